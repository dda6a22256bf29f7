// Exact symmetric group quantisation (gfx950 device code), shared by the
// residual quantiser and the quantised reference store.
//
// A scale is the fp16 nearest to max|x|/qmax and a code the integer nearest
// to x/scale, both exact round-half-even of the rational value: a cheap fp32
// estimate is corrected with comparisons that are exact in fp32 (products of
// short significands, fma remainders).
#pragma once

#include "rkv_common.h"

namespace rkv {

// fp16 nearest to a/qmax, ties to even, saturating at 65504.  a >= 0 finite.
__device__ __noinline__ inline uint16_t exact_scale_bits_slow(float a, float qmax, float inv_qmax) {
  if (a == 0.f) return 0;
  uint16_t b = f32_to_half_bits_rne(a * inv_qmax);
  if (b >= 0x7C00) b = 0x7BFF;
  float hv = half_bits_to_f32(b);
  if (b < 0x7BFF) {
    const float up = half_bits_to_f32((uint16_t)(b + 1));
    const float lim = qmax * (0.5f * (hv + up));  // exact
    if (a > lim || (a == lim && (b & 1))) {
      ++b;
      hv = up;
    }
  }
  if (b > 0) {
    const float dn = half_bits_to_f32((uint16_t)(b - 1));
    const float lim = qmax * (0.5f * (hv + dn));  // exact
    if (a < lim || (a == lim && (b & 1))) --b;
  }
  return b;
}

// Same result as exact_scale_bits_slow.  y = a * fl(1/qmax) is within 2 ulp
// of a/qmax, so its fp16 rounding is the exact one unless the 13 bits below
// fp16 precision sit within 3 of the half-way pattern 0x1000 (or y is
// outside the normal fp16 range); only those cases take the exact path.
__device__ inline uint16_t exact_scale_bits(float a, float qmax, float inv_qmax) {
  const float y = a * inv_qmax;
  const int low = (int)(__float_as_uint(y) & 0x1FFFu) - 0x1000;
  if (y >= 0x1p-14f && y < 65504.f && (low > 3 || low < -3)) return f32_to_half_bits_rne(y);
  return exact_scale_bits_slow(a, qmax, inv_qmax);
}

// exact_scale_bits, also telling whether the scale came from the plain
// rounding of a normal-range estimate.  Then the scale is within a relative
// 2^-11 of a/qmax, so |z/scale| < qmax + 1/2 for every element of the group
// (qmax <= 127) and no code of the group needs clamping.
// (The plain rounding is taken unconditionally and replaced in the rare other
// case: one divergent branch instead of a branch per condition.)
__device__ inline uint16_t exact_scale_bits_plain(float a, float qmax, float inv_qmax,
                                                  bool& plain) {
  const float y = a * inv_qmax;
  // low bits within 3 of the half-way pattern: (bits & 0x1FFF) - 0x0FFD in [0, 6]
  const uint32_t near = (__float_as_uint(y) & 0x1FFFu) - 0x0FFDu;
  plain = (y >= 0x1p-14f) & (y < 65504.f) & (near > 6u);
  uint16_t b = f32_to_half_bits_rne(y);
  if (!plain) b = exact_scale_bits_slow(a, qmax, inv_qmax);
  return b;
}

// Integer nearest to z/s (ties to even), clamped to [-qmax, qmax].  s > 0.
__device__ inline int exact_code(float z, float s, float rs, float qmax, float tol) {
  const float q = z * rs;
  float n = __builtin_rintf(q);
  if (fabsf(q - n) > 0.5f - tol) {
    // q may sit on the wrong side of a half-integer: decide exactly.
    const float n0 = n;
    const float hi = __builtin_fmaf(-(n0 + 0.5f), s, z);
    const float lo = __builtin_fmaf(-(n0 - 0.5f), s, z);
    const bool odd = ((int)n0 & 1) != 0;
    if (hi > 0.f || (hi == 0.f && odd)) n = n0 + 1.f;
    else if (lo < 0.f || (lo == 0.f && odd)) n = n0 - 1.f;
  }
  n = __builtin_amdgcn_fmed3f(n, -qmax, qmax);
  return (int)n;
}

// Codes of 8 residuals with scale s (rs ~ 1/s within 1 ulp; rs = 0 when
// s = 0).  t = fl(z*rs + 1.5*2^23) holds the integer nearest to the exact
// product z*rs (ties to even) in its low mantissa bits; r = fma(z, rs, M - t)
// is that rounding's remainder.  When a remainder is clear of 1/2 by more
// than the product's error, z*rs and z/s round alike.  Otherwise the code is
// one of the two integers either side of the half-integer b next to z*rs on
// r's side, and the sign of fma(-b, s, z) = z - b*s (exact: b*s has at most
// 19 significant bits and the difference is a multiple of 2^-149) decides it,
// ties going to the even integer (the low bit of M + code).  Returned as
// M + code (so the low bits are the two's complement code), clamped to
// [-qmax, qmax].  kClamp = false skips the clamp of the estimated codes, for
// callers that pass exact = true unless the scale keeps every code in range
// (exact_scale_bits_plain): codes that took the exact path are always
// clamped.
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

template <bool kClamp = true>
__device__ inline void codes8(const float (&z)[8], float s, float rs, float qmax, float tol,
                              uint32_t (&u)[8], bool exact = false) {
  float t[8], r[8];
  float emax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    t[e] = __builtin_fmaf(z[e], rs, kMagic);
    r[e] = __builtin_fmaf(z[e], rs, kMagic - t[e]);
    emax = fmaxf(emax, fabsf(r[e]));
  }
  if (exact || emax > 0.5f - tol) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (fabsf(r[e]) > 0.5f - tol) {
        const float lo = r[e] < 0.f ? t[e] - 1.f : t[e];   // M + the lower candidate
        const float b = (lo - kMagic) + 0.5f;              // the half-integer between them
        const float h = __builtin_fmaf(-b, s, z[e]);
        const bool odd = (__float_as_uint(lo) & 1u) != 0u;
        t[e] = (h > 0.f || (h == 0.f && odd)) ? lo + 1.f : lo;
      }
      t[e] = __builtin_amdgcn_fmed3f(t[e], kMagic - qmax, kMagic + qmax);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    u[e] = __float_as_uint(kClamp ? __builtin_amdgcn_fmed3f(t[e], kMagic - qmax, kMagic + qmax)
                                  : t[e]);
}

// Exact group quantisation of one value: scale bits of the group (a = the
// group's max |x|) and the code of x.  For code paths that are not hot.
__device__ inline int exact_code_of(float x, uint16_t sb, float qmax) {
  const float s = half_bits_to_f32(sb);
  if (!(s > 0.f)) return 0;
  const float rs = __builtin_amdgcn_rcpf(s);
  return exact_code(x, s, rs, qmax, (qmax + 1.f) * 0x1p-21f);
}

}  // namespace rkv
