// Shared device/host helpers of librkv (gfx950).
//
// Reference schedule (paper page "DeltaKV Framework Architecture": a
// reference every s-th token; news page "How ResidualKV Works": dynamic
// stride).  Position j is a reference iff j mod s(j) == 0 with s(j) = base
// below A = double_after and base * 2^b on [A*2^(b-1), A*2^b).  With A a
// multiple of 2*base every band holds A/(2*base) references and its first
// position is a reference, which gives the closed forms below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rkv {

// Lambdas that take register arrays by reference must be inlined, or the
// arrays are placed in scratch or LDS memory.
#define RKV_INLINE __attribute__((always_inline))

// Division by a constant d >= 1 for 0 <= n < 2^31 with one 32x32->64
// multiply: l = ceil(log2 d), m = floor(2^(31+l)/d) + 1, n/d = (n*m) >> (31+l)
// (Granlund-Montgomery: m*d lies in (2^(31+l), 2^(31+l) + 2^l]).
struct FastDiv {
  uint32_t d, m, s;
};

__host__ __device__ inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t m = ((1ull << (31 + l)) / d) + 1;
  return FastDiv{d, (uint32_t)m, 31 + l};
}

__host__ __device__ inline uint32_t fdiv(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}

__host__ __device__ inline int bit_width(uint32_t x) {
#ifdef __HIP_DEVICE_COMPILE__
  return x ? 32 - __clz(x) : 0;
#else
  return x ? 32 - __builtin_clz(x) : 0;
#endif
}

// Schedule constants (positions < 2^31).  A = 0: fixed stride.
struct Sched {
  int32_t base;
  int32_t A;
  int32_t c0;      // references below A: A / base
  int32_t per;     // references per doubling band: A / (2 base)
  FastDiv fb;      // / base
  FastDiv fa;      // / A
  FastDiv fp;      // / per
};

inline Sched make_sched(int64_t base, int64_t A) {
  Sched s;
  s.base = (int32_t)base;
  s.A = (int32_t)A;
  s.c0 = A ? (int32_t)(A / base) : 0;
  s.per = A ? (int32_t)(A / (2 * base)) : 1;
  s.fb = make_fastdiv((uint32_t)base);
  s.fa = make_fastdiv(A ? (uint32_t)A : 1u);
  s.fp = make_fastdiv((uint32_t)s.per);
  return s;
}

// References in [0, n), 0 <= n < 2^31.
__host__ __device__ inline int32_t sched_count(int32_t n, const Sched& s) {
  if (n <= 0) return 0;
  if (s.A == 0 || n <= s.A) return (int32_t)fdiv((uint32_t)(n + s.base - 1), s.fb);
  const int b = bit_width(fdiv((uint32_t)(n - 1), s.fa));  // band of position n-1
  const int32_t lo = s.A << (b - 1);
  const uint32_t st = (uint32_t)s.base << b;
  return s.c0 + (b - 1) * s.per +
         (int32_t)(fdiv((uint32_t)(n - lo) + st - 1, s.fb) >> b);
}

// References at positions <= i.
__host__ __device__ inline int32_t sched_count_le(int32_t i, const Sched& s) {
  return sched_count(i + 1, s);
}

// Position of reference `slot`.
__host__ __device__ inline int32_t sched_pos(int32_t slot, const Sched& s) {
  if (s.A == 0 || slot < s.c0) return slot * s.base;
  const uint32_t m = (uint32_t)(slot - s.c0);
  const uint32_t bq = fdiv(m, s.fp);
  const int band = (int)bq + 1;
  return (s.A << (band - 1)) + (int32_t)(m - bq * (uint32_t)s.per) * (s.base << band);
}

// Slot of position i if it is a reference, else -1.
__host__ __device__ inline int32_t sched_slot(int32_t i, const Sched& s) {
  if (s.A == 0 || i < s.A) {
    const uint32_t q = fdiv((uint32_t)i, s.fb);
    return (uint32_t)i == q * (uint32_t)s.base ? (int32_t)q : -1;
  }
  const int b = bit_width(fdiv((uint32_t)i, s.fa));
  const uint32_t off = (uint32_t)(i - (s.A << (b - 1)));
  const uint32_t q = fdiv(off, s.fb) >> b;
  if (off != q * ((uint32_t)s.base << b)) return -1;
  return s.c0 + (b - 1) * s.per + (int32_t)q;
}

// ---------------------------------------------------------------- numbers

// The two bf16 halves of a 32-bit word as fp32 (exact).
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline float half_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ inline uint16_t f32_to_half_bits_rne(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Load 8 consecutive elements as fp32 (exact widening).
__device__ inline void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ inline void load8(const __bf16* p, float (&x)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

__device__ inline void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

__device__ inline bool is_pow2(int v) { return (v & (v - 1)) == 0; }

// Lane exchanges inside a DPP row (16 lanes), no LDS traffic.
#define RKV_DPP_F32(v, ctrl) \
  __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), (ctrl), 0xF, 0xF, true))

// ------------------------------------------------------- latent transform
// Latent variant of the residual (paper page, "DeltaKV Framework
// Architecture": residuals of compressed projections, rebuilt by a
// decompressor).  Untrained stand-in: f_c(x) = H D x / 16, f_d(y) = D H y / 8
// with H the 128-point Walsh-Hadamard matrix (entries (-1)^popcount(i & t))
// and D = diag(+-1); f_d(f_c(x)) = x.
//
// Sign bits of D: dim t is negated iff bit t%32 of w[t/32] is set.  They are
// the top bits of the first 128 outputs of SplitMix64 started at the seed.
struct LatMask {
  uint32_t w[4];
};

inline uint64_t splitmix64_next(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline LatMask make_latmask(uint64_t seed) {
  LatMask m{{0u, 0u, 0u, 0u}};
  uint64_t st = seed;
  for (int t = 0; t < 128; ++t)
    if (splitmix64_next(st) >> 63) m.w[t >> 5] |= 1u << (t & 31);
  return m;
}

// Negate the dims of D among 8*dl .. 8*dl+7 (exact: a sign-bit flip).
__device__ inline void lat_signs8(float (&z)[8], const LatMask& lm, int dl) {
  const uint32_t word = dl < 8 ? (dl < 4 ? lm.w[0] : lm.w[1]) : (dl < 12 ? lm.w[2] : lm.w[3]);
  const uint32_t b = (word >> (8 * (dl & 3))) & 0xFFu;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = __uint_as_float(__float_as_uint(z[e]) ^ (((b >> e) & 1u) << 31));
}

// Unnormalised 128-point Walsh-Hadamard transform of a row spread over 16
// aligned lanes, lane dl holding dims 8*dl .. 8*dl+7.  Butterflies
// (a, b) -> (a + b, a - b) over index bit 0, 1, ..., 6 in that order, each
// rounded to fp32: bits 0-2 inside the lane, bits 3-6 across lanes (the lane
// holding the upper element of a pair computes partner - own).
__device__ inline void fwht128_8(float (&z)[8], int dl) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e & h) continue;
      const float a = z[e], b = z[e | h];
      z[e] = a + b;
      z[e | h] = a - b;
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    const bool hi = (dl & m) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __shfl_xor(z[e], m);
      z[e] = hi ? p - z[e] : z[e] + p;
    }
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

}  // namespace rkv
