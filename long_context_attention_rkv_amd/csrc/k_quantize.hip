// Residual quantisation and reconstruction (gfx950).
//
// Paper page "DeltaKV Framework Architecture": the residual is the token
// minus KV_R, the mean of its k nearest references, and the token comes back
// as residual + KV_R.  Section "Performance Results": the residuals suit
// token-wise quantisation.  News page "How ResidualKV Works": they are kept
// as compact quantised codes.  Section "Practical Deployment via
// Sparse-vLLM": gathering the references, the mean and the residual are one
// fused kernel.
//
// Exact rounding.  Codes and scales are decided from the fp32 residual
// z = x - fl32(fl32-sum of the selected references / k_eff), the sum taken in
// ascending slot order.  The scale is the fp16 nearest to max|z|/qmax and a
// code is the integer nearest to z/scale, both exact round-half-even of the
// rational value: a cheap fp32 estimate is corrected with comparisons that
// are exact in fp32 (products of short significands, fma remainders).
//
// Layout: 32 lanes per (token): lanes 0..15 take the K row, 16..31 the V row,
// 8 dims per lane.  A block of 512 threads covers 16 tokens per step; V codes
// are staged in LDS per tile of 32 tokens and stored transposed (for each
// dim, the tile's 32 codes are one bit string) so decode can feed them to the
// MFMA that contracts over tokens.
#include "rkv_common.h"

namespace rkv {

// fp16 nearest to a/qmax, ties to even, saturating at 65504.  a >= 0 finite.
__device__ inline uint16_t exact_scale_bits(float a, float qmax, float inv_qmax) {
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

template <int BITS>
__device__ inline void store_codes(uint8_t* p, const int (&c)[8]) {
  if constexpr (BITS == 4) {
    uint32_t w = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) w |= (uint32_t)(c[t] & 0xF) << (4 * t);
    *reinterpret_cast<uint32_t*>(p) = w;
  } else if constexpr (BITS == 8) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      w0 |= (uint32_t)(c[t] & 0xFF) << (8 * t);
      w1 |= (uint32_t)(c[t + 4] & 0xFF) << (8 * t);
    }
    *reinterpret_cast<uint2*>(p) = make_uint2(w0, w1);
  } else {
    uint32_t w = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) w |= (uint32_t)(c[t] & 0x3) << (2 * t);
    *reinterpret_cast<uint16_t*>(p) = (uint16_t)w;
  }
}

// Fixed-order fp32 mean of the selected reference rows (8 dims of them).
// All k_eff row loads are issued before the first add; the adds then run in
// ascending slot order.
template <int KM>
__device__ inline void load_slots(const uint16_t* __restrict__ irow, int k, uint32_t (&sl)[KM]) {
  if (k == KM) {
    if constexpr (KM == 4) {
      const uint2 v = *reinterpret_cast<const uint2*>(irow);
      sl[0] = v.x & 0xFFFF; sl[1] = v.x >> 16; sl[2] = v.y & 0xFFFF; sl[3] = v.y >> 16;
    } else {
#pragma unroll
      for (int c = 0; c < KM / 8; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(irow + 8 * c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sl[8 * c + 2 * e] = w[e] & 0xFFFF;
          sl[8 * c + 2 * e + 1] = w[e] >> 16;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < KM; ++j) sl[j] = j < k ? irow[j] : 0;
  }
}

template <typename T>
struct Raw8 {
  uint4 v[sizeof(T) / 2];
};

template <typename T>
__device__ inline void load_raw8(const T* p, Raw8<T>& r) {
#pragma unroll
  for (int c = 0; c < (int)(sizeof(T) / 2); ++c) r.v[c] = reinterpret_cast<const uint4*>(p)[c];
}

__device__ inline void widen8(const Raw8<__bf16>& r, float (&x)[8]) {
  x[0] = bf16_lo(r.v[0].x); x[1] = bf16_hi(r.v[0].x);
  x[2] = bf16_lo(r.v[0].y); x[3] = bf16_hi(r.v[0].y);
  x[4] = bf16_lo(r.v[0].z); x[5] = bf16_hi(r.v[0].z);
  x[6] = bf16_lo(r.v[0].w); x[7] = bf16_hi(r.v[0].w);
}

__device__ inline void widen8(const Raw8<float>& r, float (&x)[8]) {
  x[0] = __uint_as_float(r.v[0].x); x[1] = __uint_as_float(r.v[0].y);
  x[2] = __uint_as_float(r.v[0].z); x[3] = __uint_as_float(r.v[0].w);
  x[4] = __uint_as_float(r.v[1].x); x[5] = __uint_as_float(r.v[1].y);
  x[6] = __uint_as_float(r.v[1].z); x[7] = __uint_as_float(r.v[1].w);
}

template <typename T, int KM>
__device__ inline void ref_mean8(const T* __restrict__ refs, const uint16_t* __restrict__ irow,
                                 int k, int keff, float (&m)[8]) {
  uint32_t sl[KM];
  load_slots<KM>(irow, k, sl);
  Raw8<T> raw[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < keff) load_raw8(refs + (int64_t)sl[j] * 128, raw[j]);
  float acc[8];
  widen8(raw[0], acc);
#pragma unroll
  for (int j = 1; j < KM; ++j) {
    if (j < keff) {
      float r[8];
      widen8(raw[j], r);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = acc[e] + r[e];
    }
  }
  if (is_pow2(keff)) {
    const float inv = __uint_as_float((uint32_t)(127 - __builtin_ctz(keff)) << 23);  // 1/keff exactly
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = acc[e] * inv;
  } else {
    const float kf = (float)keff;
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = acc[e] / kf;  // correctly rounded
  }
}

constexpr int kQTokens = 16;   // tokens per step (512 threads)
constexpr int kVTile = 32;     // tokens per transposed V tile

template <typename T, int BITS, int KM>
__global__ __launch_bounds__(512) void k_quantize(
    const T* __restrict__ K, const T* __restrict__ V, const uint16_t* __restrict__ idx,
    const T* __restrict__ ref_kv, uint8_t* __restrict__ codes_k,
    uint8_t* __restrict__ codes_v, uint16_t* __restrict__ scales, int64_t N,
    int64_t n_refs, Sched sc, int k, int group, int chunk, int H) {
  __shared__ int8_t vt[128][kVTile + 4];
  const int tid = threadIdx.x;
  const int tok_l = tid >> 5;          // token within the step
  const int plane = (tid >> 4) & 1;    // 0 = K, 1 = V
  const int dl = tid & 15;             // dims [8*dl, 8*dl+8)
  const int64_t ih = (int64_t)blockIdx.z * H + blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  const int64_t c1 = (c0 + chunk < N) ? c0 + chunk : N;
  const T* src = (plane ? V : K) + ih * N * 128 + 8 * dl;
  const T* refs = ref_kv + (ih * 2 + plane) * n_refs * 128 + 8 * dl;
  constexpr float qmax = BITS ? (float)((1 << (BITS - 1)) - 1) : 0.f;
  const float inv_qmax = BITS ? 1.0f / qmax : 0.f;
  const float tol = (qmax + 1.f) * 0x1p-21f;  // >= 2x the error of z * rcp(s)
  const int lanes_per_group = group >> 3;
  const int n_groups = 128 / group;

  for (int64_t tb = c0; tb < c1; tb += kVTile) {
    for (int sub = 0; sub < kVTile; sub += kQTokens) {
      const int64_t tok = tb + sub + tok_l;
      int c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (tok < c1) {
        float x[8], m[8], z[8];
        load8(src + tok * 128, x);
        const int keff = (int)min((int64_t)k, sched_count_le((int32_t)tok, sc));
        ref_mean8<T, KM>(refs, idx + (ih * N + tok) * k, k, keff, m);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = x[e] - m[e];
        if constexpr (BITS == 0) {
          double* dst = reinterpret_cast<double*>(plane ? codes_v : codes_k) +
                        (ih * N + tok) * 128 + 8 * dl;
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = (double)x[e] - (double)m[e];
        } else {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(z[e]));
          for (int off = 1; off < lanes_per_group; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
          const uint16_t sb = exact_scale_bits(a, qmax, inv_qmax);
          const float s = half_bits_to_f32(sb);
          if (s > 0.f) {
            const float rs = __builtin_amdgcn_rcpf(s);  // within 1 ulp of 1/s
#pragma unroll
            for (int e = 0; e < 8; ++e) c[e] = exact_code(z[e], s, rs, qmax, tol);
          }
          if ((dl & (lanes_per_group - 1)) == 0)
            scales[((ih * N + tok) * 2 + plane) * n_groups + dl / lanes_per_group] = sb;
          if (plane == 0)
            store_codes<BITS>(codes_k + (ih * N + tok) * (128 * BITS / 8) + dl * BITS, c);
        }
      }
      if constexpr (BITS != 0) {
        if (plane == 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) vt[8 * dl + e][sub + tok_l] = (int8_t)c[e];
        }
      }
    }
    if constexpr (BITS != 0) {
      __syncthreads();
      // 512 threads: dim = tid/4, tokens 8*(tid%4) .. +7 of the tile
      const int dim = tid >> 2;
      const int u = tid & 3;
      int cc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cc[e] = vt[dim][8 * u + e];
      const int64_t tile = tb / kVTile;
      store_codes<BITS>(codes_v + ((ih * ((N + kVTile - 1) / kVTile) + tile) * 128 + dim) *
                                      (kVTile * BITS / 8) + u * BITS,
                        cc);
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------ reconstruct
template <int BITS>
__device__ inline int code_at(const uint8_t* row, int t) {
  if constexpr (BITS == 8) return (int)(int8_t)row[t];
  const int bit = t * BITS;
  const int v = (row[bit >> 3] >> (bit & 7)) & ((1 << BITS) - 1);
  return v >= (1 << (BITS - 1)) ? v - (1 << BITS) : v;
}

template <typename T, int BITS, int KM>
__global__ __launch_bounds__(512) void k_reconstruct(
    const uint16_t* __restrict__ idx, const T* __restrict__ ref_kv,
    const uint8_t* __restrict__ codes_k, const uint8_t* __restrict__ codes_v,
    const uint16_t* __restrict__ scales, float* __restrict__ Kh, float* __restrict__ Vh,
    int64_t N, int64_t n_refs, Sched sc, int k, int group, int H) {
  const int tid = threadIdx.x;
  const int plane = (tid >> 4) & 1;
  const int dl = tid & 15;
  const int64_t ih = (int64_t)blockIdx.z * H + blockIdx.y;
  const int64_t tok = (int64_t)blockIdx.x * kQTokens + (tid >> 5);
  if (tok >= N) return;
  const T* refs = ref_kv + (ih * 2 + plane) * n_refs * 128 + 8 * dl;
  float* dst = (plane ? Vh : Kh) + (ih * N + tok) * 128 + 8 * dl;
  float out[8];
  const int64_t slot = sched_slot((int32_t)tok, sc);
  if (slot >= 0) {
    load8(refs + slot * 128, out);
    store8(dst, out);
    return;
  }
  float m[8];
  const int keff = (int)min((int64_t)k, sched_count_le((int32_t)tok, sc));
  ref_mean8<T, KM>(refs, idx + (ih * N + tok) * k, k, keff, m);
  if constexpr (BITS == 0) {
    const double* r = reinterpret_cast<const double*>(plane ? codes_v : codes_k) +
                      (ih * N + tok) * 128 + 8 * dl;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)((double)m[e] + r[e]);
  } else {
    const int n_groups = 128 / group;
    const float s = half_bits_to_f32(
        scales[((ih * N + tok) * 2 + plane) * n_groups + (8 * dl) / group]);
    if (plane == 0) {
      const uint8_t* row = codes_k + (ih * N + tok) * (128 * BITS / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = m[e] + s * (float)code_at<BITS>(row, 8 * dl + e);
    } else {
      const int64_t tile = tok / kVTile;
      const int u = (int)(tok % kVTile);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint8_t* row = codes_v + ((ih * ((N + kVTile - 1) / kVTile) + tile) * 128 +
                                        8 * dl + e) * (kVTile * BITS / 8);
        out[e] = m[e] + s * (float)code_at<BITS>(row, u);
      }
    }
  }
  store8(dst, out);
}

// ------------------------------------------------------------ launchers
template <typename T, int BITS>
hipError_t launch_quantize_t(const void* K, const void* V, const uint16_t* idx,
                             const void* ref_kv, uint8_t* ck, uint8_t* cv, uint16_t* sc16,
                             int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc,
                             int k, int group, hipStream_t st) {
  const int chunk = 256;
  const int64_t nchunks = (N + chunk - 1) / chunk;
  auto kern = k <= 4 ? k_quantize<T, BITS, 4> : (k <= 8 ? k_quantize<T, BITS, 8>
                                                       : k_quantize<T, BITS, 16>);
  hipLaunchKernelGGL(kern, dim3((unsigned)nchunks, H, (unsigned)n_inst),
                     dim3(512), 0, st, (const T*)K, (const T*)V, idx, (const T*)ref_kv, ck,
                     cv, sc16, N, n_refs, sc, k, group, chunk, H);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_quantize_d(int bits, const void* K, const void* V, const uint16_t* idx,
                             const void* ref_kv, uint8_t* ck, uint8_t* cv, uint16_t* sc16,
                             int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc,
                             int k, int group, hipStream_t st) {
  switch (bits) {
    case 0: return launch_quantize_t<T, 0>(K, V, idx, ref_kv, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, st);
    case 2: return launch_quantize_t<T, 2>(K, V, idx, ref_kv, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, st);
    case 4: return launch_quantize_t<T, 4>(K, V, idx, ref_kv, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, st);
    default: return launch_quantize_t<T, 8>(K, V, idx, ref_kv, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, st);
  }
}

hipError_t launch_quantize(int dtype, int bits, const void* K, const void* V,
                           const uint16_t* idx, const void* ref_kv, uint8_t* ck, uint8_t* cv,
                           uint16_t* sc16, int64_t n_inst, int H, int64_t N, int64_t n_refs,
                           Sched sc, int k, int group, hipStream_t st) {
  if (N == 0 || n_inst == 0) return hipSuccess;
  if (dtype == 0)
    return launch_quantize_d<float>(bits, K, V, idx, ref_kv, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, st);
  return launch_quantize_d<__bf16>(bits, K, V, idx, ref_kv, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, st);
}

template <typename T, int BITS>
hipError_t launch_recon_t(const uint16_t* idx, const void* ref_kv, const uint8_t* ck,
                          const uint8_t* cv, const uint16_t* sc16, float* Kh, float* Vh,
                          int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc, int k,
                          int group, hipStream_t st) {
  const int64_t blocks = (N + kQTokens - 1) / kQTokens;
  auto kern = k <= 4 ? k_reconstruct<T, BITS, 4>
                     : (k <= 8 ? k_reconstruct<T, BITS, 8> : k_reconstruct<T, BITS, 16>);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks, H, (unsigned)n_inst),
                     dim3(512), 0, st, idx, (const T*)ref_kv, ck, cv, sc16, Kh, Vh, N, n_refs,
                     sc, k, group, H);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_recon_d(int bits, const uint16_t* idx, const void* ref_kv, const uint8_t* ck,
                          const uint8_t* cv, const uint16_t* sc16, float* Kh, float* Vh,
                          int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc, int k,
                          int group, hipStream_t st) {
  switch (bits) {
    case 0: return launch_recon_t<T, 0>(idx, ref_kv, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, st);
    case 2: return launch_recon_t<T, 2>(idx, ref_kv, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, st);
    case 4: return launch_recon_t<T, 4>(idx, ref_kv, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, st);
    default: return launch_recon_t<T, 8>(idx, ref_kv, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, st);
  }
}

hipError_t launch_reconstruct(int dtype, int bits, const uint16_t* idx, const void* ref_kv,
                              const uint8_t* ck, const uint8_t* cv, const uint16_t* sc16,
                              float* Kh, float* Vh, int64_t n_inst, int H, int64_t N,
                              int64_t n_refs, Sched sc, int k, int group, hipStream_t st) {
  if (N == 0 || n_inst == 0) return hipSuccess;
  if (dtype == 0)
    return launch_recon_d<float>(bits, idx, ref_kv, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, st);
  return launch_recon_d<__bf16>(bits, idx, ref_kv, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, st);
}

}  // namespace rkv
