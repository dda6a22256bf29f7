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
// Layout: 16 lanes per (token, plane), 8 dims per lane; waves 0-3 of a
// 512-thread block take the K rows and waves 4-7 the V rows of the same 16
// tokens per step.  V codes are staged in LDS per tile of 32 tokens and
// stored transposed (for each dim, the tile's 32 codes are one bit string) so
// decode can feed them to the MFMA that contracts over tokens.  The
// reconstruction kernel keeps 32 lanes per token (16 for K, 16 for V).
#include <type_traits>

#include <utility>

#include "rkv_common.h"
#include "rkv_quant.h"

namespace rkv {

// A word of packed codes (BITS bytes: 8 codes) and stores of it: whole, or
// only the fields of elements lo .. hi-1 (the others keep their bits).
template <int BITS>
__device__ inline void store_word(uint8_t* p, uint64_t w) {
  if constexpr (BITS == 8) *reinterpret_cast<uint64_t*>(p) = w;
  else if constexpr (BITS == 4) *reinterpret_cast<uint32_t*>(p) = (uint32_t)w;
  else *reinterpret_cast<uint16_t*>(p) = (uint16_t)w;
}

template <int BITS>
__device__ inline void store_word_range(uint8_t* p, uint64_t w, int lo, int hi) {
  const uint64_t full = BITS == 8 ? ~0ull : ((1ull << (8 * BITS)) - 1);
  const uint64_t below_hi = hi >= 8 ? full : ((1ull << (BITS * hi)) - 1);
  const uint64_t below_lo = (1ull << (BITS * lo)) - 1;  // lo <= 7 here
  const uint64_t m = below_hi & ~below_lo;
  if constexpr (BITS == 8) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    *q = (*q & ~m) | (w & m);
  } else if constexpr (BITS == 4) {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    *q = (uint32_t)((*q & ~m) | (w & m));
  } else {
    uint16_t* q = reinterpret_cast<uint16_t*>(p);
    *q = (uint16_t)((*q & ~m) | (w & m));
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

// Reference rows of one (instance, head, plane), the 8 dims of this lane:
// raw rows of T, or (RQ) int4 nibbles + one fp16 scale per group.
template <typename T, bool RQ>
struct RefSrc {
  const T* raw;           // row slot at raw + slot * 128
  const uint8_t* codes;   // row slot at codes + slot * 64 (4 bytes = 8 nibbles)
  const uint16_t* sc;     // scale of this lane's group at sc + slot * ng
  int ng;
};

// 8 nibbles of a quantised row times its scale: exact fp32 values.
__device__ inline void dequant8(uint32_t w, uint16_t sb, float (&x)[8]) {
  const float s = half_bits_to_f32(sb);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)((int32_t)(w << (28 - 4 * e)) >> 28) * s;
}

template <typename T, bool RQ>
__device__ inline void ref_row8(const RefSrc<T, RQ>& r, uint32_t slot, float (&x)[8]) {
  if constexpr (RQ) {
    dequant8(*reinterpret_cast<const uint32_t*>(r.codes + slot * 64u), r.sc[slot * (uint32_t)r.ng], x);
  } else {
    load8(r.raw + slot * 128u, x);
  }
}

// Mean of the k_eff selected rows: all loads first, then the fixed
// ascending-slot fp32 sum and one multiply by 1/k_eff (power of two) or a
// correctly rounded division.
template <typename T, int KM, bool RQ>
__device__ inline void ref_mean8_src(const RefSrc<T, RQ>& src, const uint16_t* __restrict__ irow,
                                     int k, int keff, float (&m)[8]) {
  if constexpr (!RQ) {
    ref_mean8<T, KM>(src.raw, irow, k, keff, m);
  } else {
    uint32_t sl[KM];
    load_slots<KM>(irow, k, sl);
    uint32_t w[KM];
    uint16_t sb[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < keff) {
        w[j] = *reinterpret_cast<const uint32_t*>(src.codes + sl[j] * 64u);
        sb[j] = src.sc[sl[j] * (uint32_t)src.ng];
      }
    }
    float acc[8];
    dequant8(w[0], sb[0], acc);
#pragma unroll
    for (int j = 1; j < KM; ++j) {
      if (j < keff) {
        float r[8];
        dequant8(w[j], sb[j], r);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + r[e];
      }
    }
    if (is_pow2(keff)) {
      const float inv = __uint_as_float((uint32_t)(127 - __builtin_ctz(keff)) << 23);
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = acc[e] * inv;
    } else {
      const float kf = (float)keff;
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = acc[e] / kf;
    }
  }
}


constexpr int kQTokens = 16;   // positions per step (512 threads)
constexpr int kVTile = 32;     // positions per transposed V tile

// 16 (8) bytes at byte offset `off` from a block-uniform base: one global
// load with the base in scalar registers and a 32-bit lane offset.
RKV_INLINE __device__ inline u32x4 ld16(const void* base, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + off);
}
RKV_INLINE __device__ inline uint2 ld8(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(base) + off);
}

// Largest of non-negative floats over aligned groups of `lanes` lanes (4, 8
// or 16).  For such values the bit patterns order like the values, so each
// stage is one unsigned max with a DPP operand: swaps within quads, then
// half-row and row mirrors.
__device__ inline float group_max_nonneg(float v, int lanes) {
  uint32_t u = __float_as_uint(v);
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, true));
  if (lanes >= 8) u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, true));
  if (lanes >= 16) u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x140, 0xF, 0xF, true));
  return __uint_as_float(u);
}

// Low bytes of a, b, c, d as bytes 0..3 of one word (v_perm_b32 takes
// bytes 0-3 from its second operand and 4-7 from its first; selector 0x0C
// gives a zero byte).
RKV_INLINE __device__ inline uint32_t low_bytes4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_amdgcn_perm(b, a, 0x0C0C0400u) | __builtin_amdgcn_perm(d, c, 0x04000C0Cu);
}

// The two's complement codes in the low bits of w[0..7], packed BITS to a
// field in element order (element 0 lowest).  For 4 bits the even elements'
// low nibbles stay in place and the odd elements' move up into the high
// nibble of the same byte.
template <int BITS>
RKV_INLINE __device__ inline uint64_t pack8(const uint32_t (&w)[8]) {
  if constexpr (BITS == 8) {
    return (uint64_t)low_bytes4(w[4], w[5], w[6], w[7]) << 32 | low_bytes4(w[0], w[1], w[2], w[3]);
  } else if constexpr (BITS == 4) {
    const uint32_t ev = low_bytes4(w[0], w[2], w[4], w[6]);
    const uint32_t od = low_bytes4(w[1], w[3], w[5], w[7]);
    return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
  } else {
    uint32_t v = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) v |= (w[t] & 0x3u) << (2 * t);
    return v;
  }
}

// Raw buffer descriptor of a byte range starting at p (no range limit).
RKV_INLINE __device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, -1, 0x00020000);
}

// One word of packed codes (BITS bytes) at byte offset off of a buffer.
template <int BITS>
RKV_INLINE __device__ inline void buffer_store_word(__amdgpu_buffer_rsrc_t r, uint32_t off, uint64_t w) {
  if constexpr (BITS == 8) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{(uint32_t)w, (uint32_t)(w >> 32)}, r, (int)off, 0, 0);
  } else if constexpr (BITS == 4) {
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)w, r, (int)off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)w, r, (int)off, 0, 0);
  }
}

// Eight elements as fp32 from their raw 16 bytes (bf16) or 32 bytes (fp32).
RKV_INLINE __device__ inline void widen(const u32x4 (&r)[1], float (&x)[8]) {
  x[0] = bf16_lo(r[0].x); x[1] = bf16_hi(r[0].x);
  x[2] = bf16_lo(r[0].y); x[3] = bf16_hi(r[0].y);
  x[4] = bf16_lo(r[0].z); x[5] = bf16_hi(r[0].z);
  x[6] = bf16_lo(r[0].w); x[7] = bf16_hi(r[0].w);
}
RKV_INLINE __device__ inline void widen(const u32x4 (&r)[2], float (&x)[8]) {
  x[0] = __uint_as_float(r[0].x); x[1] = __uint_as_float(r[0].y);
  x[2] = __uint_as_float(r[0].z); x[3] = __uint_as_float(r[0].w);
  x[4] = __uint_as_float(r[1].x); x[5] = __uint_as_float(r[1].y);
  x[6] = __uint_as_float(r[1].z); x[7] = __uint_as_float(r[1].w);
}

// Loads of one position issued a step ahead on the fast path: its 8
// elements of the row and its KM slots (KM = 4: the first 8 bytes).
template <typename T, int KM>
struct PosLoads {
  u32x4 x[sizeof(T) / 2];
  u32x4 sl[(KM + 7) / 8];
};

// The word holding slots j & ~1 and j | 1 of a position.
template <typename T, int KM>
RKV_INLINE __device__ inline uint32_t slot_word(const PosLoads<T, KM>& p, int j) {
  const u32x4 v = p.sl[j >> 3];
  const int q = (j >> 1) & 3;
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// Slot words of a position: lane c (c < KM/2) of its 16 lanes loaded word c;
// DPP row_newbcast:c gives every lane of the 16-lane row the word of lane c.
template <int... C>
RKV_INLINE __device__ inline void row_bcast_words(int w0, uint32_t* wd,
                                                  std::integer_sequence<int, C...>) {
  ((wd[C] = (uint32_t)__builtin_amdgcn_mov_dpp(w0, 0x150 + C, 0xF, 0xF, false)), ...);
}
template <typename T, int KM>
RKV_INLINE __device__ inline void spread_slot_words(PosLoads<T, KM>& p) {
  uint32_t wd[KM / 2];
  row_bcast_words((int)p.sl[0].x, wd, std::make_integer_sequence<int, KM / 2>{});
#pragma unroll
  for (int c = 0; c < (KM + 7) / 8; ++c)
    p.sl[c] = u32x4{wd[4 * c], wd[4 * c + 1], 4 * c + 2 < KM / 2 ? wd[4 * c + 2] : 0u,
                    4 * c + 3 < KM / 2 ? wd[4 * c + 3] : 0u};
}

// Byte offset of this lane's piece of the raw reference row whose slot is
// the low (half = 0) or high half of w: slot * 128 * sizeof(T) + 8 * dl *
// sizeof(T), from lane16 = 16 * dl < 256.  The bf16 offset is one byte
// permute (byte 0 = lane16, bytes 1-2 = the slot, byte 3 = 0); fp32 doubles it.
template <typename T>
RKV_INLINE __device__ inline uint32_t ref_piece_off(uint32_t w, int half, uint32_t lane16) {
  const uint32_t o = __builtin_amdgcn_perm(w, lane16, half ? 0x0C070600u : 0x0C050400u);
  return sizeof(T) == 2 ? o : o << 1;
}

// One block = one chunk of positions of one (instance, head).  Waves 0-3
// take the K rows and waves 4-7 the V rows, so every branch on the plane is
// uniform in a wave; a wave holds 4 positions, 16 lanes per position with 8
// dims each, and a step covers 16 positions.  When every position of the
// chunk has k = KM candidates (all but the first chunks of a sequence) a
// position's row and slots are loaded one step ahead and every load is
// unconditional (positions outside the range reread a row of the range and
// store nothing); otherwise k_eff is taken per position.
template <typename T, int BITS, int KM, bool RQ, bool LAT>
__global__ __launch_bounds__(512, KM <= 8 ? 6 : 4) void k_quantize(
    const T* __restrict__ K, const T* __restrict__ V, const uint16_t* __restrict__ idx,
    const T* __restrict__ ref_kv, const uint16_t* __restrict__ ref_scales,
    uint8_t* __restrict__ codes_k,
    uint8_t* __restrict__ codes_v, uint16_t* __restrict__ scales, int64_t N,
    int64_t n_refs, Sched sc, int k, int group, int chunk, int H, int p0, int n_in,
    LatMask lm) {
  __shared__ int8_t vt[128][kVTile + 1];  // odd pitch: the 16 writing lanes hit 16 banks
  const int tid = threadIdx.x;
  const int plane = __builtin_amdgcn_readfirstlane(tid >> 8);  // 0 = K, 1 = V
  const int tok_l = (tid >> 4) & 15;   // position within the step
  const int dl = tid & 15;             // dims [8*dl, 8*dl+8)
  // Workgroups are dealt to the 8 XCDs in turn.  When the heads split evenly
  // over them, the i-th workgroup of XCD x takes chunk i % C of head
  // 8 (i / C) + x, so the chunks of one head run together on one XCD and
  // share its L2 copy of the head's reference rows.
  int64_t ih = (int64_t)blockIdx.z * H + blockIdx.y;
  int chunk_id = (int)blockIdx.x;
  if (((gridDim.y * gridDim.z) & 7u) == 0) {
    const int64_t nc = gridDim.x;
    const int64_t L = blockIdx.x + nc * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t i = L >> 3;
    ih = 8 * (i / nc) + (L & 7);
    chunk_id = (int)(i % nc);
  }
  // positions [p0, p1) from input rows [ih][n_in][128]; chunks start on
  // tile boundaries (no two blocks share a transposed V tile); positions of
  // a chunk outside [p0, p1) are skipped and keep their codes
  const int p1 = p0 + n_in;
  const int c0 = (p0 & ~(kVTile - 1)) + chunk_id * chunk;
  const int c1 = c0 + chunk < p1 ? c0 + chunk : p1;
  const int v0 = c0 > p0 ? c0 : p0;
  const int n_groups = 128 / group;
  const int lanes_per_group = group >> 3;
  const uint32_t vspan = (uint32_t)(c1 - v0);  // t is ours iff (uint32_t)(t - v0) < vspan
  // Block-uniform bases at position c0: position t of the chunk is reached
  // with the 32-bit offset (t - c0) * (bytes per position).  Positions below
  // p0 have no input row and are never read.
  constexpr uint32_t kRowBytes = 128 * sizeof(T);
  const uint32_t lane16 = 16u * dl;
  const uint32_t lane_off = 8u * dl * sizeof(T);
  const T* xb = (plane ? V : K) + (ih * n_in + (c0 - p0)) * 128;
  const uint16_t* ib = idx + (ih * N + c0) * k;
  // the K codes and the scales are written through buffer descriptors (the
  // base stays in scalar registers; each store takes a 32-bit lane offset)
  const __amdgpu_buffer_rsrc_t kb =
      make_rsrc(codes_k + (ih * N + c0) * (128 * BITS / 8));
  const uint32_t k_lane = dl * BITS;
  const __amdgpu_buffer_rsrc_t sbb =
      make_rsrc(scales + (ih * N + c0) * 2 * n_groups + plane * n_groups);
  const uint32_t s_lane = 2u * (dl / lanes_per_group);
  const bool scale_lane = (dl & (lanes_per_group - 1)) == 0;
  const T* rb = ref_kv + (ih * 2 + plane) * n_refs * 128;  // raw rows of this plane
  RefSrc<T, RQ> refs;
  refs.ng = n_groups;
  if constexpr (RQ) {
    refs.codes = reinterpret_cast<const uint8_t*>(ref_kv) + (ih * 2 + plane) * n_refs * 64 + 4 * dl;
    refs.sc = ref_scales + (ih * 2 + plane) * n_refs * n_groups + (8 * dl) / group;
  } else {
    refs.raw = rb + 8 * dl;
  }
  constexpr float qmax = BITS ? (float)((1 << (BITS - 1)) - 1) : 0.f;
  constexpr float inv_qmax = BITS ? 1.0f / qmax : 0.f;
  constexpr float tol = (qmax + 1.f) * 0x1p-21f;  // >= 2x the error of z * rcp(s)
  const bool fast = k == KM && sched_count_le(c0, sc) >= KM;

  // Scale and codes of position c0 + r from its residual z (fp32, exact);
  // stores the scale and (K rows) the codes when `mine`, and leaves the
  // codes in the low bits of u (V rows stage them).
  auto finish = [&](uint32_t r, bool mine, float (&z)[8], uint32_t (&u)[8]) RKV_INLINE {
    if constexpr (LAT) {
      // latent residual f_c(z) = H D z / 16 (the 16 lanes of the row share r)
      lat_signs8(z, lm, dl);
      fwht128_8(z, dl);
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] *= 0.0625f;
    }
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(z[e]));
    a = group_max_nonneg(a, lanes_per_group);
    bool plain;
    const uint16_t sbits = exact_scale_bits_plain(a, qmax, inv_qmax, plain);
    const float s = half_bits_to_f32(sbits);
    const float rs = s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f;  // within 1 ulp of 1/s
    // a scale that is not plain (rare) has every code decided exactly and clamped
    codes8<false>(z, s, rs, qmax, tol, u, !plain);
    if (mine && scale_lane)
      __builtin_amdgcn_raw_buffer_store_b16(sbits, sbb, (int)(r * (4u * n_groups) + s_lane), 0, 0);
    if (plane == 0 && mine) buffer_store_word<BITS>(kb, r * (16u * BITS) + k_lane, pack8<BITS>(u));
  };
  // BITS = 0: the residual kept as fp64 x - fp64 mean.
  auto store_delta = [&](uint32_t r, const float (&x)[8], const float (&m)[8]) RKV_INLINE {
    double* dst = reinterpret_cast<double*>(plane ? codes_v : codes_k) +
                  (ih * N + c0 + r) * 128 + 8 * dl;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = (double)x[e] - (double)m[e];
  };
  auto issue = [&](int t, PosLoads<T, KM>& p) RKV_INLINE {
    const uint32_t r = (uint32_t)(t - c0);
#pragma unroll
    for (int c = 0; c < (int)(sizeof(T) / 2); ++c)
      p.x[c] = ld16(xb, r * kRowBytes + lane_off + 16u * c);
    // one slot word per lane (lanes 0 .. KM/2-1 of the position's 16 hold
    // words 0 .. KM/2-1); the step spreads them over the 16 lanes before the
    // gathers
    p.sl[0].x = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(ib) +
                                                   r * (2u * KM) + 4u * (dl & (KM / 2 - 1)));
  };
  auto clamp_pos = [&](int t) RKV_INLINE { return min(max(t, v0), c1 - 1); };
  // One step of the fast path: request the loads of position t + 16 into
  // `nxt`, then finish position t from `cur`.
  auto fast_step = [&](int t, PosLoads<T, KM>& cur, PosLoads<T, KM>& nxt,
                       uint32_t (&u)[8]) RKV_INLINE {
    issue(clamp_pos(t + kQTokens), nxt);
    const bool mine = (uint32_t)(t - v0) < vspan;
    const uint32_t r = (uint32_t)(t - c0);
    spread_slot_words<T, KM>(cur);
    // fixed ascending-slot fp32 sum of the KM rows (all loads first)
    float acc[8];
    if constexpr (RQ) {
      uint32_t w[KM];
      uint16_t sbr[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const uint32_t slot = (slot_word(cur, j) >> (16 * (j & 1))) & 0xFFFFu;
        w[j] = *reinterpret_cast<const uint32_t*>(refs.codes + slot * 64u);
        sbr[j] = refs.sc[slot * (uint32_t)n_groups];
      }
      dequant8(w[0], sbr[0], acc);
#pragma unroll
      for (int j = 1; j < KM; ++j) {
        float rr[8];
        dequant8(w[j], sbr[j], rr);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + rr[e];
      }
    } else {
      u32x4 g[KM][sizeof(T) / 2];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        const uint32_t o = ref_piece_off<T>(slot_word(cur, j), j & 1, lane16);
#pragma unroll
        for (int c = 0; c < (int)(sizeof(T) / 2); ++c) g[j][c] = ld16(rb, o + 16u * c);
      }
      widen(g[0], acc);
#pragma unroll
      for (int j = 1; j < KM; ++j) {
        float rr[8];
        widen(g[j], rr);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + rr[e];
      }
    }
    float x[8];
    widen(cur.x, x);
    constexpr float inv = 1.0f / KM;  // KM is 4, 8 or 16: exact
    if constexpr (BITS == 0) {
      float m[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) m[e] = acc[e] * inv;
      if (mine) store_delta(r, x, m);
    } else {
      float z[8];
      if constexpr (sizeof(T) == 2 || RQ) {
        // acc / KM is exact here (bf16 rows and dequantised rows are
        // multiples of 2^-133 and 2^-24, and so is their fp32 sum), so one
        // fma gives fl(x - fl(acc / KM)).
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = __builtin_fmaf(acc[e], -inv, x[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = x[e] - acc[e] * inv;
      }
      finish(r, mine, z, u);
    }
  };
  auto slow_step = [&](int t, uint32_t (&u)[8]) RKV_INLINE {
    if ((uint32_t)(t - v0) < vspan) {
      const uint32_t r = (uint32_t)(t - c0);
      float x[8], m[8];
      load8(xb + r * 128u + 8 * dl, x);
      const int keff = min(k, sched_count_le(t, sc));
      ref_mean8_src<T, KM, RQ>(refs, ib + r * (uint32_t)k, k, keff, m);
      if constexpr (BITS == 0) {
        store_delta(r, x, m);
      } else {
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = x[e] - m[e];
        finish(r, true, z, u);
      }
    }
  };
  auto stage_v = [&](int sub, const uint32_t (&u)[8]) RKV_INLINE {
    if constexpr (BITS != 0) {
      if (plane == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vt[8 * dl + e][sub + tok_l] = (int8_t)u[e];
      }
    }
  };
  auto store_v_tile = [&](int tb) RKV_INLINE {
    if constexpr (BITS != 0) {
      __syncthreads();
      // 512 threads: dim = tid/4, positions 8*(tid%4) .. +7 of the tile
      const int dim = tid >> 2;
      const int uu = tid & 3;
      uint32_t cc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cc[e] = (uint8_t)vt[dim][8 * uu + e];
      const int64_t tile = tb / kVTile;
      uint8_t* dst = codes_v + ((ih * ((N + kVTile - 1) / kVTile) + tile) * 128 + dim) *
                                   (kVTile * BITS / 8) + uu * BITS;
      const int g0 = tb + 8 * uu;  // positions g0 .. g0+7
      const uint64_t wv = pack8<BITS>(cc);
      if (g0 >= v0 && g0 + 8 <= c1) {
        store_word<BITS>(dst, wv);
      } else {
        // a tile cut by the range: only positions v0 .. c1-1 are ours
        const int lo = v0 - g0 < 0 ? 0 : v0 - g0;
        const int hi = c1 - g0 > 8 ? 8 : c1 - g0;
        if (lo < hi) store_word_range<BITS>(dst, wv, lo, hi);
      }
      __syncthreads();
    }
  };

  if (fast) {
    PosLoads<T, KM> pa, pb;
    issue(clamp_pos(c0 + tok_l), pa);
    for (int tb = c0; tb < c1; tb += kVTile) {
      uint32_t u0[8], u1[8];
      fast_step(tb + tok_l, pa, pb, u0);
      stage_v(0, u0);
      fast_step(tb + kQTokens + tok_l, pb, pa, u1);
      stage_v(kQTokens, u1);
      store_v_tile(tb);
    }
  } else {
    for (int tb = c0; tb < c1; tb += kVTile) {
      for (int sub = 0; sub < kVTile; sub += kQTokens) {
        uint32_t u[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        slow_step(tb + sub + tok_l, u);
        stage_v(sub, u);
      }
      store_v_tile(tb);
    }
  }
}

// ------------------------------------------------- quantise, LDS gathers
// The same computation with the reference rows gathered from LDS instead of
// the L1/L2 path (bf16 caches whose reference rows of one plane fit in
// 128 KB, i.e. up to 512 references): one block of 16 waves takes one plane (K or V) of one
// (instance, head) over a chunk of 32-position tiles and first copies that
// plane's reference rows (the ones positions below the range end can
// select) into LDS, so every gather of the chunk is an LDS read.  Each wave
// owns whole tiles: at step s (0..7) its four 16-lane rows take positions
// 8 r + s of the tile (r = lane / 16), so after the 8 steps a lane holds,
// for each of its 8 dims, the codes of 8 consecutive positions -- one word
// of the transposed V layout -- and writes it directly (no LDS staging, no
// block barrier after the copy).
//
// Arithmetic: the selected rows are summed with v_dot2_f32_bf16 (one
// element times -1/k plus the running fp32 sum: no unpacking, and the
// scaling is exact, so the partial sums are those of the plain sum scaled),
// then the token row enters the same way times 1: z = fl(x - sum / k)
// (positions with fewer than k candidates, in a sequence's first tiles,
// sum the rows plainly and divide by k_eff); scales and codes are the
// exact round-half-even of
// max|z| / qmax and z / scale, as in k_quantize (bf16 data puts many z /
// scale exactly on a half-integer, so the tie must be decided exactly).
//
// Loads: a wave keeps RD steps' rows and slot words in flight (a whole
// tile, 8 steps, in the common forms; 4 where registers are short): each
// step's registers are refilled with the step RD later -- of this tile or of
// the wave's next one -- as soon as the step is done.
constexpr int kLdsQWaves = 16;             // waves per block
constexpr int kLdsRefBytes = 128 * 1024;   // reference rows of one plane held in LDS
constexpr int kLdsChunkTiles = 256;        // tiles per block

// bf16 pair selectors (the low or the high element of a word times a power
// of two), held in registers: as a compile-time operand the compiler encodes
// the low selector 0x00003F80 as the inline constant 1.0, which
// v_dot2c_f32_bf16 does not read as that pattern (sums measured wrong on the
// device), so the patterns are moved into VGPRs by hand once per kernel.
// make_bf16_sel gives the factor 1; make_bf16_nsel<KM> the factor -1/KM
// (KM = 4, 8, 16: bf16 0xBE80, 0xBE00, 0xBD80), exact for every bf16 value
// that is not below 2^-122 in magnitude.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
struct Bf16Sel {
  bf16x2_t lo, hi;
};
RKV_INLINE __device__ inline Bf16Sel make_bf16_sel() {
  uint32_t lo, hi;
  asm volatile("v_mov_b32 %0, 0x3f80" : "=v"(lo));
  asm volatile("v_mov_b32 %0, 0x3f800000" : "=v"(hi));
  return Bf16Sel{__builtin_bit_cast(bf16x2_t, lo), __builtin_bit_cast(bf16x2_t, hi)};
}
template <int KM>
RKV_INLINE __device__ inline Bf16Sel make_bf16_nsel() {
  static_assert(KM == 4 || KM == 8 || KM == 16, "power-of-two slot counts");
  uint32_t lo, hi;
  if constexpr (KM == 4) {
    asm volatile("v_mov_b32 %0, 0xbe80" : "=v"(lo));
    asm volatile("v_mov_b32 %0, 0xbe800000" : "=v"(hi));
  } else if constexpr (KM == 8) {
    asm volatile("v_mov_b32 %0, 0xbe00" : "=v"(lo));
    asm volatile("v_mov_b32 %0, 0xbe000000" : "=v"(hi));
  } else {
    asm volatile("v_mov_b32 %0, 0xbd80" : "=v"(lo));
    asm volatile("v_mov_b32 %0, 0xbd800000" : "=v"(hi));
  }
  return Bf16Sel{__builtin_bit_cast(bf16x2_t, lo), __builtin_bit_cast(bf16x2_t, hi)};
}

// acc = the 8 elements of a bf16 row piece times the selectors' factor: the
// three-operand dot with a zero addend (the builtin becomes the two-operand
// form, which needs the zero moved into acc first).  The product is exact,
// so the result needs no rounding.
RKV_INLINE __device__ inline float dot2_sel0(uint32_t w, bf16x2_t sel) {
  float d;
  asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(d) : "v"(w), "v"(sel));
  return d;
}
RKV_INLINE __device__ inline void acc_set8(const u32x4 (&r)[1], float (&acc)[8], const Bf16Sel& sl) {
  const uint32_t wd[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] = dot2_sel0(wd[q], sl.lo);
    acc[2 * q + 1] = dot2_sel0(wd[q], sl.hi);
  }
}

// acc += the 8 elements of a raw row piece times the selectors' factor
// (bf16: 16 bytes; fp32: 32 bytes, factor 1).
RKV_INLINE __device__ inline void acc_add8(const u32x4 (&r)[1], float (&acc)[8], const Bf16Sel& sl) {
  const uint32_t wd[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const bf16x2_t v = __builtin_bit_cast(bf16x2_t, wd[q]);
    acc[2 * q] = __builtin_amdgcn_fdot2_f32_bf16(v, sl.lo, acc[2 * q], false);
    acc[2 * q + 1] = __builtin_amdgcn_fdot2_f32_bf16(v, sl.hi, acc[2 * q + 1], false);
  }
}
RKV_INLINE __device__ inline void acc_add8(const u32x4 (&r)[2], float (&acc)[8], const Bf16Sel&) {
  float x[8];
  widen(r, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] += x[e];
}

// LDS row piece of `slot` for this lane (byte offset from ref_piece_off).
template <typename T>
RKV_INLINE __device__ inline void lds_piece(const char* base, uint32_t off, u32x4 (&r)[sizeof(T) / 2]) {
#pragma unroll
  for (int c = 0; c < (int)(sizeof(T) / 2); ++c)
    r[c] = *reinterpret_cast<const u32x4*>(base + off + 16u * c);
}

// This lane's 8 codes of the V plane at step s (position 8 r + s of the
// tile), packed into the per-dim words (BITS = 2, 4: one word holds the 8
// positions; BITS = 8: two).
template <int BITS>
RKV_INLINE __device__ inline void v_accumulate(const uint32_t (&u)[8], int s, uint32_t (&vw)[8][BITS == 8 ? 2 : 1]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (BITS == 8) {
      vw[e][s >> 2] |= (u[e] & 0xFFu) << (8 * (s & 3));
    } else {
      vw[e][0] |= (u[e] & ((1u << BITS) - 1)) << (BITS * s);
    }
  }
}

template <typename T, int BITS, int KM, bool LAT>
__global__ __launch_bounds__(1024) void k_quantize_lds(
    const T* __restrict__ K, const T* __restrict__ V, const uint16_t* __restrict__ idx,
    const T* __restrict__ ref_kv, uint8_t* __restrict__ codes_k, uint8_t* __restrict__ codes_v,
    uint16_t* __restrict__ scales, int64_t N, int64_t n_refs, Sched sc, int k, int group, int H,
    int p0, int n_in, int chunk_tiles, LatMask lm) {
  static_assert(BITS == 2 || BITS == 4 || BITS == 8, "quantised codes only");
  static_assert(sizeof(T) == 2, "bf16 rows: 256 bytes each");
  // the plane's reference rows, 128 elements each (a static array: its LDS
  // address is known when the kernel is compiled, so gathers need no base add)
  __shared__ u32x4 rl[kLdsRefBytes / 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index: tile loop in scalars
  const int rr = lane >> 4;        // 16-lane row of the wave: positions 8 rr + s
  const int dl = lane & 15;        // dims [8 dl, 8 dl + 8)
  // grid (2 * chunks, H, inst); the chunks and planes of one head run on one
  // XCD when the heads split evenly over the 8 XCDs
  int64_t ih = (int64_t)blockIdx.z * H + blockIdx.y;
  int item = (int)blockIdx.x;
  if (((gridDim.y * gridDim.z) & 7u) == 0) {
    const int64_t nc = gridDim.x;
    const int64_t L = blockIdx.x + nc * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t i = L >> 3;
    ih = 8 * (i / nc) + (L & 7);
    item = (int)(i % nc);
  }
  const int plane = item & 1;
  const int p1 = p0 + n_in;
  const int t_first = (p0 >> 5) + (item >> 1) * chunk_tiles;
  const int t_last = (p1 + kVTile - 1) >> 5;
  const int t_end = t_first + chunk_tiles < t_last ? t_first + chunk_tiles : t_last;
  if (t_first >= t_end) return;  // whole block

  // copy the reference rows positions below p1 can select: every thread
  // requests all of its chunks before its first store (one memory round
  // trip instead of one per chunk), through a descriptor bounded by those
  // rows, so chunks past them read zeros (never gathered) and neither loop
  // needs a branch
  {
    const int nr = sched_count(p1, sc);
    constexpr int kPer = kLdsRefBytes / 16 / 1024;
    const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(ref_kv + (ih * 2 + plane) * n_refs * 128), 0,
        nr * (int)(128 * sizeof(T)), 0x00020000);
    u32x4 tmp[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      tmp[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rrs, (tid + 1024 * j) * 16, 0, 0));
#pragma unroll
    for (int j = 0; j < kPer; ++j) rl[tid + 1024 * j] = tmp[j];
  }
  __syncthreads();

  const char* lb = reinterpret_cast<const char*>(rl);
  const Bf16Sel bsel = make_bf16_sel();
  const Bf16Sel nsel = make_bf16_nsel<KM>();
  const uint32_t lane16 = 16u * dl;
  const int n_groups = 128 / group;
  const int lanes_per_group = group >> 3;
  const bool scale_lane = (dl & (lanes_per_group - 1)) == 0;
  const int sgrp = dl / lanes_per_group;
  const T* xin = (plane ? V : K) + ih * n_in * 128 + 8 * dl;  // + (position - p0) * 128
  const uint16_t* ib = idx + ih * N * k;
  // K codes and scales of this head through bounded buffer descriptors over
  // the positions [p0, p1): the hardware drops a store whose offset falls
  // outside, which takes care of positions outside the range (below p0 the
  // 32-bit offset wraps past the end), so no store sits behind a branch (a
  // branch around a store would make the compiler wait for every load in
  // flight before it).  Offset of position pos, lane piece: (pos - p0) times
  // the bytes per position (wave-uniform) plus a lane constant; lanes that
  // write no scale get a lane constant past every range.
  constexpr uint32_t kDrop = 0x80000000u;
  const uint32_t ck_bytes = (uint32_t)n_in * (16u * BITS);
  const __amdgpu_buffer_rsrc_t kb = __builtin_amdgcn_make_buffer_rsrc(
      codes_k + (ih * N + p0) * (16 * BITS), 0, (int)ck_bytes, 0x00020000);
  const uint32_t sc_bytes = (uint32_t)n_in * 4u * n_groups;
  const __amdgpu_buffer_rsrc_t sb = __builtin_amdgcn_make_buffer_rsrc(
      scales + (ih * N + p0) * 2 * n_groups, 0, (int)sc_bytes, 0x00020000);
  const uint32_t k_lane = (uint32_t)(8 * rr) * (16u * BITS) + (uint32_t)dl * BITS;
  const uint32_t s_lane = scale_lane ? (uint32_t)(8 * rr) * (4u * n_groups) +
                                           2u * (uint32_t)(plane * n_groups + sgrp)
                                     : kDrop;
  constexpr float qmax = (float)((1 << (BITS - 1)) - 1);
  constexpr float inv_qmax = 1.0f / qmax;
  constexpr float tol = (qmax + 1.f) * 0x1p-21f;

  // residual of this lane's 8 dims at position tb + 8 rr + s -> scale and
  // codes (u); stores the scale and (K plane) the codes if that position is
  // in [p0, p1)
  auto finish = [&](int tb, int s, float (&z)[8], uint32_t (&u)[8]) RKV_INLINE {
    if constexpr (LAT) {
      lat_signs8(z, lm, dl);
      fwht128_8(z, dl);
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] *= 0.0625f;
    }
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(z[e]));
    a = group_max_nonneg(a, lanes_per_group);
    bool plain;
    const uint16_t sbits = exact_scale_bits_plain(a, qmax, inv_qmax, plain);
    const float sv = half_bits_to_f32(sbits);
    const float rs = sv > 0.f ? __builtin_amdgcn_rcpf(sv) : 0.f;  // within 1 ulp of 1/s
    // a scale that is not plain (rare) has every code decided exactly and clamped
    codes8<false>(z, sv, rs, qmax, tol, u, !plain);
    const uint32_t ru = (uint32_t)(tb + s - p0);  // wave-uniform
    __builtin_amdgcn_raw_buffer_store_b16(sbits, sb, (int)(ru * (4u * n_groups) + s_lane), 0, 0);
    if (plane == 0) buffer_store_word<BITS>(kb, ru * (16u * BITS) + k_lane, pack8<BITS>(u));
  };

  // Row piece and slot word of step s of the tile at tbx, through bounded
  // buffer descriptors over the range's rows and slot rows: a position
  // outside [p0, p1) reads zeros or a row of the range (its results are
  // never stored), so no clamp is needed, and the step's offset is an
  // instruction immediate.
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>((plane ? V : K) + ih * n_in * 128), 0, n_in * 256, 0x00020000);
  const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(ib + (int64_t)p0 * KM), 0, n_in * KM * 2, 0x00020000);
  const uint32_t x_lane = 16u * dl;
  const uint32_t i_lane = 4u * (dl & (KM / 2 - 1));
  auto issue = [&](int tbx, int s, PosLoads<T, KM>& pl) RKV_INLINE {
    const uint32_t r0 = (uint32_t)(tbx + 8 * rr - p0);
    // token rows are read once: non-temporal (nt), which measured about 1 %
    // faster; the slot words stay cached (the other plane's blocks read them)
    pl.x[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            xrs, (int)(r0 * 256u + x_lane + 256u * s), 0, 2));
    pl.sl[0].x = __builtin_amdgcn_raw_buffer_load_b32(
        irs, (int)(r0 * (2u * KM) + i_lane + 2u * KM * s), 0, 0);
  };
  // steps in flight per wave: a whole tile where the registers allow
  constexpr int RD = (KM <= 8 && BITS <= 4 && !LAT && sizeof(T) == 2) ? 8 : 4;
  PosLoads<T, KM> ring[RD];
  bool ring_ok = false;  // the ring holds the current tile's first RD steps
  for (int t = t_first + w; t < t_end; t += kLdsQWaves) {
    const int tb = t * kVTile;
    const int v0 = tb > p0 ? tb : p0;
    const int v1 = tb + kVTile < p1 ? tb + kVTile : p1;
    const bool fast = k == KM && sched_count_le(tb, sc) >= KM;
    uint32_t vw[8][BITS == 8 ? 2 : 1];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int c = 0; c < (BITS == 8 ? 2 : 1); ++c) vw[e][c] = 0u;
    if (fast) {
      // every position has KM candidates: unconditional loads (positions
      // outside the range reread one inside it and store nothing)
      auto step = [&](int s, PosLoads<T, KM>& cur) RKV_INLINE {
        spread_slot_words<T, KM>(cur);
        u32x4 g[KM][sizeof(T) / 2];
#pragma unroll
        for (int j = 0; j < KM; ++j) lds_piece<T>(lb, ref_piece_off<T>(slot_word(cur, j), j & 1, lane16), g[j]);
        // acc = -(fp32 sum of the rows in slot order) / KM: the rows enter
        // scaled by -1/KM (exact), so every partial sum is the unscaled one's
        // exact image; then z = fl(x + acc) = fl(x - sum / KM)
        float acc[8];
        acc_set8(g[0], acc, nsel);
#pragma unroll
        for (int j = 1; j < KM; ++j) acc_add8(g[j], acc, nsel);
        acc_add8(cur.x, acc, bsel);
        uint32_t u[8];
        finish(tb, s, acc, u);
        if (plane == 1) v_accumulate<BITS>(u, s, vw);
      };
      if (!ring_ok) {
#pragma unroll
        for (int s = 0; s < RD; ++s) issue(tb, s, ring[s]);
      }
      // step s + RD is requested as soon as step s is done: later steps of
      // this tile, then the first steps of the wave's next tile if that one
      // is a fast tile too
      const int tn = t + kLdsQWaves;
      const bool next = tn < t_end && k == KM && sched_count_le(tn * kVTile, sc) >= KM;
      const int nb = tn * kVTile;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        step(s, ring[s % RD]);
        if (s + RD < 8) issue(tb, s + RD, ring[s % RD]);
        else if (next) issue(nb, s + RD - 8, ring[s % RD]);
      }
      ring_ok = next;
    } else {
      // first tiles of a sequence (fewer than k candidates) or k < KM
#pragma unroll 1
      for (int s = 0; s < 8; ++s) {
        const int pos = tb + 8 * rr + s;
        const bool mine = pos >= v0 && pos < v1;
        uint32_t u[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        if (mine) {
          u32x4 xr[sizeof(T) / 2];
#pragma unroll
          for (int c = 0; c < (int)(sizeof(T) / 2); ++c)
            xr[c] = *reinterpret_cast<const u32x4*>(xin + (int64_t)(pos - p0) * 128 + (16 / sizeof(T)) * c);
          const int cnt = sched_count_le(pos, sc);
          const int keff = cnt < k ? cnt : k;
          const uint16_t* irow = ib + (int64_t)pos * k;
          float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          for (int j = 0; j < keff; ++j) {
            const uint32_t slot = irow[j];
            u32x4 g[sizeof(T) / 2];
            lds_piece<T>(lb, (slot * 128u + 8u * dl) * (uint32_t)sizeof(T), g);
            acc_add8(g, acc, bsel);
          }
          float x[8], z[8];
          widen(xr, x);
          if (is_pow2(keff)) {
            const float inv = __uint_as_float((uint32_t)(127 - __builtin_ctz(keff)) << 23);
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = x[e] - acc[e] * inv;
          } else {
            const float kf = (float)keff;
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = x[e] - acc[e] / kf;
          }
          finish(tb, s, z, u);
        }
        if (plane == 1) v_accumulate<BITS>(u, s, vw);
      }
      ring_ok = false;
    }
    if (plane == 1) {
      // the words of positions 8 rr .. 8 rr + 7 of the tile, for the lane's 8
      // dims; a tile cut by the range keeps the other positions' bits
      const int g0 = tb + 8 * rr;
      const int lo = v0 - g0 < 0 ? 0 : v0 - g0;
      const int hi = v1 - g0 > 8 ? 8 : v1 - g0;
      uint8_t* dst = codes_v + ((ih * ((N + kVTile - 1) / kVTile) + t) * 128 + 8 * dl) *
                                   (kVTile * BITS / 8) + rr * BITS;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint64_t wv = BITS == 8 ? ((uint64_t)vw[e][BITS == 8 ? 1 : 0] << 32 | vw[e][0])
                                      : (uint64_t)vw[e][0];
        uint8_t* d = dst + e * (kVTile * BITS / 8);
        if (lo == 0 && hi == 8) store_word<BITS>(d, wv);
        else if (lo < hi) store_word_range<BITS>(d, wv, lo, hi);
      }
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

template <typename T, int BITS, int KM, bool RQ, bool LAT>
__global__ __launch_bounds__(512) void k_reconstruct(
    const uint16_t* __restrict__ idx, const T* __restrict__ ref_kv,
    const uint16_t* __restrict__ ref_scales,
    const uint8_t* __restrict__ codes_k, const uint8_t* __restrict__ codes_v,
    const uint16_t* __restrict__ scales, float* __restrict__ Kh, float* __restrict__ Vh,
    int64_t N, int64_t n_refs, Sched sc, int k, int group, int H, LatMask lm) {
  const int tid = threadIdx.x;
  const int plane = (tid >> 4) & 1;
  const int dl = tid & 15;
  const int64_t ih = (int64_t)blockIdx.z * H + blockIdx.y;
  const int64_t tok = (int64_t)blockIdx.x * kQTokens + (tid >> 5);
  if (tok >= N) return;
  RefSrc<T, RQ> refs;
  refs.ng = 128 / group;
  if constexpr (RQ) {
    refs.codes = reinterpret_cast<const uint8_t*>(ref_kv) + (ih * 2 + plane) * n_refs * 64 + 4 * dl;
    refs.sc = ref_scales + (ih * 2 + plane) * n_refs * refs.ng + (8 * dl) / group;
  } else {
    refs.raw = ref_kv + (ih * 2 + plane) * n_refs * 128 + 8 * dl;
  }
  float* dst = (plane ? Vh : Kh) + (ih * N + tok) * 128 + 8 * dl;
  float out[8];
  const int64_t slot = sched_slot((int32_t)tok, sc);
  if (slot >= 0) {
    ref_row8<T, RQ>(refs, (uint32_t)slot, out);
    store8(dst, out);
    return;
  }
  float m[8];
  const int keff = (int)min((int64_t)k, sched_count_le((int32_t)tok, sc));
  ref_mean8_src<T, KM, RQ>(refs, idx + (ih * N + tok) * k, k, keff, m);
  if constexpr (BITS == 0) {
    const double* r = reinterpret_cast<const double*>(plane ? codes_v : codes_k) +
                      (ih * N + tok) * 128 + 8 * dl;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)((double)m[e] + r[e]);
  } else {
    const int n_groups = 128 / group;
    const float s = half_bits_to_f32(
        scales[((ih * N + tok) * 2 + plane) * n_groups + (8 * dl) / group]);
    float y[8];  // dequantised residual (exact: fp16 scale x small integer)
    if (plane == 0) {
      const uint8_t* row = codes_k + (ih * N + tok) * (128 * BITS / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = s * (float)code_at<BITS>(row, 8 * dl + e);
    } else {
      const int64_t tile = tok / kVTile;
      const int u = (int)(tok % kVTile);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint8_t* row = codes_v + ((ih * ((N + kVTile - 1) / kVTile) + tile) * 128 +
                                        8 * dl + e) * (kVTile * BITS / 8);
        y[e] = s * (float)code_at<BITS>(row, u);
      }
    }
    if constexpr (LAT) {
      // f_d(y) = D H y / 8
      fwht128_8(y, dl);
      lat_signs8(y, lm, dl);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= 0.125f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = m[e] + y[e];
  }
  store8(dst, out);
}

// ------------------------------------------------------------ launchers
template <typename T, int BITS>
hipError_t launch_quantize_t(const void* K, const void* V, const uint16_t* idx,
                             const void* ref_kv, const uint16_t* ref_scales, int ref_bits,
                             uint8_t* ck, uint8_t* cv, uint16_t* sc16,
                             int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc,
                             int k, int group, int64_t p0, int64_t n_in, const LatMask* lm,
                             hipStream_t st) {
  const int chunk = 256;
  const int64_t start = p0 & ~(int64_t)(kVTile - 1);
  const int64_t nchunks = (p0 + n_in - start + chunk - 1) / chunk;
  // latent codes exist only with quantisation (BITS > 0)
  auto pick = [&](auto rq, auto lat) {
    constexpr bool R = decltype(rq)::value;
    constexpr bool L = decltype(lat)::value && BITS != 0;
    return k <= 4 ? k_quantize<T, BITS, 4, R, L>
                  : (k <= 8 ? k_quantize<T, BITS, 8, R, L> : k_quantize<T, BITS, 16, R, L>);
  };
  auto pick_r = [&](auto lat) {
    return ref_bits == 4 ? pick(std::true_type{}, lat) : pick(std::false_type{}, lat);
  };
  const LatMask m = lm ? *lm : LatMask{{0u, 0u, 0u, 0u}};
  // Reference rows of one plane that fit in LDS: gathers from LDS, when the
  // range is long enough to repay copying the rows into every block (at
  // least four positions per reference; a streaming append of a few
  // positions gathers through the L1/L2 instead)
  const int64_t nr_range = sched_count((int32_t)(p0 + n_in), sc);
  const size_t ref_lds = (size_t)nr_range * 128 * sizeof(T);
  if constexpr (BITS != 0 && sizeof(T) == 2) {
    if (ref_bits == 0 && ref_lds <= (size_t)kLdsRefBytes && n_in >= 4 * nr_range &&
        n_in < (int64_t{1} << 23)) {  // byte offsets of the range's rows fit 31 bits
      const int64_t ntiles = (p0 + n_in + kVTile - 1) / kVTile - p0 / kVTile;
      const int64_t nch = (ntiles + kLdsChunkTiles - 1) / kLdsChunkTiles;
      auto pick_l = [&](auto lat) {
        constexpr bool L = decltype(lat)::value;
        return k <= 4 ? k_quantize_lds<T, BITS, 4, L>
                      : (k <= 8 ? k_quantize_lds<T, BITS, 8, L> : k_quantize_lds<T, BITS, 16, L>);
      };
      auto kl = lm ? pick_l(std::true_type{}) : pick_l(std::false_type{});
      hipLaunchKernelGGL(kl, dim3((unsigned)(2 * nch), H, (unsigned)n_inst), dim3(1024),
                         0, st, (const T*)K, (const T*)V, idx, (const T*)ref_kv, ck, cv,
                         sc16, N, n_refs, sc, k, group, H, (int)p0, (int)n_in,
                         (int)kLdsChunkTiles, m);
      return hipGetLastError();
    }
  }
  auto kern = lm ? pick_r(std::true_type{}) : pick_r(std::false_type{});
  hipLaunchKernelGGL(kern, dim3((unsigned)nchunks, H, (unsigned)n_inst),
                     dim3(512), 0, st, (const T*)K, (const T*)V, idx, (const T*)ref_kv, ref_scales, ck,
                     cv, sc16, N, n_refs, sc, k, group, chunk, H, (int)p0, (int)n_in, m);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_quantize_d(int bits, const void* K, const void* V, const uint16_t* idx,
                             const void* ref_kv, const uint16_t* ref_scales, int ref_bits,
                             uint8_t* ck, uint8_t* cv, uint16_t* sc16,
                             int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc,
                             int k, int group, int64_t p0, int64_t n_in, const LatMask* lm,
                             hipStream_t st) {
  switch (bits) {
    case 0: return launch_quantize_t<T, 0>(K, V, idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, p0, n_in, lm, st);
    case 2: return launch_quantize_t<T, 2>(K, V, idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, p0, n_in, lm, st);
    case 4: return launch_quantize_t<T, 4>(K, V, idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, p0, n_in, lm, st);
    default: return launch_quantize_t<T, 8>(K, V, idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, p0, n_in, lm, st);
  }
}

hipError_t launch_quantize(int dtype, int bits, const void* K, const void* V,
                           const uint16_t* idx, const void* ref_kv, const uint16_t* ref_scales,
                           int ref_bits, uint8_t* ck, uint8_t* cv,
                           uint16_t* sc16, int64_t n_inst, int H, int64_t N, int64_t n_refs,
                           Sched sc, int k, int group, int64_t p0, int64_t n_in,
                           const LatMask* lm, hipStream_t st) {
  if (n_in == 0 || n_inst == 0) return hipSuccess;
  if (dtype == 0)
    return launch_quantize_d<float>(bits, K, V, idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, p0, n_in, lm, st);
  return launch_quantize_d<__bf16>(bits, K, V, idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, n_inst, H, N, n_refs, sc, k, group, p0, n_in, lm, st);
}

template <typename T, int BITS>
hipError_t launch_recon_t(const uint16_t* idx, const void* ref_kv, const uint16_t* ref_scales,
                          int ref_bits, const uint8_t* ck,
                          const uint8_t* cv, const uint16_t* sc16, float* Kh, float* Vh,
                          int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc, int k,
                          int group, const LatMask* lm, hipStream_t st) {
  const int64_t blocks = (N + kQTokens - 1) / kQTokens;
  auto pick = [&](auto rq, auto lat) {
    constexpr bool R = decltype(rq)::value;
    constexpr bool L = decltype(lat)::value && BITS != 0;
    return k <= 4 ? k_reconstruct<T, BITS, 4, R, L>
                  : (k <= 8 ? k_reconstruct<T, BITS, 8, R, L> : k_reconstruct<T, BITS, 16, R, L>);
  };
  auto pick_r = [&](auto lat) {
    return ref_bits == 4 ? pick(std::true_type{}, lat) : pick(std::false_type{}, lat);
  };
  auto kern = lm ? pick_r(std::true_type{}) : pick_r(std::false_type{});
  const LatMask m = lm ? *lm : LatMask{{0u, 0u, 0u, 0u}};
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks, H, (unsigned)n_inst),
                     dim3(512), 0, st, idx, (const T*)ref_kv, ref_scales, ck, cv, sc16, Kh, Vh, N, n_refs,
                     sc, k, group, H, m);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_recon_d(int bits, const uint16_t* idx, const void* ref_kv,
                          const uint16_t* ref_scales, int ref_bits, const uint8_t* ck,
                          const uint8_t* cv, const uint16_t* sc16, float* Kh, float* Vh,
                          int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc, int k,
                          int group, const LatMask* lm, hipStream_t st) {
  switch (bits) {
    case 0: return launch_recon_t<T, 0>(idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, lm, st);
    case 2: return launch_recon_t<T, 2>(idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, lm, st);
    case 4: return launch_recon_t<T, 4>(idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, lm, st);
    default: return launch_recon_t<T, 8>(idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, lm, st);
  }
}

hipError_t launch_reconstruct(int dtype, int bits, const uint16_t* idx, const void* ref_kv,
                              const uint16_t* ref_scales, int ref_bits, const uint8_t* ck, const uint8_t* cv, const uint16_t* sc16,
                              float* Kh, float* Vh, int64_t n_inst, int H, int64_t N,
                              int64_t n_refs, Sched sc, int k, int group, const LatMask* lm,
                              hipStream_t st) {
  if (N == 0 || n_inst == 0) return hipSuccess;
  if (dtype == 0)
    return launch_recon_d<float>(bits, idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, lm, st);
  return launch_recon_d<__bf16>(bits, idx, ref_kv, ref_scales, ref_bits, ck, cv, sc16, Kh, Vh, n_inst, H, N, n_refs, sc, k, group, lm, st);
}

}  // namespace rkv
