// Decode attention straight from the compressed cache (gfx950).
//
// Paper page "DeltaKV Framework Architecture": a token is rebuilt as
// KV^ = KV^_delta + KV_R; news page "How ResidualKV Works": the rebuild
// happens on the fly when attention needs the token.  Section "Practical
// Deployment via Sparse-vLLM" fuses the reference gather, the mean and the
// residual add into one kernel to save bandwidth.
//
// Rebuilding each K^_i from its k gathered references would cost k reference
// rows of on-chip traffic per token.  Attention is linear in K^ and V^, so
// the mean is folded instead:
//   q . K^_i  = q . (scale*code)_i + mean_{j in S_i} QK[j],  QK[j] = q . Kref_j
//   sum_i p_i V^_i = sum_i p_i (scale*code)_i + sum_j W[j] Vref_j,
//   W[j] = sum_{i : j in S_i} p_i / k_eff
// (a reference position i contributes QK[slot(i)] and W[slot(i)] += p_i).
//
// Kernels:
//   k_qk_table QK for every reference and query head.
//   k_decode   one block of 4 waves per (instance, KV head, split of the
//              sequence), which it walks in chunks of 1024 positions.
//              Phase A: the waves stream the K codes of 32-token tiles,
//              q.codes on 16x16x32 f16 MFMAs (codes are exact small
//              integers in f16, taken with a fixed offset that the
//              accumulators start without), scales in fp32, the reference
//              term from the QK table in LDS; every logit goes to LDS.  The
//              block takes the chunk maximum per query head (rescaling what
//              it holds only if the maximum grew).  Phase B: the waves stream
//              the V codes, p = exp(logit - max) <= 1, P.codes on the MFMA,
//              and the chunk's W in LDS as 21-bit fixed point, two query
//              heads per 64-bit atomic (integer LDS atomics are far faster
//              than float ones here), added to fp32 totals at the chunk end.
//              The block writes (m, l, O, W) per query head.
//   k_combine  one block per (instance, query head): merges the splits,
//              adds W . Vref and normalises, with its loads requested up
//              front.
#include <float.h>

#include <type_traits>

#include "rkv_common.h"

namespace rkv {

// Element order of the f16x8 operand decoded from 8 codes (see decode_codes).
template <int BITS>
__host__ __device__ constexpr int perm_of(int e) {
  return BITS == 8 ? ((e & 4) | ((e & 1) << 1) | ((e >> 1) & 1))   // 0 2 1 3 4 6 5 7
                   : (((e & 1) << 2) | (e >> 1));                  // 0 4 1 5 2 6 3 7
}
template <int BITS>
__host__ __device__ constexpr int invperm_of(int o) {
  return BITS == 8 ? perm_of<8>(o)                                   // an involution
                   : (((o & 3) << 1) | (o >> 2));                    // 0 2 4 6 1 3 5 7
}

__device__ inline f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

// A float that is the same in every lane, moved to a scalar register (the
// bits are passed through: the builtin takes an int).
__device__ inline float uniform_f32(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Unsigned maximum of the two 16-bit halves of a and b (one packed op).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Offset of a code decoded without the final subtract: 1024 + 2^(BITS-1).
template <int BITS>
constexpr float code_bias() { return 1024.f + (float)(1 << (BITS - 1)); }

// 8 two's-complement codes (BITS each) -> f16x8 exact integers, in
// perm_of<BITS> order.  Offset-binary plus the f16 exponent of 1024 puts each
// code in a mantissa; one packed subtract removes the offset.  RAW skips that
// subtract: the values are then code + code_bias<BITS>() (still exact).
template <int BITS, bool RAW = false>
__device__ inline f16x8 decode_codes(uint32_t w0, uint32_t w1) {
  f16x2 p[4];
  if constexpr (BITS == 4) {
    const uint32_t t = w0 ^ 0x88888888u;
    const f16x2 off = {(_Float16)-1032.f, (_Float16)-1032.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = as_h2(((t >> (4 * j)) & 0x000F000Fu) | 0x64006400u);
      if constexpr (!RAW) p[j] = p[j] + off;
    }
  } else if constexpr (BITS == 8) {
    const uint32_t t0 = w0 ^ 0x80808080u, t1 = w1 ^ 0x80808080u;
    const f16x2 off = {(_Float16)-1152.f, (_Float16)-1152.f};
    p[0] = as_h2((t0 & 0x00FF00FFu) | 0x64006400u);
    p[1] = as_h2(((t0 >> 8) & 0x00FF00FFu) | 0x64006400u);
    p[2] = as_h2((t1 & 0x00FF00FFu) | 0x64006400u);
    p[3] = as_h2(((t1 >> 8) & 0x00FF00FFu) | 0x64006400u);
    if constexpr (!RAW) {
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = p[j] + off;
    }
  } else {
    const uint32_t t = (w0 ^ 0xAAAAu) & 0xFFFFu;
    const uint32_t u = (t & 0xFFu) | ((t & 0xFF00u) << 8);
    const f16x2 off = {(_Float16)-1026.f, (_Float16)-1026.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = as_h2(((u >> (2 * j)) & 0x00030003u) | 0x64006400u);
      if constexpr (!RAW) p[j] = p[j] + off;
    }
  }
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = p[j][0];
    r[2 * j + 1] = p[j][1];
  }
  return r;
}

__device__ inline float quad_max(float v) {
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}
__device__ inline float quad_sum(float v) {
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int NW>
__device__ inline void load_words(const void* p, uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (NW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[c];
      w[4 * c] = v.x; w[4 * c + 1] = v.y; w[4 * c + 2] = v.z; w[4 * c + 3] = v.w;
    }
  }
}

// The same with the non-temporal hint, for words a block reads once (the K
// and V codes: one-layer decode 180 -> 162 us at 32K); the slot and scale
// words keep the default policy, because the second phase of a chunk reads
// them again (non-temporal there too measured slower).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int NW>
__device__ inline void load_words_nt(const void* p, uint32_t (&w)[NW]) {
  if constexpr (NW == 1) {
    w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  } else if constexpr (NW == 2) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    w[0] = v[0]; w[1] = v[1];
  } else {
#pragma unroll
    for (int c = 0; c < NW / 4; ++c) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + c);
      w[4 * c] = v[0]; w[4 * c + 1] = v[1]; w[4 * c + 2] = v[2]; w[4 * c + 3] = v[3];
    }
  }
}

// W of one softmax chunk is accumulated in LDS as unsigned fixed point with
// 21 fractional bits, two query heads per 64-bit word (head 2m in the low
// half, 2m+1 in the high half).  Every addend is p or p / k_eff with
// p <= 1, and a chunk holds at most 1024 positions, so a half stays below
// 2^31 and never carries into its neighbour.
constexpr float kWFix = 0x1p21f;
__device__ inline uint32_t to_fixed21(float x) {  // 0 <= x <= 1, rounded to nearest
  return (uint32_t)__builtin_rintf(x * kWFix);
}
__device__ inline unsigned long long pack_pair(uint32_t lo, uint32_t hi) {
  return (unsigned long long)lo | ((unsigned long long)hi << 32);
}

constexpr int kDecTile = 32;

// Workgroups are dealt to the 8 XCDs in turn.  For a grid of nx x (heads)
// workgroups with the heads (instance, KV head) a multiple of 8, the i-th
// workgroup of XCD x takes item i % nx of head 8 (i / nx) + x: the table,
// decode and combine workgroups of one head then all run on one XCD, and the
// QK table and partial records they pass on stay in that XCD's L2.
// `lin` is the workgroup's linear index, `nx` the items per head.
struct XcdItem {
  int64_t head;
  int item;
};
__device__ inline XcdItem xcd_item(int64_t lin, int64_t nx) {
  const int64_t i = lin >> 3;
  return XcdItem{8 * (i / nx) + (lin & 7), (int)(i % nx)};
}

// Partial record per (instance, query head, split): m, l, 2 pad, O[128], W[nrp].
__host__ __device__ inline int64_t part_rec_floats(int64_t n_refs) {
  return 132 + ((n_refs + 3) / 4) * 4;
}

// ------------------------------------------------------------------ QK table
// QK[inst][hq][slot] = q_hq . Kref_slot in fp32.  Four lanes per reference
// (32 dims each, the row piece loaded whole before the products), summed
// across the quad with DPP.  Rows of the table are padded to a multiple of 4
// (nrp) with zeros; rows from n_valid on (references not written yet) are
// zero.
template <typename T>
__global__ __launch_bounds__(256) void k_qk_table(const T* __restrict__ q,
                                                  const T* __restrict__ ref_kv,
                                                  const uint16_t* __restrict__ ref_scales,
                                                  int ref_bits, int group,
                                                  float* __restrict__ qk, int G, int H,
                                                  int64_t n_refs, int64_t n_valid) {
  // q rows as [head][part][33]: the four parts of a quad read different banks
  __shared__ float qs[16 * 4 * 33];
  int kvh = blockIdx.y;
  int64_t inst = blockIdx.z;
  int bx = (int)blockIdx.x;
  if ((((int64_t)gridDim.y * gridDim.z) & 7) == 0) {
    const XcdItem it = xcd_item(blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z),
                                gridDim.x);
    kvh = (int)(it.head % H);
    inst = it.head / H;
    bx = it.item;
  }
  const int Hq = H * G;
  const int64_t nrp = ((n_refs + 3) / 4) * 4;
  const T* qh = q + (inst * Hq + kvh * G) * 128;
  for (int e = threadIdx.x; e < G * 128; e += 256)
    qs[(e >> 5) * 33 + (e & 31)] = (float)qh[e];
  __syncthreads();
  const int part = threadIdx.x & 3;  // dims 32*part .. +31
  const int64_t j = (int64_t)bx * 64 + (threadIdx.x >> 2);
  if (j >= nrp) return;  // whole quads leave together
  float* out = qk + (inst * Hq + kvh * G) * nrp + j;
  const bool live = j < n_valid;
  const int64_t jr = live ? j : 0;  // rows past n_valid compute on row 0 and store 0
  float x[32];
  if (ref_bits == 4) {
    // quantised reference: nibbles times the fp16 scale of their group (exact)
    const int ng = 128 / group;
    const int64_t r = ((inst * H + kvh) * 2 + 0) * n_refs + jr;
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(ref_kv) +
                                                    r * 64 + 16 * part);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    const uint16_t* sr = ref_scales + r * ng;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 8 * u + e;
        const float s = half_bits_to_f32(sr[(32 * part + t) / group]);
        x[t] = (float)((int32_t)(w4[u] << (28 - 4 * e)) >> 28) * s;
      }
    }
  } else {
    const T* row = ref_kv + ((inst * H + kvh) * 2 + 0) * n_refs * 128 + jr * 128 + 32 * part;
#pragma unroll
    for (int t = 0; t < 32; t += 8) {
      float v[8];
      load8(row + t, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[t + e] = v[e];
    }
  }
  for (int h = 0; h < G; ++h) {
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 32; ++t) acc = __builtin_fmaf(qs[(4 * h + part) * 33 + t], x[t], acc);
    acc += RKV_DPP_F32(acc, 0xB1);  // quad_perm [1,0,3,2]
    acc += RKV_DPP_F32(acc, 0x4E);  // quad_perm [2,3,0,1]
    if (part == 0) out[h * nrp] = live ? acc : 0.f;
  }
}

constexpr int kChunkTiles = 32;   // tiles (x32 tokens) per softmax chunk of a block
constexpr int kLgPad = 16;

// Slot (or -1) and k_eff of position `tok` in the tile starting at `tb`.
// The tile's references are the slots [cb, ce) (wave-uniform: every lane of
// the wave works on the same tile), so a lane only compares its position
// against those few reference positions.
struct TileRefs {
  int32_t cb, ce;
};
__device__ inline TileRefs tile_refs(int32_t tb, int32_t N, const Sched& sc) {
  const int32_t te = tb + kDecTile < N ? tb + kDecTile : N;
  return TileRefs{sched_count(tb, sc), sched_count(te, sc)};
}
__device__ inline void pos_info(int32_t tok, const TileRefs& tr, const Sched& sc, int k,
                                int32_t& slot, int& keff) {
  int32_t cnt = tr.cb;
  slot = -1;
  for (int32_t r = tr.cb; r < tr.ce; ++r) {
    const int32_t p = sched_pos(r, sc);
    if (p <= tok) ++cnt;
    if (p == tok) slot = r;
  }
  keff = cnt < k ? cnt : k;
}

// Slot of position `tok` if it is one of the tile's references, else -1 (the
// k_eff of a fast tile is KM for every position).
__device__ inline int32_t ref_slot_in_tile(int32_t tok, const TileRefs& tr, const Sched& sc) {
  int32_t slot = -1;
  for (int32_t r = tr.cb; r < tr.ce; ++r)
    if (sched_pos(r, sc) == tok) slot = r;
  return slot;
}

// Blocks per CU the register allocation aims at.  The bf16 int4 forms with
// 32-dim groups and exactly KM slots per row fit three (168 VGPRs; the few
// values live across the whole position loop are spilled once before it and
// reloaded once after); the other forms keep two so that nothing spills
// inside the loop.
template <typename T, int BITS, int NG, int KM, bool EX>
constexpr int kDecodeBlocksPerCU() {
  return (sizeof(T) == 2 && BITS == 4 && NG == 4 && KM <= 8 && EX) ? 3 : 2;
}

// EX: every row of ref_idx holds exactly KM slots (k == KM).
template <typename T, int BITS, int NG, int KM, bool EX>
__global__ __launch_bounds__(256, (kDecodeBlocksPerCU<T, BITS, NG, KM, EX>())) void k_decode(
    const T* __restrict__ q, const T* __restrict__ ref_kv, const uint16_t* __restrict__ idx,
    const uint8_t* __restrict__ codes_k, const uint8_t* __restrict__ codes_v,
    const uint16_t* __restrict__ scales, const float* __restrict__ qk, float* __restrict__ part,
    float alpha, int64_t N, int64_t Nlen, int64_t n_refs, Sched sc, int k, int G, int H,
    int n_split, const int32_t* __restrict__ tile_list, int32_t n_list,
    const float* __restrict__ qrot) {
  // N: positions the cache holds (layout); Nlen <= N: positions attended
  constexpr int HPL = 4 / NG;  // query heads per lane in the score layout
  constexpr int VW = (NG + 1) / 2;  // scale words holding the V scales
  constexpr int GS = 128 / NG;  // dims per scale group
  constexpr int CT = kChunkTiles * kDecTile;  // tokens per chunk
  // logit rows padded by 16 floats: the 4 heads of one position (lane quads)
  // then fall in different banks
  constexpr int CTP = CT + kLgPad;
  extern __shared__ float lds[];
  const int64_t nrp = ((n_refs + 3) / 4) * 4;
  // Per-head LDS rows are nrp + 8 floats apart: the G heads of one token touch
  // the same slot, and this puts their words in different banks.
  const int64_t ls = nrp + 8;
  const int GP = (G + 1) / 2;                                     // head pairs
  float* qk_s = lds;                                              // [G][ls]
  unsigned long long* wc_s =
      reinterpret_cast<unsigned long long*>(qk_s + G * ls);       // [GP][ls] chunk W, fixed point
  float* wt_s = reinterpret_cast<float*>(wc_s + GP * ls);         // [G][ls] W of earlier chunks
  float* lg_s = wt_s + G * ls;                                    // [G][CT] logits of a chunk
  float* m_s = lg_s + G * CTP;                                    // [16] block max per head
  float* wm_s = m_s + 16;                                         // [4][16] wave maxima
  float* sc_s = wm_s + 64;                                        // [16] rescale factors
  // P.V operand scaling: the fp16 operand is p * scale_V * 2^-E, with 2^E
  // (vp_s[0]) above every V scale seen so far in this split, so the product
  // stays below 1 whatever the magnitude of V; the accumulators hold
  // P.V / 2^E.  vp_s[1]: the factor the accumulators take when E grows;
  // vp_s[2]: 2^-E (0 while every V scale is 0); vw_s[4]: the waves' chunk
  // maxima of the V scale bits.
  float* vp_s = sc_s + 16;                                        // [4]
  uint32_t* vw_s = reinterpret_cast<uint32_t*>(vp_s + 4);         // [4]
  _Float16* pst_all = reinterpret_cast<_Float16*>(vw_s + 4);      // [4][16][32]
  _Float16* sst_all = pst_all + 4 * 16 * kDecTile;                // [4][NG][32]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 15;
  const int quad = lane >> 4;
  int split = blockIdx.x;
  int kvh = blockIdx.y;
  int64_t inst = blockIdx.z;
  if ((((int64_t)gridDim.y * gridDim.z) & 7) == 0) {
    const XcdItem it = xcd_item(blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z),
                                gridDim.x);
    kvh = (int)(it.head % H);
    inst = it.head / H;
    split = it.item;
  }
  const int64_t ih = inst * H + kvh;
  const int Hq = H * G;
  const int32_t tiles = (int32_t)((N + kDecTile - 1) / kDecTile);       // layout
  const int32_t tiles_len = (int32_t)((Nlen + kDecTile - 1) / kDecTile);
  // The splits walk entries [0, n_ent) of the tile list (all tiles below
  // Nlen when there is no list); entry e names tile tile_of(e).
  const int32_t* tl = tile_list ? tile_list + ih * n_list : nullptr;
  const int32_t n_ent = tl ? n_list : tiles_len;
  // an entry outside [0, tiles_len) reads as the empty tile `tiles_len` (all
  // of its positions are >= Nlen: masked, nothing loaded)
  auto tile_of = [&](int32_t e) -> int32_t {
    if (!tl) return e;
    const int32_t x = tl[e];
    return (x >= 0 && x < tiles_len) ? x : tiles_len;
  };
  const int32_t tps = (n_ent + n_split - 1) / n_split;
  const int32_t t0 = split * tps;
  const int32_t t1 = (t0 + tps < n_ent) ? t0 + tps : n_ent;
  const int32_t N32 = (int32_t)Nlen;  // masking bound
  const T* qh = q + (inst * Hq + kvh * G) * 128;

  // ---- prologue: QK table into LDS, clears
  {
    const float4* src = reinterpret_cast<const float4*>(qk + (inst * Hq + kvh * G) * nrp);
    const int nq = (int)(nrp / 4);
    for (int h = 0; h < G; ++h)
      for (int c = tid; c < nq; c += 256)
        *reinterpret_cast<float4*>(qk_s + h * ls + 4 * c) = src[h * nq + c];
    for (int64_t e = tid; e < GP * ls; e += 256) wc_s[e] = 0ull;
    for (int64_t e = tid; e < G * ls; e += 256) wt_s[e] = 0.f;
    for (int e = tid; e < 4 * 16 * kDecTile; e += 256) pst_all[e] = (_Float16)0.f;
    if (tid < 16) m_s[tid] = -INFINITY;
    if (tid < 4) vp_s[tid] = 0.f;
  }

  // ---- A operand of the score MFMA: rows (h, g); lane quad covers dims
  //      32*quad .. +31, step s dims 32*quad + 8*s + perm(e).  Latent codes
  //      are scored against the rotated query qrot = H D q / 8 instead
  //      (q . f_d(y) = (H D q / 8) . y).
  f16x8 aq[4];
  // The query enters the f16 MFMA scaled by a power of two, 2^s, that puts
  // the largest |q| of the KV head's query heads in [2^8, 2^9): no fp16
  // overflow or underflow for any magnitude of q.  qinv = 2^-s (the same in
  // every lane) undoes it on the logit.
  float qinv;
  {
    // the lane's 32 query values are 4 runs of 8 dims (32*quad + 8*s): load
    // them whole (one branch for the source), then permute and mask to the
    // lane's scale group
    const int h = n / NG, g = n % NG;
    const bool live = h < G;
    const int hr = live ? h : 0;
    float qv[4][8];
    if (qrot) {
      const float* qr = qrot + ((inst * Hq + kvh * G) + hr) * 128 + 32 * quad;
#pragma unroll
      for (int s = 0; s < 4; ++s) load8(qr + 8 * s, qv[s]);
    } else {
      const T* qq = qh + hr * 128 + 32 * quad;
#pragma unroll
      for (int s = 0; s < 4; ++s) load8(qq + 8 * s, qv[s]);
    }
    float qm = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qm = fmaxf(qm, fabsf(qv[s][e]));
    if (!live) qm = 0.f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) qm = fmaxf(qm, __shfl_xor(qm, off));
    qm = uniform_f32(qm);  // largest |q| of the G heads (all 128 dims)
    int qe = 0;
    (void)frexpf(qm, &qe);                   // qm in [2^(qe-1), 2^qe), or qe = 0 for 0
    const float qs = (qm > 0.f && qm <= FLT_MAX) ? ldexpf(1.f, 9 - qe) : 1.f;
    qinv = uniform_f32(1.f / qs);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dim = 32 * quad + 8 * s + perm_of<BITS>(e);
        aq[s][e] = (_Float16)((live && dim / GS == g) ? qv[s][perm_of<BITS>(e)] * qs : 0.f);
      }
    }
  }
  // The score MFMA takes codes without their offset (decode_codes RAW: code +
  // code_bias), so each accumulator row starts at -code_bias * (sum of that
  // A row).  Lane (n, quad) accumulates rows 4*quad + i of column n.
  f32x4 qbias;
  {
    float rsum = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) rsum += (float)aq[s][e];
    rsum += __shfl_xor(rsum, 16);
    rsum += __shfl_xor(rsum, 32);  // row n's sum over all 128 dims
#pragma unroll
    for (int i = 0; i < 4; ++i) qbias[i] = -code_bias<BITS>() * __shfl(rsum, 4 * quad + i);
  }
  __syncthreads();

  _Float16* pst = pst_all + w * 16 * kDecTile;
  _Float16* sst = sst_all + w * NG * kDecTile;
  // per-row bases: K codes of row t at ck0 + t * 16*BITS (this lane's 32
  // dims), scales at sc0 + t * 2*NG
  const uint8_t* ck0 = codes_k + ih * N * (16 * BITS) + quad * (4 * BITS);
  const uint16_t* sc0 = scales + ih * N * 2 * NG;
  const uint16_t* ix = idx + ih * N * k;
  const uint8_t* cv = codes_v + ih * tiles * 128 * (4 * BITS) + n * (4 * BITS) + quad * BITS;
  const int h0 = quad * HPL;

  float l_mine[HPL];
#pragma unroll
  for (int hh = 0; hh < HPL; ++hh) l_mine[hh] = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float vinv = 0.f;  // 2^-E of the current chunk (the same in every lane)

  auto load_slots_of = [&](int32_t tok, uint32_t (&iw)[KM / 2]) RKV_INLINE {
    if constexpr (EX) {
      load_words<KM / 2>(ix + (uint32_t)tok * KM, iw);
    } else {
      const uint16_t* row = ix + (uint32_t)tok * (uint32_t)k;
#pragma unroll
      for (int j = 0; j < KM / 2; ++j) {
        const uint32_t lo = 2 * j < k ? row[2 * j] : 0;
        const uint32_t hi = 2 * j + 1 < k ? row[2 * j + 1] : 0;
        iw[j] = lo | (hi << 16);
      }
    }
  };

  struct ARegs {
    uint32_t kw[2][BITS];     // K codes, dims 32*quad .. +31 of tokens 16b+n
    uint32_t sw[2][NG];       // K then V scales of those tokens
    uint32_t iw[2][KM / 2];   // their reference slots
  };
  struct BRegs {
    uint32_t vw[8][BITS == 8 ? 2 : 1];  // V codes: dim 16*blk+n, tokens 8*quad .. +7
    uint32_t sw[2][NG];
    uint32_t iw[2][KM / 2];
  };
  // Loads are unconditional: a position at or past the attended length reads
  // the last attended row instead (its logit is -inf and its p is 0, so the
  // values never count).  With no branch around them the load counter waits
  // only for the tile being used, and the next tile's loads stay in flight.
  auto loadA = [&](int32_t t, ARegs& r) RKV_INLINE {
    const int32_t tb = tile_of(t) * kDecTile;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int32_t row = min(tb + 16 * b + n, N32 - 1);
      load_words_nt<BITS>(ck0 + (uint32_t)row * (16 * BITS), r.kw[b]);
      load_words<NG>(sc0 + (uint32_t)row * (2 * NG), r.sw[b]);
      load_slots_of(row, r.iw[b]);
    }
  };
  // Phase A of one tile.  FT (a fast tile: every position has k = KM
  // references) is chosen per tile, wave-uniformly, so each variant is
  // straight-line code.
  auto computeA_t = [&](auto ft_c, int32_t tb, int32_t t, int32_t c0, const TileRefs& tr,
                        const ARegs& r, float (&wmax)[HPL], uint32_t& vmx) RKV_INLINE {
    constexpr bool FT = decltype(ft_c)::value;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int32_t tok = tb + 16 * b + n;
      const bool valid = tok < N32;
      // largest V scale of the chunk, on the packed scale words (fp16 bits
      // of non-negative values order like the values; with one group the
      // low half is the K scale and is ignored); rows past the length
      // reread a row inside it
#pragma unroll
      for (int m = 0; m < VW; ++m) vmx = pk_max_u16(vmx, r.sw[b][(NG >> 1) + m]);
      f32x4 acc = qbias;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t w0, w1;
        if constexpr (BITS == 4) {
          w0 = r.kw[b][s]; w1 = 0;
        } else if constexpr (BITS == 8) {
          w0 = r.kw[b][2 * s]; w1 = r.kw[b][2 * s + 1];
        } else {
          w0 = (r.kw[b][s >> 1] >> (16 * (s & 1))) & 0xFFFFu; w1 = 0;
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[s], decode_codes<BITS, true>(w0, w1), acc, 0, 0, 0);
      }
      int32_t slot;
      int keff;
      if constexpr (FT) {
        slot = ref_slot_in_tile(tok, tr, sc);
        keff = KM;
      } else {
        pos_info(tok, tr, sc, k, slot, keff);
        if (!valid) { slot = -1; keff = 0; }
      }
      const float inv_keff = keff > 0 ? 1.0f / (float)keff : 0.f;
      const int u = (t - c0) * kDecTile + 16 * b + n;
#pragma unroll
      for (int hh = 0; hh < HPL; ++hh) {
        const int h = h0 + hh;
        if (FT && h < G) {
          // every position of the tile has k = KM references: no predicates
          // (positions past N read slot 0 and are masked to -inf)
          const float* qrow = qk_s + h * ls;
          // all KM lookups (and the reference position's own entry) first,
          // then a pairwise sum: one LDS wait per token.  The scheduling
          // barrier keeps the reads together when registers are tight.
          float qv[KM];
#pragma unroll
          for (int j = 0; j < KM; ++j) qv[j] = qrow[(r.iw[b][j >> 1] >> (16 * (j & 1))) & 0xFFFFu];
          const float sref = qrow[slot >= 0 ? slot : 0];
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int w2 = 1; w2 < KM; w2 *= 2)
#pragma unroll
            for (int j = 0; j + w2 < KM; j += 2 * w2) qv[j] += qv[j + w2];
          const float rs = qv[0];
          float res = 0.f;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const float sk = half_bits_to_f32((uint16_t)(r.sw[b][g >> 1] >> (16 * (g & 1))));
            res = __builtin_fmaf(sk, acc[hh * NG + g], res);
          }
          const float sc_ = slot >= 0 ? sref : __builtin_fmaf(res, qinv, rs * (1.0f / KM));
          const float lg = valid ? alpha * sc_ : -INFINITY;
          lg_s[h * CTP + u] = lg;
          wmax[hh] = fmaxf(wmax[hh], lg);
        } else if (!FT && h < G) {
          float lg = -INFINITY;
          if (valid) {
            const float* qrow = qk_s + h * ls;
            float sc_;
            if (slot >= 0) {
              sc_ = qrow[slot];
            } else {
              float rs = 0.f;
#pragma unroll
              for (int j = 0; j < KM; ++j)
                if (j < keff) rs += qrow[(r.iw[b][j >> 1] >> (16 * (j & 1))) & 0xFFFFu];
              float res = 0.f;
#pragma unroll
              for (int g = 0; g < NG; ++g) {
                const float sk = half_bits_to_f32((uint16_t)(r.sw[b][g >> 1] >> (16 * (g & 1))));
                res = __builtin_fmaf(sk, acc[hh * NG + g], res);
              }
              sc_ = __builtin_fmaf(res, qinv, rs * inv_keff);
            }
            lg = alpha * sc_;
          }
          lg_s[h * CTP + u] = lg;
          wmax[hh] = fmaxf(wmax[hh], lg);
        }
      }
    }
  };
  auto computeA = [&](int32_t t, int32_t c0, const ARegs& r, float (&wmax)[HPL],
                      uint32_t& vmx) RKV_INLINE {
    const int32_t tb = tile_of(t) * kDecTile;
    const TileRefs tr = tile_refs(tb, N32, sc);
    if (EX && tr.cb >= KM)
      computeA_t(std::true_type{}, tb, t, c0, tr, r, wmax, vmx);
    else
      computeA_t(std::false_type{}, tb, t, c0, tr, r, wmax, vmx);
  };
  auto loadB = [&](int32_t t, BRegs& r) RKV_INLINE {
    const int32_t tb = tile_of(t) * kDecTile;
    // a tile past the attended length reads tile 0 (all its p are 0)
    const uint8_t* cvt = cv + (uint32_t)(tb < N32 ? tile_of(t) : 0) * (128 * 4 * BITS);
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const uint8_t* pp = cvt + 16 * blk * (4 * BITS);
      if constexpr (BITS == 8) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pp));
        r.vw[blk][0] = v[0];
        r.vw[blk][1] = v[1];
      } else if constexpr (BITS == 4) {
        r.vw[blk][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(pp));
      } else {
        r.vw[blk][0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(pp));
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int32_t row = min(tb + 16 * b + n, N32 - 1);
      load_slots_of(row, r.iw[b]);
      load_words<NG>(sc0 + (uint32_t)row * (2 * NG), r.sw[b]);
    }
  };
  auto computeB_t = [&](auto ft_c, int32_t tb, int32_t t, int32_t c0, const TileRefs& tr,
                        const BRegs& r, const float (&mh)[HPL]) RKV_INLINE {
    constexpr bool FT = decltype(ft_c)::value;
    float psum[HPL];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) psum[hh] = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int32_t tok = tb + 16 * b + n;
      const bool valid = tok < N32;
      int32_t slot;
      int keff;
      if constexpr (FT) {
        slot = ref_slot_in_tile(tok, tr, sc);
        keff = KM;
      } else {
        pos_info(tok, tr, sc, k, slot, keff);
        if (!valid) { slot = -1; keff = 0; }
      }
      const int u = 16 * b + n;
      const int pos = 8 * (u >> 3) + invperm_of<BITS>(u & 7);
      const int uc = (t - c0) * kDecTile + u;
      uint32_t fx[HPL];  // fast tiles: this position's W addend per head
#pragma unroll
      for (int hh = 0; hh < HPL; ++hh) {
        const int h = h0 + hh;
        if (FT) {
          float pv = 0.f;
          if (h < G) {
            const float lg = lg_s[h * CTP + uc];
            pv = valid ? __expf(lg - mh[hh]) : 0.f;
            psum[hh] += pv;
            pst[h * kDecTile + pos] = (_Float16)(slot >= 0 ? 0.f : pv);
          }
          // a reference position adds p to its own slot; any other position
          // adds p / KM to each of its KM slots
          fx[hh] = to_fixed21(slot >= 0 ? pv : pv * (1.0f / KM));
        } else if (h < G) {
          const float lg = lg_s[h * CTP + uc];
          const float pv = (valid && lg > -INFINITY) ? __expf(lg - mh[hh]) : 0.f;
          psum[hh] += pv;
          unsigned long long* wrow = wc_s + (h >> 1) * ls;
          const int sh = 32 * (h & 1);  // this head's half of the pair word
          if (slot >= 0) {
            if (pv > 0.f) atomicAdd(wrow + slot, (unsigned long long)to_fixed21(pv) << sh);
            pst[h * kDecTile + pos] = (_Float16)0.f;
          } else {
            if (keff > 0 && pv > 0.f) {
              const unsigned long long pw = (unsigned long long)to_fixed21(pv / (float)keff) << sh;
#pragma unroll
              for (int j = 0; j < KM; ++j)
                if (j < keff) atomicAdd(wrow + ((r.iw[b][j >> 1] >> (16 * (j & 1))) & 0xFFFFu), pw);
            }
            pst[h * kDecTile + pos] = (_Float16)pv;
          }
        }
      }
      if constexpr (FT) {
        const bool isref = slot >= 0;
        if constexpr (HPL == 1) {
          // lane quads 2m and 2m+1 hold heads 2m and 2m+1 of one position:
          // after the swap both hold the pair word, and each adds it to half
          // of the position's slots
          const auto pr = __builtin_amdgcn_permlane16_swap(fx[0], fx[0], false, false);
          const unsigned long long v = pack_pair(pr[0], pr[1]);
          const int pp = quad >> 1;
          const bool odd = (quad & 1) != 0;
          if (2 * pp < G) {
            unsigned long long* wrow = wc_s + pp * ls;
            if (isref) {
              if (!odd) atomicAdd(wrow + slot, v);
            } else {
#pragma unroll
              for (int j = 0; j < KM / 2; ++j) {
                const uint32_t wd = odd ? r.iw[b][KM / 4 + (j >> 1)] : r.iw[b][j >> 1];
                atomicAdd(wrow + ((wd >> (16 * (j & 1))) & 0xFFFFu), v);
              }
            }
          }
        } else {
          // the lane holds both heads of each of its pairs
#pragma unroll
          for (int pp = 0; pp < HPL / 2; ++pp) {
            if (h0 + 2 * pp < G) {
              const unsigned long long v = pack_pair(fx[2 * pp], fx[2 * pp + 1]);
              unsigned long long* wrow = wc_s + ((h0 >> 1) + pp) * ls;
              if (isref) {
                atomicAdd(wrow + slot, v);
              } else {
#pragma unroll
                for (int j = 0; j < KM; ++j)
                  atomicAdd(wrow + ((r.iw[b][j >> 1] >> (16 * (j & 1))) & 0xFFFFu), v);
              }
            }
          }
        }
      }
      if (quad == 0) {
        // scale_V * 2^-E_g: below 2, so p * scale_V * 2^-E_g stays in range
#pragma unroll
        for (int g = 0; g < NG; ++g)
          sst[g * kDecTile + pos] = (_Float16)(
              half_bits_to_f32((uint16_t)(r.sw[b][(NG + g) >> 1] >> (16 * ((NG + g) & 1)))) *
              vinv);
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh)
      if (h0 + hh < G) l_mine[hh] += quad_sum(psum[hh]);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS writes landed
    __builtin_amdgcn_wave_barrier();
    f16x8 ap[NG];
    {
      const uint4 pr = *reinterpret_cast<const uint4*>(pst + n * kDecTile + 8 * quad);
      const uint32_t pw4[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const uint4 sr = *reinterpret_cast<const uint4*>(sst + g * kDecTile + 8 * quad);
        const uint32_t sw4[4] = {sr.x, sr.y, sr.z, sr.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x2 prod = as_h2(pw4[j]) * as_h2(sw4[j]);
          ap[g][2 * j] = prod[0];
          ap[g][2 * j + 1] = prod[1];
        }
      }
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const uint32_t w0 = r.vw[blk][0];
      const uint32_t w1 = BITS == 8 ? r.vw[blk][BITS == 8 ? 1 : 0] : 0;
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[(16 * blk) / GS],
                                                   decode_codes<BITS>(w0, w1), o[blk], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
  };
  auto computeB = [&](int32_t t, int32_t c0, const BRegs& r, const float (&mh)[HPL]) RKV_INLINE {
    const int32_t tb = tile_of(t) * kDecTile;
    const TileRefs tr = tile_refs(tb, N32, sc);
    if (EX && tr.cb >= KM)
      computeB_t(std::true_type{}, tb, t, c0, tr, r, mh);
    else
      computeB_t(std::false_type{}, tb, t, c0, tr, r, mh);
  };

  for (int32_t c0 = t0; c0 < t1; c0 += kChunkTiles) {
    const int32_t c1 = (c0 + kChunkTiles < t1) ? c0 + kChunkTiles : t1;
    // ================= phase A: logits of the chunk into LDS (next tile prefetched)
    float wmax[HPL];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) wmax[hh] = -INFINITY;
    uint32_t vmx = 0u;
    {
      // two register sets alternate (unrolled by 2): no copies of loads in flight
      // entries past the chunk load its last entry (never computed)
      ARegs ra, rb;
      int32_t t = c0 + w;
      loadA(min(t, c1 - 1), ra);
      while (t < c1) {
        loadA(min(t + 4, c1 - 1), rb);
        computeA(t, c0, ra, wmax, vmx);
        t += 4;
        if (t >= c1) break;
        loadA(min(t + 4, c1 - 1), ra);
        computeA(t, c0, rb, wmax, vmx);
        t += 4;
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
      const float m = quad_max(wmax[hh]);
      if (n == 0 && h0 + hh < G) wm_s[w * 16 + h0 + hh] = m;
    }
    {
      uint32_t v = vmx;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) v = pk_max_u16(v, (uint32_t)__shfl_xor((int)v, off));
      if (lane == 0) vw_s[w] = v;
    }
    __syncthreads();
    if (tid == 32) {
      // E: the smallest power of two above every V scale so far (never
      // shrinks, so the accumulators are only ever scaled down)
      uint32_t mw = pk_max_u16(pk_max_u16(vw_s[0], vw_s[1]), pk_max_u16(vw_s[2], vw_s[3]));
      if (NG == 1) mw >>= 16;  // the V scale is the high half
      const float mv = half_bits_to_f32((uint16_t)max(mw & 0xFFFFu, mw >> 16));
      const float po = vp_s[0];
      float pn = po;
      if (mv > 0.f) {
        int e = 0;
        (void)frexpf(mv, &e);  // mv < 2^e
        pn = fmaxf(po, ldexpf(1.f, e));
      }
      vp_s[1] = po > 0.f ? po / pn : 1.f;  // exact: powers of two
      vp_s[0] = pn;
      vp_s[2] = pn > 0.f ? 1.f / pn : 0.f;
    }
    if (tid < 16) {
      float f = 1.f;
      if (tid < G) {
        const float mo = m_s[tid];
        const float mn = fmaxf(mo, fmaxf(fmaxf(wm_s[tid], wm_s[16 + tid]),
                                         fmaxf(wm_s[32 + tid], wm_s[48 + tid])));
        f = (mn > mo) ? (mo > -INFINITY ? __expf(mo - mn) : 0.f) : 1.f;
        m_s[tid] = mn;
      }
      sc_s[tid] = f;
    }
    __syncthreads();
    {
      // rescale what was accumulated against the old maximum
      bool any = false;
      for (int h = 0; h < G; ++h) any |= sc_s[h] != 1.f;
      any |= vp_s[1] != 1.f;
      if (any) {
        for (int h = 0; h < G; ++h) {
          const float f = sc_s[h];
          if (f != 1.f)
            for (int j = tid; j < (int)nrp; j += 256) wt_s[h * ls + j] *= f;
        }
#pragma unroll
        for (int hh = 0; hh < HPL; ++hh)
          if (h0 + hh < G) l_mine[hh] *= sc_s[h0 + hh];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float f = (4 * quad + j < G) ? sc_s[4 * quad + j] : 1.f;
#pragma unroll
          for (int b = 0; b < 8; ++b) o[b][j] *= f * vp_s[1];
        }
      }
    }
    __syncthreads();
    // ================= phase B: p, W, P.V
    float mh[HPL];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) mh[hh] = (h0 + hh < G) ? m_s[h0 + hh] : 0.f;
    vinv = uniform_f32(vp_s[2]);

    {
      BRegs ra, rb;
      int32_t t = c0 + w;
      loadB(min(t, c1 - 1), ra);
      while (t < c1) {
        loadB(min(t + 4, c1 - 1), rb);
        computeB(t, c0, ra, mh);
        t += 4;
        if (t >= c1) break;
        loadB(min(t + 4, c1 - 1), ra);
        computeB(t, c0, rb, mh);
        t += 4;
      }
    }
    __syncthreads();
    // add the chunk's fixed-point W to the fp32 totals and clear it (each
    // thread owns whole pair words; the next use of either buffer is behind
    // the next chunk's barriers)
    for (int pp = 0; pp < GP; ++pp) {
      for (int j = tid; j < (int)nrp; j += 256) {
        const unsigned long long v = wc_s[pp * ls + j];
        wt_s[2 * pp * ls + j] += (float)(uint32_t)v * (1.0f / kWFix);
        if (2 * pp + 1 < G) wt_s[(2 * pp + 1) * ls + j] += (float)(uint32_t)(v >> 32) * (1.0f / kWFix);
        wc_s[pp * ls + j] = 0ull;
      }
    }
  }

  // ---- merge the four waves (same maximum), write the partial records.
  // Each wave stores its P.V rows in the logit buffer (free after the last
  // chunk's barrier); the four are then summed in a fixed order.
  float* lw = wm_s;  // reuse [4][16]
#pragma unroll
  for (int hh = 0; hh < HPL; ++hh)
    if (h0 + hh < G && n == 0) lw[w * 16 + h0 + hh] = l_mine[hh];
  float* ow = lg_s;  // [4][G][128]
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * quad + j;
    if (h < G) {
#pragma unroll
      for (int blk = 0; blk < 8; ++blk) ow[(w * G + h) * 128 + 16 * blk + n] = o[blk][j];
    }
  }
  __syncthreads();
  const int64_t rec = part_rec_floats(n_refs);
  float* pr0 = part + ((inst * Hq + kvh * G) * n_split + split) * rec;  // head 0's record
  const int64_t hstride = (int64_t)n_split * rec;                         // next head's
  for (int h = 0; h < G; ++h)
    for (int j = tid; j < (int)nrp; j += 256) pr0[h * hstride + 132 + j] = wt_s[h * ls + j];
  if (tid < G) {
    pr0[tid * hstride] = m_s[tid];
    pr0[tid * hstride + 1] = lw[tid] + lw[16 + tid] + lw[32 + tid] + lw[48 + tid];
  }
  for (int e = tid; e < G * 128; e += 256) {
    const int h = e >> 7, d = e & 127;
    pr0[h * hstride + 4 + d] = (((ow[h * 128 + d] + ow[(G + h) * 128 + d]) + ow[(2 * G + h) * 128 + d]) +
                                ow[(3 * G + h) * 128 + d]) * vp_s[0];
  }
}

// ------------------------------------------------------------------ combine
// One block of CT threads per (instance, query head): merge the head's
// splits (maximum, softmax sum, P.V partials and the reference weights W),
// then add W . Vref over the n_valid written references and normalise.
// Every global load is requested up front (the first comb_rows reference
// rows of each thread, the first kCombSplits partial records of W and of
// P.V), so the merge costs about two memory round trips.  Thread (dg, rg)
// takes dims 8*dg .. 8*dg+7 of references rg, rg + CT/16, ...; the CT/16
// stride groups are summed in LDS.
// CT threads per block: 1024 when the launch has few blocks (one layer),
// 256 when it has many (several blocks per CU then hide the latency).
template <typename T>
constexpr int comb_rows() { return sizeof(T) == 2 ? 8 : 4; }  // reference rows per thread requested up front
constexpr int kCombSplits = 8;              // partial records requested up front

// Dims d0 .. d0+7 of V reference row j, loaded as raw bits (bf16: one
// 16-byte word; fp32: two; int4 rows: the nibble word and the group scale)
// and widened to fp32 at use (exact).
template <typename T>
struct VRow {
  u32x4 v[sizeof(T) / 2];
};

template <typename T>
__device__ inline void vrow_load(const T* __restrict__ raw, const uint8_t* __restrict__ q4,
                                 const uint16_t* __restrict__ rsc, int ng, int group, int ref_bits,
                                 int64_t j, int d0, VRow<T>& r) {
  if (ref_bits == 4) {
    r.v[0].x = *reinterpret_cast<const uint32_t*>(q4 + j * 64 + d0 / 2);
    r.v[0].y = rsc[j * ng + d0 / group];
  } else {
#pragma unroll
    for (int c = 0; c < (int)(sizeof(T) / 2); ++c)
      r.v[c] = *reinterpret_cast<const u32x4*>(raw + j * 128 + d0 + c * (16 / sizeof(T)));
  }
}

template <typename T>
__device__ inline void vrow_widen(const VRow<T>& r, int ref_bits, float (&x)[8]) {
  if (ref_bits == 4) {
    const float s = half_bits_to_f32((uint16_t)r.v[0].y);
    const uint32_t w = r.v[0].x;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)((int32_t)(w << (28 - 4 * e)) >> 28) * s;
  } else if constexpr (sizeof(T) == 2) {
    x[0] = bf16_lo(r.v[0].x); x[1] = bf16_hi(r.v[0].x);
    x[2] = bf16_lo(r.v[0].y); x[3] = bf16_hi(r.v[0].y);
    x[4] = bf16_lo(r.v[0].z); x[5] = bf16_hi(r.v[0].z);
    x[6] = bf16_lo(r.v[0].w); x[7] = bf16_hi(r.v[0].w);
  } else {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      x[4 * c + 0] = __uint_as_float(r.v[c].x); x[4 * c + 1] = __uint_as_float(r.v[c].y);
      x[4 * c + 2] = __uint_as_float(r.v[c].z); x[4 * c + 3] = __uint_as_float(r.v[c].w);
    }
  }
}

template <typename T, int CT>
__global__ __launch_bounds__(CT) void k_combine(const float* __restrict__ part,
                                                          const T* __restrict__ ref_kv,
                                                          const uint16_t* __restrict__ ref_scales,
                                                          int ref_bits, int group,
                                                          float* __restrict__ out, int G, int H,
                                                          int64_t n_refs, int64_t n_valid,
                                                          int n_split, float* __restrict__ ores) {
  constexpr int kCombRG = CT / 16;  // reference stride groups
  constexpr int kWThreads = CT - 128;  // threads merging W (float4 chunks)
  extern __shared__ float cs[];
  const int64_t nrp = ((n_refs + 3) / 4) * 4;
  float* wt = cs;               // [nrp] merged W
  float* fs = wt + nrp;         // [n_split] split factors
  float* sm = fs + n_split;     // [2]: l, and [128] merged P.V at sm + 4
  float* red = sm + 132;        // [kCombRG][128] partial W . Vref
  // grid (H, n_inst, G): the G query heads of a KV head are its items
  int kvh = blockIdx.x;
  int64_t inst = blockIdx.y;
  int g = blockIdx.z;
  if ((((int64_t)gridDim.x * gridDim.y) & 7) == 0) {
    const XcdItem it = xcd_item(blockIdx.x + (int64_t)gridDim.x * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z),
                                gridDim.z);
    kvh = (int)(it.head % H);
    inst = it.head / H;
    g = it.item;
  }
  const int hq = kvh * G + g;
  const int Hq = H * G;
  const int tid = threadIdx.x;
  const int64_t rec = part_rec_floats(n_refs);
  const float* base = part + (inst * Hq + hq) * n_split * rec;  // split s at base + s * rec

  // reference rows for W . Vref
  const int dg = tid & 15, rg = tid >> 4;
  const int d0 = dg * 8;
  const int64_t row0 = ((inst * H + kvh) * 2 + 1) * n_refs;  // V plane
  const int ngq = ref_bits == 4 ? 128 / group : 1;
  const T* raw = ref_kv + row0 * 128;
  const uint8_t* q4 = reinterpret_cast<const uint8_t*>(ref_kv) + row0 * 64;
  const uint16_t* rsc = ref_bits == 4 ? ref_scales + row0 * ngq : nullptr;
  constexpr int kCombRows = comb_rows<T>();
  VRow<T> xr[kCombRows];
#pragma unroll
  for (int u = 0; u < kCombRows; ++u) {
    const int64_t j = rg + (int64_t)u * kCombRG;
    if (j < n_valid) vrow_load<T>(raw, q4, rsc, ngq, group, ref_bits, j, d0, xr[u]);
  }
  // roles for the merges: wave 0 the maximum and the sum, threads 64 ..
  // CT - 65 float4 chunks of W (chunk c, c + CT - 128, ...), the last 64
  // threads two dims of P.V each
  const int64_t wc = tid - 64;  // first W chunk of this thread
  const bool w_role = wc >= 0 && wc < nrp / 4 && wc < kWThreads;
  const int od = 2 * (tid - (CT - 64));  // P.V dims od, od + 1
  const bool o_role = tid >= CT - 64;
  float4 wv[kCombSplits];
  float2 ov[kCombSplits];
  if (w_role) {
#pragma unroll
    for (int s = 0; s < kCombSplits; ++s)
      if (s < n_split) wv[s] = *reinterpret_cast<const float4*>(base + s * rec + 132 + 4 * wc);
  }
  if (o_role) {
#pragma unroll
    for (int s = 0; s < kCombSplits; ++s)
      if (s < n_split) ov[s] = *reinterpret_cast<const float2*>(base + s * rec + 4 + od);
  }
  if (tid < 64) {
    float M = -INFINITY;
    for (int s = tid; s < n_split; s += 64) M = fmaxf(M, base[s * rec]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float l = 0.f;
    for (int s = tid; s < n_split; s += 64) {
      const float m = base[s * rec];
      const float f = m > -INFINITY ? __expf(m - M) : 0.f;
      fs[s] = f;
      l += f * base[s * rec + 1];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
    if (tid == 0) sm[0] = l;
  }
  __syncthreads();
  // merged W (float4 chunks) and merged P.V
  for (int64_t c = wc; wc >= 0 && wc < kWThreads && c < nrp / 4; c += kWThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = 0;
    if (c == wc && w_role) {
#pragma unroll
      for (int u = 0; u < kCombSplits; ++u) {
        if (u < n_split) {
          const float f = fs[u];
          acc.x += f * wv[u].x; acc.y += f * wv[u].y; acc.z += f * wv[u].z; acc.w += f * wv[u].w;
        }
      }
      s = kCombSplits;
    }
    // further splits in batches, each batch's loads first (the sum keeps
    // split order)
    for (; s + kCombSplits <= n_split; s += kCombSplits) {
      float4 v[kCombSplits];
#pragma unroll
      for (int u = 0; u < kCombSplits; ++u)
        v[u] = *reinterpret_cast<const float4*>(base + (s + u) * rec + 132 + 4 * c);
#pragma unroll
      for (int u = 0; u < kCombSplits; ++u) {
        const float f = fs[s + u];
        acc.x += f * v[u].x; acc.y += f * v[u].y; acc.z += f * v[u].z; acc.w += f * v[u].w;
      }
    }
    for (; s < n_split; ++s) {
      const float f = fs[s];
      const float4 v = *reinterpret_cast<const float4*>(base + s * rec + 132 + 4 * c);
      acc.x += f * v.x; acc.y += f * v.y; acc.z += f * v.z; acc.w += f * v.w;
    }
    *reinterpret_cast<float4*>(wt + 4 * c) = acc;
  }
  if (o_role) {
    float2 acc = make_float2(0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kCombSplits; ++u) {
      if (u < n_split) {
        acc.x += fs[u] * ov[u].x;
        acc.y += fs[u] * ov[u].y;
      }
    }
    int s = kCombSplits;
    for (; s + kCombSplits <= n_split; s += kCombSplits) {
      float2 v[kCombSplits];
#pragma unroll
      for (int u = 0; u < kCombSplits; ++u)
        v[u] = *reinterpret_cast<const float2*>(base + (s + u) * rec + 4 + od);
#pragma unroll
      for (int u = 0; u < kCombSplits; ++u) {
        acc.x += fs[s + u] * v[u].x;
        acc.y += fs[s + u] * v[u].y;
      }
    }
    for (; s < n_split; ++s) {
      const float2 v = *reinterpret_cast<const float2*>(base + s * rec + 4 + od);
      acc.x += fs[s] * v.x;
      acc.y += fs[s] * v.y;
    }
    sm[4 + od] = acc.x;
    sm[4 + od + 1] = acc.y;
  }
  __syncthreads();
  // W . Vref
  float a[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = 0.f;
#pragma unroll
  for (int u = 0; u < kCombRows; ++u) {
    const int64_t j = rg + (int64_t)u * kCombRG;
    if (j < n_valid) {
      const float wj = wt[j];
      float x[8];
      vrow_widen<T>(xr[u], ref_bits, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = __builtin_fmaf(wj, x[e], a[e]);
    }
  }
  // the rest in batches of kCombRows rows, all of a batch's loads first
  for (int64_t j0 = rg + (int64_t)kCombRows * kCombRG; j0 < n_valid; j0 += (int64_t)kCombRows * kCombRG) {
    VRow<T> yr[kCombRows];
#pragma unroll
    for (int u = 0; u < kCombRows; ++u) {
      const int64_t j = j0 + (int64_t)u * kCombRG;
      if (j < n_valid) vrow_load<T>(raw, q4, rsc, ngq, group, ref_bits, j, d0, yr[u]);
    }
#pragma unroll
    for (int u = 0; u < kCombRows; ++u) {
      const int64_t j = j0 + (int64_t)u * kCombRG;
      if (j < n_valid) {
        float y[8];
        vrow_widen<T>(yr[u], ref_bits, y);
        const float wj = wt[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = __builtin_fmaf(wj, y[e], a[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg * 128 + d0 + e] = a[e];
  __syncthreads();
  if (tid < 128) {
    float s = 0.f;
    for (int g = 0; g < kCombRG; ++g) s += red[g * 128 + tid];
    const float l = sm[0];
    const float o = sm[4 + tid];
    const int64_t at = (inst * Hq + hq) * 128 + tid;
    // a head that attended no position (l = 0: an empty tile selection)
    // gets a zero row
    const float il = l > 0.f ? 1.f / l : 0.f;
    if (ores) {
      // latent codes: the residual part is still rotated; f_d is applied
      // to the whole row afterwards
      ores[at] = o * il;
      out[at] = s * il;
    } else {
      out[at] = (o + s) * il;
    }
  }
}

// ------------------------------------------------------ latent transforms
// One wave per 128-dim row, lane l holding dims 2l and 2l+1: index bit 0
// inside the lane, bits 1-6 across lanes (xor 1 .. 32).
__device__ inline void fwht128_2(float& a, float& b, int l) {
  const float x = a + b, y = a - b;
  a = x;
  b = y;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const bool hi = (l & m) != 0;
    const float pa = __shfl_xor(a, m), pb = __shfl_xor(b, m);
    a = hi ? pa - a : a + pa;
    b = hi ? pb - b : b + pb;
  }
}

__device__ inline void lat_signs2(float& a, float& b, const LatMask& lm, int l) {
  const uint32_t word = l < 32 ? (l < 16 ? lm.w[0] : lm.w[1]) : (l < 48 ? lm.w[2] : lm.w[3]);
  const uint32_t bb = (word >> (2 * (l & 15))) & 3u;
  a = __uint_as_float(__float_as_uint(a) ^ ((bb & 1u) << 31));
  b = __uint_as_float(__float_as_uint(b) ^ ((bb >> 1) << 31));
}

// qrot[r] = H D q[r] / 8 (fp32), r < rows.
template <typename T>
__global__ __launch_bounds__(256) void k_latent_q(const T* __restrict__ q, LatMask lm,
                                                  float* __restrict__ qrot, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // whole waves
  const int l = threadIdx.x & 63;
  float a = (float)q[r * 128 + 2 * l], b = (float)q[r * 128 + 2 * l + 1];
  lat_signs2(a, b, lm, l);
  fwht128_2(a, b, l);
  qrot[r * 128 + 2 * l] = a * 0.125f;
  qrot[r * 128 + 2 * l + 1] = b * 0.125f;
}

// out[r] += f_d(ores[r]) = D H ores[r] / 8, r < rows.
__global__ __launch_bounds__(256) void k_latent_out(const float* __restrict__ ores, LatMask lm,
                                                    float* __restrict__ out, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int l = threadIdx.x & 63;
  float a = ores[r * 128 + 2 * l], b = ores[r * 128 + 2 * l + 1];
  fwht128_2(a, b, l);
  lat_signs2(a, b, lm, l);
  out[r * 128 + 2 * l] += a * 0.125f;
  out[r * 128 + 2 * l + 1] += b * 0.125f;
}

// ------------------------------------------------------- exact residuals
// bits = 0 keeps every residual exactly (fp64), so attention runs on the
// rebuilt cache itself: each attended position is KV_R + residual, with
// KV_R the fp32 mean the encoder took (ascending-slot fp32 sum, divided by
// k_eff), which gives back the input rows.  Plain softmax attention, one
// block per (instance, KV head, split); wave w takes positions w, w+4, ...
// of each tile, lane l dims 2l and 2l+1.  Writes the same partial records as
// k_decode (W = 0: the reference mean is already inside every row), so
// k_combine merges them unchanged.  G <= 16.
template <typename T>
__device__ inline float2 ld_pair(const T* p) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(bf16_lo(w), bf16_hi(w));
  } else {
    return *reinterpret_cast<const float2*>(p);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_decode_exact(
    const T* __restrict__ q, const T* __restrict__ ref_kv, const uint16_t* __restrict__ idx,
    const double* __restrict__ rk, const double* __restrict__ rv, float* __restrict__ part,
    float alpha, int64_t N, int64_t Nlen, int64_t n_refs, Sched sc, int k, int G, int H,
    int n_split, const int32_t* __restrict__ tile_list, int32_t n_list) {
  __shared__ float ms[4][16], ls[4][16];
  __shared__ float os[4][16][128];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int64_t inst = blockIdx.z;
  const int64_t ih = inst * H + kvh;
  const int Hq = H * G;
  const int32_t tiles_len = (int32_t)((Nlen + kDecTile - 1) / kDecTile);
  const int32_t* tl = tile_list ? tile_list + ih * n_list : nullptr;
  const int32_t n_ent = tl ? n_list : tiles_len;
  const int32_t tps = (n_ent + n_split - 1) / n_split;
  const int32_t t0 = split * tps;
  const int32_t t1 = (t0 + tps < n_ent) ? t0 + tps : n_ent;
  const int d0 = 2 * lane;
  float qa[16], qb[16], m[16], l[16], o0[16], o1[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    qa[h] = qb[h] = 0.f;
    m[h] = -INFINITY;
    l[h] = o0[h] = o1[h] = 0.f;
    if (h < G) {
      const float2 v = ld_pair(q + ((inst * Hq + kvh * G + h) * 128 + d0));
      qa[h] = v.x;
      qb[h] = v.y;
    }
  }
  const T* rkb = ref_kv + ih * 2 * n_refs * 128;   // K plane; V plane at + n_refs * 128
  for (int32_t e = t0; e < t1; ++e) {
    int32_t tile = e;
    if (tl) {
      const int32_t x = tl[e];
      tile = (x >= 0 && x < tiles_len) ? x : tiles_len;
    }
    for (int u = w; u < kDecTile; u += 4) {
      const int64_t p = (int64_t)tile * kDecTile + u;
      if (p >= Nlen) break;
      float2 kk, vv;
      const int32_t slot = sched_slot((int32_t)p, sc);
      if (slot >= 0) {
        kk = ld_pair(rkb + (int64_t)slot * 128 + d0);
        vv = ld_pair(rkb + (n_refs + slot) * 128 + d0);
      } else {
        const int32_t cnt = sched_count_le((int32_t)p, sc);
        const int keff = cnt < k ? cnt : k;
        float sk0 = 0.f, sk1 = 0.f, sv0 = 0.f, sv1 = 0.f;
        for (int j = 0; j < keff; ++j) {
          const int64_t r = idx[(ih * N + p) * k + j];
          const float2 a = ld_pair(rkb + r * 128 + d0);
          const float2 b = ld_pair(rkb + (n_refs + r) * 128 + d0);
          if (j == 0) {
            sk0 = a.x; sk1 = a.y; sv0 = b.x; sv1 = b.y;
          } else {
            sk0 += a.x; sk1 += a.y; sv0 += b.x; sv1 += b.y;
          }
        }
        const float kf = (float)keff;
        const double2 dk = *reinterpret_cast<const double2*>(rk + (ih * N + p) * 128 + d0);
        const double2 dv = *reinterpret_cast<const double2*>(rv + (ih * N + p) * 128 + d0);
        kk = make_float2((float)((double)(sk0 / kf) + dk.x), (float)((double)(sk1 / kf) + dk.y));
        vv = make_float2((float)((double)(sv0 / kf) + dv.x), (float)((double)(sv1 / kf) + dv.y));
      }
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        if (h < G) {
          float sdot = __builtin_fmaf(qa[h], kk.x, qb[h] * kk.y);
#pragma unroll
          for (int off = 32; off > 0; off >>= 1) sdot += __shfl_xor(sdot, off);
          const float lg = alpha * sdot;
          const float mn = fmaxf(m[h], lg);
          const float f = m[h] > -INFINITY ? __expf(m[h] - mn) : 0.f;
          const float pe = __expf(lg - mn);
          l[h] = l[h] * f + pe;
          o0[h] = __builtin_fmaf(pe, vv.x, o0[h] * f);
          o1[h] = __builtin_fmaf(pe, vv.y, o1[h] * f);
          m[h] = mn;
        }
      }
    }
  }
  // merge the four waves
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    if (h < G) {
      if (lane == 0) {
        ms[w][h] = m[h];
        ls[w][h] = l[h];
      }
      os[w][h][d0] = o0[h];
      os[w][h][d0 + 1] = o1[h];
    }
  }
  __syncthreads();
  const int64_t rec = part_rec_floats(n_refs);
  const int64_t nrp = ((n_refs + 3) / 4) * 4;
  for (int h = 0; h < G; ++h) {
    float* pr = part + ((inst * Hq + kvh * G + h) * n_split + split) * rec;
    const float M = fmaxf(fmaxf(ms[0][h], ms[1][h]), fmaxf(ms[2][h], ms[3][h]));
    float fw[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) fw[x] = ms[x][h] > -INFINITY ? __expf(ms[x][h] - M) : 0.f;
    if (threadIdx.x < 128) {
      const int d = threadIdx.x;
      pr[4 + d] = ((fw[0] * os[0][h][d] + fw[1] * os[1][h][d]) + fw[2] * os[2][h][d]) +
                  fw[3] * os[3][h][d];
    }
    if (threadIdx.x == 0) {
      pr[0] = M;
      pr[1] = ((fw[0] * ls[0][h] + fw[1] * ls[1][h]) + fw[2] * ls[2][h]) + fw[3] * ls[3][h];
    }
    for (int64_t j = threadIdx.x; j < nrp; j += 256) pr[132 + j] = 0.f;
  }
}

// ------------------------------------------------------------------ launchers
static size_t qk_bytes(int64_t n_inst, int n_q_heads, int64_t n_refs) {
  const size_t b = (size_t)n_inst * n_q_heads * (((n_refs + 3) / 4) * 4) * 4;
  return (b + 255) / 256 * 256;
}

static size_t part_bytes(int64_t n_inst, int n_q_heads, int n_split, int64_t n_refs) {
  const size_t b = (size_t)n_inst * n_q_heads * n_split * part_rec_floats(n_refs) * 4;
  return (b + 255) / 256 * 256;
}

// latent mode: rotated queries, then the merged rotated residual outputs
static size_t row_bytes(int64_t n_inst, int n_q_heads) {
  const size_t b = (size_t)n_inst * n_q_heads * 128 * 4;
  return (b + 255) / 256 * 256;
}

size_t decode_ws_bytes(int64_t n_inst, int H, int n_q_heads, int n_split, int64_t n_refs,
                       bool latent) {
  (void)H;
  return qk_bytes(n_inst, n_q_heads, n_refs) + part_bytes(n_inst, n_q_heads, n_split, n_refs) +
         (latent ? 2 * row_bytes(n_inst, n_q_heads) : 0);
}

size_t decode_lds_bytes(int G, int NG, int64_t n_refs) {
  const int64_t nrp = ((n_refs + 3) / 4) * 4;
  return (size_t)((2 * G + 2 * ((G + 1) / 2)) * (nrp + 8) + G * (kChunkTiles * kDecTile + kLgPad) +
                  96 + 4 + 4) * 4 +  // m_s, wm_s, sc_s; vp_s; vw_s
         (size_t)(4 * 16 + 4 * NG) * kDecTile * 2;
}

size_t combine_lds_bytes(int G, int64_t n_refs, int n_split) {
  (void)G;
  const int64_t nrp = ((n_refs + 3) / 4) * 4;
  return (size_t)(nrp + n_split + 132 + (1024 / 16) * 128) * 4;  // the 1024-thread form
}

// Whether the decode kernels' LDS fits one CU (160 KiB).  The exact-residual
// decode keeps no per-reference state; only its combine does.
bool decode_fits(int G, int group, int64_t n_refs, int n_split, bool exact) {
  const int NG = 128 / group;
  return (exact || decode_lds_bytes(G, NG, n_refs) <= 160 * 1024) &&
         combine_lds_bytes(G, n_refs, n_split) <= 160 * 1024;
}

template <typename T>
hipError_t launch_decode_exact(const void* q, int n_q_heads, const uint16_t* idx,
                               const void* ref_kv, const uint8_t* ck, const uint8_t* cv,
                               float alpha, float* out, int n_split, void* ws, int64_t n_inst,
                               int H, int64_t N, int64_t len, int64_t n_refs, Sched sc, int k,
                               const int32_t* tile_list, int32_t n_list, hipStream_t st) {
  const int G = n_q_heads / H;
  float* part = (float*)((char*)ws + qk_bytes(n_inst, n_q_heads, n_refs));
  hipLaunchKernelGGL(k_decode_exact<T>, dim3(n_split, H, (unsigned)n_inst), dim3(256), 0, st,
                     (const T*)q, (const T*)ref_kv, idx, (const double*)ck, (const double*)cv,
                     part, alpha, N, len, n_refs, sc, k, G, H, n_split, tile_list, n_list);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_valid = sched_count((int32_t)len, sc);
  const bool wide = (int64_t)H * n_inst * G <= 512;
  const size_t clds = combine_lds_bytes(G, n_refs, n_split);
  auto comb = wide ? k_combine<T, 1024> : k_combine<T, 256>;
  if (clds > 64 * 1024) {
    e = hipFuncSetAttribute((const void*)comb, hipFuncAttributeMaxDynamicSharedMemorySize, (int)clds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(comb, dim3(H, (unsigned)n_inst, G), dim3(wide ? 1024 : 256), clds, st, part,
                     (const T*)ref_kv, (const uint16_t*)nullptr, 0, 128, out, G, H, n_refs, n_valid,
                     n_split, (float*)nullptr);
  return hipGetLastError();
}

template <typename T, int BITS, int NG, int KM, bool EX>
hipError_t launch_decode_t(const void* q, int n_q_heads, const uint16_t* idx,
                           const void* ref_kv, const uint16_t* ref_scales, int ref_bits, int group_r,
                           const uint8_t* ck, const uint8_t* cv,
                           const uint16_t* sc16, float alpha, float* out, int n_split, void* ws,
                           int64_t n_inst, int H, int64_t N, int64_t len, int64_t n_refs, Sched sc, int k,
                           const int32_t* tile_list, int32_t n_list, const LatMask* lm,
                           hipStream_t st) {
  const int G = n_q_heads / H;
  float* qk = (float*)ws;
  float* part = (float*)((char*)ws + qk_bytes(n_inst, n_q_heads, n_refs));
  float* qrot = nullptr;
  float* ores = nullptr;
  const int64_t rows = n_inst * n_q_heads;
  if (lm) {
    qrot = (float*)((char*)part + part_bytes(n_inst, n_q_heads, n_split, n_refs));
    ores = (float*)((char*)qrot + row_bytes(n_inst, n_q_heads));
    hipLaunchKernelGGL(k_latent_q<T>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       (const T*)q, *lm, qrot, rows);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  const int64_t nrp = ((n_refs + 3) / 4) * 4;
  const int64_t n_valid = sched_count((int32_t)len, sc);
  hipLaunchKernelGGL(k_qk_table<T>, dim3((unsigned)((nrp + 63) / 64), H, (unsigned)n_inst),
                     dim3(256), 0, st, (const T*)q, (const T*)ref_kv, ref_scales, ref_bits,
                     group_r, qk, G, H, n_refs, n_valid);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = decode_lds_bytes(G, NG, n_refs);
  auto kern = k_decode<T, BITS, NG, KM, EX>;
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(n_split, H, (unsigned)n_inst), dim3(256), lds, st, (const T*)q,
                     (const T*)ref_kv, idx, ck, cv, sc16, qk, part, alpha, N, len, n_refs, sc, k, G, H,
                     n_split, tile_list, n_list, qrot);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 1024-thread blocks while the launch has at most about two blocks per CU
  const bool wide = (int64_t)H * n_inst * G <= 512;
  const size_t clds = combine_lds_bytes(G, n_refs, n_split);
  auto comb = wide ? k_combine<T, 1024> : k_combine<T, 256>;
  if (clds > 64 * 1024) {
    e = hipFuncSetAttribute((const void*)comb, hipFuncAttributeMaxDynamicSharedMemorySize, (int)clds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(comb, dim3(H, (unsigned)n_inst, G), dim3(wide ? 1024 : 256), clds, st, part,
                     (const T*)ref_kv, ref_scales, ref_bits, group_r, out, G, H, n_refs, n_valid,
                     n_split, ores);
  e = hipGetLastError();
  if (e != hipSuccess || !lm) return e;
  hipLaunchKernelGGL(k_latent_out, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, ores, *lm,
                     out, rows);
  return hipGetLastError();
}

template <typename T, int BITS, int NG>
hipError_t launch_decode_k(int k, const void* q, int n_q_heads, const uint16_t* idx,
                           const void* ref_kv, const uint16_t* ref_scales, int ref_bits, int group_r,
                           const uint8_t* ck, const uint8_t* cv,
                           const uint16_t* sc16, float alpha, float* out, int n_split, void* ws,
                           int64_t n_inst, int H, int64_t N, int64_t len, int64_t n_refs, Sched sc, const int32_t* tile_list,
                           int32_t n_list, const LatMask* lm, hipStream_t st) {
  if (k == 4) return launch_decode_t<T, BITS, NG, 4, true>(q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, k, tile_list, n_list, lm, st);
  if (k == 8) return launch_decode_t<T, BITS, NG, 8, true>(q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, k, tile_list, n_list, lm, st);
  if (k == 16) return launch_decode_t<T, BITS, NG, 16, true>(q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, k, tile_list, n_list, lm, st);
  if (k < 4) return launch_decode_t<T, BITS, NG, 4, false>(q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, k, tile_list, n_list, lm, st);
  if (k < 8) return launch_decode_t<T, BITS, NG, 8, false>(q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, k, tile_list, n_list, lm, st);
  return launch_decode_t<T, BITS, NG, 16, false>(q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, k, tile_list, n_list, lm, st);
}

template <typename T, int BITS>
hipError_t launch_decode_g(int group, int k, const void* q, int n_q_heads, const uint16_t* idx,
                           const void* ref_kv, const uint16_t* ref_scales, int ref_bits, int group_r,
                           const uint8_t* ck, const uint8_t* cv,
                           const uint16_t* sc16, float alpha, float* out, int n_split, void* ws,
                           int64_t n_inst, int H, int64_t N, int64_t len, int64_t n_refs, Sched sc, const int32_t* tile_list,
                           int32_t n_list, const LatMask* lm, hipStream_t st) {
  if (group == 32)
    return launch_decode_k<T, BITS, 4>(k, q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, tile_list, n_list, lm, st);
  if (group == 64)
    return launch_decode_k<T, BITS, 2>(k, q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, tile_list, n_list, lm, st);
  return launch_decode_k<T, BITS, 1>(k, q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, tile_list, n_list, lm, st);
}

template <typename T>
hipError_t launch_decode_b(int bits, int group, int k, const void* q, int n_q_heads,
                           const uint16_t* idx, const void* ref_kv, const uint16_t* ref_scales,
                           int ref_bits, int group_r, const uint8_t* ck,
                           const uint8_t* cv, const uint16_t* sc16, float alpha, float* out,
                           int n_split, void* ws, int64_t n_inst, int H, int64_t N, int64_t len, int64_t n_refs, Sched sc, const int32_t* tile_list,
                           int32_t n_list, const LatMask* lm, hipStream_t st) {
  if (bits == 2)
    return launch_decode_g<T, 2>(group, k, q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, tile_list, n_list, lm, st);
  if (bits == 4)
    return launch_decode_g<T, 4>(group, k, q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, tile_list, n_list, lm, st);
  return launch_decode_g<T, 8>(group, k, q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group_r, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, len, n_refs, sc, tile_list, n_list, lm, st);
}

hipError_t launch_decode(int dtype, int bits, const void* q, int n_q_heads, const uint16_t* idx,
                         const void* ref_kv, const uint16_t* ref_scales, int ref_bits,
                         const uint8_t* ck, const uint8_t* cv,
                         const uint16_t* sc16, float softmax_scale, float* out, int n_split,
                         void* ws, int64_t n_inst, int H, int64_t N, int64_t len, int64_t n_refs, Sched sc,
                         int k, int group, const int32_t* tile_list, int32_t n_list,
                         const LatMask* lm, hipStream_t st) {
  if (bits == 0) {
    if (dtype == 0)
      return launch_decode_exact<float>(q, n_q_heads, idx, ref_kv, ck, cv, softmax_scale, out, n_split, ws, n_inst, H, N, len, n_refs, sc, k, tile_list, n_list, st);
    return launch_decode_exact<__bf16>(q, n_q_heads, idx, ref_kv, ck, cv, softmax_scale, out, n_split, ws, n_inst, H, N, len, n_refs, sc, k, tile_list, n_list, st);
  }
  if (dtype == 0)
    return launch_decode_b<float>(bits, group, k, q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group, ck, cv, sc16, softmax_scale, out, n_split, ws, n_inst, H, N, len, n_refs, sc, tile_list, n_list, lm, st);
  return launch_decode_b<__bf16>(bits, group, k, q, n_q_heads, idx, ref_kv, ref_scales, ref_bits, group, ck, cv, sc16, softmax_scale, out, n_split, ws, n_inst, H, N, len, n_refs, sc, tile_list, n_list, lm, st);
}

}  // namespace rkv
