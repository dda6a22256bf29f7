// Reference store and reference selection (gfx950).
//
// Paper page "DeltaKV Framework Architecture": references are every s-th
// token; each token keeps the k references nearest to it in L2 distance.
// Section "Practical Deployment via Sparse-vLLM" names a batched L2-distance
// kernel for this search.  Here the search is a bf16 MFMA contraction
// (|r|^2 - 2 k.r; |k|^2 is the same for every candidate of a row and does not
// change the order) fused with an exact top-k, so the token x reference
// distance matrix never leaves registers.
//
// Top-k on a 64-wide wave: a running sorted top-k per lane costs O(k) ops per
// candidate on every lane whenever any lane inserts, which with 64 independent
// rows is almost always.  Instead each row is scanned twice:
//   pass 1  keeps, per lane, the minimum of each of its 16 accumulator
//           positions ("buckets": disjoint candidate sets), 1 op/candidate;
//           the k-th smallest of a row's 32 bucket minima is an upper bound
//           tau on the row's k-th smallest distance;
//   pass 2  recomputes the same MFMA tiles (bit-identical values) and appends
//           candidates <= tau to a per-lane LDS list (about k per row; a
//           list near capacity is cut to the lane's own k best).  The append
//           is branch-free: every candidate is written at the list's end and
//           the end advances only for a survivor (a branch per candidate
//           costs far more than the store, since some lane of the wave almost
//           always takes it);
//   final   one lane per token (the wave's 64 lanes hold two 32-token sets,
//           each token split over lanes n and n + 32; one cross-half swap
//           regroups them so that lower lanes finish set 0 and upper lanes
//           set 1) loads the token's two lists and takes the k smallest by
//           (distance, slot), lowest slot first on ties, written in ascending
//           slot order.  tau is found the same way.
#include <float.h>

#include "rkv_common.h"
#include "rkv_quant.h"

namespace rkv {

// ------------------------------------------------------------------ refstore
// One wave per new reference (slots s0 .. s0+ns-1 of every (instance,
// head), at positions inside the input range that starts at p0): copies its
// K and V rows into the cache's reference store, writes -2 x the bf16-rounded
// key (exact: a power-of-two scaling) and the squared norm of the bf16 key to
// the workspace.  Input rows are [ih][n_in][128].
// With ref_bits = 4 the rows are stored quantised (int4 nibbles, fp16 scale
// per group of `group` dims, the residual quantiser's exact rounding); the
// workspace keys and norms still come from the original key.
template <typename T>
__global__ __launch_bounds__(256) void k_refstore(
    const T* __restrict__ K, const T* __restrict__ V, void* __restrict__ ref_kv_v,
    uint16_t* __restrict__ ref_scales, int ref_bits, int group,
    __bf16* __restrict__ refkey, float* __restrict__ refnorm, int64_t n_in, int64_t p0,
    int64_t n_refs, int64_t s0, int64_t ns, Sched sc, int64_t total_refs) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= total_refs) return;
  const int64_t ih = r / ns;
  const int64_t slot = s0 + (r - ih * ns);
  const int64_t pos = sched_pos((int32_t)slot, sc);
  const T* kr = K + (ih * n_in + (pos - p0)) * 128;
  const T* vr = V + (ih * n_in + (pos - p0)) * 128;
  const int t = lane * 2;
  if (ref_bits == 4) {
    // lane t/2 holds dims t, t+1: one byte of nibbles per plane
    uint8_t* rq = reinterpret_cast<uint8_t*>(ref_kv_v);
    const int lanes_per_group = group >> 1;
    const int ng = 128 / group;
#pragma unroll
    for (int pl = 0; pl < 2; ++pl) {
      const T* xr = pl ? vr : kr;
      const float x0 = (float)xr[t], x1 = (float)xr[t + 1];
      float a = fmaxf(fabsf(x0), fabsf(x1));
      for (int off = 1; off < lanes_per_group; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
      const uint16_t sb = exact_scale_bits(a, 7.f, 1.0f / 7.f);
      const int c0 = exact_code_of(x0, sb, 7.f), c1 = exact_code_of(x1, sb, 7.f);
      const int64_t row = (ih * 2 + pl) * n_refs + slot;
      rq[row * 64 + lane] = (uint8_t)((c0 & 0xF) | ((c1 & 0xF) << 4));
      if (t % group == 0) ref_scales[row * ng + t / group] = sb;
    }
  } else {
    T* ref_kv = reinterpret_cast<T*>(ref_kv_v);
    T* dk = ref_kv + ((ih * 2 + 0) * n_refs + slot) * 128;
    T* dv = ref_kv + ((ih * 2 + 1) * n_refs + slot) * 128;
    dk[t] = kr[t];
    dk[t + 1] = kr[t + 1];
    dv[t] = vr[t];
    dv[t + 1] = vr[t + 1];
  }
  const __bf16 b0 = (__bf16)(float)kr[t];
  const __bf16 b1 = (__bf16)(float)kr[t + 1];
  const int64_t wr = ih * n_refs + slot;
  refkey[wr * 128 + t] = (__bf16)(-2.0f * (float)b0);
  refkey[wr * 128 + t + 1] = (__bf16)(-2.0f * (float)b1);
  double s = (double)(float)b0 * (double)(float)b0 + (double)(float)b1 * (double)(float)b1;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) refnorm[wr] = (float)s;
}

// ------------------------------------------------------------------ top-k
template <int KM>
__device__ inline void topk_insert(float (&top)[KM], float v) {
#pragma unroll
  for (int t = KM - 1; t > 0; --t) top[t] = __builtin_amdgcn_fmed3f(top[t - 1], v, top[t]);
  top[0] = fminf(top[0], v);
}

// k-th smallest (1 <= k <= KM) of an ascending list: the largest of its
// first k entries.  Written as a masked max so that it stays in registers
// (a select chain over t == k - 1 can be folded into a memory-indexed load).
template <int KM>
__device__ inline float topk_get(const float (&top)[KM], int k) {
  float r = -INFINITY;
#pragma unroll
  for (int t = 0; t < KM; ++t) r = fmaxf(r, t < k ? top[t] : -INFINITY);
  return r;
}

// Row of accumulator register r of a 32x32 MFMA tile for lane half `half`.
__device__ inline int acc_row(int r, int half) { return (r & 3) + 8 * (r >> 2) + 4 * half; }

// Survivor lists: per (lane, token set) entries of a distance (fp32 bits)
// and a slot.  For k <= 8 an entry is two words, laid out [entry][word][64
// lanes] so that one entry is a single two-address LDS store; capacity: the
// lane's k best, 3 more (a lane holds about k/2 + 1 survivors on average,
// rarely more than k + 3, so a list seldom needs cutting), plus the
// kCheckRows accumulator rows appended between two fullness checks.  For
// k > 8 the distances ([entry][64 lanes] words) and the slots ([entry][64
// lanes] halves) are separate arrays and the capacity has no slack (k +
// kCheckRows): 6 bytes per entry, so that two blocks fit in LDS.
constexpr int kCheckRows = 4;
template <int KM>
constexpr bool split_lists() { return KM > 8; }
template <int KM>
constexpr int surv_cap() { return split_lists<KM>() ? KM + kCheckRows : KM + 3 + kCheckRows; }
constexpr int kEntryWords = 128;  // stride of one two-word entry, in 32-bit words

// One lane's list: d = its distance of entry 0.  Split layout: a wave's
// lists are [set 0 distances][set 1 distances][slot words], each [entry][64
// lanes] words; the slot word of (entry, lane) holds set 0's slot in its low
// half and set 1's in its high half, so the slot of set c sits a fixed
// `soff` halfwords from the distance (one pointer per list, and the 64 lanes
// of a store touch 64 different words).
template <bool SPLIT>
struct LaneList {
  uint32_t* d;
  int soff;  // split layout: halfword offset of the slot from the distance
  static constexpr int kD = SPLIT ? 64 : kEntryWords;  // distance stride, in words
  __device__ uint32_t dist(int c) const { return d[c * kD]; }
  __device__ uint32_t slot(int c) const {
    if constexpr (SPLIT) return reinterpret_cast<const uint16_t*>(d)[soff + c * 128];
    else return d[c * kEntryWords + 64];
  }
  __device__ void put(int c, uint32_t dv, uint32_t sv) const {
    d[c * kD] = dv;
    if constexpr (SPLIT) reinterpret_cast<uint16_t*>(d)[soff + c * 128] = (uint16_t)sv;
    else d[c * kEntryWords + 64] = sv;
  }
};

// Loads a lane's survivor list into registers; entries past cnt read as +inf.
template <int CAP, bool SPLIT>
__device__ inline void load_list(const LaneList<SPLIT>& bl, int cnt, float (&e)[CAP], float (&js)[CAP]) {
#pragma unroll
  for (int c = 0; c < CAP; ++c) {
    const float v = __uint_as_float(bl.dist(c));
    const uint32_t j = bl.slot(c);
    e[c] = c < cnt ? v : INFINITY;
    js[c] = (float)j;
  }
}

// Cuts a lane's list to its own k best, keeping slot order; among entries
// equal to the k-th value the earlier (lower) slots stay.  Lowers tau to the
// k-th value: an entry dropped here is beaten by k kept ones, and every later
// entry has a higher slot.
template <int KM, int CAP, bool SPLIT>
__device__ __forceinline__ void lane_compact(const LaneList<SPLIT>& bl, int& cnt, float& tau, int k) {
  if (cnt <= k) return;
  float e[CAP], js[CAP];
  load_list<CAP>(bl, cnt, e, js);
  float top[KM];
#pragma unroll
  for (int t = 0; t < KM; ++t) top[t] = INFINITY;
#pragma unroll
  for (int c = 0; c < CAP; ++c) topk_insert(top, e[c]);
  const float t = topk_get(top, k);
  int nless = 0;
#pragma unroll
  for (int c = 0; c < CAP; ++c) nless += e[c] < t;
  const int quota = k - nless;
  int out = 0, ties = 0;
#pragma unroll
  for (int c = 0; c < CAP; ++c) {
    const bool tie = e[c] == t;
    const bool take = e[c] < t || (tie && ties < quota);
    ties += tie;
    if (take) {
      bl.put(out, __float_as_uint(e[c]), (uint32_t)js[c]);
      ++out;
    }
  }
  cnt = out;
  tau = fminf(tau, t);
}

// The keff nearest references of one token from its two survivor lists
// (la: cnt_a entries, lb: cnt_b entries), lowest slot first among equal
// distances; returns them in ascending slot order, 65535 past keff.
template <int KM, int CAP, bool SPLIT>
__device__ __forceinline__ void token_select(const LaneList<SPLIT>& la, int cnt_a,
                                             const LaneList<SPLIT>& lb, int cnt_b, int keff,
                                             float (&sel)[KM]) {
  float ea[CAP], ja[CAP], eb[CAP], jb[CAP];
  load_list<CAP>(la, cnt_a, ea, ja);
  load_list<CAP>(lb, cnt_b, eb, jb);
  // Entries past a list's count read +inf and change nothing below, so
  // groups of four entries past every lane's counts are skipped (the test
  // is wave-uniform); lists hold about k/2 entries against a capacity of
  // k + 7.
  const int cmax = cnt_a > cnt_b ? cnt_a : cnt_b;
  float top[KM];
#pragma unroll
  for (int t = 0; t < KM; ++t) top[t] = INFINITY;
#pragma unroll
  for (int c0 = 0; c0 < CAP; c0 += 4) {
    if (__any(c0 < cmax)) {
#pragma unroll
      for (int c = c0; c < c0 + 4 && c < CAP; ++c) {
        topk_insert(top, ea[c]);
        topk_insert(top, eb[c]);
      }
    }
  }
  const float th = topk_get(top, keff);
  int nless = 0, nties = 0;
#pragma unroll
  for (int c0 = 0; c0 < CAP; c0 += 4) {
    if (__any(c0 < cmax)) {
#pragma unroll
      for (int c = c0; c < c0 + 4 && c < CAP; ++c) {
        nless += (ea[c] < th) + (eb[c] < th);
        nties += (ea[c] == th) + (eb[c] == th);
      }
    }
  }
  const int quota = keff - nless;  // >= 1: th is the keff-th smallest
  float slot_bound = 65536.f;      // ties at th are taken up to this slot
  if (nties > quota) {
    float tl[KM];
#pragma unroll
    for (int t = 0; t < KM; ++t) tl[t] = 65536.f;
#pragma unroll
    for (int c = 0; c < CAP; ++c) {
      topk_insert(tl, ea[c] == th ? ja[c] : 65536.f);
      topk_insert(tl, eb[c] == th ? jb[c] : 65536.f);
    }
    slot_bound = topk_get(tl, quota);
  }
#pragma unroll
  for (int t = 0; t < KM; ++t) sel[t] = 65535.f;
#pragma unroll
  for (int c0 = 0; c0 < CAP; c0 += 4) {
    if (__any(c0 < cmax)) {
#pragma unroll
      for (int c = c0; c < c0 + 4 && c < CAP; ++c) {
        const bool ta = ea[c] < th || (ea[c] == th && ja[c] <= slot_bound);
        const bool tb = eb[c] < th || (eb[c] == th && jb[c] <= slot_bound);
        topk_insert(sel, ta ? ja[c] : 65535.f);
        topk_insert(sel, tb ? jb[c] : 65535.f);
      }
    }
  }
}

// Exchange between the two lane halves: returns {x of lanes 0-31 | y of
// lanes 0-31} in .a and {x of lanes 32-63 | y of lanes 32-63} in .b, i.e.
// lane l < 32 gets (x[l], x[l + 32]) and lane l >= 32 gets (y[l - 32], y[l]).
struct HalfPair {
  uint32_t a, b;
};
__device__ inline HalfPair half_swap(uint32_t x, uint32_t y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  return HalfPair{r[0], r[1]};
}

// 8 consecutive key elements as a bf16 B fragment (zeros for an invalid row):
// bf16 input as is, fp32 input rounded to nearest even.
__device__ inline bf16x8 load_key_frag(const __bf16* p, bool valid) {
  const uint4 w = valid ? *reinterpret_cast<const uint4*>(p) : make_uint4(0u, 0u, 0u, 0u);
  return __builtin_bit_cast(bf16x8, w);
}

__device__ inline bf16x8 load_key_frag(const float* p, bool valid) {
  float x[8];
  if (valid) {
    load8(p, x);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
  }
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = (__bf16)x[e];
  return b;
}

// One block = 4 waves x 64 tokens of one (instance, head); each wave holds
// the B operands of two 32-token sets, so every A fragment read from LDS
// feeds two independent MFMA chains.  Blocks are issued from the end of the
// sequence (most candidates) backwards.  Tiles of 32 reference keys (+ norms)
// are staged in LDS, double-buffered and loaded one tile ahead by the block.
constexpr int kRowPad = 136;  // bf16 per staged key row: 128 + 8 (bank spread)
constexpr int kSets = 2;      // 32-token sets per wave
constexpr int kBlockRows = 4 * 32 * kSets;

// Two blocks per CU (79 KB of LDS each).  DIRECT: the form for short ranges
// (a streaming append): one wave per block, no staging, no barriers -- each
// wave loads its A operands and norms straight from L2, one tile ahead, and
// runs the same MFMA chain (so its indices equal the staged form's).
template <typename T, int KM, bool DIRECT>
__global__ __launch_bounds__(DIRECT ? 64 : 256, 2) void k_dist_topk(
    const T* __restrict__ K, const __bf16* __restrict__ refkey,
    const float* __restrict__ refnorm, uint16_t* __restrict__ idx_out, int64_t N,
    int64_t n_refs, Sched sc, int k, int H, int n_blocks, int64_t p0, int64_t n_in) {
  // positions [p0, p1) from input rows [ih][n_in][128]; idx rows at ih * N + position
  const int64_t p1 = p0 + n_in;
  constexpr int CAP = surv_cap<KM>();
  constexpr bool SPLIT = split_lists<KM>();
  constexpr int NWV = DIRECT ? 1 : 4;           // waves per block
  constexpr int BROWS = NWV * 32 * kSets;       // tokens per block
  __shared__ uint32_t sbd[NWV][SPLIT ? kSets + 1 : kSets][CAP][SPLIT ? 64 : kEntryWords];
  // halfword offset from set c's distance to its slot (split layout)
  auto soff_of = [](int c_) RKV_INLINE { return (kSets - c_) * CAP * 128 + c_; };
  auto list_of = [&](int w_, int c_, int l_) RKV_INLINE {
    return LaneList<SPLIT>{&sbd[w_][c_][0][l_], soff_of(c_)};
  };
  __shared__ __attribute__((aligned(16))) __bf16 kbuf[DIRECT ? 1 : 2][32][kRowPad];
  __shared__ __attribute__((aligned(16))) float nbuf[DIRECT ? 1 : 2][32];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups are dealt to the 8 XCDs in turn.  When the heads split evenly
  // over them, the i-th workgroup of XCD x takes block i % n_blocks of head
  // 8 (i / n_blocks) + x, so the blocks of one head run together on one XCD
  // and share its L2 copy of the head's reference keys.  Within a head the
  // blocks still start from the end of the sequence (the most candidates).
  int64_t ih = (int64_t)blockIdx.z * H + blockIdx.y;
  int bx = (int)blockIdx.x;
  if (((gridDim.y * gridDim.z) & 7u) == 0) {
    const int64_t nb = gridDim.x;
    const int64_t L = blockIdx.x + nb * (blockIdx.y + (int64_t)gridDim.y * blockIdx.z);
    const int64_t i = L >> 3;
    ih = 8 * (i / nb) + (L & 7);
    bx = (int)(i % nb);
  }
  const int blk = n_blocks - 1 - bx;
  const int64_t blk0 = p0 + (int64_t)blk * BROWS;
  const int64_t row0 = blk0 + w * 32 * kSets;
  const bool active = row0 < p1;
  const int n = lane & 31;
  const int half = lane >> 5;
  const int64_t blk_last = (blk0 + BROWS - 1 < p1) ? blk0 + BROWS - 1 : p1 - 1;
  const int ntile_blk = (int)((sched_count_le((int32_t)blk_last, sc) + 31) / 32);
  const int64_t last_row = (row0 + 32 * kSets - 1 < p1) ? row0 + 32 * kSets - 1 : p1 - 1;
  const int ntile = active ? (int)((sched_count_le((int32_t)last_row, sc) + 31) / 32) : 0;
  const int full_tiles = active ? (int)(sched_count_le((int32_t)row0, sc) / 32) : 0;
  bool valid_row[kSets];
  int my_last[kSets];
  // B operands: bf16(key) of token row0 + 32c + n, dims 16s + 8*half + [0,8);
  // the A operands (staged reference keys) carry the factor -2.
  auto uniform_ptr = [](const void* p) RKV_INLINE {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  };
  bf16x8 bfrag[kSets][8];
  const T* krow[kSets];
#pragma unroll
  for (int c = 0; c < kSets; ++c) {
    const int64_t i = row0 + 32 * c + n;
    valid_row[c] = i < p1;
    my_last[c] = valid_row[c] ? sched_count_le((int32_t)i, sc) - 1 : -1;
    krow[c] = K + (ih * n_in + (valid_row[c] ? i - p0 : 0)) * 128 + 8 * half;
  }
  const __bf16* rk = refkey + ih * n_refs * 128;
  const float* rn = refnorm + ih * n_refs;

  // (one-wave form) slots past the last reference read the last one
  // instead: every score of such a slot is masked
  const uint32_t last_slot = (uint32_t)(n_refs - 1);
  // Cooperative staging, 512 chunks of 16 B per tile, 2 per thread, through
  // bounded buffer descriptors over this head's keys and norms: slots past
  // the last reference read zeros (every score of such a slot is masked: it
  // lies beyond every token's last candidate), the tile offset is a scalar
  // and the lane offsets are fixed, so a tile's loads take no vector address
  // arithmetic.
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(rk), 0, __builtin_amdgcn_readfirstlane((int)(n_refs * 256)), 0x00020000);
  const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(rn), 0, __builtin_amdgcn_readfirstlane((int)(n_refs * 4)), 0x00020000);
  // thread t loads chunks t and t + 256 of the tile (16 bytes each); the
  // whole offset is in the range-checked vector part
  const int kvoff = tid * 16;
  const int nvoff = (tid & 31) * 4;
  auto gload = [&](int rt, u32x4 (&v)[2], float& nv) RKV_INLINE {
    const int vo = kvoff + rt * 8192;
    v[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, vo, 0, 0));
    v[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, vo + 4096, 0, 0));
    nv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(nrs, nvoff + rt * 128, 0, 0));
  };
  auto lstore = [&](int b, const u32x4 (&v)[2], float nv) RKV_INLINE {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int chunk = tid + 256 * c;
      *reinterpret_cast<u32x4*>(&kbuf[b][chunk >> 4][(chunk & 15) * 8]) = v[c];
    }
    // (every thread stores: a branch here would let the compiler sink the
    // norm load into it, past the key loads)
    nbuf[b][tid & 31] = nv;
  };
  // The first two tiles' staging loads go out before the token keys: the
  // load counter completes in order, so the first staging store then waits
  // only for them, and the first MFMAs wait only for the key fragments they
  // use (requested in chain order: dims 16s .. 16s + 15 of both sets).
  // pa/pb: the two register sets of staged tiles in flight; pass 1 starts
  // with tiles 0 and 1 in them, and leaves pass 2's tile 0 in LDS buffer 0
  // and its tile 1 in pb (see stream)
  u32x4 pa[2], pb[2];
  float na = 0.f, nb = 0.f;
  if constexpr (!DIRECT) {
    gload(0, pa, na);
    gload(1, pb, nb);
  }
  if constexpr (sizeof(T) == 2) {
    // bf16 keys through a bounded descriptor over the range's rows: rows
    // past the range read zeros, with no branch around the loads (a branch
    // would make every later wait count conservative)
    // (the descriptor starts at the wave's first row and covers at most its
    // 64 rows, so the offsets stay small for any range length)
    const int64_t wrows = p1 - row0 < 32 * kSets ? p1 - row0 : 32 * kSets;
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(K + (ih * n_in + (active ? row0 - p0 : 0)) * 128), 0,
        __builtin_amdgcn_readfirstlane(active ? (int)wrows * 256 : 0), 0x00020000);
    int xo[kSets];
#pragma unroll
    for (int c = 0; c < kSets; ++c) xo[c] = (32 * c + n) * 256 + 16 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int c = 0; c < kSets; ++c)
        bfrag[c][s] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(xrs, xo[c] + 32 * s, 0, 0));
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int c = 0; c < kSets; ++c) bfrag[c][s] = load_key_frag(krow[c] + 16 * s, valid_row[c]);
  }

  // acc[c][r]: e = |ref|^2 - 2 k.ref of candidate slot rt*32 + acc_row(r, half)
  // for token row0 + 32c + n; +inf past the token's last candidate.
  auto tile_scores = [&](int rt, auto&& get_a, const f32x16& init, f32x16 (&acc)[kSets]) RKV_INLINE {
    {
      const bf16x8 a = get_a(0);
#pragma unroll
      for (int c = 0; c < kSets; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfrag[c][0], init, 0, 0, 0);
    }
#pragma unroll
    for (int s = 1; s < 8; ++s) {
      const bf16x8 a = get_a(s);
#pragma unroll
      for (int c = 0; c < kSets; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfrag[c][s], acc[c], 0, 0, 0);
    }
    if (rt >= full_tiles) {
      const int r0 = rt * 32 + 4 * half;
#pragma unroll
      for (int c = 0; c < kSets; ++c) {
        const int lim = my_last[c] - r0;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_row(r, 0) > lim) acc[c][r] = INFINITY;
      }
    }
  };
  // scores of the tile staged in LDS buffer b
  auto lds_scores = [&](int rt, int b, f32x16 (&acc)[kSets]) RKV_INLINE {
    f32x16 init;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 nn = *reinterpret_cast<const float4*>(&nbuf[b][8 * q4 + 4 * half]);
      init[4 * q4 + 0] = nn.x;
      init[4 * q4 + 1] = nn.y;
      init[4 * q4 + 2] = nn.z;
      init[4 * q4 + 3] = nn.w;
    }
    // all eight A fragments requested at once: one LDS round trip per tile
    bf16x8 af[8];
#pragma unroll
    for (int s_ = 0; s_ < 8; ++s_) af[s_] = *reinterpret_cast<const bf16x8*>(&kbuf[b][n][16 * s_ + 8 * half]);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads together, ahead of the chain
    tile_scores(rt, [&](int s_) RKV_INLINE { return af[s_]; }, init, acc);
  };
  // DIRECT: a tile's A operands (slot rt*32 + n, dims 16s + 8*half + [0,8))
  // and norms (rows acc_row(r, half)) straight from memory, slots past the
  // last reference clamped to it (their scores are masked)
  auto dload = [&](int rt, bf16x8 (&a)[8], f32x16& init) RKV_INLINE {
    const uint32_t slot = min((uint32_t)rt * 32 + (uint32_t)n, last_slot);
#pragma unroll
    for (int s_ = 0; s_ < 8; ++s_)
      a[s_] = *reinterpret_cast<const bf16x8*>(rk + slot * 128 + 16 * s_ + 8 * half);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      init[r] = rn[min((uint32_t)rt * 32 + (uint32_t)acc_row(r, half), last_slot)];
  };
  // Streams every candidate tile of the block through LDS; `epi(rt, acc)`
  // consumes this wave's scores of tile rt.  Global loads run two tiles
  // ahead: tile rt + 2 is requested while tile rt is scored, and tile rt + 1
  // (requested one iteration earlier) is written to the free LDS buffer
  // after it.  The loop is unrolled by two so the two register sets of tiles
  // in flight alternate without copies.  Loads and stores are unconditional
  // (tiles past the block's last read clamped slots and are never scored):
  // with no branch around them the load counter waits only for the older
  // tile, and the newer load stays in flight across the scoring.
  auto stream = [&](auto&& epi, bool pre) RKV_INLINE {
    if constexpr (DIRECT) {
      // one wave: its own tiles, the next one's operands in flight (two
      // register sets alternate)
      bf16x8 a0[8], a1[8];
      f32x16 i0, i1;
      dload(0, a0, i0);
      for (int rt = 0; rt < ntile; rt += 2) {
        dload(rt + 1, a1, i1);
        {
          f32x16 acc[kSets];
          tile_scores(rt, [&](int s_) RKV_INLINE { return a0[s_]; }, i0, acc);
          epi(rt, acc);
        }
        if (rt + 1 >= ntile) break;
        dload(rt + 2, a0, i0);
        {
          f32x16 acc[kSets];
          tile_scores(rt + 1, [&](int s_) RKV_INLINE { return a1[s_]; }, i1, acc);
          epi(rt + 1, acc);
        }
      }
    } else {
      // Pass 1 (pre): tile 0 is in pa and tile 1 in flight in pb.  Its last
      // two loads wrap to tiles 0 and 1 again, so that at its end LDS buffer
      // 0 holds tile 0 and pb tile 1 for pass 2, which then starts at once.
      const int nt_even = (ntile_blk + 1) & ~1;
      if (pre) {
        lstore(0, pa, na);
        __syncthreads();
      }
      auto step = [&](int rt, u32x4 (&st)[2], float& sn, u32x4 (&ld)[2], float& ln) RKV_INLINE {
        int tgt = rt + 2;
        if (pre && tgt >= nt_even) tgt -= nt_even;
        gload(tgt, ld, ln);
        if (rt < ntile) {
          f32x16 acc[kSets];
          lds_scores(rt, rt & 1, acc);
          epi(rt, acc);
        }
        lstore((rt + 1) & 1, st, sn);
        __syncthreads();
      };
      for (int rt = 0; rt < ntile_blk; rt += 2) {
        step(rt, pb, nb, pa, na);
        step(rt + 1, pa, na, pb, nb);
      }
    }
  };

  // ---- pass 1: bucket minima -> tau per token
  float bk[kSets][16];
#pragma unroll
  for (int c = 0; c < kSets; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) bk[c][r] = INFINITY;
  stream([&](int, const f32x16 (&acc)[kSets]) RKV_INLINE {
#pragma unroll
    for (int c = 0; c < kSets; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) bk[c][r] = fminf(bk[c][r], acc[c][r]);
  }, true);
  // one token per lane: lower lanes take set 0, upper lanes set 1, each with
  // the 16 bucket minima of both of its lanes
  static_assert(kSets == 2, "the half swap pairs two token sets");
  float tau[kSets];
  {
    float top[KM];
#pragma unroll
    for (int t = 0; t < KM; ++t) top[t] = INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const HalfPair m = half_swap(__float_as_uint(bk[0][r]), __float_as_uint(bk[1][r]));
      topk_insert(top, __uint_as_float(m.a));
      topk_insert(top, __uint_as_float(m.b));
    }
    float t = topk_get(top, k);
    if (!(t < INFINITY)) t = FLT_MAX;
    // back to every lane: tau of set 0 from the lower lane, set 1 from the upper
    const HalfPair tt = half_swap(__float_as_uint(t), __float_as_uint(t));
    tau[0] = __uint_as_float(tt.a);
    tau[1] = __uint_as_float(tt.b);
  }

  // ---- pass 2: collect candidates <= tau
  // ends[c]: the end of list c; a survivor moves it by one entry (compare,
  // select, add per candidate)
  LaneList<SPLIT> ends[kSets];
#pragma unroll
  for (int c = 0; c < kSets; ++c) ends[c] = list_of(w, c, lane);
  stream([&](int rt, const f32x16 (&acc)[kSets]) RKV_INLINE {
    const uint32_t r0 = (uint32_t)rt * 32 + 4 * half;
#pragma unroll
    for (int h = 0; h < 16 / kCheckRows; ++h) {
#pragma unroll
      for (int c = 0; c < kSets; ++c) {
#pragma unroll
        for (int r = kCheckRows * h; r < kCheckRows * h + kCheckRows; ++r) {
          // at most CAP - 1 entries here: at most kCheckRows - 1 appends
          // since the last check left at most CAP - kCheckRows
          ends[c].put(0, __float_as_uint(acc[c][r]), r0 + (uint32_t)acc_row(r, 0));
          const int inc = acc[c][r] <= tau[c] ? 1 : 0;
          ends[c].d += inc * LaneList<SPLIT>::kD;
        }
      }
      bool full = false;
#pragma unroll
      for (int c = 0; c < kSets; ++c) full |= ends[c].d > &sbd[w][c][CAP - kCheckRows][lane];
      if (__any(full)) {
#pragma unroll
        for (int c = 0; c < kSets; ++c) {
          const LaneList<SPLIT> bl = list_of(w, c, lane);
          int cnt = (int)(ends[c].d - bl.d) / LaneList<SPLIT>::kD;
          lane_compact<KM, CAP>(bl, cnt, tau[c], k);
          ends[c].d = bl.d + cnt * LaneList<SPLIT>::kD;
        }
      }
    }
  }, false);
  int cnt[kSets];
#pragma unroll
  for (int c = 0; c < kSets; ++c) cnt[c] = (int)(ends[c].d - &sbd[w][c][0][lane]) / LaneList<SPLIT>::kD;
  if (!active) return;

  // ---- final: one token per lane (set `half`, column n) from the lists of
  //      lanes n and n + 32 of that set
  {
    const HalfPair cp = half_swap((uint32_t)cnt[0], (uint32_t)cnt[1]);
    const int c = half;
    const int last = c ? my_last[1] : my_last[0];
    const int keff = (last + 1 < k) ? last + 1 : k;
    float sel[KM];
    token_select<KM, CAP>(list_of(w, c, n), (int)cp.a, list_of(w, c, n + 32), (int)cp.b,
                          keff < 1 ? 1 : keff, sel);
    if (c ? valid_row[1] : valid_row[0]) {
      uint16_t* orow = idx_out + (ih * N + row0 + 32 * c + n) * k;
      if (k == KM) {
        // the whole row as 16-byte words (rows are 2k-byte aligned)
        uint32_t wv[KM / 2];
#pragma unroll
        for (int t = 0; t < KM / 2; ++t)
          wv[t] = (uint32_t)sel[2 * t] | ((uint32_t)sel[2 * t + 1] << 16);
        if constexpr (KM == 4) {
          *reinterpret_cast<uint2*>(orow) = make_uint2(wv[0], wv[1]);
        } else {
#pragma unroll
          for (int t = 0; t < KM / 8; ++t)
            reinterpret_cast<uint4*>(orow)[t] =
                make_uint4(wv[4 * t], wv[4 * t + 1], wv[4 * t + 2], wv[4 * t + 3]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < KM; ++t)
          if (t < k) orow[t] = (uint16_t)sel[t];
      }
    }
  }
}

// ------------------------------------------------------------------ launchers

template <typename T>
hipError_t launch_refstore_t(const void* K, const void* V, void* ref_kv, uint16_t* ref_scales,
                             int ref_bits, int group, void* refkey,
                             float* refnorm, int64_t n_inst, int H, int64_t p0, int64_t n_in,
                             int64_t n_refs, Sched sc, hipStream_t st) {
  const int64_t s0 = sched_count((int32_t)p0, sc);
  const int64_t ns = sched_count((int32_t)(p0 + n_in), sc) - s0;
  const int64_t total = n_inst * H * ns;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 3) / 4;
  hipLaunchKernelGGL(k_refstore<T>, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const T*)K, (const T*)V, ref_kv, ref_scales, ref_bits, group,
                     (__bf16*)refkey, refnorm, n_in, p0, n_refs, s0, ns, sc, total);
  return hipGetLastError();
}

hipError_t launch_refstore(int dtype, const void* K, const void* V, void* ref_kv,
                           uint16_t* ref_scales, int ref_bits, int group,
                           void* refkey, float* refnorm, int64_t n_inst, int H,
                           int64_t p0, int64_t n_in, int64_t n_refs, Sched sc, hipStream_t st) {
  if (dtype == 0)
    return launch_refstore_t<float>(K, V, ref_kv, ref_scales, ref_bits, group, refkey, refnorm,
                                    n_inst, H, p0, n_in, n_refs, sc, st);
  return launch_refstore_t<__bf16>(K, V, ref_kv, ref_scales, ref_bits, group, refkey, refnorm,
                                   n_inst, H, p0, n_in, n_refs, sc, st);
}

// Ranges up to this many positions per head take the one-wave form.
constexpr int64_t kDirectMaxRows = 256;

template <typename T, int KM>
hipError_t launch_topk_t(const void* K, const void* refkey, const float* refnorm,
                         uint16_t* idx, int64_t n_inst, int H, int64_t N, int64_t n_refs,
                         Sched sc, int k, int64_t p0, int64_t n_in, hipStream_t st) {
  if (n_in <= kDirectMaxRows) {
    const int n_blocks = (int)((n_in + 32 * kSets - 1) / (32 * kSets));
    hipLaunchKernelGGL((k_dist_topk<T, KM, true>), dim3(n_blocks, H, (unsigned)n_inst),
                       dim3(64), 0, st, (const T*)K, (const __bf16*)refkey, refnorm, idx, N,
                       n_refs, sc, k, H, n_blocks, p0, n_in);
    return hipGetLastError();
  }
  const int n_blocks = (int)((n_in + kBlockRows - 1) / kBlockRows);
  hipLaunchKernelGGL((k_dist_topk<T, KM, false>), dim3(n_blocks, H, (unsigned)n_inst), dim3(256),
                     0, st, (const T*)K, (const __bf16*)refkey, refnorm, idx, N, n_refs, sc, k,
                     H, n_blocks, p0, n_in);
  return hipGetLastError();
}

hipError_t launch_dist_topk(int dtype, const void* K, const void* refkey,
                            const float* refnorm, uint16_t* idx, int64_t n_inst, int H,
                            int64_t N, int64_t n_refs, Sched sc, int k, int64_t p0,
                            int64_t n_in, hipStream_t st) {
  if (n_in == 0 || n_inst == 0) return hipSuccess;
  if (dtype == 0) {
    if (k <= 4) return launch_topk_t<float, 4>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, p0, n_in, st);
    if (k <= 8) return launch_topk_t<float, 8>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, p0, n_in, st);
    return launch_topk_t<float, 16>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, p0, n_in, st);
  }
  if (k <= 4) return launch_topk_t<__bf16, 4>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, p0, n_in, st);
  if (k <= 8) return launch_topk_t<__bf16, 8>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, p0, n_in, st);
  return launch_topk_t<__bf16, 16>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, p0, n_in, st);
}

}  // namespace rkv
