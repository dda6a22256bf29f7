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
//           candidates <= tau to a per-lane LDS list (about k per row);
//   final   one lane per row takes the k smallest of the two lists of the
//           row by (distance, slot), lowest slot first on ties.
#include <float.h>

#include "rkv_common.h"

namespace rkv {

// ------------------------------------------------------------------ refstore
// One wave per reference: copies its K and V rows into the cache's reference
// store, writes the bf16-rounded key and its squared norm to the workspace.
template <typename T>
__global__ __launch_bounds__(256) void k_refstore(
    const T* __restrict__ K, const T* __restrict__ V, T* __restrict__ ref_kv,
    __bf16* __restrict__ refkey, float* __restrict__ refnorm, int64_t N,
    int64_t n_refs, Sched sc, int64_t total_refs) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= total_refs) return;
  const int64_t ih = r / n_refs;
  const int64_t slot = r - ih * n_refs;
  const int64_t pos = sched_pos((int32_t)slot, sc);
  const T* kr = K + (ih * N + pos) * 128;
  const T* vr = V + (ih * N + pos) * 128;
  T* dk = ref_kv + ((ih * 2 + 0) * n_refs + slot) * 128;
  T* dv = ref_kv + ((ih * 2 + 1) * n_refs + slot) * 128;
  const int t = lane * 2;
  dk[t] = kr[t];
  dk[t + 1] = kr[t + 1];
  dv[t] = vr[t];
  dv[t + 1] = vr[t + 1];
  const __bf16 b0 = (__bf16)(float)kr[t];
  const __bf16 b1 = (__bf16)(float)kr[t + 1];
  refkey[r * 128 + t] = b0;
  refkey[r * 128 + t + 1] = b1;
  double s = (double)(float)b0 * (double)(float)b0 + (double)(float)b1 * (double)(float)b1;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) refnorm[r] = (float)s;
}

// ------------------------------------------------------------------ top-k
template <int KM>
__device__ inline void topk_insert(float (&top)[KM], float v) {
#pragma unroll
  for (int t = KM - 1; t > 0; --t) top[t] = __builtin_amdgcn_fmed3f(top[t - 1], v, top[t]);
  top[0] = fminf(top[0], v);
}

template <int KM>
__device__ inline float topk_get(const float (&top)[KM], int k) {
  float r = top[0];
#pragma unroll
  for (int t = 1; t < KM; ++t) r = (t == k - 1) ? top[t] : r;
  return r;
}

constexpr int kSurv = 32;  // survivor list capacity per lane

// Row of accumulator register r of a 32x32 MFMA tile for lane half `half`.
__device__ inline int acc_row(int r, int half) { return (r & 3) + 8 * (r >> 2) + 4 * half; }

// Keep this lane's own k best (distance, slot) entries; lists stay in slot
// order.  Lowers tau to the lane's k-th value.
template <int KM>
__device__ void lane_compact(float* be, uint16_t* bj, int& cnt, float& tau, int k) {
  if (cnt <= k) return;
  float top[KM];
#pragma unroll
  for (int t = 0; t < KM; ++t) top[t] = INFINITY;
  for (int c = 0; c < cnt; ++c) topk_insert(top, be[c * 64]);
  const float t = topk_get(top, k);
  int nless = 0;
  for (int c = 0; c < cnt; ++c) nless += be[c * 64] < t;
  int quota = k - nless;
  int out = 0;
  for (int c = 0; c < cnt; ++c) {
    const float e = be[c * 64];
    bool take = e < t;
    if (e == t && quota > 0) {
      take = true;
      --quota;
    }
    if (take) {
      be[out * 64] = e;
      bj[out * 64] = bj[c * 64];
      ++out;
    }
  }
  cnt = out;
  tau = fminf(tau, t);
}

template <typename T>
__device__ inline bf16x8 load_key_frag(const T* p, bool valid) {
  float x[8];
  if (valid) {
    load8(p, x);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
  }
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float r = (float)(__bf16)x[e];  // RNE to bf16 (identity for bf16 input)
    b[e] = (__bf16)(-2.0f * r);           // exact
  }
  return b;
}

// One block = 4 waves x 32 tokens of one (instance, head).  Blocks are
// issued from the end of the sequence (most candidates) backwards.  Tiles of
// 32 reference keys (+ norms) are staged in LDS, double-buffered and loaded
// one tile ahead by the whole block; each wave reads its A operands from LDS.
constexpr int kRowPad = 136;  // bf16 per staged key row: 128 + 8 (bank spread)

template <typename T, int KM>
__global__ __launch_bounds__(256, 2) void k_dist_topk(
    const T* __restrict__ K, const __bf16* __restrict__ refkey,
    const float* __restrict__ refnorm, uint16_t* __restrict__ idx_out, int64_t N,
    int64_t n_refs, Sched sc, int k, int H, int n_tiles) {
  __shared__ float sb_e[4][kSurv][64];
  __shared__ uint16_t sb_j[4][kSurv][64];
  __shared__ __attribute__((aligned(16))) __bf16 kbuf[2][32][kRowPad];
  __shared__ __attribute__((aligned(16))) float nbuf[2][32];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int tile = n_tiles - 1 - (int)blockIdx.x;
  const int64_t ih = (int64_t)blockIdx.z * H + blockIdx.y;
  const int64_t blk0 = (int64_t)tile * 128;
  const int64_t row0 = blk0 + w * 32;
  const bool active = row0 < N;
  const int n = lane & 31;
  const int half = lane >> 5;
  const int64_t i = row0 + n;
  const bool valid_row = i < N;
  const int64_t blk_last = (blk0 + 127 < N) ? blk0 + 127 : N - 1;
  const int ntile_blk = (int)((sched_count_le((int32_t)blk_last, sc) + 31) / 32);
  const int64_t last_row = (row0 + 31 < N) ? row0 + 31 : N - 1;
  const int ntile = active ? (int)((sched_count_le((int32_t)last_row, sc) + 31) / 32) : 0;
  const int full_tiles = active ? (int)(sched_count_le((int32_t)row0, sc) / 32) : 0;
  const int64_t my_last = valid_row ? sched_count_le((int32_t)i, sc) - 1 : -1;

  // B operand: -2 * bf16(key) of this lane's token, dims 16s + 8*half + [0,8).
  bf16x8 bfrag[8];
  {
    const T* krow = K + (ih * N + (valid_row ? i : 0)) * 128 + 8 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) bfrag[s] = load_key_frag(krow + 16 * s, valid_row);
  }
  const __bf16* rk = refkey + ih * n_refs * 128;
  const float* rn = refnorm + ih * n_refs;

  // cooperative staging: 512 chunks of 16 B per tile, 2 per thread
  auto gload = [&](int rt, uint4 (&v)[2], float& nv) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int chunk = tid + 256 * c;
      const int64_t slot = (int64_t)rt * 32 + (chunk >> 4);
      v[c] = slot < n_refs ? *reinterpret_cast<const uint4*>(rk + slot * 128 + (chunk & 15) * 8)
                           : make_uint4(0, 0, 0, 0);
    }
    if (tid < 32) {
      const int64_t slot = (int64_t)rt * 32 + tid;
      nv = slot < n_refs ? rn[slot] : 0.f;
    }
  };
  auto lstore = [&](int b, const uint4 (&v)[2], float nv) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int chunk = tid + 256 * c;
      *reinterpret_cast<uint4*>(&kbuf[b][chunk >> 4][(chunk & 15) * 8]) = v[c];
    }
    if (tid < 32) nbuf[b][tid] = nv;
  };
  auto tile_scores = [&](int rt, int b, f32x16& acc) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 nn = *reinterpret_cast<const float4*>(&nbuf[b][8 * q4 + 4 * half]);
      acc[4 * q4 + 0] = nn.x;
      acc[4 * q4 + 1] = nn.y;
      acc[4 * q4 + 2] = nn.z;
      acc[4 * q4 + 3] = nn.w;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&kbuf[b][n][16 * s + 8 * half]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfrag[s], acc, 0, 0, 0);
    }
    if (rt >= full_tiles) {
      const int r0 = rt * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int sl = r0 + acc_row(r, half);
        if (sl > my_last) acc[r] = INFINITY;
      }
    }
  };
  // Streams every candidate tile of the block through LDS; `epi(rt, acc)`
  // consumes this wave's scores of tile rt.
  auto stream = [&](auto&& epi) {
    uint4 pre[2];
    float pn = 0.f;
    gload(0, pre, pn);
    lstore(0, pre, pn);
    __syncthreads();
    for (int rt = 0; rt < ntile_blk; ++rt) {
      const bool more = rt + 1 < ntile_blk;
      if (more) gload(rt + 1, pre, pn);
      if (rt < ntile) {
        f32x16 acc;
        tile_scores(rt, rt & 1, acc);
        epi(rt, acc);
      }
      if (more) lstore((rt + 1) & 1, pre, pn);
      __syncthreads();
    }
  };

  // ---- pass 1: bucket minima -> tau
  float bk[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) bk[r] = INFINITY;
  stream([&](int, const f32x16& acc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) bk[r] = fminf(bk[r], acc[r]);
  });
  float tau;
  {
    float top[KM];
#pragma unroll
    for (int t = 0; t < KM; ++t) top[t] = INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      topk_insert(top, bk[r]);
      topk_insert(top, __shfl_xor(bk[r], 32));
    }
    tau = topk_get(top, k);
    if (!(tau < INFINITY)) tau = FLT_MAX;
  }

  // ---- pass 2: collect candidates <= tau
  float* be = &sb_e[w][0][lane];
  uint16_t* bj = &sb_j[w][0][lane];
  int cnt = 0;
  stream([&](int rt, const f32x16& acc) {
    const int r0 = rt * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (acc[r] <= tau) {
        be[cnt * 64] = acc[r];
        bj[cnt * 64] = (uint16_t)(r0 + acc_row(r, half));
        ++cnt;
      }
    }
    if (__any(cnt > kSurv - 16)) lane_compact<KM>(be, bj, cnt, tau, k);
  });
  if (!active) return;

  // ---- final: merge the row's two lists (this lane and lane ^ 32)
  const int cnt_b = __shfl_xor(cnt, 32);
  if (half != 0 || !valid_row) return;
  const float* pe = &sb_e[w][0][lane + 32];
  const uint16_t* pj = &sb_j[w][0][lane + 32];
  const int keff = (int)((my_last + 1 < k) ? my_last + 1 : k);
  float top[KM];
#pragma unroll
  for (int t = 0; t < KM; ++t) top[t] = INFINITY;
  for (int c = 0; c < cnt; ++c) topk_insert(top, be[c * 64]);
  for (int c = 0; c < cnt_b; ++c) topk_insert(top, pe[c * 64]);
  const float t = topk_get(top, keff);
  int nless = 0;
  for (int c = 0; c < cnt; ++c) nless += be[c * 64] < t;
  for (int c = 0; c < cnt_b; ++c) nless += pe[c * 64] < t;
  int quota = keff - nless;
  uint16_t* orow = idx_out + (ih * N + i) * k;
  int pos = 0, ia = 0, ib = 0;
  while (ia < cnt || ib < cnt_b) {
    float e;
    uint16_t j;
    const bool from_a = ib >= cnt_b || (ia < cnt && bj[ia * 64] < pj[ib * 64]);
    if (from_a) {
      e = be[ia * 64];
      j = bj[ia * 64];
      ++ia;
    } else {
      e = pe[ib * 64];
      j = pj[ib * 64];
      ++ib;
    }
    bool take = e < t;
    if (e == t && quota > 0) {
      take = true;
      --quota;
    }
    if (take && pos < keff) orow[pos++] = j;
  }
  for (; pos < k; ++pos) orow[pos] = 0xFFFF;
}

// ------------------------------------------------------------------ launchers

template <typename T>
hipError_t launch_refstore_t(const void* K, const void* V, void* ref_kv, void* refkey,
                             float* refnorm, int64_t n_inst, int H, int64_t N,
                             int64_t n_refs, Sched sc, hipStream_t st) {
  const int64_t total = n_inst * H * n_refs;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 3) / 4;
  hipLaunchKernelGGL(k_refstore<T>, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const T*)K, (const T*)V, (T*)ref_kv, (__bf16*)refkey, refnorm, N,
                     n_refs, sc, total);
  return hipGetLastError();
}

hipError_t launch_refstore(int dtype, const void* K, const void* V, void* ref_kv,
                           void* refkey, float* refnorm, int64_t n_inst, int H,
                           int64_t N, int64_t n_refs, Sched sc, hipStream_t st) {
  if (dtype == 0)
    return launch_refstore_t<float>(K, V, ref_kv, refkey, refnorm, n_inst, H, N, n_refs, sc, st);
  return launch_refstore_t<__bf16>(K, V, ref_kv, refkey, refnorm, n_inst, H, N, n_refs, sc, st);
}

template <typename T, int KM>
hipError_t launch_topk_t(const void* K, const void* refkey, const float* refnorm,
                         uint16_t* idx, int64_t n_inst, int H, int64_t N, int64_t n_refs,
                         Sched sc, int k, hipStream_t st) {
  const int n_tiles = (int)((N + 127) / 128);
  hipLaunchKernelGGL((k_dist_topk<T, KM>), dim3(n_tiles, H, (unsigned)n_inst), dim3(256), 0,
                     st, (const T*)K, (const __bf16*)refkey, refnorm, idx, N, n_refs, sc, k,
                     H, n_tiles);
  return hipGetLastError();
}

hipError_t launch_dist_topk(int dtype, const void* K, const void* refkey,
                            const float* refnorm, uint16_t* idx, int64_t n_inst, int H,
                            int64_t N, int64_t n_refs, Sched sc, int k, hipStream_t st) {
  if (N == 0 || n_inst == 0) return hipSuccess;
  if (dtype == 0) {
    if (k <= 4) return launch_topk_t<float, 4>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, st);
    if (k <= 8) return launch_topk_t<float, 8>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, st);
    return launch_topk_t<float, 16>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, st);
  }
  if (k <= 4) return launch_topk_t<__bf16, 4>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, st);
  if (k <= 8) return launch_topk_t<__bf16, 8>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, st);
  return launch_topk_t<__bf16, 16>(K, refkey, refnorm, idx, n_inst, H, N, n_refs, sc, k, st);
}

}  // namespace rkv
