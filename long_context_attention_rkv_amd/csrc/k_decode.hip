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
//   k_qk_table  QK[inst][hq][slot] in fp32.
//   k_decode    one wave per (instance, KV head, split of the sequence):
//               streams the codes of its positions; q.codes and P.codes on
//               16x16x32 f16 MFMAs (codes are exact small integers in f16),
//               scales applied in fp32, online softmax per query head,
//               W accumulated in LDS.  Writes (m, l, O, W) per query head.
//   k_combine   merges the splits and adds W . Vref.
#include <float.h>

#include "rkv_common.h"

namespace rkv {

// ------------------------------------------------------------------ QK table
template <typename T>
__global__ __launch_bounds__(256) void k_qk_table(const T* __restrict__ q,
                                                  const T* __restrict__ ref_kv,
                                                  float* __restrict__ qk, int G, int H,
                                                  int64_t n_refs) {
  __shared__ float qs[16][128];
  const int kvh = blockIdx.x;
  const int64_t inst = blockIdx.y;
  const int hq0 = kvh * G;
  const int Hq = H * G;
  for (int e = threadIdx.x; e < G * 128; e += 256)
    qs[e / 128][e % 128] = (float)q[(inst * Hq + hq0) * 128 + e];
  __syncthreads();
  const T* kref = ref_kv + ((inst * H + kvh) * 2 + 0) * n_refs * 128;
  for (int64_t j = threadIdx.x; j < n_refs; j += 256) {
    float acc[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) acc[h] = 0.f;
    for (int t = 0; t < 128; t += 8) {
      float x[8];
      load8(kref + j * 128 + t, x);
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        if (h < G) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h] = __builtin_fmaf(qs[h][t + e], x[e], acc[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 16; ++h)
      if (h < G) qk[(inst * Hq + hq0 + h) * n_refs + j] = acc[h];
  }
}

// ------------------------------------------------------------------ codes
// Decode 8 codes of one lane into an f16x8 MFMA operand.  The element order
// is a fixed permutation of the 8 code positions (perm_of<BITS>); the other
// operand is built in the same order.
template <int BITS>
__device__ inline int perm_of(int e) {
  if constexpr (BITS == 8) {
    constexpr int p[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    return p[e];
  } else {
    constexpr int p[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    return p[e];
  }
}

__device__ inline f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

template <int BITS>
__device__ inline f16x8 decode_codes(uint32_t w0, uint32_t w1) {
  f16x2 p[4];
  if constexpr (BITS == 4) {
    const uint32_t t = w0 ^ 0x88888888u;  // two's complement -> offset binary
    const f16x2 off = {(_Float16)-1032.f, (_Float16)-1032.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = as_h2(((t >> (4 * j)) & 0x000F000Fu) | 0x64006400u) + off;
  } else if constexpr (BITS == 8) {
    const uint32_t t0 = w0 ^ 0x80808080u, t1 = w1 ^ 0x80808080u;
    const f16x2 off = {(_Float16)-1152.f, (_Float16)-1152.f};
    p[0] = as_h2((t0 & 0x00FF00FFu) | 0x64006400u) + off;
    p[1] = as_h2(((t0 >> 8) & 0x00FF00FFu) | 0x64006400u) + off;
    p[2] = as_h2((t1 & 0x00FF00FFu) | 0x64006400u) + off;
    p[3] = as_h2(((t1 >> 8) & 0x00FF00FFu) | 0x64006400u) + off;
  } else {
    const uint32_t t = (w0 ^ 0xAAAAu) & 0xFFFFu;
    const uint32_t u = (t & 0xFFu) | ((t & 0xFF00u) << 8);
    const f16x2 off = {(_Float16)-1026.f, (_Float16)-1026.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = as_h2(((u >> (2 * j)) & 0x00030003u) | 0x64006400u) + off;
  }
  f16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[2 * j] = p[j][0];
    r[2 * j + 1] = p[j][1];
  }
  return r;
}

// Load the BITS bytes of 8 consecutive codes starting at byte p.
template <int BITS>
__device__ inline void load_code_words(const uint8_t* p, uint32_t& w0, uint32_t& w1) {
  if constexpr (BITS == 4) {
    w0 = *reinterpret_cast<const uint32_t*>(p);
    w1 = 0;
  } else if constexpr (BITS == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w0 = v.x;
    w1 = v.y;
  } else {
    w0 = *reinterpret_cast<const uint16_t*>(p);
    w1 = 0;
  }
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

constexpr int kDecTile = 32;

// Partial record per (instance, query head, split): m, l, 2 pad, O[128], W[nrp].
__host__ __device__ inline int64_t part_rec_floats(int64_t n_refs) {
  return 132 + ((n_refs + 3) / 4) * 4;
}

template <typename T, int BITS, int NG>
__global__ __launch_bounds__(64) void k_decode(
    const T* __restrict__ q, const uint16_t* __restrict__ idx, const uint8_t* __restrict__ codes_k,
    const uint8_t* __restrict__ codes_v, const uint16_t* __restrict__ scales,
    const float* __restrict__ qk, float* __restrict__ part, float alpha, int64_t N,
    int64_t n_refs, Sched sc, int k, int G, int H, int n_split) {
  constexpr int HPL = 4 / NG;  // query heads per lane in the score layout
  constexpr int GS = 128 / NG;  // group size
  extern __shared__ float lds[];
  const int64_t nrp = ((n_refs + 3) / 4) * 4;
  float* qk_s = lds;                 // [G][nrp]
  float* w_s = lds + G * nrp;        // [G][nrp]
  float* pst = w_s + G * nrp;        // [16][kDecTile]
  float* sst = pst + 16 * kDecTile;  // [NG][kDecTile]

  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int quad = lane >> 4;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int64_t inst = blockIdx.z;
  const int64_t ih = inst * H + kvh;
  const int Hq = H * G;
  const int64_t tiles = (N + kDecTile - 1) / kDecTile;
  const int64_t tps = (tiles + n_split - 1) / n_split;
  const int64_t t0 = split * tps;
  const int64_t t1 = (t0 + tps < tiles) ? t0 + tps : tiles;

  // ---- stage the QK table, clear W and the P staging
  const float* qk_g = qk + (inst * Hq + kvh * G) * n_refs;
  for (int64_t e = lane; e < (int64_t)G * nrp; e += 64) {
    const int64_t h = e / nrp, j = e - h * nrp;
    qk_s[e] = j < n_refs ? qk_g[h * n_refs + j] : 0.f;
    w_s[e] = 0.f;
  }
  for (int e = lane; e < 16 * kDecTile; e += 64) pst[e] = 0.f;

  // ---- A operand of the score MFMA: rows (h, g), dims of step s in lane order
  f16x8 aq[4];
  {
    const int m = n;  // row
    const int h = m / NG, g = m % NG;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dim = 32 * s + 8 * quad + perm_of<BITS>(e);
        float v = 0.f;
        if (h < G && dim / GS == g) v = (float)q[(inst * Hq + kvh * G + h) * 128 + dim];
        aq[s][e] = (_Float16)v;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();

  float m_mine[HPL], l_mine[HPL];
#pragma unroll
  for (int hh = 0; hh < HPL; ++hh) {
    m_mine[hh] = -INFINITY;
    l_mine[hh] = 0.f;
  }
  f32x4 o[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint8_t* ck = codes_k + ih * N * (16 * BITS);
  const uint16_t* sc16 = scales + ih * N * 2 * NG;
  const uint16_t* ix = idx + ih * N * k;
  const uint8_t* cv = codes_v + ih * tiles * 128 * (4 * BITS);
  const int h0 = quad * HPL;

  for (int64_t t = t0; t < t1; ++t) {
    const int64_t tb = t * kDecTile;
    float logit[2][HPL];
    int64_t slot_b[2];
    int keff_b[2];
    float sv_b[2][NG];
    // ---------------- scores of the two 16-token blocks
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t tok = tb + 16 * b + n;
      const bool valid = tok < N;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t w0 = 0, w1 = 0;
        if (valid) load_code_words<BITS>(ck + tok * (16 * BITS) + (4 * s + quad) * BITS, w0, w1);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[s], decode_codes<BITS>(w0, w1), acc, 0, 0, 0);
      }
      float sk[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        sk[g] = valid ? half_bits_to_f32(sc16[(tok * 2 + 0) * NG + g]) : 0.f;
        sv_b[b][g] = valid ? half_bits_to_f32(sc16[(tok * 2 + 1) * NG + g]) : 0.f;
      }
      const int64_t slot = valid ? sched_slot(tok, sc) : -1;
      const int keff = valid ? (int)min((int64_t)k, sched_count_le(tok, sc)) : 0;
      slot_b[b] = slot;
      keff_b[b] = keff;
      const uint16_t* irow = ix + (valid ? tok : 0) * k;
#pragma unroll
      for (int hh = 0; hh < HPL; ++hh) {
        const int h = h0 + hh;
        float lg = -INFINITY;
        if (valid && h < G) {
          const float* qrow = qk_s + h * nrp;
          float sc_ = 0.f;
          if (slot >= 0) {
            sc_ = qrow[slot];
          } else {
            float rs = 0.f;
            for (int j = 0; j < keff; ++j) rs += qrow[irow[j]];
            float res = 0.f;
#pragma unroll
            for (int g = 0; g < NG; ++g) res = __builtin_fmaf(sk[g], acc[hh * NG + g], res);
            sc_ = res + rs / (float)keff;
          }
          lg = alpha * sc_;
        }
        logit[b][hh] = lg;
      }
    }
    // ---------------- online softmax per head (this lane's heads)
    float scale_mine[HPL];
    float p[2][HPL];
#pragma unroll
    for (int hh = 0; hh < HPL; ++hh) {
      const float tm = quad_max(fmaxf(logit[0][hh], logit[1][hh]));
      const float mnew = fmaxf(m_mine[hh], tm);
      const bool live = mnew > -INFINITY;
      scale_mine[hh] = live ? __expf(m_mine[hh] - mnew) : 1.f;
      p[0][hh] = live ? __expf(logit[0][hh] - mnew) : 0.f;
      p[1][hh] = live ? __expf(logit[1][hh] - mnew) : 0.f;
      l_mine[hh] = l_mine[hh] * scale_mine[hh] + quad_sum(p[0][hh] + p[1][hh]);
      m_mine[hh] = mnew;
    }
    // rescale O (rows 4*quad + j of the PV layout) and W (this quad's heads)
    float so[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int src = 16 * min((4 * quad + j) / HPL, 3);
      so[j] = __shfl(scale_mine[j % HPL], src);
    }
    const bool any_rescale = __any(so[0] != 1.f || so[1] != 1.f || so[2] != 1.f || so[3] != 1.f);
    if (any_rescale) {
#pragma unroll
      for (int b = 0; b < 8; ++b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[b][j] *= so[j];
      }
#pragma unroll
      for (int hh = 0; hh < HPL; ++hh) {
        const int h = h0 + hh;
        if (h < G && scale_mine[hh] != 1.f) {
          for (int64_t j = n; j < n_refs; j += 16) w_s[h * nrp + j] *= scale_mine[hh];
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // ---------------- W accumulation and P staging
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t tok = tb + 16 * b + n;
      const uint16_t* irow = ix + (tok < N ? tok : 0) * k;
#pragma unroll
      for (int hh = 0; hh < HPL; ++hh) {
        const int h = h0 + hh;
        if (h < G) {
          const float pv = p[b][hh];
          float* wrow = w_s + h * nrp;
          if (slot_b[b] >= 0) {
            atomicAdd(wrow + slot_b[b], pv);
            pst[h * kDecTile + 16 * b + n] = 0.f;
          } else {
            if (keff_b[b] > 0) {
              const float pw = pv / (float)keff_b[b];
              for (int j = 0; j < keff_b[b]; ++j) atomicAdd(wrow + irow[j], pw);
            }
            pst[h * kDecTile + 16 * b + n] = pv;
          }
        }
      }
      if (quad == 0) {
#pragma unroll
        for (int g = 0; g < NG; ++g) sst[g * kDecTile + 16 * b + n] = sv_b[b][g];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    // ---------------- P.V on the MFMA, one A operand per scale group
    f16x8 ap[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tk = 8 * quad + perm_of<BITS>(e);
        ap[g][e] = (_Float16)(pst[n * kDecTile + tk] * sst[g * kDecTile + tk]);
      }
    }
    const uint8_t* cvt = cv + t * 128 * (4 * BITS);
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
      const int dim = 16 * blk + n;
      uint32_t w0, w1;
      load_code_words<BITS>(cvt + dim * (4 * BITS) + quad * BITS, w0, w1);
      o[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ap[(16 * blk) / GS], decode_codes<BITS>(w0, w1),
                                                   o[blk], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }

  // ---- write the partial record of every query head of this KV head
  const int64_t rec = part_rec_floats(n_refs);
#pragma unroll
  for (int hh = 0; hh < HPL; ++hh) {
    const int h = h0 + hh;
    if (h < G && n == 0) {
      float* r = part + ((inst * Hq + kvh * G + h) * n_split + split) * rec;
      r[0] = m_mine[hh];
      r[1] = l_mine[hh];
    }
  }
#pragma unroll
  for (int blk = 0; blk < 8; ++blk) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * quad + j;
      if (h < G) {
        float* r = part + ((inst * Hq + kvh * G + h) * n_split + split) * rec;
        r[4 + 16 * blk + n] = o[blk][j];
      }
    }
  }
  for (int64_t e = lane; e < (int64_t)G * nrp; e += 64) {
    const int64_t h = e / nrp, j = e - h * nrp;
    float* r = part + ((inst * Hq + kvh * G + h) * n_split + split) * rec;
    r[132 + j] = w_s[e];
  }
}

// ------------------------------------------------------------------ combine
template <typename T>
__global__ __launch_bounds__(128) void k_combine(const float* __restrict__ part,
                                                 const T* __restrict__ ref_kv,
                                                 float* __restrict__ out, int G, int H,
                                                 int64_t n_refs, int n_split) {
  extern __shared__ float wt[];
  const int hq = blockIdx.x;
  const int64_t inst = blockIdx.y;
  const int Hq = H * G;
  const int kvh = hq / G;
  const int t = threadIdx.x;
  const int64_t rec = part_rec_floats(n_refs);
  const float* base = part + (inst * Hq + hq) * n_split * rec;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, base[s * rec]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float ms = base[s * rec];
    const float f = ms > -INFINITY ? __expf(ms - M) : 0.f;
    l += f * base[s * rec + 1];
    o += f * base[s * rec + 4 + t];
  }
  for (int64_t j = t; j < n_refs; j += 128) {
    float w = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const float ms = base[s * rec];
      const float f = ms > -INFINITY ? __expf(ms - M) : 0.f;
      w += f * base[s * rec + 132 + j];
    }
    wt[j] = w;
  }
  __syncthreads();
  const T* vref = ref_kv + ((inst * H + kvh) * 2 + 1) * n_refs * 128;
  for (int64_t j = 0; j < n_refs; ++j) o = __builtin_fmaf(wt[j], (float)vref[j * 128 + t], o);
  out[(inst * Hq + hq) * 128 + t] = o / l;
}

// ------------------------------------------------------------------ launchers
size_t decode_ws_bytes(int64_t n_inst, int H, int n_q_heads, int n_split, int64_t n_refs) {
  const size_t qkb = (size_t)n_inst * n_q_heads * n_refs * 4;
  const size_t qka = (qkb + 255) / 256 * 256;
  const size_t pb = (size_t)n_inst * n_q_heads * n_split * part_rec_floats(n_refs) * 4;
  (void)H;
  return qka + pb;
}

template <typename T, int BITS, int NG>
hipError_t launch_decode_t(const void* q, int n_q_heads, const uint16_t* idx,
                           const void* ref_kv, const uint8_t* ck, const uint8_t* cv,
                           const uint16_t* sc16, float alpha, float* out, int n_split, void* ws,
                           int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc, int k,
                           hipStream_t st) {
  const int G = n_q_heads / H;
  float* qk = (float*)ws;
  const size_t qkb = (size_t)n_inst * n_q_heads * n_refs * 4;
  float* part = (float*)((char*)ws + (qkb + 255) / 256 * 256);
  hipLaunchKernelGGL(k_qk_table<T>, dim3(H, (unsigned)n_inst), dim3(256), 0, st, (const T*)q,
                     (const T*)ref_kv, qk, G, H, n_refs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nrp = ((n_refs + 3) / 4) * 4;
  const size_t lds = ((size_t)2 * G * nrp + 16 * kDecTile + NG * kDecTile) * 4;
  auto kern = k_decode<T, BITS, NG>;
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(n_split, H, (unsigned)n_inst), dim3(64), lds, st, (const T*)q,
                     idx, ck, cv, sc16, qk, part, alpha, N, n_refs, sc, k, G, H, n_split);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_combine<T>, dim3(n_q_heads, (unsigned)n_inst), dim3(128),
                     (size_t)nrp * 4, st, part, (const T*)ref_kv, out, G, H, n_refs, n_split);
  return hipGetLastError();
}

template <typename T, int BITS>
hipError_t launch_decode_g(int group, const void* q, int n_q_heads, const uint16_t* idx,
                           const void* ref_kv, const uint8_t* ck, const uint8_t* cv,
                           const uint16_t* sc16, float alpha, float* out, int n_split, void* ws,
                           int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc, int k,
                           hipStream_t st) {
  if (group == 32)
    return launch_decode_t<T, BITS, 4>(q, n_q_heads, idx, ref_kv, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, n_refs, sc, k, st);
  if (group == 64)
    return launch_decode_t<T, BITS, 2>(q, n_q_heads, idx, ref_kv, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, n_refs, sc, k, st);
  return launch_decode_t<T, BITS, 1>(q, n_q_heads, idx, ref_kv, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, n_refs, sc, k, st);
}

template <typename T>
hipError_t launch_decode_b(int bits, int group, const void* q, int n_q_heads, const uint16_t* idx,
                           const void* ref_kv, const uint8_t* ck, const uint8_t* cv,
                           const uint16_t* sc16, float alpha, float* out, int n_split, void* ws,
                           int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc, int k,
                           hipStream_t st) {
  if (bits == 2)
    return launch_decode_g<T, 2>(group, q, n_q_heads, idx, ref_kv, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, n_refs, sc, k, st);
  if (bits == 4)
    return launch_decode_g<T, 4>(group, q, n_q_heads, idx, ref_kv, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, n_refs, sc, k, st);
  return launch_decode_g<T, 8>(group, q, n_q_heads, idx, ref_kv, ck, cv, sc16, alpha, out, n_split, ws, n_inst, H, N, n_refs, sc, k, st);
}

hipError_t launch_decode(int dtype, int bits, const void* q, int n_q_heads, const uint16_t* idx,
                         const void* ref_kv, const uint8_t* ck, const uint8_t* cv,
                         const uint16_t* sc16, float softmax_scale, float* out, int n_split,
                         void* ws, int64_t n_inst, int H, int64_t N, int64_t n_refs, Sched sc,
                         int k, int group, hipStream_t st) {
  if (dtype == 0)
    return launch_decode_b<float>(bits, group, q, n_q_heads, idx, ref_kv, ck, cv, sc16, softmax_scale, out, n_split, ws, n_inst, H, N, n_refs, sc, k, st);
  return launch_decode_b<__bf16>(bits, group, q, n_q_heads, idx, ref_kv, ck, cv, sc16, softmax_scale, out, n_split, ws, n_inst, H, N, n_refs, sc, k, st);
}

}  // namespace rkv
