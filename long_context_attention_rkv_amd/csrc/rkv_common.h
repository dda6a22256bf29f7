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

struct Sched {
  int64_t base;
  int64_t A;  // 0 = fixed stride
};

// References in [0, n).
__host__ __device__ inline int64_t sched_count(int64_t n, Sched s) {
  if (n <= 0) return 0;
  if (s.A == 0 || n <= s.A) return (n + s.base - 1) / s.base;
  int64_t c = s.A / s.base;
  const int64_t per_band = s.A / (2 * s.base);
  int64_t lo = s.A;
  int band = 1;
  for (;;) {
    const int64_t st = s.base << band;
    if (n <= 2 * lo) return c + (n - lo + st - 1) / st;
    c += per_band;
    lo *= 2;
    ++band;
  }
}

// References at positions <= i.
__host__ __device__ inline int64_t sched_count_le(int64_t i, Sched s) {
  return sched_count(i + 1, s);
}

// Position of reference `slot`.
__host__ __device__ inline int64_t sched_pos(int64_t slot, Sched s) {
  if (s.A == 0) return slot * s.base;
  const int64_t c0 = s.A / s.base;
  if (slot < c0) return slot * s.base;
  const int64_t per = s.A / (2 * s.base);
  const int64_t m = slot - c0;
  const int band = (int)(m / per) + 1;
  return (s.A << (band - 1)) + (m % per) * (s.base << band);
}

// Slot of position i if it is a reference, else -1.
__host__ __device__ inline int64_t sched_slot(int64_t i, Sched s) {
  if (s.A == 0 || i < s.A) return (i % s.base == 0) ? i / s.base : -1;
  int64_t lo = s.A;
  int band = 1;
  while (i >= 2 * lo) {
    lo *= 2;
    ++band;
  }
  const int64_t st = s.base << band;
  if ((i - lo) % st != 0) return -1;
  return s.A / s.base + (band - 1) * (s.A / (2 * s.base)) + (i - lo) / st;
}

// ---------------------------------------------------------------- numbers

__device__ inline float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

}  // namespace rkv
