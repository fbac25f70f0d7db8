// Internal helpers shared by the kvc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "kvc.h"

namespace kvc {

// ---------------------------------------------------------------- host side

// Record a message for kvc_last_error() and return `st`.
kvc_status fail(kvc_status st, const char* fmt, ...);
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Check the last launch; on failure record the HIP error string.
kvc_status check_launch(const char* what);

// ---------------------------------------------------------------- device side

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane index within the wave, and the count of set bits of `mask` below it.
__device__ __forceinline__ int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

__device__ __forceinline__ int popc_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ unsigned wave_sum_u(unsigned x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Inclusive prefix sum across the wave (Hillis-Steele over 64 lanes).
__device__ __forceinline__ unsigned wave_incl_scan(unsigned x) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    unsigned y = __shfl_up(x, o);
    if (l >= o) x += y;
  }
  return x;
}

// Exclusive prefix sum over the whole block. `scratch` must hold one unsigned
// per wave plus one; every thread of the block must call it. Returns the
// exclusive prefix and writes the block total to *total.
template <int kThreads>
__device__ __forceinline__ unsigned block_excl_scan(unsigned x, unsigned* scratch, unsigned* total) {
  constexpr int kWaves = kThreads / kWave;
  const int w = static_cast<int>(threadIdx.x) / kWave;
  const unsigned incl = wave_incl_scan(x);
  if (lane_id() == kWave - 1) scratch[w] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned run = 0;
    for (int i = 0; i < kWaves; ++i) {
      unsigned t = scratch[i];
      scratch[i] = run;
      run += t;
    }
    scratch[kWaves] = run;
  }
  __syncthreads();
  const unsigned res = scratch[w] + incl - x;
  *total = scratch[kWaves];
  __syncthreads();
  return res;
}

template <typename T>
struct Vec16;  // a 16-byte piece of a row as float lanes
template <>
struct Vec16<uint16_t> {
  static constexpr int kN = 8;
  __device__ static void load(const void* p, float (&x)[8]) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct Vec16<float> {
  static constexpr int kN = 4;
  __device__ static void load(const void* p, float (&x)[4]) {
    const f32x4_t u = *reinterpret_cast<const f32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = u[i];
  }
};

// (m, l) pairs of a base-2 softmax: m is a running maximum, l = sum 2^(s - m).
__device__ __forceinline__ void lse2_merge(float& m, float& l, float m2, float l2) {
  const float mm = fmaxf(m, m2);
  l = l * fast_exp2(m - mm) + l2 * fast_exp2(m2 - mm);
  m = mm;
}

}  // namespace kvc
