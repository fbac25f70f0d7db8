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
typedef __attribute__((ext_vector_type(2))) unsigned long long u64x2_t;

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

// The value x holds in lane (lane ^ K) of the wave, K a power of two below 64.
// K = 1, 2, 4, 8: DPP moves within each 16-lane row (quad permutations; row
// shifts by 4 written into alternate 4-lane banks; a row rotation by 8).
// K = 16, 32: gfx950's lane-swap instructions, which exchange one half of their
// two operands (odd rows of the first with even rows of the second, or the
// upper 32 lanes of the first with the lower 32 of the second); with x as both
// operands, the two results and x hold the partner's value and x twice, so
// their XOR is the partner's value. A few cycles each, against a round trip
// through LDS for __shfl_xor (ds_bpermute).
template <int K>
__device__ __forceinline__ unsigned lane_xor_u(unsigned x) {
  static_assert(K == 1 || K == 2 || K == 4 || K == 8 || K == 16 || K == 32, "K: a power of two below 64");
  const int v = static_cast<int>(x);
  if constexpr (K == 1) {
    return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  } else if constexpr (K == 2) {
    return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  } else if constexpr (K == 4) {
    const int t = __builtin_amdgcn_update_dpp(v, v, 0x104, 0xF, 0x5, false);            // row_shl:4, banks 0 and 2
    return static_cast<unsigned>(__builtin_amdgcn_update_dpp(t, v, 0x114, 0xF, 0xA, false));  // row_shr:4, banks 1 and 3
  } else if constexpr (K == 8) {
    return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false));  // row_ror:8
  } else if constexpr (K == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return r[0] ^ r[1] ^ x;
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return r[0] ^ r[1] ^ x;
  }
}

template <int K>
__device__ __forceinline__ float lane_xor(float x) {
  return __uint_as_float(lane_xor_u<K>(__float_as_uint(x)));
}

template <int K>
__device__ __forceinline__ unsigned long long lane_xor_u64(unsigned long long x) {
  return (static_cast<unsigned long long>(lane_xor_u<K>(static_cast<unsigned>(x >> 32))) << 32) |
         lane_xor_u<K>(static_cast<unsigned>(x));
}

// lane_xor for a stride that is a constant only once the caller's loop is
// unrolled; any other stride goes through __shfl_xor.
__device__ __forceinline__ float lane_xor_n(float x, int k) {
  switch (k) {
    case 1: return lane_xor<1>(x);
    case 2: return lane_xor<2>(x);
    case 4: return lane_xor<4>(x);
    case 8: return lane_xor<8>(x);
    case 16: return lane_xor<16>(x);
    case 32: return lane_xor<32>(x);
    default: return __shfl_xor(x, k);
  }
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, lane_xor<32>(x));
  x = fmaxf(x, lane_xor<16>(x));
  x = fmaxf(x, lane_xor<8>(x));
  x = fmaxf(x, lane_xor<4>(x));
  x = fmaxf(x, lane_xor<2>(x));
  return fmaxf(x, lane_xor<1>(x));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += lane_xor<32>(x);
  x += lane_xor<16>(x);
  x += lane_xor<8>(x);
  x += lane_xor<4>(x);
  x += lane_xor<2>(x);
  return x + lane_xor<1>(x);
}

__device__ __forceinline__ unsigned wave_sum_u(unsigned x) {
  x += lane_xor_u<32>(x);
  x += lane_xor_u<16>(x);
  x += lane_xor_u<8>(x);
  x += lane_xor_u<4>(x);
  x += lane_xor_u<2>(x);
  return x + lane_xor_u<1>(x);
}

// Inclusive prefix sum across the wave: Hillis-Steele shifts within each
// 16-lane row (DPP row_shr, lanes past the row's start adding zero), then the
// row totals carried into the rows above (row_bcast:15 into rows 1 and 3,
// row_bcast:31 into rows 2 and 3).
__device__ __forceinline__ unsigned wave_incl_scan(unsigned x) {
  int v = static_cast<int>(x);
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return static_cast<unsigned>(v);
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
struct Vec16;  // a 16-byte piece of a row as float lanes (loaded with the nontemporal bit:
               // the kernels that use it stream rows they read once per call)
template <>
struct Vec16<uint16_t> {
  static constexpr int kN = 8;
  __device__ static void load(const void* p, float (&x)[8]) {
    const u32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
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
    const f32x4_t u = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
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
