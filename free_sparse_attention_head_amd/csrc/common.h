// Shared device helpers for the gfx950 kernels: bf16 conversion, MFMA vector
// types, wave/block scans, order-preserving float keys, XCD-aware work mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;  // MI355X: 8 accelerator dies, workgroups dealt round-robin

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger
// key).  -0.0 is folded onto +0.0 first so that equal scores give equal keys.
__device__ __forceinline__ uint32_t order_key(float f) {
  f = f + 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// DPP lane moves inside a 16-lane row (bound_ctrl off, all rows/banks on).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  // old = 0 with bound_ctrl: the form the compiler folds into the consuming
  // add as a DPP operand (every lane has a valid source for these patterns)
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // reverse within each 8 lanes
constexpr int kDppMirror = 0x140;     // reverse within each 16 lanes

// Sum over aligned groups of N lanes (N = 8 or 16); every lane of the group
// receives the total.  Each step pairs lanes whose partial sums are disjoint.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16, "group size");
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  if constexpr (N == 16) v += dpp_mov<kDppMirror>(v);
  return v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 dot product of 8 bf16 pairs packed in two uint4 words (v_dot2_f32_bf16).
__device__ __forceinline__ float dot8_bf16(uint4 a, uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), acc, false);
  return acc;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o, 64);
    if (l >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over the whole workgroup (blockDim.x a multiple of 64,
// at most 1024).  `tmp` is shared scratch of >= 17 ints.  Returns the
// exclusive prefix of v; *total receives the workgroup sum.  Contains
// barriers: every thread must call it.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = wave_incl_scan(v);
  if (lane_id() == 63) tmp[w] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < nw; ++i) {
      int t = tmp[i];
      tmp[i] = run;
      run += t;
    }
    tmp[16] = run;
  }
  __syncthreads();
  int r = tmp[w] + inc - v;
  *total = tmp[16];
  __syncthreads();
  return r;
}

// Map a launch of `padded` workgroups (a multiple of kXcds) onto logical work
// items so that each accelerator die (XCD) receives one contiguous range of
// logical ids: dispatch deals workgroup w to die w % 8, so the logical id is
// (w % 8) * (padded / 8) + w / 8.  Logical ids >= total are idle.
__device__ __forceinline__ int xcd_remap(int w, int padded) {
  const int per = padded / kXcds;
  return (w % kXcds) * per + w / kXcds;
}

}  // namespace fsa
