// Shared device helpers for the gfx950 kernels: bf16 conversion, MFMA vector
// types, wave/block scans, order-preserving float keys, XCD-aware work mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

namespace fsa {

// Debug builds (-DFSA_DEBUG_BOUNDS) record inputs that release builds skip
// silently: each translation unit that includes this header owns one device
// word of flag bits (FSA_DBG_* in fsa.h), raised with a device-scope atomic
// OR where a bad list entry, index or page id is met, and read back on the
// host through debug_flags_of_tu().  Release builds compile the checks out.
#ifdef FSA_DEBUG_BOUNDS
static __device__ uint32_t g_debug_flags;
#define FSA_DEBUG_RAISE(cond, bit)                                       \
  do {                                                                   \
    if (cond) __hip_atomic_fetch_or(&::fsa::g_debug_flags, (uint32_t)(bit), \
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); \
  } while (0)
#else
#define FSA_DEBUG_RAISE(cond, bit) \
  do {                             \
  } while (0)
#endif

// host: this translation unit's flags (0 in a release build), cleared if asked
static inline hipError_t debug_flags_of_tu(uint32_t* flags, bool clear) {
#ifdef FSA_DEBUG_BOUNDS
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_debug_flags), sizeof(uint32_t));
  if (e != hipSuccess || !clear) return e;
  const uint32_t zero = 0u;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &zero, sizeof(uint32_t));
#else
  (void)clear;
  *flags = 0u;
  return hipSuccess;
#endif
}

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

// op over the 64 lanes of a wave, the result in every lane: the row_shr /
// row_bcast ladder of wave_incl_scan (below) with `ident` for lanes that a
// move gives no source, then lane 63 (which has seen every lane) read into
// a scalar.  32-bit T only.
template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce(T v, T ident, Op op) {
  static_assert(sizeof(T) == 4, "32-bit lanes");
  const int id = __builtin_bit_cast(int, ident);
#define FSA_DPP_STEP(CTRL, ROWS)                                                              \
  v = op(v, __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, v), \
                                                              CTRL, ROWS, 0xf, false)))
  FSA_DPP_STEP(0x111, 0xf);  // row_shr:1
  FSA_DPP_STEP(0x112, 0xf);  // row_shr:2
  FSA_DPP_STEP(0x114, 0xf);  // row_shr:4
  FSA_DPP_STEP(0x118, 0xf);  // row_shr:8
  FSA_DPP_STEP(0x142, 0xa);  // row_bcast:15
  FSA_DPP_STEP(0x143, 0xc);  // row_bcast:31
#undef FSA_DPP_STEP
  return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_allreduce(v, T(0), [](T a, T b) { return a + b; });
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_allreduce(v, -INFINITY, [](float a, float b) { return fmaxf(a, b); });
}

// x at this lane and at lane l ^ OFF (OFF = 8, 16 or 32), as two values whose
// order may differ between the two lanes, so callers combine them
// symmetrically: v_permlane32_swap / v_permlane16_swap exchange half-waves
// or 16-lane rows, and DPP row_ror:8 rotates a 16-lane row by 8.
template <int OFF>
__device__ __forceinline__ void xor_pair(float x, float& a, float& b) {
  const uint32_t u = __float_as_uint(x);
  if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    static_assert(OFF == 8, "lane distance 8, 16 or 32");
    a = x;
    b = __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xf, 0xf, false));
  }
}

// Inclusive prefix sum over the 64 lanes of a wave, in DPP lane moves (no
// LDS round trip per step, as a __shfl_up ladder takes): a Hillis-Steele
// scan inside each row of 16 lanes (row_shr 1, 2, 4, 8; lanes without a
// source add 0), then each row's total carried forward: lane 15 into row 1
// and lane 47 into row 3 (row_bcast:15), lane 31 into rows 2 and 3
// (row_bcast:31).  Rows a move leaves out keep their value.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix sum over the whole workgroup (blockDim.x a multiple of 64,
// at most 1024).  `tmp` is shared scratch of >= 16 ints.  Returns the
// exclusive prefix of v; *total receives the workgroup sum.  Each wave
// publishes its total; then lanes 0..15 of every wave read the (at most 16)
// totals, one wave scan ranks them, and a wave takes the inclusive sum of
// the waves before it from lane w - 1 and the workgroup total from the last
// wave's lane: no thread walks the totals in a chain.  Contains barriers:
// every thread must call it.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6, l = lane_id();
  const int inc = wave_incl_scan(v);
  if (l == 63) tmp[w] = inc;
  __syncthreads();
  const int wsum = wave_incl_scan(l < nw ? tmp[l] : 0);  // lanes >= nw add 0
  const int before = w > 0 ? __builtin_amdgcn_readlane(wsum, w - 1) : 0;
  *total = __builtin_amdgcn_readlane(wsum, nw - 1);
  __syncthreads();  // tmp is free for the next call
  return before + inc - v;
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
