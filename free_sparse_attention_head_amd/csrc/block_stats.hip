// block_stats: per (batch, KV head, key block) centroid and radius.
//
// RBS-Attention post, "Key technical points" 1: the centroid base branch
// scores a key block by its mean key; the rescue branch uses the block's
// maximum key-to-centroid distance (radius).
//
// One workgroup of 256 threads per (b, g, j).  The block's T x D keys are read
// once from HBM with 16-byte loads (one key row is D contiguous elements, rows
// Hkv*D apart), kept in registers, reduced to the centroid through LDS, and
// then reused for the distances; the per-row distance is reduced across the
// lanes that share a row with xor-shuffles.  HBM-bound: T*D*elt bytes read,
// (D+1)*4 bytes written per block.
#include "common.h"
#include "launch.h"

namespace fsa {

template <typename TI, int D, int T>
__global__ __launch_bounds__(256) void block_stats_kernel(const TI* __restrict__ K,
                                                          float* __restrict__ cen,
                                                          float* __restrict__ rad, int S,
                                                          int Hkv, int total) {
  constexpr int VPT = 16 / sizeof(TI);  // elements per 16-byte load
  constexpr int DG = D / VPT;           // threads across one row
  constexpr int RG = 256 / DG;          // row groups
  constexpr int RPT = T / RG;           // rows per thread
  static_assert(RPT >= 1 && T % RG == 0, "block shape");
  __shared__ float part[RG][D + 1];
  __shared__ float cs[D];
  __shared__ float mx[RG];

  const int blk = xcd_remap(blockIdx.x, gridDim.x);
  if (blk >= total) return;
  const int nB = S / T;
  const int j = blk % nB;
  const int bg = blk / nB;  // b * Hkv + g
  const int g = bg % Hkv, b = bg / Hkv;
  const int t = threadIdx.x;
  const int dg = t % DG, rg = t / DG;

  float x[RPT][VPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int s = j * T + rg + r * RG;
    const TI* p = K + ((size_t)(b * (size_t)S + s) * Hkv + g) * D + dg * VPT;
    uint4 w = *reinterpret_cast<const uint4*>(p);
    if constexpr (sizeof(TI) == 2) {
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[r][2 * e] = bf16_lo(ws[e]);
        x[r][2 * e + 1] = bf16_hi(ws[e]);
      }
    } else {
      x[r][0] = __uint_as_float(w.x);
      x[r][1] = __uint_as_float(w.y);
      x[r][2] = __uint_as_float(w.z);
      x[r][3] = __uint_as_float(w.w);
    }
  }
  // centroid: per-thread partial sums over its rows, then over row groups
#pragma unroll
  for (int e = 0; e < VPT; ++e) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) s += x[r][e];
    part[rg][dg * VPT + e] = s;
  }
  __syncthreads();
  if (t < D) {
    float s = 0.f;
    for (int r = 0; r < RG; ++r) s += part[r][t];
    const float c = s / (float)T;
    cs[t] = c;
    cen[(size_t)blk * D + t] = c;
  }
  __syncthreads();
  // radius: max over rows of the squared distance, sqrt once at the end
  float best = 0.f;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    float d2 = 0.f;
#pragma unroll
    for (int e = 0; e < VPT; ++e) {
      const float dv = x[r][e] - cs[dg * VPT + e];
      d2 += dv * dv;
    }
#pragma unroll
    for (int o = DG / 2; o >= 1; o >>= 1) d2 += __shfl_xor(d2, o, 64);
    best = fmaxf(best, d2);
  }
  if (dg == 0) mx[rg] = best;
  __syncthreads();
  if (t == 0) {
    float m = 0.f;
    for (int r = 0; r < RG; ++r) m = fmaxf(m, mx[r]);
    rad[blk] = sqrtf(m);
  }
}

template <typename TI, int D, int T>
static hipError_t launch_bs(const void* k, float* c, float* r, const PrefillDims& d,
                            hipStream_t st) {
  const int total = d.B * d.Hkv * (d.S / T);
  const int padded = (total + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((block_stats_kernel<TI, D, T>), dim3(padded), dim3(256), 0, st,
                     static_cast<const TI*>(k), c, r, d.S, d.Hkv, total);
  return hipGetLastError();
}

hipError_t launch_block_stats(bool f32, const void* k, float* c, float* r, const PrefillDims& d,
                              hipStream_t st) {
#define FSA_BS(TY, DD, TT) \
  if (d.D == DD && d.T == TT) return launch_bs<TY, DD, TT>(k, c, r, d, st);
  if (f32) {
    FSA_BS(float, 64, 64) FSA_BS(float, 64, 128) FSA_BS(float, 128, 64) FSA_BS(float, 128, 128)
  } else {
    FSA_BS(uint16_t, 64, 64) FSA_BS(uint16_t, 64, 128) FSA_BS(uint16_t, 128, 64)
    FSA_BS(uint16_t, 128, 128)
  }
#undef FSA_BS
  return hipErrorInvalidValue;
}

}  // namespace fsa
