// select_blocks: RBS-style two-branch block selection and mask merge.
//
// RBS-Attention post, "Key technical points" 1-2: a centroid base branch and
// a radius rescue branch, each thresholded independently, masks merged, and
// the block-sparse attention path left unchanged.
//
// Three kernels, all stream-ordered:
//   1. pool_queries_kernel: qbar[b,h,i,:] = mean of the T query rows of block i
//      (one workgroup per (b, i): the T x Hq x D slab is contiguous in HBM and
//      read once with 16-byte loads).
//   2. centroid_score_kernel: Sc[b,h,i,j] = qbar_i . c_j for j <= i, as 128x128
//      fp32 register-blocked tiles of the lower triangle (LDS-staged operands,
//      8x8 outputs per thread, sequential accumulation over d).
//   3. select_rows_kernel: one wave per row (b,h,i): Sr = Sc + ||qbar||*r,
//      exact top-k of each branch by a radix select in 8-bit digits on
//      order-preserving keys held in registers (per-wave LDS histogram,
//      early stop once the k-th key's bin is kept whole; remaining ties go to
//      the lower block index through a wave scan of the equal-key counts),
//      union with the forced sink/band blocks, compaction into an ascending
//      block list with a wave scan, and the bitmask row.  Per-entry flags
//      are per-lane bit masks, which keeps the wave's registers to 75 VGPRs
//      and 86 SGPRs at 16 entries a lane (100 SGPRs as per-entry booleans).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace fsa {

// ---------------------------------------------------------------- pooling
template <typename TI>
__global__ __launch_bounds__(256) void pool_queries_kernel(const TI* __restrict__ Q,
                                                           float* __restrict__ qbar, int S,
                                                           int Hq, int D, int T) {
  constexpr int VPT = 16 / sizeof(TI);
  const int nB = S / T;
  const int i = blockIdx.x % nB, b = blockIdx.x / nB;
  const int NC = Hq * D / VPT;  // 16-byte column groups of one token row
  const size_t row_elems = (size_t)Hq * D;
  const TI* base = Q + ((size_t)b * S + (size_t)i * T) * row_elems;
  for (int cg = threadIdx.x; cg < NC; cg += blockDim.x) {
    float acc[VPT];
#pragma unroll
    for (int e = 0; e < VPT; ++e) acc[e] = 0.f;
    // kU row loads in flight per thread before they are summed (T is a
    // multiple of 64); the sum still runs over t in order
    constexpr int kU = 8;
    for (int t0 = 0; t0 < T; t0 += kU) {
      uint4 w[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        w[u] = *reinterpret_cast<const uint4*>(base + (size_t)(t0 + u) * row_elems + cg * VPT);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if constexpr (sizeof(TI) == 2) {
          const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += bf16_lo(ws[e]);
            acc[2 * e + 1] += bf16_hi(ws[e]);
          }
        } else {
          acc[0] += __uint_as_float(w[u].x);
          acc[1] += __uint_as_float(w[u].y);
          acc[2] += __uint_as_float(w[u].z);
          acc[3] += __uint_as_float(w[u].w);
        }
      }
    }
    const int h = (cg * VPT) / D, d0 = (cg * VPT) % D;
    float* out = qbar + (((size_t)b * Hq + h) * nB + i) * D + d0;
#pragma unroll
    for (int e = 0; e < VPT; ++e) out[e] = acc[e] / (float)T;
  }
}

// ---------------------------------------------------------------- scores
// 128x128 tiles of the lower triangle, 256 threads, 8x8 outputs a thread
// (rows ty*4 + {0..3} and 64 + ty*4 + {0..3}, columns likewise from tx): four
// 16-byte LDS reads feed 64 FMAs, half the LDS traffic per FMA of 4x4
// outputs a thread, which left the kernel waiting on LDS.  The dot products
// still accumulate over d in order, one fmaf per term.
constexpr int kTile = 128, kDc = 32;

__global__ __launch_bounds__(256) void centroid_score_kernel(const float* __restrict__ qbar,
                                                             const float* __restrict__ cen,
                                                             float* __restrict__ sc, int Hq,
                                                             int Hkv, int nB, int D, int tiles) {
  __shared__ __align__(16) float As[kDc][kTile + 4];
  __shared__ __align__(16) float Bs[kDc][kTile + 4];
  const int x = blockIdx.x % tiles, bh = blockIdx.x / tiles;
  const int h = bh % Hq, b = bh / Hq, g = h / (Hq / Hkv);
  // x -> (it, jt) with jt <= it, row-major over the lower triangle
  int it = (int)((sqrtf(8.f * x + 1.f) - 1.f) * 0.5f);
  while ((it + 1) * (it + 2) / 2 <= x) ++it;
  while (it * (it + 1) / 2 > x) --it;
  const int jt = x - it * (it + 1) / 2;
  const float* A = qbar + ((size_t)b * Hq + h) * nB * D;
  const float* Bm = cen + ((size_t)b * Hkv + g) * nB * D;
  const int t = threadIdx.x, ty = t / 16, tx = t % 16;
  float acc[2][4][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[a][r][c][e] = 0.f;
  for (int d0 = 0; d0 < D; d0 += kDc) {
    // stage 128 rows x 32 d of each operand, transposed to [d][row]: thread
    // e reads 4 consecutive d of row e/8 (eight threads cover a row's 128 B)
#pragma unroll
    for (int u = 0; u < kTile * kDc / 4 / 256; ++u) {
      const int e = t + 256 * u, r = e / (kDc / 4), d4 = e % (kDc / 4);
      const int ia = it * kTile + r, jb = jt * kTile + r;
      const float4 va = ia < nB ? *reinterpret_cast<const float4*>(A + (size_t)ia * D + d0 + 4 * d4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 vb = jb < nB ? *reinterpret_cast<const float4*>(Bm + (size_t)jb * D + d0 + 4 * d4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
      As[4 * d4 + 0][r] = va.x;
      As[4 * d4 + 1][r] = va.y;
      As[4 * d4 + 2][r] = va.z;
      As[4 * d4 + 3][r] = va.w;
      Bs[4 * d4 + 0][r] = vb.x;
      Bs[4 * d4 + 1][r] = vb.y;
      Bs[4 * d4 + 2][r] = vb.z;
      Bs[4 * d4 + 3][r] = vb.w;
    }
    __syncthreads();
#pragma unroll 4
    for (int dd = 0; dd < kDc; ++dd) {
      float av[2][4], bv[2][4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const float4 a4 = *reinterpret_cast<const float4*>(&As[dd][64 * h2 + ty * 4]);
        const float4 b4 = *reinterpret_cast<const float4*>(&Bs[dd][64 * h2 + tx * 4]);
        av[h2][0] = a4.x, av[h2][1] = a4.y, av[h2][2] = a4.z, av[h2][3] = a4.w;
        bv[h2][0] = b4.x, bv[h2][1] = b4.y, bv[h2][2] = b4.z, bv[h2][3] = b4.w;
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[a][r][c][e] = fmaf(av[a][r], bv[c][e], acc[a][r][c][e]);
    }
    __syncthreads();
  }
  float* out = sc + ((size_t)b * Hq + h) * nB * nB;
  // a tile left of the diagonal holds only j < i; rows are 16-byte aligned
  // when nB is a multiple of 4
  const bool vec = jt < it && (nB & 3) == 0;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = it * kTile + 64 * a + ty * 4 + r;
      if (i >= nB) continue;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int j0 = jt * kTile + 64 * c + tx * 4;
        if (vec && j0 + 3 < nB) {
          *reinterpret_cast<float4*>(&out[(size_t)i * nB + j0]) =
              make_float4(acc[a][r][c][0], acc[a][r][c][1], acc[a][r][c][2], acc[a][r][c][3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j0 + e < nB && j0 + e <= i) out[(size_t)i * nB + j0 + e] = acc[a][r][c][e];
        }
      }
    }
}

// ---------------------------------------------------------------- selection
// One wave per row (b, h, i), four rows per workgroup; no workgroup barriers.
// Lane l holds the E consecutive entries j = l*E .. l*E+E-1 of the row, so
// lane order is index order and a wave prefix sum ranks entries by index.
constexpr int kRowsPerWg = 4;

struct __align__(16) WaveShared {
  uint32_t hist[256];   // radix histogram of one pass
  uint32_t words[128];  // mask row (nB <= 4096)
};

// the wave's own LDS accesses are served in order; this keeps the compiler
// from moving them across the point
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Top-k membership of the valid entries, largest keys first, ties to the
// lower index: a radix select of the k-th largest key in 8-bit digits from
// the top (histogram of the entries still matching the digits fixed so far,
// counted from the largest bin down), stopping early once the k-th key's bin
// is kept whole; the remaining ties are ranked by index with a wave scan.
// A lane's valid entries are its first nv; the result is a per-lane bit mask
// (bit e = entry e kept), so no per-entry flags live in lane-mask registers.
template <int E>
__device__ __forceinline__ uint64_t wave_topk(const uint32_t (&key)[E], int nv, int k, int n,
                                              WaveShared& sh) {
  static_assert(E <= 64, "one mask bit per entry");
  const int l = lane_id();
  const uint64_t vm = nv >= 64 ? ~0ull : ((1ull << nv) - 1ull);
  if (k >= n) return vm;  // every valid entry
  if (k <= 0) return 0ull;
  uint32_t prefix = 0, pmask = 0;
  int kk = k;  // entries still to take among those matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    reinterpret_cast<uint4*>(sh.hist)[l] = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_fence();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (e < nv && (key[e] & pmask) == prefix)
        __hip_atomic_fetch_add(&sh.hist[(key[e] >> shift) & 255u], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WAVEFRONT);
    wave_lds_fence();
    // lane l: bins 255-4l (c0) down to 252-4l (c3); counts from the top
    const uint4 h4 = reinterpret_cast<const uint4*>(sh.hist)[63 - l];
    const int c0 = h4.w, c1 = h4.z, c2 = h4.y, c3 = h4.x;
    const int sum = c0 + c1 + c2 + c3;
    const int inc = wave_incl_scan(sum);
    const int exc = inc - sum;
    const bool mine = exc < kk && kk <= inc;
    int d, above, cd;
    {
      int a = exc;
      if (kk <= a + c0) {
        d = 255 - 4 * l, cd = c0;
      } else if (kk <= a + c0 + c1) {
        a += c0, d = 254 - 4 * l, cd = c1;
      } else if (kk <= a + c0 + c1 + c2) {
        a += c0 + c1, d = 253 - 4 * l, cd = c2;
      } else {
        a += c0 + c1 + c2, d = 252 - 4 * l, cd = c3;
      }
      above = a;
    }
    const int src = __builtin_ctzll(__ballot(mine));  // exactly one lane (kk <= total)
    d = __builtin_amdgcn_readlane(d, src);
    above = __builtin_amdgcn_readlane(above, src);
    cd = __builtin_amdgcn_readlane(cd, src);
    kk -= above;
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
    if (cd == kk) {  // the k-th key's bin is kept whole
      uint64_t sel = 0ull;
#pragma unroll
      for (int e = 0; e < E; ++e) sel |= (uint64_t)((key[e] & pmask) >= prefix) << e;
      return sel & vm;
    }
  }
  // prefix is the k-th largest key; kk of its copies are kept, lowest index first
  uint64_t gt = 0ull, eq = 0ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    gt |= (uint64_t)(key[e] > prefix) << e;
    eq |= (uint64_t)(key[e] == prefix) << e;
  }
  gt &= vm;
  eq &= vm;
  const int neq = __popcll(eq);
  const int rank = wave_incl_scan(neq) - neq;  // equal keys in lower lanes
  // keep this lane's first max(0, kk - rank) equal keys
  const int take = min(max(kk - rank, 0), neq);
  uint64_t keep_eq = eq;
  for (int x = take; x < neq; ++x) keep_eq &= ~(1ull << (63 - __builtin_clzll(keep_eq)));
  return gt | keep_eq;
}

__device__ __forceinline__ int k_of(double p, int n) {
  if (p < 0.0) return 0;
  double x = ceil(p * (double)n);
  int k = x < 1.0 ? 1 : (x > (double)n ? n : (int)x);
  return k;
}

template <int E>
__global__ __launch_bounds__(64 * kRowsPerWg) void select_rows_kernel(
    const float* __restrict__ qbar, const float* __restrict__ sc, const float* __restrict__ rad,
    uint32_t* __restrict__ mask, int32_t* __restrict__ bidx, int32_t* __restrict__ bcnt,
    float* __restrict__ score_r, int rows, int Hq, int Hkv, int nB, int D, double p_c,
    double p_r, int band, int sink) {
  __shared__ WaveShared shw[kRowsPerWg];
  const int wave = threadIdx.x >> 6, l = lane_id();
  const int row = blockIdx.x * kRowsPerWg + wave;  // (b*Hq + h)*nB + i
  if (row >= rows) return;
  WaveShared& sh = shw[wave];
  const int i = row % nB, bh = row / nB, h = bh % Hq, b = bh / Hq;
  const int g = h / (Hq / Hkv);
  const int n = i + 1;
  const int nw = (nB + 31) / 32;

  float s2 = 0.f;
  const float* qr = qbar + (size_t)row * D;
  for (int d = l; d < D; d += 64) s2 += qr[d] * qr[d];
  const float qn = sqrtf(wave_sum(s2));

  uint32_t kc[E], kr[E];
  const int nv = min(max(n - l * E, 0), E);  // this lane's valid entries
  const float* scr = sc + (size_t)row * nB;
  const float* rr = rad + ((size_t)b * Hkv + g) * nB;
  // A lane's entries are consecutive: with nB a multiple of 4 its quads start
  // on 16-byte boundaries, and each quad whose four entries are valid is read
  // with one 16-byte load of the scores and one of the radii (a lane's 16
  // single-word loads at a 64-byte lane stride touched 4x the cache lines).
  const bool quads = E % 4 == 0 && (nB & 3) == 0;
#pragma unroll
  for (int e4 = 0; e4 < (E + 3) / 4; ++e4) {
    float sv[4] = {0.f, 0.f, 0.f, 0.f}, rv[4] = {0.f, 0.f, 0.f, 0.f};
    const int e0 = 4 * e4, j0 = l * E + e0;
    if (quads && e0 + 4 <= nv) {
      const float4 s4 = *reinterpret_cast<const float4*>(scr + j0);
      const float4 r4 = *reinterpret_cast<const float4*>(rr + j0);
      sv[0] = s4.x, sv[1] = s4.y, sv[2] = s4.z, sv[3] = s4.w;
      rv[0] = r4.x, rv[1] = r4.y, rv[2] = r4.z, rv[3] = r4.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e0 + u < E && e0 + u < nv) {
          sv[u] = scr[j0 + u];
          rv[u] = rr[j0 + u];
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = e0 + u;
      if (e >= E) break;
      const bool valid = e < nv;
      const float r = valid ? fmaf(qn, rv[u], sv[u]) : 0.f;
      kc[e] = order_key(valid ? sv[u] : 0.f);
      kr[e] = order_key(r);
      if (score_r != nullptr && valid) score_r[(size_t)row * nB + j0 + u] = r;
    }
  }
  uint64_t m = wave_topk<E>(kc, nv, k_of(p_c, n), n, sh);
  m |= wave_topk<E>(kr, nv, k_of(p_r, n), n, sh);
  // forced blocks: j < sink, or j > i - band (the band's blocks)
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = l * E + e;
    const bool forced = (j < sink) || (band > 0 && j > i - band);
    m |= (uint64_t)(e < nv && forced) << e;
  }
  const int cnt = __popcll(m);
  const int inc = wave_incl_scan(cnt);
  int pos = inc - cnt;
  const int tot = __builtin_amdgcn_readlane(inc, 63);
  int32_t* lst = bidx + (size_t)row * nB;
  // mask bits of this lane's entries, gathered into 32-bit words in LDS
  for (int w = l; w < nw; w += 64) sh.words[w] = 0u;
  wave_lds_fence();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if ((m >> e) & 1ull) {
      const int j = l * E + e;
      lst[pos++] = j;
      __hip_atomic_fetch_or(&sh.words[j >> 5], 1u << (j & 31), __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_WAVEFRONT);
    }
  }
  if (l == 0) bcnt[row] = tot;
  wave_lds_fence();
  for (int w = l; w < nw; w += 64) mask[(size_t)row * nw + w] = sh.words[w];
}

size_t select_ws_bytes(const PrefillDims& d) {
  const size_t nB = d.S / d.T;
  const size_t qb = (size_t)d.B * d.Hq * nB * d.D * sizeof(float);
  const size_t sc = (size_t)d.B * d.Hq * nB * nB * sizeof(float);
  return ((qb + 255) / 256) * 256 + sc;
}

hipError_t launch_select_blocks(bool f32, const void* q, const float* cen, const float* rad,
                                const PrefillDims& d, double p_c, double p_r, int band,
                                int sink, uint32_t* mask, int32_t* bidx, int32_t* bcnt,
                                float* score_c, float* score_r, void* ws, hipStream_t st) {
  const int nB = d.S / d.T;
  float* qbar = static_cast<float*>(ws);
  const size_t qb = (size_t)d.B * d.Hq * nB * d.D * sizeof(float);
  float* sc = score_c ? score_c
                      : reinterpret_cast<float*>(static_cast<char*>(ws) + ((qb + 255) / 256) * 256);
  if (f32)
    hipLaunchKernelGGL(pool_queries_kernel<float>, dim3(d.B * nB), dim3(256), 0, st,
                       static_cast<const float*>(q), qbar, d.S, d.Hq, d.D, d.T);
  else
    hipLaunchKernelGGL(pool_queries_kernel<uint16_t>, dim3(d.B * nB), dim3(256), 0, st,
                       static_cast<const uint16_t*>(q), qbar, d.S, d.Hq, d.D, d.T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nt = (nB + kTile - 1) / kTile;
  const int tiles = nt * (nt + 1) / 2;
  hipLaunchKernelGGL(centroid_score_kernel, dim3(d.B * d.Hq * tiles), dim3(256), 0, st, qbar, cen,
                     sc, d.Hq, d.Hkv, nB, d.D, tiles);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = d.B * d.Hq * nB;
  const dim3 grid((rows + kRowsPerWg - 1) / kRowsPerWg);
#define FSA_SEL(EE)                                                                           \
  hipLaunchKernelGGL(select_rows_kernel<EE>, grid, dim3(64 * kRowsPerWg), 0, st, qbar, sc, rad, \
                     mask, bidx, bcnt, score_r, rows, d.Hq, d.Hkv, nB, d.D, p_c, p_r, band, sink)
  if (nB <= 64)
    FSA_SEL(1);
  else if (nB <= 128)
    FSA_SEL(2);
  else if (nB <= 256)
    FSA_SEL(4);
  else if (nB <= 512)
    FSA_SEL(8);
  else if (nB <= 1024)
    FSA_SEL(16);
  else if (nB <= 2048)
    FSA_SEL(32);
  else
    FSA_SEL(64);
#undef FSA_SEL
  return hipGetLastError();
}

}  // namespace fsa
