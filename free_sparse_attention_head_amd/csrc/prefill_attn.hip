// sparse_prefill_attn, fp32 inputs: block-sparse causal flash-attention on
// gfx950 MFMA (v_mfma_f32_32x32x2_f32, everything in fp32).  bf16 inputs run
// in prefill_attn_bf16.hip.
//
// RBS-Attention post, "Key technical points" 2: the merged block mask is
// executed by an otherwise unchanged block-sparse FlashAttention path.
//
// Work unit: one workgroup per (batch, query head, query block i), T/32
// waves, each wave owning 32 query rows.  The workgroup walks the ascending
// key-block list of its row in 64-key chunks:
//   * K and V chunks staged row-major in LDS, the next chunk's global loads
//     issued into registers before the current chunk's MFMAs;
//   * S^T = K Q^T with the wave's Q tile resident in registers as the MFMA B
//     operand, so each lane ends up holding one query row's scores: the row
//     max needs one cross-half swap, the row sum none until the epilogue;
//   * online softmax with exp2 and log2(e) folded into the scale;
//   * O^T += V^T P^T with P^T taken straight from registers as the B operand.
// The diagonal block applies the element-wise causal mask; list entries
// outside [0, i] are skipped.  Workgroups sweep one KV head at a time,
// longest rows first.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace fsa {

constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold, log2 units

template <int D, int BLK>
struct PrefillTraits {
  static constexpr int NW = BLK / 32;  // waves per workgroup
  static constexpr int NT = NW * 64;   // threads per workgroup
  static constexpr int KC = 64;        // keys per chunk
  static constexpr int NCH = BLK / KC; // chunks per key block
  // LDS row pitch (elements), padded against bank conflicts
  static constexpr int KP = D + 4;
  static constexpr size_t LDS = (size_t)(2 * KC * KP) * sizeof(float);
  // global->register staging work per thread: 16-byte pieces of K (and of V)
  static constexpr int PIECES = KC * D * 4 / 16 / NT;
  static_assert(PIECES >= 1, "tile shape");
};

// Global -> register -> LDS staging of one 64-key chunk of K and V, both
// row-major.  The pieces are held in wide vector types: an array of uint4 is
// not split into registers and ends up in scratch memory.
template <int D, int BLK>
struct Stage {
  using Tr = PrefillTraits<D, BLK>;
  static constexpr int KP = Tr::KP, NT = Tr::NT;
  static constexpr int PPR = D / 4;  // 16-byte pieces per key row
  typedef uint32_t vec_t __attribute__((ext_vector_type(4 * Tr::PIECES)));
  vec_t k, v;

  __device__ __forceinline__ void load(const float* Kb, const float* Vb, int s0, size_t kv_stride,
                                       int tid) {
#pragma unroll
    for (int m = 0; m < Tr::PIECES; ++m) {
      const int p = tid + m * NT;
      const int key = p / PPR, pc = p % PPR;
      const size_t off = (size_t)(s0 + key) * kv_stride + pc * 4;
      const uint4 a = *reinterpret_cast<const uint4*>(Kb + off);
      const uint4 c = *reinterpret_cast<const uint4*>(Vb + off);
      k[4 * m] = a.x; k[4 * m + 1] = a.y; k[4 * m + 2] = a.z; k[4 * m + 3] = a.w;
      v[4 * m] = c.x; v[4 * m + 1] = c.y; v[4 * m + 2] = c.z; v[4 * m + 3] = c.w;
    }
  }

  __device__ __forceinline__ void store(float* Ks, float* Vs, int tid) const {
#pragma unroll
    for (int m = 0; m < Tr::PIECES; ++m) {
      const int p = tid + m * NT;
      const int key = p / PPR, pc = p % PPR;
      *reinterpret_cast<uint4*>(Ks + key * KP + pc * 4) =
          make_uint4(k[4 * m], k[4 * m + 1], k[4 * m + 2], k[4 * m + 3]);
      *reinterpret_cast<uint4*>(Vs + key * KP + pc * 4) =
          make_uint4(v[4 * m], v[4 * m + 1], v[4 * m + 2], v[4 * m + 3]);
    }
  }
};

// D = 128 needs more than the 256 registers of two waves per SIMD (the fp32 Q
// tile alone takes 64); it runs one wave per SIMD instead of spilling.
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2, D == 128 ? 1 : 2) void prefill_attn_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const int32_t* __restrict__ bidx, const int32_t* __restrict__ bcnt, float* __restrict__ O,
    float* __restrict__ LSE, int S, int Hq, int Hkv, float scale_log2, int total) {
  using Tr = PrefillTraits<D, BLK>;
  constexpr int KC = Tr::KC, NCH = Tr::NCH, KP = Tr::KP;
  extern __shared__ __align__(16) unsigned char smem[];
  float* Ks = reinterpret_cast<float*>(smem);
  float* Vs = Ks + KC * KP;
  int32_t* Ls = reinterpret_cast<int32_t*>(smem + Tr::LDS);  // the row's block list

  // Work order: KV head major, then query blocks longest-first, then the G
  // query heads sharing that KV head.
  const int L = blockIdx.x;
  if (L >= total) return;
  const int nB = S / BLK;
  const int G = Hq / Hkv;
  const int hh = L % G;
  const int rest = L / G;
  const int i = nB - 1 - (rest % nB);
  const int bg = rest / nB;
  const int g = bg % Hkv, b = bg / Hkv;
  const int h = g * G + hh;
  const int row = (b * Hq + h) * nB + i;

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int lq = l & 31, lg = l >> 5;  // lane's query column / lane half
  const int qrow = wave * 32 + lq;     // query row inside the block
  const size_t kv_stride = (size_t)Hkv * D;
  const float* Kb = K + ((size_t)b * S * Hkv + g) * D;
  const float* Vb = V + ((size_t)b * S * Hkv + g) * D;

  // ---- Q tile -> registers (MFMA B operand, lane = query row); lane half lg
  // covers d in [lg*D/2, lg*D/2 + D/2)
  float qf[D / 2];
  {
    const float* qp = Q + (((size_t)b * S + (size_t)i * BLK + qrow) * Hq + h) * D;
#pragma unroll
    for (int kk = 0; kk < D / 2; kk += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(qp + lg * (D / 2) + kk);
      qf[kk] = v4.x; qf[kk + 1] = v4.y; qf[kk + 2] = v4.z; qf[kk + 3] = v4.w;
    }
  }

  // the row's list of causal key blocks (entries outside [0, i] dropped,
  // order kept), staged in LDS once
  __shared__ int scan_tmp[17];
  const int cnt = bidx ? min(max(bcnt[row], 0), nB) : i + 1;
  int nvalid = 0;
  for (int e0 = 0; e0 < cnt; e0 += Tr::NT) {
    const int e = e0 + tid;
    int j = -1;
    if (e < cnt) j = bidx ? bidx[(size_t)row * nB + e] : e;
    const int ok = (j >= 0 && j <= i) ? 1 : 0;
    FSA_DEBUG_RAISE(e < cnt && !ok, FSA_DBG_BLOCK_INDEX);
    int tot;
    const int pos = block_excl_scan(ok, scan_tmp, &tot);
    if (ok) Ls[nvalid + pos] = j;
    nvalid += tot;
  }
  __syncthreads();
  const int nchunks = nvalid * NCH;

  floatx16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // One 64-key chunk: S^T = K Q^T, masked online softmax, O^T += V^T P^T.
  auto compute = [&](int c) {
    const int j = Ls[c / NCH];
    const int koff = (c % NCH) * KC;  // chunk's first key inside the block
    const bool diag = (j == i);
    // a wave whose queries all precede the chunk's keys has nothing to do
    if (diag && koff > wave * 32 + 31) return;
    floatx16 s[2];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[tl][r] = 0.f;
      const float* kr = Ks + (tl * 32 + lq) * KP;
#pragma unroll
      for (int kk = 0; kk < D / 2; kk += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(kr + lg * (D / 2) + kk);
        s[tl] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.x, qf[kk], s[tl], 0, 0, 0);
        s[tl] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.y, qf[kk + 1], s[tl], 0, 0, 0);
        s[tl] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.z, qf[kk + 2], s[tl], 0, 0, 0);
        s[tl] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.w, qf[kk + 3], s[tl], 0, 0, 0);
      }
    }
    // causal mask on the diagonal block and the chunk's row max, in raw score
    // units.  Register r of tile tl holds key koff + tl*32 + (r/4)*8 + lg*4 +
    // r%4 for query qrow.
    if (diag) {
      const int rel = koff + lg * 4 - qrow;
#pragma unroll
      for (int tl = 0; tl < 2; ++tl)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (rel + tl * 32 + (r >> 2) * 8 + (r & 3) > 0) s[tl][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[tl][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescale: a row's reference max m_run moves only when the row max
    // exceeds it by more than kRescaleLog2 (log2 units).  exp2 arguments then
    // stay <= kRescaleLog2 (p <= 256) and the O^T rescale is skipped on every
    // chunk where no row of the wave grows.
    const bool grow = (mx - m_run) * scale_log2 > kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2) : 1.f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * scale_log2;
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[tl][r] = __builtin_amdgcn_exp2f(fmaf(s[tl][r], scale_log2, -mc));
        l_run += s[tl][r];
      }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int tl = 0; tl < 2; ++tl)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = tl * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
          const float a = Vs[key * KP + dt * 32 + lq];
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[tl][r], oacc[dt], 0, 0, 0);
        }
  };

  // register prefetch: while chunk c is computed, the loads of chunk c+1 are
  // in flight
  auto chunk_s0 = [&](int c) { return Ls[c / NCH] * BLK + (c % NCH) * KC; };
  Stage<D, BLK> st;
  if (0 < nchunks) st.load(Kb, Vb, chunk_s0(0), kv_stride, tid);
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();
    st.store(Ks, Vs, tid);
    __syncthreads();
    if (c + 1 < nchunks) st.load(Kb, Vb, chunk_s0(c + 1), kv_stride, tid);
    compute(c);
  }

  // ---- epilogue: O = O^T / l, LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int t = i * BLK + qrow;
  float* op = O + (((size_t)b * S + t) * Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = dt * 32 + rg * 8 + lg * 4;
      *reinterpret_cast<float4*>(op + d0) =
          make_float4(oacc[dt][rg * 4] * inv, oacc[dt][rg * 4 + 1] * inv,
                      oacc[dt][rg * 4 + 2] * inv, oacc[dt][rg * 4 + 3] * inv);
    }
  if (LSE != nullptr && lg == 0)
    LSE[((size_t)b * Hq + h) * S + t] =
        l_tot > 0.f ? (m_run * scale_log2 + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, int BLK>
static hipError_t launch_pa(const void* q, const void* k, const void* v, const PrefillDims& d,
                            const int32_t* bidx, const int32_t* bcnt, float scale, void* out,
                            float* lse, hipStream_t st) {
  using Tr = PrefillTraits<D, BLK>;
  auto kern = prefill_attn_kernel<D, BLK>;
  const size_t lds = Tr::LDS + (size_t)(d.S / BLK) * sizeof(int32_t);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int total = d.B * d.Hq * (d.S / BLK);
  hipLaunchKernelGGL(kern, dim3(total), dim3(Tr::NT), lds, st, static_cast<const float*>(q),
                     static_cast<const float*>(k), static_cast<const float*>(v), bidx, bcnt,
                     static_cast<float*>(out), lse, d.S, d.Hq, d.Hkv, scale * kLog2e, total);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(bool f32, const void* q, const void* k, const void* v,
                               const PrefillDims& d, const int32_t* bidx, const int32_t* bcnt,
                               float scale, void* out, float* lse, hipStream_t st) {
  if (!f32) return launch_prefill_attn_bf16(q, k, v, d, bidx, bcnt, scale, out, lse, st);
#define FSA_PA(DD, TT) \
  if (d.D == DD && d.T == TT) return launch_pa<DD, TT>(q, k, v, d, bidx, bcnt, scale, out, lse, st);
  FSA_PA(64, 64) FSA_PA(64, 128) FSA_PA(128, 64) FSA_PA(128, 128)
#undef FSA_PA
  return hipErrorInvalidValue;
}

hipError_t debug_flags_prefill_f32(uint32_t* flags, bool clear) {
  return debug_flags_of_tu(flags, clear);
}

}  // namespace fsa
