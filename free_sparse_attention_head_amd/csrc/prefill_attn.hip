// sparse_prefill_attn: block-sparse causal flash-attention on gfx950 MFMA.
//
// RBS-Attention post, "Key technical points" 2: the merged block mask is
// executed by an otherwise unchanged block-sparse FlashAttention path.
//
// Work unit: one workgroup per (batch, query head, query block i), T/32
// waves, each wave owning 32 query rows.  The workgroup walks the ascending
// key-block list of its row in 64-key chunks:
//   * K chunk staged row-major in LDS, V chunk staged transposed (V^T) in LDS,
//     the next chunk's global loads issued into registers before the current
//     chunk's MFMAs (register double buffering);
//   * S^T = K Q^T with the wave's Q tile resident in registers as the MFMA B
//     operand, so each lane ends up holding one query row's scores: the row
//     max needs one cross-half swap, the row sum none until the epilogue;
//   * online softmax in fp32 with exp2 and log2(e) folded into the scale;
//   * O^T += V^T P^T with P^T taken straight from registers as the B operand
//     (the key order inside a 16-key MFMA step follows the S^T register
//     layout; V^T is read from LDS in that same order).
// bf16 inputs: v_mfma_f32_32x32x16_bf16, P rounded to bf16 for the PV step.
// fp32 inputs: v_mfma_f32_32x32x2_f32, everything in fp32 (V kept row-major).
// The diagonal block applies the element-wise causal mask; list entries
// outside [0, i] are skipped.  Workgroups sweep one KV head at a time,
// longest rows first (see the work-order note in the kernel).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace fsa {

constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold, log2 units

template <typename TI, int D, int BLK>
struct PrefillTraits {
  static constexpr bool F32 = sizeof(TI) == 4;
  static constexpr int NW = BLK / 32;  // waves per workgroup
  static constexpr int NT = NW * 64;   // threads per workgroup
  static constexpr int KC = 64;        // keys per chunk
  static constexpr int NCH = BLK / KC; // chunks per key block
  // LDS row pitches (elements), padded against bank conflicts
  static constexpr int KP = F32 ? D + 4 : D + 8;
  static constexpr int VP = F32 ? D + 4 : KC + 4;
  static constexpr int VROWS = F32 ? KC : D;
  static constexpr size_t LDS = (size_t)(KC * KP + VROWS * VP) * sizeof(TI);
  // global->register staging work per thread
  static constexpr int KPIECES = KC * D * sizeof(TI) / 16 / NT;  // 16-byte K pieces
  static constexpr int VUNITS = F32 ? KPIECES : (KC / 4) * (D / 4) / NT;
  static_assert(KPIECES >= 1 && VUNITS >= 1, "tile shape");
  // two staging sets in flight when one set is small enough
  static constexpr bool DEEP = !F32 && KPIECES <= 4;
};

// V^T fragment (MFMA A operand) of step m = kc * ndt + dt: d row dt*32 + lq,
// keys kc*16 + lg*4 + {0..3} and kc*16 + 8 + lg*4 + {0..3} (vbase already
// points at row lq, column lg*4).
template <typename TI, int VP, int NDT>
__device__ __forceinline__ uint4 vt_frag(const TI* vbase, int m) {
  const int kc = m / NDT, dt = m % NDT;
  const TI* p = vbase + dt * 32 * VP + kc * 16;
  const uint2 lo = *reinterpret_cast<const uint2*>(p);
  const uint2 hi = *reinterpret_cast<const uint2*>(p + 8);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Global -> register -> LDS staging of one 64-key chunk of K and V.  K is
// copied row-major; bf16 V is transposed 4x4 in registers and written as V^T
// (fp32 V stays row-major).  All loops are fully unrolled over fixed-size
// member arrays so the staging lives in VGPRs.
template <typename TI, int D, int BLK>
struct Stage {
  using Tr = PrefillTraits<TI, D, BLK>;
  static constexpr bool F32 = Tr::F32;
  static constexpr int KC = Tr::KC, KP = Tr::KP, VP = Tr::VP, NT = Tr::NT;
  static constexpr int PPR = D * (int)sizeof(TI) / 16;  // 16-byte pieces per key row
  // K (and fp32 V) pieces are held in wide vector types: an array of uint4
  // here is not split into registers and ends up in scratch memory.
  typedef uint32_t kvec_t __attribute__((ext_vector_type(4 * Tr::KPIECES)));
  typedef uint32_t vvec_t __attribute__((ext_vector_type(4 * (F32 ? Tr::VUNITS : 1))));
  kvec_t k;
  vvec_t vf;                           // fp32 V pieces
  uint2 vb[F32 ? 1 : Tr::VUNITS][4];   // bf16 V: 4 keys x 4 d per unit

  __device__ __forceinline__ void load(const TI* Kb, const TI* Vb, int s0, size_t kv_stride,
                                       int tid) {
#pragma unroll
    for (int m = 0; m < Tr::KPIECES; ++m) {
      const int p = tid + m * NT;
      const int key = p / PPR, pc = p % PPR;
      const uint4 w = *reinterpret_cast<const uint4*>(Kb + (size_t)(s0 + key) * kv_stride +
                                                      pc * (16 / sizeof(TI)));
      k[4 * m] = w.x;
      k[4 * m + 1] = w.y;
      k[4 * m + 2] = w.z;
      k[4 * m + 3] = w.w;
    }
    if constexpr (F32) {
#pragma unroll
      for (int m = 0; m < Tr::VUNITS; ++m) {
        const int p = tid + m * NT;
        const int key = p / PPR, pc = p % PPR;
        const uint4 w = *reinterpret_cast<const uint4*>(Vb + (size_t)(s0 + key) * kv_stride + pc * 4);
        vf[4 * m] = w.x;
        vf[4 * m + 1] = w.y;
        vf[4 * m + 2] = w.z;
        vf[4 * m + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int m = 0; m < Tr::VUNITS; ++m) {
        const int u = tid + m * NT;
        const int kq = u / (D / 4), dq = u % (D / 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          vb[m][rr] = *reinterpret_cast<const uint2*>(Vb + (size_t)(s0 + kq * 4 + rr) * kv_stride +
                                                      dq * 4);
      }
    }
  }

  __device__ __forceinline__ void store(TI* Ks, TI* Vs, int tid) const {
#pragma unroll
    for (int m = 0; m < Tr::KPIECES; ++m) {
      const int p = tid + m * NT;
      const int key = p / PPR, pc = p % PPR;
      *reinterpret_cast<uint4*>(Ks + key * KP + pc * (16 / sizeof(TI))) =
          make_uint4(k[4 * m], k[4 * m + 1], k[4 * m + 2], k[4 * m + 3]);
    }
    if constexpr (F32) {
#pragma unroll
      for (int m = 0; m < Tr::VUNITS; ++m) {
        const int p = tid + m * NT;
        const int key = p / PPR, pc = p % PPR;
        *reinterpret_cast<uint4*>(Vs + key * VP + pc * 4) =
            make_uint4(vf[4 * m], vf[4 * m + 1], vf[4 * m + 2], vf[4 * m + 3]);
      }
    } else {
#pragma unroll
      for (int m = 0; m < Tr::VUNITS; ++m) {
        const int u = tid + m * NT;
        const int kq = u / (D / 4), dq = u % (D / 4);
        const uint2 r0 = vb[m][0], r1 = vb[m][1], r2 = vb[m][2], r3 = vb[m][3];
        uint2 c0, c1, c2, c3;  // column e of the 4x4 bf16 block = keys kq*4..+3 at d = dq*4+e
        c0.x = (r0.x & 0xffffu) | (r1.x << 16);
        c0.y = (r2.x & 0xffffu) | (r3.x << 16);
        c1.x = (r0.x >> 16) | (r1.x & 0xffff0000u);
        c1.y = (r2.x >> 16) | (r3.x & 0xffff0000u);
        c2.x = (r0.y & 0xffffu) | (r1.y << 16);
        c2.y = (r2.y & 0xffffu) | (r3.y << 16);
        c3.x = (r0.y >> 16) | (r1.y & 0xffff0000u);
        c3.y = (r2.y >> 16) | (r3.y & 0xffff0000u);
        TI* vt = Vs + (dq * 4) * VP + kq * 4;
        *reinterpret_cast<uint2*>(vt) = c0;
        *reinterpret_cast<uint2*>(vt + VP) = c1;
        *reinterpret_cast<uint2*>(vt + 2 * VP) = c2;
        *reinterpret_cast<uint2*>(vt + 3 * VP) = c3;
      }
    }
  }
};

template <typename TI, int D, int BLK>
__global__ __launch_bounds__(BLK * 2, 2) void prefill_attn_kernel(
    const TI* __restrict__ Q, const TI* __restrict__ K, const TI* __restrict__ V,
    const int32_t* __restrict__ bidx, const int32_t* __restrict__ bcnt, TI* __restrict__ O,
    float* __restrict__ LSE, int S, int Hq, int Hkv, float scale_log2, int total) {
  using Tr = PrefillTraits<TI, D, BLK>;
  constexpr bool F32 = Tr::F32;
  constexpr int KC = Tr::KC, NCH = Tr::NCH, KP = Tr::KP, VP = Tr::VP;
  extern __shared__ __align__(16) unsigned char smem[];
  TI* Ks = reinterpret_cast<TI*>(smem);
  TI* Vs = Ks + KC * KP;
  int32_t* Ls = reinterpret_cast<int32_t*>(smem + Tr::LDS);  // the row's block list

  // Work order: KV head major, then query blocks longest-first, then the G
  // query heads sharing that KV head.  The running window of workgroups
  // therefore touches one KV head's K/V at a time (so it stays resident in
  // the Infinity Cache), and since dispatch deals workgroups round-robin over
  // the 8 XCDs, each XCD sees the same query head for consecutive query
  // blocks, whose diagonal bands and sink blocks then hit in its L2.
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
  const int bh = b * Hq + h;
  const int row = bh * nB + i;

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int lq = l & 31, lg = l >> 5;  // lane's query column / lane half
  const int qrow = wave * 32 + lq;     // query row inside the block
  const size_t kv_stride = (size_t)Hkv * D;
  const TI* Kb = K + ((size_t)b * S * Hkv + g) * D;
  const TI* Vb = V + ((size_t)b * S * Hkv + g) * D;

  // ---- Q tile -> registers (MFMA B operand, lane = query row)
  constexpr int QREG = F32 ? D / 2 : D / 16;
  using QFrag = typename std::conditional<F32, float, bf16x8>::type;
  QFrag qf[QREG];
  {
    const TI* qp = Q + (((size_t)b * S + (size_t)i * BLK + qrow) * Hq + h) * D;
    if constexpr (F32) {
      // lane half lg covers d in [lg*D/2, lg*D/2 + D/2)
#pragma unroll
      for (int kk = 0; kk < D / 2; kk += 4) {
        float4 v4 = *reinterpret_cast<const float4*>(qp + lg * (D / 2) + kk);
        qf[kk] = v4.x; qf[kk + 1] = v4.y; qf[kk + 2] = v4.z; qf[kk + 3] = v4.w;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + kk * 16 + lg * 8));
    }
  }

  // Stage the row's list of causal key blocks (entries outside [0, i]
  // dropped, order kept) in LDS once; the loop then reads the list from LDS
  // and never waits on a global load that could also cover the K/V prefetch.
  __shared__ int scan_tmp[17];
  const int cnt = bidx ? min(max(bcnt[row], 0), nB) : i + 1;
  int nvalid = 0;
  for (int e0 = 0; e0 < cnt; e0 += Tr::NT) {
    const int e = e0 + tid;
    int j = -1;
    if (e < cnt) j = bidx ? bidx[(size_t)row * nB + e] : e;
    const int ok = (j >= 0 && j <= i) ? 1 : 0;
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
      if (!(diag && koff > wave * 32 + 31)) {
        floatx16 s[2];
  #pragma unroll
        for (int tl = 0; tl < 2; ++tl) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) s[tl][r] = 0.f;
          if constexpr (F32) {
            const TI* kr = Ks + (tl * 32 + lq) * KP;
  #pragma unroll
            for (int kk = 0; kk < D / 2; kk += 4) {
              const float4 a4 = *reinterpret_cast<const float4*>(kr + lg * (D / 2) + kk);
              s[tl] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.x, qf[kk], s[tl], 0, 0, 0);
              s[tl] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.y, qf[kk + 1], s[tl], 0, 0, 0);
              s[tl] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.z, qf[kk + 2], s[tl], 0, 0, 0);
              s[tl] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.w, qf[kk + 3], s[tl], 0, 0, 0);
            }
          }
        }
        if constexpr (!F32) {
          // K fragments of step kk+1 are read before the MFMAs of step kk, and
          // the two independent 32-key tiles alternate on the matrix pipe, so
          // LDS latency overlaps MFMA execution.
          const TI* kr0 = Ks + lq * KP + lg * 8;
          const TI* kr1 = kr0 + 32 * KP;
          uint4 a0 = *reinterpret_cast<const uint4*>(kr0);
          uint4 a1 = *reinterpret_cast<const uint4*>(kr1);
  #pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            uint4 n0 = a0, n1 = a1;
            if (kk + 1 < D / 16) {
              n0 = *reinterpret_cast<const uint4*>(kr0 + (kk + 1) * 16);
              n1 = *reinterpret_cast<const uint4*>(kr1 + (kk + 1) * 16);
            }
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0), qf[kk], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a1), qf[kk], s[1], 0, 0, 0);
            a0 = n0;
            a1 = n1;
          }
          // keep the reads one step ahead of the MFMAs in the final schedule
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  #pragma unroll
          for (int kk = 0; kk < D / 16; ++kk) {
            if (kk + 1 < D / 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          }
        }
        // causal mask on the diagonal block and the chunk's row max, in raw
        // score units.  Register r of tile tl holds key
        // koff + tl*32 + (r/4)*8 + lg*4 + r%4 for query qrow.
        if (diag) {
          // keys after the query row: key - qrow > 0 with key = koff + tl*32 +
          // (r/4)*8 + lg*4 + r%4
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
        // stay <= kRescaleLog2 (p <= 256, exact in fp32 and bf16 range) and the
        // O^T rescale is skipped on every chunk where no row of the wave grows.
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
          for (int r = 0; r < 16; ++r) s[tl][r] = __builtin_amdgcn_exp2f(fmaf(s[tl][r], scale_log2, -mc));
        // O^T += V^T P^T
        if constexpr (F32) {
  #pragma unroll
          for (int tl = 0; tl < 2; ++tl)
  #pragma unroll
            for (int r = 0; r < 16; ++r) l_run += s[tl][r];
  #pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
  #pragma unroll
            for (int tl = 0; tl < 2; ++tl)
  #pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = tl * 32 + (r >> 2) * 8 + lg * 4 + (r & 3);
                const float a = Vs[key * VP + dt * 32 + lq];
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[tl][r], oacc[dt], 0, 0, 0);
              }
        } else {
          bf16x8 pf[4];
  #pragma unroll
          for (int kc = 0; kc < 4; ++kc)
  #pragma unroll
            for (int e = 0; e < 8; ++e) pf[kc][e] = (__bf16)s[kc >> 1][(kc & 1) * 8 + e];
          // row sum of the bf16-rounded P that the PV step multiplies (v_dot2 with ones)
          const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  #pragma unroll
          for (int kc = 0; kc < 4; ++kc) {
            const uint4 w = __builtin_bit_cast(uint4, pf[kc]);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.x), ones, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.y), ones, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.z), ones, l_run, false);
            l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w.w), ones, l_run, false);
          }
          // 4*(D/32) MFMAs in (kc, dt) order: consecutive MFMAs hit different
          // accumulators, and each V^T fragment is read two MFMAs ahead.
          constexpr int NDT = D / 32, NM = 4 * NDT;
          const TI* vbase = Vs + lq * VP + lg * 4;
          uint4 f0 = vt_frag<TI, VP, NDT>(vbase, 0), f1 = vt_frag<TI, VP, NDT>(vbase, 1);
  #pragma unroll
          for (int m = 0; m < NM; ++m) {
            const uint4 f2 = (m + 2 < NM) ? vt_frag<TI, VP, NDT>(vbase, m + 2) : f0;
            oacc[m % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f0),
                                                                    pf[m / NDT], oacc[m % NDT], 0, 0, 0);
            f0 = f1;
            f1 = f2;
          }
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
  #pragma unroll
          for (int m = 0; m < NM; ++m) {
            if (m + 2 < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          }
        }
      }
  };

  // ---- register prefetch: while chunk c is computed, the loads of chunks
  // c+1 and c+2 are in flight (two staging register sets, loop unrolled by
  // two so each set keeps fixed registers).
  // Shapes whose staging set is larger (fewer threads per chunk, or fp32)
  // keep a one-deep prefetch so the registers still fit two waves per SIMD.
  auto chunk_s0 = [&](int c) { return Ls[c / NCH] * BLK + (c % NCH) * KC; };
  if constexpr (Tr::DEEP) {
    // sched_barrier(0) keeps set A's loads ahead of set B's in issue order, so
    // the wait before storing set A leaves set B's loads in flight
    // The loads are unconditional (past the end they re-read the last chunk,
    // a cache hit): conditional loads would merge wait-count state at the
    // joins and force a wait for every outstanding load.
    if (nchunks > 0) {
      const int last = nchunks - 1;
      Stage<TI, D, BLK> stA, stB;
      stA.load(Kb, Vb, chunk_s0(0), kv_stride, tid);
      __builtin_amdgcn_sched_barrier(0);
      stB.load(Kb, Vb, chunk_s0(min(1, last)), kv_stride, tid);
      __builtin_amdgcn_sched_barrier(0);
      // pairs of chunks; the loop header is reached only after both halves,
      // so the wait before storing set A never covers set B's loads
      const int pairs = nchunks >> 1;
      for (int pr = 0; pr < pairs; ++pr) {
        const int c = 2 * pr;
        __syncthreads();
        stA.store(Ks, Vs, tid);
        __syncthreads();
        stA.load(Kb, Vb, chunk_s0(min(c + 2, last)), kv_stride, tid);
        __builtin_amdgcn_sched_barrier(0);
        compute(c);
        __syncthreads();
        stB.store(Ks, Vs, tid);
        __syncthreads();
        stB.load(Kb, Vb, chunk_s0(min(c + 3, last)), kv_stride, tid);
        __builtin_amdgcn_sched_barrier(0);
        compute(c + 1);
      }
      if (nchunks & 1) {  // odd tail: set A holds chunk nchunks - 1
        __syncthreads();
        stA.store(Ks, Vs, tid);
        __syncthreads();
        compute(last);
      }
    }
  } else {
    Stage<TI, D, BLK> st;
    if (0 < nchunks) st.load(Kb, Vb, chunk_s0(0), kv_stride, tid);
    for (int c = 0; c < nchunks; ++c) {
      __syncthreads();
      st.store(Ks, Vs, tid);
      __syncthreads();
      if (c + 1 < nchunks) st.load(Kb, Vb, chunk_s0(c + 1), kv_stride, tid);
      compute(c);
    }
  }

  // ---- epilogue: O = O^T / l, LSE
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int t = i * BLK + qrow;
  TI* op = O + (((size_t)b * S + t) * Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = dt * 32 + rg * 8 + lg * 4;
      const float o0 = oacc[dt][rg * 4] * inv, o1 = oacc[dt][rg * 4 + 1] * inv;
      const float o2 = oacc[dt][rg * 4 + 2] * inv, o3 = oacc[dt][rg * 4 + 3] * inv;
      if constexpr (F32) {
        *reinterpret_cast<float4*>(op + d0) = make_float4(o0, o1, o2, o3);
      } else {
        *reinterpret_cast<uint2*>(op + d0) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      }
    }
  if (LSE != nullptr && lg == 0)
    LSE[((size_t)b * Hq + h) * S + t] =
        l_tot > 0.f ? (m_run * scale_log2 + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <typename TI, int D, int BLK>
static hipError_t launch_pa(const void* q, const void* k, const void* v, const PrefillDims& d,
                            const int32_t* bidx, const int32_t* bcnt, float scale, void* out,
                            float* lse, hipStream_t st) {
  using Tr = PrefillTraits<TI, D, BLK>;
  auto kern = prefill_attn_kernel<TI, D, BLK>;
  const size_t lds = Tr::LDS + (size_t)(d.S / BLK) * sizeof(int32_t);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int total = d.B * d.Hq * (d.S / BLK);
  const int padded = (total + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL(kern, dim3(padded), dim3(Tr::NT), lds, st, static_cast<const TI*>(q),
                     static_cast<const TI*>(k), static_cast<const TI*>(v), bidx, bcnt,
                     static_cast<TI*>(out), lse, d.S, d.Hq, d.Hkv, scale * kLog2e, total);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(bool f32, const void* q, const void* k, const void* v,
                               const PrefillDims& d, const int32_t* bidx, const int32_t* bcnt,
                               float scale, void* out, float* lse, hipStream_t st) {
#define FSA_PA(TY, DD, TT) \
  if (d.D == DD && d.T == TT) return launch_pa<TY, DD, TT>(q, k, v, d, bidx, bcnt, scale, out, lse, st);
  if (!f32) return launch_prefill_attn_bf16(q, k, v, d, bidx, bcnt, scale, out, lse, st);
  FSA_PA(float, 64, 64) FSA_PA(float, 64, 128) FSA_PA(float, 128, 64) FSA_PA(float, 128, 128)
#undef FSA_PA
  return hipErrorInvalidValue;
}

}  // namespace fsa
