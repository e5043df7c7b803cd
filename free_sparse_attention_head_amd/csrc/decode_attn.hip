// sparse_decode_attn: split-KV decode attention over a paged bf16 KV cache,
// plus the log-sum-exp combine.
//
// Kascade post, "What Kascade got right": reuse layers attend only at the
// anchor layer's per-head top-k indices (index mode; the per-KV-head variant
// shares one index set, and every K/V read, among a KV head's query heads).
// Declarative Attention post, "Declarative attention protocol": global / focus / local modes become
// block-aligned token ranges that an unmodified attention kernel reads
// (segment mode).  LoZA post, "4. From food delivery to AI":
// SplitKV-and-Combine splits the KV reads and merges partial results.
//
// HBM-bound streaming design (no matrix cores: the contraction per KV row is
// a handful of dot products):
//   * a workgroup of 4 waves owns one (sequence, head-or-KV-head, split);
//   * D/8 lanes share one 256-byte (D=128) key row: every lane issues one
//     16-byte load for K and one for V, so a row is one contiguous,
//     fully-used read; each lane group streams RB rows per step with all 2*RB
//     loads in flight before any arithmetic;
//   * scores use v_dot2_f32_bf16 on the raw bf16 pairs and a DPP butterfly
//     across the lane group; in segment/all mode the G query heads of a KV
//     head share every K/V read;
//   * the softmax is online per lane group (one rescale per RB-row step);
//     lane groups and waves merge through LDS at the end of the split and
//     write an unnormalised (max, sum, output) partial in fp32;
//   * a split takes at least kMinSplitPositions positions, so short segment
//     lists leave surplus splits empty (max -inf, sum 0);
//   * combine_kernel merges the splits of one (sequence, head): one wave
//     reads every split's (max, sum) in parallel, then the splits' outputs
//     eight at a time, all loads of a batch in flight together; with a single split the split kernel
//     normalises and writes the output itself.
#include <math.h>

#include <mutex>

#include "common.h"
#include "launch.h"

namespace fsa {

constexpr int kDecThreads = 256;
constexpr int kMaxSeg = 64;     // segments per sequence kept in LDS
constexpr int kRowBatch = 1024;  // positions resolved to pool rows at a time
// A split takes at least this many positions: the split count is fixed at
// launch from the longest possible list, but a segment list may admit far
// fewer tokens; surplus splits then take no positions and write empty
// partials, which the combine skips.
constexpr int kMinSplitPositions = 64;

template <int D, int NH, int MODE>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpool,
    const uint16_t* __restrict__ vpool, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ sl, int Hq, int Hkv, int max_pages, int num_pages,
    int max_seq_len, const int32_t* __restrict__ idx, const float* __restrict__ scores, int k,
    const int32_t* __restrict__ seg,
    const int32_t* __restrict__ nseg, int max_seg, int n_split, float scale_log2,
    float* __restrict__ part, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int LPR = D / 8;            // lanes per key row
  constexpr int RG = 64 / LPR;          // row groups per wave
  constexpr int NSLOT = 4 * RG;         // row groups per workgroup
  constexpr int RB = 4;                 // rows per row group per step
  constexpr int NHEAD_ITEM = NH;
  __shared__ float sm_m[4][NH], sm_l[4][NH];
  __shared__ float sm_o[4][NH][D];
  __shared__ int seg_lo[kMaxSeg], seg_pre[kMaxSeg + 1];
  __shared__ int s_nseg;
  __shared__ uint32_t rows_lds[kRowBatch];  // pool row of each position of the batch
  constexpr bool SCORED = MODE == FSA_SEL_INDEX_SCORED;
  // scored mode: the raw score of each position of the batch (keys not read)
  __shared__ float sc_lds[SCORED ? kRowBatch : 1];

  const int G = Hq / Hkv;
  const int s = blockIdx.x % n_split;
  const int item = blockIdx.x / n_split;  // b * (heads per item layout) + hh
  constexpr bool PER_HEAD = MODE == FSA_SEL_INDEX || MODE == FSA_SEL_INDEX_SCORED;
  const int per_b = PER_HEAD ? Hq : Hkv;
  const int hh = item % per_b, b = item / per_b;
  const int g = PER_HEAD ? hh / G : hh;
  const int h0 = PER_HEAD ? hh : hh * G;  // first query head of the item
  constexpr bool LISTED = MODE == FSA_SEL_INDEX || MODE == FSA_SEL_INDEX_KV || SCORED;
  const int n = min(max(sl[b], 0), max_seq_len);

  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int slot = wave * RG + l / LPR, dl = l % LPR;

  // ---- this split's range of list positions
  int total;
  if constexpr (MODE == FSA_SEL_SEGMENT) {
    // wave 0: lane x reads segment x (clipped to [0, n)); the non-empty ones
    // are compacted in order with their exclusive prefix of lengths
    static_assert(kMaxSeg == 64, "one segment per lane of a wave");
    if (wave == 0) {
      // the count and every segment slot are read together (one round trip)
      int ns = nseg[b];
      int a = 0, e = 0;
      if (l < min(max_seg, kMaxSeg)) {
        a = seg[((size_t)b * max_seg + l) * 2];
        e = seg[((size_t)b * max_seg + l) * 2 + 1];
      }
      FSA_DEBUG_RAISE(l == 0 && (ns < 0 || ns > max_seg), FSA_DBG_SEGMENT);
      ns = ns < 0 ? 0 : (ns > max_seg ? max_seg : ns);
      ns = ns > kMaxSeg ? kMaxSeg : ns;
#ifdef FSA_DEBUG_BOUNDS
      // ranges must be sorted and disjoint: each starts at or after the
      // previous one's end (lanes are consecutive segments)
      const int prev_end = __shfl_up(e, 1, 64);
      FSA_DEBUG_RAISE(l > 0 && l < ns && a < prev_end, FSA_DBG_SEGMENT);
#endif
      int len = 0;
      if (l < ns) {
        a = max(a, 0);
        len = max(min(e, n) - a, 0);
      } else {
        a = 0;
      }
      const uint64_t valid = __ballot(len > 0);
      const int rank = __popcll(valid & ((1ull << l) - 1ull));
      const int inc = wave_incl_scan(len);
      if (len > 0) {
        seg_lo[rank] = a;
        seg_pre[rank] = inc - len;
      }
      if (l == 63) {
        seg_pre[__popcll(valid)] = inc;
        s_nseg = __popcll(valid);
      }
    }
    __syncthreads();
    total = seg_pre[s_nseg];
  } else if constexpr (LISTED) {
    total = k;
  } else {
    total = n;
  }
  int chunk = (total + n_split - 1) / n_split;
  chunk = max((chunk + 15) & ~15, kMinSplitPositions);
  const int p0 = s * chunk;
  const int p1 = min(total, p0 + chunk);

  // ---- queries of the item: lane keeps its 8 d values of each head
  uint4 qv[NH];
#pragma unroll
  for (int x = 0; x < NH; ++x)
    qv[x] = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + h0 + x) * D + dl * 8);

  float m_run[NH], l_run[NH], o[NH][8];
#pragma unroll
  for (int x = 0; x < NH; ++x) {
    m_run[x] = -INFINITY;
    l_run[x] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[x][e] = 0.f;
  }
  const int32_t* ptb = pt + (size_t)b * max_pages;
  // index list of the item: per query head, or per KV head shared by its G heads
  const int32_t* idxr = LISTED ? idx + ((size_t)b * per_b + hh) * k : nullptr;

  // pool row of token tok, or kNoRow (out of range, or a bad page id: such
  // tokens are skipped, never read).  The page-table read is issued for every
  // token (a clamped in-range entry), so that a thread's lookups can all be
  // in flight together.
  constexpr uint32_t kNoRow = 0xffffffffu;
  auto row_of = [&](int tok) -> uint32_t {
    const int page = ptb[min(max(tok, 0), max(n - 1, 0)) >> 4];
    const bool ok = (tok >= 0) & (tok < n) & (page >= 0) & (page < num_pages);
    // -1 marks an empty slot (top-k of a short sequence, union padding)
    FSA_DEBUG_RAISE(tok < -1 || tok >= n, FSA_DBG_TOKEN_INDEX);
    FSA_DEBUG_RAISE(tok >= 0 && tok < n && (page < 0 || page >= num_pages), FSA_DBG_PAGE_ID);
    const uint32_t row = ((uint32_t)page * (uint32_t)Hkv + (uint32_t)g) * 16u + (uint32_t)(tok & 15);
    // a select, not a branch, so that the next lookup's read can issue first
    return __builtin_unpredictable(ok) ? row : kNoRow;
  };
  // token at list position pos
  auto token_of = [&](int pos) -> int {
    if constexpr (LISTED) {
      return idxr[pos];
    } else if constexpr (MODE == FSA_SEL_SEGMENT) {
      int x = 0;
      while (x + 1 < s_nseg && seg_pre[x + 1] <= pos) ++x;
      return seg_lo[x] + (pos - seg_pre[x]);
    } else {
      return pos;
    }
  };
  // Positions are resolved (index or segment, then page id) to pool rows
  // kRowBatch at a time into LDS before they are streamed, so the K/V loads
  // of a step depend on no other global load.
  for (int b0 = p0; b0 < p1; b0 += kRowBatch) {
    const int b1 = min(p1, b0 + kRowBatch);
    __syncthreads();  // the previous batch's rows have been read
    uint32_t rw[kRowBatch / kDecThreads];  // all of a thread's lookups in flight at once
#pragma unroll
    for (int u = 0; u < kRowBatch / kDecThreads; ++u) {
      const int x = u * kDecThreads + tid;
      const bool in_batch = x < b1 - b0;
      const uint32_t r = row_of(token_of(in_batch ? b0 + x : b0));
      rw[u] = in_batch ? r : kNoRow;
    }
#pragma unroll
    for (int u = 0; u < kRowBatch / kDecThreads; ++u) rows_lds[u * kDecThreads + tid] = rw[u];
    if constexpr (SCORED) {
      const float* scr = scores + ((size_t)b * per_b + hh) * k;
#pragma unroll
      for (int u = 0; u < kRowBatch / kDecThreads; ++u) {
        const int x = u * kDecThreads + tid;
        sc_lds[x] = x < b1 - b0 ? scr[b0 + x] : 0.f;
      }
    }
    __syncthreads();
    for (int base = b0; base < b1; base += NSLOT * RB) {
      uint4 kr[RB], vr[RB];
      bool ok[RB];
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const int pos = base + slot * RB + r;
        const uint32_t row = pos < b1 ? rows_lds[pos - b0] : kNoRow;
        ok[r] = row != kNoRow;
        if (ok[r]) {
          if constexpr (!SCORED)
            kr[r] = *reinterpret_cast<const uint4*>(kpool + (size_t)row * D + dl * 8);
          vr[r] = *reinterpret_cast<const uint4*>(vpool + (size_t)row * D + dl * 8);
        } else {
          kr[r] = make_uint4(0, 0, 0, 0);
          vr[r] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int x = 0; x < NHEAD_ITEM; ++x) {
        float sc[RB];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          float d;
          if constexpr (SCORED) {
            const int pos = base + slot * RB + r;
            d = sc_lds[min(pos - b0, kRowBatch - 1)];
          } else {
            d = group_sum<LPR>(dot8_bf16(qv[x], kr[r], 0.f));
          }
          sc[r] = ok[r] ? d * scale_log2 : -INFINITY;
          mx = fmaxf(mx, sc[r]);
        }
        const float m_new = fmaxf(m_run[x], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[x] - m_use);
        m_run[x] = m_new;
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[x][e] *= alpha;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const float p = __builtin_amdgcn_exp2f(sc[r] - m_use);
          ls += p;
          const uint32_t w[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[x][2 * e] = fmaf(p, bf16_lo(w[e]), o[x][2 * e]);
            o[x][2 * e + 1] = fmaf(p, bf16_hi(w[e]), o[x][2 * e + 1]);
          }
        }
        l_run[x] = l_run[x] * alpha + ls;
      }
    }
  }

  // ---- merge the row groups of each wave (lanes LPR apart hold the same d
  // values of different row groups), then the waves through LDS, and write
  // the split's unnormalised partial (max, sum, output).
  // One merge step with the row group OFF lanes away; the pair's order may
  // differ between the two lanes, and the merge is symmetric in it.
  auto merge_step = [&](auto off_c, int x) {
    constexpr int OFF = decltype(off_c)::value;
    float ma, mb, la, lb;
    xor_pair<OFF>(m_run[x], ma, mb);
    xor_pair<OFF>(l_run[x], la, lb);
    const float M = fmaxf(ma, mb);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float wa = __builtin_amdgcn_exp2f(ma - Mu);
    const float wb = __builtin_amdgcn_exp2f(mb - Mu);
    l_run[x] = la * wa + lb * wb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float oa, ob;
      xor_pair<OFF>(o[x][e], oa, ob);
      o[x][e] = oa * wa + ob * wb;
    }
    m_run[x] = M;
  };
  static_assert(LPR == 8 || LPR == 16, "row groups of 8 or 16 lanes");
#pragma unroll
  for (int x = 0; x < NH; ++x) {
    if constexpr (LPR == 8) merge_step(std::integral_constant<int, 8>{}, x);
    merge_step(std::integral_constant<int, 16>{}, x);
    merge_step(std::integral_constant<int, 32>{}, x);
    if (l < LPR) {
      if (dl == 0) {
        sm_m[wave][x] = m_run[x];
        sm_l[wave][x] = l_run[x];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wave][x][dl * 8 + e] = o[x][e];
    }
  }
  __syncthreads();
  for (int z = tid; z < NH * D; z += kDecThreads) {
    const int x = z / D, d = z % D;
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) M = fmaxf(M, sm_m[r][x]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f, Ov = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float w = __builtin_amdgcn_exp2f(sm_m[r][x] - Mu);
      L += w * sm_l[r][x];
      Ov += w * sm_o[r][x][d];
    }
    if (n_split == 1) {
      // a single split is the whole result: normalise here (the same
      // arithmetic as combine_kernel with one partial) and skip the combine
      const size_t bh = (size_t)b * Hq + h0 + x;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      out[bh * D + d] = f32_to_bf16(Ov * inv);
      if (lse != nullptr && d == 0) lse[bh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    } else {
      float* pp = part + (((size_t)b * Hq + h0 + x) * n_split + s) * (D + 2);
      if (d == 0) {
        pp[0] = M;
        pp[1] = L;
      }
      pp[2 + d] = Ov;
    }
  }
}

template <int D>
__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ part, int n_split,
                                                     uint16_t* __restrict__ out,
                                                     float* __restrict__ lse) {
  // one wave per (b, h): the lanes read the splits' (max, sum) pairs in
  // parallel, the weights go through LDS (an empty split holds max = -inf:
  // weight 0), and the output pass loads the splits' outputs in batches
  __shared__ float w_s[kMaxSplit];
  const int bh = blockIdx.x, l = threadIdx.x;
  const float* pp = part + (size_t)bh * n_split * (D + 2);
  float M = -INFINITY;
  for (int s = l; s < n_split; s += 64) M = fmaxf(M, pp[(size_t)s * (D + 2)]);
  M = wave_max(M);
  const float Mu = M == -INFINITY ? 0.f : M;
  float L = 0.f;
  for (int s = l; s < n_split; s += 64) {
    const float m = pp[(size_t)s * (D + 2)];
    const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - Mu);
    L += w * pp[(size_t)s * (D + 2) + 1];
    w_s[s] = w;
  }
  L = wave_sum(L);
  __syncthreads();
  constexpr int DPL = D / 64;
  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  // kCombineBatch splits' outputs are loaded together, then added in split
  // order.  Every split wrote a finite output (an empty one 0, with weight 0),
  // so adding w * o for a zero weight leaves the sum as skipping it would.
  constexpr int kCombineBatch = 8;
  for (int s0 = 0; s0 < n_split; s0 += kCombineBatch) {
    float v[kCombineBatch][DPL];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const float* ps = pp + (size_t)min(s0 + u, n_split - 1) * (D + 2);
#pragma unroll
      for (int e = 0; e < DPL; ++e) v[u][e] = ps[2 + l * DPL + e];
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const float w = s0 + u < n_split ? w_s[s0 + u] : 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += w * v[u][e];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) out[(size_t)bh * D + l * DPL + e] = f32_to_bf16(acc[e] * inv);
  if (lse != nullptr && l == 0) lse[bh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

int decode_pick_split(const DecodeDims& d, int mode, int k, int n_split) {
  if (n_split > 0) return n_split;
  const bool per_head = mode == FSA_SEL_INDEX || mode == FSA_SEL_INDEX_SCORED;
  const int items = per_head ? d.B * d.Hq : d.B * d.Hkv;
  const bool listed = per_head || mode == FSA_SEL_INDEX_KV;
  const int len = listed ? k : d.max_seq_len;
  // aim for >= 2048 workgroups (1024 for listed positions: a single split then
  // writes the output itself, with no combine launch) and >= 256 positions
  // per split
  const int target = listed ? 1024 : 2048;
  int ns = (target + items - 1) / items;
  const int cap = (len + kMinSplitPositions - 1) / kMinSplitPositions;
  if (ns > cap) ns = cap;
  return ns < 1 ? 1 : ns;
}

size_t decode_ws_bytes(const DecodeDims& d, int mode, int k, int n_split) {
  const int ns = decode_pick_split(d, mode, k, n_split);
  return (size_t)d.B * d.Hq * ns * (d.D + 2) * sizeof(float);
}

template <int D>
static hipError_t launch_dec_d(const void* q, const void* kp, const void* vp, const int32_t* pt,
                               const int32_t* sl, const DecodeDims& d, int mode,
                               const int32_t* idx, const float* scores, int k, const int32_t* seg,
                               const int32_t* nseg, int max_seg, int ns, float sl2,
                               void* out, float* lse, float* part, hipStream_t st) {
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* Kp = static_cast<const uint16_t*>(kp);
  const uint16_t* Vp = static_cast<const uint16_t*>(vp);
  const int G = d.Hq / d.Hkv;
  if (mode == FSA_SEL_INDEX) {
    hipLaunchKernelGGL((decode_split_kernel<D, 1, FSA_SEL_INDEX>), dim3(d.B * d.Hq * ns),
                       dim3(kDecThreads), 0, st, Q, Kp, Vp, pt, sl, d.Hq, d.Hkv, d.max_pages,
                       d.num_pages, d.max_seq_len, idx, scores, k, seg, nseg, max_seg, ns, sl2,
                       part, static_cast<uint16_t*>(out), lse);
  } else if (mode == FSA_SEL_INDEX_SCORED) {
    hipLaunchKernelGGL((decode_split_kernel<D, 1, FSA_SEL_INDEX_SCORED>), dim3(d.B * d.Hq * ns),
                       dim3(kDecThreads), 0, st, Q, Kp, Vp, pt, sl, d.Hq, d.Hkv, d.max_pages,
                       d.num_pages, d.max_seq_len, idx, scores, k, seg, nseg, max_seg, ns, sl2,
                       part, static_cast<uint16_t*>(out), lse);
  } else {
#define FSA_DEC(GG, MM)                                                                        \
  hipLaunchKernelGGL((decode_split_kernel<D, GG, MM>), dim3(d.B * d.Hkv * ns), dim3(kDecThreads), \
                     0, st, Q, Kp, Vp, pt, sl, d.Hq, d.Hkv, d.max_pages, d.num_pages,           \
                     d.max_seq_len, idx, scores, k, seg, nseg, max_seg, ns, sl2, part,        \
                     static_cast<uint16_t*>(out), lse)
#define FSA_DEC_G(GG)                         \
  if (G == GG) {                              \
    if (mode == FSA_SEL_SEGMENT)              \
      FSA_DEC(GG, FSA_SEL_SEGMENT);           \
    else if (mode == FSA_SEL_INDEX_KV)        \
      FSA_DEC(GG, FSA_SEL_INDEX_KV);          \
    else                                      \
      FSA_DEC(GG, FSA_SEL_ALL);               \
  } else
    FSA_DEC_G(1) FSA_DEC_G(2) FSA_DEC_G(4) FSA_DEC_G(8) { return hipErrorInvalidValue; }
#undef FSA_DEC_G
#undef FSA_DEC
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  hipLaunchKernelGGL(combine_kernel<D>, dim3(d.B * d.Hq), dim3(64), 0, st, part, ns,
                     static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

hipError_t launch_decode_attn(const void* q, const void* kpool, const void* vpool,
                              const int32_t* pt, const int32_t* sl, const DecodeDims& d,
                              int mode, const int32_t* idx, const float* scores, int k,
                              const int32_t* seg, const int32_t* nseg, int max_seg, int n_split,
                              float scale, void* out, float* lse, void* ws, hipStream_t st) {
  const int ns = decode_pick_split(d, mode, k, n_split);
  float* part = static_cast<float*>(ws);
  const float sl2 = scale * kLog2e;
  if (d.D == 128)
    return launch_dec_d<128>(q, kpool, vpool, pt, sl, d, mode, idx, scores, k, seg, nseg,
                             max_seg, ns, sl2, out, lse, part, st);
  if (d.D == 64)
    return launch_dec_d<64>(q, kpool, vpool, pt, sl, d, mode, idx, scores, k, seg, nseg,
                            max_seg, ns, sl2, out, lse, part, st);
  return hipErrorInvalidValue;
}


// ---- the variant that allocates nothing ---------------------------------
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// serving loops that forbid it) get the split partials from a file-scope
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): the device address is looked up once per device, with that
// device current, and kept.  Every call on a GPU shares that GPU's array, so
// calls that overlap on one GPU race.  Nothing in it has to start at zero:
// every split of a launch writes its partial before the combine reads it.
namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t debug_flags_decode(uint32_t* flags, bool clear) {
  return debug_flags_of_tu(flags, clear);
}

}  // namespace fsa
