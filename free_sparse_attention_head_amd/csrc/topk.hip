// topk_indices: exact per-head top-k over a paged bf16 key cache.
//
// Kascade post, "What Kascade got right": an anchor layer computes exact
// Top-k key indices; "Head-aware is the key to accuracy": one set per
// attention head.  Raw scores q.k in fp32; ties go to the lower token index;
// the index set is written ascending.
//
// Kernels (stream-ordered):
//   1. fill_kernel: clears the per-row digit histograms (a plain store kernel,
//      safe under graph capture).
//   2. topk_score_kernel: streams K once from HBM through the page table; the
//      G query heads of a KV head share every 256-byte key row (16 lanes x
//      16 bytes, v_dot2_f32_bf16 + DPP butterfly).  A workgroup scores one
//      tile of a row and keeps the tile's fp32 scores, and a histogram of the
//      top 11 bits of their order-preserving keys, in LDS.  At the end it
//      reads the row's histogram as it stands and takes as bound the bin of
//      the k-th largest key counted there (0 while fewer than k are counted).
//      Counts only grow, so any reading counts a subset of the row: its k-th
//      largest key is never above the row's, and the bound never exceeds the
//      bin b1 of the row's k-th largest key.  The tile then keeps only its
//      candidates, keys in bins >= bound, written (order key, index) in index
//      order as one list per tile, and adds its counts of bins >= bound to
//      the row's histogram, which is therefore exact from b1 up, the only
//      part the select reads.  Tiles run in order along the row, so later
//      tiles see tighter bounds and write few candidates.
//   3. topk_select_kernel: one 1024-thread workgroup per score row, reading
//      the row's candidate lists as one stream in index order.  Digit 1 comes
//      from the row histogram.  When few keys lie in or above the k-th key's
//      bin, one pass copies them to LDS and the rest runs there; otherwise
//      digits 2 (11 bits) and 3 (10 bits) are histogrammed over the
//      candidates sharing the prefix by re-reading the stream.  This yields
//      the exact k-th key K* and how many keys equal to K* are taken.  A
//      final pass in index order keeps key > K*, plus the first keys equal to
//      K*, compacting positions with workgroup scans so that the output is
//      ascending.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace fsa {

constexpr int kBins1 = 2048;      // digit 1: key bits 31..21
constexpr int kSelThreads = 1024;
constexpr int kTileScores = 8192;  // scores of a score workgroup's tile, staged in LDS (32 KB)
constexpr int kMaxSelTiles = kTopkMaxSeqLen / (kTileScores / 8);  // tiles of a row, at most

// tokens per score workgroup: the tile's scores of all its rows fit in LDS
constexpr int topk_tile(int rows) { return kTileScores / rows; }

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v) {
  for (size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x; x < n;
       x += (size_t)gridDim.x * blockDim.x)
    p[x] = v;
}

// POOL: one score row per KV head, the maximum of its G query heads' raw
// scores (a key counts if any head of the group rates it), instead of one
// row per query head.
//
// A workgroup scores one tile of TT tokens of one (sequence, KV head).  Its
// scores and digit-1 histograms stay in LDS until the tile is done: a wave
// issues no global store between its K row loads, so a load never waits
// behind a store's acknowledgement.
template <int D, int G, bool POOL>
__global__ __launch_bounds__(256) void topk_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kpool,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ sl, int B, int Hq, int Hkv,
    int max_pages, int num_pages, int max_seq_len, int k, int tiles, int cstride,
    uint32_t* __restrict__ ckey, uint16_t* __restrict__ cidx, uint32_t* __restrict__ ccnt,
    uint32_t* __restrict__ hist) {
  constexpr int LPR = D / 8, RG = 64 / LPR, NSLOT = 4 * RG;
  constexpr int RB = 8;                  // rows per lane group per step
  constexpr int STEP = NSLOT * RB;       // tokens per step
  constexpr int GR = POOL ? 1 : G;       // score rows per KV head
  constexpr int TT = topk_tile(GR);      // tokens per tile
  static_assert(TT % STEP == 0, "tile of whole steps");
  // page ids of the tile plus the two steps that the last loads run past it
  constexpr int TPAGES = (TT + 2 * STEP) / 16;
  // digit-1 counts of bins 2w and 2w+1 share word w (a tile holds < 65536
  // keys); the last word takes the adds of lanes with nothing to count
  constexpr int HW = GR * kBins1 / 2, TRASH = HW;
  __shared__ uint32_t lh[HW + 1];
  __shared__ __align__(16) float ssc[GR * TT + 4];  // + a spare quad for idle lanes
  __shared__ int pg[TPAGES];
  __shared__ int scan_tmp[17];
  // tile-major order: the first tiles of every row are scored first, so the
  // rows' histograms already hold several tiles when later tiles bound
  // their candidates
  const int tile = blockIdx.x / (B * Hkv);
  const int bg = blockIdx.x % (B * Hkv);
  const int g = bg % Hkv, b = bg / Hkv;
  const int n = min(max(sl[b], 0), max_seq_len);
  const int t0 = tile * TT;
  if (t0 >= n) return;
  const int t1 = min(n, t0 + TT);
  const int tid = threadIdx.x, wave = tid >> 6, l = tid & 63;
  const int slot = wave * RG + l / LPR, dl = l % LPR;
  for (int x = tid; x <= TRASH; x += 256) lh[x] = 0u;
  // the tile's page ids, read once and coalesced: row loads then depend on an
  // LDS read instead of a second global load (bad ids become -1: skipped)
  const int32_t* ptb = pt + (size_t)b * max_pages;
  for (int x = tid; x < TPAGES; x += 256) {
    const int tok = t0 + x * 16;
    int p = tok < t1 ? ptb[tok >> 4] : -1;
    pg[x] = (p >= 0 && p < num_pages) ? p : -1;
  }
  uint4 qv[G];
#pragma unroll
  for (int x = 0; x < G; ++x)
    qv[x] = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + g * G + x) * D + dl * 8);
  __syncthreads();

  // A lane group's RB rows are consecutive tokens inside one 16-token page.
  // Every wave issues all of its row loads on every step, with no branch
  // around them (rows of a missing page, or past the tile, are read from page
  // 0; their scores are replaced by 0 or never kept): the compiler then knows
  // how many loads are younger than each row buffer and waits for that
  // buffer alone.
  auto page_of = [&](int base) { return pg[(base + slot * RB - t0) >> 4]; };
  auto load_rows = [&](int base, uint4 (&kr)[RB]) {
    const int tok0 = base + slot * RB;
    const int page = max(page_of(base), 0);
    const size_t row0 = ((size_t)page * Hkv + g) * 16 + (tok0 & 15);
#pragma unroll
    for (int r = 0; r < RB; ++r)
      kr[r] = *reinterpret_cast<const uint4*>(kpool + (row0 + r) * D + dl * 8);
  };
  // After the group sums every lane of a row group holds all GR*RB scores of
  // its RB consecutive tokens, as GR*NQ quads of four consecutive tokens of
  // one score row.  Quad c = j*LPR + dl is kept by lane dl of the group with
  // its j-th 16-byte LDS store: row c / NQ, tokens 4*(c % NQ) .. +3.
  constexpr int NQ = RB / 4, NJ = (GR * NQ + LPR - 1) / LPR;
  static_assert(RB % 4 == 0, "quads of tokens");
  auto score_rows = [&](int base, const uint4 (&kr)[RB]) {
    float sc[GR][RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      if constexpr (POOL) {
        float m = group_sum<LPR>(dot8_bf16(qv[0], kr[r], 0.f));
#pragma unroll
        for (int x = 1; x < G; ++x) m = fmaxf(m, group_sum<LPR>(dot8_bf16(qv[x], kr[r], 0.f)));
        sc[0][r] = m;
      } else {
#pragma unroll
        for (int x = 0; x < G; ++x) sc[x][r] = group_sum<LPR>(dot8_bf16(qv[x], kr[r], 0.f));
      }
    }
    const bool page_ok = page_of(base) >= 0;  // a missing page scores 0
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = j * LPR + dl;
      const int sx = c / NQ, sq = c % NQ;        // the quad's score row and place
      const int tq = base + slot * RB + 4 * sq;  // its first token
      floatx4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float w = 0.f;
#pragma unroll
        for (int cc = j * LPR; cc < GR * NQ && cc < (j + 1) * LPR; ++cc)
          w = c == cc ? sc[cc / NQ][4 * (cc % NQ) + e] : w;
        v[e] = page_ok ? w + 0.0f : 0.f;  // + 0 folds -0 onto +0
      }
      const bool ok = (c < GR * NQ) & (tq < t1);
      *reinterpret_cast<floatx4*>(&ssc[ok ? sx * TT + (tq - t0) : GR * TT]) = v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t bin = (uint32_t)sx * kBins1 + (order_key(v[e]) >> 21);
        const bool oke = ok & (tq + e < t1);
        atomicAdd(&lh[oke ? bin >> 1 : TRASH], (bin & 1) ? 0x10000u : 1u);
      }
    }
  };
  // two row buffers: the next step's rows are in flight while this step is scored
  uint4 ka[RB], kb[RB];
  load_rows(t0, ka);
  int base = t0;
  for (; base + STEP < t1; base += 2 * STEP) {
    // scheduling barriers keep each step's scoring after the loads of the
    // next step and before the loads after it, so no score instruction waits
    // for rows that were only just requested
    load_rows(base + STEP, kb);
    __builtin_amdgcn_sched_barrier(0);
    score_rows(base, ka);
    __builtin_amdgcn_sched_barrier(0);
    load_rows(base + 2 * STEP, ka);  // past the tile: rows of page 0, never kept
    __builtin_amdgcn_sched_barrier(0);
    score_rows(base + STEP, kb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (base < t1) score_rows(base, ka);
  __syncthreads();
  const size_t row0 = POOL ? (size_t)b * Hkv + g : (size_t)b * Hq + (size_t)g * G;
  constexpr int BPT = kBins1 / 256;  // histogram bins per thread
  constexpr int PER = TT / 256;      // tile tokens per thread
  // the compaction below reads each thread's tokens as 16-byte quads
  static_assert(PER >= 4 && PER % 4 == 0, "tile of whole 16-byte quads per thread");
  __shared__ uint32_t sbound[GR];
  const int nt = t1 - t0;
  // Candidate bounds: per row, the bin of the k-th largest key counted in
  // the row's histogram as it stands (0 while fewer than k keys are
  // counted).  Thread t reads bins [top, top + BPT), the threads in
  // descending bin order; all rows' reads are issued together.
  const int top = kBins1 - BPT * (tid + 1);
  uint32_t hc[GR][BPT];
#pragma unroll
  for (int x = 0; x < GR; ++x)
#pragma unroll
    for (int e = 0; e < BPT; ++e)
      hc[x][e] = __hip_atomic_load(hist + (row0 + x) * kBins1 + top + e, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  if (tid < GR) sbound[tid] = 0u;
#pragma unroll
  for (int x = 0; x < GR; ++x) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) c += (int)hc[x][e];
    int tot;
    const int above = block_excl_scan(c, scan_tmp, &tot);  // keys in higher bins
    if (above < k && k <= above + c) {
      int acc = above;
#pragma unroll
      for (int e = BPT - 1; e >= 0; --e) {
        acc += (int)hc[x][e];
        if (acc >= k) {
          sbound[x] = (uint32_t)(top + e);
          break;
        }
      }
    }
  }
  __syncthreads();
  // The tile's counts into the rows' histograms, from each row's bound up:
  // the select reads exact counts only from the k-th key's bin up, and that
  // bin is at or above every tile's bound.
  for (int y = tid; y < HW; y += 256) {
    const int x = y / (kBins1 / 2), bin = 2 * (y % (kBins1 / 2));
    const uint32_t cc = lh[y], bound = sbound[x];
    uint32_t* hr = hist + (row0 + x) * kBins1 + bin;
    if ((cc & 0xffffu) && (uint32_t)bin >= bound) atomicAdd(hr, cc & 0xffffu);
    if ((cc >> 16) && (uint32_t)(bin + 1) >= bound) atomicAdd(hr + 1, cc >> 16);
  }
  // Each row's candidates of this tile, compacted in index order: thread t
  // takes tokens [t*PER, t*PER + PER), a workgroup scan places them.
  const int j0 = tid * PER;
#pragma unroll 1
  for (int x = 0; x < GR; ++x) {
    const uint32_t bound = sbound[x];
    uint32_t key[PER];
    int nc = 0;
#pragma unroll
    for (int e = 0; e < PER; e += 4) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(&ssc[x * TT + j0 + e]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        key[e + u] = order_key(v[u]);
        nc += (j0 + e + u < nt && (key[e + u] >> 21) >= bound) ? 1 : 0;
      }
    }
    int ntot;
    int pos = block_excl_scan(nc, scan_tmp, &ntot);
    const size_t cbase = (row0 + x) * (size_t)cstride + t0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (j0 + e < nt && (key[e] >> 21) >= bound) {
        ckey[cbase + pos] = key[e];
        cidx[cbase + pos] = (uint16_t)(j0 + e);
        ++pos;
      }
    }
    if (tid == 0) ccnt[(row0 + x) * tiles + tile] = (uint32_t)ntot;
  }
}

struct TopkShared {
  uint32_t hist[kBins1];
  int scan[17];
  int dig, above;
};

// Among nbins (1024 or 2048) histogram bins in LDS, find the bin holding the
// kk-th largest element (bins scanned from the top).  Every thread calls it.
__device__ void find_digit(TopkShared& sh, int nbins, int kk, int& digit, int& above) {
  const int t = threadIdx.x;
  const int per = nbins / kSelThreads;  // 1 or 2, bins owned by thread t, descending
  const int top = nbins - 1 - per * t;
  int c0 = (int)sh.hist[top];
  int c1 = per == 2 ? (int)sh.hist[top - 1] : 0;
  int tot;
  const int exc = block_excl_scan(c0 + c1, sh.scan, &tot);
  if (exc < kk && kk <= exc + c0 + c1) {
    if (kk <= exc + c0) {
      sh.dig = top;
      sh.above = exc;
    } else {
      sh.dig = top - 1;
      sh.above = exc + c0;
    }
  }
  __syncthreads();
  digit = sh.dig;
  above = sh.above;
  __syncthreads();
}

// A row's candidates as one stream in index order: the lists of its tiles
// one after another.  seg[i] = candidates in tiles before i (seg[nt] = all).
struct CandStream {
  const uint32_t* key;  // the row's candidate keys, tile i's list at i * tt
  const uint16_t* idx;  // their indices inside the tile
  const int* seg;       // LDS
  int nt, tt, m;
  // element p < m: the tile holding it is the last i with seg[i] <= p;
  // hint = a tile at or before it
  __device__ void at(int p, int& hint, uint32_t& k, int& tok) const {
    int lo = hint, hi = nt - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg[mid] <= p) lo = mid; else hi = mid - 1;
    }
    hint = lo;
    const int o = lo * tt + (p - seg[lo]);
    k = key[o];
    tok = lo * tt + (int)idx[o];
  }
  // this thread's four consecutive elements from p0 (invalid past the end)
  __device__ void quad(int p0, uint32_t (&k)[4], int (&tok)[4], bool (&valid)[4]) const {
    int hint = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      valid[e] = p0 + e < m;
      k[e] = 0u;
      tok[e] = -1;
      if (valid[e]) at(p0 + e, hint, k[e], tok[e]);
    }
  }
};

// Fast path, used when the keys in or above the k-th key's top-11-bit bin
// number at most kCandCap: one pass over the candidate stream copies them
// (key, index) into LDS in index order; digits 2-3 and the ordered output
// then run on LDS only.  `need` = how many keys of bin b1 still have to be
// taken.
constexpr int kCandCap = 6144;
__device__ void select_from_candidates(const CandStream& cs, int k, uint32_t b1, int need,
                                       TopkShared& sh, int32_t* __restrict__ out,
                                       float* __restrict__ kth) {
  __shared__ uint32_t ck[kCandCap];
  __shared__ int ci[kCandCap];
  const int t = threadIdx.x;
  int ncand = 0;
  for (int base = 0; base < cs.m; base += 4 * kSelThreads) {
    uint32_t key[4];
    int tok[4];
    bool f[4];
    cs.quad(base + 4 * t, key, tok, f);
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = f[e] && (key[e] >> 21) >= b1;
      c += f[e] ? 1 : 0;
    }
    int tot;
    int pos = ncand + block_excl_scan(c, sh.scan, &tot);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (f[e]) {
        ck[pos] = key[e];
        ci[pos] = tok[e];
        ++pos;
      }
    ncand += tot;
  }
  __syncthreads();
  // digits 2 (11 bits) and 3 (10 bits) among the candidates of bin b1
  const int E = (ncand + kSelThreads - 1) / kSelThreads;
  const int e0 = min(ncand, t * E), e1 = min(ncand, e0 + E);
  uint32_t prefix = b1 << 21, pmask = 0xffe00000u;
  const int shifts[2] = {10, 0};
  const int nbins[2] = {2048, 1024};
  for (int pass = 0; pass < 2; ++pass) {
    for (int x = t; x < nbins[pass]; x += kSelThreads) sh.hist[x] = 0u;
    __syncthreads();
    const uint32_t dmask = (uint32_t)nbins[pass] - 1u;
    for (int e = e0; e < e1; ++e) {
      const uint32_t key = ck[e];
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shifts[pass]) & dmask], 1u);
    }
    __syncthreads();
    int d, above;
    find_digit(sh, nbins[pass], need, d, above);
    need -= above;
    prefix |= (uint32_t)d << shifts[pass];
    pmask |= dmask << shifts[pass];
  }
  const uint32_t ks = prefix;
  // ordered output: candidates are in index order and each thread owns a
  // contiguous range, so one scan of (equal, greater) counts places them
  int neq = 0, ngt = 0;
  for (int e = e0; e < e1; ++e) {
    neq += ck[e] == ks ? 1 : 0;
    ngt += ck[e] > ks ? 1 : 0;
  }
  int tot;
  const int ex = block_excl_scan((neq << 16) | ngt, sh.scan, &tot);
  int eq_rank = ex >> 16;
  int pos = (ex & 0xffff) + min(eq_rank, need);
  for (int e = e0; e < e1; ++e) {
    const uint32_t key = ck[e];
    if (key > ks) {
      if (pos < k) out[pos] = ci[e];
      ++pos;
    } else if (key == ks) {
      if (eq_rank < need) {
        if (pos < k) out[pos] = ci[e];
        ++pos;
      }
      ++eq_rank;
    }
  }
  if (kth != nullptr && t == 0) *kth = key_to_float(ks);
}

// One workgroup per score row; rows_per_b rows (query heads, or KV heads when
// pooled) per sequence.
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(
    const uint32_t* __restrict__ ckey, const uint16_t* __restrict__ cidx,
    const uint32_t* __restrict__ ccnt, const uint32_t* __restrict__ hist,
    const int32_t* __restrict__ sl, int rows_per_b, int max_seq_len, int tt, int tiles,
    int cstride, int k, int32_t* __restrict__ idx, float* __restrict__ kth) {
  __shared__ TopkShared sh;
  __shared__ int seg[kMaxSelTiles + 1];
  const int row = blockIdx.x, b = row / rows_per_b;
  const int n = min(max(sl[b], 0), max_seq_len);
  const int t = threadIdx.x;
  int32_t* out = idx + (size_t)row * k;
  if (n < k) {
    for (int x = t; x < k; x += kSelThreads) out[x] = x < n ? x : -1;
    if (kth != nullptr && t == 0) kth[row] = -INFINITY;
    return;
  }
  // the candidate stream: exclusive prefix of the tiles' list lengths
  const int nt = (n + tt - 1) / tt;
  {
    constexpr int TPT = kMaxSelTiles / kSelThreads;  // tiles per thread, consecutive
    int c[TPT], sum = 0;
#pragma unroll
    for (int e = 0; e < TPT; ++e) {
      const int i = t * TPT + e;
      c[e] = i < nt ? (int)ccnt[(size_t)row * tiles + i] : 0;
      sum += c[e];
    }
    int tot;
    int run = block_excl_scan(sum, sh.scan, &tot);
#pragma unroll
    for (int e = 0; e < TPT; ++e) {
      const int i = t * TPT + e;
      if (i <= nt) seg[i] = run;
      run += c[e];
    }
    if (t == 0) seg[nt] = tot;
  }
  __syncthreads();
  const CandStream cs{ckey + (size_t)row * cstride, cidx + (size_t)row * cstride, seg, nt, tt,
                      seg[nt]};
  // digit 1 from the row histogram (exact from the k-th key's bin up)
  for (int x = t; x < kBins1; x += kSelThreads) sh.hist[x] = hist[(size_t)row * kBins1 + x];
  __syncthreads();
  int kk = k, d, above;
  find_digit(sh, kBins1, kk, d, above);
  kk -= above;
  const int cand = above + (int)sh.hist[d];
  __syncthreads();
  if (cand <= kCandCap) {
    select_from_candidates(cs, k, (uint32_t)d, kk, sh, out, kth ? kth + row : nullptr);
    return;
  }
  // general path: refine digits 2 and 3 by re-reading the candidate stream
  uint32_t prefix = (uint32_t)d << 21, pmask = 0xffe00000u;
  const int shifts[2] = {10, 0};
  const int nbins[2] = {2048, 1024};
  for (int pass = 0; pass < 2; ++pass) {
    for (int x = t; x < nbins[pass]; x += kSelThreads) sh.hist[x] = 0u;
    __syncthreads();
    const uint32_t dmask = (uint32_t)nbins[pass] - 1u;
    for (int p0 = 4 * t; p0 < cs.m; p0 += 4 * kSelThreads) {
      uint32_t key[4];
      int tok[4];
      bool valid[4];
      cs.quad(p0, key, tok, valid);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (valid[e] && (key[e] & pmask) == prefix)
          atomicAdd(&sh.hist[(key[e] >> shifts[pass]) & dmask], 1u);
    }
    __syncthreads();
    find_digit(sh, nbins[pass], kk, d, above);
    kk -= above;
    prefix |= (uint32_t)d << shifts[pass];
    pmask |= dmask << shifts[pass];
  }
  const uint32_t kstar = prefix;
  const int need_eq = kk;
  // output pass in index order: keep key > K*, and the first need_eq keys == K*
  int eq_before = 0, out_before = 0;
  for (int base = 0; base < cs.m; base += 4 * kSelThreads) {
    uint32_t key[4];
    int tok[4];
    bool valid[4];
    cs.quad(base + 4 * t, key, tok, valid);
    int neq = 0, ngt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      neq += (valid[e] && key[e] == kstar) ? 1 : 0;
      ngt += (valid[e] && key[e] > kstar) ? 1 : 0;
    }
    // one scan carries both counts: equal keys in the high half
    int tot;
    const int ex = block_excl_scan((neq << 16) | ngt, sh.scan, &tot);
    int eq_rank = eq_before + (ex >> 16);
    int gt_rank = ex & 0xffff;
    // output position = keys kept before this thread's first element: all of
    // out_before, this iteration's greater keys before it, and the equal keys
    // before it that still fit under need_eq
    int pos = out_before + gt_rank + min(eq_rank, need_eq) - min(eq_before, need_eq);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!valid[e]) continue;
      if (key[e] > kstar) {
        if (pos < k) out[pos] = tok[e];
        ++pos;
      } else if (key[e] == kstar) {
        if (eq_rank < need_eq) {
          if (pos < k) out[pos] = tok[e];
          ++pos;
        }
        ++eq_rank;
      }
    }
    const int teq = tot >> 16, tgt = tot & 0xffff;
    out_before += tgt + max(0, min(teq, need_eq - eq_before));
    eq_before += teq;
  }
  if (kth != nullptr && t == 0) kth[row] = key_to_float(kstar);
}

// Workspace: candidate keys and tile indices (one TT-entry list per tile of
// every score row), list lengths, and the rows' digit-1 histograms.
struct TopkLayout {
  int rows, tt, tiles, cstride;
  size_t idx_off, cnt_off, hist_off, bytes;
};

static TopkLayout topk_layout(const DecodeDims& d, bool pooled) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  TopkLayout L;
  L.rows = d.B * (pooled ? d.Hkv : d.Hq);
  L.tt = topk_tile(pooled ? 1 : d.Hq / d.Hkv);
  L.tiles = (d.max_seq_len + L.tt - 1) / L.tt;
  L.cstride = L.tiles * L.tt;
  L.idx_off = up((size_t)L.rows * L.cstride * sizeof(uint32_t));
  L.cnt_off = L.idx_off + up((size_t)L.rows * L.cstride * sizeof(uint16_t));
  L.hist_off = L.cnt_off + up((size_t)L.rows * L.tiles * sizeof(uint32_t));
  L.bytes = L.hist_off + (size_t)L.rows * kBins1 * sizeof(uint32_t);
  return L;
}

size_t topk_ws_bytes(const DecodeDims& d, int k) {
  (void)k;
  const size_t a = topk_layout(d, false).bytes, b = topk_layout(d, true).bytes;
  return a > b ? a : b;
}

hipError_t launch_topk(const void* q, const void* kpool, const int32_t* pt, const int32_t* sl,
                       const DecodeDims& d, int k, bool pooled, int32_t* idx, float* kth, void* ws,
                       hipStream_t st) {
  const int rows_per_b = pooled ? d.Hkv : d.Hq;  // score rows (and index sets) per sequence
  const TopkLayout L = topk_layout(d, pooled);
  char* w = static_cast<char*>(ws);
  uint32_t* ckey = reinterpret_cast<uint32_t*>(w);
  uint16_t* cidx = reinterpret_cast<uint16_t*>(w + L.idx_off);
  uint32_t* ccnt = reinterpret_cast<uint32_t*>(w + L.cnt_off);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w + L.hist_off);
  const size_t nh = (size_t)L.rows * kBins1;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((nh + 255) / 256 < 4096 ? (nh + 255) / 256 : 4096)),
                     dim3(256), 0, st, hist, nh, 0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = d.Hq / d.Hkv;
  const uint16_t* Q = static_cast<const uint16_t*>(q);
  const uint16_t* Kp = static_cast<const uint16_t*>(kpool);
  const dim3 grid(d.B * d.Hkv * L.tiles);
#define FSA_TS(DD, GG, PP)                                                                   \
  hipLaunchKernelGGL((topk_score_kernel<DD, GG, PP>), grid, dim3(256), 0, st, Q, Kp, pt, sl,  \
                     d.B, d.Hq, d.Hkv, d.max_pages, d.num_pages, d.max_seq_len, k, L.tiles,    \
                     L.cstride, ckey, cidx, ccnt, hist)
#define FSA_TS_G(DD, GG)                  \
  if (d.D == DD && G == GG) {             \
    if (pooled)                           \
      FSA_TS(DD, GG, true);               \
    else                                  \
      FSA_TS(DD, GG, false);              \
  } else
  FSA_TS_G(128, 1) FSA_TS_G(128, 2) FSA_TS_G(128, 4) FSA_TS_G(128, 8) FSA_TS_G(64, 1)
  FSA_TS_G(64, 2) FSA_TS_G(64, 4) FSA_TS_G(64, 8) { return hipErrorInvalidValue; }
#undef FSA_TS_G
#undef FSA_TS
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_select_kernel, dim3(d.B * rows_per_b), dim3(kSelThreads), 0, st, ckey,
                     cidx, ccnt, hist, sl, rows_per_b, d.max_seq_len, L.tt, L.tiles, L.cstride, k,
                     idx, kth);
  return hipGetLastError();
}

}  // namespace fsa
