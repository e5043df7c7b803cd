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
//      tile of a row.  Before its first scores it reads the row's histogram
//      of the top 11 bits of the order-preserving keys as it stands (64
//      coarse buckets of 32 bins first, then the 32 bins of one bucket) and
//      takes as bound the bin of the k-th largest key counted there (0 while
//      fewer than k are counted).  Counts only grow, and a bin never counts
//      more keys than the row holds in it, so any reading counts a subset of
//      the row: the bound never exceeds the bin b1 of the row's k-th largest
//      key.  The tile keeps its fp32 scores in LDS and histograms only keys
//      in bins >= bound; at its end it writes those keys, its candidates, as
//      (order key, index) in index order as one list per tile, and adds their
//      counts to the row's histogram (both levels), which is therefore exact
//      from b1 up, the only part the select reads.  Tiles run in order along
//      the row, so later tiles see tighter bounds and keep few candidates.
//   3. topk_select_kernel: one 1024-thread workgroup per score row, reading
//      the row's candidate lists as one stream in index order.  Digit 1 comes
//      from the row histogram.  When few keys lie in or above the k-th key's
//      bin, one pass copies them to LDS and the rest runs there; otherwise
//      digits 2 (11 bits) and 3 (10 bits) are histogrammed over the
//      candidates sharing the prefix by re-reading the stream.  This yields
//      the exact k-th key K* and how many keys equal to K* are taken.  A
//      final pass in index order keeps key > K*, plus the first keys equal to
//      K*, ranking positions with wave ballots and one workgroup scan per
//      pass so that the output is ascending.  Each load instruction of a
//      pass reads 64 consecutive list entries.
#include <limits.h>
#include <math.h>

#include "common.h"
#include "launch.h"

namespace fsa {

constexpr int kBins1 = 2048;      // digit 1: key bits 31..21
constexpr int kCoarse = 64;       // coarse buckets of digit 1 (32 bins each)
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
  // digit-1 counts of bins 2w and 2w+1 share word w (a tile holds < 65536 keys)
  constexpr int HW = GR * kBins1 / 2;
  __shared__ __align__(16) uint32_t lh[HW];
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
  for (int x = tid; x < HW; x += 256) lh[x] = 0u;
  // the tile's page ids, read once and coalesced: row loads then depend on an
  // LDS read instead of a second global load (bad ids become -1: skipped)
  const int32_t* ptb = pt + (size_t)b * max_pages;
  for (int x = tid; x < TPAGES; x += 256) {
    const int tok = t0 + x * 16;
    int p = tok < t1 ? ptb[tok >> 4] : -1;
    FSA_DEBUG_RAISE(tok < t1 && (p < 0 || p >= num_pages), FSA_DBG_PAGE_ID);
    pg[x] = (p >= 0 && p < num_pages) ? p : -1;
  }
  uint4 qv[G];
#pragma unroll
  for (int x = 0; x < G; ++x)
    qv[x] = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + g * G + x) * D + dl * 8);
  const size_t row0 = POOL ? (size_t)b * Hkv + g : (size_t)b * Hq + (size_t)g * G;
  const int rows_total = B * (POOL ? Hkv : Hq);
  uint32_t* coarse = hist + (size_t)rows_total * kBins1;  // [rows, kCoarse] after the bins
  constexpr int BPC = kBins1 / kCoarse;                   // bins per coarse bucket
  static_assert(kCoarse == 64 && BPC <= 64, "one coarse bucket per lane");
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
    const size_t prow = ((size_t)page * Hkv + g) * 16 + (tok0 & 15);
#pragma unroll
    for (int r = 0; r < RB; ++r)
      kr[r] = *reinterpret_cast<const uint4*>(kpool + (prow + r) * D + dl * 8);
  };
  __shared__ uint32_t sbound[GR];
  __syncthreads();  // the tile's page ids are in LDS
  // two row buffers: the next step's rows are in flight while this step is
  // scored; the first step's rows are requested before the bounds are read
  uint4 ka[RB], kb[RB];
  load_rows(t0, ka);
  // Candidate bounds, read before the tile is scored: per row, the bin of the
  // k-th largest key counted in the row's histogram as it stands (0 while
  // fewer than k keys are counted).  Wave w takes rows w, w + 4, ...: lane l
  // reads coarse bucket 63 - l (descending), a wave scan finds the bucket of
  // the k-th key, then lanes 0..BPC-1 read that bucket's bins, descending.
  for (int x = wave; x < GR; x += 4) {
    const uint32_t cb = __hip_atomic_load(coarse + (row0 + x) * kCoarse + (kCoarse - 1 - l),
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int inc = wave_incl_scan((int)cb);
    const uint64_t hit = __ballot(inc >= k);
    uint32_t bound = 0u;
    if (hit != 0ull) {
      const int lb = __ffsll((unsigned long long)hit) - 1;  // first lane reaching k
      const int above = __builtin_amdgcn_readlane(inc - (int)cb, lb);  // keys in higher buckets
      const int bucket = kCoarse - 1 - lb;
      uint32_t fc = 0u;
      if (l < BPC)
        fc = __hip_atomic_load(hist + (row0 + x) * kBins1 + bucket * BPC + (BPC - 1 - l),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int finc = above + wave_incl_scan((int)fc);
      const uint64_t fhit = __ballot(l < BPC && finc >= k);
      // The two levels are read at different times, so the bins may not add
      // up to the bucket's count; a bin reaching k, or else the bucket's
      // lowest bin, is then still at or below b1.
      const int lf = fhit != 0ull ? __ffsll((unsigned long long)fhit) - 1 : BPC - 1;
      bound = (uint32_t)(bucket * BPC + (BPC - 1 - lf));
    }
    if (l == 0) sbound[x] = bound;
  }
  __syncthreads();

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
      const uint32_t bnd = sbound[sx < GR ? sx : 0];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t kb = order_key(v[e]) >> 21;
        const uint32_t bin = (uint32_t)sx * kBins1 + kb;
        // keys below the bound are never candidates: they are not counted
        if (ok & (tq + e < t1) & (kb >= bnd)) atomicAdd(&lh[bin >> 1], (bin & 1) ? 0x10000u : 1u);
      }
    }
  };
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
  const int nt = t1 - t0;
  // The tile's counts into the rows' histograms: the LDS counts hold only
  // keys at or above each row's bound, and the select reads exact counts only
  // from the k-th key's bin up, which is at or above every tile's bound.
  // Thread u takes one coarse bucket of one row: its BPC/2 count words, read
  // with 16-byte LDS loads all at once (one at a time they were a chain of
  // LDS round trips), then its bins and its total.
  constexpr int WPU = BPC / 2;  // count words per coarse bucket
  static_assert(WPU % 4 == 0, "buckets of whole 16-byte words");
  for (int u = tid; u < GR * kCoarse; u += 256) {
    const int x = u / kCoarse, cbk = u % kCoarse;
    uint4 cw[WPU / 4];
#pragma unroll
    for (int w = 0; w < WPU / 4; ++w)
      cw[w] = reinterpret_cast<const uint4*>(lh)[x * (kBins1 / 8) + cbk * (WPU / 4) + w];
    uint32_t tot = 0u;
#pragma unroll
    for (int w = 0; w < WPU; ++w) {
      const uint32_t cc = (w & 3) == 0 ? cw[w / 4].x : (w & 3) == 1 ? cw[w / 4].y
                        : (w & 3) == 2 ? cw[w / 4].z : cw[w / 4].w;
      // bins 2w and 2w+1 are adjacent words of the row's histogram: one
      // 64-bit add covers both (a bin never counts 2^32 keys: no carry)
      if (cc)
        atomicAdd(reinterpret_cast<unsigned long long*>(hist + (row0 + x) * kBins1 + cbk * BPC + 2 * w),
                  ((unsigned long long)(cc >> 16) << 32) | (cc & 0xffffu));
      tot += (cc & 0xffffu) + (cc >> 16);
    }
    if (tot) atomicAdd(coarse + (row0 + x) * kCoarse + cbk, tot);
  }
  // Each row's candidates of this tile, compacted in index order.
  if constexpr (GR >= 4) {
    // A wave per row: lane l reads quads l, l + 64, ... (consecutive 16-byte
    // LDS reads), one wave scan per 64 quads.  The candidates are compacted
    // in LDS first (keys in place over the row's scores: a candidate's place
    // never passes the quads still to be read; token offsets over the row's
    // histogram words, flushed above), then copied out with coalesced
    // stores; a lane's own candidates are consecutive, so stores straight
    // from the scan would touch every fourth element.
    static_assert(GR * TT <= 2 * HW, "token offsets fit over the histogram words");
    __syncthreads();  // every row's histogram words are flushed
#pragma unroll 1
    for (int x = wave; x < GR; x += 4) {
      const uint32_t bound = sbound[x];
      uint32_t* kst = reinterpret_cast<uint32_t*>(&ssc[x * TT]);
      uint16_t* ist = reinterpret_cast<uint16_t*>(lh) + x * TT;
      int done = 0;
#pragma unroll
      for (int it = 0; it < TT / 256; ++it) {
        const int j = 4 * (it * 64 + l);
        const floatx4 v = *reinterpret_cast<const floatx4*>(&ssc[x * TT + j]);
        uint32_t key[4];
        int nc = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          key[u] = order_key(v[u]);
          nc += (j + u < nt && (key[u] >> 21) >= bound) ? 1 : 0;
        }
        const int inc = wave_incl_scan(nc);
        int pos = done + inc - nc;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (j + u < nt && (key[u] >> 21) >= bound) {
            kst[pos] = key[u];
            ist[pos] = (uint16_t)(j + u);
            ++pos;
          }
        }
        done += __builtin_amdgcn_readlane(inc, 63);
      }
      const size_t cbase = (row0 + x) * (size_t)cstride + t0;
      for (int e = l; e < done; e += 64) {
        ckey[cbase + e] = kst[e];
        cidx[cbase + e] = ist[e];
      }
      if (l == 0) ccnt[(row0 + x) * tiles + tile] = (uint32_t)done;
    }
  } else {
    // fewer rows than waves: thread t takes tokens [t*PER, t*PER + PER), a
    // workgroup scan places them
    constexpr int PER = TT / 256;
    static_assert(PER >= 4 && PER % 4 == 0, "tile of whole 16-byte quads per thread");
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
  // elements p0, p0 + 64, ..., p0 + 64 (N - 1) (invalid past the end): one
  // tile search for the first, then a walk over the tile ends that the rest
  // cross (lists may be empty), so that all 2N loads are in flight together.
  // The 64 lanes of a wave take 64 consecutive positions, so each load
  // instruction reads consecutive list entries.
  template <int N>
  __device__ void strided(int p0, uint32_t (&k)[N], int (&tok)[N], bool (&valid)[N]) const {
    int tile = 0;
    if (p0 < m) {
      int lo = 0, hi = nt - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg[mid] <= p0) lo = mid; else hi = mid - 1;
      }
      tile = lo;
    }
    int start = seg[tile], next = seg[tile + 1];
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const int p = p0 + 64 * e;
      valid[e] = p < m;
      // p < m = seg[nt], so the walk stops at a tile <= nt - 1
      while (valid[e] && p >= next) {
        ++tile;
        start = next;
        next = seg[tile + 1];
      }
      const int o = tile * tt + (p - start);
      k[e] = valid[e] ? key[o] : 0u;
      tok[e] = valid[e] ? tile * tt + (int)idx[o] : -1;
    }
  }
};

// Fast path, used when the keys in or above the k-th key's top-11-bit bin
// number at most kCandCap: one pass over the candidate stream copies them
// (key, index) into LDS in index order; digits 2-3 and the ordered output
// then run on LDS only.  `need` = how many keys of bin b1 still have to be
// taken.
constexpr int kCandCap = 6144;
constexpr int kSelPer = 8;  // stream elements a thread takes per pass
__device__ void select_from_candidates(const CandStream& cs, int k, uint32_t b1, int need,
                                       TopkShared& sh, int32_t* __restrict__ out,
                                       float* __restrict__ sco, float* __restrict__ kth) {
  __shared__ uint32_t ck[kCandCap];
  __shared__ int ci[kCandCap];
  const int t = threadIdx.x;
  // A pass covers kSelPer * kSelThreads stream positions: wave w the
  // kSelPer * 64 from base + w * kSelPer * 64, lane l every 64th of them
  // from l.  Ranks inside the wave come from ballots (element e of every
  // lane precedes element e + 1 of any), the waves' offsets from one scan.
  const int lane = t & 63, wave = t >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  int ncand = 0;
  for (int base = 0; base < cs.m; base += kSelPer * kSelThreads) {
    uint32_t key[kSelPer];
    int tok[kSelPer];
    bool f[kSelPer];
    cs.strided(base + wave * kSelPer * 64 + lane, key, tok, f);
    int rank[kSelPer], wtot = 0;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
      f[e] = f[e] && (key[e] >> 21) >= b1;
      const uint64_t mk = __ballot(f[e]);
      rank[e] = wtot + __popcll(mk & below);
      wtot += __popcll(mk);
    }
    int tot;
    const int wo = __builtin_amdgcn_readlane(block_excl_scan(lane == 0 ? wtot : 0, sh.scan, &tot), 0);
#pragma unroll
    for (int e = 0; e < kSelPer; ++e)
      if (f[e]) {
        ck[ncand + wo + rank[e]] = key[e];
        ci[ncand + wo + rank[e]] = tok[e];
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
      if (pos < k) {
        out[pos] = ci[e];
        if (sco != nullptr) sco[pos] = key_to_float(key);
      }
      ++pos;
    } else if (key == ks) {
      if (eq_rank < need) {
        if (pos < k) {
          out[pos] = ci[e];
          if (sco != nullptr) sco[pos] = key_to_float(key);
        }
        ++pos;
      }
      ++eq_rank;
    }
  }
  if (kth != nullptr && t == 0) *kth = key_to_float(ks);
}

// One workgroup per score row; rows_per_b rows (query heads, or KV heads when
// pooled) per sequence.  A row's select is a chain of latencies, so rows in
// flight set the pace: two 1024-thread workgroups share a CU only while a
// wave holds at most 64 VGPRs and about 72 SGPRs (with 78 SGPRs, or 71
// VGPRs, a CU ran one), hence the register caps (surplus SGPRs go to VGPR
// lanes).
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_num_sgpr(72), amdgpu_num_vgpr(64))) void topk_select_kernel(
    const uint32_t* __restrict__ ckey, const uint16_t* __restrict__ cidx,
    const uint32_t* __restrict__ ccnt, const uint32_t* __restrict__ hist,
    const int32_t* __restrict__ sl, int rows_per_b, int max_seq_len, int tt, int tiles,
    int cstride, int k, int32_t* __restrict__ idx, float* __restrict__ scores,
    float* __restrict__ kth) {
  __shared__ TopkShared sh;
  // tile offsets of the candidate stream: tiles + 1 entries, sized at launch
  // (a static array for the longest supported row would take 32 KB of LDS
  // and halve the workgroups a CU holds)
  extern __shared__ int seg[];
  const int row = blockIdx.x, b = row / rows_per_b;
  const int t = threadIdx.x;
  // The sequence length, the tiles' list lengths and the row histogram are
  // read together (one round trip); lengths of tiles past the sequence's end
  // are dropped once its length is known.
  constexpr int TPT = kMaxSelTiles / kSelThreads;  // tiles per thread, consecutive
  constexpr int HPT = kBins1 / kSelThreads;        // histogram bins per thread
  static_assert(kMaxSelTiles % kSelThreads == 0 && kBins1 % kSelThreads == 0, "per-thread shares");
  const int n_in = sl[b];
  int c[TPT];
#pragma unroll
  for (int e = 0; e < TPT; ++e) {
    const int i = t * TPT + e;
    c[e] = i < tiles ? (int)ccnt[(size_t)row * tiles + i] : 0;
  }
  uint32_t hv[HPT];
#pragma unroll
  for (int x = 0; x < HPT; ++x) hv[x] = hist[(size_t)row * kBins1 + x * kSelThreads + t];
  const int n = min(max(n_in, 0), max_seq_len);
  int32_t* out = idx + (size_t)row * k;
  float* sco = scores != nullptr ? scores + (size_t)row * k : nullptr;
  if (n < k && sco == nullptr) {
    for (int x = t; x < k; x += kSelThreads) out[x] = x < n ? x : -1;
    if (kth != nullptr && t == 0) kth[row] = -INFINITY;
    return;
  }
  // the candidate stream: exclusive prefix of the tiles' list lengths
  const int nt = (n + tt - 1) / tt;
  {
    int sum = 0;
#pragma unroll
    for (int e = 0; e < TPT; ++e) {
      c[e] = t * TPT + e < nt ? c[e] : 0;
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
  if (n < k) {
    // every key is kept (no reading of the histogram ever counted k keys, so
    // every tile's bound was 0): the stream holds token x at position x
    for (int x = t; x < k; x += kSelThreads) {
      int hint = 0, tok = -1;
      uint32_t key = 0u;
      if (x < n) cs.at(x, hint, key, tok);
      out[x] = x < n ? tok : -1;
      sco[x] = x < n ? key_to_float(key) : -INFINITY;
    }
    if (kth != nullptr && t == 0) kth[row] = -INFINITY;
    return;
  }
  // digit 1 from the row histogram (exact from the k-th key's bin up)
#pragma unroll
  for (int x = 0; x < HPT; ++x) sh.hist[x * kSelThreads + t] = hv[x];
  __syncthreads();
  int kk = k, d, above;
  find_digit(sh, kBins1, kk, d, above);
  kk -= above;
  const int cand = above + (int)sh.hist[d];
  __syncthreads();
  if (cand <= kCandCap) {
    select_from_candidates(cs, k, (uint32_t)d, kk, sh, out, sco, kth ? kth + row : nullptr);
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
    for (int base = 0; base < cs.m; base += kSelPer * kSelThreads) {
      uint32_t key[kSelPer];
      int tok[kSelPer];
      bool valid[kSelPer];
      cs.strided(base + (t >> 6) * kSelPer * 64 + (t & 63), key, tok, valid);
#pragma unroll
      for (int e = 0; e < kSelPer; ++e)
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
  // output pass in index order: keep key > K*, and the first need_eq keys
  // == K*.  An element's output place is the greater keys before it plus
  // min(equal keys before it, need_eq); positions are laid out as in the
  // fast path's pass, ranks from ballots and one scan per pass.
  const int lane = t & 63, wave = t >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  int gt_before = 0, eq_before = 0;
  for (int base = 0; base < cs.m; base += kSelPer * kSelThreads) {
    uint32_t key[kSelPer];
    int tok[kSelPer];
    bool valid[kSelPer];
    cs.strided(base + wave * kSelPer * 64 + lane, key, tok, valid);
    int gr[kSelPer], er[kSelPer], wgt = 0, weq = 0;
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
      const uint64_t mg = __ballot(valid[e] && key[e] > kstar);
      const uint64_t me = __ballot(valid[e] && key[e] == kstar);
      gr[e] = wgt + __popcll(mg & below);
      er[e] = weq + __popcll(me & below);
      wgt += __popcll(mg);
      weq += __popcll(me);
    }
    // one scan carries both counts (at most 16384 each): equal keys high
    int tot;
    const int ex =
        __builtin_amdgcn_readlane(block_excl_scan(lane == 0 ? ((weq << 16) | wgt) : 0, sh.scan, &tot), 0);
    const int g0 = gt_before + (ex & 0xffff), e0 = eq_before + (ex >> 16);
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
      if (!valid[e]) continue;
      const int gb = g0 + gr[e], eb = e0 + er[e];
      const bool keep = key[e] > kstar || (key[e] == kstar && eb < need_eq);
      const int pos = gb + min(eb, need_eq);
      if (keep && pos < k) {
        out[pos] = tok[e];
        if (sco != nullptr) sco[pos] = key_to_float(key[e]);
      }
    }
    gt_before += tot & 0xffff;
    eq_before += tot >> 16;
  }
  if (kth != nullptr && t == 0) kth[row] = key_to_float(kstar);
}

// ---- union of a KV head's per-query-head index sets -----------------------
//
// Kascade post, "Head-aware is the key to accuracy": per-head sets keep each
// head's own choice; sharing one set among a KV head's G query heads lets
// them share every K/V read.  The union of the G sets is the shared set that
// keeps every head's own top-k (each head then attends over a superset of
// its own choice) and reads each chosen key once per KV head.
//
// One workgroup per (sequence, KV head): the G lists (any order; negative
// slots are empty) go to LDS, padded to a power of two with INT_MAX, a
// bitonic sort orders them, and a workgroup scan keeps the first of each run
// of equal entries.  Output: the distinct entries ascending, then -1 to the
// end of the row (G * k entries).
__global__ __launch_bounds__(kUnionThreads) void union_sets_kernel(
    const int32_t* __restrict__ idx, int Hq, int Hkv, int k, int n,
    int32_t* __restrict__ out, int32_t* __restrict__ cnt) {
  __shared__ int key[kUnionMax];
  __shared__ int scan_tmp[17];
  const int G = Hq / Hkv;
  const int row = blockIdx.x;  // b * Hkv + g: its G heads' lists are contiguous in idx
  const int t = threadIdx.x;
  const int m = G * k;  // entries of the G lists
  const int32_t* src = idx + (size_t)row * m;
  for (int e = t; e < n; e += kUnionThreads) {
    int v = INT_MAX;
    if (e < m) {
      const int w = src[e];
      v = w >= 0 ? w : INT_MAX;
    }
    key[e] = v;
  }
  __syncthreads();
  // bitonic sort, ascending: stage sizes 2..n, compare distances size/2..1
  for (int size = 2; size <= n; size <<= 1) {
    for (int d = size >> 1; d >= 1; d >>= 1) {
      for (int e = t; e < n / 2; e += kUnionThreads) {
        const int a = 2 * d * (e / d) + (e % d), b = a + d;
        const bool up = (a & size) == 0;  // direction of this bitonic run
        const int x = key[a], y = key[b];
        if ((x > y) == up) {
          key[a] = y;
          key[b] = x;
        }
      }
      __syncthreads();
    }
  }
  // keep the first of each run of equal valid entries; thread t owns a
  // contiguous range, so one scan places them in order
  const int per = (n + kUnionThreads - 1) / kUnionThreads;
  const int e0 = min(n, t * per), e1 = min(n, e0 + per);
  int c = 0;
  for (int e = e0; e < e1; ++e) {
    const int v = key[e];
    c += (v != INT_MAX && (e == 0 || key[e - 1] != v)) ? 1 : 0;
  }
  int tot;
  int pos = block_excl_scan(c, scan_tmp, &tot);
  int32_t* dst = out + (size_t)row * m;
  for (int e = e0; e < e1; ++e) {
    const int v = key[e];
    if (v != INT_MAX && (e == 0 || key[e - 1] != v)) dst[pos++] = v;
  }
  for (int e = tot + t; e < m; e += kUnionThreads) dst[e] = -1;
  if (cnt != nullptr && t == 0) cnt[row] = tot;
}

hipError_t launch_union_sets(const int32_t* idx, int B, int Hq, int Hkv, int k, int32_t* out,
                             int32_t* cnt, hipStream_t st) {
  const int m = (Hq / Hkv) * k;
  int n = 1;
  while (n < m) n <<= 1;
  if (n > kUnionMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(union_sets_kernel, dim3(B * Hkv), dim3(kUnionThreads), 0, st, idx, Hq, Hkv, k,
                     n, out, cnt);
  return hipGetLastError();
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
  L.bytes = L.hist_off + (size_t)L.rows * (kBins1 + kCoarse) * sizeof(uint32_t);
  return L;
}

size_t topk_ws_bytes(const DecodeDims& d, int k) {
  (void)k;
  const size_t a = topk_layout(d, false).bytes, b = topk_layout(d, true).bytes;
  return a > b ? a : b;
}

hipError_t launch_topk(const void* q, const void* kpool, const int32_t* pt, const int32_t* sl,
                       const DecodeDims& d, int k, bool pooled, int32_t* idx, float* scores,
                       float* kth, void* ws, hipStream_t st) {
  const int rows_per_b = pooled ? d.Hkv : d.Hq;  // score rows (and index sets) per sequence
  const TopkLayout L = topk_layout(d, pooled);
  char* w = static_cast<char*>(ws);
  uint32_t* ckey = reinterpret_cast<uint32_t*>(w);
  uint16_t* cidx = reinterpret_cast<uint16_t*>(w + L.idx_off);
  uint32_t* ccnt = reinterpret_cast<uint32_t*>(w + L.cnt_off);
  uint32_t* hist = reinterpret_cast<uint32_t*>(w + L.hist_off);
  const size_t nh = (size_t)L.rows * (kBins1 + kCoarse);  // bins, then coarse buckets
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
  hipLaunchKernelGGL(topk_select_kernel, dim3(d.B * rows_per_b), dim3(kSelThreads),
                     (L.tiles + 1) * sizeof(int), st, ckey,
                     cidx, ccnt, hist, sl, rows_per_b, d.max_seq_len, L.tt, L.tiles, L.cstride, k,
                     idx, scores, kth);
  return hipGetLastError();
}

hipError_t debug_flags_topk(uint32_t* flags, bool clear) {
  return debug_flags_of_tu(flags, clear);
}

}  // namespace fsa
