/*
 * fsa.h -- C ABI of the head-aware sparse attention library for AMD MI355X
 * (gfx950).  Five entry points run the hot path on the GPU; three helpers
 * size workspaces, build decode segment masks on the host and name status
 * codes.
 *
 * Conventions shared by every call
 *   - Pointers marked (device) are HIP device memory owned by the caller;
 *     the library never allocates, frees or keeps them.  Pointers marked
 *     (host) are ordinary host memory read before the call returns.
 *   - Tensors are dense, row-major (C order), with the shapes given below;
 *     bf16 is IEEE bfloat16 stored in 16 bits, fp32 is IEEE binary32.
 *   - bf16 / fp32 data tensors (queries, keys, values, KV pools, centroids,
 *     radii, scores of select_blocks, outputs) and workspaces start on a
 *     16-byte boundary, index / count / length arrays on a 4-byte boundary,
 *     else FSA_ERR_ARG (the kernels move them in 16- and 4-byte words).
 *   - Every entry point validates its host-side arguments before any launch
 *     and returns FSA_OK (0) or a negative FSA_ERR_* code; nothing aborts,
 *     exits or throws across the ABI.  Kernel work is enqueued
 *     asynchronously on the caller's stream `st` (0 = the null stream);
 *     launch failures are reported as FSA_ERR_LAUNCH, device faults surface
 *     at the caller's next synchronisation.
 *   - Calls are re-entrant; consecutive calls on one stream see each other's
 *     results (stream order).  The library keeps no mutable global state,
 *     apart from a per-device "is gfx950" cache and the per-GPU device array
 *     that sparse_decode_attn_noalloc alone uses (see there).
 *
 * Prefill shapes: batch B, prompt length S, query heads Hq, KV heads Hkv
 * (Hq % Hkv == 0, G = Hq / Hkv, query head h reads KV head h / G), head dim
 * D in {64, 128}, block size T in {64, 128} (query block = key block),
 * S % T == 0, nB = S / T <= 4096, Hq <= 1024, B * S < 2^31 and
 * B * Hq * nB < 2^31 (else FSA_ERR_SHAPE).
 * Decode shapes: page size 16 tokens, KV pool [num_pages, Hkv, 16, D] bf16
 * with num_pages * Hkv * 16 < 2^32 - 1 (else FSA_ERR_SHAPE),
 * token j of sequence b at pool[page_table[b * max_pages + j / 16], g,
 * j % 16, :].
 */
#ifndef FSA_H
#define FSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  FSA_OK = 0,
  FSA_ERR_NULL = -1,      /* a required pointer is NULL                          */
  FSA_ERR_SHAPE = -2,     /* a shape or size rule is violated                    */
  FSA_ERR_DTYPE = -3,     /* dtype not supported by this call                    */
  FSA_ERR_WORKSPACE = -4, /* ws_bytes smaller than fsa_workspace_size() asks for */
  FSA_ERR_NO_DEVICE = -5, /* no usable gfx950 device is current                  */
  FSA_ERR_LAUNCH = -6,    /* the HIP runtime rejected a kernel launch            */
  FSA_ERR_ARG = -7        /* another argument is out of range                    */
};

/* Element type of a call's tensors.  A plain 32-bit integer (not an enum
 * type), so that any value a caller passes is well defined to inspect:
 * values other than these two are rejected with FSA_ERR_DTYPE. */
typedef int32_t fsa_dtype;
enum { FSA_BF16 = 0, FSA_F32 = 1 };

typedef struct {
  int32_t B, S, Hq, Hkv, D, T;
} fsa_prefill_shape;

/* Two-branch selector parameters (host struct).
 * Branch keep counts per query block i with n_i = i + 1 visible key blocks:
 * k = max(1, ceil(p * n_i)) capped at n_i, the product formed in IEEE
 * double; p < 0 switches that branch off.  Forced blocks: key blocks
 * j < sink_blocks and i - band_blocks < j <= i. */
typedef struct {
  double p_centroid;
  double p_rescue;
  int32_t band_blocks;
  int32_t sink_blocks;
} fsa_select_params;

typedef struct {
  int32_t B, Hq, Hkv, D;
  int32_t page_size;   /* must be 16                                   */
  int32_t num_pages;   /* pages in each pool                           */
  int32_t max_pages;   /* row stride of page_table (pages per sequence) */
  int32_t max_seq_len; /* upper bound of seq_lens[b], <= 16*max_pages   */
} fsa_decode_shape;

enum {
  FSA_SEL_ALL = 0,
  FSA_SEL_INDEX = 1,
  FSA_SEL_SEGMENT = 2,
  FSA_SEL_INDEX_KV = 3,
  FSA_SEL_INDEX_SCORED = 4
};

/* Which cached tokens a decode query reads (host struct).
 *   FSA_SEL_ALL:     tokens [0, seq_lens[b]).
 *   FSA_SEL_INDEX:   idx (device) int32 [B, Hq, k], per query head; entries
 *                    outside [0, seq_lens[b]) are skipped.
 *   FSA_SEL_INDEX_KV: idx (device) int32 [B, Hkv, k], one list per KV head
 *                    shared by its G query heads (each K/V row is read once
 *                    for the group); entries outside [0, seq_lens[b]) are
 *                    skipped.
 *   FSA_SEL_INDEX_SCORED: idx as FSA_SEL_INDEX plus scores (device) fp32
 *                    [B, Hq, k], the raw q . k of each listed key (as
 *                    topk_indices_scored writes them); the keys are not read
 *                    (k_pool may be NULL), only V at the indices.  The
 *                    anchor layer of a Kascade group attends this way at its
 *                    own top-k without reading K twice.
 *   FSA_SEL_SEGMENT: segments (device) int32 [B, max_seg, 2] token ranges
 *                    [start, end), n_seg (device) int32 [B]; ranges of one
 *                    sequence must be sorted and disjoint, and are clipped
 *                    to [0, seq_lens[b]); shared by all heads.
 * n_split: split-KV factor per (sequence, head), 0 <= n_split <= 4096; 0
 * picks one.  A split takes at least 64 list positions, so splits beyond
 * what a short list needs stay empty (their partials carry no weight). */
typedef struct {
  int32_t mode;
  const int32_t* idx;
  int32_t k;
  const int32_t* segments;
  const int32_t* n_seg;
  int32_t max_seg;
  int32_t n_split;
  const float* scores; /* FSA_SEL_INDEX_SCORED only */
} fsa_kv_select;

/* ---- entry points -------------------------------------------------------- */

/* block_stats -- key-block centroid and radius.
 * RBS-Attention post, "Key technical points" 1: the centroid base branch
 * scores a block by its average key; the rescue branch uses the maximum
 * key-block radius.  centroid[b,g,j,:] = mean of the T keys K[b, jT..jT+T-1,
 * g, :]; radius[b,g,j] = max over those keys of ||k - centroid||_2 (whole
 * block, causality ignored).  Computed in fp32.
 *   k        (device) [B, S, Hkv, D] bf16 or fp32 (dt)
 *   centroid (device) fp32 [B, Hkv, nB, D]   written
 *   radius   (device) fp32 [B, Hkv, nB]      written */
int block_stats(fsa_dtype dt, const void* k, const fsa_prefill_shape* s, float* centroid,
                float* radius, hipStream_t st);

/* select_blocks -- two-branch block selection and mask merge.
 * RBS-Attention post, "Key technical points" 1-2: centroid and rescue
 * branches are thresholded independently and their masks merged.  With
 * qbar = mean of the T queries of query block i (head h) and j <= i:
 *   Sc[i,j] = qbar . centroid[g(h), j]
 *   Sr[i,j] = Sc[i,j] + ||qbar|| * radius[g(h), j]
 * C = top k(p_centroid) by Sc, R = top k(p_rescue) by Sr (ties to the lower
 * j), M = C u R u forced, j <= i.  Scores in fp32.
 *   q          (device) [B, S, Hq, D] bf16 or fp32
 *   centroid, radius (device) from block_stats
 *   p          (host) selector parameters
 *   mask_bits  (device) uint32 [B, Hq, nB, ceil(nB/32)]; bit j%32 of word j/32
 *              set iff M[i,j]; every word written
 *   block_idx  (device) int32 [B, Hq, nB, nB]; the j with M[i,j], ascending;
 *              entries past block_cnt are not written
 *   block_cnt  (device) int32 [B, Hq, nB]
 *   score_c, score_r (device, nullable) fp32 [B, Hq, nB, nB]; j <= i written
 *   ws         (device) at least fsa_workspace_size(FSA_OP_SELECT_BLOCKS) bytes */
int select_blocks(fsa_dtype dt, const void* q, const float* centroid, const float* radius,
                  const fsa_prefill_shape* s, const fsa_select_params* p, uint32_t* mask_bits,
                  int32_t* block_idx, int32_t* block_cnt, float* score_c, float* score_r,
                  void* ws, size_t ws_bytes, hipStream_t st);

/* sparse_prefill_attn -- block-sparse causal flash-attention.
 * RBS-Attention post, "Key technical points" 2: the merged mask runs on an
 * unchanged block-sparse FlashAttention path.  For token t of query block i
 * and head h: O[b,t,h,:] = sum over s in A softmax(scale * Q.K_s) V_s with
 * A = {s <= t : s / T listed in block_idx[b,h,i,0..block_cnt)}; list entries
 * outside [0, i] are skipped.  block_idx == NULL (and block_cnt == NULL)
 * means every causal block (dense causal attention).  bf16 inputs use bf16
 * MFMA with fp32 accumulation and an fp32 online softmax; fp32 inputs use
 * fp32 MFMA throughout.  An empty list gives O = 0, lse = -inf.  scale must
 * be finite and > 0 (else FSA_ERR_ARG).
 *   q (device) [B,S,Hq,D]; k, v (device) [B,S,Hkv,D]; all of dtype dt
 *   out (device) [B,S,Hq,D] dtype dt; lse (device, nullable) fp32 [B,Hq,S]
 *   (natural log).  ws may be NULL when the workspace size is 0. */
int sparse_prefill_attn(fsa_dtype dt, const void* q, const void* k, const void* v,
                        const fsa_prefill_shape* s, const int32_t* block_idx,
                        const int32_t* block_cnt, float scale, void* out, float* lse, void* ws,
                        size_t ws_bytes, hipStream_t st);

/* topk_indices -- exact per-head top-k over the whole paged context.
 * Kascade post, "What Kascade got right": an anchor layer computes exact
 * Top-k key indices that later layers reuse; "Head-aware is the key to
 * accuracy": one index set per attention (query) head.  Scores are raw
 * q . k in fp32 over tokens [0, seq_lens[b]); the k largest are kept, ties
 * to the lower token index, written ascending.  If seq_lens[b] < k the
 * missing entries are -1 and kth is -inf.  max_seq_len <= 2^23 (else
 * FSA_ERR_SHAPE).
 *   q (device) bf16 [B, Hq, D]; k_pool (device) bf16 [num_pages, Hkv, 16, D]
 *   page_table (device) int32 [B, max_pages]; seq_lens (device) int32 [B]
 *   idx (device) int32 [B, Hq, k]; kth (device, nullable) fp32 [B, Hq]
 *   ws (device) at least fsa_workspace_size(FSA_OP_TOPK) bytes */
int topk_indices(fsa_dtype dt, const void* q, const void* k_pool, const int32_t* page_table,
                 const int32_t* seq_lens, const fsa_decode_shape* s, int k, int32_t* idx,
                 float* kth, void* ws, size_t ws_bytes, hipStream_t st);

/* topk_indices_scored -- topk_indices that also returns each kept key's
 * score: scores (device) fp32 [B, Hq, k], scores[b,h,x] = the raw fp32
 * q . k of token idx[b,h,x] as the scan computed it (-inf for the -1 slots
 * of a sequence shorter than k).  Kascade post, "What Kascade got right": the
 * anchor layer scores every key to pick its top-k, so its own attention at
 * those keys needs only their values (FSA_SEL_INDEX_SCORED).  Other
 * arguments and errors as topk_indices; scores must not be NULL. */
int topk_indices_scored(fsa_dtype dt, const void* q, const void* k_pool,
                        const int32_t* page_table, const int32_t* seq_lens,
                        const fsa_decode_shape* s, int k, int32_t* idx, float* scores,
                        float* kth, void* ws, size_t ws_bytes, hipStream_t st);

/* topk_indices_kv -- exact top-k per KV head over a pooled score, the
 * GQA-shared counterpart of topk_indices.  Kascade post, "Head-aware is the
 * key to accuracy", favours one set per query head; one set per KV head lets
 * the G query heads share every index and K/V read (FSA_SEL_INDEX_KV), at the
 * accuracy cost that post describes.  The pooled score of a token is the
 * maximum over the KV head's G query heads of the raw q . k (fp32); the k
 * largest are kept, ties to the lower token index, written ascending; if
 * seq_lens[b] < k the missing entries are -1 and kth is -inf.
 *   q, k_pool, page_table, seq_lens, ws: as topk_indices
 *   idx (device) int32 [B, Hkv, k]; kth (device, nullable) fp32 [B, Hkv] */
int topk_indices_kv(fsa_dtype dt, const void* q, const void* k_pool, const int32_t* page_table,
                    const int32_t* seq_lens, const fsa_decode_shape* s, int k, int32_t* idx,
                    float* kth, void* ws, size_t ws_bytes, hipStream_t st);

/* topk_union_kv -- one shared index set per KV head: the union of its G
 * query heads' sets.  Kascade post, "Head-aware is the key to accuracy":
 * per-head sets keep each head's own choice, and sharing one set lets a KV
 * head's query heads share every K/V read.  The union keeps every head's own
 * top-k (each head attends over a superset of it, FSA_SEL_INDEX_KV with
 * k' = G * k) and reads each chosen key once per KV head.
 *   idx (device) int32 [B, Hq, k]: per-query-head sets as topk_indices
 *       writes them (any order is accepted; negative entries are empty)
 *   out (device) int32 [B, Hkv, G * k]: the distinct entries ascending, then
 *       -1 to the end of each row
 *   cnt (device, nullable) int32 [B, Hkv]: distinct entries per row
 * G = Hq / Hkv; G * k rounded up to a power of two must not exceed 16384
 * (else FSA_ERR_ARG). */
int topk_union_kv(const int32_t* idx, int B, int Hq, int Hkv, int k, int32_t* out,
                  int32_t* cnt, hipStream_t st);

/* sparse_decode_attn -- split-KV decode attention over a paged cache.
 * Kascade post, "What Kascade got right" (reuse layers attend only at the
 * anchor's indices); Declarative Attention post, "Declarative attention
 * protocol" (block-aligned global/focus/local token ranges over a paged
 * cache); LoZA post, "4. From food delivery to AI" (SplitKV-and-Combine).
 * o[b,h,:] = sum over admitted tokens j softmax(scale * q.K_j) V_j; the key
 * set is split, each split writes (max, sum, output) partials in fp32, and
 * a log-sum-exp combine merges them.  An empty key set gives o = 0 and
 * lse = -inf.
 *   q (device) bf16 [B, Hq, D]; k_pool, v_pool (device) bf16 pools
 *   sel (host) key selection, see fsa_kv_select
 *   out (device) bf16 [B, Hq, D]; lse (device, nullable) fp32 [B, Hq]
 *   ws (device) at least fsa_workspace_size(FSA_OP_DECODE_ATTN) bytes */
int sparse_decode_attn(fsa_dtype dt, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* page_table, const int32_t* seq_lens,
                       const fsa_decode_shape* s, const fsa_kv_select* sel, float scale,
                       void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t st);

/* sparse_decode_attn_noalloc -- sparse_decode_attn without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * serving loops and harnesses that forbid allocation.  Arguments, results and
 * errors are those of sparse_decode_attn; the split partials live instead in
 * a library-owned device array of FSA_NOALLOC_SCRATCH_BYTES (16 MiB) per
 * GPU, held from the first call on that GPU until the process ends.  The
 * call allocates nothing.  It returns FSA_ERR_WORKSPACE when the partials
 * (fsa_workspace_size(FSA_OP_DECODE_ATTN, ...) bytes) would exceed the array.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (several streams, or several host threads) race and must be ordered
 * by the caller. */
#define FSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int sparse_decode_attn_noalloc(fsa_dtype dt, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* page_table,
                               const int32_t* seq_lens, const fsa_decode_shape* s,
                               const fsa_kv_select* sel, float scale, void* out, float* lse,
                               hipStream_t st);

/* ---- helpers --------------------------------------------------------------- */

enum { FSA_OP_SELECT_BLOCKS = 1, FSA_OP_PREFILL_ATTN = 2, FSA_OP_TOPK = 3, FSA_OP_DECODE_ATTN = 4 };

/* Workspace bytes a call needs.  shape: fsa_prefill_shape* for ops 1-2,
 * fsa_decode_shape* for ops 3-4; params: NULL for ops 1-2, int* k for op 3,
 * fsa_kv_select* for op 4.  Returns 0 for an unknown op or bad arguments. */
size_t fsa_workspace_size(int op, const void* shape, const void* params);

enum { FSA_SEG_GLOBAL = 0, FSA_SEG_FOCUS = 1, FSA_SEG_LOCAL = 2, FSA_SEG_STREAMING = 3 };

/* fsa_build_segments -- host-only segment builder for one sequence of n
 * cached tokens.  Declarative Attention post, "Declarative attention
 * protocol" (global / focus / local; kept ranges rounded outward to
 * KV-block boundaries) and LoZA post, "2. ZigZag architecture" (streaming
 * window).  Ranges written to out (host) int32 [*n_seg, 2], sorted, merged:
 *   GLOBAL    [0, n)
 *   FOCUS     [chunk_start, chunk_start + chunk_len) u [n - local_len, n),
 *             each rounded outward to `page`, clipped to [0, n)
 *   LOCAL     [n - local_len, n) rounded outward to `page`
 *   STREAMING [0, n_sink) u [n - local_len, n), token-exact
 * out must hold 2 ranges.  Returns FSA_ERR_ARG for a bad mode or sizes. */
int fsa_build_segments(int mode, int n, int chunk_start, int chunk_len, int local_len,
                       int n_sink, int page, int32_t* out, int* n_seg);

/* fsa_build_segments_nb -- fsa_build_segments with a minimum neighbourhood
 * around the focused region, one of the safeguards the million-token-context
 * post lists ("Not a free lunch").  In FOCUS mode the chunk is first widened
 * to [chunk_start - min_nb, chunk_start + chunk_len + min_nb), then rounded
 * outward and clipped as above; the other modes ignore min_nb.
 * fsa_build_segments(...) is fsa_build_segments_nb(..., min_nb = 0, ...).
 * Returns FSA_ERR_ARG for min_nb < 0 and as fsa_build_segments otherwise. */
int fsa_build_segments_nb(int mode, int n, int chunk_start, int chunk_len, int local_len,
                          int n_sink, int page, int min_nb, int32_t* out, int* n_seg);

/* fsa_debug_flags -- inputs that the kernels skip, recorded by a debug build.
 * Release builds skip bad inputs silently (see each call); a library built
 * with FSA_DEBUG_BOUNDS (python -m free_sparse_attention_head_amd.build
 * --debug-bounds, libfsa_debug.so) also raises, on the device, one flag bit
 * per kind of bad input it met:
 *   FSA_DBG_BLOCK_INDEX  a prefill block-list entry outside [0, i]
 *   FSA_DBG_TOKEN_INDEX  a decode index entry below -1 or at or past seq_len
 *                        (-1 marks an empty slot and is not flagged)
 *   FSA_DBG_PAGE_ID      a page-table entry outside [0, num_pages) for a
 *                        token inside the sequence (decode and top-k)
 *   FSA_DBG_SEGMENT      an n_seg outside [0, max_seg], or segment ranges
 *                        that are not sorted and disjoint
 * flags (host) receives the bits raised since the last clear, on every GPU
 * call of this process; clear != 0 resets them.  The read synchronises with
 * the null stream: synchronise other streams first.  A release build sets
 * only FSA_DBG_UNAVAILABLE. */
enum {
  FSA_DBG_BLOCK_INDEX = 1,
  FSA_DBG_TOKEN_INDEX = 2,
  FSA_DBG_PAGE_ID = 4,
  FSA_DBG_SEGMENT = 8,
  FSA_DBG_UNAVAILABLE = (int)0x80000000u
};
int fsa_debug_flags(uint32_t* flags, int clear);

/* Static text for a status code. */
const char* fsa_status_string(int status);

/* FSA_OK when the current HIP device is a gfx950 GPU, else FSA_ERR_NO_DEVICE. */
int fsa_device_check(void);

#ifdef __cplusplus
}
#endif

#endif /* FSA_H */
