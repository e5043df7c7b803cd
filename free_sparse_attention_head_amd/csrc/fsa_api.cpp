// C-ABI layer of the library: host-side validation, workspace sizing, device
// check and dispatch to the kernel launchers.  No allocation, no global
// mutable state besides the per-device "is gfx950" cache (and, in
// decode_attn.hip, the per-device address of the allocation-free entry
// point's array).
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <initializer_list>

#include "fsa.h"
#include "launch.h"

namespace {

using fsa::DecodeDims;
using fsa::PrefillDims;

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int device_check() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FSA_ERR_NO_DEVICE;
  if (dev < kMaxDevices) {
    const int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return FSA_OK;
    if (st == 2) return FSA_ERR_NO_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FSA_ERR_NO_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FSA_OK : FSA_ERR_NO_DEVICE;
}

int launch_status(hipError_t e) { return e == hipSuccess ? FSA_OK : FSA_ERR_LAUNCH; }

// The kernels move data tensors and workspaces in 16-byte vectors and index
// arrays in 4-byte words; a pointer off that grain is rejected, never read.
// Null pointers pass here (the null checks come first).
bool off_grain(std::initializer_list<const void*> ptrs, uintptr_t grain) {
  for (const void* ptr : ptrs)
    if (reinterpret_cast<uintptr_t>(ptr) & (grain - 1)) return true;
  return false;
}
bool misaligned16(std::initializer_list<const void*> ptrs) { return off_grain(ptrs, 16); }
bool misaligned4(std::initializer_list<const void*> ptrs) { return off_grain(ptrs, 4); }

int check_prefill_shape(const fsa_prefill_shape* s, PrefillDims* d) {
  if (s == nullptr) return FSA_ERR_NULL;
  if (s->B < 1 || s->S < 1 || s->Hq < 1 || s->Hkv < 1) return FSA_ERR_SHAPE;
  if (s->Hq % s->Hkv != 0) return FSA_ERR_SHAPE;
  if (s->D != 64 && s->D != 128) return FSA_ERR_SHAPE;
  if (s->T != 64 && s->T != 128) return FSA_ERR_SHAPE;
  if (s->S % s->T != 0 || s->S / s->T > 4096) return FSA_ERR_SHAPE;
  // element counts used as 64-bit offsets; token rows, (b, h, i) rows and
  // byte strides of one token row (Hq * D * 4 bytes) as 32-bit ints
  if ((long long)s->B * s->S > (1LL << 31) - 1) return FSA_ERR_SHAPE;
  if (s->Hq > 1024) return FSA_ERR_SHAPE;
  if ((long long)s->B * s->Hq * (s->S / s->T) > (1LL << 31) - 1) return FSA_ERR_SHAPE;
  *d = PrefillDims{s->B, s->S, s->Hq, s->Hkv, s->D, s->T};
  return FSA_OK;
}

int check_dtype_prefill(fsa_dtype dt) {
  return (dt == FSA_BF16 || dt == FSA_F32) ? FSA_OK : FSA_ERR_DTYPE;
}

int check_decode_shape(const fsa_decode_shape* s, DecodeDims* d) {
  if (s == nullptr) return FSA_ERR_NULL;
  if (s->B < 1 || s->Hq < 1 || s->Hkv < 1 || s->Hq % s->Hkv != 0) return FSA_ERR_SHAPE;
  const int G = s->Hq / s->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return FSA_ERR_SHAPE;
  if (s->D != 64 && s->D != 128) return FSA_ERR_SHAPE;
  if (s->page_size != 16) return FSA_ERR_SHAPE;
  if (s->num_pages < 1 || s->max_pages < 1 || s->max_seq_len < 1) return FSA_ERR_SHAPE;
  if ((long long)s->max_seq_len > 16LL * s->max_pages) return FSA_ERR_SHAPE;
  if (s->max_seq_len > (1 << 30)) return FSA_ERR_SHAPE;
  // pool rows (page, head, slot) are 32-bit indices, the top one reserved
  if ((long long)s->num_pages * s->Hkv * 16 >= 0xffffffffLL) return FSA_ERR_SHAPE;
  *d = DecodeDims{s->B, s->Hq, s->Hkv, s->D, s->num_pages, s->max_pages, s->max_seq_len};
  return FSA_OK;
}

using fsa::kMaxSplit;
constexpr int kMaxSegments = 64;

int check_kv_select(const fsa_kv_select* sel, const DecodeDims& d) {
  if (sel == nullptr) return FSA_ERR_NULL;
  if (sel->n_split < 0 || sel->n_split > kMaxSplit) return FSA_ERR_ARG;
  switch (sel->mode) {
    case FSA_SEL_ALL:
      return FSA_OK;
    case FSA_SEL_INDEX:
    case FSA_SEL_INDEX_KV:
      if (sel->idx == nullptr) return FSA_ERR_NULL;
      if (sel->k < 1) return FSA_ERR_ARG;
      return FSA_OK;
    case FSA_SEL_INDEX_SCORED:
      if (sel->idx == nullptr || sel->scores == nullptr) return FSA_ERR_NULL;
      if (sel->k < 1) return FSA_ERR_ARG;
      return FSA_OK;
    case FSA_SEL_SEGMENT:
      if (sel->segments == nullptr || sel->n_seg == nullptr) return FSA_ERR_NULL;
      if (sel->max_seg < 1 || sel->max_seg > kMaxSegments) return FSA_ERR_ARG;
      return FSA_OK;
    default:
      return FSA_ERR_ARG;
  }
  (void)d;
}

}  // namespace

extern "C" {

int fsa_debug_flags(uint32_t* flags, int clear) {
  if (!flags) return FSA_ERR_NULL;
  int rc = device_check();
  if (rc) return rc;
  uint32_t all = 0u;
  hipError_t (*const readers[])(uint32_t*, bool) = {
      fsa::debug_flags_prefill_f32, fsa::debug_flags_prefill_bf16, fsa::debug_flags_topk,
      fsa::debug_flags_decode};
  for (auto rd : readers) {
    uint32_t f = 0u;
    if (rd(&f, clear != 0) != hipSuccess) return FSA_ERR_LAUNCH;
    all |= f;
  }
#ifndef FSA_DEBUG_BOUNDS
  all |= FSA_DBG_UNAVAILABLE;
#endif
  *flags = all;
  return FSA_OK;
}

const char* fsa_status_string(int status) {
  switch (status) {
    case FSA_OK: return "ok";
    case FSA_ERR_NULL: return "required pointer is NULL";
    case FSA_ERR_SHAPE: return "shape or size rule violated";
    case FSA_ERR_DTYPE: return "dtype not supported by this call";
    case FSA_ERR_WORKSPACE: return "workspace too small";
    case FSA_ERR_NO_DEVICE: return "no usable gfx950 device";
    case FSA_ERR_LAUNCH: return "kernel launch failed";
    case FSA_ERR_ARG: return "argument out of range";
    default: return "unknown status";
  }
}

int fsa_device_check(void) { return device_check(); }

size_t fsa_workspace_size(int op, const void* shape, const void* params) {
  if (shape == nullptr) return 0;
  if (op != FSA_OP_SELECT_BLOCKS && op != FSA_OP_PREFILL_ATTN && op != FSA_OP_TOPK &&
      op != FSA_OP_DECODE_ATTN)
    return 0;  // the shape is not read: its type depends on the op
  if (op == FSA_OP_SELECT_BLOCKS || op == FSA_OP_PREFILL_ATTN) {
    PrefillDims d;
    if (check_prefill_shape(static_cast<const fsa_prefill_shape*>(shape), &d) != FSA_OK) return 0;
    return op == FSA_OP_SELECT_BLOCKS ? fsa::select_ws_bytes(d) : 0;
  }
  DecodeDims d;
  if (check_decode_shape(static_cast<const fsa_decode_shape*>(shape), &d) != FSA_OK) return 0;
  if (op == FSA_OP_TOPK) {
    const int k = params ? *static_cast<const int*>(params) : 1;
    return fsa::topk_ws_bytes(d, k);
  }
  if (op == FSA_OP_DECODE_ATTN) {
    // sizing depends on mode, k and n_split only; pointers are not needed yet
    const fsa_kv_select* sel = static_cast<const fsa_kv_select*>(params);
    if (sel == nullptr || sel->n_split < 0 || sel->n_split > kMaxSplit) return 0;
    if (sel->mode != FSA_SEL_ALL && sel->mode != FSA_SEL_INDEX && sel->mode != FSA_SEL_SEGMENT &&
        sel->mode != FSA_SEL_INDEX_KV && sel->mode != FSA_SEL_INDEX_SCORED)
      return 0;
    if ((sel->mode == FSA_SEL_INDEX || sel->mode == FSA_SEL_INDEX_KV ||
         sel->mode == FSA_SEL_INDEX_SCORED) && sel->k < 1)
      return 0;
    return fsa::decode_ws_bytes(d, sel->mode, sel->k, sel->n_split);
  }
  return 0;
}

int block_stats(fsa_dtype dt, const void* k, const fsa_prefill_shape* s, float* centroid,
                float* radius, hipStream_t st) {
  PrefillDims d;
  int rc = check_prefill_shape(s, &d);
  if (rc) return rc;
  if ((rc = check_dtype_prefill(dt))) return rc;
  if (!k || !centroid || !radius) return FSA_ERR_NULL;
  if (misaligned16({k, centroid, radius})) return FSA_ERR_ARG;
  if ((rc = device_check())) return rc;
  return launch_status(fsa::launch_block_stats(dt == FSA_F32, k, centroid, radius, d, st));
}

int select_blocks(fsa_dtype dt, const void* q, const float* centroid, const float* radius,
                  const fsa_prefill_shape* s, const fsa_select_params* p, uint32_t* mask_bits,
                  int32_t* block_idx, int32_t* block_cnt, float* score_c, float* score_r,
                  void* ws, size_t ws_bytes, hipStream_t st) {
  PrefillDims d;
  int rc = check_prefill_shape(s, &d);
  if (rc) return rc;
  if ((rc = check_dtype_prefill(dt))) return rc;
  if (!q || !centroid || !radius || !p || !mask_bits || !block_idx || !block_cnt) return FSA_ERR_NULL;
  if (isnan(p->p_centroid) || isnan(p->p_rescue)) return FSA_ERR_ARG;
  if (p->band_blocks < 0 || p->sink_blocks < 0) return FSA_ERR_ARG;
  if (!ws) return FSA_ERR_NULL;
  if (misaligned16({q, centroid, radius, score_c, score_r, ws}) ||
      misaligned4({mask_bits, block_idx, block_cnt}))
    return FSA_ERR_ARG;
  if (ws_bytes < fsa::select_ws_bytes(d)) return FSA_ERR_WORKSPACE;
  if ((rc = device_check())) return rc;
  return launch_status(fsa::launch_select_blocks(dt == FSA_F32, q, centroid, radius, d,
                                                 p->p_centroid, p->p_rescue, p->band_blocks,
                                                 p->sink_blocks, mask_bits, block_idx, block_cnt,
                                                 score_c, score_r, ws, st));
}

int sparse_prefill_attn(fsa_dtype dt, const void* q, const void* k, const void* v,
                        const fsa_prefill_shape* s, const int32_t* block_idx,
                        const int32_t* block_cnt, float scale, void* out, float* lse, void* ws,
                        size_t ws_bytes, hipStream_t st) {
  (void)ws;
  (void)ws_bytes;
  PrefillDims d;
  int rc = check_prefill_shape(s, &d);
  if (rc) return rc;
  if ((rc = check_dtype_prefill(dt))) return rc;
  if (!q || !k || !v || !out) return FSA_ERR_NULL;
  if ((block_idx == nullptr) != (block_cnt == nullptr)) return FSA_ERR_NULL;
  // the kernels track the running row maximum in unscaled score units, which
  // orders scaled scores the same way only for a positive scale
  if (!isfinite(scale) || !(scale > 0.f)) return FSA_ERR_ARG;
  if (misaligned16({q, k, v, out}) || misaligned4({block_idx, block_cnt, lse})) return FSA_ERR_ARG;
  if ((rc = device_check())) return rc;
  return launch_status(fsa::launch_prefill_attn(dt == FSA_F32, q, k, v, d, block_idx, block_cnt,
                                                scale, out, lse, st));
}

static int topk_common(fsa_dtype dt, const void* q, const void* k_pool,
                       const int32_t* page_table, const int32_t* seq_lens,
                       const fsa_decode_shape* s, int k, bool pooled, int32_t* idx,
                       float* scores, float* kth, void* ws, size_t ws_bytes, hipStream_t st) {
  DecodeDims d;
  int rc = check_decode_shape(s, &d);
  if (rc) return rc;
  if (dt != FSA_BF16) return FSA_ERR_DTYPE;
  if (!q || !k_pool || !page_table || !seq_lens || !idx) return FSA_ERR_NULL;
  if (k < 1 || k > d.max_seq_len) return FSA_ERR_ARG;
  if (d.max_seq_len > fsa::kTopkMaxSeqLen) return FSA_ERR_SHAPE;
  if (!ws) return FSA_ERR_NULL;
  if (misaligned16({q, k_pool, ws}) || misaligned4({page_table, seq_lens, idx, scores, kth}))
    return FSA_ERR_ARG;
  if (ws_bytes < fsa::topk_ws_bytes(d, k)) return FSA_ERR_WORKSPACE;
  if ((rc = device_check())) return rc;
  return launch_status(
      fsa::launch_topk(q, k_pool, page_table, seq_lens, d, k, pooled, idx, scores, kth, ws, st));
}

int topk_indices(fsa_dtype dt, const void* q, const void* k_pool, const int32_t* page_table,
                 const int32_t* seq_lens, const fsa_decode_shape* s, int k, int32_t* idx,
                 float* kth, void* ws, size_t ws_bytes, hipStream_t st) {
  return topk_common(dt, q, k_pool, page_table, seq_lens, s, k, false, idx, nullptr, kth, ws,
                     ws_bytes, st);
}

int topk_indices_scored(fsa_dtype dt, const void* q, const void* k_pool,
                        const int32_t* page_table, const int32_t* seq_lens,
                        const fsa_decode_shape* s, int k, int32_t* idx, float* scores,
                        float* kth, void* ws, size_t ws_bytes, hipStream_t st) {
  if (!scores) return FSA_ERR_NULL;
  return topk_common(dt, q, k_pool, page_table, seq_lens, s, k, false, idx, scores, kth, ws,
                     ws_bytes, st);
}

int topk_indices_kv(fsa_dtype dt, const void* q, const void* k_pool, const int32_t* page_table,
                    const int32_t* seq_lens, const fsa_decode_shape* s, int k, int32_t* idx,
                    float* kth, void* ws, size_t ws_bytes, hipStream_t st) {
  return topk_common(dt, q, k_pool, page_table, seq_lens, s, k, true, idx, nullptr, kth, ws,
                     ws_bytes, st);
}

int topk_union_kv(const int32_t* idx, int B, int Hq, int Hkv, int k, int32_t* out,
                  int32_t* cnt, hipStream_t st) {
  if (!idx || !out) return FSA_ERR_NULL;
  if (misaligned4({idx, out, cnt})) return FSA_ERR_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return FSA_ERR_SHAPE;
  if (k < 1) return FSA_ERR_ARG;
  if ((long long)(Hq / Hkv) * k > fsa::kUnionMax) return FSA_ERR_ARG;
  if ((long long)B * Hq * k > (1LL << 31) - 1) return FSA_ERR_SHAPE;
  int rc = device_check();
  if (rc) return rc;
  return launch_status(fsa::launch_union_sets(idx, B, Hq, Hkv, k, out, cnt, st));
}

int sparse_decode_attn(fsa_dtype dt, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* page_table, const int32_t* seq_lens,
                       const fsa_decode_shape* s, const fsa_kv_select* sel, float scale,
                       void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t st) {
  DecodeDims d;
  int rc = check_decode_shape(s, &d);
  if (rc) return rc;
  if (dt != FSA_BF16) return FSA_ERR_DTYPE;
  if ((rc = check_kv_select(sel, d))) return rc;
  // keys are not read when their scores come with the indices
  if (!q || (!k_pool && sel->mode != FSA_SEL_INDEX_SCORED) || !v_pool || !page_table ||
      !seq_lens || !out)
    return FSA_ERR_NULL;
  if (!isfinite(scale)) return FSA_ERR_ARG;
  if (!ws) return FSA_ERR_NULL;
  if (misaligned16({q, k_pool, v_pool, out, ws}) ||
      misaligned4({page_table, seq_lens, lse, sel->idx, sel->scores, sel->segments, sel->n_seg}))
    return FSA_ERR_ARG;
  if (ws_bytes < fsa::decode_ws_bytes(d, sel->mode, sel->k, sel->n_split)) return FSA_ERR_WORKSPACE;
  if ((rc = device_check())) return rc;
  return launch_status(fsa::launch_decode_attn(q, k_pool, v_pool, page_table, seq_lens, d,
                                               sel->mode, sel->idx, sel->scores, sel->k,
                                               sel->segments, sel->n_seg, sel->max_seg,
                                               sel->n_split, scale, out, lse, ws, st));
}

int sparse_decode_attn_noalloc(fsa_dtype dt, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* page_table,
                               const int32_t* seq_lens, const fsa_decode_shape* s,
                               const fsa_kv_select* sel, float scale, void* out, float* lse,
                               hipStream_t st) {
  DecodeDims d;
  int rc = check_decode_shape(s, &d);
  if (rc) return rc;
  if (dt != FSA_BF16) return FSA_ERR_DTYPE;
  if ((rc = check_kv_select(sel, d))) return rc;
  if (!q || (!k_pool && sel->mode != FSA_SEL_INDEX_SCORED) || !v_pool || !page_table ||
      !seq_lens || !out)
    return FSA_ERR_NULL;
  if (!isfinite(scale)) return FSA_ERR_ARG;
  if (misaligned16({q, k_pool, v_pool, out}) ||
      misaligned4({page_table, seq_lens, lse, sel->idx, sel->scores, sel->segments, sel->n_seg}))
    return FSA_ERR_ARG;
  if (fsa::decode_ws_bytes(d, sel->mode, sel->k, sel->n_split) > fsa::kNoAllocScratchBytes)
    return FSA_ERR_WORKSPACE;
  if ((rc = device_check())) return rc;
  void* scratch = nullptr;
  if (fsa::noalloc_scratch(&scratch) != hipSuccess) return FSA_ERR_NO_DEVICE;
  return launch_status(fsa::launch_decode_attn(q, k_pool, v_pool, page_table, seq_lens, d,
                                               sel->mode, sel->idx, sel->scores, sel->k,
                                               sel->segments, sel->n_seg, sel->max_seg,
                                               sel->n_split, scale, out, lse, scratch, st));
}

int fsa_build_segments(int mode, int n, int chunk_start, int chunk_len, int local_len,
                       int n_sink, int page, int32_t* out, int* n_seg) {
  return fsa_build_segments_nb(mode, n, chunk_start, chunk_len, local_len, n_sink, page, 0, out,
                               n_seg);
}

int fsa_build_segments_nb(int mode, int n, int chunk_start, int chunk_len, int local_len,
                          int n_sink, int page, int min_nb, int32_t* out, int* n_seg) {
  if (!out || !n_seg) return FSA_ERR_NULL;
  if (n < 0 || page < 1 || local_len < 0 || chunk_len < 0 || n_sink < 0 || chunk_start < 0 ||
      min_nb < 0)
    return FSA_ERR_ARG;
  long long r[2][2];
  int c = 0;
  auto add = [&](long long a, long long b) {
    a = std::max(0LL, a);
    b = std::min((long long)n, b);
    if (b > a) {
      r[c][0] = a;
      r[c][1] = b;
      ++c;
    }
  };
  auto down = [&](long long x) { return x < 0 ? 0 : (x / page) * page; };
  auto up = [&](long long x) { return ((x + page - 1) / page) * page; };
  switch (mode) {
    case FSA_SEG_GLOBAL:
      add(0, n);
      break;
    case FSA_SEG_LOCAL:
      add(down((long long)n - local_len), n);
      break;
    case FSA_SEG_FOCUS:
      add(down((long long)chunk_start - min_nb), up((long long)chunk_start + chunk_len + min_nb));
      add(down((long long)n - local_len), n);
      break;
    case FSA_SEG_STREAMING:
      add(0, n_sink);
      add((long long)n - local_len, n);
      break;
    default:
      return FSA_ERR_ARG;
  }
  // sort the (at most two) ranges and merge overlapping or touching ones
  if (c == 2 && r[1][0] < r[0][0]) {
    std::swap(r[0][0], r[1][0]);
    std::swap(r[0][1], r[1][1]);
  }
  if (c == 2 && r[1][0] <= r[0][1]) {
    r[0][1] = std::max(r[0][1], r[1][1]);
    c = 1;
  }
  for (int x = 0; x < c; ++x) {
    out[2 * x] = (int32_t)r[x][0];
    out[2 * x + 1] = (int32_t)r[x][1];
  }
  *n_seg = c;
  return FSA_OK;
}

}  // extern "C"
