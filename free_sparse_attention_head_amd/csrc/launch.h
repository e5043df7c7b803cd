// Internal launcher declarations shared by the C-ABI layer (fsa_api.cpp) and
// the kernel translation units.  Host arguments arrive validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fsa.h"

namespace fsa {

struct PrefillDims {
  int B, S, Hq, Hkv, D, T;
};

struct DecodeDims {
  int B, Hq, Hkv, D, num_pages, max_pages, max_seq_len;
};

// block_stats.hip
hipError_t launch_block_stats(bool f32, const void* k, float* cen, float* rad,
                              const PrefillDims& d, hipStream_t st);

// select_blocks.hip
size_t select_ws_bytes(const PrefillDims& d);
hipError_t launch_select_blocks(bool f32, const void* q, const float* cen, const float* rad,
                                const PrefillDims& d, double p_c, double p_r, int band,
                                int sink, uint32_t* mask, int32_t* bidx, int32_t* bcnt,
                                float* score_c, float* score_r, void* ws, hipStream_t st);

// prefill_attn.hip
hipError_t launch_prefill_attn(bool f32, const void* q, const void* k, const void* v,
                               const PrefillDims& d, const int32_t* bidx, const int32_t* bcnt,
                               float scale, void* out, float* lse, hipStream_t st);

// prefill_attn_bf16.hip
hipError_t launch_prefill_attn_bf16(const void* q, const void* k, const void* v,
                                    const PrefillDims& d, const int32_t* bidx,
                                    const int32_t* bcnt, float scale, void* out, float* lse,
                                    hipStream_t st);

// flag bits (FSA_DBG_*) each translation unit with input checks has raised
// since its last clear; all 0 unless built with FSA_DEBUG_BOUNDS
hipError_t debug_flags_prefill_f32(uint32_t* flags, bool clear);
hipError_t debug_flags_prefill_bf16(uint32_t* flags, bool clear);
hipError_t debug_flags_topk(uint32_t* flags, bool clear);
hipError_t debug_flags_decode(uint32_t* flags, bool clear);

// topk.hip
constexpr int kTopkMaxSeqLen = 1 << 23;  // tokens per sequence that top-k supports
// decode splits per (sequence, head item), at most (n_split argument and combine)
constexpr int kMaxSplit = 4096;
size_t topk_ws_bytes(const DecodeDims& d, int k);
// pooled: one index set per KV head from the max over its query heads' scores
// scores (nullable): the raw score of each kept key, beside idx
hipError_t launch_topk(const void* q, const void* kpool, const int32_t* pt, const int32_t* sl,
                       const DecodeDims& d, int k, bool pooled, int32_t* idx, float* scores,
                       float* kth, void* ws, hipStream_t st);

// union of a KV head's G per-query-head index sets: G * k entries, padded
// to a power of two, at most kUnionMax
constexpr int kUnionMax = 16384;
constexpr int kUnionThreads = 1024;
hipError_t launch_union_sets(const int32_t* idx, int B, int Hq, int Hkv, int k, int32_t* out,
                             int32_t* cnt, hipStream_t st);

// decode_attn.hip
// bytes of the device array that the allocation-free decode entry point uses
// for split partials (one per GPU)
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
// device address of this GPU's array (looked up once per device)
hipError_t noalloc_scratch(void** ptr);
int decode_pick_split(const DecodeDims& d, int mode, int k, int n_split);
size_t decode_ws_bytes(const DecodeDims& d, int mode, int k, int n_split);
hipError_t launch_decode_attn(const void* q, const void* kpool, const void* vpool,
                              const int32_t* pt, const int32_t* sl, const DecodeDims& d,
                              int mode, const int32_t* idx, const float* scores, int k,
                              const int32_t* seg,
                              const int32_t* nseg, int max_seg, int n_split, float scale,
                              void* out, float* lse, void* ws, hipStream_t st);

}  // namespace fsa
