// Host-side exercise of the C ABI for a sanitizer build (no GPU needed):
// every entry point with missing, malformed and extreme arguments, workspace
// sizing over a sweep of shapes, and the segment builders over random and
// extreme inputs, checking the documented status codes and output
// invariants.  Valid calls end in the device check, which reports
// FSA_ERR_NO_DEVICE on a host without a GPU.  Exit status 0 = every check
// held; the sanitizer reports memory errors on its own.
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "fsa.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static void* const FAKE = reinterpret_cast<void*>(0x1000);  // never dereferenced

int main() {
  std::mt19937 rng(12345);
  const bool no_gpu = fsa_device_check() == FSA_ERR_NO_DEVICE;
  for (int c = 1; c >= -9; --c) CHECK(fsa_status_string(c) != nullptr);

  // prefill shapes: a sweep including invalid and extreme values
  const int Bs[] = {0, 1, 2, 600, INT_MAX};
  const int Ss[] = {0, 64, 1000, 131072, 524288, 524352, INT_MAX};
  const int Hs[] = {0, 1, 2, 32, 1024, 2048};
  const int Ds[] = {0, 64, 96, 128};
  const int Ts[] = {32, 64, 128};
  for (int B : Bs)
    for (int S : Ss)
      for (int Hq : Hs)
        for (int D : Ds)
          for (int T : Ts) {
            fsa_prefill_shape s{B, S, Hq, Hq > 1 ? Hq / 2 : 1, D, T};
            (void)fsa_workspace_size(FSA_OP_SELECT_BLOCKS, &s, nullptr);
            (void)fsa_workspace_size(FSA_OP_PREFILL_ATTN, &s, nullptr);
            const int rc = block_stats(FSA_BF16, FAKE, &s, (float*)FAKE, (float*)FAKE, nullptr);
            CHECK(rc == FSA_ERR_SHAPE || rc == (no_gpu ? FSA_ERR_NO_DEVICE : FSA_OK));
            if (rc == FSA_OK) return 2;  // a launch on fake pointers: never on this host
          }
  fsa_prefill_shape ps{1, 1024, 2, 2, 64, 64};
  CHECK(block_stats(FSA_BF16, nullptr, &ps, (float*)FAKE, (float*)FAKE, nullptr) == FSA_ERR_NULL);
  CHECK(block_stats((fsa_dtype)9, FAKE, &ps, (float*)FAKE, (float*)FAKE, nullptr) == FSA_ERR_DTYPE);
  CHECK(sparse_prefill_attn(FSA_BF16, FAKE, FAKE, FAKE, &ps, nullptr, nullptr, -1.f, FAKE, nullptr,
                            nullptr, 0, nullptr) == FSA_ERR_ARG);
  fsa_select_params sp{0.25, 0.1, 0, 0};
  const size_t sws = fsa_workspace_size(FSA_OP_SELECT_BLOCKS, &ps, nullptr);
  CHECK(select_blocks(FSA_F32, FAKE, (float*)FAKE, (float*)FAKE, &ps, &sp, (uint32_t*)FAKE,
                      (int32_t*)FAKE, (int32_t*)FAKE, nullptr, nullptr, FAKE, sws - 1,
                      nullptr) == FSA_ERR_WORKSPACE);
  CHECK(select_blocks(FSA_F32, FAKE, (float*)FAKE, (float*)FAKE, &ps, nullptr, (uint32_t*)FAKE,
                      (int32_t*)FAKE, (int32_t*)FAKE, nullptr, nullptr, FAKE, sws,
                      nullptr) == FSA_ERR_NULL);

  // decode shapes and selections
  for (int trial = 0; trial < 20000; ++trial) {
    fsa_decode_shape s;
    s.B = (int)(rng() % 70) - 2;
    s.Hkv = 1 << (rng() % 5);
    s.Hq = s.Hkv * ((rng() % 10) + 1);
    s.D = (rng() % 3 == 0) ? 96 : ((rng() & 1) ? 64 : 128);
    s.page_size = (rng() % 10 == 0) ? 32 : 16;
    s.num_pages = (int)(rng() % 1000000) - 5;
    s.max_pages = (int)(rng() % 70000) - 5;
    s.max_seq_len = (int)(rng() % (1u << 24)) - 5;
    int k = (int)(rng() % 5000) - 2;
    (void)fsa_workspace_size(FSA_OP_TOPK, &s, &k);
    fsa_kv_select sel{(int32_t)(rng() % 5), (const int32_t*)FAKE, (int32_t)(rng() % 5000) - 2,
                      (const int32_t*)FAKE, (const int32_t*)FAKE, (int32_t)(rng() % 70) - 2,
                      (int32_t)(rng() % 5000) - 2};
    (void)fsa_workspace_size(FSA_OP_DECODE_ATTN, &s, &sel);
    const int rc = sparse_decode_attn(FSA_BF16, FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                      (const int32_t*)FAKE, &s, &sel, 0.1f, FAKE, nullptr, FAKE,
                                      (size_t)1 << 40, nullptr);
    CHECK(rc < 0);
    if (rc == FSA_OK) return 2;
    const int rc2 = sparse_decode_attn_noalloc(FSA_BF16, FAKE, FAKE, FAKE, (const int32_t*)FAKE,
                                               (const int32_t*)FAKE, &s, &sel, 0.1f, FAKE,
                                               nullptr, nullptr);
    CHECK(rc2 < 0);
    if (rc2 == FSA_OK) return 2;
    const int rc3 = topk_indices(FSA_BF16, FAKE, FAKE, (const int32_t*)FAKE, (const int32_t*)FAKE,
                                 &s, k, (int32_t*)FAKE, nullptr, FAKE, (size_t)1 << 40, nullptr);
    CHECK(rc3 < 0);
    if (rc3 == FSA_OK) return 2;
    const int rc4 = topk_union_kv((const int32_t*)FAKE, s.B, s.Hq, s.Hkv, k, (int32_t*)FAKE,
                                  nullptr, nullptr);
    CHECK(rc4 < 0);
    if (rc4 == FSA_OK) return 2;
  }
  CHECK(fsa_workspace_size(FSA_OP_DECODE_ATTN, nullptr, nullptr) == 0);
  CHECK(fsa_workspace_size(77, FAKE, nullptr) == 0);

  // segment builders: random and extreme arguments; outputs sorted, disjoint,
  // non-touching, inside [0, n), at most two ranges
  int32_t out[4];
  int nseg = -1;
  const int ext[] = {INT_MIN, -1, 0, 1, 15, 16, 17, 1023, 1024, 2048, 1 << 20, INT_MAX - 16,
                     INT_MAX};
  for (int trial = 0; trial < 200000; ++trial) {
    const bool wild = rng() % 4 == 0;
    auto pick = [&](int hi) {
      return wild ? ext[rng() % (sizeof(ext) / sizeof(ext[0]))] : (int)(rng() % (unsigned)hi);
    };
    const int mode = (int)(rng() % 6) - 1, n = pick(1 << 21), st = pick(1 << 21),
              len = pick(4096), loc = pick(4096), sink = pick(8), page = wild ? pick(64) : 16,
              nb = pick(5000);
    nseg = -1;
    const int rc = fsa_build_segments_nb(mode, n, st, len, loc, sink, page, nb, out, &nseg);
    if (rc != FSA_OK) {
      CHECK(rc == FSA_ERR_ARG);
      continue;
    }
    CHECK(nseg >= 0 && nseg <= 2);
    for (int x = 0; x < nseg; ++x) {
      CHECK(0 <= out[2 * x] && out[2 * x] < out[2 * x + 1] && out[2 * x + 1] <= n);
      if (x) CHECK(out[2 * x - 1] < out[2 * x]);
    }
  }
  CHECK(fsa_build_segments(FSA_SEG_GLOBAL, 10, 0, 0, 0, 0, 16, nullptr, &nseg) == FSA_ERR_NULL);

  std::printf("abi driver: %d failed checks\n", failures);
  return failures ? 1 : 0;
}
