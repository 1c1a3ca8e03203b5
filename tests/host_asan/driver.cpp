// Host-side check of the C ABI's argument validation under AddressSanitizer.
//
// Every call below hands the library arguments that its validation must
// reject (or a call with nothing to compute), so no call reaches the device:
// the pointers are fake, suitably aligned addresses.  The library's host code
// is built with -fsanitize=address; any out-of-bounds read of an argument
// array, use of freed memory or overflow in the validation paths aborts the
// process.  Exit status 0: every call returned the expected class of status.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "fmha_mqa.h"

namespace {

int g_failures = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++g_failures;
  }
}

void* const A = reinterpret_cast<void*>(uintptr_t(1) << 20);  // 16-byte aligned, never touched
float* const AF = static_cast<float*>(A);
const int32_t* const AI = static_cast<const int32_t*>(A);

}  // namespace

int main() {
  // status text for every code, known or not
  for (int s = -3; s < 12; ++s) {
    const char* t = fmha_status_string(s);
    if (t == nullptr || strlen(t) == 0) ++g_failures;
  }
  // workspace sizes, including arguments that size nothing
  (void)fmha_mqa_workspace_bytes(32, 1, 128, 256, 8);
  (void)fmha_mqa_workspace_bytes(-1, 1, 1, 64, 2);
  (void)fmha_mqa_workspace_bytes(1 << 20, 1 << 10, 128, 512, 64);

  // the forward: nothing to compute, then one bad argument at a time
  expect("fwd B=0", fmha_mqa_fwd(A, A, A, nullptr, A, AF, 0, 1, 1, 8, 64, 0, 0.125f, 0, 1,
                                 nullptr, 0, nullptr), FMHA_OK);
  expect("fwd hd", fmha_mqa_fwd(A, A, A, nullptr, A, AF, 1, 1, 1, 8, 96, 0, 0.125f, 0, 1,
                                nullptr, 0, nullptr), FMHA_ERR_UNSUPPORTED);
  expect("fwd q", fmha_mqa_fwd(nullptr, A, A, nullptr, A, AF, 1, 1, 1, 8, 64, 0, 0.125f, 0, 1,
                               nullptr, 0, nullptr), FMHA_ERR_INVALID_ARG);
  expect("fwd splits", fmha_mqa_fwd(A, A, A, nullptr, A, AF, 1, 1, 1, 8, 64, 0, 0.125f, 0, 9,
                                    nullptr, 0, nullptr), FMHA_ERR_INVALID_ARG);
  expect("fwd align", fmha_mqa_fwd(static_cast<char*>(A) + 8, A, A, nullptr, A, AF, 1, 1, 1, 8,
                                   64, 0, 0.125f, 0, 1, nullptr, 0, nullptr), FMHA_ERR_ALIGNMENT);
  expect("fwd pool", fmha_mqa_fwd(A, A, A, AI, A, AF, 1, 1, 1, 8, 64, 0, 0.125f, 0, 1, nullptr, 0,
                                  nullptr), FMHA_ERR_INVALID_ARG);
  expect("fwd scale", fmha_mqa_fwd(A, A, A, nullptr, A, AF, 1, 1, 1, 8, 64, 0, 0.f, 0, 1,
                                   nullptr, 0, nullptr), FMHA_ERR_INVALID_ARG);
  expect("sink align", fmha_mqa_fwd_sink(A, A, A, nullptr, A, AF, 1, 1, 1, 8, 64, 0, 0.125f, 0,
                                         1, nullptr, 0, nullptr,
                                         reinterpret_cast<const float*>(static_cast<char*>(A) + 2)),
         FMHA_ERR_ALIGNMENT);
  expect("noalloc limit", fmha_mqa_fwd_noalloc(A, A, A, nullptr, A, AF, 32, 1, 128, 1024, 512, 0,
                                               0.125f, 1, 8, nullptr), FMHA_ERR_SCRATCH_LIMIT);
  expect("partials o", fmha_mqa_fwd_partials(A, A, A, nullptr, nullptr, AF, 1, 1, 1, 8, 64, 0,
                                             0.125f, 1, nullptr), FMHA_ERR_INVALID_ARG);

  // several sources: an empty list, then five sources with the bad one last
  expect("sources none", fmha_mqa_fwd_sources_partials(A, nullptr, 1, AF, AF, 1, 1, 1, 512,
                                                       0.125f, nullptr), FMHA_ERR_INVALID_ARG);
  std::vector<fmha_kv_source> src(5, fmha_kv_source{A, A, nullptr, 64, 0, 2});
  src[4].num_splits = 65;  // more splits than keys
  expect("sources last", fmha_mqa_fwd_sources_partials(A, src.data(), (int)src.size(), AF, AF, 1,
                                                       1, 1, 512, 0.125f, nullptr),
         FMHA_ERR_INVALID_ARG);
  src[4].num_splits = 1;
  src[2].kv_idx = AI;  // a gather source without a pool
  expect("sources pool", fmha_mqa_fwd_sources_partials(A, src.data(), (int)src.size(), AF, AF, 1,
                                                       1, 1, 512, 0.125f, nullptr),
         FMHA_ERR_INVALID_ARG);
  expect("sources rows=0", fmha_mqa_fwd_sources_partials(A, src.data() + 3, 2, AF, AF, 0, 1, 1,
                                                         512, 0.125f, nullptr), FMHA_OK);

  // the merge, the sink, the indexer and the measurement helpers
  expect("merge parts", fmha_lse_merge(AF, AF, 0, 4, 64, A, 0, AF, nullptr),
         FMHA_ERR_INVALID_ARG);
  expect("merge hd", fmha_lse_merge(AF, AF, 2, 4, 6, A, 0, AF, nullptr), FMHA_ERR_INVALID_ARG);
  expect("attention sink", fmha_attention_sink(A, AF, nullptr, 4, 1, 64, 0, nullptr),
         FMHA_ERR_INVALID_ARG);
  expect("index scores", fmha_index_scores(A, A, AF, AF, 1, 1, 48, 128, 100, nullptr),
         FMHA_ERR_UNSUPPORTED);
  expect("topk", fmha_topk_select(AF, const_cast<int32_t*>(AI), 1, 100, 0, nullptr),
         FMHA_ERR_INVALID_ARG);
  expect("gather floor", fmha_gather_floor(A, A, AI, static_cast<uint32_t*>(A), 1, 1, 8, 64, 0,
                                           nullptr), FMHA_ERR_INVALID_ARG);
  expect("read floor", fmha_read_floor(A, A, A, static_cast<uint32_t*>(A), 1, 1, 8, 128, 256, 0,
                                       nullptr), FMHA_ERR_INVALID_ARG);
  expect("mfma ceiling", fmha_mfma_ceiling(A, AF, static_cast<uint64_t*>(A), 0, 1, nullptr),
         FMHA_ERR_INVALID_ARG);

  if (g_failures) {
    fprintf(stderr, "%d unexpected statuses\n", g_failures);
    return 1;
  }
  printf("host validation under AddressSanitizer: ok\n");
  return 0;
}
