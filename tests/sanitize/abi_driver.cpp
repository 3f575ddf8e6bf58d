// Drives every entry point of the C ABI layer (api.hip, built host-only with
// AddressSanitizer and UBSan and linked against abi_stubs.cpp) through valid
// and invalid arguments: each call must return the documented status, and a
// call that fails must launch nothing.  The pointers are host addresses that
// nothing dereferences (the stubs only count launches), so what the
// sanitizers check is the layer's own host code: validation, the size
// arithmetic of the workspaces (also at the largest sizes), and the carving
// of the workspace into its parts.  Exit status 0 when every check held.
#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "dsa.h"

extern "C" int dsa_stub_launches();
extern "C" void dsa_stub_reset();

namespace {

int g_failures = 0;

#define EXPECT(cond)                                                           \
  do {                                                                         \
    if (!(cond)) {                                                             \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);       \
      ++g_failures;                                                            \
    }                                                                          \
  } while (0)

// A call's status and how many launches it made.
struct Result {
  int status;
  int launches;
};
template <class F>
Result run(F&& f) {
  dsa_stub_reset();
  const int st = f();
  return Result{st, dsa_stub_launches()};
}
void expect_fail(Result r, int status, int line) {
  if (r.status != status || r.launches != 0) {
    fprintf(stderr, "line %d: status %d (want %d), launches %d (want 0)\n", line, r.status,
            status, r.launches);
    ++g_failures;
  }
}
void expect_ok(Result r, int launches, int line) {
  if (r.status != DSA_OK || r.launches != launches) {
    fprintf(stderr, "line %d: status %d (want 0), launches %d (want %d)\n", line, r.status,
            r.launches, launches);
    ++g_failures;
  }
}
#define FAILS(status, call) expect_fail(run([&] { return call; }), status, __LINE__)
#define OK(launches, call) expect_ok(run([&] { return call; }), launches, __LINE__)

alignas(256) unsigned char g_mem[1 << 16];
void* const P = g_mem;            // aligned, never dereferenced
void* const ODD = g_mem + 2;      // 2-byte aligned only
float* const PF = reinterpret_cast<float*>(g_mem);
int32_t* const PI = reinterpret_cast<int32_t*>(g_mem);
// A "workspace" pointer for any size: only compared and offset, never read.
void* const WS = g_mem;

void sizes() {
  const int32_t M = INT32_MAX;
  // Non-positive or too many rows: 0.
  EXPECT(dsa_topk_workspace_size(0, 1, 100, 1) == 0);
  EXPECT(dsa_forward_workspace_size(1, 1, 0, 2048) == 0);
  EXPECT(dsa_forward_workspace_size(M, M, M, M) == 0);
  EXPECT(dsa_sparse_mla_workspace_size(M, 2, 2048) == 0);
  EXPECT(dsa_dense_mla_workspace_size(1 << 12, 1 << 13, 1) == 0);
  EXPECT(dsa_sparse_mha_prefill_workspace_size(M, M) == 0);
  EXPECT(dsa_forward_workspace_size(1, 1, (1 << 28) + 1, 2048) == 0);
  EXPECT(dsa_dense_mla_workspace_size(1, 1, M) == 0);
  EXPECT(dsa_topk_workspace_size(1, 1, M, 2048) == 0);
  // The largest accepted shapes: sizes grow with every argument and do not wrap.
  const int32_t S = 1 << 28;
  const size_t big = dsa_forward_workspace_size(1 << 12, 1 << 12, S, 2048);
  EXPECT(big >= (size_t)(1 << 24) * (size_t)S * 4);
  EXPECT(dsa_forward_workspace_size(1, 1, 32768, 2048) <
         dsa_forward_workspace_size(2, 1, 32768, 2048));
  EXPECT(dsa_forward_workspace_size(1, 1, S, 2048) > (size_t)S * 4);
  EXPECT(dsa_sparse_mha_prefill_workspace_size(1, 1 << 24) > 0);
  EXPECT(dsa_dense_mla_workspace_size(1 << 12, 1 << 12, S) > 0);
}

void index_scores() {
  OK(1, dsa_index_scores(P, nullptr, PF, P, nullptr, PI, 2, 1, 100, 100, 1.f, DSA_BF16, PF, nullptr));
  OK(1, dsa_index_scores(P, PF, PF, P, PF, PI, 2, 1, 100, 100, 1.f, DSA_FP8_E4M3, PF, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_index_scores(nullptr, nullptr, PF, P, nullptr, PI, 2, 1, 100, 100, 1.f, 0, PF, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_index_scores(P, nullptr, PF, P, nullptr, PI, 2, 1, 100, 100, 1.f, 0, nullptr, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_index_scores(P, nullptr, PF, P, nullptr, PI, 2, 5, 100, 4, 1.f, 0, PF, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_index_scores(P, nullptr, PF, P, nullptr, PI, 2, 1, 100, 101, 1.f, 0, PF, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_index_scores(P, nullptr, PF, P, nullptr, PI, 2, 1, 100, 100, 1.f, DSA_FP8_E4M3, PF, nullptr));
  FAILS(DSA_ERR_UNSUPPORTED, dsa_index_scores(P, nullptr, PF, P, nullptr, PI, 2, 1, 100, 100, 1.f, 7, PF, nullptr));
  FAILS(DSA_ERR_UNSUPPORTED, dsa_index_scores(P, nullptr, PF, P, nullptr, PI, INT32_MAX, 2, 100, 100, 1.f, 0, PF, nullptr));
  FAILS(DSA_ERR_UNSUPPORTED, dsa_index_scores(P, nullptr, PF, P, nullptr, PI, 1, 1, INT32_MAX, INT32_MAX, 1.f, 0, PF, nullptr));
  OK(1, dsa_index_scores(P, nullptr, PF, P, nullptr, PI, 1 << 12, 1 << 12, 1 << 28, 1 << 28, 1.f, 0, PF, nullptr));
  FAILS(DSA_ERR_MISALIGNED, dsa_index_scores(ODD, nullptr, PF, P, nullptr, PI, 2, 1, 100, 100, 1.f, 0, PF, nullptr));
}

void topk() {
  for (int32_t S : {100, 4096, 32768, 131072, 1 << 20, 1 << 28}) {
    for (int32_t B : {1, 64, 1024, 4096}) {
      const size_t need = dsa_topk_workspace_size(B, 1, S, 2048);
      OK(1, dsa_topk(PF, PI, B, 1, S, S, 2048, PI, need ? WS : nullptr, need, nullptr));
      if (need > 0)
        FAILS(DSA_ERR_WORKSPACE_TOO_SMALL, dsa_topk(PF, PI, B, 1, S, S, 2048, PI, WS, need - 1, nullptr));
    }
  }
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_topk(PF, PI, 1, 1, 100, 100, 0, PI, WS, 1 << 20, nullptr));
  FAILS(DSA_ERR_UNSUPPORTED, dsa_topk(PF, PI, 1, 1, 100, 100, 2049, PI, WS, 1 << 20, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_topk(nullptr, PI, 1, 1, 100, 100, 16, PI, WS, 1 << 20, nullptr));
  FAILS(DSA_ERR_MISALIGNED, dsa_topk(PF, PI, 1, 1, 100, 100, 16, PI, g_mem + 16, 1 << 20, nullptr));
}

void attention() {
  const size_t need = dsa_sparse_mla_workspace_size(1, 1, 2048);
  EXPECT(need > 0);
  OK(1, dsa_sparse_mla(P, P, P, P, PI, 1, 1, 4096, 2048, 0.07f, P, PF, WS, need, nullptr));
  OK(1, dsa_sparse_mla(P, P, P, P, PI, 1, 1, 4096, 2048, 0.07f, P, nullptr, WS, need, nullptr));
  for (float bad : {0.f, -1.f, INFINITY, NAN})
    FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_sparse_mla(P, P, P, P, PI, 1, 1, 4096, 2048, bad, P, PF, WS, need, nullptr));
  FAILS(DSA_ERR_WORKSPACE_TOO_SMALL, dsa_sparse_mla(P, P, P, P, PI, 1, 1, 4096, 2048, 0.07f, P, PF, WS, need - 1, nullptr));
  FAILS(DSA_ERR_UNSUPPORTED, dsa_sparse_mla(P, P, P, P, PI, 1, 1, 4096, 4096, 0.07f, P, PF, WS, need, nullptr));
  FAILS(DSA_ERR_MISALIGNED, dsa_sparse_mla(P, ODD, P, P, PI, 1, 1, 4096, 2048, 0.07f, P, PF, WS, need, nullptr));
  const size_t dneed = dsa_dense_mla_workspace_size(8, 1, 65536);
  OK(1, dsa_dense_mla(P, P, P, P, PI, 8, 1, 65536, 65536, 0.07f, P, PF, WS, dneed, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_dense_mla(P, P, P, P, PI, 8, 1, 65536, 65537, 0.07f, P, PF, WS, dneed, nullptr));
  if (dneed > 0)
    FAILS(DSA_ERR_WORKSPACE_TOO_SMALL, dsa_dense_mla(P, P, P, P, PI, 8, 1, 65536, 65536, 0.07f, P, PF, WS, dneed - 1, nullptr));
}

void forward() {
  struct Shape {
    int32_t B, T, S;
  };
  for (Shape s : {Shape{1, 1, 4096}, Shape{1, 1, 32768}, Shape{64, 1, 131072}, Shape{1, 8192, 8192},
                  Shape{8, 1, 1024}, Shape{3, 5, 777}}) {
    const size_t need = dsa_forward_workspace_size(s.B, s.T, s.S, 2048);
    EXPECT(need >= (size_t)s.B * s.T * s.S * 4 + (size_t)s.B * s.T * 2048 * 4);
    OK(3, dsa_forward(P, nullptr, PF, P, nullptr, PI, P, P, P, P, s.B, s.T, s.S, s.S, 2048, 1.f,
                      0.07f, DSA_BF16, P, PF, PI, WS, need, nullptr));
    OK(3, dsa_forward(P, PF, PF, P, PF, PI, P, P, P, P, s.B, s.T, s.S, s.S, 2048, 1.f, 0.07f,
                      DSA_FP8_E4M3, P, nullptr, nullptr, WS, need, nullptr));
    FAILS(DSA_ERR_WORKSPACE_TOO_SMALL,
          dsa_forward(P, nullptr, PF, P, nullptr, PI, P, P, P, P, s.B, s.T, s.S, s.S, 2048, 1.f,
                      0.07f, DSA_BF16, P, PF, PI, WS, need - 1, nullptr));
  }
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_forward(P, nullptr, PF, P, nullptr, PI, nullptr, P, P, P, 1, 1, 100, 100, 2048, 1.f, 0.07f, 0, P, PF, PI, WS, 1 << 20, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_forward(P, nullptr, PF, P, nullptr, PI, P, P, P, P, 1, 1, 100, 100, 2048, 1.f, 0.f, 0, P, PF, PI, WS, 1 << 20, nullptr));
  FAILS(DSA_ERR_UNSUPPORTED, dsa_forward(P, nullptr, PF, P, nullptr, PI, P, P, P, P, 1, 1, 100, 100, 2049, 1.f, 0.07f, 0, P, PF, PI, WS, 1 << 20, nullptr));
  FAILS(DSA_ERR_MISALIGNED, dsa_forward(P, nullptr, PF, P, nullptr, PI, P, P, P, P, 1, 1, 100, 100, 2048, 1.f, 0.07f, 0, P, PF, reinterpret_cast<int32_t*>(g_mem + 2), WS, 1 << 20, nullptr));
  // The no-allocation form: too large for its scratch, refused before any
  // HIP call; within it, either it runs (3 launches) or, with no GPU, the
  // scratch address cannot be had (DSA_ERR_HIP, nothing launched).
  FAILS(DSA_ERR_WORKSPACE_TOO_SMALL, dsa_forward_noalloc(P, nullptr, PF, P, nullptr, PI, P, P, P, P, 2, 1, 1 << 24, 1 << 24, 2048, 1.f, 0.07f, 0, P, PF, PI, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_forward_noalloc(nullptr, nullptr, PF, P, nullptr, PI, P, P, P, P, 1, 1, 100, 100, 2048, 1.f, 0.07f, 0, P, PF, PI, nullptr));
  const Result r = run([&] {
    return dsa_forward_noalloc(P, nullptr, PF, P, nullptr, PI, P, P, P, P, 1, 1, 32768, 32768, 2048,
                               1.f, 0.07f, 0, P, PF, PI, nullptr);
  });
  EXPECT((r.status == DSA_OK && r.launches == 3) || (r.status == DSA_ERR_HIP && r.launches == 0));
}

void products() {
  OK(1, dsa_q_absorb(P, P, 4, 3, P, nullptr));
  OK(1, dsa_out_proj(P, P, 4, 3, P, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_q_absorb(P, P, 1 << 12, 1 << 13, P, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_out_proj(nullptr, P, 1, 1, P, nullptr));
  const size_t need = dsa_sparse_mha_prefill_workspace_size(1, 8192);
  OK(1, dsa_sparse_mha_prefill(P, P, P, P, PI, 1, 8192, 2048, 0.07f, P, PF, WS, need, nullptr));
  FAILS(DSA_ERR_WORKSPACE_TOO_SMALL, dsa_sparse_mha_prefill(P, P, P, P, PI, 1, 8192, 2048, 0.07f, P, PF, WS, need - 1, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_sparse_mha_prefill(P, P, P, P, PI, 1, 8192, 2048, NAN, P, PF, WS, need, nullptr));
  OK(1, dsa_indexer_prep(P, P, PF, PF, PI, 64, 1, 4096, DSA_FP8_E4M3, P, PF, P, PF, nullptr));
  OK(1, dsa_indexer_prep(P, P, PF, PF, PI, 1, 8192, 8192, DSA_BF16, P, nullptr, P, nullptr, nullptr));
  FAILS(DSA_ERR_INVALID_ARGUMENT, dsa_indexer_prep(P, P, PF, PF, PI, 1, 8192, 8191, DSA_BF16, P, nullptr, P, nullptr, nullptr));
}

}  // namespace

int main() {
  for (int st = -6; st <= 1; ++st) EXPECT(dsa_status_string(st) != nullptr);
  sizes();
  index_scores();
  topk();
  attention();
  forward();
  products();
  if (g_failures) {
    fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  printf("abi driver: all checks passed\n");
  return 0;
}
