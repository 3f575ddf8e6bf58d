// Host-only stand-ins for the kernel launchers and planners of libdsa, for
// the sanitizer build of the C ABI layer (api.hip).  Nothing here touches
// memory behind the pointers it gets: each launcher only counts its call and
// checks that the pointers it must write through are non-null, so AddressSan
// and UBSan see api.hip's own host code (validation, size arithmetic,
// workspace carving) and the driver can tell whether anything was launched.
#include <stddef.h>
#include <stdint.h>

#include "dsa_launch.h"

namespace {
int g_launches = 0;
int launched(bool ok) {
  ++g_launches;
  return ok ? 0 : -5;
}
}  // namespace

extern "C" int dsa_stub_launches() { return g_launches; }
extern "C" void dsa_stub_reset() { g_launches = 0; }

namespace dsa {

int launch_index_scores(const void* q, const float*, const float* w, const void* k, const float*,
                        const int32_t* end_pos, int B, int T, int S_max, int max_end_pos, float,
                        int, float* out, uint32_t*, hipStream_t) {
  return launched(q && w && k && end_pos && out && B > 0 && T > 0 && max_end_pos <= S_max);
}

size_t topk_workspace_bytes(int B, int T, int S_max, int) {
  const size_t rows = (size_t)B * T;
  return rows > 1024 ? 0 : rows * (S_max <= 4096 ? 65536 : 262144);
}
uint32_t* topk_counters(void* workspace, int B, int T, int max_end_pos) {
  return ((long)B * T <= 1024 && (max_end_pos <= 4096 || max_end_pos > 32768))
             ? reinterpret_cast<uint32_t*>(workspace)
             : nullptr;
}
int launch_topk(const float* scores, const int32_t* end_pos, int B, int T, int, int, int k,
                int32_t* out, void* ws, bool, hipStream_t) {
  return launched(scores && end_pos && out && k > 0 &&
                  ((long)B * T > 1024 || ws != nullptr));
}

MlaPlan sparse_mla_plan(int B, int T, int k) {
  const long rows = (long)B * T;
  const int rps = rows <= 16 ? 64 : 512;
  return MlaPlan{rps, (k + rps - 1) / rps, rows <= 16 ? 4 : 8, rows <= 16};
}
MlaPlan dense_mla_plan(int B, int T, int S_max, int max_end_pos) {
  const int ext = max_end_pos > 0 ? max_end_pos : S_max;
  (void)B;
  (void)T;
  return MlaPlan{512, (ext + 511) / 512, 8};  // callers keep S_max <= 2^28
}
size_t mla_workspace_bytes(int B, int T, const MlaPlan& plan) {
  if (plan.n_splits <= 1) return 0;
  return (size_t)B * T * plan.n_splits * (128 * 512 * 2 + 128 * 16);
}
int launch_sparse_mla(const void* qn, const void* qp, const void* kv, const void* pe,
                      const int32_t* idx, int, int, int, int, float, void* out, float*, void*,
                      hipStream_t, const int32_t*) {
  return launched(qn && qp && kv && pe && idx && out);
}
int launch_dense_mla(const void* qn, const void* qp, const void* kv, const void* pe,
                     const int32_t* end_pos, int, int, int, int, float, void* out, float*, void*,
                     hipStream_t) {
  return launched(qn && qp && kv && pe && end_pos && out);
}
int launch_q_absorb(const void* q, const void* w, int rows, void* out, hipStream_t) {
  return launched(q && w && out && rows > 0);
}
int launch_out_proj(const void* x, const void* w, int rows, void* y, hipStream_t) {
  return launched(x && w && y && rows > 0);
}
size_t mha_prefill_workspace_bytes(int B, int T) { return (size_t)B * T * 256; }
int launch_mha_prefill(const void* q, const void* kn, const void* kp, const void* v,
                       const int32_t* idx, int, int, int, float, void* out, float*, void* ws,
                       hipStream_t) {
  return launched(q && kn && kp && v && idx && out && ws);
}
int launch_indexer_prep(const void* qi, const void* ki, const float* c, const float* s,
                        const int32_t* ep, int, int, int, int, void* qo, float*, void* kc, float*,
                        hipStream_t) {
  return launched(qi && ki && c && s && ep && qo && kc);
}

}  // namespace dsa
