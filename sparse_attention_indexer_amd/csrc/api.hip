// C ABI of libdsa.so (declared in include/dsa.h): argument validation on the
// host, workspace carving, and kernel launches on the caller's stream.  No
// device allocation and no synchronisation.  The only global state is the
// device scratch of dsa_forward_noalloc and the table of its per-device
// addresses; dsa_forward_graph_create returns a captured step the caller owns.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <new>

#include "dsa.h"

#include "dsa_launch.h"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

enum {
  kOk = 0,
  kErrInvalid = -1,
  kErrUnsupported = -2,
  kErrMisaligned = -3,
  kErrWorkspace = -4,
  kErrHip = -5,
};

constexpr int kMaxTopk = 2048;
constexpr size_t kWsAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
// A softmax scale must be a positive finite number (the kernels take the
// running maximum on unscaled scores).
bool good_softmax_scale(float s) { return s > 0.f && __builtin_isfinite(s); }
size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Query rows (B*T) a call may cover, and cache positions per sequence: grids,
// row indices and position arithmetic (rounding up to whole tiles included)
// stay well inside 32-bit integers.  2^28 positions of one sequence's latent
// cache alone would be 309 GB.
constexpr long kMaxRows = 1L << 24;
constexpr int32_t kMaxPositions = 1 << 28;
bool rows_ok(int32_t B, int32_t T) { return B >= 1 && T >= 1 && (long)B * T <= kMaxRows; }
bool positions_ok(int32_t S_max) { return S_max >= 1 && S_max <= kMaxPositions; }

// Shared checks of the (B, T, S_max, max_end_pos) geometry.
int check_geometry(int32_t B, int32_t T, int32_t S_max, int32_t max_end_pos) {
  if (B < 1 || T < 1 || S_max < 1) return kErrInvalid;
  if (!rows_ok(B, T) || !positions_ok(S_max)) return kErrUnsupported;
  if (max_end_pos < T || max_end_pos > S_max) return kErrInvalid;
  return kOk;
}

int check_indexer(const void* q, const float* q_scale, const float* w, const void* k_cache,
                  const float* k_scale, const int32_t* end_pos, int32_t B, int32_t T,
                  int32_t S_max, int32_t max_end_pos, int32_t dtype) {
  if (!q || !w || !k_cache || !end_pos) return kErrInvalid;
  int st = check_geometry(B, T, S_max, max_end_pos);
  if (st) return st;
  if (dtype != 0 && dtype != 1) return kErrUnsupported;
  if (dtype == 1 && (!q_scale || !k_scale)) return kErrInvalid;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(w) || !aligned4(end_pos))
    return kErrMisaligned;
  if (dtype == 1 && (!aligned16(q_scale) || !aligned4(k_scale))) return kErrMisaligned;
  return kOk;
}

int check_topk(const float* scores, const int32_t* end_pos, int32_t B, int32_t T, int32_t S_max,
               int32_t max_end_pos, int32_t k, const int32_t* out) {
  if (!scores || !end_pos || !out) return kErrInvalid;
  int st = check_geometry(B, T, S_max, max_end_pos);
  if (st) return st;
  if (k < 1) return kErrInvalid;
  if (k > kMaxTopk) return kErrUnsupported;
  if (!aligned4(scores) || !aligned4(end_pos) || !aligned4(out)) return kErrMisaligned;
  return kOk;
}

int check_mla_tensors(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                      const void* out, const float* lse) {
  if (!q_nope || !q_pe || !kv || !pe || !out) return kErrInvalid;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(kv) || !aligned16(pe) ||
      !aligned16(out) || (lse && !aligned4(lse)))
    return kErrMisaligned;
  return kOk;
}

int check_workspace(const void* ws, size_t have, size_t need) {
  if (have < need) return kErrWorkspace;
  if (need > 0 && !ws) return kErrInvalid;
  if (need > 0 && (reinterpret_cast<uintptr_t>(ws) & (kWsAlign - 1)) != 0) return kErrMisaligned;
  return kOk;
}

size_t sparse_mla_ws(int32_t B, int32_t T, int32_t k) {
  return dsa::mla_workspace_bytes(B, T, dsa::sparse_mla_plan(B, T, k));
}

struct ForwardLayout {
  size_t scores, indices, topk_ws, mla_ws, total;
};

ForwardLayout forward_layout(int32_t B, int32_t T, int32_t S_max, int32_t k) {
  ForwardLayout L;
  const size_t rows = (size_t)B * T;
  L.scores = 0;
  L.indices = L.scores + align_up(rows * (size_t)S_max * sizeof(float));
  L.topk_ws = L.indices + align_up(rows * (size_t)k * sizeof(int32_t));
  L.mla_ws = L.topk_ws + align_up(dsa::topk_workspace_bytes(B, T, S_max, k));
  L.total = L.mla_ws + align_up(sparse_mla_ws(B, T, k));
  return L;
}

}  // namespace

DSA_EXPORT const char* dsa_status_string(int status) {
  switch (status) {
    case kOk: return "DSA_OK: success";
    case kErrInvalid: return "DSA_ERR_INVALID_ARGUMENT: null pointer or inconsistent size";
    case kErrUnsupported: return "DSA_ERR_UNSUPPORTED: dtype or shape outside the specialisation";
    case kErrMisaligned: return "DSA_ERR_MISALIGNED: tensor or workspace pointer misaligned";
    case kErrWorkspace: return "DSA_ERR_WORKSPACE_TOO_SMALL: workspace smaller than required";
    case kErrHip: return "DSA_ERR_HIP: kernel launch failed";
    default: return "unknown dsa status";
  }
}

DSA_EXPORT int dsa_index_scores(const void* q, const float* q_scale, const float* weights,
                                const void* k_cache, const float* k_scale,
                                const int32_t* end_pos, int32_t B, int32_t T, int32_t S_max,
                                int32_t max_end_pos, float scale, int32_t dtype,
                                float* index_score, hipStream_t stream) {
  int st = check_indexer(q, q_scale, weights, k_cache, k_scale, end_pos, B, T, S_max,
                         max_end_pos, dtype);
  if (st) return st;
  if (!index_score) return kErrInvalid;
  if (!aligned4(index_score)) return kErrMisaligned;
  return dsa::launch_index_scores(q, q_scale, weights, k_cache, k_scale, end_pos, B, T, S_max,
                                  max_end_pos, scale, dtype, index_score, nullptr, stream);
}

DSA_EXPORT size_t dsa_topk_workspace_size(int32_t B, int32_t T, int32_t S_max, int32_t k) {
  if (!rows_ok(B, T) || !positions_ok(S_max) || k < 1) return 0;
  return dsa::topk_workspace_bytes(B, T, S_max, k);
}

DSA_EXPORT int dsa_topk(const float* index_score, const int32_t* end_pos, int32_t B, int32_t T,
                        int32_t S_max, int32_t max_end_pos, int32_t k, int32_t* topk_indices,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_topk(index_score, end_pos, B, T, S_max, max_end_pos, k, topk_indices);
  if (st) return st;
  st = check_workspace(workspace, workspace_bytes, dsa::topk_workspace_bytes(B, T, S_max, k));
  if (st) return st;
  return dsa::launch_topk(index_score, end_pos, B, T, S_max, max_end_pos, k, topk_indices,
                          workspace, /*counters_clear=*/false, stream);
}

DSA_EXPORT size_t dsa_sparse_mla_workspace_size(int32_t B, int32_t T, int32_t k) {
  if (!rows_ok(B, T) || k < 1) return 0;
  return sparse_mla_ws(B, T, k);
}

DSA_EXPORT int dsa_sparse_mla(const void* q_nope, const void* q_pe, const void* kv_cache,
                              const void* pe_cache, const int32_t* topk_indices, int32_t B,
                              int32_t T, int32_t S_max, int32_t k, float softmax_scale,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  int st = check_mla_tensors(q_nope, q_pe, kv_cache, pe_cache, out, lse);
  if (st) return st;
  if (!topk_indices) return kErrInvalid;
  if (B < 1 || T < 1 || S_max < 1 || k < 1) return kErrInvalid;
  if (!rows_ok(B, T) || !positions_ok(S_max)) return kErrUnsupported;
  if (!good_softmax_scale(softmax_scale)) return kErrInvalid;
  if (k > kMaxTopk) return kErrUnsupported;
  if (!aligned4(topk_indices)) return kErrMisaligned;
  st = check_workspace(workspace, workspace_bytes, sparse_mla_ws(B, T, k));
  if (st) return st;
  return dsa::launch_sparse_mla(q_nope, q_pe, kv_cache, pe_cache, topk_indices, B, T, S_max, k,
                                softmax_scale, out, lse, workspace, stream);
}

DSA_EXPORT size_t dsa_forward_workspace_size(int32_t B, int32_t T, int32_t S_max, int32_t k) {
  if (!rows_ok(B, T) || !positions_ok(S_max) || k < 1) return 0;
  return forward_layout(B, T, S_max, k).total;
}

namespace {

// Everything dsa_forward checks before its first launch.
int check_forward(const void* q, const float* q_scale, const float* weights, const void* k_cache,
                  const float* k_scale, const int32_t* end_pos, const void* q_nope,
                  const void* q_pe, const void* kv_cache, const void* pe_cache, int32_t B,
                  int32_t T, int32_t S_max, int32_t max_end_pos, int32_t k, float softmax_scale,
                  int32_t dtype, const void* out, const float* lse,
                  const int32_t* topk_indices_out) {
  int st = check_indexer(q, q_scale, weights, k_cache, k_scale, end_pos, B, T, S_max,
                         max_end_pos, dtype);
  if (st) return st;
  if (!good_softmax_scale(softmax_scale)) return kErrInvalid;
  st = check_mla_tensors(q_nope, q_pe, kv_cache, pe_cache, out, lse);
  if (st) return st;
  if (k < 1) return kErrInvalid;
  if (k > kMaxTopk) return kErrUnsupported;
  if (topk_indices_out && !aligned4(topk_indices_out)) return kErrMisaligned;
  return kOk;
}

// The three stages on `stream` over a checked workspace.
int run_forward(const void* q, const float* q_scale, const float* weights, const void* k_cache,
                const float* k_scale, const int32_t* end_pos, const void* q_nope,
                const void* q_pe, const void* kv_cache, const void* pe_cache, int32_t B,
                int32_t T, int32_t S_max, int32_t max_end_pos, int32_t k, float index_scale,
                float softmax_scale, int32_t dtype, void* out, float* lse,
                int32_t* topk_indices_out, char* ws, const ForwardLayout& L,
                hipStream_t stream) {
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  int32_t* indices =
      topk_indices_out ? topk_indices_out : reinterpret_cast<int32_t*>(ws + L.indices);
  // The indexer also clears the top-k's per-row counters (when that path has them).
  uint32_t* topk_ctr = dsa::topk_counters(ws + L.topk_ws, B, T, max_end_pos);
  int st = dsa::launch_index_scores(q, q_scale, weights, k_cache, k_scale, end_pos, B, T, S_max,
                                    max_end_pos, index_scale, dtype, scores, topk_ctr, stream);
  if (st) return st;
  st = dsa::launch_topk(scores, end_pos, B, T, S_max, max_end_pos, k, indices, ws + L.topk_ws,
                        /*counters_clear=*/topk_ctr != nullptr, stream);
  if (st) return st;
  // The selection fills each list's first min(k, causal bound) slots, so the
  // attention skips the rest (whole tiles of -1 for early prefill queries).
  return dsa::launch_sparse_mla(q_nope, q_pe, kv_cache, pe_cache, indices, B, T, S_max, k,
                                softmax_scale, out, lse, ws + L.mla_ws, stream, end_pos);
}

}  // namespace

DSA_EXPORT int dsa_forward(const void* q, const float* q_scale, const float* weights,
                           const void* k_cache, const float* k_scale, const int32_t* end_pos,
                           const void* q_nope, const void* q_pe, const void* kv_cache,
                           const void* pe_cache, int32_t B, int32_t T, int32_t S_max,
                           int32_t max_end_pos, int32_t k, float index_scale,
                           float softmax_scale, int32_t dtype, void* out, float* lse,
                           int32_t* topk_indices_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  // Validate everything before the first launch.
  int st = check_forward(q, q_scale, weights, k_cache, k_scale, end_pos, q_nope, q_pe, kv_cache,
                         pe_cache, B, T, S_max, max_end_pos, k, softmax_scale, dtype, out, lse,
                         topk_indices_out);
  if (st) return st;
  const ForwardLayout L = forward_layout(B, T, S_max, k);
  st = check_workspace(workspace, workspace_bytes, L.total);
  if (st) return st;
  return run_forward(q, q_scale, weights, k_cache, k_scale, end_pos, q_nope, q_pe, kv_cache,
                     pe_cache, B, T, S_max, max_end_pos, k, index_scale, softmax_scale, dtype,
                     out, lse, topk_indices_out, reinterpret_cast<char*>(workspace), L, stream);
}

// ---- dsa_forward_noalloc: dsa_forward's workspace in a library-held array ----
// Every GPU the library runs on holds its own copy of `scratch` from module
// load until the process ends.  In host code the name only stands for the
// symbol: its device address on the current device comes from
// hipGetSymbolAddress, taken once per device and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[DSA_FORWARD_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once known

// The address of the current device's scratch (looked up on its first use).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return kErrHip;
  if (dev < 0 || dev >= kMaxDevices) return kErrUnsupported;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return kErrHip;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return kOk;
}

}  // namespace

DSA_EXPORT int dsa_forward_noalloc(const void* q, const float* q_scale, const float* weights,
                                   const void* k_cache, const float* k_scale,
                                   const int32_t* end_pos, const void* q_nope, const void* q_pe,
                                   const void* kv_cache, const void* pe_cache, int32_t B,
                                   int32_t T, int32_t S_max, int32_t max_end_pos, int32_t k,
                                   float index_scale, float softmax_scale, int32_t dtype,
                                   void* out, float* lse, int32_t* topk_indices_out,
                                   hipStream_t stream) {
  int st = check_forward(q, q_scale, weights, k_cache, k_scale, end_pos, q_nope, q_pe, kv_cache,
                         pe_cache, B, T, S_max, max_end_pos, k, softmax_scale, dtype, out, lse,
                         topk_indices_out);
  if (st) return st;
  const ForwardLayout L = forward_layout(B, T, S_max, k);
  if (L.total > DSA_FORWARD_SCRATCH_BYTES) return kErrWorkspace;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  // Nothing in the workspace has to start at any particular value (the
  // indexer clears the top-k counters that need it), so no clearing here.
  return run_forward(q, q_scale, weights, k_cache, k_scale, end_pos, q_nope, q_pe, kv_cache,
                     pe_cache, B, T, S_max, max_end_pos, k, index_scale, softmax_scale, dtype,
                     out, lse, topk_indices_out, reinterpret_cast<char*>(ws), L, stream);
}

// ---- dsa_forward_graph_*: the decode step captured into a HIP graph ----
struct dsa_forward_graph {
  hipGraphExec_t exec;
};

DSA_EXPORT int dsa_forward_graph_create(const void* q, const float* q_scale,
                                        const float* weights, const void* k_cache,
                                        const float* k_scale, const int32_t* end_pos,
                                        const void* q_nope, const void* q_pe,
                                        const void* kv_cache, const void* pe_cache, int32_t B,
                                        int32_t T, int32_t S_max, int32_t max_end_pos,
                                        int32_t k, float index_scale, float softmax_scale,
                                        int32_t dtype, void* out, float* lse,
                                        int32_t* topk_indices_out, void* workspace,
                                        size_t workspace_bytes, dsa_forward_graph_t* graph) {
  if (!graph) return kErrInvalid;
  *graph = nullptr;
  int st = check_forward(q, q_scale, weights, k_cache, k_scale, end_pos, q_nope, q_pe, kv_cache,
                         pe_cache, B, T, S_max, max_end_pos, k, softmax_scale, dtype, out, lse,
                         topk_indices_out);
  if (st) return st;
  const ForwardLayout L = forward_layout(B, T, S_max, k);
  st = check_workspace(workspace, workspace_bytes, L.total);
  if (st) return st;
  // Capture on a private stream (default priority), thread-local mode, so
  // other threads' HIP calls are not drawn into the capture.
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return kErrHip;
  hipGraph_t g = nullptr;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    st = kErrHip;
  } else {
    st = run_forward(q, q_scale, weights, k_cache, k_scale, end_pos, q_nope, q_pe, kv_cache,
                     pe_cache, B, T, S_max, max_end_pos, k, index_scale, softmax_scale, dtype,
                     out, lse, topk_indices_out, reinterpret_cast<char*>(workspace), L, cs);
    const hipError_t e = hipStreamEndCapture(cs, &g);  // ends the capture whatever st is
    if (!st && (e != hipSuccess || !g)) st = kErrHip;
  }
  hipGraphExec_t exec = nullptr;
  if (!st && hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess) st = kErrHip;
  if (g) (void)hipGraphDestroy(g);
  (void)hipStreamDestroy(cs);
  if (st) return st;
  dsa_forward_graph* h = new (std::nothrow) dsa_forward_graph{exec};
  if (!h) {
    (void)hipGraphExecDestroy(exec);
    return kErrHip;
  }
  *graph = h;
  return kOk;
}

DSA_EXPORT int dsa_forward_graph_launch(dsa_forward_graph_t graph, hipStream_t stream) {
  if (!graph) return kErrInvalid;
  return hipGraphLaunch(graph->exec, stream) == hipSuccess ? kOk : kErrHip;
}

DSA_EXPORT int dsa_forward_graph_destroy(dsa_forward_graph_t graph) {
  if (!graph) return kOk;
  const hipError_t e = hipGraphExecDestroy(graph->exec);
  delete graph;
  return e == hipSuccess ? kOk : kErrHip;
}

DSA_EXPORT size_t dsa_dense_mla_workspace_size(int32_t B, int32_t T, int32_t S_max) {
  if (!rows_ok(B, T) || !positions_ok(S_max)) return 0;
  return dsa::mla_workspace_bytes(B, T, dsa::dense_mla_plan(B, T, S_max, S_max));
}

DSA_EXPORT int dsa_dense_mla(const void* q_nope, const void* q_pe, const void* kv_cache,
                             const void* pe_cache, const int32_t* end_pos, int32_t B, int32_t T,
                             int32_t S_max, int32_t max_end_pos, float softmax_scale, void* out,
                             float* lse, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  int st = check_mla_tensors(q_nope, q_pe, kv_cache, pe_cache, out, lse);
  if (st) return st;
  if (!good_softmax_scale(softmax_scale)) return kErrInvalid;
  if (!end_pos) return kErrInvalid;
  st = check_geometry(B, T, S_max, max_end_pos);
  if (st) return st;
  if (!aligned4(end_pos)) return kErrMisaligned;
  st = check_workspace(workspace, workspace_bytes,
                       dsa::mla_workspace_bytes(B, T, dsa::dense_mla_plan(B, T, S_max, S_max)));
  if (st) return st;
  return dsa::launch_dense_mla(q_nope, q_pe, kv_cache, pe_cache, end_pos, B, T, S_max,
                               max_end_pos, softmax_scale, out, lse, workspace, stream);
}

DSA_EXPORT int dsa_q_absorb(const void* q_nope, const void* wkv_b, int32_t B, int32_t T,
                            void* q_abs, hipStream_t stream) {
  if (!q_nope || !wkv_b || !q_abs) return kErrInvalid;
  if (B < 1 || T < 1 || (long)B * T > (1L << 24)) return kErrInvalid;
  if (!aligned16(q_nope) || !aligned16(wkv_b) || !aligned16(q_abs)) return kErrMisaligned;
  return dsa::launch_q_absorb(q_nope, wkv_b, B * T, q_abs, stream);
}

DSA_EXPORT int dsa_out_proj(const void* x, const void* wkv_b, int32_t B, int32_t T, void* y,
                            hipStream_t stream) {
  if (!x || !wkv_b || !y) return kErrInvalid;
  if (B < 1 || T < 1 || (long)B * T > (1L << 24)) return kErrInvalid;
  if (!aligned16(x) || !aligned16(wkv_b) || !aligned16(y)) return kErrMisaligned;
  return dsa::launch_out_proj(x, wkv_b, B * T, y, stream);
}

DSA_EXPORT int dsa_indexer_prep(const void* q_in, const void* k_in, const float* rope_cos,
                                const float* rope_sin, const int32_t* end_pos, int32_t B,
                                int32_t T, int32_t S_max, int32_t dtype, void* q_out,
                                float* q_scale, void* k_cache, float* k_scale,
                                hipStream_t stream) {
  if (!q_in || !k_in || !rope_cos || !rope_sin || !end_pos || !q_out || !k_cache)
    return kErrInvalid;
  if (B < 1 || T < 1 || S_max < T || (long)B * T > (1L << 24)) return kErrInvalid;
  if (!positions_ok(S_max)) return kErrUnsupported;
  if (dtype != 0 && dtype != 1) return kErrUnsupported;
  if (dtype == 1 && (!q_scale || !k_scale)) return kErrInvalid;
  if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(rope_cos) || !aligned16(rope_sin) ||
      !aligned4(end_pos) || !aligned16(q_out) || !aligned16(k_cache))
    return kErrMisaligned;
  if (dtype == 1 && (!aligned4(q_scale) || !aligned4(k_scale))) return kErrMisaligned;
  return dsa::launch_indexer_prep(q_in, k_in, rope_cos, rope_sin, end_pos, B, T, S_max, dtype,
                                  q_out, dtype == 1 ? q_scale : nullptr, k_cache,
                                  dtype == 1 ? k_scale : nullptr, stream);
}

DSA_EXPORT size_t dsa_sparse_mha_prefill_workspace_size(int32_t B, int32_t T) {
  if (B < 1 || T < 1 || (long)B * T > (1L << 24)) return 0;
  return dsa::mha_prefill_workspace_bytes(B, T);
}

DSA_EXPORT int dsa_sparse_mha_prefill(const void* q, const void* k_nope, const void* k_pe,
                                      const void* v, const int32_t* topk_indices, int32_t B,
                                      int32_t T, int32_t k, float softmax_scale, void* out,
                                      float* lse, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  if (!q || !k_nope || !k_pe || !v || !topk_indices || !out) return kErrInvalid;
  if (B < 1 || T < 1 || k < 1 || (long)B * T > (1L << 24)) return kErrInvalid;
  if (!good_softmax_scale(softmax_scale)) return kErrInvalid;
  if (!aligned16(q) || !aligned16(k_nope) || !aligned16(k_pe) || !aligned16(v) ||
      !aligned4(topk_indices) || !aligned16(out) || (lse && !aligned4(lse)))
    return kErrMisaligned;
  int st = check_workspace(workspace, workspace_bytes, dsa::mha_prefill_workspace_bytes(B, T));
  if (st) return st;
  return dsa::launch_mha_prefill(q, k_nope, k_pe, v, topk_indices, B, T, k, softmax_scale, out,
                                 lse, workspace, stream);
}
