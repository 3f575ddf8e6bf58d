// Host-side launchers of the libdsa kernels (one per .hip file).  Arguments
// are assumed validated by the C ABI layer; each returns 0 or -5 (launch
// failure) and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// With topk_ctr != nullptr the indexer also clears the top-k's per-row
// counters (the first 2 of 4 words per row, see topk_counters), so that launch_topk can run
// with counters_clear = true and skip its own clearing kernel.
int launch_index_scores(const void* q, const float* q_scale, const float* w, const void* k,
                        const float* k_scale, const int32_t* end_pos, int B, int T, int S_max,
                        int max_end_pos, float scale, int dtype, float* out, uint32_t* topk_ctr,
                        hipStream_t stream);

size_t topk_workspace_bytes(int B, int T, int S_max, int k);
// The per-row counters at the start of the top-k workspace, or nullptr when
// B*T rows of at most max_end_pos positions take a path without them.
uint32_t* topk_counters(void* workspace, int B, int T, int max_end_pos);
int launch_topk(const float* scores, const int32_t* end_pos, int B, int T, int S_max,
                int max_end_pos, int k, int32_t* out, void* workspace, bool counters_clear,
                hipStream_t stream);

// Split plan of the attention kernel: rows per split and number of splits.
struct MlaPlan {
  int rows_per_split;
  int n_splits;
  int waves;  // 4 (the tile form: 32 heads, one 64-row tile per block) or 8 (all 128 heads)
  bool tile = false;  // the 4-wave, 32-head form with one 64-row tile per block
};
MlaPlan sparse_mla_plan(int B, int T, int k);
MlaPlan dense_mla_plan(int B, int T, int S_max, int max_end_pos);
size_t mla_workspace_bytes(int B, int T, const MlaPlan& plan);

// prefix_end_pos: NULL, or the end positions when idx comes from the top-k
// selection (kept positions in the first min(k, causal bound) slots, -1
// after): the kernels then skip the empty tail of each list.
int launch_sparse_mla(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                      const int32_t* idx, int B, int T, int S_max, int k, float softmax_scale,
                      void* out, float* lse, void* workspace, hipStream_t stream,
                      const int32_t* prefix_end_pos = nullptr);
int launch_dense_mla(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                     const int32_t* end_pos, int B, int T, int S_max, int max_end_pos,
                     float softmax_scale, void* out, float* lse, void* workspace,
                     hipStream_t stream);

// Head-batched products around the absorbed attention (rows = B*T).
int launch_q_absorb(const void* q_nope, const void* wkv_b, int rows, void* q_abs,
                    hipStream_t stream);
int launch_out_proj(const void* x, const void* wkv_b, int rows, void* y, hipStream_t stream);
// MHA-form prefill attention over per-head keys/values with a selection
// bitmap built in the workspace.
size_t mha_prefill_workspace_bytes(int B, int T);
int launch_mha_prefill(const void* q, const void* k_nope, const void* k_pe, const void* v,
                       const int32_t* idx, int B, int T, int k, float softmax_scale, void* out,
                       float* lse, void* workspace, hipStream_t stream);
// Indexer input preparation (RoPE, Hadamard rotation, fp8 block quantisation or
// bf16 rounding, key append); dtype 0 = bf16, 1 = fp8.
int launch_indexer_prep(const void* q_in, const void* k_in, const float* rope_cos,
                        const float* rope_sin, const int32_t* end_pos, int B, int T, int S_max,
                        int dtype, void* q_out, float* q_scale, void* k_cache, float* k_scale,
                        hipStream_t stream);

}  // namespace dsa
