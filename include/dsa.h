/*
 * dsa.h - C ABI of libdsa.so: the DeepSeek Sparse Attention (DSA) decode hot
 * path on AMD Instinct MI355X (gfx950).
 *
 * The path has three stages, each a HIP kernel:
 *   (a) lightning-indexer scores  I[b,t,s] = scale * sum_h w[b,t,h] *
 *       ReLU(q[b,t,h,:] . k[b,s,:]) over 64 heads x 128 dims, for the
 *       causally valid positions (dsa_index_scores);
 *   (b) per-query selection of the top-k positions by that score
 *       (dsa_topk);
 *   (c) absorbed-MLA attention over only the selected cached rows: 128
 *       heads, 512-wide latent plus 64-wide rope part, softmax, 512-wide
 *       latent output (dsa_sparse_mla).
 * dsa_forward runs (a)->(b)->(c) on one stream; dsa_dense_mla is (c) over
 * every valid position (the dense baseline).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are DEVICE pointers to row-major, contiguous arrays with the
 *   shapes given below, 16-byte aligned, owned by the caller.  The library
 *   never allocates, frees or synchronises; every launch is enqueued on
 *   `stream` (NULL = the null stream) and the pointers must stay valid until
 *   that work has completed.  Intermediates live in a caller-provided
 *   workspace whose size the matching *_workspace_size function returns.
 * - Sequence b holds T new queries; query t sits at position
 *   end_pos[b] - T + t and may attend to cached positions
 *   0 .. end_pos[b] - T + t (its causal bound).  end_pos lives on the
 *   device, so the host cannot check it: the caller guarantees
 *   T <= end_pos[b] <= max_end_pos <= S_max.  Kernels clamp every position
 *   to [0, S_max) and never read out of bounds, whatever end_pos holds.
 * - bf16 is bfloat16; fp8 is OCP FP8 E4M3 ("e4m3fn", max 448), the native
 *   fp8 of gfx950.
 * - A call covers at most 2^24 query rows (B*T) and caches of at most 2^28
 *   positions (S_max); more give DSA_ERR_UNSUPPORTED, and the
 *   *_workspace_size functions return 0 for them (as for non-positive
 *   sizes).
 * - Every call returns DSA_OK (0) or a negative status.  Arguments are
 *   validated on the host before anything is launched; on failure nothing
 *   is enqueued.  DSA_ERR_HIP reports a failed launch (hipGetLastError).
 *   Calls are re-entrant and thread-safe; the one global state is the
 *   per-device scratch of dsa_forward_noalloc (the captured step of
 *   dsa_forward_graph_create is an object the caller owns).
 *
 * Sources of the definitions (web pages on DeepSeek-V3.2's sparse
 * attention): the indexer score and its output shape follow kernelpool's
 * fix in "mlx-lm PR #512 [WIP] deepseek v32" (ReLU of each head's dot, then
 * the head weight, then the sum over heads, no head dimension in the
 * output) and the Indexer.forward excerpt on "DeepSeek-V3.2-Exp - Keep top-k
 * positions" (fp8_index(q, weights, k_cache, k_scale), causal mask, then
 * topk(min(index_topk, end_pos))); the attention follows the MQA decode
 * excerpt on "DeepSeek-V3.2-Exp - Apply sparse mask" (absorbed query,
 * latent+rope scores times softmax_scale, index mask, softmax, latent-
 * weighted sum).  Sizes: 64 indexer heads x 128 dims and top-2048 from the
 * config list of "MaxText PR #2933"; 128 heads x (512+64) from the cost
 * model in "llama.cpp discussion #17692".
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle (identical to the typedef in hip_runtime_api.h). */
typedef struct ihipStream_t* hipStream_t;

enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = -1,   /* null pointer, non-positive or inconsistent size */
  DSA_ERR_UNSUPPORTED = -2,        /* dtype or shape outside the compiled specialisation */
  DSA_ERR_MISALIGNED = -3,         /* a tensor pointer is not 16-byte aligned */
  DSA_ERR_WORKSPACE_TOO_SMALL = -4,
  DSA_ERR_HIP = -5                 /* a kernel launch failed */
};

typedef enum { DSA_BF16 = 0, DSA_FP8_E4M3 = 1 } dsa_dtype;

/* Fixed sizes of this specialisation. */
#define DSA_INDEX_HEADS 64
#define DSA_INDEX_DIM 128
#define DSA_MLA_HEADS 128
#define DSA_LATENT_DIM 512
#define DSA_ROPE_DIM 64
#define DSA_MAX_TOPK 2048

/* Human-readable text for a status code (static storage, never NULL). */
const char* dsa_status_string(int status);

/* (a) Indexer scores - the fp8_index(q, weights, k_cache, k_scale) call of
 * Indexer.forward ("DeepSeek-V3.2-Exp - Keep top-k positions"), with the
 * ReLU -> weight -> head-sum order of "mlx-lm PR #512":
 *   I[b,t,s] = scale * sum_{h<64} w'[b,t,h] * ReLU(q[b,t,h,:] . k[b,s,:]) * ks[b,s]
 * with w' = w and ks = 1 for bf16, and w' = w*q_scale, ks = k_scale for fp8
 * (the scales are positive, so this equals the score of the dequantised
 * values code*scale).
 *   q        [B,T,64,128] bf16 or fp8 codes
 *   q_scale  [B,T,64] fp32, one scale per 128-element head block (fp8 only, else NULL)
 *   weights  [B,T,64] fp32 per-head weights (the caller folds in any
 *            n_heads^-0.5 / softmax-scale factors)
 *   k_cache  [B,S_max,128] bf16 or fp8 codes (one shared key per cached token)
 *   k_scale  [B,S_max] fp32, one scale per key (fp8 only, else NULL)
 *   end_pos  [B] int32 (device)
 *   scale    applied once, after the head sum
 *   index_score [B,T,S_max] fp32 out; entries past each query's causal
 *            bound are left untouched.
 * Arithmetic: products on MFMA with fp32 accumulation; ReLU, weighting,
 * head sum and scaling in fp32.  1 <= T <= max_end_pos <= S_max. */
int dsa_index_scores(const void* q, const float* q_scale, const float* weights,
                     const void* k_cache, const float* k_scale, const int32_t* end_pos,
                     int32_t B, int32_t T, int32_t S_max, int32_t max_end_pos, float scale,
                     int32_t dtype, float* index_score, hipStream_t stream);

/* (b) Top-k selection - topk(min(index_topk, end_pos)) after the causal mask
 * in Indexer.forward ("DeepSeek-V3.2-Exp - Keep top-k positions").
 * For each query row the k_eff = min(k, bound+1) positions with the largest
 * score are kept; equal scores (IEEE equality, so -0 == +0) go to the
 * smaller position.  Output: topk_indices [B,T,k] int32 with the kept
 * positions in ASCENDING order followed by -1 in the k - k_eff empty slots.
 * Scores must not be NaN (the order of NaN is unspecified).
 * Integer-only selection (order-preserving 32-bit keys): the result is
 * exact.  1 <= k <= 2048.
 * Workspace: dsa_topk_workspace_size bytes, 256-byte aligned (0 bytes, and
 * NULL allowed, when B*T > 1024; otherwise just over 64 KiB per row when
 * S_max <= 4096 and just over 384 KiB per row above that: 16 candidate
 * regions of 3072 (key, position) pairs each).  It holds the per-row candidate lists of
 * one call; its contents on entry do not matter (the call clears whatever it
 * needs cleared) and are unspecified afterwards.  Calls that overlap in time
 * must not share a workspace. */
size_t dsa_topk_workspace_size(int32_t B, int32_t T, int32_t S_max, int32_t k);
int dsa_topk(const float* index_score, const int32_t* end_pos, int32_t B, int32_t T,
             int32_t S_max, int32_t max_end_pos, int32_t k, int32_t* topk_indices,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* (c) Sparse absorbed-MLA attention - the MQA decode branch of
 * "DeepSeek-V3.2-Exp - Apply sparse mask", restricted to the selected rows:
 *   z[h,j] = (q_nope[h,:] . kv[idx_j,:] + q_pe[h,:] . pe[idx_j,:]) * softmax_scale
 *   p = softmax_j(z),  out[h,:] = sum_j p[h,j] * kv[idx_j,:]
 * over the valid entries idx_j of the query's index row (entries that are
 * negative or >= S_max are empty slots and are skipped; valid entries must
 * be distinct).  The 512-wide latent is both key and value; the query has
 * already been absorbed into the latent space.
 *   q_nope   [B,T,128,512] bf16     q_pe     [B,T,128,64] bf16
 *   kv_cache [B,S_max,512] bf16     pe_cache [B,S_max,64] bf16
 *   topk_indices [B,T,k] int32 (as produced by dsa_topk)
 *   out      [B,T,128,512] bf16 (fp32 accumulation, rounded to nearest even)
 *   lse      [B,T,128] fp32 natural-log sum of exp(z) over the kept rows, or NULL
 * A row with no valid entry produces out = 0 and lse = -inf.  softmax_scale
 * must be positive and finite (else DSA_ERR_INVALID_ARGUMENT); this holds for
 * dsa_dense_mla and dsa_forward too.
 * Arithmetic: both contractions on bf16 MFMA with fp32 accumulation, fp32
 * online softmax; the probabilities enter the value contraction as bf16. */
size_t dsa_sparse_mla_workspace_size(int32_t B, int32_t T, int32_t k);
int dsa_sparse_mla(const void* q_nope, const void* q_pe, const void* kv_cache,
                   const void* pe_cache, const int32_t* topk_indices, int32_t B, int32_t T,
                   int32_t S_max, int32_t k, float softmax_scale, void* out, float* lse,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* (a)+(b)+(c) on one stream: the decode step of "DeepSeek-V3.2-Exp - Apply
 * sparse mask" with the indexer of "Keep top-k positions".  Arguments are
 * those of the three calls; index_score, the indices, the top-k lists and
 * the attention's split partials live in the workspace, whose contents on
 * entry do not matter.  topk_indices_out [B,T,k] receives the selection if
 * not NULL.  When every query has at most k valid positions every position
 * is kept, which equals dense attention (the short-context case). */
size_t dsa_forward_workspace_size(int32_t B, int32_t T, int32_t S_max, int32_t k);
int dsa_forward(const void* q, const float* q_scale, const float* weights, const void* k_cache,
                const float* k_scale, const int32_t* end_pos, const void* q_nope,
                const void* q_pe, const void* kv_cache, const void* pe_cache, int32_t B,
                int32_t T, int32_t S_max, int32_t max_end_pos, int32_t k, float index_scale,
                float softmax_scale, int32_t dtype, void* out, float* lse,
                int32_t* topk_indices_out, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/* dsa_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, which lives instead in a device
 * array held by the library, DSA_FORWARD_SCRATCH_BYTES on every GPU it runs
 * on, from the library's load until the process ends.  Returns
 * DSA_ERR_WORKSPACE_TOO_SMALL, launching nothing, when
 * dsa_forward_workspace_size(B, T, S_max, k) exceeds that (96 MiB holds batch
 * 64 at 131072 positions, or one 4096-query prefill); the other errors are
 * dsa_forward's.  The call makes no allocation of any kind.  The current
 * device must be the one `stream` runs on; the array's address on it is
 * looked up on the first call there (DSA_ERR_HIP if that fails).  Every call
 * on one GPU uses the same array and nothing in it needs clearing: calls that
 * overlap in time on one GPU (other streams, other host threads) race and
 * must be serialised by the caller. */
#define DSA_FORWARD_SCRATCH_BYTES ((size_t)96 << 20)
int dsa_forward_noalloc(const void* q, const float* q_scale, const float* weights,
                        const void* k_cache, const float* k_scale, const int32_t* end_pos,
                        const void* q_nope, const void* q_pe, const void* kv_cache,
                        const void* pe_cache, int32_t B, int32_t T, int32_t S_max,
                        int32_t max_end_pos, int32_t k, float index_scale, float softmax_scale,
                        int32_t dtype, void* out, float* lse, int32_t* topk_indices_out,
                        hipStream_t stream);

/* The decode step captured once and replayed: dsa_forward recorded into a
 * HIP graph for fixed tensors, sizes and workspace, so that a serving loop
 * pays one graph launch per step instead of one launch per kernel, and
 * rewrites the inputs in place between steps (new query, weights, end_pos,
 * appended cache rows).  The path needs no memset, no allocation and nothing
 * carried in the workspace from one step to the next, so every replay
 * computes exactly what a dsa_forward call on the buffers' current contents
 * would.  Callers: serving loops that replay one decode step per token.
 *   dsa_forward_graph_create  takes dsa_forward's arguments without the
 *       stream, validates them as dsa_forward does (nothing is created on
 *       failure, *graph = NULL), then captures the step on a private stream
 *       of the current device and instantiates it; DSA_ERR_HIP if capture or
 *       instantiation fails.  The tensors and workspace must outlive the
 *       graph; end_pos and max_end_pos keep their meaning for every replay.
 *   dsa_forward_graph_launch  enqueues one replay on `stream` (a stream of
 *       the same device); replays of one graph on different streams must not
 *       overlap in time (they share the workspace).
 *   dsa_forward_graph_destroy  releases the graph (NULL is a no-op); no
 *       replay may still be pending.
 * This is the one part of the library that creates runtime objects (a
 * stream during capture, the graph); it still allocates no device memory of
 * its own. */
typedef struct dsa_forward_graph* dsa_forward_graph_t;
int dsa_forward_graph_create(const void* q, const float* q_scale, const float* weights,
                             const void* k_cache, const float* k_scale, const int32_t* end_pos,
                             const void* q_nope, const void* q_pe, const void* kv_cache,
                             const void* pe_cache, int32_t B, int32_t T, int32_t S_max,
                             int32_t max_end_pos, int32_t k, float index_scale,
                             float softmax_scale, int32_t dtype, void* out, float* lse,
                             int32_t* topk_indices_out, void* workspace, size_t workspace_bytes,
                             dsa_forward_graph_t* graph);
int dsa_forward_graph_launch(dsa_forward_graph_t graph, hipStream_t stream);
int dsa_forward_graph_destroy(dsa_forward_graph_t graph);

/* Dense baseline: (c) over every causally valid position 0..bound, no index
 * list (the unmasked form of the same decode branch).  Same tensors and
 * arithmetic as dsa_sparse_mla.  Used to measure where sparse wins. */
size_t dsa_dense_mla_workspace_size(int32_t B, int32_t T, int32_t S_max);
int dsa_dense_mla(const void* q_nope, const void* q_pe, const void* kv_cache,
                  const void* pe_cache, const int32_t* end_pos, int32_t B, int32_t T,
                  int32_t S_max, int32_t max_end_pos, float softmax_scale, void* out, float* lse,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Query absorption and output up-projection: the two per-head products on
 * either side of (c) in the MQA decode branch of "DeepSeek-V3.2-Exp - Apply
 * sparse mask", with the key/value up-projection wkv_b viewed as
 * [128 heads, 128 + 128, 512] (its first 128 rows per head act on the query's
 * non-rope part, its last 128 = v_head_dim rows produce the head's output):
 *   dsa_q_absorb:  q_abs[b,t,h,c] = sum_{d<128} q_nope[b,t,h,d] * wkv_b[h,d,c]
 *   dsa_out_proj:  y[b,t,h,d]     = sum_{c<512} x[b,t,h,c] * wkv_b[h,128+d,c]
 *   q_nope [B,T,128,128] bf16   wkv_b [128,256,512] bf16 (dequantised weight)
 *   q_abs  [B,T,128,512] bf16   x [B,T,128,512] bf16 (the latent output of (c))
 *   y      [B,T,128,128] bf16
 * Arithmetic: bf16 MFMA with fp32 accumulation, rounded to nearest even.
 * No workspace; 1 <= B*T <= 2^24; pointers 16-byte aligned. */
int dsa_q_absorb(const void* q_nope, const void* wkv_b, int32_t B, int32_t T, void* q_abs,
                 hipStream_t stream);
int dsa_out_proj(const void* x, const void* wkv_b, int32_t B, int32_t T, void* y,
                 hipStream_t stream);

/* MHA-form prefill attention - the `mask is not None` branch of the attention
 * excerpt on "DeepSeek-V3.2-Exp - Keep top-k positions": keys and values
 * up-projected per head (by the caller), a head's key = its 128 non-rotary
 * dims followed by the 64 rotary dims shared by all heads, scores times
 * softmax_scale, plus the index mask (0 at the selected positions, -inf
 * elsewhere; a position listed twice counts once) and the causal mask,
 * softmax, weighted sum of the head's values.  B sequences of T tokens each,
 * token s at position s (a prefill from position 0); query s sees key t iff t
 * is in s's list and t <= s.
 *   q      [B,T,128,192] bf16 (non-rotary 128 dims, then rotary 64)
 *   k_nope [B,T,128,128] bf16   k_pe [B,T,64] bf16   v [B,T,128,128] bf16
 *   topk_indices [B,T,k] int32: entries outside 0..T-1 select nothing
 *   out    [B,T,128,128] bf16 (fp32 accumulation, round to nearest even)
 *   lse    [B,T,128] fp32 natural-log sum of exp(z) over the kept keys, or NULL
 * A query that keeps no key gets out = 0 and lse = -inf.  The workspace holds
 * the selection as a bitmap (B * ceil(T/32) * roundup(T,256) words).
 * Arithmetic: bf16 MFMA with fp32 accumulation, fp32 online softmax, the
 * probabilities enter the value product as bf16.  1 <= B*T <= 2^24;
 * softmax_scale positive and finite. */
size_t dsa_sparse_mha_prefill_workspace_size(int32_t B, int32_t T);
int dsa_sparse_mha_prefill(const void* q, const void* k_nope, const void* k_pe, const void* v,
                           const int32_t* topk_indices, int32_t B, int32_t T, int32_t k,
                           float softmax_scale, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Indexer input preparation - the weight-free steps of the Indexer.forward
 * excerpt on "DeepSeek-V3.2-Exp - Keep top-k positions" between the
 * projections (wq_b, wk + k_norm) and fp8_index: RoPE on the first 64 dims of
 * every query head and of the key, in the concatenated layout that "MaxText
 * PR #2933" gives for the indexer (dim i and dim i+32, i < 32, are the two
 * parts of one pair turned by the angle of frequency i); the rotation
 * rotate_activation, read as the orthonormal Walsh-Hadamard transform
 * (Sylvester order, 128^-1/2); then, for fp8, act_quant with 128-element
 * blocks (scale = max|x| / 448, codes = nearest e4m3 of x / scale, ties to
 * even) and, for either dtype, the key written at its position.
 *   q_in  [B,T,64,128] bf16 (rope dims first)   k_in [B,T,128] bf16
 *   rope_cos, rope_sin [S_max,32] fp32: cos and sin of the pair angles at each
 *         absolute position; token t of sequence b uses row end_pos[b]-T+t
 *   end_pos [B] int32 (device), T <= end_pos[b] <= S_max
 *   dtype DSA_FP8_E4M3: q_out [B,T,64,128] fp8 codes, q_scale [B,T,64] fp32,
 *         k_cache [B,S_max,128] fp8 and k_scale [B,S_max] fp32 get row
 *         end_pos[b]-T+t of each token -- the inputs of dsa_index_scores.
 *   dtype DSA_BF16: q_out / k_cache get the rotated values rounded to bf16;
 *         q_scale and k_scale are ignored (may be NULL).
 * Other cache rows are not touched.  Arithmetic in fp32 (the rotation's sums
 * unscaled, the 128^-1/2 folded into the scale), IEEE divisions for the
 * scale and the codes; an all-zero block gets scale 0 and zero codes.  A
 * token whose position falls outside [0, S_max) (end_pos out of contract)
 * writes no key.  No workspace; 1 <= B*T <= 2^24; tensors 16-byte aligned,
 * scales 4-byte aligned. */
int dsa_indexer_prep(const void* q_in, const void* k_in, const float* rope_cos,
                     const float* rope_sin, const int32_t* end_pos, int32_t B, int32_t T,
                     int32_t S_max, int32_t dtype, void* q_out, float* q_scale, void* k_cache,
                     float* k_scale, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
