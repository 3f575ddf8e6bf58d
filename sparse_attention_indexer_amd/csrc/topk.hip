// Per-query top-k selection on gfx950 (topk(min(index_topk, end_pos)) of
// Indexer.forward, "DeepSeek-V3.2-Exp - Keep top-k positions").
//
// Integer-only radix select.  Each score becomes an order-preserving 32-bit
// key (score_key: -0 folded into +0, sign-magnitude flipped so unsigned order
// equals float order).  Three histogram passes over the row (11, 11, 10 key
// bits, most significant first) narrow down the key T of the k-th largest
// element and how many of the elements equal to T are kept (need_eq).  A last
// pass walks the row in index order and writes, in ascending position order,
// every element with key > T and the first need_eq elements with key == T:
// ties go to the smaller position.  The output is unique, so it can be
// compared bit for bit.
//
// One 1024-thread workgroup per query row.  Rows of up to kLdsKeys positions
// keep their keys in LDS after the first pass (128 KiB of gfx950's 160 KiB);
// longer rows are re-read from global memory (L2) on each pass.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kLdsKeys = 32768;
constexpr int kMaxBins = 2048;

// Exclusive prefix sum over the block of one value per thread; also returns the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave,
                                                        uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  uint32_t before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const uint32_t c = s_wave[w];
    before += (w < wave) ? c : 0u;
    sum += c;
  }
  __syncthreads();
  total = sum;
  return before + incl - v;
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ end_pos,
                                                          int T, int S_max, int k,
                                                          int32_t* __restrict__ out) {
  __shared__ uint32_t s_keys[kLdsKeys];
  __shared__ uint32_t s_hist[kMaxBins];
  __shared__ uint32_t s_wave[kTkWaves];
  __shared__ uint32_t s_cnt[2][kTkWaves];
  __shared__ uint32_t s_sel[2];

  const int row = blockIdx.x;
  const int b = row / T, t = row - b * T;
  const int ep = min(max(end_pos[b], T), S_max);
  const int n = ep - T + t + 1;  // valid positions 0..n-1
  const float* x = scores + (size_t)row * S_max;
  int32_t* o = out + (size_t)row * k;
  const int tid = threadIdx.x;

  if (n <= k) {  // every valid position is kept
    for (int i = tid; i < k; i += kTkThreads) o[i] = i < n ? i : -1;
    return;
  }
  const bool in_lds = n <= kLdsKeys;

  // ---- radix passes: find the threshold key and how many ties to keep ----
  uint32_t prefix = 0, prefix_mask = 0, remaining = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < nbins; i += kTkThreads) s_hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTkThreads) {
      uint32_t key;
      if (pass == 0) {
        key = score_key(x[i]);
        if (in_lds) s_keys[i] = key;
      } else {
        key = in_lds ? s_keys[i] : score_key(x[i]);
      }
      if ((key & prefix_mask) == prefix) atomicAdd(&s_hist[(key >> shift) & (nbins - 1)], 1u);
    }
    __syncthreads();
    // Scan the bins from the top: thread tid owns reversed bins 2*tid, 2*tid+1.
    const int r0 = 2 * tid, r1 = 2 * tid + 1;
    const uint32_t c0 = r0 < nbins ? s_hist[nbins - 1 - r0] : 0u;
    const uint32_t c1 = r1 < nbins ? s_hist[nbins - 1 - r1] : 0u;
    uint32_t total;
    const uint32_t above0 = block_exclusive_scan(c0 + c1, s_wave, total);
    const uint32_t above1 = above0 + c0;
    // The unique bin whose elements straddle the remaining count.
    if (r0 < nbins && above0 < remaining && remaining <= above0 + c0) {
      s_sel[0] = (uint32_t)(nbins - 1 - r0);
      s_sel[1] = above0;
    }
    if (r1 < nbins && above1 < remaining && remaining <= above1 + c1) {
      s_sel[0] = (uint32_t)(nbins - 1 - r1);
      s_sel[1] = above1;
    }
    __syncthreads();
    const uint32_t digit = s_sel[0];
    remaining -= s_sel[1];
    prefix |= digit << shift;
    prefix_mask |= (uint32_t)(nbins - 1) << shift;
    __syncthreads();
  }
  const uint32_t thr = prefix;        // key of the k-th largest element
  const uint32_t need_eq = remaining;  // elements equal to thr that are kept

  // ---- ordered compaction: ascending positions, ties to the smaller position ----
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t run_gt = 0, run_eq = 0;
#pragma unroll 1
  for (int base = 0; base < n; base += kTkThreads) {
    const int i = base + tid;
    uint32_t key = 0;
    if (i < n) key = in_lds ? s_keys[i] : score_key(x[i]);
    const bool gt = i < n && key > thr;
    const bool eq = i < n && key == thr;
    const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
    if (lane == 0) {
      s_cnt[0][wave] = (uint32_t)__popcll(mgt);
      s_cnt[1][wave] = (uint32_t)__popcll(meq);
    }
    __syncthreads();
    uint32_t off_gt = 0, off_eq = 0, tot_gt = 0, tot_eq = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      const uint32_t a = s_cnt[0][w], e = s_cnt[1][w];
      off_gt += (w < wave) ? a : 0u;
      off_eq += (w < wave) ? e : 0u;
      tot_gt += a;
      tot_eq += e;
    }
    const uint32_t gt_before = run_gt + off_gt + (uint32_t)__popcll(mgt & lt_mask);
    const uint32_t eq_before = run_eq + off_eq + (uint32_t)__popcll(meq & lt_mask);
    // Positions are distinct and below k by construction; the bound check only
    // keeps a wrong threshold from ever writing outside the row.
    const uint32_t pos = gt ? gt_before + min(eq_before, need_eq) : gt_before + eq_before;
    if ((gt || (eq && eq_before < need_eq)) && pos < (uint32_t)k) o[pos] = i;
    run_gt += tot_gt;
    run_eq += tot_eq;
    __syncthreads();
  }
}

size_t topk_workspace_bytes(int, int, int, int) { return 0; }

int launch_topk(const float* scores, const int32_t* end_pos, int B, int T, int S_max, int,
                int k, int32_t* out, void*, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((long)B * T)), dim3(kTkThreads), 0, stream,
                     scores, end_pos, T, S_max, k, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace dsa
