// Per-query top-k selection on gfx950 (topk(min(index_topk, end_pos)) of
// Indexer.forward, "DeepSeek-V3.2-Exp - Keep top-k positions").
//
// Integer-only radix select.  Each score becomes an order-preserving 32-bit
// key (score_key: -0 folded into +0, sign-magnitude flipped so unsigned order
// equals float order).  Histogram rounds over the key bits (11, 11, 10, most
// significant first) find the key `thr` of the k-th largest element and how
// many elements equal to thr are kept (need_eq).  The output is every
// position with key > thr plus the first need_eq positions with key == thr,
// in ascending position order, so ties go to the smaller position and the
// result is unique.
//
// Three ways to run it, chosen on the host:
//  * rows of at most 32768 positions: topk_lean_kernel, one 512-thread
//    workgroup per row holding the whole row in registers (no workspace);
//  * longer rows, up to 1024 of them: the row is spread over many workgroups
//    (topk_hist_kernel, topk_classify_kernel) and a last one per row
//    finishes the selection (topk_final_kernel);
//  * more rows than that: full_row_topk, one workgroup per row, chunk by
//    chunk (topk_row_kernel).
// The first two build bitmaps of the certain winners and of the ties and read
// the ordered output off them; full_row_topk (also their fallback for rows
// whose candidate set is too crowded) compacts keys held in LDS.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kSeg = 64;                   // positions per thread per chunk
constexpr int kChunk = kTkThreads * kSeg;  // 32768 positions per chunk
constexpr int kBins = 2048;
constexpr int kCandCap = 4096;             // candidate keys
constexpr int kHistWords = kBins + kBins / 32;

// Histogram bins are stored with one pad word per 32 so that a lane reading
// 32 consecutive bins (the bin search) does not collide with other lanes.
__device__ __forceinline__ int hpad(uint32_t bin) { return (int)(bin + (bin >> 5)); }

// Word of element j of segment t in the LDS chunk: 16-byte group j/4 is
// XOR-swizzled with the low bits of t, so lanes reading the same group of
// consecutive segments hit different 4-bank sets.
__device__ __forceinline__ int swz(int t, int j) {
  return kSeg * t + 4 * ((j >> 2) ^ (t & (kSeg / 4 - 1))) + (j & 3);
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  return v;
}

// Exclusive prefix sums over the block of two per-thread values, plus totals.
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t* s_wave,
                                                      uint32_t& ex_a, uint32_t& ex_b,
                                                      uint32_t& tot_a, uint32_t& tot_b) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) {
    s_wave[wave] = ia;
    s_wave[kTkWaves + wave] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w4 = 0; w4 < kTkWaves; w4 += 4) {
    const uint4 wa = *reinterpret_cast<const uint4*>(s_wave + w4);
    const uint4 wb = *reinterpret_cast<const uint4*>(s_wave + kTkWaves + w4);
    const uint32_t va[4] = {wa.x, wa.y, wa.z, wa.w}, vb[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pa += (w4 + u < wave) ? va[u] : 0u;
      pb += (w4 + u < wave) ? vb[u] : 0u;
      sa += va[u];
      sb += vb[u];
    }
  }
  __syncthreads();
  ex_a = pa + ia - a;
  ex_b = pb + ib - b;
  tot_a = sa;
  tot_b = sb;
}

// Keys of chunk positions [base, base+len): coalesced global loads -> keys ->
// LDS (swizzled).  With hist != nullptr the top 11 bits of every valid key are
// counted on the way.  Returns how many positions of this thread's segment are
// valid.  Ends with the block synchronised.
__device__ __forceinline__ int load_chunk(const float* __restrict__ x, int base, int len,
                                          uint32_t* s_keys, uint32_t* hist) {
  const int t = threadIdx.x;
  // Unconditional loads (index clamped into the chunk), 32 in flight at a
  // time; positions past len are never counted or selected.
  __syncthreads();  // the previous chunk's LDS copy is no longer read
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float v[kSeg / 2];
#pragma unroll
    for (int j = 0; j < kSeg / 2; ++j)
      v[j] = x[base + min(t + kTkThreads * (half * (kSeg / 2) + j), len - 1)];
#pragma unroll
    for (int j = 0; j < kSeg / 2; ++j) {
      const int i = t + kTkThreads * (half * (kSeg / 2) + j);
      const uint32_t key = score_key(v[j]);
      s_keys[swz(i / kSeg, i % kSeg)] = key;
      if (hist != nullptr) atomicAdd(&hist[hpad(key >> 21)], i < len ? 1u : 0u);
    }
  }
  __syncthreads();
  const int nv = len - kSeg * t;
  return nv < 0 ? 0 : (nv > kSeg ? kSeg : nv);
}

// 16 consecutive keys (batch bt) of this thread's segment from the LDS copy.
__device__ __forceinline__ void read_batch(const uint32_t* s_keys, int bt, uint32_t (&kb)[16]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint4 q4 = *reinterpret_cast<const uint4*>(s_keys + swz(t, 16 * bt + 4 * c));
    kb[4 * c] = q4.x;
    kb[4 * c + 1] = q4.y;
    kb[4 * c + 2] = q4.z;
    kb[4 * c + 3] = q4.w;
  }
}

// One wave finds the bin holding the `remaining`-th largest counted element
// (counting from the top bin down): returns its digit and the count of
// elements in higher bins.  Lane l owns the 32 (or 16) bins just below the
// bins of lane l-1.
template <bool kPadded = true>
__device__ __forceinline__ void wave_select_bin(const uint32_t* hist, int nbins,
                                                uint32_t remaining, uint32_t& digit,
                                                uint32_t& above_out) {
  const int lane = threadIdx.x & 63;
  const int per = nbins / kWave;  // 32 or 16
  uint32_t c[32];
  uint32_t sum = 0;
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    // Unconditional (clamped) read, masked afterwards: no branch per bin.
    const int bin = max(nbins - 1 - (lane * per + u), 0);
    const uint32_t v = hist[kPadded ? hpad((uint32_t)bin) : bin];
    c[u] = u < per ? v : 0u;
    sum += c[u];
  }
  const uint32_t incl = wave_incl_scan(sum);
  uint32_t above = incl - sum;
  uint32_t my_digit = 0, my_above = 0;
  bool found = false;
#pragma unroll
  for (int u = 0; u < 32; ++u) {
    if (u < per && above < remaining && remaining <= above + c[u]) {
      my_digit = (uint32_t)(nbins - 1 - (lane * per + u));
      my_above = above;
      found = true;
    }
    above += c[u];
  }
  const uint64_t who = __ballot(found);
  const int src = __ffsll((long long)who) - 1;
  digit = __shfl(my_digit, src, 64);
  above_out = __shfl(my_above, src, 64);
}

// Block-wide version: wave 0 searches, everyone receives the result.
__device__ __forceinline__ uint32_t select_bin(const uint32_t* hist, int nbins,
                                               uint32_t& remaining, uint32_t* s_sel) {
  __syncthreads();  // histogram complete
  if (threadIdx.x < kWave) {
    uint32_t digit, above;
    wave_select_bin(hist, nbins, remaining, digit, above);
    if (threadIdx.x == 0) {
      s_sel[0] = digit;
      s_sel[1] = above;
    }
  }
  __syncthreads();
  const uint32_t digit = s_sel[0];
  remaining -= s_sel[1];
  return digit;
}

// Exact selection over a whole row, one workgroup (the general path, and the
// fallback of the candidate path below).  n > k.
struct TopkShared {
  uint32_t keys[kChunk];
  uint32_t hist[kHistWords];
  uint32_t cand[kCandCap];
  uint32_t wave[2 * kTkWaves];
  uint32_t sel[2];
  uint32_t ncand;
};

__device__ void full_row_topk(const float* __restrict__ x, int n, int k,
                              int32_t* __restrict__ o, TopkShared& sh) {
  uint32_t* s_keys = sh.keys;
  uint32_t* s_hist = sh.hist;
  uint32_t* s_cand = sh.cand;
  uint32_t* s_wave = sh.wave;
  uint32_t* s_sel = sh.sel;
  uint32_t& s_ncand = sh.ncand;
  const int tid = threadIdx.x;

  const int n_chunks = (n + kChunk - 1) / kChunk;
  const bool resident = n_chunks == 1;
  int nv = 0;

  // ---- round 1: histogram of the top 11 key bits, counted while loading ----
  for (int i = tid; i < kHistWords; i += kTkThreads) s_hist[i] = 0;
  if (tid == 0) s_ncand = 0;
#pragma unroll 1
  for (int c = 0; c < n_chunks; ++c)
    nv = load_chunk(x, c * kChunk, min(kChunk, n - c * kChunk), s_keys, s_hist);
  uint32_t remaining = (uint32_t)k;
  const uint32_t d0 = select_bin(s_hist, kBins, remaining, s_sel);
  const uint32_t bin_count = s_hist[hpad(d0)];
  const bool use_list = bin_count <= (uint32_t)kCandCap;

  // ---- candidates: the keys that fell into bin d0 ----
  if (use_list) {
#pragma unroll 1
    for (int c = 0; c < n_chunks; ++c) {
      if (!resident) nv = load_chunk(x, c * kChunk, min(kChunk, n - c * kChunk), s_keys, nullptr);
      uint64_t hits = 0;  // bit j: element j of the segment is a candidate
#pragma unroll 1
      for (int bt = 0; bt < kSeg / 16; ++bt) {
        uint32_t kb[16];
        read_batch(s_keys, bt, kb);
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 16; ++j) m |= ((kb[j] >> 21) == d0 ? 1u : 0u) << j;
        hits |= (uint64_t)m << (16 * bt);
      }
      hits &= nv >= kSeg ? ~0ull : ((1ull << nv) - 1);
      const uint32_t cnt = (uint32_t)__popcll(hits);
      // One LDS atomic per wave reserves the wave's slots.
      const uint32_t incl = wave_incl_scan(cnt);
      uint32_t base_slot = 0;
      if ((tid & 63) == 63 && incl > 0) base_slot = atomicAdd(&s_ncand, incl);
      base_slot = __shfl(base_slot, 63, 64);
      uint32_t slot = base_slot + incl - cnt;
      while (hits != 0) {
        const int j = __ffsll((long long)hits) - 1;
        hits &= hits - 1;
        if (slot < (uint32_t)kCandCap) s_cand[slot] = s_keys[swz(tid, j)];
        ++slot;
      }
    }
  }

  // ---- rounds 2 and 3: the next 11 bits, then the last 10 ----
  uint32_t prefix = d0 << 21, prefix_mask = 0xFFE00000u;
  if (use_list) {
    // The candidate list is small: wave 0 finishes the selection alone.
    __syncthreads();  // candidate list complete
    if (tid < kWave) {
#pragma unroll 1
      for (int round = 1; round < 3; ++round) {
        const int shift = round == 1 ? 10 : 0;
        const uint32_t nbins = round == 1 ? 2048u : 1024u;
        for (int i = tid; i < kHistWords; i += kWave) s_hist[i] = 0;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        for (int i0 = 0; i0 < (int)bin_count; i0 += 4 * kWave) {
          uint32_t key[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) key[u] = s_cand[min(i0 + u * kWave + tid, kCandCap - 1)];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            atomicAdd(&s_hist[hpad((key[u] >> shift) & (nbins - 1))],
                      (i0 + u * kWave + tid < (int)bin_count && (key[u] & prefix_mask) == prefix)
                          ? 1u : 0u);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        uint32_t digit, above;
        wave_select_bin(s_hist, (int)nbins, remaining, digit, above);
        remaining -= above;
        prefix |= digit << shift;
        prefix_mask |= (nbins - 1) << shift;
      }
      if (tid == 0) {
        s_sel[0] = prefix;
        s_sel[1] = remaining;
      }
    }
    __syncthreads();
    prefix = s_sel[0];
    remaining = s_sel[1];
  } else {
#pragma unroll 1
    for (int round = 1; round < 3; ++round) {
      const int shift = round == 1 ? 10 : 0;
      const uint32_t nbins = round == 1 ? 2048u : 1024u;
      __syncthreads();  // previous readers of s_hist are done
      for (int i = tid; i < kHistWords; i += kTkThreads) s_hist[i] = 0;
      __syncthreads();
#pragma unroll 1
      for (int c = 0; c < n_chunks; ++c) {
        if (!resident) nv = load_chunk(x, c * kChunk, min(kChunk, n - c * kChunk), s_keys, nullptr);
#pragma unroll 1
        for (int bt = 0; bt < kSeg / 16; ++bt) {
          uint32_t kb[16];
          read_batch(s_keys, bt, kb);
#pragma unroll
          for (int j = 0; j < 16; ++j)
            atomicAdd(&s_hist[hpad((kb[j] >> shift) & (nbins - 1))],
                      (16 * bt + j < nv && (kb[j] & prefix_mask) == prefix) ? 1u : 0u);
        }
      }
      const uint32_t digit = select_bin(s_hist, (int)nbins, remaining, s_sel);
      prefix |= digit << shift;
      prefix_mask |= (nbins - 1) << shift;
    }
  }
  const uint32_t thr = prefix;         // key of the k-th largest element
  const uint32_t need_eq = remaining;  // elements equal to thr that are kept

  // ---- ordered compaction: ascending positions, ties to the smaller position ----
  uint32_t run_gt = 0, run_eq = 0;
#pragma unroll 1
  for (int c = 0; c < n_chunks; ++c) {
    if (!resident) nv = load_chunk(x, c * kChunk, min(kChunk, n - c * kChunk), s_keys, nullptr);
    uint32_t n_gt = 0, n_eq = 0;
    uint64_t sel = 0;  // bit j: element j of the segment has key >= thr
#pragma unroll 1
    for (int bt = 0; bt < kSeg / 16; ++bt) {
      uint32_t kb[16];
      read_batch(s_keys, bt, kb);
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) m |= (kb[j] >= thr ? 1u : 0u) << j;
      sel |= (uint64_t)m << (16 * bt);
    }
    sel &= nv >= kSeg ? ~0ull : ((1ull << nv) - 1);
    // Elements equal to thr among the selected ones (rare: they are re-read).
    uint64_t rest = sel;
    while (rest != 0) {
      const int j = __ffsll((long long)rest) - 1;
      rest &= rest - 1;
      n_eq += s_keys[swz(tid, j)] == thr ? 1u : 0u;
    }
    n_gt = (uint32_t)__popcll(sel) - n_eq;
    uint32_t gt_before, eq_before, tot_gt, tot_eq;
    block_exclusive_scan2(n_gt, n_eq, s_wave, gt_before, eq_before, tot_gt, tot_eq);
    gt_before += run_gt;
    eq_before += run_eq;
    const int first = c * kChunk + kSeg * tid;
    while (sel != 0) {
      const int j = __ffsll((long long)sel) - 1;
      sel &= sel - 1;
      const uint32_t key = s_keys[swz(tid, j)];
      // Positions are distinct and below k by construction; the bound check
      // only keeps a wrong threshold from ever writing outside the row.
      if (key > thr) {
        const uint32_t pos = gt_before + min(eq_before, need_eq);
        if (pos < (uint32_t)k) o[pos] = first + j;
        ++gt_before;
      } else {
        if (eq_before < need_eq) {
          const uint32_t pos = gt_before + eq_before;
          if (pos < (uint32_t)k) o[pos] = first + j;
        }
        ++eq_before;
      }
    }
    run_gt += tot_gt;
    run_eq += tot_eq;
  }
}

// ---------------------------------------------------------------------------
// Candidate path.  A row is cut into blocks of kBlk positions processed by
// separate workgroups:
//   topk_hist_kernel  counts the top 11 key bits of each block into the row's
//                     histogram (LDS, then one global atomic per non-empty bin);
//   topk_cand_kernel  reads the histogram, takes the lower edge L of the bin
//                     holding the k-th largest key, and writes the (key,
//                     position) of every element >= L of its block, in
//                     position order, to the block's slot (or marks overflow);
//   topk_kernel       concatenates the slots (ascending positions), checks that
//                     they hold every element >= L and at least k of them, and
//                     then selects exactly among them.  Otherwise it falls back
//                     to full_row_topk.  It leaves the row's histogram zeroed.
// The histogram only chooses L: whatever it contains, the selection is exact
// (a candidate set holding every element >= L with at least k elements
// contains the top k).  A zero-filled workspace gets the fast path at once.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Few rows: the row is spread over many workgroups.
//   1. topk_hist_kernel: a histogram of the top 11 key bits per row (blocks of
//      2048 positions count in LDS and add their non-zero bins to the row's
//      histogram in the workspace); it also clears the row's candidate count.
//   2. topk_classify_kernel: every block finds the bin d0 holding the k-th
//      largest key from that histogram, then splits its positions into sure
//      winners (top 11 bits above d0: one ballot per 64 positions, stored as
//      a global bitmap) and candidates (in bin d0: appended, in any order, as
//      (key, position) pairs to the row's candidate list).
//   3. topk_final_kernel, one workgroup per row: loads the winner bitmap and
//      the candidates into LDS, runs rounds 2 and 3 over the candidates only,
//      adds those above the threshold to the winner bitmap and those equal to
//      it to a tie bitmap, and reads the ordered output off the two bitmaps
//      (winners, plus the first need_eq ties in position order).  It leaves
//      the histogram zeroed for the next call.
// The histogram only steers the work: the final kernel counts the winners S
// and candidates C itself and, unless S < k <= S + C (the k-th largest key is
// in bin d0) and the candidates fit, selects the row from scratch with
// full_row_topk.  Any workspace content thus gives the exact result.
// Many rows: full_row_topk, one workgroup per row (topk_row_kernel).
constexpr int kBlk = 2048;           // positions per histogram / classify block
constexpr int kBlkThreads = 256;     // 8 positions per thread
constexpr int kMultiRows = 1024;     // up to this many rows take the multi-block path
constexpr int kSelMaxN = 262144;     // longest row the final kernel's bitmaps cover
constexpr int kSelWords = kSelMaxN / 32;
constexpr int kSelCap = 8192;        // candidates per row

struct TopkWs {
  uint32_t* hist;   // [rows][kBins]
  uint32_t* ctr;    // [rows][2]: candidate count, bin d0
  uint64_t* win;    // [rows][n_blk * 32] winner bitmap, 64 positions a word
  uint2* cand;      // [rows][kSelCap] (key, position)
  int n_blk;        // blocks of kBlk positions per row (covering S_max)
};

__host__ __device__ inline int topk_blocks(int S_max) { return (S_max + kBlk - 1) / kBlk; }

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__host__ inline TopkWs carve_topk_ws(void* ws, int rows, int S_max) {
  TopkWs w;
  w.n_blk = topk_blocks(S_max);
  char* p = reinterpret_cast<char*>(ws);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * kBins * 4);
  w.ctr = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * 2 * 4);
  w.win = reinterpret_cast<uint64_t*>(p);
  p += align256((size_t)rows * w.n_blk * (kBlk / 8));
  w.cand = reinterpret_cast<uint2*>(p);
  return w;
}

size_t topk_workspace_bytes(int B, int T, int S_max, int) {
  const size_t rows = (size_t)B * T;
  // Rows that fit one workgroup's registers (max_end_pos <= S_max <= 32768),
  // or too many rows for the histogram path, need no workspace.
  if (S_max <= kChunk || rows > (size_t)kMultiRows) return 0;
  return align256(rows * kBins * 4) + align256(rows * 2 * 4) +
         align256(rows * topk_blocks(S_max) * (kBlk / 8)) + rows * kSelCap * 8;
}

__device__ __forceinline__ int row_len(const int32_t* end_pos, int row, int T, int S_max) {
  const int b = row / T, t = row - b * T;
  const int ep = min(max(end_pos[b], T), S_max);
  return ep - T + t + 1;
}

__global__ __launch_bounds__(kBlkThreads) void topk_hist_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, TopkWs ws) {
  __shared__ uint32_t s_h[kBins];
  const int row = blockIdx.x / ws.n_blk, blk = blockIdx.x - row * ws.n_blk;
  const int n = row_len(end_pos, row, T, S_max);
  const int base = blk * kBlk;
  if (n <= k || base >= n) return;
  const int len = min(kBlk, n - base);
  const float* x = scores + (size_t)row * S_max + base;
  const int tid = threadIdx.x;
  float v[kBlk / kBlkThreads];
#pragma unroll
  for (int j = 0; j < kBlk / kBlkThreads; ++j) v[j] = x[min(tid + kBlkThreads * j, len - 1)];
  for (int i = tid; i < kBins; i += kBlkThreads) s_h[i] = 0;
  if (blk == 0 && tid == 0) ws.ctr[2 * row] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kBlk / kBlkThreads; ++j)
    atomicAdd(&s_h[score_key(v[j]) >> 21], tid + kBlkThreads * j < len ? 1u : 0u);
  __syncthreads();
  uint32_t* gh = ws.hist + (size_t)row * kBins;
  for (int i = tid; i < kBins; i += kBlkThreads)
    if (s_h[i] != 0) atomicAdd(&gh[i], s_h[i]);
}

__global__ __launch_bounds__(kBlkThreads) void topk_classify_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, TopkWs ws) {
  __shared__ uint32_t s_wsum[kBlkThreads / kWave];
  __shared__ uint32_t s_d0;
  const int row = blockIdx.x / ws.n_blk, blk = blockIdx.x - row * ws.n_blk;
  const int n = row_len(end_pos, row, T, S_max);
  const int base = blk * kBlk;
  if (n <= k || base >= n) return;
  const int len = min(kBlk, n - base);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* x = scores + (size_t)row * S_max + base;

  // Positions base + tid + 256j; the loads stay in flight during the bin search.
  constexpr int kPer = kBlk / kBlkThreads;
  float v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = x[min(tid + kBlkThreads * j, len - 1)];

  // Bin d0: thread t owns bins 2047-8t down to 2040-8t.
  const uint32_t* gh = ws.hist + (size_t)row * kBins;
  const uint4 h_hi = *reinterpret_cast<const uint4*>(gh + kBins - 8 * tid - 4);
  const uint4 h_lo = *reinterpret_cast<const uint4*>(gh + kBins - 8 * tid - 8);
  const uint32_t c[8] = {h_hi.w, h_hi.z, h_hi.y, h_hi.x, h_lo.w, h_lo.z, h_lo.y, h_lo.x};
  uint32_t sum = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) sum += c[u];
  // No crossing (an inconsistent histogram) leaves d0 = 0 and the final kernel
  // falls back.  With garbage counts several bins may look like the crossing:
  // the highest one is taken, so that every block of the row, reading the same
  // histogram, classifies against the same d0.
  if (tid == 0) s_d0 = 0;
  const uint32_t incl = wave_incl_scan(sum);
  if (lane == 63) s_wsum[wave] = incl;
  lds_barrier();
  uint32_t above = incl - sum;
#pragma unroll
  for (int w = 0; w < kBlkThreads / kWave; ++w) above += w < wave ? s_wsum[w] : 0u;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    if (above < (uint32_t)k && (uint32_t)k <= above + c[u])
      atomicMax(&s_d0, (uint32_t)(kBins - 1 - (8 * tid + u)));
    above += c[u];
  }
  lds_barrier();
  const uint32_t d0 = s_d0;
  if (blk == 0 && tid == 0) ws.ctr[2 * row + 1] = d0;

  // Winners (bitmap) and candidates (count) of each 64-position group.
  uint64_t my_win = 0;
  uint32_t n_cand = 0;
  uint64_t cm[kPer];
  uint32_t key[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const bool valid = tid + kBlkThreads * j < len;
    key[j] = score_key(v[j]);
    const uint32_t d = key[j] >> 21;
    const uint64_t wm = __ballot(valid && d > d0);
    cm[j] = __ballot(valid && d == d0);
    n_cand += (uint32_t)__popcll(cm[j]);
    my_win = lane == j ? wm : my_win;
  }
  // Lane j < 8 holds the mask of positions base + 256j + 64*wave .. +63.
  uint64_t* win = ws.win + (size_t)row * ws.n_blk * (kBlk / 64) + blk * (kBlk / 64);
  if (lane < kPer) win[kBlkThreads / 64 * lane + wave] = my_win;
  if (n_cand == 0) return;  // wave-uniform
  uint32_t at = 0;
  if (lane == 0) at = atomicAdd(&ws.ctr[2 * row], n_cand);
  at = (uint32_t)__builtin_amdgcn_readfirstlane((int)at);
  uint2* cand = ws.cand + (size_t)row * kSelCap;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(cm[j] >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)cm[j], 0u));
    if (((cm[j] >> lane) & 1u) && at + rank < (uint32_t)kSelCap)
      cand[at + rank] = uint2{key[j], (uint32_t)(base + tid + kBlkThreads * j)};
    at += (uint32_t)__popcll(cm[j]);
  }
}

struct SelShared {
  uint32_t sure[kSelWords];  // bit p: position p is selected for certain
  uint32_t eq[kSelWords];    // bit p: the key of p equals the threshold
  uint32_t ck[kSelCap];      // candidate keys
  uint32_t cp[kSelCap];      // candidate positions
  uint32_t hist[kHistWords];
  uint32_t wave[2 * kTkWaves];
  uint32_t sel[2];
  uint32_t small[kWave];     // the few keys left after round 2
  uint32_t nsmall;
};

union TopkLds {
  TopkShared full;
  SelShared sel;
};

static_assert(kSelMaxN % kBlk == 0, "the bitmaps cover whole classify blocks");

// select_bin with LDS-only barriers.
template <bool kPadded = true>
__device__ __forceinline__ uint32_t sel_select_bin(const uint32_t* hist, int nbins,
                                                   uint32_t& remaining, uint32_t* s_sel) {
  lds_barrier();
  if (threadIdx.x < kWave) {
    uint32_t digit, above;
    wave_select_bin<kPadded>(hist, nbins, remaining, digit, above);
    if (threadIdx.x == 0) {
      s_sel[0] = digit;
      s_sel[1] = above;
    }
  }
  lds_barrier();
  const uint32_t digit = s_sel[0];
  remaining -= s_sel[1];
  return digit;
}

__global__ __launch_bounds__(kTkThreads) void topk_final_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, int32_t* __restrict__ out, TopkWs ws) {
  __shared__ __align__(16) TopkLds lds;
  SelShared& sh = lds.sel;
  const int row = blockIdx.x;
  const int n = row_len(end_pos, row, T, S_max);
  const float* x = scores + (size_t)row * S_max;
  int32_t* o = out + (size_t)row * k;
  uint4* gh = reinterpret_cast<uint4*>(ws.hist + (size_t)row * kBins) + threadIdx.x;
  const int tid = threadIdx.x;

  if (n <= k) {  // every valid position is kept
    for (int i = tid; i < k; i += kTkThreads) o[i] = i < n ? i : -1;
    *gh = uint4{0u, 0u, 0u, 0u};
    return;
  }
  bool ok = n <= kSelMaxN;
  if (ok) {
    // Everything the selection reads goes out at once: the counters, the
    // winner bitmap (16-byte pieces, at most 4 per thread) and the first 2048
    // candidate slots (4 per thread; the count then says which are real).
    // Loads are clamped; only the stores are conditional.
    const int nwords = (n + 31) >> 5;
    const int n16 = (nwords + 3) >> 2;
    const uint4* wsrc =
        reinterpret_cast<const uint4*>(ws.win + (size_t)row * ws.n_blk * (kBlk / 64));
    const uint2* cs = ws.cand + (size_t)row * kSelCap;
    const uint32_t C = ws.ctr[2 * row], d0 = ws.ctr[2 * row + 1];
    uint4 q[4];
    uint2 e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = wsrc[min(tid + kTkThreads * u, n16 - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) e[u] = cs[tid + kTkThreads * u];
    for (int i = tid; i < kHistWords; i += kTkThreads) sh.hist[i] = 0;  // round 2
    if (tid == 0) sh.nsmall = 0;
    uint32_t n_win = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + kTkThreads * u;
      if (i < n16) {
        reinterpret_cast<uint4*>(sh.sure)[i] = q[u];
        reinterpret_cast<uint4*>(sh.eq)[i] = uint4{0u, 0u, 0u, 0u};
        n_win += (uint32_t)(__popc(q[u].x) + __popc(q[u].y) + __popc(q[u].z) + __popc(q[u].w));
      }
    }
    const int nc = (int)min(C, (uint32_t)kSelCap);
    // A position outside the row can only come from a corrupted list.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + kTkThreads * u;
      if (i < nc) {
        sh.ck[i] = e[u].x;
        sh.cp[i] = min(e[u].y, (uint32_t)(n - 1));
      }
    }
#pragma unroll 1
    for (int b0 = 4 * kTkThreads; b0 < nc; b0 += 4 * kTkThreads) {
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = cs[min(b0 + tid + kTkThreads * u, nc - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = b0 + tid + kTkThreads * u;
        if (i < nc) {
          sh.ck[i] = e[u].x;
          sh.cp[i] = min(e[u].y, (uint32_t)(n - 1));
        }
      }
    }
    uint32_t S, dummy_ex, dummy_ex2, dummy_tot;
    block_exclusive_scan2(n_win, 0u, sh.wave, dummy_ex, dummy_ex2, S, dummy_tot);
    ok = S < (uint32_t)k && (uint32_t)k <= S + C && C <= (uint32_t)kSelCap;
    if (ok) {
      // Round 2 over the candidates (their top 11 bits are d0): bits 10..20.
      uint32_t remaining = (uint32_t)k - S;
      for (int i = tid; i < nc; i += kTkThreads)
        atomicAdd(&sh.hist[hpad((sh.ck[i] >> 10) & (kBins - 1))], 1u);
      const uint32_t d1 = sel_select_bin(sh.hist, kBins, remaining, sh.sel);
      const uint32_t pre = (d0 << 11) | d1;
      const uint32_t m = sh.hist[hpad(d1)];  // keys left in the running
      uint32_t thr, need_eq;
      if (m <= (uint32_t)kWave) {
        // Few keys left: gather them and let one wave rank them directly.
        for (int i = tid; i < nc; i += kTkThreads) {
          const uint32_t key = sh.ck[i];
          if ((key >> 10) == pre) sh.small[atomicAdd(&sh.nsmall, 1u)] = key;
        }
        lds_barrier();
        if (tid < kWave) {
          const bool valid = tid < (int)m;
          const uint32_t mine = sh.small[min(tid, (int)m - 1)];
          uint32_t gt = 0, ge = 0;
          for (int j2 = 0; j2 < (int)m; ++j2) {
            const uint32_t other = sh.small[j2];
            gt += other > mine ? 1u : 0u;
            ge += other >= mine ? 1u : 0u;
          }
          // The remaining-th largest key: fewer than `remaining` keys above it,
          // at least `remaining` at or above it.
          const bool hit = valid && gt < remaining && remaining <= ge;
          const uint64_t who = __ballot(hit);
          const int src = (int)__ffsll((long long)who) - 1;
          const uint32_t t_key = (uint32_t)__builtin_amdgcn_readlane((int)mine, src < 0 ? 0 : src);
          const uint32_t t_gt = (uint32_t)__builtin_amdgcn_readlane((int)gt, src < 0 ? 0 : src);
          if (tid == 0) {
            sh.sel[0] = t_key;
            sh.sel[1] = remaining - t_gt;
          }
        }
        lds_barrier();
        thr = sh.sel[0];
        need_eq = sh.sel[1];
      } else {
        // Round 3: the last 10 bits.
        for (int i = tid; i < kHistWords; i += kTkThreads) sh.hist[i] = 0;
        lds_barrier();
        for (int i = tid; i < nc; i += kTkThreads) {
          const uint32_t key = sh.ck[i];
          atomicAdd(&sh.hist[hpad(key & 1023u)], (key >> 10) == pre ? 1u : 0u);
        }
        const uint32_t d2 = sel_select_bin(sh.hist, 1024, remaining, sh.sel);
        thr = (pre << 10) | d2;
        need_eq = remaining;
      }
      for (int i = tid; i < nc; i += kTkThreads) {
        const uint32_t key = sh.ck[i], p = sh.cp[i];
        if (key > thr) atomicOr(&sh.sure[p >> 5], 1u << (p & 31));
        else if (key == thr) atomicOr(&sh.eq[p >> 5], 1u << (p & 31));
      }
      lds_barrier();
      // Ordered output: thread t owns bitmap words [w0, w1).
      const int wpt = (nwords + kTkThreads - 1) / kTkThreads;
      const int w0 = min(tid * wpt, nwords), w1 = min(w0 + wpt, nwords);
      uint32_t n_gt = 0, n_eq = 0;
      for (int w = w0; w < w1; ++w) {
        n_gt += (uint32_t)__popc(sh.sure[w]);
        n_eq += (uint32_t)__popc(sh.eq[w]);
      }
      uint32_t gt, eqb, tot_gt, tot_eq;
      block_exclusive_scan2(n_gt, n_eq, sh.wave, gt, eqb, tot_gt, tot_eq);
      for (int w = w0; w < w1; ++w) {
        const uint32_t s = sh.sure[w], e = sh.eq[w];
        uint32_t bits = s | e;
        while (bits != 0u) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1u;
          const int32_t p = 32 * w + b;
          if ((s >> b) & 1u) {
            const uint32_t at = gt + min(eqb, need_eq);
            if (at < (uint32_t)k) o[at] = p;
            ++gt;
          } else {
            if (eqb < need_eq && gt + eqb < (uint32_t)k) o[gt + eqb] = p;
            ++eqb;
          }
        }
      }
    }
  }
  // A fallback starts after the scan's last barrier: no wave reads the
  // selection's LDS any more.
  if (!ok) full_row_topk(x, n, k, o, lds.full);
  *gh = uint4{0u, 0u, 0u, 0u};  // leave the row's histogram zeroed for the next call
}

__global__ __launch_bounds__(kTkThreads) void topk_row_kernel(const float* __restrict__ scores,
                                                              const int32_t* __restrict__ end_pos,
                                                              int T, int S_max, int k,
                                                              int32_t* __restrict__ out) {
  __shared__ __align__(16) TopkShared sh;
  const int row = blockIdx.x;
  const int n = row_len(end_pos, row, T, S_max);
  int32_t* o = out + (size_t)row * k;
  if (n <= k) {
    for (int i = threadIdx.x; i < k; i += kTkThreads) o[i] = i < n ? i : -1;
    return;
  }
  full_row_topk(scores + (size_t)row * S_max, n, k, o, sh);
}

// ---------------------------------------------------------------------------
// Rows of up to 32768 positions: one workgroup per row with the whole row in
// registers (64 keys per thread), no workspace.  Wave w takes the 64-position
// groups w, w+8, w+16, ... (one coalesced 256-byte load each), so a run of
// high scores is spread over all waves.
//   1. Keys of all positions; LDS histogram of the top 11 bits; bin d0.
//   2. One pass over the registers: per group, a ballot of the winners (top
//      bits above d0) goes to the winner bitmap and the candidates (in bin
//      d0) are appended to the wave's own region of the candidate list.
//   3. Round 2 over the candidates, then either a direct rank of the few keys
//      left (one wave) or round 3; candidates above the threshold join the
//      winner bitmap, those equal to it go to the tie bitmap.
//   4. Ordered output from the two bitmaps.
// If a wave's region overflows (more than 1024 candidates in its groups) the
// row is redone by full_row_topk.
constexpr int kLeanMaxN = kChunk;               // 32768
constexpr int kLeanGroups = kLeanMaxN / kWave / kTkWaves;  // 64 groups per wave
constexpr int kLeanRegion = kSelCap / kTkWaves;  // 1024 candidates per wave

struct LeanShared {
  uint32_t hist[kHistWords];   // round 1 (and round 3)
  uint32_t hist2[kHistWords];  // round 2
  uint32_t sure[kLeanMaxN / 32];
  uint32_t eq[kLeanMaxN / 32];
  uint32_t ck[kSelCap];        // wave w's candidates at [1024 w, 1024 w + ncw[w])
  uint32_t cp[kSelCap];
  uint32_t ncw[kTkWaves];
  uint32_t wave[2 * kTkWaves];
  uint32_t sel[2];
  uint32_t small[kWave];
  uint32_t nsmall;
};

union LeanLds {
  TopkShared full;
  LeanShared lean;
};

__global__ __launch_bounds__(kTkThreads) void topk_lean_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, int32_t* __restrict__ out) {
  __shared__ __align__(16) LeanLds lds;
  LeanShared& sh = lds.lean;
  const int row = blockIdx.x;
  const int n = row_len(end_pos, row, T, S_max);
  const float* x = scores + (size_t)row * S_max;
  int32_t* o = out + (size_t)row * k;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (n <= k) {  // every valid position is kept
    for (int i = tid; i < k; i += kTkThreads) o[i] = i < n ? i : -1;
    return;
  }
  bool ok = n <= kLeanMaxN;
  if (ok) {
    // Position of group i of this wave, lane l: 64 (8 i + wave) + l.
    uint32_t key[kLeanGroups];
#pragma unroll
    for (int i = 0; i < kLeanGroups; ++i)
      key[i] = __float_as_uint(x[min(kWave * (kTkWaves * i + wave) + lane, n - 1)]);
    for (int i = tid; i < kHistWords; i += kTkThreads) {
      sh.hist[i] = 0;
      sh.hist2[i] = 0;
    }
    for (int i = tid; i < kLeanMaxN / 32; i += kTkThreads) sh.eq[i] = 0;
    if (tid == 0) sh.nsmall = 0;
    lds_barrier();
    // 1. Round 1 (unpadded histogram).  Every lane counts; the lanes past the
    // row end loaded position n-1 again, and thread 0 takes those 32768 - n
    // extra counts back out of that key's bin.
#pragma unroll
    for (int i = 0; i < kLeanGroups; ++i) {
      key[i] = score_key(__uint_as_float(key[i]));
      atomicAdd(&sh.hist[key[i] >> 21], 1u);
    }
    if (tid == 0)
      atomicSub(&sh.hist[score_key(x[n - 1]) >> 21], (uint32_t)(kLeanMaxN - n));
    uint32_t remaining = (uint32_t)k;
    const uint32_t d0 = sel_select_bin<false>(sh.hist, kBins, remaining, sh.sel);
    // 2. Winners and candidates.
    uint32_t win_lo = 0, win_hi = 0, nc = 0;
    const int region = wave * kLeanRegion;
#pragma unroll
    for (int i = 0; i < kLeanGroups; ++i) {
      const int base = kWave * (kTkWaves * i + wave);
      const bool in_row = lane < n - base;
      const uint32_t d = key[i] >> 21;
      const bool c = in_row && d == d0;
      const uint64_t wm = __builtin_amdgcn_ballot_w64(in_row && d > d0);
      const uint64_t cm = __builtin_amdgcn_ballot_w64(c);
      win_lo = lane == i ? (uint32_t)wm : win_lo;
      win_hi = lane == i ? (uint32_t)(wm >> 32) : win_hi;
      const uint32_t at = nc + __builtin_amdgcn_mbcnt_hi((uint32_t)(cm >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)cm, 0u));
      if (c && at < (uint32_t)kLeanRegion) {
        sh.ck[region + at] = key[i];
        sh.cp[region + at] = (uint32_t)(base + lane);
      }
      nc += (uint32_t)__popcll(cm);
    }
    // Lane i holds the winner mask of group 8 i + wave.
    reinterpret_cast<uint2*>(sh.sure)[kTkWaves * lane + wave] = uint2{win_lo, win_hi};
    if (lane == 0) sh.ncw[wave] = nc;
    lds_barrier();
    uint32_t over = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) over |= sh.ncw[w] > (uint32_t)kLeanRegion ? 1u : 0u;
    ok = over == 0;
    if (ok) {
      // 3. Round 2 over each wave's own candidates: bits 10..20.
      const int my_nc = (int)nc;
      for (int j = lane; j < my_nc; j += kWave)
        atomicAdd(&sh.hist2[hpad((sh.ck[region + j] >> 10) & (kBins - 1))], 1u);
      const uint32_t d1 = sel_select_bin(sh.hist2, kBins, remaining, sh.sel);
      const uint32_t pre = (d0 << 11) | d1;
      const uint32_t m = sh.hist2[hpad(d1)];  // keys left in the running
      uint32_t thr, need_eq;
      if (m <= (uint32_t)kWave) {
        for (int j = lane; j < my_nc; j += kWave) {
          const uint32_t kk = sh.ck[region + j];
          if ((kk >> 10) == pre) sh.small[atomicAdd(&sh.nsmall, 1u)] = kk;
        }
        lds_barrier();
        if (wave == 0) {
          const bool valid = lane < (int)m;
          const uint32_t mine = sh.small[min(lane, (int)m - 1)];
          uint32_t gt = 0, ge = 0;
          for (int j = 0; j < (int)m; ++j) {
            const uint32_t other = sh.small[j];
            gt += other > mine ? 1u : 0u;
            ge += other >= mine ? 1u : 0u;
          }
          const bool hit = valid && gt < remaining && remaining <= ge;
          const uint64_t who = __ballot(hit);
          const int src = who ? (int)__ffsll((long long)who) - 1 : 0;
          const uint32_t t_key = (uint32_t)__builtin_amdgcn_readlane((int)mine, src);
          const uint32_t t_gt = (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
          if (lane == 0) {
            sh.sel[0] = t_key;
            sh.sel[1] = remaining - t_gt;
          }
        }
        lds_barrier();
        thr = sh.sel[0];
        need_eq = sh.sel[1];
      } else {
        for (int i = tid; i < kHistWords; i += kTkThreads) sh.hist[i] = 0;
        lds_barrier();
        for (int j = lane; j < my_nc; j += kWave) {
          const uint32_t kk = sh.ck[region + j];
          atomicAdd(&sh.hist[hpad(kk & 1023u)], (kk >> 10) == pre ? 1u : 0u);
        }
        const uint32_t d2 = sel_select_bin(sh.hist, 1024, remaining, sh.sel);
        thr = (pre << 10) | d2;
        need_eq = remaining;
      }
      for (int j = lane; j < my_nc; j += kWave) {
        const uint32_t kk = sh.ck[region + j], p = sh.cp[region + j];
        if (kk > thr) atomicOr(&sh.sure[p >> 5], 1u << (p & 31));
        else if (kk == thr) atomicOr(&sh.eq[p >> 5], 1u << (p & 31));
      }
      lds_barrier();
      // 4. Ordered output: thread t owns 32-bit words 2t and 2t+1.
      const int nwords = (n + 31) >> 5;
      const int w0 = min(2 * tid, nwords), w1 = min(w0 + 2, nwords);
      uint32_t n_gt = 0, n_eq = 0;
      for (int w = w0; w < w1; ++w) {
        n_gt += (uint32_t)__popc(sh.sure[w]);
        n_eq += (uint32_t)__popc(sh.eq[w]);
      }
      uint32_t gt, eqb, tot_gt, tot_eq;
      block_exclusive_scan2(n_gt, n_eq, sh.wave, gt, eqb, tot_gt, tot_eq);
      for (int w = w0; w < w1; ++w) {
        const uint32_t sw = sh.sure[w], ew = sh.eq[w];
        uint32_t bits = sw | ew;
        while (bits != 0u) {
          const int b = __ffs(bits) - 1;
          bits &= bits - 1u;
          const int32_t p = 32 * w + b;
          if ((sw >> b) & 1u) {
            const uint32_t at = gt + min(eqb, need_eq);
            if (at < (uint32_t)k) o[at] = p;
            ++gt;
          } else {
            if (eqb < need_eq && gt + eqb < (uint32_t)k) o[gt + eqb] = p;
            ++eqb;
          }
        }
      }
    }
  }
  if (!ok) {
    __syncthreads();  // the overflow check's reads are done before the LDS is reused
    full_row_topk(x, n, k, o, lds.full);
  }
}

static_assert(kLeanGroups * kWave * kTkWaves == kLeanMaxN, "row fits the registers");
static_assert(kTkThreads * 2 * 32 == kLeanMaxN, "two bitmap words per thread");

static_assert(kTkThreads * 4 == kBins, "one 16-byte histogram piece per thread");

int launch_topk(const float* scores, const int32_t* end_pos, int B, int T, int S_max,
                int max_end_pos, int k, int32_t* out, void* workspace, hipStream_t stream) {
  const int rows = B * T;
  if (max_end_pos <= kLeanMaxN) {
    hipLaunchKernelGGL(topk_lean_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, stream,
                       scores, end_pos, T, S_max, k, out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  if (rows > kMultiRows) {
    hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, stream,
                       scores, end_pos, T, S_max, k, out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  const TopkWs ws = carve_topk_ws(workspace, rows, S_max);
  const dim3 blk_grid((unsigned)((long)rows * ws.n_blk));
  hipLaunchKernelGGL(topk_hist_kernel, blk_grid, dim3(kBlkThreads), 0, stream, scores, end_pos,
                     T, S_max, k, ws);
  if (hipGetLastError() != hipSuccess) return -5;
  hipLaunchKernelGGL(topk_classify_kernel, blk_grid, dim3(kBlkThreads), 0, stream, scores,
                     end_pos, T, S_max, k, ws);
  if (hipGetLastError() != hipSuccess) return -5;
  hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, stream,
                     scores, end_pos, T, S_max, k, out, ws);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace dsa
