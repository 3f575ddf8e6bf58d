// Per-query top-k selection on gfx950 (topk(min(index_topk, end_pos)) of
// Indexer.forward, "DeepSeek-V3.2-Exp - Keep top-k positions").
//
// Integer-only radix select.  Each score becomes an order-preserving 32-bit
// key (score_key: -0 folded into +0, sign-magnitude flipped so unsigned order
// equals float order).  Three histogram rounds (11, 11, 10 key bits, most
// significant first) find the key `thr` of the k-th largest element and how
// many elements equal to thr are kept (need_eq).  A compaction pass then
// writes, in ascending position order, every element with key > thr and the
// first need_eq elements with key == thr, so ties go to the smaller position
// and the output is unique.
//
// One 512-thread workgroup (8 waves, two per SIMD) per query row, working on
// chunks of up to 32768 positions.  A chunk is read with coalesced loads and
// turned into keys, which are counted for the first round's histogram (top 11
// bits, LDS atomics with no return value) and stored in LDS.  Thread t owns
// the 64 consecutive positions 64t..64t+63 and reads them 16 at a time with
// 16-byte loads (the LDS copy is swizzled in 16-byte groups so both the
// scattered writes and the segment reads are free of bank conflicts).  Then:
//   1. the keys of the winning bin are appended to a small candidate list and
//      rounds 2 and 3 histogram only that list (if the bin is too crowded,
//      e.g. under heavy ties, they scan the whole row instead);
//   2. per-thread (greater, equal) counts, one scan, and each thread writes
//      its own selected positions in order, visiting only those (bit masks
//      over its segment, keys re-read from the LDS copy).
// Bin searches, and rounds 2 and 3 over a candidate list, are done by one wave.  A row that fits in one chunk is read
// from memory once; longer rows are re-read chunk by chunk in each phase
// (they sit in L2 / the last-level cache right after the indexer wrote them).
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
    const uint32_t v = hist[hpad((uint32_t)bin)];
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

__global__ __launch_bounds__(kTkThreads) void topk_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ end_pos,
                                                          int T, int S_max, int k,
                                                          int32_t* __restrict__ out) {
  __shared__ __align__(16) uint32_t s_keys[kChunk];
  __shared__ uint32_t s_hist[kHistWords];
  __shared__ uint32_t s_cand[kCandCap];
  __shared__ __align__(16) uint32_t s_wave[2 * kTkWaves];
  __shared__ uint32_t s_sel[2];
  __shared__ uint32_t s_ncand;

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

size_t topk_workspace_bytes(int, int, int, int) { return 0; }

int launch_topk(const float* scores, const int32_t* end_pos, int B, int T, int S_max, int,
                int k, int32_t* out, void*, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((long)B * T)), dim3(kTkThreads), 0, stream,
                     scores, end_pos, T, S_max, k, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace dsa
