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
// Four ways to run it, chosen on the host from the row count and the
// longest row:
//  * up to 1024 rows of 4097..131072 positions (decode): topk_cut_kernel
//    spreads each row over workgroups of 2048 positions (8192 above 32768)
//    that cut it down to position-ordered candidate regions, and
//    topk_pick_kernel, one workgroup per row, selects among them (two
//    launches);
//  * other rows when there are at most 1024: topk_split_kernel spreads each
//    row over workgroups that append their candidates to one list per row,
//    and topk_finish_kernel selects among them (one launch when a row fits
//    one workgroup, else two);
//  * more rows, each of at most 32768 positions (prefill): topk_lean_kernel,
//    one 512-thread workgroup per row holding the whole row in registers;
//  * otherwise: full_row_topk, one workgroup per row, chunk by chunk
//    (topk_row_kernel).
// The candidate paths fall back to full_row_topk for a row whose candidates
// cannot be trusted (fewer than k of them, or more than the lists hold), so
// the result is exact whatever the sample says.  Only the split path needs
// anything in the workspace beforehand: its per-row list counters must be
// zero when it starts (dsa_forward has the indexer clear them, dsa_topk
// launches a small clearing kernel).
#include "dsa_device.h"
#include "dsa_launch.h"
#include "select.h"

#include <cstddef>
#include <type_traits>

namespace dsa {

constexpr int kTkThreads = 512;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kSeg = 64;                   // positions per thread per chunk
constexpr int kChunk = kTkThreads * kSeg;  // 32768 positions per chunk
constexpr int kCandCap = 4096;             // candidate keys
static_assert(kTkThreads == kSplitThreads && kChunk == kSpShortMax, "split workspace layout");

// Word of element j of segment t in the LDS chunk: 16-byte group j/4 is
// XOR-swizzled with the low bits of t, so lanes reading the same group of
// consecutive segments hit different 4-bank sets.
__device__ __forceinline__ int swz(int t, int j) {
  return kSeg * t + 4 * ((j >> 2) ^ (t & (kSeg / 4 - 1))) + (j & 3);
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

__device__ __noinline__ void full_row_topk(const float* __restrict__ x, int n, int k,
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
// Up to 1024 rows of at most 4096 (or more than 131072) positions: each row
// is spread over workgroups of 512 * kSpPer positions (topk_split_kernel), and
// a second launch with one workgroup per row finishes it (topk_finish_kernel).
//   1. Every workgroup derives the same cut L from the same 2048 sampled
//      positions of the row, 128 evenly spaced runs of 16 consecutive ones
//      (run g starts at floor(g (n - 16) / 127); one 64-byte segment per run,
//      where single positions at a stride cost a cache line each and made
//      the sample most of a long row's traffic): the 22-bit key prefix of the
//      sample's T_s-th largest key, T_s being the sample's expected count of
//      keys above the k-th largest plus four standard deviations (and 16).
//   2. It appends its keys >= L with their positions to the row's list in the
//      workspace (one device-scope atomic per workgroup reserves the slots).
//   3. The finishing workgroup loads the list into registers, runs up to
//      three radix rounds over it (the last one a direct rank when at most 64
//      keys are left), marks the keys above the threshold in a winner bitmap
//      and those equal to it in a tie bitmap, and writes the ordered output.
// The launch boundary makes the lists visible to the finishing workgroups
// (one release for the whole grid; fences in every workgroup cost more).  A
// row that fits one workgroup is selected by it directly from its registers.
// If the list holds fewer than k keys (the sample misjudged the row), more
// than it can hold, or the row is longer than the bitmaps, the finishing
// workgroup selects the row from scratch (full_row_topk).  The list counter
// of each row must be zero when the first launch starts: the indexer clears
// it in the fused call, a small kernel otherwise.
constexpr int kSpSample = 2048;                       // sampled positions per row
constexpr int kSpSamplePer = kSpSample / kTkThreads;  // 4 per thread
constexpr int kSpListPer = kSpCap / kTkThreads;       // 16 per thread


union SplitLds {
  TopkShared full;
  SelectShared sp;
};

// Exact selection of the k largest among M >= k keys, all >= L, held in
// registers: entry tid + 512u of the set is (ek[u], ep[u]) for every
// tid + 512u < M.  Writes the row's ordered output.
template <int kEnt, class Sh>
__device__ __forceinline__ void split_select(const uint32_t (&ek)[kEnt], const uint32_t (&ep)[kEnt],
                                             int M, int n, int k, int32_t* __restrict__ o,
                                             uint32_t L, Sh& sh) {
  RegCandidates<kTkThreads, kEnt> cand;
#pragma unroll
  for (int u = 0; u < kEnt; ++u) {
    cand.d[u] = ek[u] - L;
    cand.p[u] = ep[u];
  }
  cand.M = M;
  uint32_t thr, need_eq;
  block_select<kTkThreads>(cand, n, k, sh, thr, need_eq);
  // Each winner writes its position at its rank among the winners by position.
  cand.each([&](uint32_t d, uint32_t p) {
    if (d >= thr) {
      const int at = winner_slot(sh.sure, sh.eq, sh.pre, p, d > thr, need_eq);
      if (at >= 0 && at < k) o[at] = (int32_t)p;
    }
  });
}

// Step 3 for the row's last workgroup: the list -> registers -> selection.
__device__ __forceinline__ void split_finish(const float* __restrict__ x, int n, int k, int32_t* __restrict__ o,
                             const uint32_t* count, const uint2* __restrict__ list, uint32_t L,
                             SplitLds& lds) {
  const int tid = threadIdx.x;
  const uint32_t M = __hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool ok = M >= (uint32_t)k && M <= (uint32_t)kSpCap && n <= kSpMaxN;
  if (!ok) {
    full_row_topk(x, n, k, o, lds.full);
    return;
  }
  uint32_t ek[kSpListPer], ep[kSpListPer];
#pragma unroll
  for (int u = 0; u < kSpListPer; ++u) {
    const uint2 e = list[min(tid + kTkThreads * u, (int)M - 1)];
    ek[u] = e.x;
    ep[u] = min(e.y, (uint32_t)(n - 1));  // a position outside the row cannot occur
  }
  split_select<kSpListPer>(ek, ep, (int)M, n, k, o, L, lds.sp);
}

// kFallback: this launch is the only one (every row fits one workgroup), so
// it also selects rows longer than max_end_pos promised (full_row_topk, with
// its large LDS); otherwise the finishing launch does, and this one's LDS is
// sized for its own positions only (several workgroups per CU).
template <int kSpPer, bool kFallback>
struct SplitKernelLds {
  using Sel = SelectSharedT<kTkThreads * kSpPer>;
  union U {
    TopkShared full;
    Sel sp;
  };
  using Type = typename std::conditional<kFallback, U, Sel>::type;
};

// Without kFallback: at most 128 registers (4 waves per SIMD), two
// workgroups per CU.
template <int kSpPer, bool kFallback>
__global__ __launch_bounds__(kTkThreads, kFallback ? 1 : 4) void topk_split_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, int32_t* __restrict__ out, SplitWs ws) {
  constexpr int kSpBlk = kTkThreads * kSpPer;  // positions per workgroup
  using Lds = typename SplitKernelLds<kSpPer, kFallback>::Type;
  __shared__ __align__(16) Lds lds;
  auto& sh = [&]() -> typename SplitKernelLds<kSpPer, kFallback>::Sel& {
    if constexpr (kFallback) return lds.sp;
    else return lds;
  }();
  const int row = blockIdx.x / ws.n_blk, blk = blockIdx.x - row * ws.n_blk;
  const int n = row_len(end_pos, row, T, S_max);
  const float* x = scores + (size_t)row * S_max;
  int32_t* o = out + (size_t)row * k;
  const int tid = threadIdx.x, lane = tid & 63;
  if (n <= k) {  // every valid position is kept
    if (blk == 0)
      for (int i = tid; i < k; i += kTkThreads) o[i] = i < n ? i : -1;
    return;
  }
  if (n > ws.n_blk * kSpBlk) {  // longer than max_end_pos promised: not split
    if constexpr (kFallback) {
      if (blk == 0) full_row_topk(x, n, k, o, lds.full);
    }
    return;  // (without kFallback, the finishing launch selects the row)
  }
  const int base = blk * kSpBlk;
  if (base >= n) return;
  const int nb = (n + kSpBlk - 1) / kSpBlk;  // workgroups that take part for this row

  // This workgroup's positions base + tid + 512u, and the row's sample.
  uint32_t kv[kSpPer], ks[kSpSamplePer];
#pragma unroll
  for (int u = 0; u < kSpPer; ++u)
    kv[u] = __float_as_uint(x[min(base + tid + kTkThreads * u, n - 1)]);
#pragma unroll
  for (int u = 0; u < kSpSamplePer; ++u) {
    const int s = tid + kTkThreads * u;  // sample s: run s / 16, position s % 16 in it
    const int pos = n >= kSpSample
                        ? (int)(((uint64_t)(s >> 4) * (uint64_t)(n - 16)) / (kSpSample / 16 - 1)) + (s & 15)
                        : (int)(((uint64_t)s * (uint64_t)n) / (uint64_t)kSpSample);
    ks[u] = __float_as_uint(x[pos]);
  }
  if (nb == 1) {
    // The whole row is in this workgroup's registers: select over it directly.
    uint32_t pv[kSpPer];
#pragma unroll
    for (int u = 0; u < kSpPer; ++u) {
      kv[u] = score_key(__uint_as_float(kv[u]));
      pv[u] = (uint32_t)(tid + kTkThreads * u);
    }
    split_select<kSpPer>(kv, pv, n, n, k, o, 0u, sh);
    return;
  }
  for (int i = tid; i < kHistWords; i += kTkThreads) {
    sh.hist[i] = 0;
    sh.hist2[i] = 0;
  }
  lds_barrier();

  // 1. The cut L.
#pragma unroll
  for (int u = 0; u < kSpSamplePer; ++u) {
    ks[u] = score_key(__uint_as_float(ks[u]));
    atomicAdd(&sh.hist[hpad(ks[u] >> 21)], 1u);
  }
  const float mean = (float)k * (float)kSpSample / (float)n;
  uint32_t rem = min((uint32_t)kSpSample, (uint32_t)(mean + 4.0f * sqrtf(mean) + 16.0f));
  const uint32_t s0 = sel_select_bin(sh.hist, kBins, rem, sh.sel);
#pragma unroll
  for (int u = 0; u < kSpSamplePer; ++u)
    if ((ks[u] >> 21) == s0) atomicAdd(&sh.hist2[hpad((ks[u] >> 10) & (kBins - 1))], 1u);
  const uint32_t s1 = sel_select_bin(sh.hist2, kBins, rem, sh.sel);
  const uint32_t L = (s0 << 21) | (s1 << 10);

  // 2. Keys >= L -> the row's list.
  bool ge[kSpPer];
  uint32_t cnt = 0;
#pragma unroll
  for (int u = 0; u < kSpPer; ++u) {
    kv[u] = score_key(__uint_as_float(kv[u]));
    ge[u] = base + tid + kTkThreads * u < n && kv[u] >= L;
    cnt += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(ge[u]));
  }
  // One device-scope atomic per workgroup reserves the slots of all its waves.
  const int wave = tid >> 6;
  if (lane == 0) sh.wave[wave] = cnt;
  lds_barrier();
  if (tid == 0) {
    uint32_t tot = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) tot += sh.wave[w];
    sh.wave[kTkWaves] = tot != 0 ? atomicAdd(&ws.ctr[kCtrWords * row + 1], tot) : 0u;
    if (blk == 0) ws.ctr[kCtrWords * row + 2] = L;
  }
  lds_barrier();
  uint32_t at = sh.wave[kTkWaves];
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) at += w < wave ? sh.wave[w] : 0u;
  uint2* list = ws.list + (size_t)row * kSpCap;
#pragma unroll
  for (int u = 0; u < kSpPer; ++u) {
    const uint64_t mk = __builtin_amdgcn_ballot_w64(ge[u]);
    const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
    if (ge[u] && at + r < (uint32_t)kSpCap)
      list[at + r] = uint2{kv[u], (uint32_t)(base + tid + kTkThreads * u)};
    at += (uint32_t)__popcll(mk);
  }
}

// Second launch: one workgroup per row finishes the rows that the first
// launch spread over several workgroups.
template <int kSpPer>
__global__ __launch_bounds__(kTkThreads) void topk_finish_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, int32_t* __restrict__ out, SplitWs ws) {
  constexpr int kSpBlk = kTkThreads * kSpPer;
  __shared__ __align__(16) SplitLds lds;
  const int row = blockIdx.x;
  const int n = row_len(end_pos, row, T, S_max);
  if (n <= k || n <= ws.blk_pos) return;  // done by the first launch
  const float* x = scores + (size_t)row * S_max;
  if (n > ws.n_blk * ws.blk_pos) {  // longer than max_end_pos promised: not split
    full_row_topk(x, n, k, out + (size_t)row * k, lds.full);
    return;
  }
  split_finish(x, n, k, out + (size_t)row * k, ws.ctr + kCtrWords * row + 1,
               ws.list + (size_t)row * kSpCap, ws.ctr[kCtrWords * row + 2], lds);
}

// ---------------------------------------------------------------------------
// Decode rows (up to 1024 rows of 4097..131072 positions), two launches.
//   topk_cut_kernel: a row is spread over workgroups of 512 * kPer positions
//     (2048, or 8192 for rows above 32768; wave w of a workgroup owns its
//     64 * kPer consecutive positions, so every load instruction reads 256
//     contiguous bytes).  Every workgroup derives the same cut L from the
//     row's 2048-position sample (as the split top-k) and writes its keys >= L
//     with their positions to its own region of the row's list, in position
//     order (waves in order, a wave's entries by ballot rank), and a header
//     (count, L).  No atomics, nothing to clear.
//   topk_pick_kernel: one workgroup per row copies the regions into LDS in
//     position order (32 threads per region load its first entries together
//     with the headers; the whole workgroup copies what a region holds beyond
//     them), takes entries 8t..8t+7 (16 for the long rows) of their
//     concatenation into thread t's registers and selects among them with
//     ordered_select (radix rounds over key - L, each winner's slot from one
//     block scan).
// When the list misses (fewer than k keys, a region over its capacity, more
// entries than the pick holds, or a row longer than promised) the pick
// workgroup selects the row from scratch (full_row_topk), which is exact
// whatever the sample said.
// List entries per region: a 2048-position region can never overflow; an
// 8192-position region of a row of ~8-12K positions keeps ~2500 candidates
// (the sample's margin over k grows as 4 sqrt(n)), the rest far fewer.
constexpr int kCutCap = 2048;
constexpr int kCutCapLong = 3072;
constexpr int kCutMaxRegions = 16;
constexpr int kCutPer = 4;                       // positions per thread of a cut workgroup
constexpr int kCutPerLong = 16;                  // the same for rows of 32769..131072
constexpr int kCutMaxN = kCutMaxRegions * kTkThreads * kCutPer;          // 32768
constexpr int kCutMaxNLong = kCutMaxRegions * kTkThreads * kCutPerLong;  // 131072
// Entries the pick workgroup selects over (8 or 16 a thread), and how many
// of each region's entries a thread loads together with the headers: a
// 131072-position row keeps ~4500 candidates, ~280 a region.
template <int kPer> struct PickShape {
  static constexpr int kRegCap = kPer == kCutPer ? kCutCap : kCutCapLong;  // entries per region
  static constexpr int kCap = kPer == kCutPer ? 4096 : 8192;
  static constexpr int kEnt = kCap / kTkThreads;
  static constexpr int kSpec = kPer == kCutPer ? 8 : 12;
};

struct CutHdr {
  uint32_t count, L, pad0, pad1;
};
struct CutWs {
  CutHdr* hdr;  // [rows][kCutMaxRegions]
  uint2* list;  // [rows][kCutMaxRegions][PickShape<per>::kRegCap]: (key, position)
  int n_reg;    // regions (workgroups) per row
};

// Rows of 4097..131072 positions take the cut path: at batch 8 x 131072 its
// top-k took 15.8 us against 18.4 us for the split path, at batch 64 (rows of
// 8192..131072 positions) 22.4 us against 24.7 us.
__host__ inline bool cut_path(int rows, int max_end_pos) {
  return rows <= kMultiRows && max_end_pos > kSplitThreads * kSpPerShort &&
         max_end_pos <= kCutMaxNLong;
}
static_assert(kSplitThreads * kSpPerShort == 4096 && kCutMaxNLong > kSpShortMax,
              "the split path sees rows of at most 4096 positions (one workgroup, 8 a "
              "thread) or longer than the cut path's 131072 (16 a thread)");
// Positions per thread of the cut workgroups for rows of at most max_end_pos.
__host__ inline int cut_per(int max_end_pos) {
  return max_end_pos <= kCutMaxN ? kCutPer : kCutPerLong;
}
__host__ inline size_t cut_ws_bytes(int rows) {
  return align256((size_t)rows * kCutMaxRegions * sizeof(CutHdr)) +
         (size_t)rows * kCutMaxRegions * kCutCapLong * sizeof(uint2);
}
__host__ inline CutWs carve_cut_ws(void* ws, int rows, int max_end_pos) {
  CutWs w;
  char* p = reinterpret_cast<char*>(ws);
  w.hdr = reinterpret_cast<CutHdr*>(p);
  w.list = reinterpret_cast<uint2*>(p + align256((size_t)rows * kCutMaxRegions * sizeof(CutHdr)));
  const int blk = kTkThreads * cut_per(max_end_pos);
  w.n_reg = (max_end_pos + blk - 1) / blk;
  return w;
}

template <int kPer>
__global__ __launch_bounds__(kTkThreads) void topk_cut_kernel(const float* __restrict__ scores,
                                                              const int32_t* __restrict__ end_pos,
                                                              int T, int S_max, int k,
                                                              int32_t* __restrict__ out, CutWs ws) {
  constexpr int kBlk = kTkThreads * kPer;
  __shared__ uint32_t s_hist[kHistWords];
  __shared__ uint32_t s_hist2[kHistWords];
  __shared__ uint32_t s_sel[2];
  __shared__ uint32_t s_cnt[kTkWaves];
  const int row = blockIdx.x / ws.n_reg, blk = blockIdx.x - row * ws.n_reg;
  const int n = row_len(end_pos, row, T, S_max);
  const float* x = scores + (size_t)row * S_max;
  const int tid = threadIdx.x, lane = tid & 63;
  if (n <= k) {  // every valid position is kept
    if (blk == 0) {
      int32_t* o = out + (size_t)row * k;
      for (int i = tid; i < k; i += kTkThreads) o[i] = i < n ? i : -1;
    }
    return;
  }
  if (n > ws.n_reg * kBlk) return;  // longer than max_end_pos promised: the pick launch selects it
  const int base = blk * kBlk;
  if (base >= n) return;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wbase = base + wave * kWave * kPer;  // this wave's first position

  uint32_t kv[kPer], ks[kSpSamplePer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) kv[u] = __float_as_uint(x[min(wbase + kWave * u + lane, n - 1)]);
#pragma unroll
  for (int u = 0; u < kSpSamplePer; ++u) {
    const int s = tid + kTkThreads * u;  // sample s: run s / 16, position s % 16 in it
    const int pos = n >= kSpSample
                        ? (int)(((uint64_t)(s >> 4) * (uint64_t)(n - 16)) / (kSpSample / 16 - 1)) + (s & 15)
                        : (int)(((uint64_t)s * (uint64_t)n) / (uint64_t)kSpSample);
    ks[u] = __float_as_uint(x[pos]);
  }
  for (int i = tid; i < kHistWords; i += kTkThreads) {
    s_hist[i] = 0;
    s_hist2[i] = 0;
  }
  lds_barrier();

  // The cut L: the 22-bit key prefix of the sample's T_s-th largest key.
#pragma unroll
  for (int u = 0; u < kSpSamplePer; ++u) {
    ks[u] = score_key(__uint_as_float(ks[u]));
    atomicAdd(&s_hist[hpad(ks[u] >> 21)], 1u);
  }
  const float mean = (float)k * (float)kSpSample / (float)n;
  uint32_t rem = min((uint32_t)kSpSample, (uint32_t)(mean + 4.0f * sqrtf(mean) + 16.0f));
  const uint32_t c0 = sel_select_bin(s_hist, kBins, rem, s_sel);
#pragma unroll
  for (int u = 0; u < kSpSamplePer; ++u)
    if ((ks[u] >> 21) == c0) atomicAdd(&s_hist2[hpad((ks[u] >> 10) & (kBins - 1))], 1u);
  const uint32_t c1 = sel_select_bin(s_hist2, kBins, rem, s_sel);
  const uint32_t L = (c0 << 21) | (c1 << 10);

  // Keys >= L: this wave's count, then the workgroup's.
  uint64_t mk[kPer];
  uint32_t cnt = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    kv[u] = score_key(__uint_as_float(kv[u]));
    const bool ge = wbase + kWave * u + lane < n && kv[u] >= L;
    mk[u] = __builtin_amdgcn_ballot_w64(ge);
    cnt += (uint32_t)__popcll(mk[u]);
  }
  if (lane == 0) s_cnt[wave] = cnt;
  lds_barrier();
  uint32_t at = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    const uint32_t c = s_cnt[w];
    at += w < wave ? c : 0u;
    total += c;
  }
  constexpr int kRegCap = PickShape<kPer>::kRegCap;
  if (total <= (uint32_t)kRegCap) {
    uint2* reg = ws.list + ((size_t)row * kCutMaxRegions + blk) * kRegCap;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint64_t m = mk[u];
      if ((m >> lane) & 1ull) {
        const uint32_t r = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        reg[at + r] = uint2{kv[u], (uint32_t)(wbase + kWave * u + lane)};
      }
      at += (uint32_t)__popcll(m);
    }
  }
  if (tid == 0) ws.hdr[(size_t)row * kCutMaxRegions + blk] = CutHdr{total, L, 0u, 0u};
}

union PickLds {
  TopkShared full;                 // full_row_topk (the fallback)
  uint2 list[PickShape<kCutPerLong>::kCap];  // the regions' entries, concatenated (position order)
  SelectSharedT<kCutMaxN> sel;     // the selection, once the list is in registers
};

template <int kPer>
__global__ __launch_bounds__(kTkThreads) void topk_pick_kernel(const float* __restrict__ scores,
                                                               const int32_t* __restrict__ end_pos,
                                                               int T, int S_max, int k,
                                                               int32_t* __restrict__ out, CutWs ws) {
  constexpr int kBlk = kTkThreads * kPer;
  constexpr int kSpec = PickShape<kPer>::kSpec;  // entries per thread loaded with the headers
  constexpr int kPickCap = PickShape<kPer>::kCap, kPickEnt = PickShape<kPer>::kEnt;
  constexpr int kRegCap = PickShape<kPer>::kRegCap;
  constexpr uint32_t kHead = 32 * kSpec;  // entries of a region staged by its own 32 threads
  constexpr int kRem = (kRegCap - (int)kHead + kTkThreads - 1) / kTkThreads;
  static_assert(kTkThreads == kCutMaxRegions * 32 && (int)kHead <= kRegCap, "32 threads per region");
  __shared__ __align__(16) PickLds lds;
  __shared__ uint2 s_reg[kCutMaxRegions];  // (first slot, count) of each region
  const int row = blockIdx.x;
  const int n = row_len(end_pos, row, T, S_max);
  if (n <= k) return;  // done by the cut launch
  const float* x = scores + (size_t)row * S_max;
  int32_t* o = out + (size_t)row * k;
  if (n > ws.n_reg * kBlk) {  // longer than max_end_pos promised
    full_row_topk(x, n, k, o, lds.full);
    return;
  }
  const int tid = threadIdx.x;
  const int nr = (n + kBlk - 1) / kBlk;  // regions holding positions of this row
  const CutHdr* hdr = ws.hdr + (size_t)row * kCutMaxRegions;
  const uint2* list = ws.list + (size_t)row * kCutMaxRegions * kRegCap;
  // Thread (w, r) = (tid / 32, tid % 32) copies entries r + 32 j of region w.
  // The first kSpec of them are loaded together with the headers.
  const int w = tid >> 5, r = tid & 31;
  uint2 e[kSpec];
#pragma unroll
  for (int j = 0; j < kSpec; ++j) e[j] = list[(size_t)w * kRegCap + r + 32 * j];
  uint32_t M = 0, ok = 1, P = 0, cw = 0, over = 0;
  const uint32_t L = hdr[0].L;
#pragma unroll
  for (int i = 0; i < kCutMaxRegions; ++i) {
    const CutHdr h = i < nr ? hdr[i] : CutHdr{0u, 0u, 0u, 0u};
    ok &= h.count <= (uint32_t)kRegCap ? 1u : 0u;
    P += i < w ? h.count : 0u;
    cw = i == w ? h.count : cw;
    M += h.count;
    over |= (h.count > kHead ? 1u : 0u) << i;
  }
  if (!ok || M < (uint32_t)k || M > (uint32_t)kPickCap) {
    full_row_topk(x, n, k, o, lds.full);
    return;
  }
  // Stage the list in LDS, in position order: first the entries already
  // loaded, then, region by region, what a region holds beyond its first
  // kHead entries, spread over the whole workgroup (all of a region's loads
  // issued before its stores).
  if (w < nr) {
#pragma unroll
    for (int j = 0; j < kSpec; ++j)
      if ((uint32_t)(r + 32 * j) < cw) lds.list[P + r + 32 * j] = e[j];
  }
  if (over != 0u) {  // uniform
    if (r == 0) s_reg[w] = uint2{P, cw};
    lds_barrier();
    do {
      const int i = __builtin_ctz(over);
      over &= over - 1u;
      const uint2 pc = s_reg[i];
      const uint32_t rem = pc.y - kHead;
      const uint2* src = list + (size_t)i * kRegCap + kHead;
      uint2* dst = lds.list + pc.x + kHead;
      uint2 rv[kRem];
#pragma unroll
      for (int u = 0; u < kRem; ++u) {
        const uint32_t ei = (uint32_t)tid + kTkThreads * u;
        rv[u] = ei < rem ? src[ei] : uint2{0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kRem; ++u) {
        const uint32_t ei = (uint32_t)tid + kTkThreads * u;
        if (ei < rem) dst[ei] = rv[u];
      }
    } while (over != 0u);
  }
  lds_barrier();
  // Thread tid takes entries 8 tid .. 8 tid + 7 of the position-ordered list,
  // so the winners' slots come from one scan of per-thread counts.
  BlockedCandidates<kTkThreads, kPickEnt> cand;
  cand.M = (int)M;
#pragma unroll
  for (int u = 0; u < kPickEnt; ++u) cand.d[u] = cand.p[u] = 0u;
  if (kPickEnt * tid < (int)M) {
    const uint4* src = reinterpret_cast<const uint4*>(lds.list + kPickEnt * tid);
#pragma unroll
    for (int u = 0; u < kPickEnt / 2; ++u) {
      const uint4 v = src[u];
      cand.d[2 * u] = v.x - L;
      cand.p[2 * u] = v.y;
      cand.d[2 * u + 1] = v.z - L;
      cand.p[2 * u + 1] = v.w;
    }
  }
  lds_barrier();  // the selection's LDS overlaps the staged list
  ordered_select(cand, k, o, lds.sel);
}

__global__ __launch_bounds__(256) void topk_reset_kernel(uint32_t* __restrict__ ctr, int words) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < words) ctr[i] = 0u;
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
// groups w, w+8, w+16, ... (one coalesced 256-byte load each).
//   1. A cut L below the k-th largest key: a histogram of the top 11 key bits
//      over every position (rows up to 8192) or over every 4th group of each
//      wave (longer rows, a quarter of the row in blocks of 512), and the bin
//      where the count from the top reaches k (scaled to the sample, plus a
//      margin of four standard deviations) gives L.
//   2. One pass over the registers appends every key >= L with its position
//      to the wave's own region of an LDS list (typically 1.2-2 k entries).
//   3. If the list holds at least k keys, the k-th largest is among them: three
//      radix rounds over the list (the last one a direct rank when few keys
//      are left) give the threshold and need_eq; list entries above it go to a
//      winner bitmap, those equal to it to a tie bitmap.
//   4. Ordered output from the two bitmaps, staged in LDS and stored with
//      coalesced writes.
// Too short a list (the sample misjudged the row) or an overflowing region
// sends the row to full_row_topk.
constexpr int kLeanMaxN = kChunk;                          // 32768
constexpr int kLeanExactN = 8192;                          // histogram every position up to here
constexpr int kLeanSample = 4;                             // else every 4th group

// kMaxN = 32768, or 8192 when S_max <= 8192 (prefill of up to 8192 tokens):
// then every row takes the exact histogram, no wave region can overflow
// (region = the wave's 1024 positions) and the list always holds k keys, so
// full_row_topk and its LDS are never needed, and the lighter registers and
// LDS let two workgroups share a CU.
template <int kMaxN>
struct LeanSharedT {
  static constexpr int kCap = kMaxN > kLeanExactN ? 16384 : kMaxN;  // keys >= L per row
  static constexpr int kRegion = kCap / kTkWaves;                  // per wave
  uint32_t hist[kHistWords];   // round 0 (the sample), then round 1, then round 3
  uint32_t hist2[kHistWords];  // round 2
  uint32_t ck[kCap];           // keys >= L; wave w's at [kRegion w, kRegion w + ncw[w])
  uint16_t cp[kCap];           // their positions
  uint32_t sure[kMaxN / 32];
  uint32_t eq[kMaxN / 32];
  uint32_t pre[kMaxN / 32];    // per-word prefixes of sure / eq (bitmap_prefixes)
  uint32_t ncw[kTkWaves];
  uint32_t wave[2 * kTkWaves];
  uint32_t sel[2];
  alignas(16) uint32_t small[kWave];
  uint32_t nsmall;
};

template <int kMaxN>
union LeanLdsFull {
  TopkShared full;
  LeanSharedT<kMaxN> lean;
};
template <int kMaxN>
struct LeanLdsOnly {
  LeanSharedT<kMaxN> lean;
};
template <int kMaxN>
using LeanLds = typename std::conditional<(kMaxN > kLeanExactN), LeanLdsFull<kMaxN>,
                                          LeanLdsOnly<kMaxN>>::type;

template <int kMaxN>
__global__ __launch_bounds__(kTkThreads, kMaxN > kLeanExactN ? 1 : 4) void topk_lean_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, int32_t* __restrict__ out) {
  constexpr int kLeanGroups = kMaxN / kWave / kTkWaves;  // 64-position groups per wave
  constexpr int kLeanRegion = LeanSharedT<kMaxN>::kRegion;
  static_assert(kLeanGroups * kWave * kTkWaves == kMaxN, "row fits the registers");
  static_assert(kMaxN > kLeanExactN || kLeanRegion >= kLeanGroups * kWave,
                "a wave's keys always fit its region");
  __shared__ __align__(16) LeanLds<kMaxN> lds;
  LeanSharedT<kMaxN>& sh = lds.lean;
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
  bool ok = n <= kMaxN;
  if (ok) {
    // Group i of this wave holds positions 64 (8 i + wave) + lane.
    uint32_t key[kLeanGroups];
#pragma unroll
    for (int i = 0; i < kLeanGroups; ++i)
      key[i] = __float_as_uint(x[min(kWave * (kTkWaves * i + wave) + lane, n - 1)]);
    for (int i = tid; i < kHistWords; i += kTkThreads) {
      sh.hist[i] = 0;
      sh.hist2[i] = 0;
    }
    for (int i = tid; i < kMaxN / 32; i += kTkThreads) {
      sh.sure[i] = 0;
      sh.eq[i] = 0;
    }
    if (tid == 0) sh.nsmall = 0;
    lds_barrier();

    // 1. Histogram of all positions, or of the sample, and the cut L.
    const bool exact = n <= kLeanExactN;
#pragma unroll
    for (int i = 0; i < kLeanGroups; ++i) {
      key[i] = score_key(__uint_as_float(key[i]));
      const int base = kWave * (kTkWaves * i + wave);
      if (base < n && (exact || i % kLeanSample == 0))
        atomicAdd(&sh.hist[hpad(key[i] >> 21)], lane < n - base ? 1u : 0u);
    }
    lds_barrier();
    if (wave == 0) {
      // Lane l sums bins 2047-32l down to 2016-32l; the scan gives the count
      // above each of them.
      uint32_t c[32], sum = 0;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        c[u] = sh.hist[hpad((uint32_t)(kBins - 1 - (32 * lane + u)))];
        sum += c[u];
      }
      const uint32_t incl = wave_incl_scan(sum);
      const uint32_t ns = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);  // counted keys
      uint32_t target = (uint32_t)k;
      if (!exact) {
        const float mean = (float)k * (float)ns / (float)n;
        target = min(ns, (uint32_t)(mean + 4.0f * sqrtf(mean) + 16.0f));
      }
      uint32_t above = incl - sum, bin = 0;
      bool found = false;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        if (!found && above + c[u] >= target) {
          bin = (uint32_t)(kBins - 1 - (32 * lane + u));
          found = true;
        }
        above += c[u];
      }
      // The highest bin where the count from the top reaches the target.
      const uint64_t who = __builtin_amdgcn_ballot_w64(found);
      const int src = who ? (int)__ffsll((long long)who) - 1 : 0;
      bin = who ? (uint32_t)__builtin_amdgcn_readlane((int)bin, src) : 0u;
      if (lane == 0) sh.sel[0] = bin << 21;
    }
    lds_barrier();
    const uint32_t L = sh.sel[0];
    for (int i = tid; i < kHistWords; i += kTkThreads) sh.hist[i] = 0;  // round 1

    // 2. Keys >= L -> the wave's region.
    uint32_t nc = 0;
    const int region = wave * kLeanRegion;
#pragma unroll
    for (int i = 0; i < kLeanGroups; ++i) {
      const int base = kWave * (kTkWaves * i + wave);
      if (base < n) {
        const bool ge = lane < n - base && key[i] >= L;
        const uint64_t m = __builtin_amdgcn_ballot_w64(ge);
        const uint32_t at = nc + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (ge && at < (uint32_t)kLeanRegion) {
          sh.ck[region + at] = key[i];
          sh.cp[region + at] = (uint16_t)(base + lane);
        }
        nc += (uint32_t)__popcll(m);
      }
    }
    if (lane == 0) sh.ncw[wave] = nc;
    lds_barrier();
    uint32_t M = 0, over = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w) {
      const uint32_t c = sh.ncw[w];
      M += c;
      over |= c > (uint32_t)kLeanRegion ? 1u : 0u;
    }
    ok = over == 0 && M >= (uint32_t)k;
    if (ok) {
      // 3. Exact selection over the list.  Round 1: bits 21..31.
      const int my_nc = (int)nc;
      for (int j = lane; j < my_nc; j += kWave)
        atomicAdd(&sh.hist[hpad(sh.ck[region + j] >> 21)], 1u);
      uint32_t remaining = (uint32_t)k;
      const uint32_t d0 = sel_select_bin(sh.hist, kBins, remaining, sh.sel);
      // Round 2: bits 10..20 of the keys in bin d0.
      for (int j = lane; j < my_nc; j += kWave) {
        const uint32_t kk = sh.ck[region + j];
        if ((kk >> 21) == d0) atomicAdd(&sh.hist2[hpad((kk >> 10) & (kBins - 1))], 1u);
      }
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
          const uint64_t who = __builtin_amdgcn_ballot_w64(hit);
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
        // Round 3: the last 10 bits.
        for (int i = tid; i < kHistWords; i += kTkThreads) sh.hist[i] = 0;
        lds_barrier();
        for (int j = lane; j < my_nc; j += kWave) {
          const uint32_t kk = sh.ck[region + j];
          if ((kk >> 10) == pre) atomicAdd(&sh.hist[hpad(kk & 1023u)], 1u);
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
      // 4. Ordered output: each winner writes its position at its rank.
      bitmap_prefixes<kTkThreads, kMaxN / 32>(sh.sure, sh.eq, sh.pre, (n + 31) >> 5, sh.wave);
      lds_barrier();
      for (int j = lane; j < my_nc; j += kWave) {
        const uint32_t kk = sh.ck[region + j], p = sh.cp[region + j];
        if (kk >= thr) {
          const int at = winner_slot(sh.sure, sh.eq, sh.pre, p, kk > thr, need_eq);
          if (at >= 0 && at < k) o[at] = (int32_t)p;
        }
      }
    }
  }
  if constexpr (kMaxN > kLeanExactN) {
    if (!ok) {
      __syncthreads();  // the list checks' reads are done before the LDS is reused
      full_row_topk(x, n, k, o, lds.full);
    }
  }
}

size_t topk_workspace_bytes(int B, int T, int S_max, int) {
  const size_t rows = (size_t)B * T;
  if (rows > (size_t)kMultiRows) return 0;
  const size_t split = align256(rows * kCtrWords * 4) + rows * kSpCap * 8;
  if (S_max <= kSplitThreads * kSpPerShort) return split;
  return max(split, cut_ws_bytes((int)rows));
}

uint32_t* topk_counters(void* workspace, int B, int T, int max_end_pos) {
  const int rows = B * T;
  if (rows > kMultiRows || cut_path(rows, max_end_pos)) return nullptr;
  return reinterpret_cast<uint32_t*>(workspace);
}

static_assert(kTkThreads * 4 == kBins, "one 16-byte histogram piece per thread");

int launch_topk(const float* scores, const int32_t* end_pos, int B, int T, int S_max,
                int max_end_pos, int k, int32_t* out, void* workspace, bool counters_clear,
                hipStream_t stream) {
  const int rows = B * T;
  if (cut_path(rows, max_end_pos)) {
    const CutWs ws = carve_cut_ws(workspace, rows, max_end_pos);
    const dim3 grid((unsigned)((long)rows * ws.n_reg)), block(kTkThreads);
    if (cut_per(max_end_pos) == kCutPer) {
      hipLaunchKernelGGL(topk_cut_kernel<kCutPer>, grid, block, 0, stream, scores, end_pos, T,
                         S_max, k, out, ws);
      if (hipGetLastError() != hipSuccess) return -5;
      hipLaunchKernelGGL(topk_pick_kernel<kCutPer>, dim3((unsigned)rows), block, 0, stream,
                         scores, end_pos, T, S_max, k, out, ws);
    } else {
      hipLaunchKernelGGL(topk_cut_kernel<kCutPerLong>, grid, block, 0, stream, scores, end_pos, T,
                         S_max, k, out, ws);
      if (hipGetLastError() != hipSuccess) return -5;
      hipLaunchKernelGGL(topk_pick_kernel<kCutPerLong>, dim3((unsigned)rows), block, 0, stream,
                         scores, end_pos, T, S_max, k, out, ws);
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  if (rows <= kMultiRows) {
    const SplitWs ws = carve_split_ws(workspace, rows, max_end_pos);
    if (!counters_clear && ws.n_blk > 1) {  // the lists are only used with several workgroups
      hipLaunchKernelGGL(topk_reset_kernel, dim3((unsigned)((kCtrWords * rows + 255) / 256)),
                         dim3(256), 0, stream, ws.ctr, kCtrWords * rows);
      if (hipGetLastError() != hipSuccess) return -5;
    }
    const dim3 grid((unsigned)((long)rows * ws.n_blk));
    // The cut path takes every row count here with max_end_pos in 4097..131072,
    // so this path sees max_end_pos <= 4096 (8 positions a thread, one
    // workgroup per row) or above 131072 (16 a thread, several workgroups).
    // With one workgroup per row the first launch selects every row itself
    // (or sends it to full_row_topk): no list, no second launch.
    if (ws.n_blk == 1) {
      hipLaunchKernelGGL((topk_split_kernel<kSpPerShort, true>), grid, dim3(kTkThreads), 0,
                         stream, scores, end_pos, T, S_max, k, out, ws);
      return hipGetLastError() == hipSuccess ? 0 : -5;
    }
    hipLaunchKernelGGL((topk_split_kernel<kSpPerLong, false>), grid, dim3(kTkThreads), 0,
                       stream, scores, end_pos, T, S_max, k, out, ws);
    if (hipGetLastError() != hipSuccess) return -5;
    hipLaunchKernelGGL(topk_finish_kernel<kSpPerLong>, dim3((unsigned)rows), dim3(kTkThreads),
                       0, stream, scores, end_pos, T, S_max, k, out, ws);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  if (S_max <= kLeanExactN) {  // every row is at most 8192 long
    hipLaunchKernelGGL(topk_lean_kernel<kLeanExactN>, dim3((unsigned)rows), dim3(kTkThreads), 0,
                       stream, scores, end_pos, T, S_max, k, out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  if (max_end_pos <= kLeanMaxN) {
    hipLaunchKernelGGL(topk_lean_kernel<kLeanMaxN>, dim3((unsigned)rows), dim3(kTkThreads), 0,
                       stream, scores, end_pos, T, S_max, k, out);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, stream, scores,
                     end_pos, T, S_max, k, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace dsa
