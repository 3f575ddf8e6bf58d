// In-workgroup exact top-k selection over an explicit candidate set: the part
// of "DeepSeek-V3.2-Exp - Keep top-k positions" (topk(min(index_topk,
// end_pos)) of Indexer.forward) that runs after the candidates are known (the
// split top-k's finishing launch, and the workgroups that select a whole row
// held in registers), with the split top-k's workspace layout.
//
// Keys are order-preserving 32-bit images of the scores (score_key).  The
// candidates are handed over as D = key - L, all >= 0, with L a lower bound of
// every candidate key.  Radix rounds over D (11 bits, then 11, then the rest,
// or a direct rank once at most 64 keys are left) give the threshold D value
// thr of the k-th largest candidate and the number need_eq of candidates equal
// to it that are kept.  Two position bitmaps, `sure` (D > thr) and `eq`
// (D == thr), and per-word prefix counts of both then give every winner its
// slot in the output row: ascending positions, ties to the smaller position.
#pragma once
#include "dsa_device.h"

namespace dsa {

constexpr int kBins = 2048;
constexpr int kHistWords = kBins + kBins / 32;
constexpr int kMaxK = 2048;

// Histogram bins are stored with one pad word per 32 so that a lane reading
// 32 consecutive bins (the bin search) does not collide with other lanes.
__device__ __forceinline__ int hpad(uint32_t bin) { return (int)(bin + (bin >> 5)); }

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active): sums
// within rows of 16 lanes by DPP row shifts, then the row totals are carried
// over with row broadcasts (lane 15 into row 1 and 3, lane 31 into rows 2, 3).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Maximum over the 64 lanes of a wave (all lanes active), in every lane:
// the scan pattern of wave_incl_scan with max, read back from lane 63.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Exclusive prefix sums over the workgroup (kWaves waves) of two per-thread
// values, plus totals.  s_wave holds 2 * kWaves words.  kLdsOnly: the barrier
// is an LDS-only one (global accesses in flight stay in flight) and there is
// no trailing barrier, for callers that synchronise before s_wave is written
// again.
template <bool kLdsOnly = false, int kWaves = 8>
__device__ __forceinline__ void block_exclusive_scan2(uint32_t a, uint32_t b, uint32_t* s_wave,
                                                      uint32_t& ex_a, uint32_t& ex_b,
                                                      uint32_t& tot_a, uint32_t& tot_b) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ia = wave_incl_scan(a), ib = wave_incl_scan(b);
  if (lane == 63) {
    s_wave[wave] = ia;
    s_wave[kWaves + wave] = ib;
  }
  if constexpr (kLdsOnly) lds_barrier();
  else __syncthreads();
  uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t va = s_wave[w], vb = s_wave[kWaves + w];
    pa += w < wave ? va : 0u;
    pb += w < wave ? vb : 0u;
    sa += va;
    sb += vb;
  }
  if constexpr (!kLdsOnly) __syncthreads();
  ex_a = pa + ia - a;
  ex_b = pb + ib - b;
  tot_a = sa;
  tot_b = sb;
}

// One wave finds the bin holding the `remaining`-th largest counted element
// (counting from the top bin down): returns its digit and the count of
// elements in higher bins.  Lane l owns the kNB/64 bins just below those of
// lane l-1 (they share one pad offset, so a lane reads them at fixed offsets
// from one address, and consecutive lanes hit different banks).  The crossing
// lane comes from the scan of the per-lane sums; then its bins are scanned
// with one bin per lane.  All 64 lanes must be active.  With no crossing (an
// inconsistent histogram) the digit is meaningless but in range.
template <int kNB, bool kPadded>
__device__ __forceinline__ void wave_select_bin_t(const uint32_t* hist, uint32_t remaining,
                                                  uint32_t& digit, uint32_t& above_out) {
  constexpr int kPer = kNB / kWave;  // 32 or 16
  const int lane = threadIdx.x & 63;
  auto lane_bins = [&](int l) {
    const int low = kNB - kPer * (l + 1);  // lowest bin of lane l
    return hist + (kPadded ? low + (low >> 5) : low);
  };
  const uint32_t* hb = lane_bins(lane);
  uint32_t sum = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) sum += hb[u];
  const uint32_t incl = wave_incl_scan(sum);
  const uint32_t excl = incl - sum;
  const uint64_t who = __builtin_amdgcn_ballot_w64(excl < remaining && remaining <= incl);
  const int src = who ? (int)__ffsll((long long)who) - 1 : 0;
  const uint32_t above_src = (uint32_t)__builtin_amdgcn_readlane((int)excl, src);
  // Lane j < kPer takes bin (top bin of lane src) - j.
  const uint32_t v = lane_bins(src)[kPer - 1 - min(lane, kPer - 1)];
  const uint32_t cj = lane < kPer ? v : 0u;
  const uint32_t incl2 = wave_incl_scan(cj) + above_src;
  const uint32_t excl2 = incl2 - cj;
  const uint64_t who2 =
      __builtin_amdgcn_ballot_w64(lane < kPer && excl2 < remaining && remaining <= incl2);
  const int j = who2 ? (int)__ffsll((long long)who2) - 1 : 0;
  digit = (uint32_t)(kNB - 1 - kPer * src - j);
  above_out = (uint32_t)__builtin_amdgcn_readlane((int)excl2, j);
}

template <bool kPadded = true>
__device__ __forceinline__ void wave_select_bin(const uint32_t* hist, int nbins,
                                                uint32_t remaining, uint32_t& digit,
                                                uint32_t& above_out) {
  if (nbins == kBins) wave_select_bin_t<kBins, kPadded>(hist, remaining, digit, above_out);
  else wave_select_bin_t<kBins / 2, kPadded>(hist, remaining, digit, above_out);
}

// Row length of query row `row` = b*T + t: positions 0 .. end_pos[b]-T+t
// (end_pos clamped to [T, S_max]).
__device__ __forceinline__ int row_len(const int32_t* end_pos, int row, int T, int S_max) {
  const int b = row / T, t = row - b * T;
  const int ep = min(max(end_pos[b], T), S_max);
  return ep - T + t + 1;
}

// Wave 0 searches the histogram, everyone receives the digit (LDS-only
// barriers: global loads in flight stay in flight).
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

// The few keys (at most 64) left after a round, gathered in s_small: one wave
// ranks them and publishes the `remaining`-th largest (thr) and how many keys
// equal to it are kept (need_eq).
__device__ __forceinline__ void rank_small(const uint32_t* s_small, uint32_t m,
                                           uint32_t remaining, uint32_t* s_sel) {
  const int lane = threadIdx.x & 63;
  const bool valid = lane < (int)m;
  const uint32_t mine = s_small[min(lane, (int)m - 1)];
  // Only the m gathered keys are compared (m is uniform and usually a handful:
  // a single wave pays the full latency of every instruction, so a loop over
  // all 64 slots cost more than the rest of the selection), four per 16-byte
  // broadcast read, with four counters per relation.
  const uint4* s4 = reinterpret_cast<const uint4*>(s_small);
  uint32_t gt4[4] = {0u, 0u, 0u, 0u}, ge4[4] = {0u, 0u, 0u, 0u};
  const int groups = ((int)m + 3) >> 2;
  for (int q = 0; q < groups; ++q) {
    const uint4 o4 = s4[q];
    const uint32_t other[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = 4 * q + i < (int)m;
      gt4[i] += in && other[i] > mine ? 1u : 0u;
      ge4[i] += in && other[i] >= mine ? 1u : 0u;
    }
  }
  const uint32_t gt = (gt4[0] + gt4[1]) + (gt4[2] + gt4[3]);
  const uint32_t ge = (ge4[0] + ge4[1]) + (ge4[2] + ge4[3]);
  // Fewer than `remaining` keys above it, at least `remaining` at or above it.
  const bool hit = valid && gt < remaining && remaining <= ge;
  const uint64_t who = __builtin_amdgcn_ballot_w64(hit);
  const int src = who ? (int)__ffsll((long long)who) - 1 : 0;
  const uint32_t t_key = (uint32_t)__builtin_amdgcn_readlane((int)mine, src);
  const uint32_t t_gt = (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
  if (lane == 0) {
    s_sel[0] = t_key;
    s_sel[1] = remaining - t_gt;
  }
}

// Ordered output from the two position bitmaps (winners strictly above the
// threshold in `sure`, keys equal to it in `eq`, of which the need_eq
// smallest positions are kept).  bitmap_prefixes stores, per 32-position
// word, the number of set `sure` bits before the word (bits 0..15) and of
// set `eq` bits before it (bits 16..31), each capped at 65535 (both are only
// compared with k <= 2048); thread t owns a run of consecutive words.  The
// caller synchronises before reading `pre`.  A winner then finds its output
// slot from three LDS words, with no loop over set bits.
template <int kThreads, int kMaxWords>
__device__ __forceinline__ void bitmap_prefixes(const uint32_t* sure, const uint32_t* eq,
                                                uint32_t* pre, int nwords, uint32_t* s_wave) {
  // A thread's words are read once into registers: the second pass would
  // otherwise read them again behind its own stores to `pre`, one LDS round
  // trip per word.
  constexpr int kWpt = (kMaxWords + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  const int wpt = (nwords + kThreads - 1) / kThreads;
  const int w0 = min(tid * wpt, nwords), w1 = min(w0 + wpt, nwords);
  uint32_t cs[kWpt], ce[kWpt];
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < kWpt; ++i) {
    const bool in = w0 + i < w1;
    cs[i] = in ? (uint32_t)__popc(sure[w0 + i]) : 0u;
    ce[i] = in ? (uint32_t)__popc(eq[w0 + i]) : 0u;
    n_gt += cs[i];
    n_eq += ce[i];
  }
  uint32_t gt, eqb, tot_gt, tot_eq;
  block_exclusive_scan2<true, kThreads / kWave>(n_gt, n_eq, s_wave, gt, eqb, tot_gt, tot_eq);
#pragma unroll
  for (int i = 0; i < kWpt; ++i) {
    if (w0 + i < w1) pre[w0 + i] = min(gt, 0xFFFFu) | (min(eqb, 0xFFFFu) << 16);
    gt += cs[i];
    eqb += ce[i];
  }
}

// Output slot of position p (marked in `sure` when above the threshold, else
// in `eq`), or -1 when p is an equal key beyond the first need_eq.
__device__ __forceinline__ int winner_slot(const uint32_t* sure, const uint32_t* eq,
                                           const uint32_t* pre, uint32_t p, bool above,
                                           uint32_t need_eq) {
  const uint32_t w = p >> 5, below = (1u << (p & 31)) - 1u;
  const uint32_t pw = pre[w];
  const uint32_t n_gt = (pw & 0xFFFFu) + (uint32_t)__popc(sure[w] & below);
  const uint32_t n_eq = (pw >> 16) + (uint32_t)__popc(eq[w] & below);
  if (above) return (int)(n_gt + min(n_eq, need_eq));
  return n_eq < need_eq ? (int)(n_gt + n_eq) : -1;
}

// ---------------------------------------------------------------------------
// Workspace of the split top-k (up to kMultiRows query rows): per row a few
// counters and a list of (key, position) candidates.  Each row is spread over
// workgroups of kSplitThreads * per-thread positions; every one of them
// derives the same cut L from a sample of the row and appends its keys >= L
// to the row's list.
constexpr int kMultiRows = 1024;
constexpr int kSplitThreads = 512;
constexpr int kSpPerShort = 8;      // positions per thread, rows <= kSpShortMax
constexpr int kSpPerLong = 16;      // longer rows (fewer workgroups per row)
constexpr int kSpShortMax = 32768;
constexpr int kSpCap = 8192;        // list entries per row
constexpr int kSpMaxN = 131072;     // longest row the bitmaps cover
constexpr int kCtrWords = 4;        // per row: unused, list length, cut L, unused

struct SplitWs {
  uint32_t* ctr;  // [rows][kCtrWords]
  uint2* list;    // [rows][kSpCap]: (key, position) of the keys >= L
  int n_blk;      // workgroups per row
  int blk_pos;    // positions per workgroup
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__host__ inline int split_per_thread(int max_end_pos) {
  return max_end_pos <= kSpShortMax ? kSpPerShort : kSpPerLong;
}

// Workgroups per row of the split top-k for rows of at most max_end_pos positions.
__host__ inline int split_blocks(int max_end_pos) {
  const int blk = kSplitThreads * split_per_thread(max_end_pos);
  return max(1, (max_end_pos + blk - 1) / blk);
}

__host__ inline SplitWs carve_split_ws(void* ws, int rows, int max_end_pos) {
  SplitWs w;
  char* p = reinterpret_cast<char*>(ws);
  w.ctr = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)rows * kCtrWords * 4);
  w.list = reinterpret_cast<uint2*>(p);
  w.blk_pos = kSplitThreads * split_per_thread(max_end_pos);
  w.n_blk = split_blocks(max_end_pos);
  return w;
}

// A row whose selection is finished from its candidate list (the others are
// selected completely by the first launch: rows with at most k positions,
// rows that fit one workgroup, rows longer than max_end_pos promised).
__device__ __forceinline__ bool row_uses_list(int n, int k, const SplitWs& ws) {
  return n > k && n > ws.blk_pos && n <= ws.n_blk * ws.blk_pos;
}

// LDS of a selection over rows of at most kMaxN positions.
template <int kMaxN>
struct SelectSharedT {
  static constexpr int kMaxPositions = kMaxN;
  uint32_t hist[kHistWords];
  uint32_t hist2[kHistWords];
  uint32_t sure[kMaxN / 32];
  uint32_t eq[kMaxN / 32];
  uint32_t pre[kMaxN / 32];  // per-word prefixes of sure / eq (bitmap_prefixes)
  uint32_t wave[2 * 16];
  uint32_t sel[2];
  alignas(16) uint32_t small[kWave];
  uint32_t nsmall;
};
using SelectShared = SelectSharedT<kSpMaxN>;

// Candidates held in registers: entry tid + kThreads*u is (d[u], p[u]) for
// every tid + kThreads*u < M.
template <int kThreads, int kEnt>
struct RegCandidates {
  uint32_t d[kEnt], p[kEnt];
  int M;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
#pragma unroll
    for (int u = 0; u < kEnt; ++u) {
      if (kThreads * u >= M) break;  // uniform: no thread has slot u or later
      if ((int)threadIdx.x + kThreads * u < M) f(d[u], p[u]);
    }
  }
  // f(d, p, valid) for every slot some thread holds, with no branch on the
  // lane's own slot (so the LDS operations of successive slots are issued
  // together rather than each behind its own branch); the entries of
  // invalid slots are other candidates' and must not be counted.
  template <class F>
  __device__ __forceinline__ void each_all(F&& f) const {
#pragma unroll
    for (int u = 0; u < kEnt; ++u) {
      if (kThreads * u >= M) break;  // uniform
      f(d[u], p[u], (int)threadIdx.x + kThreads * u < M);
    }
  }
};

// Candidates held in registers in list order: thread tid holds entries
// kEnt*tid .. kEnt*tid + kEnt - 1 (those below M are valid).
template <int kThreads, int kEnt>
struct BlockedCandidates {
  uint32_t d[kEnt], p[kEnt];
  int M;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    const int first = kEnt * (int)threadIdx.x;
    if (first >= M) return;
#pragma unroll
    for (int u = 0; u < kEnt; ++u)
      if (first + u < M) f(d[u], p[u]);
  }
  template <class F>
  __device__ __forceinline__ void each_all(F&& f) const {
    const int first = kEnt * (int)threadIdx.x;
    if (first >= M) return;  // whole waves past the list skip
#pragma unroll
    for (int u = 0; u < kEnt; ++u) f(d[u], p[u], first + u < M);
  }
};

// Threshold of the k largest among the candidates (at least k of them), by a
// workgroup of kThreads threads: the D value thr of the k-th largest and the
// number need_eq of candidates equal to it that are kept (the others equal to
// it are dropped, the larger positions first).  dmax is an upper bound of
// every D when known (known_dmax), else the rounds find the largest D first.
// Ends with the workgroup synchronised on LDS.
template <int kThreads, class Cand, class Sh>
__device__ __forceinline__ void block_threshold(const Cand& cand, int k, Sh& sh, bool known_dmax,
                                                uint32_t dmax, uint32_t& thr,
                                                uint32_t& need_eq) {
  constexpr int kWaves = kThreads / kWave;
  static_assert(kThreads % kWave == 0 && kWaves <= 16, "up to 16 waves");
  const int tid = threadIdx.x;
  for (int i = tid; i < kHistWords; i += kThreads) {
    sh.hist[i] = 0;
    sh.hist2[i] = 0;
  }
  if (tid == 0) sh.nsmall = 0;
  // The rounds work on D, whose range is known from the largest one, so the
  // first digit spreads the keys over the histogram instead of piling them
  // into the few top-bit bins they share.
  uint32_t mx = dmax;
  if (!known_dmax) {
    mx = 0;
    cand.each_all([&](uint32_t d, uint32_t, bool v) { mx = max(mx, v ? d : 0u); });
    mx = wave_max(mx);
    if ((tid & 63) == 0) sh.wave[tid >> 6] = mx;
  }
  lds_barrier();  // also orders the clearing above before the rounds
  if (!known_dmax) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = max(mx, sh.wave[w]);
  }
  const int bits = 32 - __clz((int)mx);      // D < 2^bits
  const int s1 = bits > 11 ? bits - 11 : 0;  // round 1: D >> s1 (< 2048)
  const int s2 = s1 > 11 ? s1 - 11 : 0;      // round 2: bits s2.. of D
  // Round 1.
  cand.each_all([&](uint32_t d, uint32_t, bool v) {
    atomicAdd(&sh.hist[hpad(min(d >> s1, (uint32_t)kBins - 1u))], v ? 1u : 0u);
  });
  uint32_t remaining = (uint32_t)k;
  const uint32_t d1 = sel_select_bin(sh.hist, kBins, remaining, sh.sel);
  const uint32_t m1 = sh.hist[hpad(d1)];  // keys left in the running
  // The keys whose D >> shift equals pre are gathered and ranked directly.
  auto rank_direct = [&](int shift, uint32_t pre, uint32_t m) {
    // One LDS atomic per thread that holds any of the few matching keys.
    uint32_t cnt = 0;
    cand.each_all([&](uint32_t d, uint32_t, bool v) { cnt += v && (d >> shift) == pre ? 1u : 0u; });
    if (cnt != 0) {
      uint32_t at = atomicAdd(&sh.nsmall, cnt);
      cand.each_all([&](uint32_t d, uint32_t, bool v) {
        if (v && (d >> shift) == pre) sh.small[min(at++, (uint32_t)kWave - 1u)] = d;
      });
    }
    lds_barrier();
    if (tid < kWave) rank_small(sh.small, m, remaining, sh.sel);
    lds_barrier();
    thr = sh.sel[0];
    need_eq = sh.sel[1];
  };
  if (s1 == 0) {
    thr = d1;
    need_eq = remaining;
  } else if (m1 <= (uint32_t)kWave) {
    rank_direct(s1, d1, m1);
  } else {
    // Round 2: bits s2 .. s1-1 of D (with the constant bits above when the
    // span is shorter than 11).
    cand.each([&](uint32_t d, uint32_t) {
      if ((d >> s1) == d1) atomicAdd(&sh.hist2[hpad((d >> s2) & (kBins - 1))], 1u);
    });
    const uint32_t d2 = sel_select_bin(sh.hist2, kBins, remaining, sh.sel);
    const uint32_t m2 = sh.hist2[hpad(d2)];
    const uint32_t low = (1u << (s1 - s2)) - 1u;
    const uint32_t p2 = (d1 << (s1 - s2)) | (d2 & low);  // D >> s2 of the survivors
    if (s2 == 0) {
      thr = p2;
      need_eq = remaining;
    } else if (m2 <= (uint32_t)kWave) {
      rank_direct(s2, p2, m2);
    } else {
      // Round 3: the last s2 (<= 10) bits.
      for (int i = tid; i < kHistWords; i += kThreads) sh.hist[i] = 0;
      lds_barrier();
      cand.each([&](uint32_t d, uint32_t) {
        if ((d >> s2) == p2) atomicAdd(&sh.hist[hpad(d & ((1u << s2) - 1u))], 1u);
      });
      const uint32_t d3 = sel_select_bin(sh.hist, 1024, remaining, sh.sel);
      thr = (p2 << s2) | d3;
      need_eq = remaining;
    }
  }
}

// Exact selection of the k largest among the candidates (at least k of them,
// positions < n <= Sh::kMaxPositions), by a workgroup of kThreads threads.  Returns the
// threshold D value and need_eq; on return the bitmaps and their prefixes are
// complete (the workgroup is synchronised), so that
//   winner_slot(sh.sure, sh.eq, sh.pre, p, d > thr, need_eq)
// gives the output slot of every candidate (d, p) with d >= thr.
template <int kThreads, class Cand, class Sh>
__device__ __forceinline__ void block_select(const Cand& cand, int n, int k, Sh& sh,
                                             uint32_t& thr, uint32_t& need_eq) {
  const int tid = threadIdx.x;
  const int nwords = (n + 31) >> 5;
  for (int i = tid; i < nwords; i += kThreads) {
    sh.sure[i] = 0;
    sh.eq[i] = 0;
  }
  block_threshold<kThreads>(cand, k, sh, false, 0u, thr, need_eq);
  const uint32_t t = thr;
  cand.each([&](uint32_t d, uint32_t p) {
    if (d > t) atomicOr(&sh.sure[p >> 5], 1u << (p & 31));
    else if (d == t) atomicOr(&sh.eq[p >> 5], 1u << (p & 31));
  });
  lds_barrier();
  bitmap_prefixes<kThreads, Sh::kMaxPositions / 32>(sh.sure, sh.eq, sh.pre, nwords, sh.wave);
  lds_barrier();
}

// Exact selection of the k largest among M >= k candidates that are held in
// position order (BlockedCandidates: thread tid holds list entries kEnt*tid
// ..), all with D >= 0.  A winner's output slot is the number of winners
// before it in the list, so one block scan of two per-thread counts (keys
// above the threshold, keys equal to it) replaces the position bitmaps: the
// slot of an entry above is gt_before + min(eq_before, need_eq), an equal
// entry is kept when eq_before < need_eq, at slot gt_before + eq_before.
template <int kThreads, int kEnt, class Sh>
__device__ __forceinline__ void ordered_select(const BlockedCandidates<kThreads, kEnt>& cand,
                                               int k, int32_t* __restrict__ o, Sh& sh) {
  uint32_t thr, need_eq;
  block_threshold<kThreads>(cand, k, sh, false, 0u, thr, need_eq);
  const int first = kEnt * (int)threadIdx.x;
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int u = 0; u < kEnt; ++u) {
    const bool v = first + u < cand.M;
    n_gt += v && cand.d[u] > thr ? 1u : 0u;
    n_eq += v && cand.d[u] == thr ? 1u : 0u;
  }
  uint32_t gt, eq, tot_gt, tot_eq;
  block_exclusive_scan2<true, kThreads / kWave>(n_gt, n_eq, sh.wave, gt, eq, tot_gt, tot_eq);
  if (n_gt + n_eq == 0) return;
#pragma unroll
  for (int u = 0; u < kEnt; ++u) {
    if (first + u >= cand.M) break;
    const uint32_t d = cand.d[u];
    if (d > thr) {
      const uint32_t at = gt + min(eq, need_eq);
      if (at < (uint32_t)k) o[at] = (int32_t)cand.p[u];
      ++gt;
    } else if (d == thr) {
      if (eq < need_eq && gt + eq < (uint32_t)k) o[gt + eq] = (int32_t)cand.p[u];
      ++eq;
    }
  }
}

}  // namespace dsa
