// Absorbed-MLA attention over gathered cached rows on gfx950 (the MQA decode
// branch of "DeepSeek-V3.2-Exp - Apply sparse mask", restricted to the rows the
// indexer selected; the dense variant takes every causally valid row).
//
//   z[h,j] = (q_nope[h,:] . kv[pos_j,:] + q_pe[h,:] . pe[pos_j,:]) * softmax_scale
//   out[h,:] = sum_j softmax_j(z[h,:]) * kv[pos_j,:]
//
// Work item: one query row and one split of its row list.  Two forms:
//   narrow (mla_kernel, few query rows, i.e. small-batch decode): a 2-wave
//     workgroup takes 32 of the 128 heads, so one query spreads over many CUs;
//   wide (mla_wide_kernel, many query rows): an 8-wave workgroup takes all
//     128 heads, so every gathered row is read from HBM once for all heads;
//     its layout and pipeline are described above the kernel.
// The rest of this header describes the narrow form; the wide one shares its
// gathers, score layout and online softmax.
//
// Gathers.  Rows are copied from HBM straight into LDS (global_load_lds, 16
// bytes a lane, no register staging) into a 2-slot ring, so the next tile is
// in flight while one is computed.  A 512-wide latent row (1 KiB) is one
// instruction; the 64-wide rope part of 8 rows is another, with its 16-byte
// chunks XOR-swizzled by row so the score reads do not collide on banks.  The
// split's row positions are first staged in LDS.  Barriers are plain
// s_barrier with explicit waits (vmcnt for this wave's copies, lgkmcnt for LDS
// writes), so the copies for the next tile stay in flight across them.
//
// Math, transposed so that each lane owns one head.  Scores are computed as
// S^T[row][head] = KV[row] . Q[head] (16x16x32 bf16 MFMA, rows as M, the
// wave's 16 heads as N, K = 576): the lane holding head h gets 16 of the
// tile's 64 rows.  The online softmax state (running max, partial sum) is
// therefore per lane; the max over rows needs only two cross-lane swaps
// (v_permlane32_swap / v_permlane16_swap).  The probabilities stay in
// registers: the rows a lane holds become the B operand of the value
// contraction O^T[c][head] += V^T[c][rows] . P[rows][head], whose A operand is
// read from the row-major LDS tile with ds_read_tr16_b64 (the same K order,
// rows 16s+4g..16s+4g+3 for lane group g, is used on both sides).  O^T has
// the head in the lane too, so rescaling by exp2(m_old - m_new) is one
// multiply per accumulator; it is done lazily, only when a tile's max exceeds
// the running reference by more than 2^8 (probabilities stay below 256).  The
// 16x512 fp32 accumulator lives in registers.  With several splits per row,
// unnormalised partial outputs plus (max, sum) go to the workspace and a
// combine kernel merges them.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kHeads = 128;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kNbuf = 2;                     // tiles in the LDS ring
constexpr int kKvPitch = 1040;               // bytes per latent row in LDS (+16: bank spread)
constexpr int kMaxSplitRows = 2048;

// Shape of one workgroup: kWaves waves of 16 heads; every wave copies kRw
// rows of each tile (one instruction per latent row, one per 8 rope rows),
// so a tile has kRw*kWaves rows.
template <int kWaves, int kRw>
struct MlaShape {
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kHeadsPerBlock = 16 * kWaves;
  static constexpr int kHeadGroups = kHeads / kHeadsPerBlock;
  static constexpr int kRt = kRw * kWaves;                // gathered rows per tile
  static constexpr int kLoadsPerTile = kRw + kRw / 8;     // per wave
  static constexpr int kMt = kRt / 16;                    // 16-row M-tiles per tile
  static constexpr int kKs = kRt / 32;                    // 32-row K-steps of the value product
  static constexpr int kTileKv = kRt * kKvPitch;
  static constexpr int kTileBytes = kTileKv + kRt * 128;  // + rope rows (128 B each)
};
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;


__device__ __forceinline__ uint32_t pack_bf16(float a, float b) { return pack2_bf16(a, b); }

// Most positions a split of the narrow form holds (its plans stay below).
constexpr int kNarrowMaxRows = 512;

template <bool kDense, int kWaves, int kRw>
__global__ __launch_bounds__(kWaves * 64) void mla_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ pe,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, int rows_per_split, int n_splits, int n_items, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float4* __restrict__ part_ml) {
  using S = MlaShape<kWaves, kRw>;
  constexpr int kLoadsPerTile = S::kLoadsPerTile;
  constexpr int kThreads = S::kThreads, kRt = S::kRt, kMt = S::kMt, kKs = S::kKs;
  constexpr int kTileKv = S::kTileKv, kTileBytes = S::kTileBytes;
  __shared__ __align__(16) uint8_t s_ring[kNbuf * kTileBytes];
  __shared__ int s_pos[kNbuf][kRt];  // positions of the tiles in the ring (-1 = empty)
  __shared__ int s_idx[kDense ? 1 : kNarrowMaxRows];  // the split's positions

  // Block -> (item = row * n_splits + split, head group).  The head groups of
  // one item get ids that are 8 apart, i.e. fall on the same XCD (ids are dealt
  // round-robin over the 8 XCDs), so later groups find the rows in its L2.
  int X, hg;
  if constexpr (S::kHeadGroups == 1) {
    X = blockIdx.x;
    hg = 0;
  } else {
    constexpr int G = S::kHeadGroups;
    const int bid = blockIdx.x;
    X = (bid / (8 * G)) * 8 + (bid & 7);
    hg = (bid >> 3) % G;
  }
  if (X >= n_items) return;
  const int row = X / n_splits, split = X - row * n_splits;
  const int b = row / T, t = row - b * T;

  // Entries in this row's list.  Dense: the causal bound.  Sparse: k, or,
  // when end_pos is given (a list from the top-k selection, whose kept
  // positions fill its first min(k, bound) slots), only those slots.
  int n_list;
  if (kDense || end_pos != nullptr) {
    const int ep = min(max(end_pos[b], T), S_max);
    n_list = ep - T + t + 1;
    if (!kDense) n_list = min(n_list, k);
  } else {
    n_list = k;
  }
  const int j_begin = split * rows_per_split;
  const int j_end = min(j_begin + rows_per_split, n_list);
  const int n_rows = max(j_end - j_begin, 0);
  const int n_tiles = (n_rows + kRt - 1) / kRt;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r16 = lane & 15;

  // Position of split entry j (-1 = empty slot, also past the end).
  auto entry_pos = [&](int j) {
    int pos = -1;
    if (j < n_rows) {
      if constexpr (kDense) pos = j_begin + j;
      else pos = s_idx[j];
    }
    return pos;
  };

  // The split's positions are loaded first and the query's fragments right
  // after them; the positions go to LDS as soon as they arrive, so the first
  // tiles' copies start while the query loads are still in flight (the
  // positions are a few hundred bytes, the query 36 KiB a workgroup).
  constexpr int kIdxPer = (kNarrowMaxRows + kThreads - 1) / kThreads;
  int pv[kIdxPer];
  if constexpr (!kDense) {
    const int32_t* src = idx + (size_t)row * k + j_begin;
#pragma unroll
    for (int u = 0; u < kIdxPer; ++u) {
      const int j = threadIdx.x + u * kThreads;
      pv[u] = j < n_rows ? src[j] : -1;
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the position loads go out before the query's

  // Query fragment (B operand of S^T = KV . Q^T): head hg*16*kWaves + wave*16 + r16;
  // K-step kk holds dims kk*32 + 8g .. +7 of [q_nope | q_pe].
  const int head = hg * S::kHeadsPerBlock + wave * 16 + r16;
  uint4 qb[18];
  {
    const uint16_t* qn = q_nope + ((size_t)row * kHeads + head) * kDc;
    const uint16_t* qp = q_pe + ((size_t)row * kHeads + head) * kDr;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qb[kk] = ldg16(qn + kk * 32 + g * 8);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) qb[16 + kk] = ldg16(qp + kk * 32 + g * 8);
  }
  if constexpr (!kDense) {
#pragma unroll
    for (int u = 0; u < kIdxPer; ++u) {
      const int j = threadIdx.x + u * kThreads;
      if (j < n_rows) s_idx[j] = (pv[u] < 0 || pv[u] >= S_max) ? -1 : pv[u];
    }
    lds_barrier();  // LDS only: the query loads stay in flight
  }

  const uint8_t* kv_b = reinterpret_cast<const uint8_t*>(kv) + (size_t)b * S_max * kDc * 2;
  const uint8_t* pe_b = reinterpret_cast<const uint8_t*>(pe) + (size_t)b * S_max * kDr * 2;

  // This wave copies rows kRw*wave .. kRw*wave+kRw-1 of tile `tile` into ring
  // slot tile % kNbuf.  Empty slots copy row 0 (masked in the softmax).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int tile) {
    uint8_t* base = s_ring + (tile % kNbuf) * kTileBytes;
    int rpos[kRw];
#pragma unroll
    for (int r = 0; r < kRw; ++r) rpos[r] = entry_pos(tile * kRt + kRw * wv + r);
    // The tile's positions for the softmax's validity test (published by the
    // barrier that follows the wait for this tile).
    {
      int mine = rpos[0];
#pragma unroll
      for (int r = 1; r < kRw; ++r) mine = lane == r ? rpos[r] : mine;
      if (lane < kRw) s_pos[tile % kNbuf][kRw * wv + lane] = mine;
    }
#pragma unroll
    for (int r = 0; r < kRw; ++r) rpos[r] = max(rpos[r], 0);
#pragma unroll
    for (int r = 0; r < kRw; ++r) {
      const int trow = kRw * wv + r;
      const int pu = __builtin_amdgcn_readfirstlane(rpos[r]);
      lds_copy16(kv_b + (size_t)pu * (kDc * 2), lane * 16,
                 __builtin_amdgcn_readfirstlane(lds_addr(base + trow * kKvPitch)));
    }
    // Rope parts, 8 rows per instruction: lane L writes chunk L%8 of row L/8,
    // holding the row's global chunk (L%8) ^ (row & 7).
#pragma unroll
    for (int q8 = 0; q8 < kRw / 8; ++q8) {
      const int r = 8 * q8 + (lane >> 3);
      int pos = rpos[0];
#pragma unroll
      for (int rr = 1; rr < kRw; ++rr) pos = r == rr ? rpos[rr] : pos;
      const int trow = kRw * wv + r;
      const int chunk = (lane & 7) ^ (trow & 7);
      lds_copy16_v(pe_b + (size_t)pos * (kDr * 2) + chunk * 16,
                   __builtin_amdgcn_readfirstlane(lds_addr(base + kTileKv + (kRw * wv + 8 * q8) * 128)));
    }
  };

  // Running softmax state for head `head` (base 2): reference max, and this
  // lane's share of the sum relative to it.
  float m_run = -INFINITY, l_part = 0.f;
  f32x4 o[32];  // O^T: tile ct holds latent dims ct*16 + 4g + i for this lane's head
#pragma unroll
  for (int c = 0; c < 32; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int p = 0; p < kNbuf - 1 && p < n_tiles; ++p) issue(p);

#pragma unroll 1
  for (int tile = 0; tile < n_tiles; ++tile) {
    if (tile + kNbuf - 1 < n_tiles) issue(tile + kNbuf - 1);
    static_assert(kNbuf == 2, "the wait below assumes one tile in flight");
    if (tile + 1 < n_tiles)  // the next tile's copies may still be in flight
      __builtin_amdgcn_s_waitcnt(wait_vm(kLoadsPerTile));
    else
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
    lds_barrier();  // every wave's copies for this tile have landed

    const uint8_t* buf = s_ring + (tile % kNbuf) * kTileBytes;

    // ---- scores S^T[row][head], rows mt*16 + 4g + i ----
    f32x4 sc[kMt];
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt) sc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
#pragma unroll
      for (int mt = 0; mt < kMt; ++mt) {
        const int trow = mt * 16 + r16;
        const uint8_t* a;
        if (kk < 16) {
          a = buf + trow * kKvPitch + (kk * 32 + 8 * g) * 2;
        } else {
          const int chunk = ((kk - 16) * 4 + g) ^ (trow & 7);
          a = buf + kTileKv + trow * 128 + chunk * 16;
        }
        sc[mt] = mfma_bf16_16x16x32(as_bf16x8(*reinterpret_cast<const uint4*>(a)),
                                    as_bf16x8(qb[kk]), sc[mt]);
      }
    }

    // ---- online softmax for this lane's head ----
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = s_pos[tile % kNbuf][mt * 16 + 4 * g + i] >= 0;
        sc[mt][i] = valid ? sc[mt][i] * scale_log2 : -INFINITY;  // now log2-domain score
        mx = fmaxf(mx, sc[mt][i]);
      }
    mx = group_max(mx);
    // Lazy rescaling: the reference m_run moves only when this tile's max
    // exceeds it by more than kRescaleSlack (log2 units), so probabilities stay
    // below 2^kRescaleSlack and the accumulators are rarely touched.
    // Until a head has seen a valid row its accumulators and sum are zero, so
    // its first reference needs no rescaling.
    const bool grow = mx > m_run + kRescaleSlack;
    const bool fresh = m_run == -INFINITY;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = fresh ? 0.f : exp2f(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
      if (__ballot(grow && !fresh) != 0) {
#pragma unroll
        for (int ct = 0; ct < 32; ++ct) o[ct] *= alpha;
      }
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
    uint4 pb[kKs];  // B operands of the value contraction, one per 32-row K-step
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      float p[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[h][i] = exp2f(sc[2 * ks + h][i] - m_use);
          psum += p[h][i];
        }
      // K-step ks covers M-tiles 2ks and 2ks+1: rows 32ks + 4g + i, then 32ks + 16 + 4g + i.
      pb[ks] = uint4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                     pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
    }
    l_part += psum;

    // ---- values: O^T[c][head] += V^T . P ----
    // Transposed reads: lane r16 of group g gets V[32ks + 16h + 4g + j][c0 + r16]
    // (j = 0..3) from the 8-byte rows addressed by lanes 4j + r16/4.
    const uint8_t* vrow = buf + (4 * g + (r16 >> 2)) * kKvPitch + 8 * (r16 & 3);
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        const i16x4 lo = lds_read_tr16(vrow + (32 * ks) * kKvPitch + ct * 32);
        const i16x4 hi = lds_read_tr16(vrow + (32 * ks + 16) * kKvPitch + ct * 32);
        const uint4 va = uint4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                               (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                               (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                               (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
        o[ct] = mfma_bf16_16x16x32(as_bf16x8(va), as_bf16x8(pb[ks]), o[ct]);
      }
    }
    lds_barrier();  // every wave is done with this slot before it is refilled
  }

  // ---- finish ----
  const float l_tot = group_sum(l_part);
  if (n_splits == 1) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* orow = out + ((size_t)row * kHeads + head) * kDc + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct)
      *reinterpret_cast<uint2*>(orow + ct * 16) =
          uint2{pack_bf16(o[ct][0] * inv, o[ct][1] * inv), pack_bf16(o[ct][2] * inv, o[ct][3] * inv)};
    if (lse != nullptr && g == 0)
      lse[(size_t)row * kHeads + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    // Partial output: the unnormalised accumulator rounded to bf16 (the
    // range of fp32, so no scaling is needed), plus (max, sum) in fp32.  The
    // layout is [item][16-dim tile][head][16]: each store instruction writes
    // 512 contiguous bytes (the wave's 16 heads), i.e. whole cache lines.
    uint16_t* prow = part_o + (size_t)X * kHeads * kDc + head * 16 + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct)
      *reinterpret_cast<uint2*>(prow + ct * kHeads * 16) =
          uint2{pack_bf16(o[ct][0], o[ct][1]), pack_bf16(o[ct][2], o[ct][3])};
    if (g == 0) part_ml[(size_t)X * kHeads + head] = float4{m_run, l_tot, 0.f, 0.f};
  }
}

// ---- Wide form: many query rows -------------------------------------------
//
// Eight waves (two per SIMD).  The two contractions are split differently:
//   scores  S^T[row][head]: the wave pair 2p, 2p+1 takes heads 32p..32p+31,
//           wave 2p+d the half d of the 576 score dims (latent 0..287, or
//           latent 288..511 and the rope part), its query fragments of both
//           16-head tiles in registers.  Each K fragment read from LDS then
//           feeds two MFMAs, so a tile's K is read from LDS four times, not
//           eight (those reads bound the kernel).  The pair swaps the partial
//           scores of the head tile it does not keep through LDS (2 KiB a
//           wave), and wave w finishes head tile w, as in the narrow form;
//   values  O^T[c][head]: wave w takes latent dims 64w..64w+63 for all 128
//           heads (4 x 8 accumulator tiles, 128 registers), so each transposed
//           V fragment feeds 8 head tiles and V is read from LDS once per tile
//           instead of once per wave (in the narrow form the 8-fold re-reading
//           of V through the transposing LDS read dominates).
// The probabilities cross between the two through LDS: the lane of a score
// wave that holds head n and rows {4g+i, 16+4g+i} holds exactly the B
// fragment (same K order) that lane (n, g) of every value wave needs for that
// head tile, so P is 16 bytes per lane per head tile (8 KiB a tile), plus one
// rescale factor per head for tiles where some head's running maximum moved.
// Tiles are 32 rows in a 3-slot ring, so two tiles are in flight during the
// math; each wave copies 4 rows (one copy per latent row, one per rope part).
constexpr int kWdWaves = 8;
constexpr int kWdThreads = kWdWaves * 64;
constexpr int kWdRt = 32;                               // rows per tile
constexpr int kWdRw = kWdRt / kWdWaves;                 // rows each wave copies (4)
constexpr int kWdNbuf = 3;
// Latent rows sit 1056 bytes apart (8 banks), and the 16-byte chunks of rows
// 8..15 and 24..31 of a tile are XOR-swizzled by 1: chunk c of row r is at
// position c ^ ((r >> 3) & 1).  The score reads (16 rows, one chunk each per
// quarter wave) and the transposing value reads (8 rows, two chunks each per
// half wave) are then both free of bank conflicts.
constexpr int kWdPitch = 1056;
__device__ __forceinline__ int wd_swz(int row) { return (row >> 3) & 1; }
constexpr int kWdTileKv = kWdRt * kWdPitch;
constexpr int kWdTileBytes = kWdTileKv + kWdRt * 128;
constexpr int kWdDims = kDc / kWdWaves;                 // latent dims per value wave (64)
constexpr int kWdCt = kWdDims / 16;                     // their 16-dim tiles (4)
constexpr int kWdSteps = (kDc + kDr) / 32 / 2;          // 32-dim score steps per dim half (9)
static_assert(kWdSteps == 9 && kDc / 32 == 16, "dim halves: latent steps 0-8 | 9-15 and rope 0-1");
static_assert(kWdRw == 4, "rope copies use lanes 8r..8r+7 for row r");

template <bool kDense>
__global__ __launch_bounds__(kWdThreads) void mla_wide_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ pe,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, int rows_per_split, int n_splits, int n_items, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o,
    float4* __restrict__ part_ml) {
  __shared__ __align__(16) uint8_t s_ring[kWdNbuf * kWdTileBytes];
  __shared__ __align__(16) uint4 s_p[2][kHeads / 16][64];  // P fragments per head tile
  __shared__ float s_alpha[2][kHeads];                    // a tile's rescale per head
  __shared__ float s_fin[2][kHeads];                    // m, l per head
  __shared__ __align__(8) uint8_t s_vmask[kWdNbuf][kWdWaves];  // bit r: row 4w+r is valid
  __shared__ __align__(16) float4 s_x[kWdWaves][2][64];     // partial scores for the pair wave
  __shared__ int s_grow[2];                             // last tile (per parity) whose max moved
  __shared__ int s_idx[kDense ? 1 : kMaxSplitRows];     // the split's positions

  const int X = blockIdx.x;
  if (X >= n_items) return;
  const int row = X / n_splits, split = X - row * n_splits;
  const int b = row / T, t = row - b * T;
  // Entries in this row's list.  Dense: the causal bound.  Sparse: k, or,
  // when end_pos is given (a list from the top-k selection, whose kept
  // positions fill its first min(k, bound) slots), only those slots.
  int n_list;
  if (kDense || end_pos != nullptr) {
    const int ep = min(max(end_pos[b], T), S_max);
    n_list = ep - T + t + 1;
    if (!kDense) n_list = min(n_list, k);
  } else {
    n_list = k;
  }
  const int j_begin = split * rows_per_split;
  const int j_end = min(j_begin + rows_per_split, n_list);
  const int n_rows = max(j_end - j_begin, 0);
  const int n_tiles = (n_rows + kWdRt - 1) / kWdRt;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // The split's positions are copied into LDS once, so the gathers of later
  // tiles never wait on a load of their positions.
  if constexpr (!kDense) {
    const int32_t* src = idx + (size_t)row * k + j_begin;
    for (int j = threadIdx.x; j < n_rows; j += kWdThreads) {
      const int pos = src[j];
      s_idx[j] = (pos < 0 || pos >= S_max) ? -1 : pos;
    }
  }
  auto entry_pos = [&](int j) {
    int pos = -1;
    if (j < n_rows) {
      if constexpr (kDense) pos = j_begin + j;
      else pos = s_idx[j];
    }
    return pos;
  };

  // Query fragments of the pair's two head tiles (heads 32*(wave/2) + 16*ht
  // + r16) over this wave's dim half: step j is score step 9*dh + j, latent
  // dims 32*step.. for steps below 16, the rope part after.
  const int head = 16 * wave + r16;  // the head this lane finishes
  const int dh = wv & 1;
  uint4 qb[2][kWdSteps];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int hq = 16 * ((wave & ~1) + ht) + r16;
    const uint16_t* qn = q_nope + ((size_t)row * kHeads + hq) * kDc + 9 * 32 * dh + g * 8;
    const uint16_t* qp = q_pe + ((size_t)row * kHeads + hq) * kDr + g * 8;
#pragma unroll
    for (int j = 0; j < kWdSteps; ++j)
      qb[ht][j] = ldg16(j < 7 || dh == 0 ? qn + j * 32 : qp + (j - 7) * 32);
  }

  const uint8_t* kv_b = reinterpret_cast<const uint8_t*>(kv) + (size_t)b * S_max * kDc * 2;
  const uint8_t* pe_b = reinterpret_cast<const uint8_t*>(pe) + (size_t)b * S_max * kDr * 2;

  // This wave copies rows 4*wave .. 4*wave+3 of tile `tile` into its ring
  // slot (empty entries copy row 0 and are masked by their position -1).
  auto issue = [&](int tile) {
    uint8_t* base = s_ring + (tile % kWdNbuf) * kWdTileBytes;
    int rpos[kWdRw];
#pragma unroll
    for (int r = 0; r < kWdRw; ++r) rpos[r] = entry_pos(tile * kWdRt + kWdRw * wv + r);
    {
      uint32_t vm = 0;
#pragma unroll
      for (int r = 0; r < kWdRw; ++r) vm |= (rpos[r] >= 0 ? 1u : 0u) << r;
      if (lane == 0) s_vmask[tile % kWdNbuf][wv] = (uint8_t)vm;
    }
#pragma unroll
    for (int r = 0; r < kWdRw; ++r) rpos[r] = max(rpos[r], 0);
#pragma unroll
    for (int r = 0; r < kWdRw; ++r) {
      // The position is uniform over the wave: the row's address is scalar.
      const int pu = __builtin_amdgcn_readfirstlane(rpos[r]);
      const uint8_t* rowp = kv_b + (size_t)pu * (kDc * 2);
      const int trow = kWdRw * wv + r;
      // Lane L writes position L, so it fetches chunk L ^ swizzle.
      lds_copy16(rowp, (opaque_lane() ^ wd_swz(trow)) * 16,
                 __builtin_amdgcn_readfirstlane(lds_addr(base + trow * kWdPitch)));
    }
    // Rope parts of the 4 rows, one copy per row by lanes 8r..8r+7 (so the
    // row's address is scalar): lane 8r+c writes chunk c of row r, holding the
    // row's global chunk c ^ (row & 7).
    {
      const int ln = opaque_lane();
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(base + kWdTileKv + kWdRw * wv * 128));
#pragma unroll
      for (int r = 0; r < kWdRw; ++r) {
        const int trow = kWdRw * wv + r;
        const int pu = __builtin_amdgcn_readfirstlane(rpos[r]);
        if ((ln >> 3) == r)
          lds_copy16(pe_b + (size_t)pu * (kDr * 2), (uint32_t)(((ln & 7) ^ (trow & 7)) * 16), m0);
      }
    }
  };

  float m_run = -INFINITY, l_part = 0.f;
  f32x4 o[kWdCt][8];  // [c-tile kWdCt*wave + j][head tile]: dims ct*16 + 4g + i, head 16*h + r16
#pragma unroll
  for (int j = 0; j < kWdCt; ++j)
#pragma unroll
    for (int h = 0; h < 8; ++h) o[j][h] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (threadIdx.x < 2) s_grow[threadIdx.x] = -1;
  __syncthreads();  // s_idx and s_grow

  if (n_tiles > 0) issue(0);

  // Iteration it: scores and softmax of tile it, then the values of tile it-1
  // (whose P was written in the previous iteration): one barrier per tile, and
  // one between the two halves of the scores.
#pragma unroll 1
  for (int it = 0; it <= n_tiles; ++it) {
    static_assert(kWdNbuf == 3, "slots: tile it-1 (values), tile it (scores), tile it+1 (copies)");
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // this wave's copies of tile it have landed
    lds_barrier();  // ... and every wave's; P(it-1) is visible; slot (it+1)%3 is free
    if (it + 1 < n_tiles) issue(it + 1);
    const int lane = opaque_lane(), g = lane >> 4, r16 = lane & 15;  // recomputed addresses
    const int head = 16 * wave + r16;

    // ---- scores of tile it, this wave's dim half for the pair's 32 heads;
    //      rows mt*16 + 4g + i ----
    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const bool have_s = it < n_tiles;
    const int slot = it % kWdNbuf;
    if (have_s) {
      const uint8_t* buf = s_ring + slot * kWdTileBytes;
      // Rows r16 and 16 + r16 share their swizzle (r16 >> 3): latent step s
      // of row tile mt is at the offset mt*16*pitch + 64*s from one base.
      // The rope chunks (4j' + g) ^ (r16 & 7) differ per lane.
      const uint8_t* kb = buf + r16 * kWdPitch + ((g ^ (r16 >> 3)) << 4) + 9 * 64 * dh;
      const uint8_t* rb = buf + kWdTileKv + r16 * 128;
      f32x4 sp[2][2] = {{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}},
                        {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
      for (int j = 0; j < kWdSteps; ++j) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint8_t* a = kb + mt * 16 * kWdPitch + 64 * j;
          if (j >= 7 && dh == 1) a = rb + mt * 16 * 128 + ((((j - 7) * 4 + g) ^ (r16 & 7)) << 4);
          const uint4 kf = *reinterpret_cast<const uint4*>(a);
#pragma unroll
          for (int ht = 0; ht < 2; ++ht)
            sp[ht][mt] = mfma_bf16_16x16x32(as_bf16x8(kf), as_bf16x8(qb[ht][j]), sp[ht][mt]);
        }
      }
      // Keep head tile dh, hand the other one's partial to the pair wave.
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        sc[mt] = dh ? sp[1][mt] : sp[0][mt];
        const f32x4 give = dh ? sp[0][mt] : sp[1][mt];
        s_x[wv][mt][lane] = float4{give[0], give[1], give[2], give[3]};
      }
      lds_barrier();  // the pair's partials are visible
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const float4 got = s_x[wv ^ 1][mt][lane];
        sc[mt][0] += got.x, sc[mt][1] += got.y, sc[mt][2] += got.z, sc[mt][3] += got.w;
      }
    }

    // ---- online softmax of tile it for this lane's head (branch-free) ----
    if (have_s) {
      const int cp = it & 1;
      // Rows 4g+i were copied by wave g, rows 16+4g+i by wave 4+g.
      const uint32_t vm = (uint32_t)s_vmask[slot][g] | ((uint32_t)s_vmask[slot][4 + g] << 4);
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[mt][i] = (vm >> (4 * mt + i)) & 1u ? sc[mt][i] : -INFINITY;  // raw score, masked
          mx = fmaxf(mx, sc[mt][i]);
        }
      mx = group_max(mx) * scale_log2;  // log2-domain tile max
      // Lazy rescaling: the reference moves only when the tile's max exceeds
      // it by more than kRescaleSlack, so probabilities stay below 2^8.
      const bool grow = mx > m_run + kRescaleSlack;
      const bool fresh = m_run == -INFINITY;
      const float alpha = grow ? (fresh ? 0.f : __builtin_amdgcn_exp2f(m_run - mx)) : 1.f;
      m_run = grow ? mx : m_run;
      l_part *= alpha;
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float p[2][4], psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[mt][i] = __builtin_amdgcn_exp2f(fmaf(sc[mt][i], scale_log2, -m_use));
          psum += p[mt][i];
        }
      l_part += psum;
      s_p[cp][wave][lane] = uint4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                                  pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
      if (g == 0) s_alpha[cp][head] = alpha;
      // A head's first reference needs no rescaling (its accumulators are zero).
      if (__ballot(grow && !fresh) != 0 && lane == 0) s_grow[cp] = it;
    }

    // ---- values of tile it-1 for this wave's 64 latent dims, all heads ----
    if (it > 0) {
      const int pt = it - 1, pp = pt & 1;
      if (s_grow[pp] == pt) {  // some head's reference moved at tile it-1
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const float al = s_alpha[pp][16 * h + r16];
#pragma unroll
          for (int j = 0; j < kWdCt; ++j) o[j][h] *= al;
        }
      }
      // Rows 4g + r16/4 (+16): their swizzle is g >> 1 for both halves.
      const uint8_t* vrow = s_ring + (pt % kWdNbuf) * kWdTileBytes +
                            (4 * g + (r16 >> 2)) * kWdPitch + 8 * (r16 & 1);
      const int vsw = g >> 1, vch = (r16 & 3) >> 1;
#pragma unroll
      for (int jh = 0; jh < kWdCt; jh += 2) {
        uint4 va[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int ct = kWdCt * wave + jh + jj;
          const int off = ((2 * ct + vch) ^ vsw) << 4;  // this lane's 16-byte chunk
          const i16x4 lo = lds_read_tr16(vrow + off);
          const i16x4 hi = lds_read_tr16(vrow + 16 * kWdPitch + off);
          va[jj] = uint4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                         (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                         (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                         (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
        }
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          const uint4 pb = s_p[pp][h][lane];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            o[jh + jj][h] = mfma_bf16_16x16x32(as_bf16x8(va[jj]), as_bf16x8(pb), o[jh + jj][h]);
        }
      }
    }
  }

  // ---- finish: (m, l) per head from the score waves to the value waves ----
  {
    const float l_tot = group_sum(l_part);
    if (g == 0) {
      s_fin[0][head] = m_run;
      s_fin[1][head] = l_tot;
      if (n_splits == 1 && lse != nullptr)
        lse[(size_t)row * kHeads + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
  lds_barrier();
  float inv[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const float l = s_fin[1][16 * h + r16];
    inv[h] = l > 0.f ? 1.f / l : 0.f;
  }
  if (n_splits == 1) {
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      uint16_t* orow = out + ((size_t)row * kHeads + 16 * h + r16) * kDc + 4 * g;
#pragma unroll
      for (int j = 0; j < kWdCt; ++j) {
        const int ct = kWdCt * wave + j;
        *reinterpret_cast<uint2*>(orow + ct * 16) =
            uint2{pack_bf16(o[j][h][0] * inv[h], o[j][h][1] * inv[h]),
                  pack_bf16(o[j][h][2] * inv[h], o[j][h][3] * inv[h])};
      }
    }
  } else {
    // Partial output: the unnormalised accumulators rounded to bf16, plus
    // (max, sum) per head in fp32.
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const int hd = 16 * h + r16;
      uint16_t* prow = part_o + (size_t)X * kHeads * kDc + hd * 16 + 4 * g;  // [item][tile][head][16]
#pragma unroll
      for (int j = 0; j < kWdCt; ++j) {
        const int ct = kWdCt * wave + j;
        *reinterpret_cast<uint2*>(prow + ct * kHeads * 16) =
            uint2{pack_bf16(o[j][h][0], o[j][h][1]), pack_bf16(o[j][h][2], o[j][h][3])};
      }
      if (wave == 0 && g == 0)
        part_ml[(size_t)X * kHeads + hd] = float4{s_fin[0][hd], s_fin[1][hd], 0.f, 0.f};
    }
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Maximum and sum over the 64 lanes of a wave (all lanes active), returned in
// every lane: an inclusive scan by DPP row shifts and row broadcasts, read
// back from lane 63.  Lanes a shift leaves without a source take the
// identity (-inf for the maximum, 0 for the sum).
__device__ __forceinline__ float wave_max_f(float v) {
  const int id = __float_as_int(-INFINITY);
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(v), 0x111, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(v), 0x112, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(v), 0x114, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(v), 0x118, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Merge the per-split partial outputs of four heads of one row per 512-thread
// block.  Thread t owns 4 latent dims of one head: 16-dim tile t/16, head
// t/4 % 4, quarter t % 4, so a wave's load of one split covers 4 tiles x 4
// heads x 32 bytes, i.e. four whole 128-byte lines of the [tile][head][16]
// partial layout.  The splits are read kBatch at a time (their loads all in
// flight together; kBatch = 4, 8, 16 or 32, the least that covers the splits,
// so no load is spent on a missing split), so a row with up to 32 splits costs
// one round trip to memory.  Wave q < 4 turns the batch's (max, sum) pairs of head q into one
// weight per split, 2^(its max - M) with M the running maximum, and the factor
// that rescales what was accumulated before; every thread then only reads its
// head's weights and accumulates.
constexpr int kCbHeads = 4;
constexpr int kCbThreads = 512;
static_assert(kCbThreads == (kDc / 16) * kCbHeads * 4 && kHeads % kCbHeads == 0,
              "one thread per (16-dim tile, head, quarter of the tile)");
// kParts > 1 (few rows): each workgroup takes 1/kParts of the 32 dim tiles
// with kCbThreads/kParts threads, so more workgroups share the loads (every
// part repeats the weights of its four heads; with fewer than four waves a
// wave makes the weights of several heads).
template <int kBatch, int kParts>
__global__ __launch_bounds__(kCbThreads / kParts) void mla_combine_kernel(
    const uint16_t* __restrict__ part_o, const float4* __restrict__ part_ml, int n_splits,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  static_assert(kBatch % 4 == 0 && kBatch <= 32, "batches of 4 to 32 splits");
  constexpr int kWavesB = kCbThreads / kParts / 64;
  constexpr int kHpw = kCbHeads > kWavesB ? kCbHeads / kWavesB : 1;  // heads whose weights a wave makes
  static_assert(kHpw * kWavesB >= kCbHeads, "every head's weights have a wave");
  constexpr int kGroups = kHeads / kCbHeads;
  const int part = blockIdx.x % kParts, gid = blockIdx.x / kParts;
  const int row = gid / kGroups, h0 = (gid - row * kGroups) * kCbHeads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ct = (tid >> 4) + part * (kDc / 16 / kParts), q = (tid >> 2) & 3, quarter = tid & 3;
  const int head = h0 + q;
  const size_t item0 = (size_t)row * n_splits;
  const uint16_t* src = part_o + item0 * kHeads * kDc + ((size_t)ct * kHeads + head) * 16 + 4 * quarter;
  const size_t stride = (size_t)kHeads * kDc;  // one split
  __shared__ __align__(16) float s_w[2][kCbHeads][kBatch];  // by batch parity
  __shared__ float s_alpha[2][kCbHeads];
  __shared__ float s_inv[kCbHeads];
  float4 acc = float4{0.f, 0.f, 0.f, 0.f};
  float L[kHpw], M[kHpw];  // kept by wave q for heads h0 + q + kWavesB * i
#pragma unroll
  for (int i = 0; i < kHpw; ++i) L[i] = 0.f, M[i] = -INFINITY;
  int par = 0;
  for (int s0 = 0; s0 < n_splits; s0 += kBatch, par ^= 1) {
    uint2 a[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      a[u] = *reinterpret_cast<const uint2*>(src + (size_t)min(s0 + u, n_splits - 1) * stride);
#pragma unroll
    for (int i = 0; i < kHpw; ++i) {
      const int hq = wave + kWavesB * i;
      if (hq < kCbHeads) {
        const int s = min(s0 + min(lane, kBatch - 1), n_splits - 1);
        const float4 v = part_ml[(item0 + s) * kHeads + h0 + hq];
        const bool valid = lane < kBatch && s0 + lane < n_splits && v.y > 0.f;
        const float mb = fmaxf(M[i], wave_max_f(valid ? v.x : -INFINITY));
        // Nothing was accumulated while M was -inf, so the factor is then moot.
        const float alpha = M[i] == -INFINITY ? 0.f : exp2f(M[i] - mb);
        const float w = valid ? exp2f(v.x - mb) : 0.f;
        L[i] = L[i] * alpha + wave_sum_f(w * v.y);
        M[i] = mb;
        if (lane < kBatch) s_w[par][hq][lane] = w;
        if (lane == 0) s_alpha[par][hq] = alpha;
      }
    }
    // One barrier per batch: a wave can only refill this parity's weights
    // after every wave has passed the next batch's barrier.
    __syncthreads();
    const float alpha = s_alpha[par][q];
    acc.x *= alpha;
    acc.y *= alpha;
    acc.z *= alpha;
    acc.w *= alpha;
#pragma unroll
    for (int u4 = 0; u4 < kBatch; u4 += 4) {
      const float4 w4 = *reinterpret_cast<const float4*>(&s_w[par][q][u4]);
      const float ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 av = a[u4 + j];
        acc.x += bf16_lo(av.x) * ws[j];
        acc.y += bf16_hi(av.x) * ws[j];
        acc.z += bf16_lo(av.y) * ws[j];
        acc.w += bf16_hi(av.y) * ws[j];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kHpw; ++i) {
    const int hq = wave + kWavesB * i;
    if (hq < kCbHeads && lane == 0) {
      s_inv[hq] = L[i] > 0.f ? 1.f / L[i] : 0.f;
      if (lse != nullptr && part == 0)
        lse[(size_t)row * kHeads + h0 + hq] = L[i] > 0.f ? (M[i] + log2f(L[i])) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  const float inv = s_inv[q];
  *reinterpret_cast<uint2*>(out + ((size_t)row * kHeads + head) * kDc + ct * 16 + 4 * quarter) =
      uint2{pack_bf16(acc.x * inv, acc.y * inv), pack_bf16(acc.z * inv, acc.w * inv)};
}

static int round_up(int x, int m) { return (x + m - 1) / m * m; }

#ifndef DSA_MLA_TARGET_BLOCKS
#define DSA_MLA_TARGET_BLOCKS 256
#endif
#ifndef DSA_CB_SPLIT_ROWS
#define DSA_CB_SPLIT_ROWS 2
#endif
#ifndef DSA_MLA_SMALL_ROWS
#define DSA_MLA_SMALL_ROWS 16
#endif
#ifndef DSA_MLA_SMALL_SPLIT_MIN
#define DSA_MLA_SMALL_SPLIT_MIN 64
#endif
#ifndef DSA_MLA_DENSE_SMALL_WORK
#define DSA_MLA_DENSE_SMALL_WORK 65536
#endif

// Few query rows (decode at small batch): blocks of 2 waves (32 heads, 16 rows
// per wave per tile) for one or two rows, else of 4 waves (64 heads, 8 rows
// per wave per tile: half the L2 re-reads of each gathered row, which pays
// once several rows fill the chip), and short splits, so one query is spread
// over many CUs.
// Otherwise 8-wave blocks of all 128 heads (every gathered row read once) and
// about one block per CU.
static int narrow_waves(long rows) { return rows <= 2 ? 2 : 4; }

MlaPlan sparse_mla_plan(int B, int T, int k) {
  const long rows = (long)B * T;
  if (rows <= DSA_MLA_SMALL_ROWS) {
    // Splits of k*rows/128 rows (a power of two, at least DSA_MLA_SMALL_SPLIT_MIN):
    // about 128 items of 2 head groups each.
    int rps = DSA_MLA_SMALL_SPLIT_MIN;
    while (rps < kMaxSplitRows && (long)rps * 128 < (long)k * rows) rps *= 2;
    if (rps <= kNarrowMaxRows) return MlaPlan{rps, (k + rps - 1) / rps, narrow_waves(rows)};
  }
  long ns = DSA_MLA_TARGET_BLOCKS / rows;
  const long max_ns = (k + 63) / 64;
  ns = ns < 1 ? 1 : (ns > max_ns ? max_ns : ns);
  int rps = round_up((int)((k + ns - 1) / ns), 64);
  if (rps > kMaxSplitRows) rps = kMaxSplitRows;
  return MlaPlan{rps, (k + rps - 1) / rps, 8};
}

MlaPlan dense_mla_plan(int B, int T, int S_max, int max_end_pos) {
  const long rows = (long)B * T;
  const int ext = max_end_pos > 0 ? max_end_pos : S_max;
  // Rows per split depend only on the allocation sizes, so the workspace
  // computed from S_max always covers the launch.
  // Few rows over a short context: the small-batch shape, as on the sparse
  // path; otherwise 8-wave blocks, which gather every row once for all heads.
  if (rows <= DSA_MLA_SMALL_ROWS && (long)S_max * rows <= DSA_MLA_DENSE_SMALL_WORK) {
    int rps = DSA_MLA_SMALL_SPLIT_MIN;
    while (rps < kMaxSplitRows && (long)rps * 128 < (long)S_max * rows) rps *= 2;
    if (rps <= kNarrowMaxRows) return MlaPlan{rps, (ext + rps - 1) / rps, narrow_waves(rows)};
  }
  long rps = (long)S_max * rows / DSA_MLA_TARGET_BLOCKS;
  rps = rps < 512 ? 512 : (rps > kMaxSplitRows ? kMaxSplitRows : rps);
  const int r = round_up((int)rps, 64);
  return MlaPlan{r, (ext + r - 1) / r, 8};
}

size_t mla_workspace_bytes(int B, int T, const MlaPlan& plan) {
  if (plan.n_splits <= 1) return 0;
  const size_t items = (size_t)B * T * plan.n_splits;
  return items * kHeads * kDc * sizeof(uint16_t) + items * kHeads * sizeof(float4);
}

template <bool kDense, int kWaves, int kRw>
static int launch_mla_shape(const void* q_nope, const void* q_pe, const void* kv,
                            const void* pe, const int32_t* idx, const int32_t* end_pos, int T,
                            int S_max, int k, const MlaPlan& plan, int rows, float softmax_scale,
                            void* out, float* lse, uint16_t* part_o, float4* part_ml,
                            hipStream_t stream) {
  using S = MlaShape<kWaves, kRw>;
  const int n_items = rows * plan.n_splits;
  const unsigned grid = S::kHeadGroups == 1
                            ? (unsigned)n_items
                            : (unsigned)(((n_items + 7) / 8) * 8 * S::kHeadGroups);
  hipLaunchKernelGGL((mla_kernel<kDense, kWaves, kRw>), dim3(grid), dim3(S::kThreads), 0, stream,
                     reinterpret_cast<const uint16_t*>(q_nope),
                     reinterpret_cast<const uint16_t*>(q_pe), reinterpret_cast<const uint16_t*>(kv),
                     reinterpret_cast<const uint16_t*>(pe), idx, end_pos, T, S_max, k,
                     plan.rows_per_split, plan.n_splits, n_items, softmax_scale * kLog2e,
                     reinterpret_cast<uint16_t*>(out), lse, part_o, part_ml);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <bool kDense>
static int launch_mla(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                      const int32_t* idx, const int32_t* end_pos, int B, int T, int S_max, int k,
                      const MlaPlan& plan, float softmax_scale, void* out, float* lse,
                      void* workspace, hipStream_t stream) {
  const int rows = B * T;
  const int n_items = rows * plan.n_splits;
  uint16_t* part_o = nullptr;
  float4* part_ml = nullptr;
  if (plan.n_splits > 1) {
    part_o = reinterpret_cast<uint16_t*>(workspace);
    part_ml = reinterpret_cast<float4*>(part_o + (size_t)n_items * kHeads * kDc);
  }
  int st;
  if (plan.waves == 8) {
    hipLaunchKernelGGL((mla_wide_kernel<kDense>), dim3((unsigned)n_items), dim3(kWdThreads), 0,
                       stream, reinterpret_cast<const uint16_t*>(q_nope),
                       reinterpret_cast<const uint16_t*>(q_pe),
                       reinterpret_cast<const uint16_t*>(kv), reinterpret_cast<const uint16_t*>(pe),
                       idx, end_pos, T, S_max, k, plan.rows_per_split, plan.n_splits, n_items,
                       softmax_scale * kLog2e, reinterpret_cast<uint16_t*>(out), lse, part_o,
                       part_ml);
    st = hipGetLastError() == hipSuccess ? 0 : -5;
  } else if (plan.waves == 4) {
    st = launch_mla_shape<kDense, 4, 8>(q_nope, q_pe, kv, pe, idx, end_pos, T, S_max, k, plan,
                                        rows, softmax_scale, out, lse, part_o, part_ml, stream);
  } else {
    st = launch_mla_shape<kDense, 2, 16>(q_nope, q_pe, kv, pe, idx, end_pos, T, S_max, k, plan,
                                         rows, softmax_scale, out, lse, part_o, part_ml, stream);
  }
  if (st) return st;
  if (plan.n_splits > 1) {
    uint16_t* o16 = reinterpret_cast<uint16_t*>(out);
    const unsigned groups = (unsigned)(rows * (kHeads / kCbHeads));
    if (rows <= DSA_CB_SPLIT_ROWS) {
      // Few rows: four workgroups per head group, so four times as many CUs load.
      const dim3 grid(4 * groups), block(kCbThreads / 4);
      if (plan.n_splits <= 16)
        hipLaunchKernelGGL((mla_combine_kernel<16, 4>), grid, block, 0, stream, part_o, part_ml,
                           plan.n_splits, o16, lse);
      else
        hipLaunchKernelGGL((mla_combine_kernel<32, 4>), grid, block, 0, stream, part_o, part_ml,
                           plan.n_splits, o16, lse);
    } else {
      const dim3 grid(groups), block(kCbThreads);
      if (plan.n_splits <= 4)
        hipLaunchKernelGGL((mla_combine_kernel<4, 1>), grid, block, 0, stream, part_o, part_ml,
                           plan.n_splits, o16, lse);
      else if (plan.n_splits <= 8)
        hipLaunchKernelGGL((mla_combine_kernel<8, 1>), grid, block, 0, stream, part_o, part_ml,
                           plan.n_splits, o16, lse);
      else if (plan.n_splits <= 16)
        hipLaunchKernelGGL((mla_combine_kernel<16, 1>), grid, block, 0, stream, part_o, part_ml,
                           plan.n_splits, o16, lse);
      else
        hipLaunchKernelGGL((mla_combine_kernel<32, 1>), grid, block, 0, stream, part_o, part_ml,
                           plan.n_splits, o16, lse);
    }
    if (hipGetLastError() != hipSuccess) return -5;
  }
  return 0;
}

int launch_sparse_mla(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                      const int32_t* idx, int B, int T, int S_max, int k, float softmax_scale,
                      void* out, float* lse, void* workspace, hipStream_t stream,
                      const int32_t* prefix_end_pos) {
  const MlaPlan plan = sparse_mla_plan(B, T, k);
  return launch_mla<false>(q_nope, q_pe, kv, pe, idx, prefix_end_pos, B, T, S_max, k, plan,
                           softmax_scale, out, lse, workspace, stream);
}

int launch_dense_mla(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                     const int32_t* end_pos, int B, int T, int S_max, int max_end_pos,
                     float softmax_scale, void* out, float* lse, void* workspace,
                     hipStream_t stream) {
  const MlaPlan plan = dense_mla_plan(B, T, S_max, max_end_pos);
  return launch_mla<true>(q_nope, q_pe, kv, pe, nullptr, end_pos, B, T, S_max, 0, plan,
                          softmax_scale, out, lse, workspace, stream);
}

}  // namespace dsa
