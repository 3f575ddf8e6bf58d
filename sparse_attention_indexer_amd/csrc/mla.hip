// Absorbed-MLA attention over gathered cached rows on gfx950 (the MQA decode
// branch of "DeepSeek-V3.2-Exp - Apply sparse mask", restricted to the rows the
// indexer selected; the dense variant takes every causally valid row).
//
//   z[h,j] = (q_nope[h,:] . kv[pos_j,:] + q_pe[h,:] . pe[pos_j,:]) * softmax_scale
//   out[h,:] = sum_j softmax_j(z[h,:]) * kv[pos_j,:]
//
// Work item: one query row and one split of its row list.  Two forms:
//   tile (mla_tile_kernel, at most 4 query rows, i.e. small-batch decode): a
//     4-wave workgroup takes 32 of the 128 heads and one 64-row tile of the
//     list, so one query spreads over 128 workgroups;
//   wide (mla_wide_kernel, more rows): an 8-wave workgroup takes all 128
//     heads, so every gathered row is read from HBM once for all heads, and
//     walks its split in 32-row tiles through a 3-slot ring.
// Their layouts and pipelines are described above each kernel; they share:
//
// Gathers.  Rows are copied from HBM straight into LDS (global_load_lds, 16
// bytes a lane, no register staging).  A 512-wide latent row (1 KiB) is one
// instruction; the 64-wide rope parts of 8 rows are another, with their
// 16-byte chunks XOR-swizzled by row so the score reads do not collide on
// banks.  The positions are first staged in LDS.  Barriers are plain
// s_barrier with explicit waits (vmcnt for this wave's copies, lgkmcnt for
// LDS writes), so copies still in flight stay in flight across them.
//
// Math, transposed so that each lane owns one head.  Scores are computed as
// S^T[row][head] = KV[row] . Q[head] (16x16x32 bf16 MFMA, rows as M, 16 heads
// as N, K = 576): the lane holding head h gets 4 rows of each 16-row M-tile.
// The softmax state (running max, partial sum) is therefore per lane; the max
// over rows needs only two cross-lane swaps (v_permlane32_swap /
// v_permlane16_swap).  The probabilities are the B operand of the value
// contraction O^T[c][head] += V^T[c][rows] . P[rows][head], whose A operand is
// read from the row-major LDS tile with ds_read_tr16_b64 (the same K order of
// rows on both sides).  O^T has the head in the lane too, so rescaling by
// exp2(m_old - m_new) is one multiply per accumulator.  With several splits
// per row, unnormalised partial outputs plus (max, sum) go to the workspace
// and a combine kernel merges them.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kHeads = 128;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kMaxSplitRows = 2048;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.f;


__device__ __forceinline__ uint32_t pack_bf16(float a, float b) { return pack2_bf16(a, b); }

// ---- Tile form: few query rows, one 64-row tile per workgroup -------------
//
// Four waves (one per SIMD) and 32 heads (a head group) per workgroup, and one
// tile of 64 rows of the list per workgroup, so a decode query spreads over
// (k / 64) * 4 workgroups with every SIMD of a CU busy.  The two contractions
// are split differently between the waves:
//   scores  S^T[row][head]: wave w takes rows 16w..16w+15 of the tile for all
//           32 heads, so every K fragment read from LDS feeds two MFMAs (the
//           query fragments of both 16-head tiles, 36 x 16 bytes a lane, come
//           from an LDS copy of the head group's query);
//   values  O^T[c][head]: wave w takes latent dims 128w..128w+127 for all 32
//           heads (8 x 2 accumulator tiles), each transposed V fragment
//           feeding two MFMAs.
// The probabilities cross through LDS: value K-step s covers tile rows
// 32s..32s+31 in the order rows 32s+4g+i then 32s+16+4g+i (i < 4) for lane
// group g, so score wave 2s+h's lane holds exactly half (h) of the B fragment
// that the same lane of every value wave needs.  The tile's maximum per head
// (over the four score waves, through LDS) is the softmax reference, so there
// is no rescaling.  Latent rows sit 1056 bytes apart, unswizzled, as in the
// wide form; rope parts are 128-byte rows with chunk c at c ^ (r & 7).
constexpr int kTfWaves = 4;
constexpr int kTfThreads = kTfWaves * 64;
constexpr int kTfHeads = 32;
constexpr int kTfRows = 64;
constexpr int kTfPitch = 1056;
constexpr int kTfGroups = kHeads / kTfHeads;  // 4 head groups
constexpr int kTfQPitch = kDc * 2 + 16;       // q_nope rows in LDS, 16 bytes apart in bank

template <bool kDense>
__global__ __launch_bounds__(kTfThreads) void mla_tile_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ pe,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, int n_splits, int n_items, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, uint16_t* __restrict__ part_o, float4* __restrict__ part_ml) {
  __shared__ __align__(16) uint8_t s_qn[kTfHeads * kTfQPitch];  // the head group's q_nope rows
  __shared__ __align__(16) uint8_t s_qp[kTfHeads * kDr * 2];   // and q_pe rows
  __shared__ __align__(16) uint8_t s_kv[kTfRows * kTfPitch];   // the tile's latent rows
  __shared__ __align__(16) uint8_t s_pe[kTfRows * kDr * 2];    // and rope parts
  __shared__ __align__(16) uint4 s_p[2][2][64];               // P fragments [K-step][head tile][lane]
  __shared__ float s_red[2][kTfWaves][kTfHeads];              // per-wave max, then sum, per head
  __shared__ int s_pos[kTfRows];

  // Block -> (item, head group): the head groups of one item get ids 8 apart
  // (the same XCD under round-robin dispatch), so they share its L2.
  const int bid = blockIdx.x;
  const int X = (bid / (8 * kTfGroups)) * 8 + (bid & 7);
  const int hg = (bid >> 3) % kTfGroups;
  if (X >= n_items) return;
  const int row = X / n_splits, split = X - row * n_splits;
  const int b = row / T, t = row - b * T;
  int n_list;
  if (kDense || end_pos != nullptr) {
    const int ep = min(max(end_pos[b], T), S_max);
    n_list = ep - T + t + 1;
    if (!kDense) n_list = min(n_list, k);
  } else {
    n_list = k;
  }
  const int j_begin = split * kTfRows;
  const int n_rows = max(min(kTfRows, n_list - j_begin), 0);

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

  // The tile's positions first (they address the gathers), then the query.
  int pos = -1;
  if (tid < kTfRows && tid < n_rows) {
    if constexpr (kDense) pos = j_begin + tid;
    else {
      pos = idx[(size_t)row * k + j_begin + tid];
      if (pos < 0 || pos >= S_max) pos = -1;
    }
  }
  {
    // Query: 32 rows of 1 KiB (one per head) and 4 KiB of rope parts, 36
    // copies of 1 KiB, nine a wave.
    const int ln = opaque_lane();
    const size_t h0 = (size_t)row * kHeads + hg * kTfHeads;
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const int cc = wv * 9 + c;
      if (cc < kTfHeads) {
        lds_copy16_v(reinterpret_cast<const uint8_t*>(q_nope + (h0 + cc) * kDc) + ln * 16,
                     __builtin_amdgcn_readfirstlane(lds_addr(s_qn + cc * kTfQPitch)));
      } else {
        const int c4 = cc - kTfHeads;  // 8 heads' rope parts
        lds_copy16_v(reinterpret_cast<const uint8_t*>(q_pe + (h0 + 8 * c4) * kDr) + ln * 16,
                     __builtin_amdgcn_readfirstlane(lds_addr(s_qp + c4 * 1024)));
      }
    }
  }
  if (tid < kTfRows) s_pos[tid] = pos;
  lds_barrier();  // positions visible; the query copies stay in flight

  // Gathers: wave w copies rows 16w..16w+15 (one instruction per latent row,
  // two for the sixteen rope parts).
  const uint8_t* kv_b = reinterpret_cast<const uint8_t*>(kv) + (size_t)b * S_max * kDc * 2;
  const uint8_t* pe_b = reinterpret_cast<const uint8_t*>(pe) + (size_t)b * S_max * kDr * 2;
  {
    const int ln = opaque_lane();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int trow = 16 * wv + r;
      const int pu = max(__builtin_amdgcn_readfirstlane(s_pos[trow]), 0);
      lds_copy16(kv_b + (size_t)pu * (kDc * 2), ln * 16,
                 __builtin_amdgcn_readfirstlane(lds_addr(s_kv + trow * kTfPitch)));
    }
#pragma unroll
    for (int q8 = 0; q8 < 2; ++q8) {
      const int trow = 16 * wv + 8 * q8 + (ln >> 3);
      const int pu = max(s_pos[trow], 0);
      const int chunk = (ln & 7) ^ (trow & 7);
      lds_copy16_v(pe_b + (size_t)pu * (kDr * 2) + chunk * 16,
                   __builtin_amdgcn_readfirstlane(lds_addr(s_pe + (16 * wv + 8 * q8) * 128)));
    }
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  lds_barrier();  // every wave's copies have landed

  // Query fragments (B operand): head 16 ht + r16 of the group, K-step kk
  // holds dims 32 kk + 8g .. +7 of [q_nope | q_pe].
  uint4 qb[2][18];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int h = 16 * ht + r16;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      qb[ht][kk] = *reinterpret_cast<const uint4*>(s_qn + h * kTfQPitch + kk * 64 + g * 16);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      qb[ht][16 + kk] = *reinterpret_cast<const uint4*>(s_qp + h * kDr * 2 + kk * 64 + g * 16);
  }

  // ---- scores S^T[row][head] for rows 16w + 4g + i ----
  f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  {
    const int trow = 16 * wv + r16;
    const uint8_t* kb = s_kv + trow * kTfPitch;
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      const uint8_t* a = kk < 16 ? kb + ((4 * kk + g) << 4)
                                 : s_pe + trow * 128 + ((((kk - 16) * 4 + g) ^ (trow & 7)) << 4);
      const uint4 kf = *reinterpret_cast<const uint4*>(a);
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) sc[ht] = mfma_bf16_16x16x32(as_bf16x8(kf), as_bf16x8(qb[ht][kk]), sc[ht]);
    }
  }
  // Mask the empty rows, then the tile's maximum per head.
  float mx[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    mx[ht] = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = s_pos[16 * wv + 4 * g + i] >= 0;
      sc[ht][i] = valid ? sc[ht][i] * scale_log2 : -INFINITY;  // log2-domain score
      mx[ht] = fmaxf(mx[ht], sc[ht][i]);
    }
    mx[ht] = group_max(mx[ht]);
    if (g == 0) s_red[0][wv][16 * ht + r16] = mx[ht];
  }
  lds_barrier();
  float m_ref[2], psum[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    float m = s_red[0][0][16 * ht + r16];
#pragma unroll
    for (int w = 1; w < kTfWaves; ++w) m = fmaxf(m, s_red[0][w][16 * ht + r16]);
    m_ref[ht] = m;
    const float m_use = m == -INFINITY ? 0.f : m;
    float p[4];
    psum[ht] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2f(sc[ht][i] - m_use);
      psum[ht] += p[i];
    }
    // Half (wv & 1) of K-step wv / 2's B fragment for this head tile.
    uint32_t* dst = reinterpret_cast<uint32_t*>(&s_p[wv >> 1][ht][lane]) + 2 * (wv & 1);
    *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
    psum[ht] = group_sum(psum[ht]);
    if (g == 0) s_red[1][wv][16 * ht + r16] = psum[ht];
  }
  lds_barrier();  // P fragments and the per-wave sums are visible

  // ---- values O^T[c][head] for dims 128w .. 128w + 127 ----
  f32x4 o[8][2];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j][0] = o[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const uint8_t* vrow = s_kv + (4 * g + (r16 >> 2)) * kTfPitch + 8 * (r16 & 1);
    const int vch = (r16 & 3) >> 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 pb0 = s_p[ks][0][lane], pb1 = s_p[ks][1][lane];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ct = 8 * wv + j;
        const int off = (2 * ct + vch) << 4;
        const uint8_t* base = vrow + 32 * ks * kTfPitch + off;
        const i16x4 lo = lds_read_tr16(base);
        const i16x4 hi = lds_read_tr16(base + 16 * kTfPitch);
        const uint4 va = uint4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                               (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                               (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                               (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
        o[j][0] = mfma_bf16_16x16x32(as_bf16x8(va), as_bf16x8(pb0), o[j][0]);
        o[j][1] = mfma_bf16_16x16x32(as_bf16x8(va), as_bf16x8(pb1), o[j][1]);
      }
    }
  }

  // ---- finish ----
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int hl = 16 * ht + r16;  // head within the group
    const int head = hg * kTfHeads + hl;
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kTfWaves; ++w) l += s_red[1][w][hl];
    const float m = m_ref[ht];
    if (n_splits == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* orow = out + ((size_t)row * kHeads + head) * kDc + 4 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ct = 8 * wv + j;
        *reinterpret_cast<uint2*>(orow + ct * 16) =
            uint2{pack_bf16(o[j][ht][0] * inv, o[j][ht][1] * inv),
                  pack_bf16(o[j][ht][2] * inv, o[j][ht][3] * inv)};
      }
      if (lse != nullptr && wv == 0 && g == 0)
        lse[(size_t)row * kHeads + head] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
    } else {
      // Partial: the accumulator relative to 2^m, bf16, [item][tile][head][16].
      uint16_t* prow = part_o + (size_t)X * kHeads * kDc + head * 16 + 4 * g;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ct = 8 * wv + j;
        *reinterpret_cast<uint2*>(prow + ct * kHeads * 16) =
            uint2{pack_bf16(o[j][ht][0], o[j][ht][1]), pack_bf16(o[j][ht][2], o[j][ht][3])};
      }
      if (wv == 0 && g == 0) part_ml[(size_t)X * kHeads + head] = float4{m, l, 0.f, 0.f};
    }
  }
}

// ---- Wide form: many query rows -------------------------------------------
//
// Eight waves (two per SIMD).  The two contractions are split differently:
//   scores  S^T[row][head]: wave w takes head tile w (heads 16w..16w+15) over
//           all 576 score dims, its 18 query fragments in registers, with two
//           accumulators per 16-row tile (even and odd dim steps) so that four
//           MFMA chains are in flight.  Each wave reads the whole tile's K from
//           LDS; no partial scores cross between waves, so a tile needs one
//           barrier.  (Splitting the dims between the waves of a pair, so that
//           each K fragment fed two MFMAs and a tile's K was read four times
//           instead of eight, cost the exchange of partial scores and a second
//           barrier per tile, and was slower: batch-64 decode 67.7 against 64.5
//           us, prefill 5.44 against 5.04 ms);
//   values  O^T[c][head]: wave w takes latent dims 64w..64w+63 for all 128
//           heads (4 x 8 accumulator tiles, 128 registers), so each transposed
//           V fragment feeds 8 head tiles and V is read from LDS once per tile
//           instead of once per wave (a split by heads alone would read V
//           eight times through the transposing LDS read).
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
// Latent rows sit 1056 bytes apart (8 banks), chunks in order.  Measured with
// the LDS bank-conflict counter on gfx950, both the score reads (16 rows, one
// chunk each per quarter wave) and the transposing value reads (8 rows, two
// chunks each per half wave) are then free of conflicts; an XOR swizzle of
// the chunks of rows 8..15 by one, which a 16-lane model of the banks called
// neutral, made 40 % of the score reads' LDS cycles conflict cycles.
constexpr int kWdPitch = 1056;
constexpr int kWdTileKv = kWdRt * kWdPitch;
constexpr int kWdTileBytes = kWdTileKv + kWdRt * 128;
constexpr int kWdDims = kDc / kWdWaves;                 // latent dims per value wave (64)
constexpr int kWdCt = kWdDims / 16;                     // their 16-dim tiles (4)
constexpr int kWdSteps = (kDc + kDr) / 32;              // 32-dim score steps (16 latent, 2 rope)
static_assert(kWdSteps == 18 && kDc / 32 == 16, "latent steps 0-15, rope steps 16-17");
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

  // Query fragments of this wave's head tile: step j covers latent dims
  // 32j.. for j < 16, the rope part after.
  const int head = 16 * wave + r16;  // the head this lane scores and finishes
  uint4 qb[kWdSteps];
  {
    const uint16_t* qn = q_nope + ((size_t)row * kHeads + head) * kDc + g * 8;
    const uint16_t* qp = q_pe + ((size_t)row * kHeads + head) * kDr + g * 8;
#pragma unroll
    for (int j = 0; j < kWdSteps; ++j) qb[j] = ldg16(j < 16 ? qn + j * 32 : qp + (j - 16) * 32);
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
      // Lane L writes chunk L.
      lds_copy16(rowp, opaque_lane() * 16,
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
  // (whose P was written in the previous iteration): one barrier per tile.
#pragma unroll 1
  for (int it = 0; it <= n_tiles; ++it) {
    static_assert(kWdNbuf == 3, "slots: tile it-1 (values), tile it (scores), tile it+1 (copies)");
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // this wave's copies of tile it have landed
    lds_barrier();  // ... and every wave's; P(it-1) is visible; slot (it+1)%3 is free
    if (it + 1 < n_tiles) issue(it + 1);
    const int lane = opaque_lane(), g = lane >> 4, r16 = lane & 15;  // recomputed addresses
    const int head = 16 * wave + r16;

    // ---- scores of tile it for this wave's 16 heads; rows mt*16 + 4g + i ----
    f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const bool have_s = it < n_tiles;
    const int slot = it % kWdNbuf;
    if (have_s) {
      const uint8_t* buf = s_ring + slot * kWdTileBytes;
      // Latent step j of row tile mt is at the offset mt*16*pitch + 64*j from
      // one base.  The rope chunks (4j' + g) ^ (r16 & 7) differ per lane.
      const uint8_t* kb = buf + r16 * kWdPitch + (g << 4);
      const uint8_t* rb = buf + kWdTileKv + r16 * 128;
      // Two accumulators per row tile (even and odd steps): four independent
      // MFMA chains.
      f32x4 sh[2][2] = {{f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}},
                        {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
      for (int j = 0; j < kWdSteps; ++j) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint8_t* a = j < 16 ? kb + mt * 16 * kWdPitch + 64 * j
                                    : rb + mt * 16 * 128 + ((((j - 16) * 4 + g) ^ (r16 & 7)) << 4);
          const uint4 kf = *reinterpret_cast<const uint4*>(a);
          sh[j & 1][mt] = mfma_bf16_16x16x32(as_bf16x8(kf), as_bf16x8(qb[j]), sh[j & 1][mt]);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) sc[mt] = sh[0][mt] + sh[1][mt];
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
      // Rows 4g + r16/4 (+16).
      const uint8_t* vrow = s_ring + (pt % kWdNbuf) * kWdTileBytes +
                            (4 * g + (r16 >> 2)) * kWdPitch + 8 * (r16 & 1);
      const int vch = (r16 & 3) >> 1;
#pragma unroll
      for (int jh = 0; jh < kWdCt; jh += 2) {
        uint4 va[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int ct = kWdCt * wave + jh + jj;
          const int off = (2 * ct + vch) << 4;  // this lane's 16-byte chunk
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
#ifndef DSA_MLA_DENSE_SMALL_WORK
#define DSA_MLA_DENSE_SMALL_WORK 65536
#endif

// Few query rows (decode at small batch): the tile form, 32 heads and 64 rows
// per workgroup, so one query is spread over many CUs.  Otherwise 8-wave
// blocks of all 128 heads (every gathered row read once) and about one block
// per CU.
// The tile form up to 4 query rows: measured at 32K contexts, the stage takes
// 13.6 / 19.7 / 29.1 / 52.2 us at 2 / 4 / 8 / 16 rows with it and 20.4 / 23.0 /
// 25.1 / 30.4 us with the wide form, whose 8-wave workgroups gather each row
// once for all heads.  The dense baseline keeps its own threshold.
#ifndef DSA_MLA_TILE_ROWS
#define DSA_MLA_TILE_ROWS 4
#endif
#ifndef DSA_MLA_DENSE_TILE_ROWS
#define DSA_MLA_DENSE_TILE_ROWS 16
#endif

MlaPlan sparse_mla_plan(int B, int T, int k) {
  const long rows = (long)B * T;
  if (rows <= DSA_MLA_TILE_ROWS)  // one 64-row tile per workgroup of 32 heads
    return MlaPlan{kTfRows, (k + kTfRows - 1) / kTfRows, kTfWaves, true};
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
  // Few rows over a short context: the tile form, as on the sparse path;
  // otherwise 8-wave blocks, which gather every row once for all heads.
  if (rows <= DSA_MLA_DENSE_TILE_ROWS && (long)S_max * rows <= DSA_MLA_DENSE_SMALL_WORK)
    return MlaPlan{kTfRows, (ext + kTfRows - 1) / kTfRows, kTfWaves, true};
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
  if (plan.tile) {
    const unsigned grid = (unsigned)(((n_items + 7) / 8) * 8 * kTfGroups);
    hipLaunchKernelGGL((mla_tile_kernel<kDense>), dim3(grid), dim3(kTfThreads), 0, stream,
                       reinterpret_cast<const uint16_t*>(q_nope),
                       reinterpret_cast<const uint16_t*>(q_pe),
                       reinterpret_cast<const uint16_t*>(kv), reinterpret_cast<const uint16_t*>(pe),
                       idx, end_pos, T, S_max, k, plan.n_splits, n_items, softmax_scale * kLog2e,
                       reinterpret_cast<uint16_t*>(out), lse, part_o, part_ml);
    st = hipGetLastError() == hipSuccess ? 0 : -5;
  } else {
    hipLaunchKernelGGL((mla_wide_kernel<kDense>), dim3((unsigned)n_items), dim3(kWdThreads), 0,
                       stream, reinterpret_cast<const uint16_t*>(q_nope),
                       reinterpret_cast<const uint16_t*>(q_pe),
                       reinterpret_cast<const uint16_t*>(kv), reinterpret_cast<const uint16_t*>(pe),
                       idx, end_pos, T, S_max, k, plan.rows_per_split, plan.n_splits, n_items,
                       softmax_scale * kLog2e, reinterpret_cast<uint16_t*>(out), lse, part_o,
                       part_ml);
    st = hipGetLastError() == hipSuccess ? 0 : -5;
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
