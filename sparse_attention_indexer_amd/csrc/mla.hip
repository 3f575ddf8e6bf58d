// Absorbed-MLA attention over gathered cached rows on gfx950 (the MQA decode
// branch of "DeepSeek-V3.2-Exp - Apply sparse mask", restricted to the rows the
// indexer selected; the dense variant takes every causally valid row).
//
//   z[h,j] = (q_nope[h,:] . kv[pos_j,:] + q_pe[h,:] . pe[pos_j,:]) * softmax_scale
//   out[h,:] = sum_j softmax_j(z[h,:]) * kv[pos_j,:]
//
// Work item: one query row and one split of its row list, all 128 heads.  A
// 512-thread workgroup has 8 waves of 16 heads (two waves per SIMD, so one
// wave's LDS reads overlap the other's MFMAs); it walks its split 64 rows at a
// time, so every gathered row is read from HBM once for all heads.
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

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

__device__ __forceinline__ i16x4 lds_read_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// max / sum over the 4 lanes l%16 + 16j that hold the same head.
__device__ __forceinline__ float group_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = __int_as_float(a[0]) + __int_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}
__device__ __forceinline__ uint32_t pack_half(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

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

  int n_list;  // entries in this row's list
  if constexpr (kDense) {
    const int ep = min(max(end_pos[b], T), S_max);
    n_list = ep - T + t + 1;
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
      if constexpr (kDense) {
        pos = j_begin + j;
      } else {
        pos = idx[(size_t)row * k + j_begin + j];
        if (pos < 0 || pos >= S_max) pos = -1;
      }
    }
    return pos;
  };

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
      __builtin_amdgcn_global_load_lds((glb_void*)(kv_b + (size_t)rpos[r] * (kDc * 2) + lane * 16),
                                       (lds_void*)(base + trow * kKvPitch), 16, 0, 0);
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
      __builtin_amdgcn_global_load_lds((glb_void*)(pe_b + (size_t)pos * (kDr * 2) + chunk * 16),
                                       (lds_void*)(base + kTileKv + (kRw * wv + 8 * q8) * 128),
                                       16, 0, 0);
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
    const bool grow = mx > m_run + kRescaleSlack;
    if (__ballot(grow) != 0) {
      const float m_new = grow ? mx : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - m_new);
      m_run = m_new;
      l_part *= alpha;
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) o[ct] *= alpha;
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
    // Partial output o/l in fp16, scaled by a power of two that puts its
    // largest element in [2^14, 2^15) (fp16 keeps 11 significant bits at any
    // magnitude of the cache values), plus (max, sum, 1/scale) in fp32.
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float amax = 0.f;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[ct][i]));
    amax = group_max(amax) * inv;
    int e;
    frexpf(amax, &e);  // amax < 2^e
    e = min(max(e, -100), 100);
    const float sc = ldexpf(inv, 15 - e);
    uint16_t* prow = part_o + ((size_t)X * kHeads + head) * kDc + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 32; ++ct)
      *reinterpret_cast<uint2*>(prow + ct * 16) =
          uint2{pack_half(o[ct][0] * sc, o[ct][1] * sc), pack_half(o[ct][2] * sc, o[ct][3] * sc)};
    if (g == 0) part_ml[(size_t)X * kHeads + head] = float4{m_run, l_tot, ldexpf(1.f, e - 15), 0.f};
  }
}

__device__ __forceinline__ float half_lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Merge the per-split partial outputs of one (row, head) per 128-thread block;
// each thread owns 4 latent dims.  The splits are read 32 at a time (their
// loads all in flight together), with an online maximum across batches, so a
// decode row with up to 32 splits costs one round trip to memory.
__global__ __launch_bounds__(128) void mla_combine_kernel(const uint16_t* __restrict__ part_o,
                                                          const float4* __restrict__ part_ml,
                                                          int n_splits, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  constexpr int kBatch = 32;
  const int rh = blockIdx.x;  // row * 128 + head
  const int row = rh / kHeads, head = rh - row * kHeads;
  const int tid = threadIdx.x;
  const float4* ml = part_ml + (size_t)row * n_splits * kHeads + head;
  const int c0 = tid * 4;
  const uint16_t* src = part_o + ((size_t)row * n_splits * kHeads + head) * kDc + c0;
  const size_t stride = (size_t)kHeads * kDc;
  float4 acc = float4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f, M = -INFINITY;
  __shared__ float4 s_ml[kBatch];
  for (int s0 = 0; s0 < n_splits; s0 += kBatch) {
    // The batch's partials and its (max, sum, 1/scale) triples, all in
    // flight at once; the triples go through LDS to every thread.
    uint2 a[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      a[u] = *reinterpret_cast<const uint2*>(src + (size_t)min(s0 + u, n_splits - 1) * stride);
    if (tid < kBatch) s_ml[tid] = ml[(size_t)min(s0 + tid, n_splits - 1) * kHeads];
    __syncthreads();
    float4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = s_ml[u];
    __syncthreads();  // s_ml is refilled by the next batch
    float mb = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (s0 + u < n_splits && v[u].y > 0.f) mb = fmaxf(mb, v[u].x);
    if (mb == -INFINITY) continue;  // nothing kept so far
    const float alpha = M == -INFINITY ? 0.f : exp2f(M - mb);
    M = mb;
    L *= alpha;
    acc.x *= alpha;
    acc.y *= alpha;
    acc.z *= alpha;
    acc.w *= alpha;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      // Split weight: its sum times 2^(its max - M); the stored partial is
      // o/sum times a power-of-two scale whose inverse is v.z.
      const float w = (s0 + u < n_splits && v[u].y > 0.f) ? v[u].y * exp2f(v[u].x - M) : 0.f;
      const float ws = w * v[u].z;
      L += w;
      acc.x += half_lo(a[u].x) * ws;
      acc.y += half_hi(a[u].x) * ws;
      acc.z += half_lo(a[u].y) * ws;
      acc.w += half_hi(a[u].y) * ws;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<uint2*>(out + (size_t)rh * kDc + c0) =
      uint2{pack_bf16(acc.x * inv, acc.y * inv), pack_bf16(acc.z * inv, acc.w * inv)};
  if (lse != nullptr && tid == 0) lse[rh] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

static int round_up(int x, int m) { return (x + m - 1) / m * m; }

#ifndef DSA_MLA_TARGET_BLOCKS
#define DSA_MLA_TARGET_BLOCKS 256
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

// Few query rows (decode at small batch): 2-wave blocks of 32 heads (16 rows
// per wave per tile) and short splits, so one query is spread over many CUs.
// Otherwise 8-wave blocks of all 128 heads (every gathered row read once) and
// about one block per CU.
MlaPlan sparse_mla_plan(int B, int T, int k) {
  const long rows = (long)B * T;
  if (rows <= DSA_MLA_SMALL_ROWS) {
    // Splits of k*rows/128 rows (a power of two, at least DSA_MLA_SMALL_SPLIT_MIN):
    // about 128 items of 2 head groups each.
    int rps = DSA_MLA_SMALL_SPLIT_MIN;
    while (rps < kMaxSplitRows && (long)rps * 128 < (long)k * rows) rps *= 2;
    return MlaPlan{rps, (k + rps - 1) / rps, 2};
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
    return MlaPlan{rps, (ext + rps - 1) / rps, 2};
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
  if (plan.waves == 2)
    st = launch_mla_shape<kDense, 2, 16>(q_nope, q_pe, kv, pe, idx, end_pos, T, S_max, k, plan,
                                         rows, softmax_scale, out, lse, part_o, part_ml, stream);
  else
    st = launch_mla_shape<kDense, 8, 8>(q_nope, q_pe, kv, pe, idx, end_pos, T, S_max, k, plan,
                                        rows, softmax_scale, out, lse, part_o, part_ml, stream);
  if (st) return st;
  if (plan.n_splits > 1) {
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)(rows * kHeads)), dim3(128), 0, stream,
                       part_o, part_ml, plan.n_splits, reinterpret_cast<uint16_t*>(out), lse);
    if (hipGetLastError() != hipSuccess) return -5;
  }
  return 0;
}

int launch_sparse_mla(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                      const int32_t* idx, int B, int T, int S_max, int k, float softmax_scale,
                      void* out, float* lse, void* workspace, hipStream_t stream) {
  const MlaPlan plan = sparse_mla_plan(B, T, k);
  return launch_mla<false>(q_nope, q_pe, kv, pe, idx, nullptr, B, T, S_max, k, plan,
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
