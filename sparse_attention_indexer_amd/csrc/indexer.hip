// Lightning-indexer scores on gfx950.
//
//   I[b,t,s] = scale * ks[b,s] * sum_{h<64} w'[b,t,h] * ReLU(q[b,t,h,:] . k[b,s,:])
//
// (ReLU of each head's dot, then the head weight, then the sum over heads, as in
// kernelpool's fix in "mlx-lm PR #512 [WIP] deepseek v32"; fp8_index call of
// Indexer.forward on "DeepSeek-V3.2-Exp - Keep top-k positions".)
//
// Mapping: the 64 heads are the M dimension of 16x16 MFMA tiles (4 M-tiles),
// 16 cached keys are the N dimension, and the 128-dim dot is the K dimension.
// A workgroup stages its query (64x128) in LDS once; each wave then keeps the
// A fragments in registers for its whole key range and streams keys straight
// from HBM into B-operand registers, one tile ahead of the math: a lane reads
// 64 contiguous bytes (bf16) or 32 (fp8) of one key row, 4 lanes cover a row,
// so every byte fetched is used once.  In the result tile a lane holds 4
// heads of one key; ReLU, weighting and the sum over its 16 head values happen
// in registers, and two cross-lane adds finish the sum over 64 heads.
#include "dsa_device.h"
#include "dsa_launch.h"
#include "select.h"

namespace dsa {

// ReLU in one instruction: the IEEE-2019 maximum (v_maximum3_f32 on gfx950),
// which maps -0 to +0 like fmaxf but, unlike it, needs no NaN-quieting
// instruction before it (fmaxf(x, 0) cost two per element; the 8192-query
// prefill indexer went from 538 to 495 us with this form).
__device__ __forceinline__ float relu(float x) {
  return __builtin_elementwise_maximum(x, 0.0f);
}

constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kIdxWaves = 4;
constexpr int kIdxTile = 16;

#ifndef DSA_IDX_TARGET_BLOCKS
#define DSA_IDX_TARGET_BLOCKS 1024
#endif

// Key fragment of one 16-key tile for this lane: 64 bytes (bf16) or 32 (fp8)
// of key s, starting at dim 32*g, and (fp8) the key's scale, loaded with it so
// the epilogue never waits on a load of its own.
template <bool kFp8>
struct KeyFrag {
  uint4 v[kFp8 ? 2 : 4];
  float ks;
};

template <bool kFp8>
__device__ __forceinline__ KeyFrag<kFp8> load_key_frag(const uint8_t* kbase, const float* ksrow,
                                                       int s, int g) {
  KeyFrag<kFp8> f;
  constexpr int kRowBytes = kFp8 ? kIdxDim : 2 * kIdxDim;
  const uint8_t* p = kbase + (size_t)s * kRowBytes + g * (kRowBytes / 4);
#pragma unroll
  for (int u = 0; u < (kFp8 ? 2 : 4); ++u) f.v[u] = ldg16(p + 16 * u);
  f.ks = kFp8 ? ksrow[s] : 1.0f;
  return f;
}

template <bool kFp8>
__global__ __launch_bounds__(256) void indexer_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ end_pos, int T, int S_max, float scale, int blocks_per_row,
    int tiles_per_wave, float* __restrict__ out, uint32_t* __restrict__ topk_ctr) {
  // The block's 64x128 query in LDS, rows padded by 16 bytes so the 16 rows a
  // fragment read touches start on different banks.
  constexpr int kRowBytes = kFp8 ? kIdxDim : 2 * kIdxDim;
  constexpr int kQPitch = kRowBytes + 16;
  __shared__ __align__(16) uint8_t s_q[kIdxHeads * kQPitch];

  const int row = blockIdx.x / blocks_per_row;
  const int blk = blockIdx.x - row * blocks_per_row;
  const int b = row / T, t = row - b * T;
  const int ep = min(max(end_pos[b], T), S_max);
  const int bound = ep - T + t;  // last valid position, in [0, S_max)
  const int keys_per_block = kIdxWaves * tiles_per_wave * kIdxTile;
  const int blk_start = blk * keys_per_block;
  if (blk_start > bound) return;
  if (topk_ctr != nullptr && blk == 0 && threadIdx.x < 2) topk_ctr[4 * row + threadIdx.x] = 0u;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;     // lane group: which 32 of the 128 dims this lane carries
  const int r16 = lane & 15;   // head within an M-tile (A) / key within a tile (B)
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(k) + (size_t)b * S_max * kRowBytes;
  const float* ksrow = kFp8 ? k_scale + (size_t)b * S_max : nullptr;
  auto tile_start = [&](int tile) { return blk_start + (tile * kIdxWaves + wave) * kIdxTile; };

  // First key tile in flight before anything else.
  KeyFrag<kFp8> cur = load_key_frag<kFp8>(kbase, ksrow, min(tile_start(0) + r16, bound), g);

  // Query -> LDS: thread tid copies a quarter of head tid/4.
  {
    const int h = threadIdx.x >> 2, part = threadIdx.x & 3;
    const uint8_t* src = reinterpret_cast<const uint8_t*>(q) +
                         ((size_t)row * kIdxHeads + h) * kRowBytes + part * (kRowBytes / 4);
    uint8_t* dst = s_q + h * kQPitch + part * (kRowBytes / 4);
#pragma unroll
    for (int u = 0; u < kRowBytes / 64; ++u)
      *reinterpret_cast<uint4*>(dst + 16 * u) = ldg16(src + 16 * u);
  }

  // Per-lane weights for the 16 heads whose results this lane will hold:
  // head = mt*16 + 4*g + i for M-tile mt and result element i.
  float wv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = mt * 16 + 4 * g + i;
      float wh = w[(size_t)row * kIdxHeads + h];
      if constexpr (kFp8) wh *= q_scale[(size_t)row * kIdxHeads + h];
      wv[mt][i] = wh;
    }
  __syncthreads();

  // A fragments: head mt*16 + r16, bytes [g*R/4, (g+1)*R/4) of its row.
  uint4 qa[4][kFp8 ? 2 : 4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int u = 0; u < (kFp8 ? 2 : 4); ++u)
      qa[mt][u] = *reinterpret_cast<const uint4*>(s_q + (mt * 16 + r16) * kQPitch +
                                                  g * (kRowBytes / 4) + 16 * u);

  float* orow = out + (size_t)row * S_max;

  for (int tile = 0; tile < tiles_per_wave; ++tile) {
    const int s0 = tile_start(tile);
    if (s0 > bound) break;
    const int s0n = tile_start(tile + 1);
    const bool has_next = tile + 1 < tiles_per_wave && s0n <= bound;
    KeyFrag<kFp8> nxt;
    if (has_next) nxt = load_key_frag<kFp8>(kbase, ksrow, min(s0n + r16, bound), g);

    float v = 0.f;
    if constexpr (!kFp8) {
      f32x4 acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt] = mfma_bf16_16x16x32(as_bf16x8(qa[mt][kk]), as_bf16x8(cur.v[kk]), acc[mt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v += wv[mt][i] * relu(acc[mt][i]);
    } else {
      const i32x8 kb = i32x8{(int)cur.v[0].x, (int)cur.v[0].y, (int)cur.v[0].z, (int)cur.v[0].w,
                             (int)cur.v[1].x, (int)cur.v[1].y, (int)cur.v[1].z, (int)cur.v[1].w};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const i32x8 a = i32x8{(int)qa[mt][0].x, (int)qa[mt][0].y, (int)qa[mt][0].z,
                              (int)qa[mt][0].w, (int)qa[mt][1].x, (int)qa[mt][1].y,
                              (int)qa[mt][1].z, (int)qa[mt][1].w};
        const f32x4 acc = mfma_fp8_16x16x128(a, kb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) v += wv[mt][i] * relu(acc[i]);
      }
    }
    v = group_sum(v);
    const int s = s0 + r16;
    if (g == 0 && s <= bound) {
      if constexpr (kFp8) v *= cur.ks;
      orow[s] = v * scale;
    }
    if (has_next) cur = nxt;
  }
}

// Streaming form of the decode kernel, for long key ranges per wave (at least
// 4 tiles): the same products, but each wave copies its key tiles straight
// from HBM into its own LDS ring (global_load_lds, 16 bytes a lane, issued
// through inline asm so that the compiler's waits never cover them, with the
// non-temporal hint: each key is read once, and a single pass over a large
// buffer runs closer to the HBM peak that way) and keeps
// kDepth tiles in flight; a tile's wait is a fixed vmcnt (every copy is
// issued, clamped to the workgroup's last key), and no barrier is needed since
// a wave reads only the slots it filled.  The 16-byte chunks of key row r sit
// XOR-swizzled by r & 7, so the B-fragment reads (16 rows, one or two chunks
// each) spread over the banks.  Scores are collected in LDS and stored after
// the wave's last tile, so no store sits between the copies the loop waits
// for.
constexpr int kIdxMaxTpw = 16;  // key tiles per wave, at most

template <bool kFp8>
__global__ __launch_bounds__(256) void indexer_stream_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ end_pos, int T, int S_max, float scale, int blocks_per_row,
    int tiles_per_wave, float* __restrict__ out, uint32_t* __restrict__ topk_ctr) {
  constexpr int kRowBytes = kFp8 ? kIdxDim : 2 * kIdxDim;
  constexpr int kDepth = kFp8 ? 4 : 2;                      // tiles in flight per wave
  constexpr int kLanesPerKey = kRowBytes / 16;              // 8 (fp8) or 16 (bf16)
  constexpr int kKeysPerCopy = kWave / kLanesPerKey;        // 8 or 4
  constexpr int kKeyCopies = kIdxTile / kKeysPerCopy;       // 2 or 4
  constexpr int kCopies = kKeyCopies + (kFp8 ? 1 : 0);      // + the tile's 16 scales
  constexpr int kSlotBytes = kIdxTile * kRowBytes + (kFp8 ? 16 * 4 : 0);
  __shared__ __align__(16) uint8_t s_q[kIdxHeads * kRowBytes];
  __shared__ __align__(16) uint8_t s_ring[kIdxWaves][kDepth][kSlotBytes];
  __shared__ float s_out[kIdxWaves][kIdxMaxTpw * kIdxTile];
  __shared__ __align__(16) float s_w[2][kIdxHeads];  // head weights, then (fp8) q scales

  const int row = blockIdx.x / blocks_per_row;
  const int blk = blockIdx.x - row * blocks_per_row;
  const int b = row / T, t = row - b * T;
  const int ep = min(max(end_pos[b], T), S_max);
  const int bound = ep - T + t;  // last valid position, in [0, S_max)
  const int keys_per_block = kIdxWaves * tiles_per_wave * kIdxTile;
  const int blk_start = blk * keys_per_block;
  if (blk_start > bound) return;
  if (topk_ctr != nullptr && blk == 0 && threadIdx.x < 2) topk_ctr[4 * row + threadIdx.x] = 0u;

  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(k) + (size_t)b * S_max * kRowBytes;
  const float* ksrow = kFp8 ? k_scale + (size_t)b * S_max : nullptr;
  const int last = min(bound, blk_start + keys_per_block - 1);  // the workgroup's last key
  auto tile_start = [&](int tile) { return blk_start + (tile * kIdxWaves + wave) * kIdxTile; };
  // Tiles of this wave that hold a valid key.
  const int first = blk_start + wave * kIdxTile;
  const int n_tiles = first > bound ? 0 : min(tiles_per_wave, (bound - first) / (kIdxWaves * kIdxTile) + 1);

  // The query and the head weights go to LDS by copies as well, issued before
  // the first tiles' copies: one wait covers them and leaves the tiles in
  // flight.  The query is unpadded, chunk c of head h at chunk c ^ (h & 7)
  // (as the keys), the weights and (fp8) query scales one float a lane.
  {
    constexpr int kHeadsPerCopy = kWave / kLanesPerKey;                    // 8 or 4
    constexpr int kQCopiesPerWave = kIdxHeads / kHeadsPerCopy / kIdxWaves;  // 2 or 4
    const int ln = opaque_lane();
    const uint8_t* qrow =
        reinterpret_cast<const uint8_t*>(q) + (size_t)row * kIdxHeads * kRowBytes;
#pragma unroll
    for (int c = 0; c < kQCopiesPerWave; ++c) {
      const int cc = wave * kQCopiesPerWave + c;
      const int h = cc * kHeadsPerCopy + ln / kLanesPerKey;
      const int chunk = (ln % kLanesPerKey) ^ (h & 7);
      lds_copy16_v(qrow + h * kRowBytes + chunk * 16,
                   __builtin_amdgcn_readfirstlane(lds_addr(s_q + cc * 1024)));
    }
    if (wave == 0)
      lds_copy4_v(reinterpret_cast<const uint8_t*>(w + (size_t)row * kIdxHeads + ln),
                  __builtin_amdgcn_readfirstlane(lds_addr(&s_w[0][0])));
    if (kFp8 && wave == 1)
      lds_copy4_v(reinterpret_cast<const uint8_t*>(q_scale + (size_t)row * kIdxHeads + ln),
                  __builtin_amdgcn_readfirstlane(lds_addr(&s_w[1][0])));
  }

  // Copies of tile `tile` into ring slot tile % kDepth: copy c puts keys
  // kKeysPerCopy*c .. +kKeysPerCopy-1 (lane L: key L / kLanesPerKey, slot
  // chunk L % kLanesPerKey, holding the row's chunk (L % kLanesPerKey) ^
  // (key & 7)); with fp8 one more copy puts the 16 scales (lanes 0..15).
  auto issue = [&](int tile) {
    uint8_t* slot = &s_ring[wave][tile % kDepth][0];
    const int s0 = tile_start(tile);
    const int ln = opaque_lane();
#pragma unroll
    for (int c = 0; c < kKeyCopies; ++c) {
      const int key = c * kKeysPerCopy + ln / kLanesPerKey;
      const int chunk = (ln % kLanesPerKey) ^ (key & 7);
      const int s = min(s0 + key, last);
      lds_copy16_v_nt(kbase + (size_t)s * kRowBytes + chunk * 16,
                      __builtin_amdgcn_readfirstlane(lds_addr(slot + c * 1024)));
    }
    if constexpr (kFp8) {
      if (ln < kIdxTile)
        lds_copy4_v_nt(reinterpret_cast<const uint8_t*>(ksrow + min(s0 + ln, last)),
                       __builtin_amdgcn_readfirstlane(lds_addr(slot + kIdxTile * kRowBytes)));
    }
  };
#pragma unroll
  for (int j = 0; j < kDepth; ++j) issue(j);

  // Everything but the first tiles has landed (this wave's copies), and the
  // other waves' too after the barrier.
  __builtin_amdgcn_s_waitcnt(wait_vm(kDepth * kCopies));
  lds_barrier();
  float wv[4][4];  // weights of the 16 heads whose results this lane holds
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = mt * 16 + 4 * g + i;
      wv[mt][i] = kFp8 ? s_w[0][h] * s_w[1][h] : s_w[0][h];
    }
  uint4 qa[4][kFp8 ? 2 : 4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int h = mt * 16 + r16;
#pragma unroll
    for (int u = 0; u < (kFp8 ? 2 : 4); ++u)
      qa[mt][u] = *reinterpret_cast<const uint4*>(
          s_q + h * kRowBytes + ((((kRowBytes / 64) * g + u) ^ (h & 7)) << 4));
  }

#pragma unroll 1
  for (int tile = 0; tile < n_tiles; ++tile) {
    __builtin_amdgcn_s_waitcnt(wait_vm((kDepth - 1) * kCopies));  // this tile's copies have landed
    const uint8_t* slot = &s_ring[wave][tile % kDepth][0];
    const uint8_t* krow = slot + r16 * kRowBytes;
    float v = 0.f;
    if constexpr (!kFp8) {
      uint4 kb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        kb[u] = *reinterpret_cast<const uint4*>(krow + (((4 * g + u) ^ (r16 & 7)) << 4));
      f32x4 acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt] = mfma_bf16_16x16x32(as_bf16x8(qa[mt][kk]), as_bf16x8(kb[kk]), acc[mt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v += wv[mt][i] * relu(acc[mt][i]);
    } else {
      const uint4 k0 = *reinterpret_cast<const uint4*>(krow + (((2 * g) ^ (r16 & 7)) << 4));
      const uint4 k1 = *reinterpret_cast<const uint4*>(krow + (((2 * g + 1) ^ (r16 & 7)) << 4));
      const i32x8 kb = i32x8{(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w,
                             (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const i32x8 a = i32x8{(int)qa[mt][0].x, (int)qa[mt][0].y, (int)qa[mt][0].z,
                              (int)qa[mt][0].w, (int)qa[mt][1].x, (int)qa[mt][1].y,
                              (int)qa[mt][1].z, (int)qa[mt][1].w};
        const f32x4 acc = mfma_fp8_16x16x128(a, kb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) v += wv[mt][i] * relu(acc[i]);
      }
      v *= reinterpret_cast<const float*>(slot + kIdxTile * kRowBytes)[r16];
    }
    v = group_sum(v);
    if (g == 0) s_out[wave][tile * kIdxTile + r16] = v * scale;
    // The slot's reads are done (their values fed the math): refill it.
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    issue(tile + kDepth);
  }
  // No copy may still be writing LDS when the workgroup ends.
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  float* orow = out + (size_t)row * S_max;
  for (int i = lane; i < n_tiles * kIdxTile; i += kWave) {
    const int s = tile_start(i / kIdxTile) + (i % kIdxTile);
    if (s <= bound) orow[s] = s_out[wave][i];
  }
}

// ---------------------------------------------------------------------------
// Prefill form (many queries per sequence): the same products as one GEMM of
// the queries' [T*64, 128] against the keys' [S, 128]^T.  A 256-thread
// workgroup takes 8 consecutive queries (two per wave, their 64 heads held
// as A fragments in registers) and a chunk of up to 2048 keys of the causal
// range (8192-token prefill: 535 us, against 578 us with 512 threads, 16
// queries and 1024 keys).  Key tiles of 64 rows are copied into LDS (global_load_lds, 16
// bytes a lane, two tiles in flight) with their 16-byte chunks XOR-swizzled
// by row so the B-fragment reads hit distinct banks; every B fragment feeds
// eight MFMAs (2 queries x 4 head tiles).  The ReLU, head weights and the sum
// over heads stay in registers as in the decode form.
constexpr int kPfWaves = 4;
constexpr int kPfQ = 2 * kPfWaves;      // queries per workgroup
constexpr int kPfTile = 64;             // keys per LDS tile
constexpr int kPfChunk = 2048;          // keys per workgroup

// Position of 16-byte chunk c of key row r inside the row's LDS copy.
template <bool kFp8>
__device__ __forceinline__ int pf_swz(int r, int c) {
  return kFp8 ? (c ^ ((r >> 1) & 7)) : (c ^ (r & 15));
}


typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

template <bool kFp8>
__global__ __launch_bounds__(kPfWaves * 64) void indexer_prefill_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ end_pos, int T, int S_max, float scale, int n_qblk,
    int n_chunks, float* __restrict__ out, uint32_t* __restrict__ topk_ctr) {
  constexpr int kRowBytes = kFp8 ? kIdxDim : 2 * kIdxDim;
  constexpr int kChunks = kRowBytes / 16;                  // 16-byte chunks per key row
  constexpr int kTileBytes = kPfTile * kRowBytes;
  constexpr int kCopies = kTileBytes / 1024 / kPfWaves;    // 1 KiB copies per wave per tile
  constexpr int kRowsPerCopy = 1024 / kRowBytes;
  __shared__ __align__(16) uint8_t s_k[2][kTileBytes];

  // The query block varies fastest: workgroups go to the 8 XCDs round robin,
  // and with the key chunk fastest XCD x would get chunk x of every query
  // block, so the XCDs holding the early chunks (active for every causal
  // query block) would carry most of the work.
  const int bid = blockIdx.x;
  const int qblk = bid % n_qblk, rest = bid / n_qblk;
  const int chunk = rest % n_chunks, b = rest / n_chunks;
  const int t0 = qblk * kPfQ;
  const int ep = min(max(end_pos[b], T), S_max);
  const int t_last = min(t0 + kPfQ - 1, T - 1);
  const int bound_max = ep - T + t_last;  // last key any query of the block may see
  const int s_begin = chunk * kPfChunk;
  if (s_begin > bound_max) return;
  const int n_keys = min(kPfChunk, bound_max + 1 - s_begin);
  const int n_tiles = (n_keys + kPfTile - 1) / kPfTile;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  if (topk_ctr != nullptr && chunk == 0 && tid < 2 * kPfQ && t0 + tid / 2 < T)
    topk_ctr[4 * ((size_t)b * T + t0 + tid / 2) + (tid & 1)] = 0u;

  const uint8_t* kb = reinterpret_cast<const uint8_t*>(k) + (size_t)b * S_max * kRowBytes;
  // Wave w copies rows [kRowsPerCopy*(kCopies*w + j), +kRowsPerCopy) of a tile.
  auto issue = [&](int tile) {
    uint8_t* dst = s_k[tile & 1];
#pragma unroll
    for (int j = 0; j < kCopies; ++j) {
      const int r = kRowsPerCopy * (kCopies * wave + j) + lane / kChunks;
      const int p = lane % kChunks;
      const int s = min(s_begin + tile * kPfTile + r, S_max - 1);
      __builtin_amdgcn_global_load_lds(
          (glb_void_t*)(kb + (size_t)s * kRowBytes + pf_swz<kFp8>(r, p) * 16),
          (lds_void_t*)(dst + kRowsPerCopy * (kCopies * wave + j) * kRowBytes), 16, 0, 0);
    }
  };
  issue(0);
  if (n_tiles > 1) issue(1);

  // A fragments of the wave's two queries: head mt*16 + r16, dims of K-step kk.
  int tq[2];
  uint4 qa[2][4][kFp8 ? 2 : 4];
  float wv[2][4][4];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    tq[qq] = t0 + 2 * wave + qq;
    const int tt = min(tq[qq], T - 1);
    const size_t qrow = (size_t)b * T + tt;
    const uint8_t* qbase = reinterpret_cast<const uint8_t*>(q) + qrow * kIdxHeads * kRowBytes;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int u = 0; u < (kFp8 ? 2 : 4); ++u)
        qa[qq][mt][u] = ldg16(qbase + (mt * 16 + r16) * kRowBytes + g * (kRowBytes / 4) + 16 * u);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = mt * 16 + 4 * g + i;
        float wh = w[qrow * kIdxHeads + h];
        if constexpr (kFp8) wh *= q_scale[qrow * kIdxHeads + h];
        wv[qq][mt][i] = tq[qq] < T ? wh : 0.f;
      }
  }
  const int bound0 = ep - T + tq[0], bound1 = ep - T + tq[1];
  float* orow0 = out + ((size_t)b * T + min(tq[0], T - 1)) * S_max;
  float* orow1 = out + ((size_t)b * T + min(tq[1], T - 1)) * S_max;
  const float* ksrow = kFp8 ? k_scale + (size_t)b * S_max : nullptr;

#pragma unroll 1
  for (int tile = 0; tile < n_tiles; ++tile) {
    if (tile + 1 < n_tiles)
      __builtin_amdgcn_s_waitcnt(wait_vm(kCopies));  // the next tile may stay in flight
    else
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
    lds_barrier();
    const uint8_t* buf = s_k[tile & 1];
#pragma unroll
    for (int nt = 0; nt < kPfTile / 16; ++nt) {
      const int r = nt * 16 + r16;  // key row of this lane's B fragment
      f32x4 acc[2][4];
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[qq][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (!kFp8) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          // Same K order as the A fragments: lane group g, step kk holds dims
          // 32g + 8kk .. +7, i.e. chunk 4g + kk of the key row.
          const uint4 bv =
              *reinterpret_cast<const uint4*>(buf + r * kRowBytes + pf_swz<false>(r, 4 * g + kk) * 16);
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
              acc[qq][mt] = mfma_bf16_16x16x32(as_bf16x8(qa[qq][mt][kk]), as_bf16x8(bv), acc[qq][mt]);
        }
      } else {
        const uint4 b0 =
            *reinterpret_cast<const uint4*>(buf + r * kRowBytes + pf_swz<true>(r, 2 * g) * 16);
        const uint4 b1 =
            *reinterpret_cast<const uint4*>(buf + r * kRowBytes + pf_swz<true>(r, 2 * g + 1) * 16);
        const i32x8 bb = i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                               (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const i32x8 a = i32x8{(int)qa[qq][mt][0].x, (int)qa[qq][mt][0].y,
                                  (int)qa[qq][mt][0].z, (int)qa[qq][mt][0].w,
                                  (int)qa[qq][mt][1].x, (int)qa[qq][mt][1].y,
                                  (int)qa[qq][mt][1].z, (int)qa[qq][mt][1].w};
            acc[qq][mt] = mfma_fp8_16x16x128(a, bb, acc[qq][mt]);
          }
      }
      // Epilogue: ReLU, head weights, sum over the 64 heads.
      float v[2];
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        float x = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) x += wv[qq][mt][i] * relu(acc[qq][mt][i]);
        v[qq] = group_sum(x);
      }
      const int s = s_begin + tile * kPfTile + nt * 16 + r16;
      if (g == 0) {
        const float ks = kFp8 ? ksrow[min(s, S_max - 1)] : 1.f;
        if (s <= bound0 && tq[0] < T) orow0[s] = v[0] * ks * scale;
        if (s <= bound1 && tq[1] < T) orow1[s] = v[1] * ks * scale;
      }
    }
    lds_barrier();  // every wave is done with this buffer before it is refilled
    if (tile + 2 < n_tiles) issue(tile + 2);
  }
}

int launch_index_scores(const void* q, const float* q_scale, const float* w, const void* k,
                        const float* k_scale, const int32_t* end_pos, int B, int T, int S_max,
                        int max_end_pos, float scale, int dtype, float* out, uint32_t* topk_ctr,
                        hipStream_t stream) {
  const long rows = (long)B * T;
  if (T >= kPfQ) {  // prefill form
    const int n_qblk = (T + kPfQ - 1) / kPfQ;
    const int n_chunks = (max_end_pos + kPfChunk - 1) / kPfChunk;
    const dim3 grid((unsigned)((long)B * n_qblk * n_chunks));
    if (dtype == 0)
      hipLaunchKernelGGL(indexer_prefill_kernel<false>, grid, dim3(kPfWaves * 64), 0, stream, q,
                         q_scale, w, k, k_scale, end_pos, T, S_max, scale, n_qblk, n_chunks, out,
                         topk_ctr);
    else
      hipLaunchKernelGGL(indexer_prefill_kernel<true>, grid, dim3(kPfWaves * 64), 0, stream, q,
                         q_scale, w, k, k_scale, end_pos, T, S_max, scale, n_qblk, n_chunks, out,
                         topk_ctr);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  const long tiles_per_row = (max_end_pos + kIdxTile - 1) / kIdxTile;
  // About 1024 workgroups (four per CU), at least one 16-key tile per wave and
  // at most 16: long key ranges per wave then take the streaming form.
  long tpw = rows * tiles_per_row / ((long)DSA_IDX_TARGET_BLOCKS * kIdxWaves);
  tpw = tpw < 1 ? 1 : (tpw > kIdxMaxTpw ? kIdxMaxTpw : tpw);
  const int keys_per_block = (int)(kIdxWaves * tpw * kIdxTile);
  const int blocks_per_row = (max_end_pos + keys_per_block - 1) / keys_per_block;
  const dim3 grid((unsigned)(rows * blocks_per_row));
  if (tpw >= 4) {  // long key ranges per wave: the streaming form
    if (dtype == 0)
      hipLaunchKernelGGL(indexer_stream_kernel<false>, grid, dim3(256), 0, stream, q, q_scale, w,
                         k, k_scale, end_pos, T, S_max, scale, blocks_per_row, (int)tpw, out,
                         topk_ctr);
    else
      hipLaunchKernelGGL(indexer_stream_kernel<true>, grid, dim3(256), 0, stream, q, q_scale, w,
                         k, k_scale, end_pos, T, S_max, scale, blocks_per_row, (int)tpw, out,
                         topk_ctr);
    return hipGetLastError() == hipSuccess ? 0 : -5;
  }
  if (dtype == 0)
    hipLaunchKernelGGL(indexer_kernel<false>, grid, dim3(256), 0, stream, q, q_scale, w, k,
                       k_scale, end_pos, T, S_max, scale, blocks_per_row, (int)tpw, out,
                       topk_ctr);
  else
    hipLaunchKernelGGL(indexer_kernel<true>, grid, dim3(256), 0, stream, q, q_scale, w, k,
                       k_scale, end_pos, T, S_max, scale, blocks_per_row, (int)tpw, out,
                       topk_ctr);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace dsa
