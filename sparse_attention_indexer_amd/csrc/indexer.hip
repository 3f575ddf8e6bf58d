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
// Each wave keeps its query's 64x128 fragment in registers for its whole key
// range and streams keys straight from HBM into B-operand registers: a lane
// reads 64 contiguous bytes (bf16) or 32 (fp8) of one key row, 4 lanes cover a
// row, so every byte fetched is used once.  In the result tile a lane holds 4
// heads of one key; ReLU, weighting and the sum over its 16 head values happen
// in registers, and two cross-lane adds finish the sum over 64 heads.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kIdxHeads = 64;
constexpr int kIdxDim = 128;
constexpr int kIdxWaves = 4;
constexpr int kIdxTile = 16;

template <bool kFp8>
__global__ __launch_bounds__(256) void indexer_kernel(
    const void* __restrict__ q, const float* __restrict__ q_scale, const float* __restrict__ w,
    const void* __restrict__ k, const float* __restrict__ k_scale,
    const int32_t* __restrict__ end_pos, int T, int S_max, float scale, int blocks_per_row,
    int tiles_per_wave, float* __restrict__ out) {
  const int row = blockIdx.x / blocks_per_row;
  const int blk = blockIdx.x - row * blocks_per_row;
  const int b = row / T, t = row - b * T;
  const int ep = min(max(end_pos[b], T), S_max);
  const int bound = ep - T + t;  // last valid position, in [0, S_max)
  const int keys_per_block = kIdxWaves * tiles_per_wave * kIdxTile;
  const int blk_start = blk * keys_per_block;
  if (blk_start > bound) return;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;     // lane group: which 32 of the 128 dims this lane carries
  const int r16 = lane & 15;   // head within an M-tile (A) / key within a tile (B)

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

  float* orow = out + (size_t)row * S_max;

  if constexpr (!kFp8) {
    // A fragments: head mt*16 + r16, dims g*32 + kk*8 .. +7 for K-step kk.
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(q) + (size_t)row * kIdxHeads * kIdxDim;
    uint4 qa[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        qa[mt][kk] = ldg16(qrow + (mt * 16 + r16) * kIdxDim + g * 32 + kk * 8);
    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(k) + (size_t)b * S_max * kIdxDim;

    for (int tile = 0; tile < tiles_per_wave; ++tile) {
      const int s0 = blk_start + (tile * kIdxWaves + wave) * kIdxTile;
      if (s0 > bound) break;
      const int s = min(s0 + r16, bound);
      const uint16_t* kp = kbase + (size_t)s * kIdxDim + g * 32;
      uint4 kb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) kb[kk] = ldg16(kp + kk * 8);
      f32x4 acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt] = mfma_bf16_16x16x32(as_bf16x8(qa[mt][kk]), as_bf16x8(kb[kk]), acc[mt]);
      float v = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v += wv[mt][i] * fmaxf(acc[mt][i], 0.f);
      v += xor_shfl(v, 16);
      v += xor_shfl(v, 32);
      if (g == 0 && s0 + r16 <= bound) orow[s0 + r16] = v * scale;
    }
  } else {
    // A fragments: head mt*16 + r16, the 32 bytes g*32 .. g*32+31 of its 128 codes.
    const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q) + (size_t)row * kIdxHeads * kIdxDim;
    i32x8 qa[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint8_t* p = qrow + (mt * 16 + r16) * kIdxDim + g * 32;
      const uint4 lo = ldg16(p), hi = ldg16(p + 16);
      qa[mt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(k) + (size_t)b * S_max * kIdxDim;
    const float* ksrow = k_scale + (size_t)b * S_max;

    for (int tile = 0; tile < tiles_per_wave; ++tile) {
      const int s0 = blk_start + (tile * kIdxWaves + wave) * kIdxTile;
      if (s0 > bound) break;
      const int s = min(s0 + r16, bound);
      const uint8_t* kp = kbase + (size_t)s * kIdxDim + g * 32;
      const uint4 lo = ldg16(kp), hi = ldg16(kp + 16);
      const i32x8 kb = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const float ks = ksrow[s];
      float v = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 acc = mfma_fp8_16x16x128(qa[mt], kb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) v += wv[mt][i] * fmaxf(acc[i], 0.f);
      }
      v += xor_shfl(v, 16);
      v += xor_shfl(v, 32);
      if (g == 0 && s0 + r16 <= bound) orow[s0 + r16] = (v * ks) * scale;
    }
  }
}

int launch_index_scores(const void* q, const float* q_scale, const float* w, const void* k,
                        const float* k_scale, const int32_t* end_pos, int B, int T, int S_max,
                        int max_end_pos, float scale, int dtype, float* out, hipStream_t stream) {
  const long rows = (long)B * T;
  const long tiles_per_row = (max_end_pos + kIdxTile - 1) / kIdxTile;
  // Enough blocks to cover all 256 CUs several times over, but at least one
  // 16-key tile per wave and at most 16.
  long tpw = rows * tiles_per_row / (2048L * kIdxWaves);
  tpw = tpw < 1 ? 1 : (tpw > 16 ? 16 : tpw);
  const int keys_per_block = (int)(kIdxWaves * tpw * kIdxTile);
  const int blocks_per_row = (max_end_pos + keys_per_block - 1) / keys_per_block;
  const dim3 grid((unsigned)(rows * blocks_per_row));
  if (dtype == 0)
    hipLaunchKernelGGL(indexer_kernel<false>, grid, dim3(256), 0, stream, q, q_scale, w, k,
                       k_scale, end_pos, T, S_max, scale, blocks_per_row, (int)tpw, out);
  else
    hipLaunchKernelGGL(indexer_kernel<true>, grid, dim3(256), 0, stream, q, q_scale, w, k,
                       k_scale, end_pos, T, S_max, scale, blocks_per_row, (int)tpw, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace dsa
