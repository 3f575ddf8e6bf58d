// Query absorption and output up-projection on gfx950: the two per-head
// products on either side of the absorbed attention in the MQA decode branch
// of "DeepSeek-V3.2-Exp - Apply sparse mask" (wkv_b viewed as [heads,
// 128 + v_head_dim, 512]):
//
//   q_abs[r,h,c] = sum_{d<128} q_nope[r,h,d] * wkv_b[h, d, c]          (absorb)
//   y[r,h,d]     = sum_{c<512} x[r,h,c]      * wkv_b[h, 128 + d, c]    (up-projection)
//
// r runs over the B*T query rows.  Both are head-batched GEMMs on 16x16x32
// bf16 MFMA with fp32 accumulation; a workgroup takes a quarter of one head's
// 128 KiB weight slice and 64 query rows, so the slice is read from HBM once
// per 64 rows (at decode, once in all: these products are weight-bandwidth
// bound there, and four workgroups per head spread the stream over the CUs;
// the up-projection of many rows keeps one workgroup per head and row block).
//
// Absorb.  The contraction runs over d, which is the row index of the weight
// slice (its rows are 512 contiguous c values), so the product is computed
// transposed, q_abs^T[c][r] = W^T[c][d] . q^T[d][r]: the workgroup's 128
// columns of the slice are copied into LDS (rows padded by 16 bytes) and the
// A fragments W^T are read from it with ds_read_b64_tr_b16; the query rows
// are staged in LDS too and read as B fragments in the same K order
// (d = 32s + 4g + j and 32s + 16 + 4g + j for lane group g).  Eight waves
// each take 16 columns for all 64 rows.
//
// Up-projection.  Here the contraction runs over c, contiguous in both the
// weight rows and the latent rows, so y^T[d][r] = W_v[d][c] . x^T[c][r] takes
// its A fragments straight from HBM (each wave owns 16 of the 128 output
// dims, 16 KiB of weights) and its B fragments from the latent rows staged in
// LDS.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kPjHeads = 128;
constexpr int kPjNope = 128;    // query dims before absorption
constexpr int kPjV = 128;       // output dims after the up-projection
constexpr int kPjLat = 512;     // latent dims
constexpr int kPjRows = 64;     // query rows per workgroup
constexpr int kAbCols = 128;    // absorb: latent columns per workgroup (4 per head)
constexpr int kAbWaves = 8;     // absorb: 16 columns per wave
constexpr int kAbPitch = 2 * kAbCols + 16;   // LDS bytes per weight row chunk
constexpr int kPjQPitch = 2 * kPjNope + 16;  // LDS bytes per 128-wide query row
constexpr int kUpSplitRows = 256;  // up-projection: up to this many rows, 4 workgroups per head
constexpr int kPjPitch = 2 * kPjLat + 16;    // LDS bytes per 512-wide latent row

typedef __attribute__((address_space(3))) void lds_void_p;
typedef __attribute__((address_space(1))) void glb_void_p;

__device__ __forceinline__ i16x4 lds_tr16(const uint8_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Workgroup (head h, latent columns c0 .. c0+127, query rows r0 .. r0+63).
__global__ __launch_bounds__(kAbWaves * 64) void absorb_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ wkv,
                                                               int R, uint16_t* __restrict__ out) {
  __shared__ __align__(16) uint8_t s_w[kPjNope * kAbPitch];
  __shared__ __align__(16) uint8_t s_q[kPjRows * kPjQPitch];
  constexpr int kChunks = kPjLat / kAbCols;
  const int h = blockIdx.x % kPjHeads;
  const int cc = (blockIdx.x / kPjHeads) % kChunks;
  const int r0 = (blockIdx.x / (kPjHeads * kChunks)) * kPjRows;
  const int c0 = cc * kAbCols;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;

  // Weight rows d = 0..127, columns c0..c0+127 -> LDS (rows padded by 16 bytes),
  // and the query rows (rows past R repeat row R-1 and are not stored).
  const uint8_t* wh = reinterpret_cast<const uint8_t*>(wkv) + (size_t)h * (kPjNope + kPjV) * kPjLat * 2;
  constexpr int kWParts = kAbCols * 2 / 16;  // 16-byte pieces per row chunk
  uint4 wv[kPjNope * kWParts / (kAbWaves * 64)];
#pragma unroll
  for (int u = 0; u < kPjNope * kWParts / (kAbWaves * 64); ++u) {
    const int i = tid + kAbWaves * 64 * u, d = i / kWParts, part = i % kWParts;
    wv[u] = ldg16(wh + (size_t)d * kPjLat * 2 + c0 * 2 + part * 16);
  }
  constexpr int kQParts = kPjNope * 2 / 16;
  uint4 qv[kPjRows * kQParts / (kAbWaves * 64)];
#pragma unroll
  for (int u = 0; u < kPjRows * kQParts / (kAbWaves * 64); ++u) {
    const int i = tid + kAbWaves * 64 * u, rr = i / kQParts, part = i % kQParts;
    const int r = min(r0 + rr, R - 1);
    qv[u] = ldg16(reinterpret_cast<const uint8_t*>(q) + ((size_t)r * kPjHeads + h) * kPjNope * 2 + part * 16);
  }
#pragma unroll
  for (int u = 0; u < kPjNope * kWParts / (kAbWaves * 64); ++u) {
    const int i = tid + kAbWaves * 64 * u, d = i / kWParts, part = i % kWParts;
    *reinterpret_cast<uint4*>(s_w + d * kAbPitch + part * 16) = wv[u];
  }
#pragma unroll
  for (int u = 0; u < kPjRows * kQParts / (kAbWaves * 64); ++u) {
    const int i = tid + kAbWaves * 64 * u, rr = i / kQParts, part = i % kQParts;
    *reinterpret_cast<uint4*>(s_q + rr * kPjQPitch + part * 16) = qv[u];
  }
  __syncthreads();

  // Wave w: columns c0 + 16w .. +15 (one M-tile) for the 64 rows (4 N-tiles).
  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Transposed reads: lane r16 of group g gets W[32s + 16e + 4g + j][16w + r16]
  // (j = 0..3, e = 0 then 1) from the 8-byte rows addressed by lanes 4j + r16/4.
  const uint8_t* wrow = s_w + (4 * g + (r16 >> 2)) * kAbPitch + 8 * (r16 & 3) + 32 * wave;
#pragma unroll
  for (int s = 0; s < kPjNope / 32; ++s) {
    const i16x4 lo = lds_tr16(wrow + (32 * s) * kAbPitch);
    const i16x4 hi = lds_tr16(wrow + (32 * s + 16) * kAbPitch);
    const uint4 a = uint4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                          (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                          (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                          (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const uint8_t* qr = s_q + (nt * 16 + r16) * kPjQPitch + (32 * s + 4 * g) * 2;
      const uint2 qlo = *reinterpret_cast<const uint2*>(qr);
      const uint2 qhi = *reinterpret_cast<const uint2*>(qr + 32);
      const uint4 b = uint4{qlo.x, qlo.y, qhi.x, qhi.y};
      acc[nt] = mfma_bf16_16x16x32(as_bf16x8(a), as_bf16x8(b), acc[nt]);
    }
  }
  // acc[nt][i] = q_abs[row r0 + 16nt + r16][c0 + 16w + 4g + i].
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int r = r0 + nt * 16 + r16;
    if (r < R)
      *reinterpret_cast<uint2*>(out + ((size_t)r * kPjHeads + h) * kPjLat + c0 + 16 * wave + 4 * g) =
          uint2{pack2_bf16(acc[nt][0], acc[nt][1]), pack2_bf16(acc[nt][2], acc[nt][3])};
  }
}

// Workgroup (head h, kUpDims output dims, query rows r0 .. r0+63): 32 dims
// (four workgroups per head) for few rows, where the weight stream is what
// counts; all 128 for many rows, so each latent row is staged once.
template <int kUpDims>
__global__ __launch_bounds__(kUpDims / 16 * 64) void out_proj_kernel(const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ wkv,
                                                                     int R, uint16_t* __restrict__ y) {
  constexpr int kUpWaves = kUpDims / 16;
  __shared__ __align__(16) uint8_t s_x[kPjRows * kPjPitch];
  constexpr int kChunks = kPjV / kUpDims;
  const int h = blockIdx.x % kPjHeads;
  const int dc = (blockIdx.x / kPjHeads) % kChunks;
  const int r0 = (blockIdx.x / (kPjHeads * kChunks)) * kPjRows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int d0 = dc * kUpDims + 16 * wave;  // this wave's 16 output dims

  // A fragments first (weight rows 128 + d0 + r16, 8 values of c per lane group,
  // 16 K-steps of 32), then the latent rows r0 .. r0+63 of head h -> LDS.
  const uint8_t* wr = reinterpret_cast<const uint8_t*>(wkv) +
                      ((size_t)h * (kPjNope + kPjV) + kPjNope + d0 + r16) * kPjLat * 2 + g * 16;
  uint4 wa[kPjLat / 32];
#pragma unroll
  for (int s = 0; s < kPjLat / 32; ++s) wa[s] = ldg16(wr + s * 64);
#pragma unroll
  for (int j = 0; j < kPjRows / kUpWaves; ++j) {
    const int rr = (kPjRows / kUpWaves) * wave + j;
    const int r = min(r0 + rr, R - 1);
    __builtin_amdgcn_global_load_lds(
        (glb_void_p*)(reinterpret_cast<const uint8_t*>(x) + ((size_t)r * kPjHeads + h) * kPjLat * 2 + lane * 16),
        (lds_void_p*)(s_x + rr * kPjPitch), 16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));
  __syncthreads();

  f32x4 acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kPjLat / 32; ++s)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const uint4 b = *reinterpret_cast<const uint4*>(s_x + (nt * 16 + r16) * kPjPitch + s * 64 + g * 16);
      acc[nt] = mfma_bf16_16x16x32(as_bf16x8(wa[s]), as_bf16x8(b), acc[nt]);
    }
  // acc[nt][i] = y[row r0 + 16nt + r16][d0 + 4g + i].
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int r = r0 + nt * 16 + r16;
    if (r < R)
      *reinterpret_cast<uint2*>(y + ((size_t)r * kPjHeads + h) * kPjV + d0 + 4 * g) =
          uint2{pack2_bf16(acc[nt][0], acc[nt][1]), pack2_bf16(acc[nt][2], acc[nt][3])};
  }
}

static_assert(kPjNope * (kAbCols * 2 / 16) % (kAbWaves * 64) == 0, "whole weight pieces per thread");
static_assert(kPjRows * (kPjNope * 2 / 16) % (kAbWaves * 64) == 0, "whole query pieces per thread");

int launch_q_absorb(const void* q_nope, const void* wkv_b, int rows, void* q_abs,
                    hipStream_t stream) {
  const dim3 grid((unsigned)(kPjHeads * (kPjLat / kAbCols) * ((rows + kPjRows - 1) / kPjRows)));
  hipLaunchKernelGGL(absorb_kernel, grid, dim3(kAbWaves * 64), 0, stream,
                     reinterpret_cast<const uint16_t*>(q_nope), reinterpret_cast<const uint16_t*>(wkv_b),
                     rows, reinterpret_cast<uint16_t*>(q_abs));
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_out_proj(const void* x, const void* wkv_b, int rows, void* y, hipStream_t stream) {
  const unsigned rchunks = (unsigned)((rows + kPjRows - 1) / kPjRows);
  if (rows <= kUpSplitRows)
    hipLaunchKernelGGL(out_proj_kernel<32>, dim3(kPjHeads * 4 * rchunks), dim3(2 * 64), 0, stream,
                       reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(wkv_b),
                       rows, reinterpret_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(out_proj_kernel<128>, dim3(kPjHeads * rchunks), dim3(8 * 64), 0, stream,
                       reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(wkv_b),
                       rows, reinterpret_cast<uint16_t*>(y));
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace dsa
