// Indexer input preparation on gfx950: the weight-free steps between the
// indexer's projections and its score kernel in the Indexer.forward excerpt
// on "DeepSeek-V3.2-Exp - Keep top-k positions" -- RoPE on the first 64 of
// every 128 dims (query heads and key), the Walsh-Hadamard rotation
// (rotate_activation), block-128 fp8 quantisation (act_quant) and the key's
// write into k_cache / k_scale_cache at its position.  RoPE uses the
// concatenated (non-interleaved) layout that "MaxText PR #2933" describes
// for the indexer: dim i and dim i+32 are the two parts of one rotated pair.
//
// Work split.  One workgroup per token (64 query heads, then the key).  Up
// to 512 tokens (decode) one 128-dim vector per 16 lanes, 8 consecutive dims
// per lane (one 16-byte load), described below; more tokens take
// indexer_prep_wide_kernel, 4 lanes per vector and 32 dims per lane, which
// needs fewer cross-lane exchanges (described above it).  Either way only
// 16-byte loads, several in flight per lane, and no LDS: 256 bytes in and 132
// (fp8) or 256 (bf16) bytes out per vector.
//
//   RoPE.  Lane l < 4 of a group holds dims 8l..8l+7 and lane l+4 the dims
//     32 above them, so each pair is one xor-4 exchange away.
//   Rotation.  In Sylvester order H[i][j] = (-1)^popcount(i & j), and the
//     transform factors into one butterfly per index bit.  Bits 0-2 of the
//     dim index are the element within a lane (three stages in registers),
//     bits 3-6 the lane within the group (four stages over xor-1/2/4/8
//     exchanges).  The butterflies are left unscaled; the 128^-1/2 is folded
//     into the stored scale (fp8) or applied once at the end (bf16).
//   Quantisation.  amax over the vector by an xor reduction, scale = amax /
//     448 and codes = e4m3(u / scale): the scale and the quotients are the
//     correctly rounded fp32 values (the quotients from one reciprocal per
//     vector and an fma correction each), rounded to the nearest e4m3 value
//     with ties to even; an all-zero vector gets scale 0 and zero codes.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kPrepDim = 128;
constexpr int kPrepHeads = 64;
constexpr int kPrepRopeHalf = 32;
constexpr float kE4m3Max = 448.0f;
constexpr float kInvSqrtDim = 0.08838834764831845f;   // 128^-1/2, nearest fp32
// Below this block scale the reciprocal could overflow; such blocks (max |x|
// under 448 * 2^-100) take plain divisions.
constexpr float kTinyScale = 0x1p-100f;

// Two fp32 values to OCP e4m3fn codes, rounded to nearest even, in the low
// 16 bits (v_cvt_pk_fp8_f32; on gfx950 it produces the OCP format).  Its
// inputs here never exceed 448 (1 + 2^-23) in magnitude, where it agrees
// with rounding the fp32 value to the nearest e4m3 value, ties to even.
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Lane exchanges within a row of 16 lanes (one vector's group) by DPP, which
// rides on a VALU move instead of a trip through the LDS crossbar:
//   xor 1, xor 2: quad_perm [1,0,3,2] and [2,3,0,1];
//   xor 4: row_half_mirror (lane j reads j^7) then quad_perm [3,2,1,0] (j^3);
//   xor 8: row_ror:8.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  // Every source lane is inside the row, so no lane keeps an old value.
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}

template <int kMask>
__device__ __forceinline__ float row_xor(float v) {
  if constexpr (kMask == 1) return dpp_f32<0xB1>(v);
  else if constexpr (kMask == 2) return dpp_f32<0x4E>(v);
  else if constexpr (kMask == 4) return dpp_f32<0x1B>(dpp_f32<0x141>(v));
  else return dpp_f32<0x128>(v);
}

// One cross-lane butterfly stage: the lane whose mask bit is clear holds the
// lower index a and keeps a + b; its partner keeps a - b (sgn = +1 / -1).
template <int kMask>
__device__ __forceinline__ void lane_stage(float (&e)[8], float sgn) {
#pragma unroll
  for (int k = 0; k < 8; ++k) e[k] = fmaf(sgn, e[k], row_xor<kMask>(e[k]));
}

__device__ __forceinline__ void bf16x8_to_f32(const uint4& v, float (&e)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e[2 * i] = __uint_as_float(w[i] << 16);
    e[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// The rotation and output of one 128-dim vector held by a 16-lane group
// (8 dims per lane, e[] already roped).  sg[m] = -1 where lane bit m is set.
__device__ __forceinline__ void rotate_store(float (&e)[8], int gl, const float (&sg)[4],
                                             bool fp8, bool store, void* dst,
                                             float* scale_dst) {
  // In-register butterfly stages (index bits 0-2)...
#pragma unroll
  for (int h = 1; h < 8; h *= 2) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k & h) continue;
      const float a = e[k], d = e[k + h];
      e[k] = a + d;
      e[k + h] = a - d;
    }
  }
  // ...then across the 16 lanes (index bits 3-6).
  lane_stage<1>(e, sg[0]);
  lane_stage<2>(e, sg[1]);
  lane_stage<4>(e, sg[2]);
  lane_stage<8>(e, sg[3]);
  if (fp8) {
    float amax = fmaxf(fmaxf(fmaxf(fabsf(e[0]), fabsf(e[1])), fmaxf(fabsf(e[2]), fabsf(e[3]))),
                       fmaxf(fmaxf(fabsf(e[4]), fabsf(e[5])), fmaxf(fabsf(e[6]), fabsf(e[7]))));
    amax = fmaxf(amax, row_xor<1>(amax));
    amax = fmaxf(amax, row_xor<2>(amax));
    amax = fmaxf(amax, row_xor<4>(amax));
    amax = fmaxf(amax, row_xor<8>(amax));
    const float su = amax / kE4m3Max;
    float q[8];
    if (su >= kTinyScale) {
      // x / su, correctly rounded, from the correctly rounded reciprocal y and
      // one correction: q0 = x y, r = q0 su - x (exact by fma), q = q0 - r y
      // (Markstein's theorem: y = RN(1/su) and q0 within an ulp make the
      // corrected value RN(x / su)).  Written this way a -0 input stays -0.
      const float y = 1.0f / su;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float q0 = e[k] * y;
        q[k] = fmaf(-fmaf(q0, su, -e[k]), y, q0);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) q[k] = su > 0.0f ? e[k] / su : 0.0f;
    }
    uint32_t w0 = 0, w1 = 0;
    if (su > 0.0f) {
      w0 = e4m3_pack2(q[0], q[1]) | (e4m3_pack2(q[2], q[3]) << 16);
      w1 = e4m3_pack2(q[4], q[5]) | (e4m3_pack2(q[6], q[7]) << 16);
    }
    if (store) {
      reinterpret_cast<uint2*>(dst)[gl] = make_uint2(w0, w1);
      if (gl == 0) *scale_dst = su * kInvSqrtDim;
    }
  } else if (store) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)f32_to_bf16_bits(e[2 * k] * kInvSqrtDim) |
             ((uint32_t)f32_to_bf16_bits(e[2 * k + 1] * kInvSqrtDim) << 16);
    reinterpret_cast<uint4*>(dst)[gl] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// One workgroup per token: kGroups groups of 16 lanes, each taking
// 64 / kGroups query heads (heads g, g + kGroups, ...: consecutive groups read
// consecutive heads, so each round of a wave reads 1 KiB contiguously); group
// 0 also takes the key.  The position is uniform over the workgroup, so
// end_pos and the table row are scalar; every lane loads its query heads
// before it needs the position, and its 8 cos/sin values once for all heads.
template <int kGroups>
__global__ __launch_bounds__(16 * kGroups) void indexer_prep_kernel(
    const uint16_t* __restrict__ q_in, const uint16_t* __restrict__ k_in,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
    const int32_t* __restrict__ end_pos, int T, int S_max, int fp8,
    void* __restrict__ q_out, float* __restrict__ q_scale, void* __restrict__ k_cache,
    float* __restrict__ k_scale) {
  constexpr int kPer = kPrepHeads / kGroups;
  const int token = blockIdx.x;                           // b * T + t
  const int gl = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const uint16_t* qsrc = q_in + (size_t)token * kPrepHeads * kPrepDim;
  uint4 raw[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) raw[i] = ldg16(qsrc + (grp + kGroups * i) * kPrepDim + 8 * gl);
  const bool has_key = grp == 0;
  uint4 kraw = make_uint4(0, 0, 0, 0);
  if (has_key) kraw = ldg16(k_in + (size_t)token * kPrepDim + 8 * gl);

  const int b = token / T;
  const int t = token - b * T;
  const int pos = end_pos[b] - T + t;
  const int row = min(max(pos, 0), S_max - 1);            // table row (clamped)
  const float* cs = rope_cos + (size_t)row * kPrepRopeHalf + 8 * (gl & 3);
  const float* sn = rope_sin + (size_t)row * kPrepRopeHalf + 8 * (gl & 3);
  const float4 c0 = *reinterpret_cast<const float4*>(cs);
  const float4 c1 = *reinterpret_cast<const float4*>(cs + 4);
  const float4 s0 = *reinterpret_cast<const float4*>(sn);
  const float4 s1 = *reinterpret_cast<const float4*>(sn + 4);
  // RoPE on dims 0..63 (lanes 0..7 of the group): pair i = 8*(gl&3)+k with
  // i+32 in lane gl^4.  lower: x1 c - x2 s;  upper: x1 s + x2 c -- i.e.
  // e c + p s' with s' = -s in the lower lane (p = the partner's value).
  const bool rope = gl < 8;
  const float ssgn = (gl & 4) ? 1.0f : -1.0f;
  const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float s[8] = {ssgn * s0.x, ssgn * s0.y, ssgn * s0.z, ssgn * s0.w,
                      ssgn * s1.x, ssgn * s1.y, ssgn * s1.z, ssgn * s1.w};
  const float sg[4] = {(gl & 1) ? -1.0f : 1.0f, (gl & 2) ? -1.0f : 1.0f,
                       (gl & 4) ? -1.0f : 1.0f, (gl & 8) ? -1.0f : 1.0f};
  auto rope_in = [&](const uint4& v, float (&e)[8]) {
    bf16x8_to_f32(v, e);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float r = fmaf(row_xor<4>(e[k]), s[k], e[k] * c[k]);
      e[k] = rope ? r : e[k];
    }
  };

  const size_t qbase = (size_t)token * kPrepHeads;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int h = grp + kGroups * i;
    float e[8];
    rope_in(raw[i], e);
    void* dst = fp8 ? (void*)(reinterpret_cast<uint8_t*>(q_out) + (qbase + h) * kPrepDim)
                    : (void*)(reinterpret_cast<uint16_t*>(q_out) + (qbase + h) * kPrepDim);
    rotate_store(e, gl, sg, fp8, true, dst, fp8 ? q_scale + qbase + h : nullptr);
  }
  if (has_key) {
    const bool in_cache = pos >= 0 && pos < S_max;
    const size_t krow = (size_t)b * S_max + (size_t)(in_cache ? pos : 0);
    float e[8];
    rope_in(kraw, e);
    void* dst = fp8 ? (void*)(reinterpret_cast<uint8_t*>(k_cache) + krow * kPrepDim)
                    : (void*)(reinterpret_cast<uint16_t*>(k_cache) + krow * kPrepDim);
    rotate_store(e, gl, sg, fp8, in_cache, dst, fp8 ? k_scale + krow : nullptr);
  }
}

// Many tokens: 4 lanes per vector, 32 dims per lane.  Lane gl holds the four
// 8-dim chunks 32q + 8gl .. +7 (q = 0..3; four 16-byte loads), element 8q + j
// being dim 32q + 8gl + j.  So every RoPE pair (i, i+32), i = 8gl + j, sits in
// one lane as elements j and 8 + j, and of the rotation's index bits, 0-2 (j)
// and 5-6 (q) are a lane's own elements (five butterfly stages in registers)
// while only bits 3-4 (gl) cross lanes (two DPP stages, both quad permutes).  With 8 dims per lane the same vector took four cross-lane stages,
// one of them two DPP moves, and a two-move RoPE exchange.  A group of 4 lanes
// takes 64 / kGroups4 heads of its token; group 0 also the key.
template <int kGroups4>
__global__ __launch_bounds__(4 * kGroups4) void indexer_prep_wide_kernel(
    const uint16_t* __restrict__ q_in, const uint16_t* __restrict__ k_in,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
    const int32_t* __restrict__ end_pos, int T, int S_max, int fp8,
    void* __restrict__ q_out, float* __restrict__ q_scale, void* __restrict__ k_cache,
    float* __restrict__ k_scale) {
  constexpr int kPer = kPrepHeads / kGroups4;
  const int token = blockIdx.x;
  const int gl = threadIdx.x & 3;
  const int grp = threadIdx.x >> 2;
  const uint16_t* qsrc = q_in + (size_t)token * kPrepHeads * kPrepDim;
  uint4 raw[kPer][4];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      raw[i][q] = ldg16(qsrc + (grp + kGroups4 * i) * kPrepDim + 32 * q + 8 * gl);
  const bool has_key = grp == 0;
  uint4 kraw[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0),
                   make_uint4(0, 0, 0, 0)};
  if (has_key) {
#pragma unroll
    for (int q = 0; q < 4; ++q) kraw[q] = ldg16(k_in + (size_t)token * kPrepDim + 32 * q + 8 * gl);
  }

  const int b = token / T;
  const int t = token - b * T;
  const int pos = end_pos[b] - T + t;
  const int row = min(max(pos, 0), S_max - 1);
  // RoPE pairs i = 8gl + j: lower dim i is element j, upper dim i + 32 element 8 + j;
  // lower' = x1 c - x2 s, upper' = x1 s + x2 c.
  const float* cs = rope_cos + (size_t)row * kPrepRopeHalf + 8 * gl;
  const float* sn = rope_sin + (size_t)row * kPrepRopeHalf + 8 * gl;
  const float4 c0 = *reinterpret_cast<const float4*>(cs);
  const float4 c1 = *reinterpret_cast<const float4*>(cs + 4);
  const float4 s0 = *reinterpret_cast<const float4*>(sn);
  const float4 s1 = *reinterpret_cast<const float4*>(sn + 4);
  const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sr[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const float sg1 = (gl & 1) ? -1.0f : 1.0f, sg2 = (gl & 2) ? -1.0f : 1.0f;

  auto process = [&](const uint4 (&v)[4], bool store, void* dst, float* scale_dst) {
    float e[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float f[8];
      bf16x8_to_f32(v[q], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) e[8 * q + j] = f[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x1 = e[j], x2 = e[8 + j];
      e[j] = fmaf(x2, -sr[j], x1 * c[j]);  // the rounding order of rotate_store's callers
      e[8 + j] = fmaf(x1, sr[j], x2 * c[j]);
    }
    // Rotation: element bits (dim bits 0-2 and 5-6) in registers...
#pragma unroll
    for (int h = 1; h < 32; h *= 2) {
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        if (k & h) continue;
        const float a = e[k], d = e[k + h];
        e[k] = a + d;
        e[k + h] = a - d;
      }
    }
    // ...dim bits 3 and 4 across the 4 lanes.
#pragma unroll
    for (int k = 0; k < 32; ++k) e[k] = fmaf(sg1, e[k], row_xor<1>(e[k]));
#pragma unroll
    for (int k = 0; k < 32; ++k) e[k] = fmaf(sg2, e[k], row_xor<2>(e[k]));
    if (fp8) {
      float amax = 0.0f;
#pragma unroll
      for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(e[k]));
      amax = fmaxf(amax, row_xor<1>(amax));
      amax = fmaxf(amax, row_xor<2>(amax));
      const float su = amax / kE4m3Max;
      uint32_t w[8];  // chunk q: words 2q, 2q + 1
      if (su >= kTinyScale) {
        // Correctly rounded x / su as in rotate_store (Markstein correction).
        const float y = 1.0f / su;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          float qv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = e[4 * m + j];
            const float q0 = x * y;
            qv[j] = fmaf(-fmaf(q0, su, -x), y, q0);
          }
          w[m] = e4m3_pack2(qv[0], qv[1]) | (e4m3_pack2(qv[2], qv[3]) << 16);
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          float qv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) qv[j] = su > 0.0f ? e[4 * m + j] / su : 0.0f;
          w[m] = su > 0.0f ? (e4m3_pack2(qv[0], qv[1]) | (e4m3_pack2(qv[2], qv[3]) << 16)) : 0u;
        }
      }
      if (store) {
        uint8_t* d8 = reinterpret_cast<uint8_t*>(dst) + 8 * gl;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(d8 + 32 * q) = make_uint2(w[2 * q], w[2 * q + 1]);
        if (gl == 0) *scale_dst = su * kInvSqrtDim;
      }
    } else if (store) {
      uint16_t* d16 = reinterpret_cast<uint16_t*>(dst) + 8 * gl;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = (uint32_t)f32_to_bf16_bits(e[8 * q + 2 * j] * kInvSqrtDim) |
                 ((uint32_t)f32_to_bf16_bits(e[8 * q + 2 * j + 1] * kInvSqrtDim) << 16);
        *reinterpret_cast<uint4*>(d16 + 32 * q) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  };

  const size_t qbase = (size_t)token * kPrepHeads;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int h = grp + kGroups4 * i;
    void* dst = fp8 ? (void*)(reinterpret_cast<uint8_t*>(q_out) + (qbase + h) * kPrepDim)
                    : (void*)(reinterpret_cast<uint16_t*>(q_out) + (qbase + h) * kPrepDim);
    process(raw[i], true, dst, fp8 ? q_scale + qbase + h : nullptr);
  }
  if (has_key) {
    const bool in_cache = pos >= 0 && pos < S_max;
    const size_t krow = (size_t)b * S_max + (size_t)(in_cache ? pos : 0);
    void* dst = fp8 ? (void*)(reinterpret_cast<uint8_t*>(k_cache) + krow * kPrepDim)
                    : (void*)(reinterpret_cast<uint16_t*>(k_cache) + krow * kPrepDim);
    process(kraw, in_cache, dst, fp8 ? k_scale + krow : nullptr);
  }
}

// Few tokens: 64 groups of 16 lanes (1024 lanes), one head each, to spread the
// vectors of a token over more SIMDs; many tokens: 64 groups of 4 lanes (32 dims a
// lane), one head each (8192 tokens: 74.4 us with 8 dims a lane, 62 us with 32
// consecutive dims, 55.8 us with the four chunks; 600 tokens: 9.8, 8.9, 7.5 us).
constexpr int kPrepSmallTokens = 512;

int launch_indexer_prep(const void* q_in, const void* k_in, const float* rope_cos,
                        const float* rope_sin, const int32_t* end_pos, int B, int T, int S_max,
                        int dtype, void* q_out, float* q_scale, void* k_cache, float* k_scale,
                        hipStream_t stream) {
  const int tokens = B * T;
  auto qi = static_cast<const uint16_t*>(q_in);
  auto ki = static_cast<const uint16_t*>(k_in);
  if (tokens <= kPrepSmallTokens)
    hipLaunchKernelGGL(indexer_prep_kernel<64>, dim3(tokens), dim3(1024), 0, stream, qi, ki,
                       rope_cos, rope_sin, end_pos, T, S_max, dtype, q_out, q_scale, k_cache,
                       k_scale);
  else
    hipLaunchKernelGGL(indexer_prep_wide_kernel<64>, dim3(tokens), dim3(4 * 64), 0, stream, qi,
                       ki, rope_cos, rope_sin, end_pos, T, S_max, dtype, q_out, q_scale, k_cache,
                       k_scale);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace dsa
