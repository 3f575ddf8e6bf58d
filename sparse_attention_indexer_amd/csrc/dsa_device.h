// Device-side helpers shared by the gfx950 kernels of libdsa.
//
// MFMA lane layouts used throughout (wave64, checked on gfx950):
//   v_mfma_f32_16x16x32_bf16: A[m][k] is held by lane m + 16*(k/8), element k%8;
//     B[k][n] by lane n + 16*(k/8), element k%8; C[m][n] by lane n + 16*(m/4),
//     element m%4.
//   v_mfma_f32_16x16x128_f8f6f4 (fp8 e4m3 operands): A row m and B column n sit
//     in lanes m + 16*g and n + 16*g (g = 0..3), 32 bytes each; a lane's A and
//     B bytes at the same (g, byte) position are multiplied together, so any
//     assignment of the 128 dot-product terms to (g, byte) slots works as long
//     as A and B use the same one.  C as for the bf16 form.
//   ds_read_tr16_b64 (LDS transposing read): within each group of 16 lanes,
//     lane i receives element i%4 of the 8-byte rows addressed by lanes
//     4*j + i/4, j = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(const bf16x8& a, const bf16x8& b,
                                                    const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp8 e4m3 x fp8 e4m3, K = 128, unscaled.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(const i32x8& a, const i32x8& b,
                                                    const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite here; NaN keeps a quiet payload).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values to packed bf16 (a in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Order-preserving map from an fp32 score to an unsigned key: larger score,
// larger key.  -0 is first turned into +0 so the two compare equal.
__device__ __forceinline__ uint32_t score_key(float x) {
  // x + 0 turns -0 into +0.  Negative values: all bits flipped; others: the
  // sign bit set.  (An arithmetic shift spreads the sign over the mask.)
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T xor_shfl(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// s_waitcnt immediates (gfx9 encoding): wait for LDS ops, or for all but N of
// this wave's outstanding vector-memory ops.
constexpr int kWaitLgkm0 = 0xC07F;
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then s_barrier.  Unlike __syncthreads it does not wait for the
// wave's outstanding global loads (or global->LDS copies), so they stay in
// flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

// Row copies issued through inline asm: global_load_lds
// with M0 = the LDS destination of lane 0 (lane i writes 16 bytes at M0 +
// 16 i).  Written as a builtin, the compiler treats the copy as an LDS write
// that may alias every later LDS read of the ring array and makes those reads
// wait for all copies in flight, which serialises the gathers with the math;
// here the kernel itself orders each slot's reads after that slot's copies
// (a vmcnt wait, then a barrier).  The instruction has no register result.
__device__ __forceinline__ void lds_copy16(const uint8_t* row, uint32_t lane_off, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0), "v"(lane_off), "s"(row) : "m0");
}
__device__ __forceinline__ void lds_copy16_v(const uint8_t* addr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0), "v"(addr) : "m0");
}
// The same with the non-temporal hint, for data read once (a streamed key
// cache): a single pass over a large buffer runs closer to the HBM peak.
__device__ __forceinline__ void lds_copy16_v_nt(const uint8_t* addr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :: "s"(m0), "v"(addr) : "m0");
}
__device__ __forceinline__ void lds_copy4_v_nt(const uint8_t* addr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off nt"
               :: "s"(m0), "v"(addr) : "m0");
}
// 4 bytes a lane (lane i writes at M0 + 4 i).
__device__ __forceinline__ void lds_copy4_v(const uint8_t* addr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m0), "v"(addr) : "m0");
}
// The lane id through an empty asm: the compiler cannot hoist what is derived
// from it out of a loop, so per-lane addresses are recomputed (a few VALU
// ops) instead of being kept live across the loop or spilled.
__device__ __forceinline__ int opaque_lane() {
  int l = __lane_id();
  asm volatile("" : "+v"(l));
  return l;
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const lds_void*)p);
}

// Transposing LDS read (ds_read_b64_tr_b16): 4 bf16 of a 16x16 block's column.
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

}  // namespace dsa
