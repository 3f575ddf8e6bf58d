// Absorbed-MLA attention over gathered cached rows on gfx950 (the MQA decode
// branch of "DeepSeek-V3.2-Exp - Apply sparse mask", restricted to the rows the
// indexer selected; the dense variant takes every causally valid row).
//
//   z[h,j] = (q_nope[h,:] . kv[pos_j,:] + q_pe[h,:] . pe[pos_j,:]) * softmax_scale
//   out[h,:] = sum_j softmax_j(z[h,:]) * kv[pos_j,:]
//
// Work item: one query row, one group of 64 heads, one split of its row list.
// A 256-thread workgroup (4 waves, 16 heads each) walks the split 32 rows at a
// time.  Each tile of 32 gathered rows (512 latent + 64 rope bf16 = 1152 B a
// row) is staged in LDS once and read by all four waves twice:
//   - scores: 16 heads x 32 rows, K = 576, on 16x16x32 bf16 MFMA, the query
//     fragment held in registers for the whole split;
//   - values: 16 heads x 512 latent dims, K = 32 rows, the row-major tile read
//     back transposed with ds_read_tr16_b64 so the same LDS copy serves both.
// The softmax is online (running max and sum per head, in base 2), the
// probabilities go through LDS as bf16 to become the A operand of the value
// contraction, and the 16x512 fp32 accumulator stays in registers.  The next
// tile's global loads are issued before the current tile is computed.
// With several splits per row, unnormalised partial outputs plus (max, sum)
// go to the workspace and a combine kernel merges them.
//
// Head groups of the same (row, split) are given block ids that fall on the
// same XCD (ids are dealt round-robin over the 8 XCDs), so the second group
// finds the gathered rows in that XCD's L2.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kHeads = 128;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kDqk = kDc + kDr;
constexpr int kHpb = 64;            // heads per workgroup
constexpr int kRt = 32;             // gathered rows per tile
constexpr int kKvPitch = kDqk + 8;  // bf16 per LDS row (1168 B): spreads rows over banks
constexpr int kPPitch = kRt + 8;    // bf16 per probability row (80 B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

template <bool kDense>
__global__ __launch_bounds__(256) void mla_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const uint16_t* __restrict__ kv, const uint16_t* __restrict__ pe,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ end_pos, int T, int S_max,
    int k, int rows_per_split, int n_splits, int n_items, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
    float2* __restrict__ part_ml) {
  __shared__ __align__(16) uint16_t s_kv[kRt * kKvPitch];
  __shared__ __align__(16) uint16_t s_p[4][16 * kPPitch];
  __shared__ int s_valid[kRt];

  const int bid = blockIdx.x;
  const int X = (bid >> 4) * 8 + (bid & 7);  // item = row * n_splits + split
  const int hg = (bid >> 3) & 1;            // head group
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

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r16 = lane & 15;

  // Query fragment (A operand): head hg*64 + wave*16 + r16; K-step kk holds dims
  // kk*32 + 8g .. +7 of [q_nope | q_pe].
  uint4 qa[18];
  {
    const int head = hg * kHpb + wave * 16 + r16;
    const uint16_t* qn = q_nope + ((size_t)row * kHeads + head) * kDc;
    const uint16_t* qp = q_pe + ((size_t)row * kHeads + head) * kDr;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qa[kk] = ldg16(qn + kk * 32 + g * 8);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) qa[16 + kk] = ldg16(qp + kk * 32 + g * 8);
  }

  // Running softmax state for the 4 heads 4g+i whose results this lane holds.
  float m_run[4], l_part[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_part[i] = 0.f;
  }
  f32x4 o[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Gather assignment: thread -> tile row lr, 1/8 of that row.
  const int lr = threadIdx.x >> 3, lp = threadIdx.x & 7;
  uint4 pf[9];
  int pf_valid = 0;
  auto issue = [&](int j0) {
    const int j = j0 + lr;
    int pos;
    bool valid;
    if constexpr (kDense) {
      pos = j;
      valid = j < j_end;
    } else {
      pos = j < j_end ? idx[(size_t)row * k + j] : -1;
      valid = pos >= 0 && pos < S_max;
    }
    if (!valid) pos = 0;  // a safe address; the row is masked out below
    const uint16_t* src = kv + ((size_t)b * S_max + pos) * kDc + lp * 64;
#pragma unroll
    for (int u = 0; u < 8; ++u) pf[u] = ldg16(src + u * 8);
    pf[8] = ldg16(pe + ((size_t)b * S_max + pos) * kDr + lp * 8);
    pf_valid = valid ? 1 : 0;
  };

  if (j_begin < j_end) issue(j_begin);
#pragma unroll 1
  for (int j0 = j_begin; j0 < j_end; j0 += kRt) {
    __syncthreads();  // every wave is done with the previous tile
    {
      uint16_t* dst = s_kv + lr * kKvPitch;
#pragma unroll
      for (int u = 0; u < 8; ++u) *reinterpret_cast<uint4*>(dst + lp * 64 + u * 8) = pf[u];
      *reinterpret_cast<uint4*>(dst + kDc + lp * 8) = pf[8];
      if (lp == 0) s_valid[lr] = pf_valid;
    }
    __syncthreads();
    if (j0 + kRt < j_end) issue(j0 + kRt);  // next tile's loads overlap this tile's math

    // ---- scores: S[head 4g+i][row nt*16 + r16] ----
    f32x4 sc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      sc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* brow = s_kv + (nt * 16 + r16) * kKvPitch + g * 8;
#pragma unroll
      for (int kk = 0; kk < 18; ++kk)
        sc[nt] = mfma_bf16_16x16x32(as_bf16x8(qa[kk]),
                                    as_bf16x8(*reinterpret_cast<const uint4*>(brow + kk * 32)),
                                    sc[nt]);
    }

    // ---- online softmax (base 2) ----
    float p[2][4], alpha[4];
    const bool v0 = s_valid[r16] != 0, v1 = s_valid[16 + r16] != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s0 = v0 ? sc[0][i] * scale_log2 : -INFINITY;
      const float s1 = v1 ? sc[1][i] * scale_log2 : -INFINITY;
      float mx = fmaxf(s0, s1);
      mx = fmaxf(mx, xor_shfl(mx, 1));
      mx = fmaxf(mx, xor_shfl(mx, 2));
      mx = fmaxf(mx, xor_shfl(mx, 4));
      mx = fmaxf(mx, xor_shfl(mx, 8));
      const float m_new = fmaxf(m_run[i], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[i] = exp2f(m_run[i] - m_use);
      m_run[i] = m_new;
      p[0][i] = exp2f(s0 - m_use);
      p[1][i] = exp2f(s1 - m_use);
      l_part[i] = l_part[i] * alpha[i] + p[0][i] + p[1][i];
    }

    // ---- probabilities: C layout -> LDS (bf16) -> A layout ----
    uint16_t* pw = s_p[wave];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[(4 * g + i) * kPPitch + nt * 16 + r16] = f32_to_bf16_bits(p[nt][i]);
    __syncthreads();
    const uint4 pa = *reinterpret_cast<const uint4*>(pw + r16 * kPPitch + 8 * g);

    // ---- values: O[head][c] = alpha * O + P . V ----
    const uint16_t* vbase = s_kv + (8 * g + (r16 >> 2)) * kKvPitch + 4 * (r16 & 3);
#pragma unroll
    for (int ct = 0; ct < 32; ++ct) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[ct][i] *= alpha[i];
      const i16x4 lo = lds_read_tr16(vbase + ct * 16);
      const i16x4 hi = lds_read_tr16(vbase + 4 * kKvPitch + ct * 16);
      const uint4 vb = uint4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                             (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                             (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                             (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
      o[ct] = mfma_bf16_16x16x32(as_bf16x8(pa), as_bf16x8(vb), o[ct]);
    }
  }

  // ---- finish: sum l over the 16 lanes holding each head's columns ----
  float l_tot[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float l = l_part[i];
    l += xor_shfl(l, 1);
    l += xor_shfl(l, 2);
    l += xor_shfl(l, 4);
    l += xor_shfl(l, 8);
    l_tot[i] = l;
  }
  const int head0 = hg * kHpb + wave * 16 + 4 * g;
  if (n_splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float inv = l_tot[i] > 0.f ? 1.f / l_tot[i] : 0.f;
      uint16_t* orow = out + ((size_t)row * kHeads + head0 + i) * kDc;
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) orow[ct * 16 + r16] = f32_to_bf16_bits(o[ct][i] * inv);
      if (lse != nullptr && r16 == 0)
        lse[(size_t)row * kHeads + head0 + i] =
            l_tot[i] > 0.f ? (m_run[i] + log2f(l_tot[i])) * kLn2 : -INFINITY;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* prow = part_o + ((size_t)X * kHeads + head0 + i) * kDc;
#pragma unroll
      for (int ct = 0; ct < 32; ++ct) prow[ct * 16 + r16] = o[ct][i];
      if (r16 == 0) part_ml[(size_t)X * kHeads + head0 + i] = float2{m_run[i], l_tot[i]};
    }
  }
}

// Merge the per-split partial outputs of one (row, head): 64 threads per head,
// 8 latent dims each.
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float2* __restrict__ part_ml,
                                                          int n_rows, int n_splits,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int rh = blockIdx.x * 4 + (threadIdx.x >> 6);  // row * 128 + head
  if (rh >= n_rows * kHeads) return;
  const int row = rh / kHeads, head = rh - row * kHeads;
  const int c0 = (threadIdx.x & 63) * 8;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s)
    M = fmaxf(M, part_ml[((size_t)row * n_splits + s) * kHeads + head].x);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const size_t item = (size_t)row * n_splits + s;
      const float2 ml = part_ml[item * kHeads + head];
      if (ml.y <= 0.f) continue;
      const float f = exp2f(ml.x - M);
      L += ml.y * f;
      const float* src = part_o + (item * kHeads + head) * kDc + c0;
      const float4 a = *reinterpret_cast<const float4*>(src);
      const float4 c = *reinterpret_cast<const float4*>(src + 4);
      acc[0] += a.x * f; acc[1] += a.y * f; acc[2] += a.z * f; acc[3] += a.w * f;
      acc[4] += c.x * f; acc[5] += c.y * f; acc[6] += c.z * f; acc[7] += c.w * f;
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint32_t packed[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    packed[u] = (uint32_t)f32_to_bf16_bits(acc[2 * u] * inv) |
                ((uint32_t)f32_to_bf16_bits(acc[2 * u + 1] * inv) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)rh * kDc + c0) =
      uint4{packed[0], packed[1], packed[2], packed[3]};
  if (lse != nullptr && (threadIdx.x & 63) == 0)
    lse[rh] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

static int round_up(int x, int m) { return (x + m - 1) / m * m; }

MlaPlan sparse_mla_plan(int B, int T, int k) {
  const long rows = (long)B * T;
  // Aim for ~512 workgroups (2 head groups each item) without splits under 128 rows.
  long ns = 512 / (2 * rows);
  const long max_ns = (k + 127) / 128;
  ns = ns < 1 ? 1 : (ns > max_ns ? max_ns : ns);
  const int rps = round_up((int)((k + ns - 1) / ns), kRt);
  return MlaPlan{rps, (k + rps - 1) / rps};
}

MlaPlan dense_mla_plan(int B, int T, int S_max, int max_end_pos) {
  const long rows = (long)B * T;
  // Rows per split depend only on the allocation sizes, so the workspace
  // computed from S_max always covers the launch.
  long rps = (long)S_max * 2 * rows / 1024;
  rps = rps < 512 ? 512 : (rps > 8192 ? 8192 : rps);
  const int r = round_up((int)rps, kRt);
  const int ext = max_end_pos > 0 ? max_end_pos : S_max;
  return MlaPlan{r, (ext + r - 1) / r};
}

size_t mla_workspace_bytes(int B, int T, const MlaPlan& plan) {
  if (plan.n_splits <= 1) return 0;
  const size_t items = (size_t)B * T * plan.n_splits;
  return items * kHeads * kDc * sizeof(float) + items * kHeads * sizeof(float2);
}

template <bool kDense>
static int launch_mla(const void* q_nope, const void* q_pe, const void* kv, const void* pe,
                      const int32_t* idx, const int32_t* end_pos, int B, int T, int S_max, int k,
                      const MlaPlan& plan, float softmax_scale, void* out, float* lse,
                      void* workspace, hipStream_t stream) {
  const int rows = B * T;
  const int n_items = rows * plan.n_splits;
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  if (plan.n_splits > 1) {
    part_o = reinterpret_cast<float*>(workspace);
    part_ml = reinterpret_cast<float2*>(part_o + (size_t)n_items * kHeads * kDc);
  }
  const unsigned grid = (unsigned)(((n_items + 7) / 8) * 16);
  hipLaunchKernelGGL(mla_kernel<kDense>, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(q_nope),
                     reinterpret_cast<const uint16_t*>(q_pe), reinterpret_cast<const uint16_t*>(kv),
                     reinterpret_cast<const uint16_t*>(pe), idx, end_pos, T, S_max, k,
                     plan.rows_per_split, plan.n_splits, n_items, softmax_scale * kLog2e,
                     reinterpret_cast<uint16_t*>(out), lse, part_o, part_ml);
  if (hipGetLastError() != hipSuccess) return -5;
  if (plan.n_splits > 1) {
    hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)((rows * kHeads + 3) / 4)), dim3(256),
                       0, stream, part_o, part_ml, rows, plan.n_splits,
                       reinterpret_cast<uint16_t*>(out), lse);
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
