// MHA-form prefill attention on gfx950: the `mask is not None` branch of the
// attention excerpt on "DeepSeek-V3.2-Exp - Keep top-k positions".  Keys and
// values are per head (up-projected from the latent by the caller); a head's
// key is its 128 non-rotary dims followed by the 64 rotary dims shared by all
// heads; scores are scaled, the index mask (0 at the selected positions, -inf
// elsewhere) and the causal mask are added, and the softmax weights the
// head's 128-dim values.
//
//   z[s,h,t] = softmax_scale * (q[s,h,:128] . k_nope[t,h,:] + q[s,h,128:] . k_pe[t,:])
//   out[s,h,:] = sum_{t in J(s)} softmax_t(z[s,h,t]) v[t,h,:],
//   J(s) = {t selected for s} intersect {t <= s}
//
// Two kernels.
//   mha_select_bitmap_kernel turns the index lists into a bitmap, bit t of
//     row s meaning "t is selected for s" (a set, like the excerpt's scatter),
//     stored key-word-major: word w of queries s0..s0+255 are 1 KiB of
//     contiguous bytes, exactly what the attention kernel copies per key tile.
//   mha_prefill_kernel: one workgroup per (sequence, head, block of 256
//     queries), 8 waves of 32 queries (two groups of 16).  Rather than
//     gathering each query's 2048 selected positions (64 KiB per position over
//     all heads), it walks the contiguous key tiles of 32 positions up to the
//     block's causal limit, so each key and value row is read once per 256
//     queries, and masks with the bitmap; every key and value fragment read
//     from LDS feeds the MFMAs of both query groups of a wave, and a wave
//     skips a tile none of its queries selected from.  Tiles come from HBM straight into a 3-slot LDS ring
//     (global_load_lds through inline asm, see mh_copy16); the math is
//     transposed as in the latent attention kernel: S^T[key][query] =
//     K . Q^T with the query fragments in registers, the online softmax per
//     lane (one query per lane, 8 keys per lane, two lane swaps for a
//     maximum), and O^T[d][query] += V^T . P with V^T read by
//     ds_read_b64_tr_b16 and P in registers in the same K order.
//
// LDS layout of a tile (16-byte chunks XOR-swizzled by row so that the score
// reads, 16 rows by one chunk per quarter wave, and the transposing value
// reads, 8 rows by two chunks per half wave, are free of bank conflicts):
//   k_nope 32 rows x 256 B, chunk c of row r at c ^ (r & 15);
//   k_pe   32 rows x 128 B, chunk c of row r at c ^ ((r >> 1) & 7);
//   v      32 rows x 256 B, chunk c of row r at c ^ ((r & 7) << 1);
//   bits   256 words: the tile's bitmap word of each query of the block.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kMhHeads = 128;
constexpr int kMhDn = 128;                 // non-rotary key / query dims
constexpr int kMhDr = 64;                  // rotary dims
constexpr int kMhDq = kMhDn + kMhDr;       // 192
constexpr int kMhDv = 128;
constexpr int kMhWaves = 8;
constexpr int kMhQg = 2;                   // 16-query groups per wave
constexpr int kMhQw = 16 * kMhQg;          // queries per wave (32)
constexpr int kMhQb = kMhWaves * kMhQw;    // queries per workgroup (256)
constexpr int kMhKt = 32;                  // keys per tile (one bitmap word)
constexpr int kMhNbuf = 3;
constexpr int kMhThreads = 256;            // the bitmap kernel
constexpr int kMhPfThreads = kMhWaves * 64;
// Byte offsets of the regions inside a slot: k_nope at 0.
constexpr int kMhOffKp = kMhKt * 256;              // k_pe
constexpr int kMhOffV = kMhOffKp + kMhKt * 128;    // v
constexpr int kMhOffBits = kMhOffV + kMhKt * 256;  // bitmap words
constexpr int kMhSlot = kMhOffBits + kMhQb * 4;
static_assert(kMhSlot == 21504, "slot layout");
static_assert(kMhKt == 4 * kMhWaves, "each wave copies 4 rows of a tile");
constexpr int kMhLoads = 4;                // copies per wave per tile
constexpr float kMhLog2e = 1.4426950408889634f;
constexpr float kMhLn2 = 0.6931471805599453f;
constexpr float kMhSlack = 8.f;

// Bitmap [B][W][Tp] uint32 (W = ceil(T/32) words per query, Tp = T rounded up
// to the 256-query block): bit t%32 of word t/32 of query s is set when t (0 <= t < T) is in
// s's list.  One workgroup per (sequence, 64 queries, 256 words); each thread
// keeps 16 index loads in flight (16 rows at one column) before its atomics.
constexpr int kBmQ = 64, kBmW = 256, kBmRows = 16;
__global__ __launch_bounds__(kMhThreads) void mha_select_bitmap_kernel(
    const int32_t* __restrict__ idx, int T, int k, int W, int Tp, uint32_t* __restrict__ bits) {
  __shared__ uint32_t s_bits[kBmW][kBmQ + 1];
  const int nqb = (T + kBmQ - 1) / kBmQ;
  const int b = blockIdx.x / nqb, s0 = (blockIdx.x - b * nqb) * kBmQ;
  const int w0 = blockIdx.y * kBmW;
  for (int i = threadIdx.x; i < kBmW * (kBmQ + 1); i += kMhThreads) (&s_bits[0][0])[i] = 0u;
  __syncthreads();
  const int nq = min(kBmQ, T - s0);
  const int32_t* src = idx + ((size_t)b * T + s0) * k;
  for (int q0 = 0; q0 < nq; q0 += kBmRows) {
    for (int e = threadIdx.x; e < k; e += kMhThreads) {
      int t[kBmRows];
#pragma unroll
      for (int u = 0; u < kBmRows; ++u) t[u] = q0 + u < nq ? src[(size_t)(q0 + u) * k + e] : -1;
#pragma unroll
      for (int u = 0; u < kBmRows; ++u) {
        const int w = (t[u] >> 5) - w0;
        if (t[u] >= 0 && t[u] < T && w >= 0 && w < kBmW)
          atomicOr(&s_bits[w][q0 + u], 1u << (t[u] & 31));
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBmW * kBmQ; i += kMhThreads) {
    const int w = i / kBmQ, q = i - w * kBmQ;
    if (w0 + w < W && s0 + q < Tp) bits[((size_t)b * W + w0 + w) * Tp + s0 + q] = s_bits[w][q];
  }
}

__global__ __launch_bounds__(kMhPfThreads) void mha_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_nope,
    const uint16_t* __restrict__ k_pe, const uint16_t* __restrict__ v,
    const uint32_t* __restrict__ bits, int B, int T, int W, int Tp, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ __align__(16) uint8_t s_ring[kMhNbuf * kMhSlot];

  // Block -> (sequence, head, query block).  Blocks are dealt round-robin to
  // the 8 XCDs; each XCD gets the heads h = xcd (mod 8), a head's query blocks
  // consecutively (heaviest first), so that head's keys stay in that XCD's L2.
  const int nqb = (T + kMhQb - 1) / kMhQb;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int per_head = nqb, heads_x = kMhHeads / 8;
  const int bh = j / per_head;  // (b, hh)
  const int b = bh / heads_x, h = 8 * (bh - b * heads_x) + xcd;
  const int qb = nqb - 1 - (j - bh * per_head);
  if (b >= B) return;
  const int s0 = qb * kMhQb;
  const int s_last = min(s0 + kMhQb, T) - 1;
  const int n_tiles = s_last / kMhKt + 1;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // This lane's queries (may be >= T in the tail): group qq holds s_me + 16 qq.
  const int s_me = s0 + kMhQw * wave + r16;

  const uint8_t* kn_h = reinterpret_cast<const uint8_t*>(k_nope) + ((size_t)b * T * kMhHeads + h) * 256;
  const uint8_t* kp_b = reinterpret_cast<const uint8_t*>(k_pe) + (size_t)b * T * 128;
  const uint8_t* v_h = reinterpret_cast<const uint8_t*>(v) + ((size_t)b * T * kMhHeads + h) * 256;
  const uint8_t* bt_b = reinterpret_cast<const uint8_t*>(bits + (size_t)b * W * Tp);

  // This wave's share of tile `kt`: k_nope, v and k_pe rows 4w .. 4w+3 (one
  // copy each: 16, 16 and 8 lanes a row) and its 32 queries' bitmap words
  // (8 lanes).  Rows past T read row T-1: no query selects them.
  auto issue = [&](int kt) {
    uint8_t* base = s_ring + (kt % kMhNbuf) * kMhSlot;
    const int t0 = kt * kMhKt;
    {
      const int r = 4 * wv + (lane >> 4);
      const int t = min(t0 + r, T - 1);
      const int cn = (lane & 15) ^ (r & 15);
      lds_copy16_v(kn_h + (size_t)t * (kMhHeads * 256) + cn * 16,
                   __builtin_amdgcn_readfirstlane(lds_addr(base + 4 * wv * 256)));
      const int cv = (lane & 15) ^ ((r & 7) << 1);
      lds_copy16_v(v_h + (size_t)t * (kMhHeads * 256) + cv * 16,
                   __builtin_amdgcn_readfirstlane(lds_addr(base + kMhOffV + 4 * wv * 256)));
    }
    if (lane < 32) {
      const int r = 4 * wv + (lane >> 3);
      const int t = min(t0 + r, T - 1);
      const int cp = (lane & 7) ^ ((r >> 1) & 7);
      lds_copy16_v(kp_b + (size_t)t * 128 + cp * 16,
                   __builtin_amdgcn_readfirstlane(lds_addr(base + kMhOffKp + 4 * wv * 128)));
    }
    if (lane < 8)
      lds_copy16_v(bt_b + ((size_t)kt * Tp + s0 + kMhQw * wv) * 4 + lane * 16,
                   __builtin_amdgcn_readfirstlane(lds_addr(base + kMhOffBits + 4 * kMhQw * wv)));
  };

  float m_run[kMhQg], l_part[kMhQg];
  f32x4 o[kMhQg][8];  // O^T: dims 16ct + 4g + i of this lane's query of group qq
#pragma unroll
  for (int qq = 0; qq < kMhQg; ++qq) {
    m_run[qq] = -INFINITY;
    l_part[qq] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[qq][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  issue(0);
  if (n_tiles > 1) issue(1);
  // Query fragments (B operand of S^T = K . Q^T): dims 32kk + 8g .. +7,
  // loaded behind the first copies and waited for here, once: the compiler
  // does not see the copies, and a wait it placed at the first use inside the
  // loop would drain every tile's copies.
  uint4 qf[kMhQg][6];
#pragma unroll
  for (int qq = 0; qq < kMhQg; ++qq) {
    const uint16_t* qs = q + (((size_t)b * T + min(s_me + 16 * qq, T - 1)) * kMhHeads + h) * kMhDq;
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) qf[qq][kk] = ldg16(qs + kk * 32 + g * 8);
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

#pragma unroll 1
  for (int kt = 0; kt < n_tiles; ++kt) {
    static_assert(kMhNbuf == 3, "the wait below assumes at most one more tile in flight");
    if (kt + 1 < n_tiles)
      __builtin_amdgcn_s_waitcnt(wait_vm(kMhLoads));
    else
      __builtin_amdgcn_s_waitcnt(wait_vm(0));
    lds_barrier();  // tile kt landed for every wave; every wave is done with tile kt-1
    if (kt + 2 < n_tiles) issue(kt + 2);

    const uint8_t* buf = s_ring + (kt % kMhNbuf) * kMhSlot;
    const int t0 = kt * kMhKt;
    // Each query's selections in the tile, restricted to t <= s.
    uint32_t word[kMhQg];
    bool any = false;
#pragma unroll
    for (int qq = 0; qq < kMhQg; ++qq) {
      const int s = s_me + 16 * qq;
      uint32_t w = reinterpret_cast<const uint32_t*>(buf + kMhOffBits)[kMhQw * wave + 16 * qq + r16];
      const int lim = s - t0;  // keys t0 + j with j <= lim are causal for this query
      w = lim >= 31 ? w : (lim < 0 ? 0u : w & ((2u << lim) - 1u));
      word[qq] = s >= T ? 0u : w;
      any |= word[qq] != 0u;
    }
    if (__ballot(any) == 0) continue;  // no query of this wave looks at this tile

    // ---- scores S^T[key][query]: keys 16mt + 4g + i; each K fragment read
    //      from LDS feeds both query groups ----
    f32x4 sc[kMhQg][2];
#pragma unroll
    for (int qq = 0; qq < kMhQg; ++qq) sc[qq][0] = sc[qq][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int r = 16 * mt + r16;
        const uint8_t* a;
        if (kk < 4) a = buf + r * 256 + (((4 * kk + g) ^ (r & 15)) << 4);
        else a = buf + kMhOffKp + r * 128 + (((4 * (kk - 4) + g) ^ ((r >> 1) & 7)) << 4);
        const uint4 kf = *reinterpret_cast<const uint4*>(a);
#pragma unroll
        for (int qq = 0; qq < kMhQg; ++qq)
          sc[qq][mt] = mfma_bf16_16x16x32(as_bf16x8(kf), as_bf16x8(qf[qq][kk]), sc[qq][mt]);
      }
    }
    // ---- online softmax for each of this lane's queries ----
    uint4 pb[kMhQg];
#pragma unroll
    for (int qq = 0; qq < kMhQg; ++qq) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool sel = (word[qq] >> (16 * mt + 4 * g + i)) & 1u;
          sc[qq][mt][i] = sel ? sc[qq][mt][i] : -INFINITY;  // raw score, masked
          mx = fmaxf(mx, sc[qq][mt][i]);
        }
      mx = group_max(mx) * scale_log2;
      const bool grow = mx > m_run[qq] + kMhSlack;
      if (__ballot(grow) != 0) {
        const float alpha =
            grow ? (m_run[qq] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qq] - mx)) : 1.f;
        m_run[qq] = grow ? mx : m_run[qq];
        l_part[qq] *= alpha;
#pragma unroll
        for (int c = 0; c < 8; ++c) o[qq][c] *= alpha;
      }
      const float m_use = m_run[qq] == -INFINITY ? 0.f : m_run[qq];
      float p[2][4], psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[mt][i] = __builtin_amdgcn_exp2f(fmaf(sc[qq][mt][i], scale_log2, -m_use));
          psum += p[mt][i];
        }
      l_part[qq] += psum;
      pb[qq] = uint4{pack2_bf16(p[0][0], p[0][1]), pack2_bf16(p[0][2], p[0][3]),
                     pack2_bf16(p[1][0], p[1][1]), pack2_bf16(p[1][2], p[1][3])};
    }
    // ---- values O^T[d][query] += V^T . P: rows {4g + j, 16 + 4g + j}; each
    //      V fragment feeds both query groups ----
    const int vr = 4 * g + (r16 >> 2);  // row of this lane's 8-byte read (and vr + 16)
    const uint8_t* vrow = buf + kMhOffV + vr * 256 + 8 * (r16 & 1);
    const int vsw = (vr & 7) << 1, vch = (r16 & 3) >> 1;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int off = ((2 * ct + vch) ^ vsw) << 4;
      const i16x4 lo = lds_read_tr16(vrow + off);
      const i16x4 hi = lds_read_tr16(vrow + 16 * 256 + off);
      const uint4 va = uint4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                             (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                             (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                             (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
#pragma unroll
      for (int qq = 0; qq < kMhQg; ++qq)
        o[qq][ct] = mfma_bf16_16x16x32(as_bf16x8(va), as_bf16x8(pb[qq]), o[qq][ct]);
    }
  }

  // ---- finish ----
#pragma unroll
  for (int qq = 0; qq < kMhQg; ++qq) {
    const int s = s_me + 16 * qq;
    const float l_tot = group_sum(l_part[qq]);
    if (s < T) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      uint16_t* orow = out + (((size_t)b * T + s) * kMhHeads + h) * kMhDv + 4 * g;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        *reinterpret_cast<uint2*>(orow + ct * 16) =
            uint2{pack2_bf16(o[qq][ct][0] * inv, o[qq][ct][1] * inv),
                  pack2_bf16(o[qq][ct][2] * inv, o[qq][ct][3] * inv)};
      if (lse != nullptr && g == 0)
        lse[((size_t)b * T + s) * kMhHeads + h] =
            l_tot > 0.f ? (m_run[qq] + log2f(l_tot)) * kMhLn2 : -INFINITY;
    }
  }
}

size_t mha_prefill_workspace_bytes(int B, int T) {
  const size_t W = ((size_t)T + 31) / 32, Tp = ((size_t)T + kMhQb - 1) / kMhQb * kMhQb;
  return (size_t)B * W * Tp * sizeof(uint32_t);
}

int launch_mha_prefill(const void* q, const void* k_nope, const void* k_pe, const void* v,
                       const int32_t* idx, int B, int T, int k, float softmax_scale, void* out,
                       float* lse, void* workspace, hipStream_t stream) {
  const int W = (T + 31) / 32, Tp = (T + kMhQb - 1) / kMhQb * kMhQb;
  uint32_t* bits = reinterpret_cast<uint32_t*>(workspace);
  const int nbq = (T + kBmQ - 1) / kBmQ;
  hipLaunchKernelGGL(mha_select_bitmap_kernel, dim3((unsigned)(B * nbq), (unsigned)((W + kBmW - 1) / kBmW)),
                     dim3(kMhThreads), 0, stream, idx, T, k, W, Tp, bits);
  if (hipGetLastError() != hipSuccess) return -5;
  const int nqb = (T + kMhQb - 1) / kMhQb;
  const unsigned grid = (unsigned)B * kMhHeads * nqb;
  hipLaunchKernelGGL(mha_prefill_kernel, dim3(grid), dim3(kMhPfThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_nope),
                     static_cast<const uint16_t*>(k_pe), static_cast<const uint16_t*>(v), bits, B,
                     T, W, Tp, softmax_scale * kMhLog2e, static_cast<uint16_t*>(out), lse);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace dsa
