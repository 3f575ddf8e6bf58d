"""Seeded synthetic inputs for the DSA decode hot path.

This module draws tensors; it contains none of the method's arithmetic.
Both the HIP path and the CPU oracle are fed from it, so they see the same
bytes.  Random numbers come from a seeded ``torch.Generator`` on the device
the tensors are made on (CPU draws are reproducible across machines; GPU
draws are reproducible on the same software stack).

Shapes and distributions follow the workloads the pages describe:

* indexer: 64 heads x 128 dims of query, one shared 128-dim key per cached
  token, one fp32 weight per head ("DeepSeek-V3.2-Exp - Keep top-k
  positions", Indexer.forward excerpt; MaxText PR #2933 config list
  ``index_n_heads 64, index_head_dim 128, index_topk 2048``);
* fp8 variant: OCP e4m3fn codes with one fp32 scale per 128-element block
  (one per query head and one per key), like ``act_quant`` with block 128;
* MLA: 128 heads, a 512-wide latent plus a 64-wide rope part per cached
  token, and the absorbed query in the same 512+64 space ("DeepSeek-V3.2-Exp
  - Apply sparse mask", MQA decode excerpt).

Encodings used here are conversions done by torch: fp32 -> bf16 and
fp32 -> float8_e4m3fn are round-to-nearest-even.  fp8 indexer inputs are
drawn as codes and block scales directly (``fp8_draw``), not quantised from
fp32 data.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, fields
from typing import Optional

import numpy as np
import torch

N_IDX_HEADS = 64
IDX_DIM = 128
N_HEADS = 128
D_LATENT = 512
D_ROPE = 64
QK_HEAD_DIM = 192  # per-head query/key width before absorption: 128 non-rope + 64 rope
TOPK = 2048
FP8_MAX = 448.0


@dataclass
class Case:
    """One decode (or prefill-shaped) batch: every input of the hot path.

    Query ``t`` of sequence ``b`` sits at position ``end_pos[b] - T + t`` and
    may attend to cached positions ``0..end_pos[b]-T+t``.
    """

    name: str
    B: int
    T: int
    S_max: int
    dtype: str                      # "bf16" or "fp8" (indexer q/k storage)
    end_pos: torch.Tensor           # [B] int32
    q: torch.Tensor                 # [B,T,64,128] bf16 or float8_e4m3fn
    w: torch.Tensor                 # [B,T,64] fp32
    k_cache: torch.Tensor           # [B,S_max,128] bf16 or float8_e4m3fn
    q_scale: Optional[torch.Tensor]  # [B,T,64] fp32 (fp8 only)
    k_scale: Optional[torch.Tensor]  # [B,S_max] fp32 (fp8 only)
    q_nope: torch.Tensor            # [B,T,128,512] bf16
    q_pe: torch.Tensor              # [B,T,128,64] bf16
    kv_cache: torch.Tensor          # [B,S_max,512] bf16
    pe_cache: torch.Tensor          # [B,S_max,64] bf16
    scale: float = 1.0 / math.sqrt(IDX_DIM)
    softmax_scale: float = 1.0 / math.sqrt(QK_HEAD_DIM)
    topk: int = TOPK
    recipe: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def max_end_pos(self) -> int:
        return int(self.end_pos.max().item())

    def to(self, device) -> "Case":
        kw = {}
        for f in fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Case(**kw)

    def numpy(self) -> dict:
        """Host copies in the oracle's conventions (bf16 -> uint16 bits, fp8 -> uint8 codes)."""
        out = {}
        for f in fields(self):
            v = getattr(self, f.name)
            if isinstance(v, torch.Tensor):
                out[f.name] = to_numpy(v)
        return out


def to_numpy(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _ints(shape, lo, hi, g, device):
    """Integers uniform in [lo, hi] as fp32."""
    return torch.randint(lo, hi + 1, shape, generator=g, device=device).to(torch.float32)


def _pow2_weights(shape, g, device, emin=-3, emax=3):
    """+-2^e with e uniform in [emin, emax]: exact in every format used."""
    e = torch.randint(emin, emax + 1, shape, generator=g, device=device).to(torch.float32)
    sign = torch.randint(0, 2, shape, generator=g, device=device).to(torch.float32) * 2 - 1
    return sign * torch.exp2(e)


def _layer_norm(x, eps=1e-6):
    """Synthetic stand-in for the key normalisation: zero mean, unit variance per row."""
    mu = x.mean(-1, keepdim=True)
    var = ((x - mu) ** 2).mean(-1, keepdim=True)
    return (x - mu) / torch.sqrt(var + eps)


def fp8_draw(shape, g, device):
    """Synthetic fp8 data of the shape act_quant produces, drawn directly: e4m3fn
    codes of N(0,1) * 150 clamped to +-448 (so a 128-element block spans the
    code range up to near its top) and fp32 block scales uniform in
    [0.005, 0.01] (about the scale unit-variance data gets), one per block of
    the last dim."""
    x = (_normal(shape, g, device) * 150.0).clamp(-FP8_MAX, FP8_MAX)
    scale = torch.rand(shape[:-1], generator=g, device=device, dtype=torch.float32)
    return x.to(torch.float8_e4m3fn), (0.005 + 0.005 * scale).contiguous()


def make_case(name: str, B: int, T: int, end_pos, S_max: int, *, dtype: str = "bf16",
              index_dist: str = "normal", k_norm: bool = False, seed: int = 0,
              device="cpu", topk: int = TOPK, key_pattern: Optional[str] = None,
              dup_period: int = 1024, recipe: str = "") -> Case:
    """Draw every input of one batch.

    index_dist "normal": q, k, w ~ N(0,1) fp32 before encoding (fp8: codes and
                         scales drawn by fp8_draw instead of q and k).
    index_dist "int":    q, k integers in [-4,4] and w = +-2^e, e in [-3,3];
                         with these every fp32 partial sum of the score is an
                         exact integer multiple of 2^-3 below 2^20.
    key_pattern "dup":   k[s] = k[s mod dup_period] (forces ties at the cut);
                "equal": every key row equal (every score equal).
    The MLA inputs are always ~N(0,1) bf16.
    """
    g = _gen(seed, device)
    end_pos_t = torch.as_tensor(end_pos, dtype=torch.int32).reshape(-1).to(device)
    assert end_pos_t.numel() == B
    H, D = N_IDX_HEADS, IDX_DIM
    if index_dist == "normal":
        qf = _normal((B, T, H, D), g, device)
        kf = _normal((B, S_max, D), g, device)
        wf = _normal((B, T, H), g, device)
    elif index_dist == "int":
        qf = _ints((B, T, H, D), -4, 4, g, device)
        kf = _ints((B, S_max, D), -4, 4, g, device)
        wf = _pow2_weights((B, T, H), g, device)
    else:
        raise ValueError(index_dist)
    if key_pattern == "dup":
        src = kf[:, :dup_period].clone()
        reps = (S_max + dup_period - 1) // dup_period
        kf = src.repeat(1, reps, 1)[:, :S_max].contiguous()
    elif key_pattern == "equal":
        kf = kf[:, :1].expand(B, S_max, D).contiguous()
    if k_norm:
        kf = _layer_norm(kf)
    q_scale = k_scale = None
    if dtype == "bf16":
        q = qf.to(torch.bfloat16)
        k_cache = kf.to(torch.bfloat16)
    elif dtype == "fp8":
        if index_dist == "int":  # integers in [-4,4] are exact e4m3 codes; scale 1
            q = qf.to(torch.float8_e4m3fn)
            k_cache = kf.to(torch.float8_e4m3fn)
            q_scale = torch.ones((B, T, H), dtype=torch.float32, device=device)
            k_scale = torch.ones((B, S_max), dtype=torch.float32, device=device)
        else:
            q, q_scale = fp8_draw((B, T, H, D), g, device)
            k_cache, k_scale = fp8_draw((B, S_max, D), g, device)
    else:
        raise ValueError(dtype)
    q_nope = _normal((B, T, N_HEADS, D_LATENT), g, device).to(torch.bfloat16)
    q_pe = _normal((B, T, N_HEADS, D_ROPE), g, device).to(torch.bfloat16)
    kv_cache = _normal((B, S_max, D_LATENT), g, device).to(torch.bfloat16)
    pe_cache = _normal((B, S_max, D_ROPE), g, device).to(torch.bfloat16)
    return Case(name=name, B=B, T=T, S_max=S_max, dtype=dtype, end_pos=end_pos_t, q=q,
                w=wf.contiguous(), k_cache=k_cache, q_scale=q_scale, k_scale=k_scale,
                q_nope=q_nope, q_pe=q_pe, kv_cache=kv_cache, pe_cache=pe_cache, topk=topk,
                recipe=recipe)


# --- the named workloads -----------------------------------------------------

def tiny_decode(variant: str = "base", seed: int = 1, device="cpu") -> Case:
    """1 query over 4096 cached tokens, integer-valued indexer inputs (exact fp32 sums).

    variants: base; dup (k[s] = k[s mod 1024], ties at the cut); equal (all
    keys equal); short (1001 cached tokens, fewer than k); fp8int (same
    integers stored as e4m3 codes with scale 1).
    """
    n = 1001 if variant == "short" else 4096
    dtype = "fp8" if variant == "fp8int" else "bf16"
    kp = {"dup": "dup", "equal": "equal"}.get(variant)
    return make_case(f"tiny_decode_{variant}", 1, 1, [n], n, dtype=dtype, index_dist="int",
                     seed=seed, device=device, key_pattern=kp,
                     recipe="B=1 T=1; q,k int U[-4,4]; w=+-2^U[-3,3]; MLA N(0,1) bf16")


def decode_32k(seed: int = 2, device="cpu", n: int = 32768) -> Case:
    """Batch 1 decode at 32768 cached tokens, bf16 throughout, k layer-normed."""
    return make_case("decode_32k_bf16", 1, 1, [n], n, dtype="bf16", index_dist="normal",
                     k_norm=True, seed=seed, device=device,
                     recipe="B=1 T=1 n=32768; q,k,w N(0,1), k layer-normed; bf16")


def decode_b64_varlen(seed: int = 3, device="cpu", B: int = 64, lo: int = 8192,
                      hi: int = 131072) -> Case:
    """Batch 64 decode, context lengths uniform in [8192, 131072], fp8 indexer."""
    g = _gen(seed + 1000, "cpu")
    end_pos = torch.randint(lo, hi + 1, (B,), generator=g).to(torch.int32)
    return make_case("decode_b64_varlen_fp8", B, 1, end_pos, hi, dtype="fp8",
                     index_dist="normal", seed=seed, device=device,
                     recipe=f"B={B} T=1 end_pos~U[{lo},{hi}] S_max={hi}; fp8 q,k block-128; bf16 MLA")


def prefill(T: int = 8192, seed: int = 4, device="cpu") -> Case:
    """One causal sequence of T queries starting at position 0, bf16."""
    return make_case(f"prefill_{T}_bf16", 1, T, [T], T, dtype="bf16", index_dist="normal",
                     seed=seed, device=device, recipe=f"B=1 T={T} start_pos=0; bf16 N(0,1)")


def sweep(n: int, seed: int = 5, device="cpu", B: int = 8) -> Case:
    """Batch 8 decode at a fixed context n, fp8 indexer, bf16 MLA."""
    return make_case(f"sweep_b{B}_n{n}_fp8", B, 1, [n] * B, n, dtype="fp8",
                     index_dist="normal", seed=seed, device=device,
                     recipe=f"B={B} T=1 n={n}; fp8 q,k block-128; bf16 MLA")


SWEEP_CONTEXTS = (1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072)


# --- the products around the attention ----------------------------------------

def make_prep(B: int, T: int, end_pos, S_max: int, kind: str = "normal", seed: int = 0,
              device="cpu"):
    """Inputs of the indexer input preparation: (q_in [B,T,64,128] bf16,
    k_in [B,T,128] bf16, rope_cos [S_max,32] fp32, rope_sin [S_max,32] fp32,
    end_pos [B] int32).

    kind "normal": q ~ N(0,1) (the query projection's output), k ~ N(0,1)
      centred and scaled to unit variance per row (standing in for k_norm), and
      cos/sin of angles drawn uniform in [-pi, pi) per (position, pair).
    kind "int": q, k integers in [-8, 8] and cos = 1, sin = 0, so every sum of
      the rotation is an exact integer in fp32.
    kind "zero": as "normal" but with some query heads and keys all zero.
    """
    g = _gen(seed, device)
    end_pos_t = torch.as_tensor(end_pos, dtype=torch.int32).reshape(-1).to(device)
    assert end_pos_t.numel() == B
    shp_q, shp_k = (B, T, N_IDX_HEADS, IDX_DIM), (B, T, IDX_DIM)
    if kind == "int":
        q, k = _ints(shp_q, -8, 8, g, device), _ints(shp_k, -8, 8, g, device)
        cos = torch.ones((S_max, 32), dtype=torch.float32, device=device)
        sin = torch.zeros((S_max, 32), dtype=torch.float32, device=device)
    elif kind in ("normal", "zero"):
        q, k = _normal(shp_q, g, device), _layer_norm(_normal(shp_k, g, device))
        ang = (torch.rand((S_max, 32), generator=g, device=device) * 2 - 1) * math.pi
        cos, sin = torch.cos(ang), torch.sin(ang)
        if kind == "zero":
            q[..., ::7, :] = 0.0
            k[..., ::3, :] = 0.0
    else:
        raise ValueError(kind)
    bf = torch.bfloat16
    return q.to(bf), k.to(bf), cos.contiguous(), sin.contiguous(), end_pos_t


def make_mha(B: int, T: int, seed: int = 0, device="cpu"):
    """Inputs of the MHA-form prefill attention, standing in for keys and values
    up-projected from the latent: q [B,T,128,192] (non-rotary 128, rotary 64),
    k_nope [B,T,128,128], k_pe [B,T,64], v [B,T,128,128], all N(0,1) in bf16."""
    g = _gen(seed, device)
    bf = torch.bfloat16
    q = _normal((B, T, N_HEADS, 192), g, device).to(bf)
    kn = _normal((B, T, N_HEADS, 128), g, device).to(bf)
    kp = _normal((B, T, D_ROPE), g, device).to(bf)
    v = _normal((B, T, N_HEADS, 128), g, device).to(bf)
    return q, kn, kp, v


def make_proj(B: int, T: int, seed: int = 0, device="cpu"):
    """Inputs of the query absorption and output up-projection: q_nope
    [B,T,128,128] ~N(0,1), a synthetic wkv_b [128,256,512] ~N(0,1)/sqrt(fan-in)
    (128 for the key rows, 512 for the value rows, so outputs are O(1)), and a
    latent attention output x [B,T,128,512] ~N(0,1); all bf16."""
    g = _gen(seed, device)
    qn = _normal((B, T, N_HEADS, 128), g, device)
    wk = _normal((N_HEADS, 128, D_LATENT), g, device) / math.sqrt(128)
    wv = _normal((N_HEADS, 128, D_LATENT), g, device) / math.sqrt(D_LATENT)
    x = _normal((B, T, N_HEADS, D_LATENT), g, device)
    bf = torch.bfloat16
    return qn.to(bf), torch.cat([wk, wv], 1).to(bf), x.to(bf)


# --- standalone inputs for the selection and attention stages ----------------

def make_scores(B: int, T: int, S_max: int, kind: str = "normal", seed: int = 0,
                device="cpu") -> torch.Tensor:
    """Synthetic fp32 score rows [B,T,S_max] for exercising top-k on its own.

    kinds: normal (N(0,1)); ties (integers 0..63, many equal values at the
    cut); equal (all 1.0); zeros (+0/-0 mixed with a few +-1: signed-zero
    ties); relu (70% exact zeros of either sign, the rest |N(0,1)|);
    wide (N(0,1) times 2^U[-60,60], spread over the exponent range).
    """
    g = _gen(seed, device)
    shape = (B, T, S_max)
    if kind == "normal":
        x = _normal(shape, g, device)
    elif kind == "ties":
        x = _ints(shape, 0, 63, g, device)
    elif kind == "equal":
        x = torch.ones(shape, device=device)
    elif kind == "zeros":
        u = torch.rand(shape, generator=g, device=device)
        x = torch.where(u < 0.45, torch.zeros_like(u), -torch.zeros_like(u))
        x = torch.where(u > 0.95, torch.ones_like(u), x)
        x = torch.where((u > 0.90) & (u <= 0.95), -torch.ones_like(u), x)
    elif kind == "relu":
        u = torch.rand(shape, generator=g, device=device)
        mag = _normal(shape, g, device).abs()
        z = torch.where(u < 0.35, torch.zeros_like(u), -torch.zeros_like(u))
        x = torch.where(u < 0.7, z, mag)
    elif kind == "wide":
        e = torch.randint(-60, 61, shape, generator=g, device=device).to(torch.float32)
        x = _normal(shape, g, device) * torch.exp2(e)
    else:
        raise ValueError(kind)
    return x.contiguous()


def make_indices(B: int, T: int, end_pos, k: int, seed: int = 0, fill: str = "random",
                 device="cpu") -> torch.Tensor:
    """Synthetic selections [B,T,k] int32 for exercising attention on its own.

    Each row holds min(k, valid) distinct positions of 0..bound in ascending
    order followed by -1 (the layout top-k produces).  fill "random": a
    uniformly random subset; "first": 0..k_eff-1; "last": the k_eff most
    recent positions.
    """
    g = _gen(seed, "cpu")
    ep = torch.as_tensor(end_pos, dtype=torch.int64).reshape(-1)
    out = torch.full((B, T, k), -1, dtype=torch.int32)
    for b in range(B):
        for t in range(T):
            n = int(ep[b]) - T + t + 1
            ke = min(k, n)
            if fill == "random":
                sel = torch.randperm(n, generator=g)[:ke].sort().values
            elif fill == "first":
                sel = torch.arange(ke)
            elif fill == "last":
                sel = torch.arange(n - ke, n)
            else:
                raise ValueError(fill)
            out[b, t, :ke] = sel.to(torch.int32)
    return out.to(device)
