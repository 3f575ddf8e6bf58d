"""Plain CPU oracle for the DeepSeek Sparse Attention decode hot path.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``sparse_attention_indexer_amd``) never imports this package, and this
package never imports the product.

The arithmetic of the three decode stages lives in ``dsa_oracle.c`` (plain
C, fp64 sums, OpenMP over query rows), built with gcc into ``liboracle.so``;
for them this module only marshals numpy arrays.  The two per-head products
around the attention (``q_absorb``, ``out_proj``) are written out below as
fp64 numpy contractions, and so are the weight-free indexer input preparation
(``indexer_prep``: RoPE, Hadamard rotation, fp8 block quantisation; its code
decisions are taken in fp32, the precision of the quantiser on the GPU) and
the MHA-form prefill attention (``sparse_mha_prefill``).  Conventions for array arguments:

* bf16 tensors are ``np.uint16`` arrays of raw bfloat16 bits;
* fp8 tensors are ``np.uint8`` arrays of OCP e4m3fn codes;
* everything else is ``np.float32`` / ``np.int32`` as documented per call.

Every function accepts ``rows``: an optional list of flattened query rows
``b*T + t`` to compute (the rest of the output is left as NaN / -2), so a
large workload can be checked on a sample of rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16 = 0
FP8_E4M3 = 1

_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (IEEE semantics: no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load(path: str | None = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _bind(lib):
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.oracle_index_scores.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                        vp, i64, vp]
    lib.oracle_topk.argtypes = [vp, vp, i32, i32, i32, i32, vp, i64, vp]
    lib.oracle_mla.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32,
                               vp, i64, vp, vp]
    for fn in (lib.oracle_index_scores, lib.oracle_topk, lib.oracle_mla):
        fn.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, int(r.size)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = {-1: "bad argument", -2: "non-finite input", -3: "position out of range"}
        raise ValueError(f"oracle {what}: {msg.get(status, status)}")


def index_scores(q, w, k_cache, end_pos, scale, T=None, q_scale=None, k_scale=None, rows=None,
                 lib=None):
    """Indexer scores I[b,t,s] = scale * sum_h w[b,t,h] * ReLU(q[b,t,h] . k[b,s]).

    q: [B,T,H,D] uint16 (bf16 bits) or uint8 (e4m3 codes, then q_scale [B,T,H]
    and k_scale [B,S_max] are required); w: [B,T,H] float32; k_cache:
    [B,S_max,D] same dtype as q; end_pos: [B] int32.  Returns float32
    [B,T,S_max] with NaN past each row's causal bound (and in skipped rows).
    """
    lib = lib or _load()
    dtype = BF16 if q.dtype == np.uint16 else FP8_E4M3
    if dtype == FP8_E4M3 and q.dtype != np.uint8:
        raise TypeError("q must be uint16 (bf16 bits) or uint8 (e4m3 codes)")
    B, T_, H, D = q.shape
    S_max = k_cache.shape[1]
    q = _c(q, q.dtype)
    k_cache = _c(k_cache, k_cache.dtype)
    w = _c(w, np.float32)
    end_pos = _c(end_pos, np.int32)
    q_scale = _c(q_scale, np.float32)
    k_scale = _c(k_scale, np.float32)
    out = np.full((B, T_, S_max), np.nan, dtype=np.float32)
    r, nr = _rows(rows)
    st = lib.oracle_index_scores(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache), _ptr(k_scale),
                                 _ptr(end_pos), B, T_, S_max, H, D, float(scale), dtype,
                                 _ptr(r), nr, _ptr(out))
    _check(st, "index_scores")
    return out


def topk(scores, end_pos, k, rows=None, lib=None):
    """Top-k positions per row: ascending order, ties to the smaller position, -1 padded.

    scores: [B,T,S_max] float32; end_pos: [B] int32.  Returns int32 [B,T,k]
    (rows not in ``rows`` are filled with -2).
    """
    lib = lib or _load()
    B, T, S_max = scores.shape
    scores = _c(scores, np.float32)
    end_pos = _c(end_pos, np.int32)
    out = np.full((B, T, k), -2, dtype=np.int32)
    r, nr = _rows(rows)
    st = lib.oracle_topk(_ptr(scores), _ptr(end_pos), B, T, S_max, int(k), _ptr(r), nr, _ptr(out))
    _check(st, "topk")
    return out


def mla(q_nope, q_pe, kv_cache, pe_cache, end_pos, softmax_scale, indices=None, rows=None,
        lib=None):
    """Absorbed MLA attention with an additive index mask (dense if indices is None).

    q_nope: [B,T,H,Dc], q_pe: [B,T,H,Dr], kv_cache: [B,S_max,Dc], pe_cache:
    [B,S_max,Dr], all uint16 bf16 bits; indices: [B,T,k] int32 (-1 = empty)
    or None; end_pos: [B] int32.  Returns (out float64 [B,T,H,Dc],
    lse float64 [B,T,H]), NaN in rows that were not computed.
    """
    lib = lib or _load()
    B, T, H, Dc = q_nope.shape
    Dr = q_pe.shape[-1]
    S_max = kv_cache.shape[1]
    arrs = [_c(a, np.uint16) for a in (q_nope, q_pe, kv_cache, pe_cache)]
    idx = _c(indices, np.int32)
    k = 0 if idx is None else idx.shape[-1]
    end_pos = _c(end_pos, np.int32)
    out = np.full((B, T, H, Dc), np.nan, dtype=np.float64)
    lse = np.full((B, T, H), np.nan, dtype=np.float64)
    r, nr = _rows(rows)
    st = lib.oracle_mla(*[_ptr(a) for a in arrs], _ptr(idx), _ptr(end_pos), B, T, S_max, H, Dc,
                        Dr, k, float(softmax_scale), _ptr(r), nr, _ptr(out), _ptr(lse))
    _check(st, "mla")
    return out, lse


# --- query absorption and output up-projection ------------------------------
# MQA decode branch of "DeepSeek-V3.2-Exp - Apply sparse mask": wkv_b viewed
# as [heads, qk_nope_head_dim + v_head_dim, kv_lora_rank] = [128, 128+128, 512].

QK_NOPE = 128
V_HEAD = 128


def bf16_to_f64(bits):
    """bfloat16 bits (uint16) -> float64 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _as_f64(a):
    """bf16 bits (uint16) are decoded; float arrays are taken as they are."""
    a = np.asarray(a)
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def q_absorb(q_nope, wkv_b):
    """q_abs[b,t,h,c] = sum_d q_nope[b,t,h,d] * wkv_b[h,d,c] over the first 128 rows of
    each head's slice (the query absorption).  q_nope [B,T,128,128] and wkv_b
    [128,256,512] as bf16 bits (or float arrays); returns float64 [B,T,128,512]."""
    q = _as_f64(q_nope)
    w = _as_f64(wkv_b)[:, :QK_NOPE, :]
    return np.einsum("bthd,hdc->bthc", q, w)


def out_proj(x, wkv_b):
    """y[b,t,h,d] = sum_c x[b,t,h,c] * wkv_b[h,128+d,c] over the last v_head_dim rows of
    each head's slice (the output up-projection).  x [B,T,128,512] and wkv_b as bf16
    bits (or float arrays); returns float64 [B,T,128,128]."""
    xx = _as_f64(x)
    w = _as_f64(wkv_b)[:, -V_HEAD:, :]
    return np.einsum("bthc,hdc->bthd", xx, w)


# --- indexer input preparation (weight-free part) -----------------------------
# The Indexer.forward excerpt on "DeepSeek-V3.2-Exp - Keep top-k positions":
# RoPE on the first 64 dims ("not interleaved"), those dims first, then
# rotate_activation, then act_quant with 128-element blocks, and the key
# written to k_cache / k_scale_cache at its position.  The pages name these
# steps but do not spell them out; the readings taken here:
#   * RoPE "not interleaved": dim i pairs with dim i + 32 of the 64 rope dims,
#     (x_i + j x_{i+32}) times (cos_i + j sin_i) for the token's position;
#   * rotate_activation: the orthonormal Walsh-Hadamard transform of the
#     128-dim vector (Sylvester order, scaled by 128^-1/2);
#   * act_quant(x, 128): scale = max|x| / 448 (fp32), codes = x / scale
#     rounded to the nearest e4m3 value (ties to even), saturating at 448.

ROPE_DIM = 64
E4M3_MAX = 448.0


def rope_halves(x, cos, sin):
    """x [..., 64] rotated pairwise: (x_i, x_{i+32}) -> (x_i c - x_{i+32} s, x_i s + x_{i+32} c)."""
    x1, x2 = x[..., :ROPE_DIM // 2], x[..., ROPE_DIM // 2:ROPE_DIM]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], -1)


def hadamard128(x, scaled=True):
    """Walsh-Hadamard transform over the last axis (128), Sylvester order, built from the
    recursion H_2n = [[H_n, H_n], [H_n, -H_n]] one doubling at a time; times 128^-1/2
    when ``scaled``."""
    y = np.array(x, dtype=np.float64)
    lead = y.shape[:-1]
    h = 1
    while h < 128:
        y = y.reshape(lead + (128 // (2 * h), 2, h))
        a, b = y[..., 0, :], y[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2)
        h *= 2
    y = y.reshape(lead + (128,))
    return y / np.sqrt(128.0) if scaled else y


def _e4m3_table():
    """The 127 non-negative finite e4m3fn values, indexed by code 0..126."""
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


_E4M3 = _e4m3_table()


def e4m3_encode(x):
    """Nearest e4m3fn code (ties to the even code), saturating at +-448; the sign bit
    follows the sign of x (so -0 and small negatives give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3, a, side="left")          # first value >= a
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3[lo], _E4M3[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a >= _E4M3[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(x)
    return (code | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def act_quant_128(u, post_scale):
    """Block-128 quantisation of u [..., 128] (u = the rotation before its 128^-1/2
    factor, post_scale = that factor): the code decision is taken in fp32 --
    scale_u = fp32(max|u| / 448), codes = e4m3(fp32(u / scale_u)) -- and the
    returned scale is fp32(scale_u * post_scale), the scale of u * post_scale.
    An all-zero block gets scale 0 and zero codes."""
    u32 = np.asarray(u, dtype=np.float64).astype(np.float32)
    amax = np.max(np.abs(u32), axis=-1)
    scale_u = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale_u > 0, scale_u, np.float32(1.0))
    q = (u32 / safe[..., None]).astype(np.float32)
    codes = e4m3_encode(q)
    codes = np.where((scale_u > 0)[..., None], codes, np.uint8(0))
    return codes, (scale_u * np.float32(post_scale)).astype(np.float32)


def indexer_prep(q_in, k_in, rope_cos, rope_sin, end_pos, fp8=True):
    """Weight-free indexer input preparation for B sequences of T new tokens.

    q_in [B,T,64,128] and k_in [B,T,128] as bf16 bits; rope_cos / rope_sin
    [S_max,32] float32 tables by absolute position; token t of sequence b sits at
    position end_pos[b] - T + t.  Returns (q, q_scale, k, k_scale, pos): with fp8,
    q [B,T,64,128] / k [B,T,128] are uint8 e4m3 codes and the scales float32
    [B,T,64] / [B,T]; otherwise q and k are the rotated values in float64 (no
    scales).  pos [B,T] are the cache rows the keys go to."""
    q = _as_f64(q_in).copy()
    k = _as_f64(k_in).copy()
    B, T = q.shape[:2]
    pos = np.asarray(end_pos, np.int64)[:, None] - T + np.arange(T)[None, :]
    c = np.asarray(rope_cos, np.float32).astype(np.float64)[pos]    # [B,T,32]
    s = np.asarray(rope_sin, np.float32).astype(np.float64)[pos]
    q[..., :ROPE_DIM] = rope_halves(q[..., :ROPE_DIM], c[:, :, None, :], s[:, :, None, :])
    k[..., :ROPE_DIM] = rope_halves(k[..., :ROPE_DIM], c, s)
    post = float(np.float32(1.0 / np.sqrt(128.0)))
    if not fp8:
        return hadamard128(q), None, hadamard128(k), None, pos
    qc, qs = act_quant_128(hadamard128(q, scaled=False), post)
    kc, ks = act_quant_128(hadamard128(k, scaled=False), post)
    return qc, qs, kc, ks, pos


# --- MHA-form prefill attention (the `mask is not None` branch) ----------------
# The MHA prefill excerpt on "DeepSeek-V3.2-Exp - Keep top-k positions": keys
# and values are up-projected per head from the latent; each head's key is its
# non-rotary part followed by the shared rotary key; scores are scaled, the
# index mask (0 at the selected positions, -inf elsewhere, built by a scatter,
# so a position listed twice counts once) and the causal mask are added, then
# softmax and the weighted sum of the values.  Token s of a sequence is query
# position s and sees key positions t <= s of the same sequence.

def sparse_mha_prefill(q, k_nope, k_pe, v, indices, softmax_scale, rows=None):
    """q [B,T,H,192] (non-rotary 128 then rotary 64), k_nope [B,T,H,128],
    k_pe [B,T,64], v [B,T,H,128] as bf16 bits; indices [B,T,k] int32 (entries
    outside 0..T-1 select nothing).  Returns (out [B,T,H,128] float64,
    lse [B,T,H] float64, natural log); rows selects flattened b*T+s rows to
    compute (others NaN).  A query with no position both selected and causal
    gets out 0 and lse -inf."""
    qf, kn, kp, vf = _as_f64(q), _as_f64(k_nope), _as_f64(k_pe), _as_f64(v)
    idx = np.asarray(indices)
    B, T, H = qf.shape[:3]
    dv = vf.shape[-1]
    out = np.full((B, T, H, dv), np.nan)
    lse = np.full((B, T, H), np.nan)
    todo = range(B * T) if rows is None else rows
    for r in todo:
        b, s = divmod(int(r), T)
        sel = idx[b, s]
        sel = np.unique(sel[(sel >= 0) & (sel < T)])
        sel = sel[sel <= s]                                   # the causal mask
        if sel.size == 0:
            out[b, s], lse[b, s] = 0.0, -np.inf
            continue
        keys = np.concatenate([kn[b, sel], np.broadcast_to(kp[b, sel][:, None, :],
                                                           (sel.size, H, kp.shape[-1]))], -1)
        z = np.einsum("hd,nhd->hn", qf[b, s], keys) * float(softmax_scale)
        m = z.max(-1, keepdims=True)
        p = np.exp(z - m)
        l = p.sum(-1, keepdims=True)
        out[b, s] = np.einsum("hn,nhd->hd", p, vf[b, sel]) / l
        lse[b, s] = (m + np.log(l))[:, 0]
    return out, lse
