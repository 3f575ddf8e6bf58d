"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``check_*`` function takes a loaded oracle library (``lib``), so the same
pins can be run against deliberately broken builds of the oracle source (see
test_oracle_mutants.py).  What each pin compares against:

* hand-derived worked examples stored under tests/golden/ (with citations);
* library routines on special cases: torch matmul (single-head indexer),
  torch's own bf16/fp8 decoding, torch stable sort (top-k), torch
  scaled_dot_product_attention and logsumexp in float64 (attention);
* brute force over every subset of tiny rows (top-k);
* exact algebraic invariants on integer inputs (sum over heads, linearity in
  the weights, head permutation) and closed forms (one kept row returns that
  row, a zero query returns the mean of the kept rows);
* for the absorption and up-projection: selector weights, and the identity
  between the pages' two attention forms (absorbed decode vs MHA prefill);
* for the indexer input preparation: torch's complex multiply (RoPE), scipy's
  Hadamard matrix (rotation), torch's float8_e4m3fn cast (encoder), RoPE's
  relative-position property, the position convention of the k_cache write,
  and e4m3's half-step error bound (block quantisation);
* for the MHA-form prefill attention: torch scaled_dot_product_attention and
  logsumexp with a boolean (selected and causal) mask, closed forms, and the
  identity with the absorbed form (q_absorb -> mla -> up-projection) on
  up-projected keys and values.
"""
from __future__ import annotations

import itertools
import os

import numpy as np
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def read_golden(name):
    """Parse a tests/golden fixture: '# comment' lines and 'key = values' entries."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = [float(x) for x in val.split()]
    return out


# --- encodings done by torch (independent of the oracle's decoders) ----------

def bf16(x) -> np.ndarray:
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_val(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .to(torch.float64).numpy()


def fp8_val(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def valid_mask(end_pos, T, S_max):
    """[B,T,S_max] bool: s <= end_pos[b] - T + t."""
    ep = np.asarray(end_pos).reshape(-1, 1, 1)
    t = np.arange(T).reshape(1, -1, 1)
    s = np.arange(S_max).reshape(1, 1, -1)
    return s <= ep - T + t


def close32(a, b, rel=2.0 ** -21):
    """Agreement of fp32 results whose fp64 sums may have run in another order."""
    return np.all(np.abs(a - b) <= rel * np.abs(b) + 1e-30)


# --- indexer -------------------------------------------------------------------

def check_indexer_golden(lib):
    g = read_golden("indexer_worked_example.txt")
    q = bf16(np.array(g["q_t0"] + g["q_t1"]).reshape(1, 2, 2, 2))
    w = np.array([g["w_t0"], g["w_t1"]], np.float32).reshape(1, 2, 2)
    k = bf16(np.array(g["k"]).reshape(1, 4, 2))
    ep = np.array([3], np.int32)
    out = oracle.index_scores(q, w, k, ep, g["scale"][0], lib=lib)
    expect = np.array([g["scores_t0"], g["scores_t1"]], np.float32)[None]
    assert np.array_equal(out, expect, equal_nan=True), out
    for kk in (2, 4):
        sel = oracle.topk(out, ep, kk, lib=lib)
        assert sel[0, 0].tolist() == [int(x) for x in g[f"topk{kk}_t0"]], sel
        assert sel[0, 1].tolist() == [int(x) for x in g[f"topk{kk}_t1"]], sel


def check_fp8_decoding(lib):
    """Every finite e4m3 code decodes like torch.float8_e4m3fn (q=code, k=+-1, H=D=1)."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    B = codes.size
    q = codes.reshape(B, 1, 1, 1)
    k = np.tile(np.array([0x38, 0xB8], np.uint8).reshape(1, 2, 1), (B, 1, 1))  # +1, -1
    ones_q = np.ones((B, 1, 1), np.float32)
    ones_k = np.ones((B, 2), np.float32)
    out = oracle.index_scores(q, ones_q, k, np.full(B, 2, np.int32), 1.0, q_scale=ones_q,
                              k_scale=ones_k, lib=lib)
    got = out[:, 0, 0].astype(np.float64) - out[:, 0, 1].astype(np.float64)
    assert np.array_equal(got, fp8_val(codes)), np.nonzero(got != fp8_val(codes))


def check_bf16_decoding(lib):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 16, size=600, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF][:512]  # finite only
    B = bits.size
    q = bits.reshape(B, 1, 1, 1)
    k = np.tile(bf16([1.0, -1.0]).reshape(1, 2, 1), (B, 1, 1))
    out = oracle.index_scores(q, np.ones((B, 1, 1), np.float32), k, np.full(B, 2, np.int32), 1.0,
                              lib=lib)
    got = out[:, 0, 0].astype(np.float64) - out[:, 0, 1].astype(np.float64)
    assert np.array_equal(got, bf16_val(bits))


def check_single_head_matmul(lib):
    """H=1: I = fl32(fl32(w * ReLU(q.k)) * scale), with q.k from torch matmul; causal tail unwritten."""
    rng = np.random.default_rng(3)
    B, T, S, D = 2, 3, 40, 5
    ep = np.array([37, 40], np.int32)
    q = bf16(rng.standard_normal((B, T, 1, D)))
    k = bf16(rng.standard_normal((B, S, D)))
    w = rng.standard_normal((B, T, 1)).astype(np.float32)
    scale = np.float32(0.37)
    out = oracle.index_scores(q, w, k, ep, scale, lib=lib)
    dots = torch.matmul(torch.from_numpy(bf16_val(q)[:, :, 0, :]),
                        torch.from_numpy(bf16_val(k)).transpose(1, 2)).numpy()
    acc = w.astype(np.float64) * np.maximum(dots, 0.0)
    expect = acc.astype(np.float32) * scale
    m = valid_mask(ep, T, S)
    assert close32(out[m], expect[m])
    assert np.all(np.isnan(out[~m]))


def check_fp8_single_head_matmul(lib):
    """fp8 values are code * block scale: compare with torch's decoding and matmul."""
    rng = np.random.default_rng(5)
    B, T, S, D = 2, 2, 24, 16
    ep = np.array([24, 19], np.int32)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    q = rng.choice(codes, size=(B, T, 1, D)).astype(np.uint8)
    k = rng.choice(codes, size=(B, S, D)).astype(np.uint8)
    q_scale = (rng.random((B, T, 1)) * 0.01 + 1e-3).astype(np.float32)
    k_scale = (rng.random((B, S)) * 0.01 + 1e-3).astype(np.float32)
    w = rng.standard_normal((B, T, 1)).astype(np.float32)
    out = oracle.index_scores(q, w, k, ep, 0.25, q_scale=q_scale, k_scale=k_scale, lib=lib)
    qd = fp8_val(q)[:, :, 0, :] * q_scale.astype(np.float64)
    kd = fp8_val(k) * k_scale.astype(np.float64)[..., None]
    dots = torch.matmul(torch.from_numpy(qd), torch.from_numpy(kd).transpose(1, 2)).numpy()
    expect = (w.astype(np.float64) * np.maximum(dots, 0.0)).astype(np.float32) * np.float32(0.25)
    m = valid_mask(ep, T, S)
    assert close32(out[m], expect[m])


def _int_case(rng, B, T, H, D, S):
    q = bf16(rng.integers(-4, 5, size=(B, T, H, D)))
    k = bf16(rng.integers(-4, 5, size=(B, S, D)))
    w = (rng.choice([-1.0, 1.0], size=(B, T, H)) *
         np.exp2(rng.integers(-3, 4, size=(B, T, H)))).astype(np.float32)
    return q, k, w


def check_head_sum_and_linearity(lib):
    """Integer inputs (exact): the score is the sum of single-head scores, each equal to the
    H=1 result on that head's slice; linear in w; invariant under head permutation."""
    rng = np.random.default_rng(9)
    B, T, H, D, S = 2, 2, 4, 6, 11
    ep = np.array([11, 7], np.int32)
    q, k, w = _int_case(rng, B, T, H, D, S)
    m = valid_mask(ep, T, S)
    full = oracle.index_scores(q, w, k, ep, 1.0, lib=lib).astype(np.float64)
    parts = np.zeros_like(full)
    for h in range(H):
        wh = np.zeros_like(w)
        wh[:, :, h] = w[:, :, h]
        part = oracle.index_scores(q, wh, k, ep, 1.0, lib=lib)
        single = oracle.index_scores(np.ascontiguousarray(q[:, :, h:h + 1]),
                                     np.ascontiguousarray(w[:, :, h:h + 1]), k, ep, 1.0, lib=lib)
        assert np.array_equal(part[m], single[m])
        parts += part
    assert np.array_equal(full[m], parts[m])
    double = oracle.index_scores(q, 2 * w, k, ep, 1.0, lib=lib).astype(np.float64)
    assert np.array_equal(double[m], 2 * full[m])
    perm = rng.permutation(H)
    permuted = oracle.index_scores(np.ascontiguousarray(q[:, :, perm]),
                                   np.ascontiguousarray(w[:, :, perm]), k, ep, 1.0, lib=lib)
    assert np.array_equal(permuted[m], full[m])


# --- top-k -----------------------------------------------------------------------

def _brute_topk(vals, k):
    """The unique subset of size min(k,n) such that every kept x beats every dropped y:
    vals[x] > vals[y], or equal and x < y.  Found by enumerating all subsets."""
    n = len(vals)
    ke = min(k, n)
    found = []
    for sub in itertools.combinations(range(n), ke):
        s = set(sub)
        ok = all(vals[x] > vals[y] or (vals[x] == vals[y] and x < y)
                 for x in s for y in range(n) if y not in s)
        if ok:
            found.append(list(sub))
    assert len(found) == 1
    return found[0] + [-1] * (k - ke)


def check_topk_bruteforce(lib):
    rng = np.random.default_rng(21)
    S = 8
    pools = [np.array([0.0, -0.0, 1.0, -1.0, 2.0], np.float32),
             np.array([3.0, 3.0, 3.0, 1.5], np.float32)]
    for trial in range(12):
        B = 4
        ep = rng.integers(1, S + 1, size=B).astype(np.int32)
        if trial < 6:
            scores = rng.choice(pools[trial % 2], size=(B, 1, S)).astype(np.float32)
        else:
            scores = rng.standard_normal((B, 1, S)).astype(np.float32)
        for k in range(1, S + 2):
            got = oracle.topk(scores, ep, k, lib=lib)
            for b in range(B):
                assert got[b, 0].tolist() == _brute_topk(scores[b, 0, :ep[b]].tolist(), k)


def check_topk_stable_sort(lib):
    """Against torch's stable descending sort (ties keep the smaller position first)."""
    from sparse_attention_indexer_amd import inputs
    B, T, S = 3, 4, 300
    ep = np.array([300, 250, 17], np.int32)
    for kind in ("normal", "ties", "zeros", "relu", "wide"):
        scores = inputs.make_scores(B, T, S, kind=kind, seed=4).numpy()
        for k in (1, 5, 64, 300):
            got = oracle.topk(scores, ep, k, lib=lib)
            for b in range(B):
                for t in range(T):
                    n = ep[b] - T + t + 1
                    row = torch.from_numpy(scores[b, t, :n].copy())
                    order = torch.sort(row, descending=True, stable=True).indices[:min(k, n)]
                    exp = sorted(order.tolist()) + [-1] * (k - min(k, n))
                    assert got[b, t].tolist() == exp, (kind, k, b, t)


def check_topk_special_cases(lib):
    g = read_golden("short_context.txt")
    n, k = int(g["n"][0]), int(g["k"][0])
    scores = np.random.default_rng(2).standard_normal((1, 1, n)).astype(np.float32)
    got = oracle.topk(scores, np.array([n], np.int32), k, lib=lib)[0, 0]
    assert got[:int(g["kept"][0])].tolist() == list(range(n))
    assert np.all(got[n:] == -1) and got.size - n == int(g["padding"][0])
    eq = np.ones((1, 1, 5000), np.float32)
    got = oracle.topk(eq, np.array([5000], np.int32), 2048, lib=lib)[0, 0]
    assert got.tolist() == list(range(2048))


# --- attention ---------------------------------------------------------------------

def check_mla_golden(lib):
    g = read_golden("mla_worked_example.txt")
    kv = bf16(np.array(g["kv"]).reshape(1, 3, 2))
    pe = bf16(np.array(g["pe"]).reshape(1, 3, 1))
    ep = np.array([3], np.int32)
    for case in ("A", "B"):
        qn = bf16(np.array(g[f"{case}_q_nope"]).reshape(1, 1, 1, 2))
        qp = bf16(np.array(g[f"{case}_q_pe"]).reshape(1, 1, 1, 1))
        o, lse = oracle.mla(qn, qp, kv, pe, ep, 1.0, lib=lib)
        assert np.allclose(o[0, 0, 0], g[f"{case}_dense_o"], rtol=1e-14, atol=0)
        assert np.allclose(lse[0, 0, 0], g[f"{case}_dense_lse"][0], rtol=1e-14, atol=0)
    qn = bf16(np.array(g["A_q_nope"]).reshape(1, 1, 1, 2))
    qp = bf16(np.array(g["A_q_pe"]).reshape(1, 1, 1, 1))
    for idx, key in (([0, 2], "idx02"), ([2, 0], "idx02"), ([1, -1], "idx1")):
        o, lse = oracle.mla(qn, qp, kv, pe, ep, 1.0, indices=np.array(idx, np.int32)
                            .reshape(1, 1, 2), lib=lib)
        assert np.allclose(o[0, 0, 0], g[f"A_{key}_o"], rtol=1e-14, atol=0), (idx, o)
        assert np.allclose(lse[0, 0, 0], g[f"A_{key}_lse"][0], rtol=1e-14, atol=0), (idx, lse)


def _mla_case(rng, B, T, H, Dc, Dr, S):
    return (bf16(rng.standard_normal((B, T, H, Dc))), bf16(rng.standard_normal((B, T, H, Dr))),
            bf16(rng.standard_normal((B, S, Dc))), bf16(rng.standard_normal((B, S, Dr))))


def _sdpa(qn, qp, kv, pe, rows, scale):
    """torch SDPA (float64) of one (b,t) over the given cached rows; returns (o [H,Dc], lse [H])."""
    q = torch.from_numpy(np.concatenate([bf16_val(qn), bf16_val(qp)], -1))       # [H, Dc+Dr]
    kk = torch.from_numpy(np.concatenate([bf16_val(kv[rows]), bf16_val(pe[rows])], -1))
    v = torch.from_numpy(bf16_val(kv[rows]))
    o = torch.nn.functional.scaled_dot_product_attention(q[None], kk[None].expand(1, -1, -1),
                                                         v[None], scale=scale)[0]
    lse = torch.logsumexp(q @ kk.T * scale, dim=-1)
    return o.numpy(), lse.numpy()


def check_mla_sdpa(lib):
    """Dense (causal) and index-masked attention against torch SDPA over the gathered rows."""
    rng = np.random.default_rng(31)
    B, T, H, Dc, Dr, S, k = 2, 2, 3, 8, 4, 20, 6
    ep = np.array([20, 13], np.int32)
    qn, qp, kv, pe = _mla_case(rng, B, T, H, Dc, Dr, S)
    scale = float(np.float32(0.3))
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = ep[b] - T + t + 1
            ke = min(k - t, n)  # leave some empty slots
            idx[b, t, :ke] = np.sort(rng.choice(n, size=ke, replace=False))
    od, lsed = oracle.mla(qn, qp, kv, pe, ep, scale, lib=lib)
    osp, lsesp = oracle.mla(qn, qp, kv, pe, ep, scale, indices=idx, lib=lib)
    for b in range(B):
        for t in range(T):
            n = ep[b] - T + t + 1
            o_ref, l_ref = _sdpa(qn[b, t], qp[b, t], kv[b], pe[b], np.arange(n), scale)
            assert np.allclose(od[b, t], o_ref, rtol=1e-12, atol=1e-12)
            assert np.allclose(lsed[b, t], l_ref, rtol=1e-12, atol=1e-12)
            rows = idx[b, t][idx[b, t] >= 0]
            o_ref, l_ref = _sdpa(qn[b, t], qp[b, t], kv[b], pe[b], rows, scale)
            assert np.allclose(osp[b, t], o_ref, rtol=1e-12, atol=1e-12)
            assert np.allclose(lsesp[b, t], l_ref, rtol=1e-12, atol=1e-12)


def check_mla_closed_forms(lib):
    rng = np.random.default_rng(41)
    B, T, H, Dc, Dr, S, k = 1, 1, 4, 16, 8, 30, 7
    ep = np.array([30], np.int32)
    qn, qp, kv, pe = _mla_case(rng, B, T, H, Dc, Dr, S)
    # one kept row -> that row, exactly
    one = np.full((1, 1, k), -1, np.int32)
    one[0, 0, 0] = 17
    o, lse = oracle.mla(qn, qp, kv, pe, ep, 0.5, indices=one, lib=lib)
    assert np.array_equal(o[0, 0], np.tile(bf16_val(kv[0, 17]), (H, 1)))
    # zero query -> mean of kept rows
    sel = np.sort(rng.choice(30, size=k, replace=False)).astype(np.int32)
    zq = np.zeros_like(qn)
    zp = np.zeros_like(qp)
    o, lse = oracle.mla(zq, zp, kv, pe, ep, 0.5, indices=sel.reshape(1, 1, k), lib=lib)
    mean = bf16_val(kv[0, sel]).mean(0)
    assert np.allclose(o[0, 0], np.tile(mean, (H, 1)), rtol=1e-14, atol=1e-15)
    assert np.allclose(lse[0, 0], np.log(k), rtol=1e-14)
    # every valid position kept == dense, bit for bit; index order does not matter
    allk = np.arange(30, dtype=np.int32).reshape(1, 1, 30)
    od, ld = oracle.mla(qn, qp, kv, pe, ep, 0.5, lib=lib)
    oa, la = oracle.mla(qn, qp, kv, pe, ep, 0.5, indices=allk, lib=lib)
    assert np.array_equal(od, oa) and np.array_equal(ld, la)
    shuffled = np.ascontiguousarray(allk[..., rng.permutation(30)])
    os_, ls_ = oracle.mla(qn, qp, kv, pe, ep, 0.5, indices=shuffled, lib=lib)
    assert np.array_equal(os_, oa) and np.array_equal(ls_, la)


# --- query absorption and output up-projection -------------------------------

def check_proj_identity(lib, mod=oracle):
    """Selector weights: the absorption's first 128 rows per head as the identity
    (q_abs = [q_nope, 0]); the up-projection's rows picking latent dims 256..383."""
    rng = np.random.default_rng(51)
    H = 3
    w = np.zeros((H, 256, 512), np.float32)
    for d in range(128):
        w[:, d, d] = 1.0
        w[:, 128 + d, 256 + d] = 1.0
    wb = bf16(w)
    qn = bf16(rng.standard_normal((2, 1, H, 128)))
    x = bf16(rng.standard_normal((2, 1, H, 512)))
    qa = mod.q_absorb(qn, wb)
    assert np.array_equal(qa[..., :128], bf16_val(qn)) and not qa[..., 128:].any()
    assert np.array_equal(mod.out_proj(x, wb), bf16_val(x)[..., 256:384])


def check_absorbed_equals_mha(lib, mod=oracle):
    """The decode branch's absorbed form (query absorbed into the latent space,
    attention over the latent cache, output up-projected) against the prefill
    branch's MHA form (keys and values up-projected from the latent first, then
    attention): "DeepSeek-V3.2-Exp - Apply sparse mask" and "Keep top-k positions".
    Integer query and key-part weights keep the absorbed query exact in bf16, so
    the two associations agree to fp64 rounding; the MHA side is torch SDPA."""
    rng = np.random.default_rng(53)
    H, Dr, n = 4, 8, 12
    scale = float(np.float32(0.05))  # the oracle takes the scale as an fp32
    qn = bf16(rng.integers(-2, 3, (1, 1, H, 128)))
    wk = rng.integers(-1, 2, (H, 128, 512)) * (rng.random((H, 128, 512)) < 0.5)
    wv = rng.standard_normal((H, 128, 512)) * 0.05
    wb = bf16(np.concatenate([wk, wv], axis=1))
    qp = bf16(rng.standard_normal((1, 1, H, Dr)))
    kv = bf16(rng.standard_normal((1, n, 512)))
    pe = bf16(rng.standard_normal((1, n, Dr)))
    # Absorbed: oracle.q_absorb -> oracle.mla over all n rows -> oracle.out_proj.
    qa = mod.q_absorb(qn, wb)
    assert np.abs(qa).max() <= 256 and np.array_equal(qa, np.round(qa))  # exact in bf16
    x, _ = oracle.mla(bf16(qa), qp, kv, pe, np.array([n], np.int32), scale, lib=lib)
    y = mod.out_proj(x, wb)[0, 0]
    # MHA: per-head keys [k_nope, k_pe] and values from the latent rows.
    W = torch.from_numpy(bf16_val(wb))                       # [H, 256, 512]
    C = torch.from_numpy(bf16_val(kv[0]))                    # [n, 512]
    k_nope = torch.einsum("hdc,tc->htd", W[:, :128], C)      # [H, n, 128]
    v = torch.einsum("hdc,tc->htd", W[:, 128:], C)           # [H, n, 128]
    k_pe = torch.from_numpy(bf16_val(pe[0]))[None].expand(H, -1, -1)
    q = torch.cat([torch.from_numpy(bf16_val(qn[0, 0])), torch.from_numpy(bf16_val(qp[0, 0]))], -1)
    k = torch.cat([k_nope, k_pe], -1)
    o = torch.nn.functional.scaled_dot_product_attention(q[:, None], k, v, scale=scale)[:, 0]
    assert np.allclose(y, o.numpy(), rtol=1e-10, atol=1e-12)


# --- indexer input preparation (rope, rotation, fp8 block quantisation) -------
# These checks take the oracle module as ``mod`` so that planted mistakes in a
# patched copy of its Python source can be run against them.

def _rope_table(S, rng):
    """cos/sin tables [S, 32] of angles theta_i * p with random per-dim frequencies."""
    theta = rng.uniform(0.01, 1.5, 32)
    ang = np.arange(S)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def check_prep_rope_complex(lib, mod=oracle):
    """RoPE in the indexer's non-interleaved ("concatenated") layout as a complex
    multiply: dims i and i+32 of the 64 rope dims are the real and imaginary parts
    of one complex number, turned by that dim's angle (MaxText PR #2933, "What
    this PR does", the indexer RoPE note; Indexer.forward excerpt on "Keep top-k
    positions").  The product is torch's complex multiply by torch.polar."""
    rng = np.random.default_rng(61)
    x = rng.standard_normal((5, 64))
    th = rng.uniform(-np.pi, np.pi, (5, 32))
    z = torch.complex(torch.from_numpy(x[:, :32]), torch.from_numpy(x[:, 32:]))
    z = z * torch.polar(torch.ones(5, 32, dtype=torch.float64), torch.from_numpy(th))
    want = torch.cat([z.real, z.imag], -1).numpy()
    got = mod.rope_halves(x, np.cos(th), np.sin(th))
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def check_prep_hadamard(lib, mod=oracle):
    """rotate_activation as the orthonormal Walsh-Hadamard transform: scipy's
    Sylvester-ordered hadamard(128) over 128**0.5; the unscaled form on the
    identity is that integer matrix; the scaled transform is its own inverse."""
    import scipy.linalg
    H = scipy.linalg.hadamard(128).astype(np.float64)
    rng = np.random.default_rng(62)
    x = rng.standard_normal((3, 4, 128))
    assert np.allclose(mod.hadamard128(x), x @ H.T / np.sqrt(128.0), rtol=1e-12, atol=1e-12)
    assert np.array_equal(mod.hadamard128(np.eye(128), scaled=False), H.T)
    assert np.allclose(mod.hadamard128(mod.hadamard128(x)), x, rtol=1e-12, atol=1e-12)


def check_prep_e4m3_encoding(lib, mod=oracle):
    """The e4m3 encoder against torch's float32 -> float8_e4m3fn cast: random values
    across the whole range, exact ties between neighbouring codes (which go to the
    even code), subnormals, signed zeros and values past 448 (which saturate)."""
    rng = np.random.default_rng(63)
    vals = [rng.uniform(-460, 460, 20000), rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000),
            rng.standard_normal(20000) * 10]
    grid = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    grid = np.unique(grid[np.isfinite(grid)])
    vals.append((grid[1:] + grid[:-1]) / 2)                  # midpoints: ties
    vals.append(grid)
    vals.append([448.0, 449.0, 464.0, -464.0, 0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -11])
    x = np.concatenate([np.asarray(v, np.float64) for v in vals]).astype(np.float32)
    x = x[np.abs(x) <= 464]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mod.e4m3_encode(x), want)
    # Past 464 torch's cast gives NaN; the quantiser never sees such values (its
    # scale puts the block maximum at 448) and the encoder saturates them instead.
    big = np.array([464.5, 1e6, -479.9, -1e30], np.float32)
    assert mod.e4m3_encode(big).tolist() == [0x7E, 0x7E, 0xFE, 0xFE]


def check_prep_act_quant(lib, mod=oracle):
    """Block-128 quantisation: the scale is the block's max |u| over 448 (times the
    post factor), the largest element maps to the top code, every element comes back
    within half an e4m3 step (2^-4 relative for normal codes, 2^-10 absolute below),
    signs are kept, and an all-zero block has scale 0 and zero codes."""
    rng = np.random.default_rng(64)
    u = (rng.standard_normal((6, 128)) * rng.uniform(0.01, 100, (6, 1))).astype(np.float32)
    u[1, 7] = -50 * np.abs(u[1]).max()                       # a block led by a negative value
    u[2, :] = 0.0
    u[3, :] = np.float32(3.0)
    codes, scale = mod.act_quant_128(u, 0.25)
    amax = np.abs(u).max(-1)
    su = (amax / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(scale, (su * np.float32(0.25)).astype(np.float32))
    assert scale[2] == 0 and not codes[2].any()
    dq = pinlib_fp8_values(codes)
    nz = su > 0
    x = u[nz] / su[nz, None].astype(np.float64)
    err = np.abs(dq[nz] - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10) * (1 + 1e-6))
    assert np.all(np.abs(dq[nz]).max(-1) == 448.0)
    assert np.all((codes[nz] >= 0x80) == (u[nz] < 0) | ((u[nz] == 0) & np.signbit(u[nz])))


def pinlib_fp8_values(codes):
    """e4m3fn codes decoded by torch."""
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(
        torch.float8_e4m3fn).double().numpy()


def check_prep_positions(lib, mod=oracle):
    """The T new tokens of a sequence take positions start_pos..end_pos-1 with
    end_pos = start_pos + T (the k_cache slice write and end_pos of the
    Indexer.forward excerpt): with cos = p, sin = 0 the inverse rotation of the
    prepared vectors gives back the rope dims times the token's position and the
    other 64 dims untouched."""
    rng = np.random.default_rng(65)
    S, T = 8, 2
    cos = np.repeat(np.arange(S, dtype=np.float32)[:, None], 32, 1)
    sin = np.zeros((S, 32), np.float32)
    qb = bf16(rng.standard_normal((1, T, 2, 128)))
    kb = bf16(rng.standard_normal((1, T, 128)))
    q, _, k, _, pos = mod.indexer_prep(qb, kb, cos, sin, np.array([5], np.int32), fp8=False)
    assert pos.tolist() == [[3, 4]]
    q0, k0 = bf16_val(qb), bf16_val(kb)
    qi, ki = mod.hadamard128(q), mod.hadamard128(k)
    for t, p in enumerate((3, 4)):
        assert np.allclose(qi[0, t, :, :64], q0[0, t, :, :64] * p, atol=1e-12)
        assert np.allclose(qi[0, t, :, 64:], q0[0, t, :, 64:], atol=1e-12)
        assert np.allclose(ki[0, t, :64], k0[0, t, :64] * p, atol=1e-12)
        assert np.allclose(ki[0, t, 64:], k0[0, t, 64:], atol=1e-12)


def check_prep_relative_position(lib, mod=oracle):
    """With tables of angles theta_i * p, the prepared query of a token at position
    p1 dotted with the prepared key of a token at p2 depends on p1 - p2 only (RoPE's
    relative-position property; the rotation is orthonormal so it keeps dot
    products), and both the query and the key are rotated."""
    rng = np.random.default_rng(66)
    cos, sin = _rope_table(300, rng)
    qb = bf16(rng.standard_normal((1, 1, 3, 128)))
    kb = bf16(rng.standard_normal((1, 1, 128)))

    def dot(p1, p2):
        q, _, _, _, _ = mod.indexer_prep(qb, kb, cos, sin, np.array([p1 + 1], np.int32), fp8=False)
        _, _, k, _, _ = mod.indexer_prep(qb, kb, cos, sin, np.array([p2 + 1], np.int32), fp8=False)
        return q[0, 0] @ k[0, 0]

    # the tables are fp32, so equality holds to their rounding only
    a, b, c = dot(10, 3), dot(207, 200), dot(3, 10)
    assert np.allclose(a, b, rtol=1e-5, atol=1e-5) and not np.allclose(a, c, rtol=1e-3)
    assert np.allclose(dot(0, 0), bf16_val(qb)[0, 0] @ bf16_val(kb)[0, 0], rtol=1e-12)


def check_prep_quantised_pipeline(lib, mod=oracle):
    """End to end with the identity rotation of RoPE (cos 1, sin 0): the prepared
    fp8 codes times their scales give scipy's hadamard(128) @ x / 128**0.5 within
    half an e4m3 step of the block scale, for the query heads and the key."""
    import scipy.linalg
    rng = np.random.default_rng(67)
    H = scipy.linalg.hadamard(128).astype(np.float64) / np.sqrt(128.0)
    cos, sin = np.ones((4, 32), np.float32), np.zeros((4, 32), np.float32)
    qb = bf16(rng.standard_normal((2, 1, 5, 128)))
    kb = bf16(rng.standard_normal((2, 1, 128)))
    qc, qs, kc, ks, _ = mod.indexer_prep(qb, kb, cos, sin, np.array([1, 4], np.int32))
    for codes, sc, x in ((qc, qs, bf16_val(qb)), (kc, ks, bf16_val(kb))):
        want = x @ H.T
        got = pinlib_fp8_values(codes) * sc[..., None].astype(np.float64)
        step = np.abs(want).max(-1, keepdims=True) * 2.0 ** -4
        assert np.all(np.abs(got - want) <= step * (1 + 1e-5))
        assert np.allclose(sc, np.abs(want).max(-1) / 448.0, rtol=1e-6)


# --- MHA-form prefill attention ----------------------------------------------

def _mha_case(rng, B, T, H, k):
    q = bf16(rng.standard_normal((B, T, H, 192)))
    kn = bf16(rng.standard_normal((B, T, H, 128)))
    kp = bf16(rng.standard_normal((B, T, 64)))
    v = bf16(rng.standard_normal((B, T, H, 128)))
    idx = rng.integers(-2, T + 2, (B, T, k)).astype(np.int32)   # some out of range, duplicates
    return q, kn, kp, v, idx


def check_mha_sdpa(lib, mod=oracle):
    """Against torch scaled_dot_product_attention in float64 with a boolean mask
    that is true at the selected positions (a set) that are also causal."""
    rng = np.random.default_rng(81)
    B, T, H, k = 2, 9, 3, 5
    q, kn, kp, v, idx = _mha_case(rng, B, T, H, k)
    scale = 0.07
    out, lse = mod.sparse_mha_prefill(q, kn, kp, v, idx, scale)
    for b in range(B):
        mask = torch.zeros(T, T, dtype=torch.bool)
        for s in range(T):
            for t in idx[b, s]:
                if 0 <= t <= s:
                    mask[s, t] = True
        qq = torch.from_numpy(bf16_val(q[b])).permute(1, 0, 2)          # [H,T,192]
        kk = torch.cat([torch.from_numpy(bf16_val(kn[b])),
                        torch.from_numpy(bf16_val(kp[b]))[:, None, :].expand(T, H, 64)], -1)
        kk = kk.permute(1, 0, 2)
        vv = torch.from_numpy(bf16_val(v[b])).permute(1, 0, 2)
        for s in range(T):
            if not mask[s].any():
                assert not out[b, s].any() and np.all(np.isneginf(lse[b, s]))
                continue
            o = torch.nn.functional.scaled_dot_product_attention(
                qq[:, s:s + 1], kk, vv, attn_mask=mask[s:s + 1], scale=scale)[:, 0]
            assert np.allclose(out[b, s], o.numpy(), rtol=1e-10, atol=1e-12)
            z = torch.einsum("hd,htd->ht", qq[:, s], kk) * scale
            ref_lse = torch.logsumexp(z.masked_fill(~mask[s], float("-inf")), -1)
            assert np.allclose(lse[b, s], ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def check_mha_closed_forms(lib, mod=oracle):
    """One selected causal position returns its value row for every head; a zero
    query weighs the selected causal positions equally (their mean); a query
    whose selections all lie in its future gets 0 and lse -inf."""
    rng = np.random.default_rng(82)
    B, T, H = 1, 6, 2
    q, kn, kp, v, _ = _mha_case(rng, B, T, H, 1)
    idx = np.full((B, T, 3), -1, np.int32)
    idx[0, 4, :] = [2, 2, 5]           # position 2 twice, position 5 in the future
    idx[0, 3, :] = [4, 5, -1]          # only future positions
    out, lse = mod.sparse_mha_prefill(q, kn, kp, v, idx, 0.1)
    assert np.array_equal(out[0, 4], bf16_val(v)[0, 2])
    assert not out[0, 3].any() and np.all(np.isneginf(lse[0, 3]))
    q0 = np.zeros_like(q)
    idx[0, 5, :] = [0, 3, 5]
    out0, lse0 = mod.sparse_mha_prefill(q0, kn, kp, v, idx, 0.1)
    assert np.allclose(out0[0, 5], bf16_val(v)[0, [0, 3, 5]].mean(0), rtol=1e-12, atol=1e-12)
    assert np.allclose(lse0[0, 5], np.log(3.0))


def check_mha_equals_absorbed(lib, mod=oracle):
    """The prefill branch's MHA form against the decode branch's absorbed form on
    the same latent cache ("Keep top-k positions" and "Apply sparse mask"): with
    k_nope = W_k c and v = W_v c per head, MHA attention over the selection equals
    absorbing the query (oracle.q_absorb), attending over the latent rows
    (oracle.mla with the same index lists) and up-projecting (oracle.out_proj).
    Small integers keep every bf16 operand exact on both sides."""
    rng = np.random.default_rng(83)
    B, T, H, k = 1, 7, 128, 4
    scale = float(np.float32(0.03))
    c = rng.integers(-2, 3, (B, T, 512)).astype(np.float64)      # latent rows
    wk = rng.integers(-1, 2, (H, 128, 512)) * (rng.random((H, 128, 512)) < 0.05)
    wv = rng.integers(-1, 2, (H, 128, 512)) * (rng.random((H, 128, 512)) < 0.05)
    qn = rng.integers(-2, 3, (B, T, H, 128))
    qp = rng.integers(-2, 3, (B, T, H, 64))
    kp = rng.integers(-2, 3, (B, T, 64))
    k_nope = np.einsum("hdc,btc->bthd", wk, c)
    v = np.einsum("hdc,btc->bthd", wv, c)
    assert np.abs(k_nope).max() <= 256 and np.abs(v).max() <= 256  # exact in bf16
    idx = np.full((1, T, k), -1, np.int32)          # causal selections (the decode form's contract)
    for t in range(T):
        sel = rng.permutation(t + 1)[:k]
        idx[0, t, :sel.size] = np.sort(sel)
    out, lse = mod.sparse_mha_prefill(bf16(np.concatenate([qn, qp], -1)), bf16(k_nope), bf16(kp),
                                      bf16(v), idx, scale)
    wb = bf16(np.concatenate([wk, wv], 1))
    qa = oracle.q_absorb(bf16(qn), wb)
    assert np.abs(qa).max() <= 256 and np.array_equal(qa, np.round(qa))
    x, lse_a = oracle.mla(bf16(qa), bf16(qp), bf16(c), bf16(kp), np.array([T], np.int32), scale,
                          indices=idx, lib=lib)
    y = np.einsum("bthc,hdc->bthd", x, wv)          # the up-projection, on the fp64 latent output
    assert np.allclose(out, y, rtol=1e-9, atol=1e-9)
    assert np.allclose(lse, lse_a, rtol=1e-9, atol=1e-9)


ALL_CHECKS = [
    check_indexer_golden, check_fp8_decoding, check_bf16_decoding, check_single_head_matmul,
    check_fp8_single_head_matmul, check_head_sum_and_linearity, check_topk_bruteforce,
    check_topk_stable_sort, check_topk_special_cases, check_mla_golden, check_mla_sdpa,
    check_mla_closed_forms, check_proj_identity, check_absorbed_equals_mha,
]
PREP_CHECKS = [
    check_prep_rope_complex, check_prep_hadamard, check_prep_e4m3_encoding, check_prep_act_quant,
    check_prep_positions, check_prep_relative_position, check_prep_quantised_pipeline,
]
MHA_CHECKS = [check_mha_sdpa, check_mha_closed_forms, check_mha_equals_absorbed]
PROJ_CHECKS = [check_proj_identity, check_absorbed_equals_mha]
ALL_CHECKS += PREP_CHECKS + MHA_CHECKS
