"""Parity of the HIP path (through the C ABI) with the CPU oracle on the same seeded inputs.

Bars:
* top-k indices: bit-exact (integer work) - on synthetic score rows fed to both
  sides, and end to end wherever the scores themselves are exact (integer-valued
  indexer inputs, where every fp32 partial sum is exact);
* indexer scores: per query row, max |I_gpu - I_ref| / max |I_ref| <= 2e-3 (bf16)
  or 1e-2 (fp8), I_ref the oracle's score of the same stored inputs;
* attention output: max |o_gpu - o_ref| <= 2e-2 over all elements (bf16 output);
  lse within 1e-3 absolute.
Large workloads are checked on sampled rows the oracle computes one by one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_indexer_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCORE_TOL = {"bf16": 2e-3, "fp8": 1e-2}
OUT_TOL = 2e-2
LSE_TOL = 1e-3


def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_indexer_amd as m
    m.lib()
    return m


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def np_case(case, rows_b=None):
    """Host copies (oracle conventions); optionally only the sequences in rows_b."""
    out = {}
    for name in ("q", "w", "k_cache", "q_scale", "k_scale", "end_pos", "q_nope", "q_pe",
                 "kv_cache", "pe_cache"):
        v = getattr(case, name)
        if v is None:
            out[name] = None
            continue
        if rows_b is not None:
            v = v[rows_b]
        out[name] = inputs.to_numpy(v)
    return out


def oracle_scores(case, h, rows=None):
    return oracle.index_scores(h["q"], h["w"], h["k_cache"], h["end_pos"], case.scale,
                               q_scale=h["q_scale"], k_scale=h["k_scale"], rows=rows)


def valid_mask(end_pos, T, S_max):
    ep = np.asarray(end_pos).reshape(-1, 1, 1)
    t = np.arange(T).reshape(1, -1, 1)
    s = np.arange(S_max).reshape(1, 1, -1)
    return s <= ep - T + t


def assert_scores_close(gpu, ref, end_pos, T, tol, rows=None):
    B, _, S = ref.shape
    m = valid_mask(end_pos, T, S)
    for b in range(B):
        for t in range(T):
            if rows is not None and b * T + t not in rows:
                continue
            r = ref[b, t][m[b, t]].astype(np.float64)
            g = gpu[b, t][m[b, t]].astype(np.float64)
            denom = max(np.abs(r).max(), 1e-30)
            err = np.abs(g - r).max() / denom
            assert err <= tol, f"row ({b},{t}): relative score error {err:.3e} > {tol}"


def assert_out_close(out_gpu, lse_gpu, o_ref, lse_ref, rows=None):
    og = out_gpu.float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.cpu().numpy().astype(np.float64)
    B, T = og.shape[:2]
    for b in range(B):
        for t in range(T):
            if rows is not None and b * T + t not in rows:
                continue
            err = np.abs(og[b, t] - o_ref[b, t]).max()
            assert err <= OUT_TOL, f"row ({b},{t}): max |out error| {err:.3e}"
            same = lg[b, t] == lse_ref[b, t]  # also -inf on both sides (nothing kept)
            with np.errstate(invalid="ignore"):
                lerr = np.where(same, 0.0, np.abs(lg[b, t] - lse_ref[b, t])).max()
            assert lerr <= LSE_TOL, f"row ({b},{t}): max |lse error| {lerr:.3e}"


def check_topk_invariants(idx, end_pos, T, k):
    B = idx.shape[0]
    for b in range(B):
        for t in range(T):
            n = int(end_pos[b]) - T + t + 1
            ke = min(k, n)
            row = idx[b, t]
            sel = row[:ke]
            assert np.all(row[ke:] == -1)
            assert np.all(sel >= 0) and np.all(sel < n)
            assert np.all(np.diff(sel) > 0)


# --- indexer --------------------------------------------------------------------

@pytest.mark.parametrize("variant", ["base", "dup", "equal", "short", "fp8int"])
def test_indexer_integer_inputs_exact(variant):
    m = dsa()
    banner(f"indexer tiny_decode {variant}")
    case = inputs.tiny_decode(variant).to(DEV)
    gpu = m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale,
                         q_scale=case.q_scale, k_scale=case.k_scale)
    h = np_case(case)
    ref = oracle_scores(case, h)
    msk = valid_mask(h["end_pos"], case.T, case.S_max)
    g = gpu.cpu().numpy()
    assert np.array_equal(g[msk], ref[msk])  # -0 == +0 numerically


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_indexer_ragged_batch(dtype):
    """Several sequences, T>1, causal rows, lengths not multiples of any tile."""
    m = dsa()
    banner(f"indexer ragged {dtype}")
    case = inputs.make_case("ragged", 3, 3, [3001, 17, 2050], 3001, dtype=dtype, seed=7,
                            device=DEV)
    gpu = m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale,
                         q_scale=case.q_scale, k_scale=case.k_scale, max_end_pos=3001)
    h = np_case(case)
    ref = oracle_scores(case, h)
    assert_scores_close(gpu.cpu().numpy(), ref, h["end_pos"], case.T, SCORE_TOL[dtype])


def test_indexer_integer_prefill_exact():
    m = dsa()
    banner("indexer integer prefill T=70 start_pos=200")
    case = inputs.make_case("prefill_int", 2, 70, [270, 70], 300, index_dist="int", seed=8,
                            device=DEV)
    gpu = m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale)
    h = np_case(case)
    ref = oracle_scores(case, h)
    msk = valid_mask(h["end_pos"], case.T, case.S_max)
    assert np.array_equal(gpu.cpu().numpy()[msk], ref[msk])


@pytest.mark.parametrize("dtype,T,ep0,S", [("bf16", 37, 2300, 2300), ("fp8", 37, 2300, 2300),
                                           ("bf16", 8, 4100, 4200), ("fp8", 15, 2049, 2100)])
def test_indexer_prefill_ragged(dtype, T, ep0, S):
    """The prefill form (8 queries per workgroup, 64-key LDS tiles, 2048-key
    chunks): T not a multiple of 8 (or exactly the smallest T that takes the
    form), a sequence whose queries start deep in its cache (ranges ending
    just past a chunk), and one starting at position 0."""
    m = dsa()
    banner(f"indexer prefill ragged {dtype} T={T} end_pos={ep0}")
    case = inputs.make_case("prefill_ragged", 2, T, [ep0, T], S, dtype=dtype, seed=11,
                            device=DEV)
    gpu = m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale,
                         q_scale=case.q_scale, k_scale=case.k_scale, max_end_pos=ep0)
    h = np_case(case)
    ref = oracle_scores(case, h)
    assert_scores_close(gpu.cpu().numpy(), ref, h["end_pos"], case.T, SCORE_TOL[dtype])


def test_indexer_prefill_untouched_past_bound():
    m = dsa()
    banner("indexer prefill poison past bound")
    case = inputs.make_case("poison_pf", 1, 40, [1500], 1600, seed=12, device=DEV)
    out = torch.full((1, 40, 1600), float("nan"), device=DEV)
    m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale, out=out)
    msk = valid_mask(case.end_pos.cpu().numpy(), 40, 1600)
    g = out.cpu().numpy()
    assert not np.isnan(g[msk]).any()
    assert np.isnan(g[~msk]).all()


def test_indexer_decode_32k_full_row():
    m = dsa()
    banner("indexer decode_32k full row")
    case = inputs.decode_32k(device=DEV)
    gpu = m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale)
    h = np_case(case)
    ref = oracle_scores(case, h)
    assert_scores_close(gpu.cpu().numpy(), ref, h["end_pos"], 1, SCORE_TOL["bf16"])


@pytest.mark.parametrize("dtype,dist", [("bf16", "int"), ("fp8", "normal")])
def test_indexer_streaming_form(dtype, dist):
    """Long decode rows (4 x 131072 cached positions: at least 4 key tiles per wave) take
    the streaming form (per-wave LDS ring of key tiles, 4 or 2 in flight): ragged lengths
    ending inside a workgroup, a tile and a 16-key group; integer bf16 inputs exactly,
    fp8 within tolerance; entries past each bound untouched."""
    m = dsa()
    banner(f"indexer streaming form {dtype} {dist}")
    S = 131072
    ep = [S, 100003, 5000, 4097]
    case = inputs.make_case("stream", 4, 1, ep, S, dtype=dtype, index_dist=dist, seed=19,
                            device=DEV)
    out = torch.full((4, 1, S), float("nan"), device=DEV)
    m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale,
                   q_scale=case.q_scale, k_scale=case.k_scale, max_end_pos=S, out=out)
    g = out.cpu().numpy()
    h = np_case(case)
    msk = valid_mask(h["end_pos"], 1, S)
    assert not np.isnan(g[msk]).any() and np.isnan(g[~msk]).all()
    ref = oracle_scores(case, h)
    if dist == "int":
        assert np.array_equal(g[msk], ref[msk])
    else:
        assert_scores_close(g, ref, h["end_pos"], 1, SCORE_TOL[dtype])


def test_untouched_past_bound():
    """Entries past each causal bound are left as they were (poisoned with NaN here)."""
    m = dsa()
    banner("indexer poison past bound")
    case = inputs.make_case("poison", 2, 2, [1000, 37], 1100, seed=9, device=DEV)
    out = torch.full((2, 2, 1100), float("nan"), device=DEV)
    m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale, out=out)
    msk = valid_mask(case.end_pos.cpu().numpy(), 2, 1100)
    g = out.cpu().numpy()
    assert not np.isnan(g[msk]).any()
    assert np.isnan(g[~msk]).all()


# --- top-k ------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["normal", "ties", "equal", "zeros", "relu", "wide"])
@pytest.mark.parametrize("S", [2047, 2048, 2049, 4095, 4097, 32768, 32769, 70001])
def test_topk_exact(kind, S):
    m = dsa()
    banner(f"topk {kind} S={S}")
    B, T, k = 2, 2, 2048
    ep = np.array([S, max(2, S // 3)], np.int32)
    scores = inputs.make_scores(B, T, S, kind=kind, seed=S % 97, device=DEV)
    end_pos = torch.from_numpy(ep).to(DEV)
    out = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    m.topk(scores, end_pos, k, max_end_pos=int(ep.max()), out=out)
    ref = oracle.topk(scores.cpu().numpy(), ep, k)
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("k", [1, 7, 64, 1000, 2048])
def test_topk_small_k_and_causal_rows(k):
    m = dsa()
    banner(f"topk causal rows k={k}")
    B, T, S = 2, 40, 3000
    ep = np.array([3000, 1500], np.int32)
    scores = inputs.make_scores(B, T, S, kind="ties", seed=k, device=DEV)
    out = m.topk(scores, torch.from_numpy(ep).to(DEV), k, max_end_pos=3000)
    ref = oracle.topk(scores.cpu().numpy(), ep, k)
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("kind", ["normal", "ties", "relu", "equal"])
@pytest.mark.parametrize("S", [70001, 140001])
def test_topk_many_long_rows(kind, S):
    """Twenty rows: sixteen long ones and four of 8200..16384 positions.  Up to 131072
    positions the cut path (8192-position regions) takes them; the short rows fill a
    region past the share its own threads stage, and "equal" overflows every region
    (the pick then selects the row from the scores).  Longer rows take the split path
    (lists appended under one device-scope atomic per workgroup, then one finishing
    workgroup per row)."""
    m = dsa()
    banner(f"topk many long rows {kind} S={S}")
    T, k = 1, 2048
    ep = np.array([S - 997 * i for i in range(16)] + [8200, 12000, 16384, 9000], np.int32)
    B = len(ep)
    scores = inputs.make_scores(B, T, S, kind=kind, seed=31, device=DEV)
    out = m.topk(scores, torch.from_numpy(ep).to(DEV), k, max_end_pos=S)
    ref = oracle.topk(scores.cpu().numpy(), ep, k)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_topk_longest_rows():
    m = dsa()
    banner("topk 131072-long rows")
    B, T, S, k = 3, 1, 131072, 2048
    ep = np.array([131072, 100000, 8192], np.int32)
    scores = inputs.make_scores(B, T, S, kind="normal", seed=3, device=DEV)
    out = m.topk(scores, torch.from_numpy(ep).to(DEV), k, max_end_pos=S)
    ref = oracle.topk(scores.cpu().numpy(), ep, k)
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("max_end_pos", [9000, 4000])
def test_topk_row_longer_than_promised(max_end_pos):
    """A row longer than max_end_pos (a broken promise the host cannot see) is still
    selected exactly: by the finishing launch when rows are split over several
    workgroups (9000: 3 per row), by the single launch otherwise (4000)."""
    m = dsa()
    banner(f"topk row longer than max_end_pos={max_end_pos}")
    B, T, S, k = 2, 1, 40000, 2048
    ep = np.array([40000, 3000], np.int32)
    scores = inputs.make_scores(B, T, S, kind="normal", seed=23, device=DEV)
    out = m.topk(scores, torch.from_numpy(ep).to(DEV), k, max_end_pos=max_end_pos)
    ref = oracle.topk(scores.cpu().numpy(), ep, k)
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("B,T,S,kind", [(1, 1100, 3000, "ties"), (2, 520, 33000, "normal"),
                                        (1, 1100, 8192, "equal"), (1, 1030, 8192, "relu"),
                                        (2, 520, 8193, "zeros")])
def test_topk_many_rows(B, T, S, kind):
    """More than 1024 query rows: one workgroup per row (rows of up to 32768
    positions held in registers, longer ones chunk by chunk; with S_max <= 8192
    the lighter form whose list always holds k keys - an all-equal row puts
    every position in it)."""
    m = dsa()
    banner(f"topk many rows B={B} T={T} S={S}")
    k = 2048
    ep = np.array([S] + [S - 7] * (B - 1), np.int32)
    scores = inputs.make_scores(B, T, S, kind=kind, seed=T, device=DEV)
    out = m.topk(scores, torch.from_numpy(ep).to(DEV), k, max_end_pos=S)
    ref = oracle.topk(scores.cpu().numpy(), ep, k)
    assert np.array_equal(out.cpu().numpy(), ref)


@pytest.mark.parametrize("seed", list(range(12)))
def test_topk_random_shapes(seed):
    """dsa_topk alone on seeded shapes across its paths: row counts on either side of
    1024 (the candidate paths against one workgroup per row), lengths on either side
    of 4096, 8192, 32768 and 131072, ragged end_pos, any k up to 2048 and every score
    kind; bit-exact against the oracle's full sort."""
    m = dsa()
    rng = np.random.default_rng(3000 + seed)
    rows = int(rng.choice([1, 3, 17, 700, 1024, 1025, 1500]))
    T = int(rng.choice([1, 2, 5])) if rows > 1 else 1
    B = max(1, rows // T)
    S = int(rng.choice([1000, 4096, 4097, 8192, 8193, 32768, 32769, 131072, 131073]))
    if B * T > 64:
        S = min(S, 33000)  # keeps the oracle's sort within seconds
    k = int(rng.choice([1, 7, 300, 2047, 2048]))
    kind = str(rng.choice(["normal", "ties", "equal", "zeros", "relu", "wide"]))
    ep = rng.integers(T, S + 1, size=B).astype(np.int32)
    ep[int(rng.integers(0, B))] = S
    banner(f"topk random seed={seed}: B={B} T={T} S={S} k={k} kind={kind}")
    scores = inputs.make_scores(B, T, S, kind=kind, seed=4000 + seed, device=DEV)
    out = m.topk(scores, torch.from_numpy(ep).to(DEV), k, max_end_pos=S)
    ref = oracle.topk(scores.cpu().numpy(), ep, k)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_topk_rows_around_bitmap_limit():
    """Rows up to 262144 positions are selected through LDS bitmaps; longer
    ones take the general path.  Both sides of that limit, and a row whose
    threshold bin is too crowded for the candidate list (a narrow score
    range), must match the oracle."""
    m = dsa()
    banner("topk rows of 262144 / 262145 / 300000 positions")
    B, T, S, k = 4, 1, 300000, 2048
    ep = np.array([262144, 262145, 300000, 50000], np.int32)
    scores = inputs.make_scores(B, T, S, kind="normal", seed=8, device=DEV)
    scores[3] = 1000.0 + scores[3] * 1e-3  # ~all of row 3 in one histogram bin
    out = m.topk(scores, torch.from_numpy(ep).to(DEV), k, max_end_pos=S)
    ref = oracle.topk(scores.cpu().numpy(), ep, k)
    assert np.array_equal(out.cpu().numpy(), ref)


# --- attention --------------------------------------------------------------------

def _mla_inputs(B, T, S, ep, seed):
    case = inputs.make_case("mla", B, T, ep, S, seed=seed, device=DEV)
    return case


@pytest.mark.parametrize("fill", ["random", "first", "last"])
def test_sparse_mla_vs_oracle(fill):
    m = dsa()
    banner(f"sparse_mla fill={fill}")
    B, T, S, k = 2, 2, 5000, 2048
    ep = [5000, 1500]  # second sequence has fewer than k valid positions
    case = _mla_inputs(B, T, S, ep, 11)
    idx = inputs.make_indices(B, T, ep, k, seed=5, fill=fill, device=DEV)
    out, lse = m.sparse_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, idx,
                            case.softmax_scale)
    h = np_case(case)
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale, indices=idx.cpu().numpy())
    assert_out_close(out, lse, o_ref, lse_ref)


@pytest.mark.parametrize("k", [1, 33, 100, 257])
def test_sparse_mla_ragged_k(k):
    m = dsa()
    banner(f"sparse_mla k={k}")
    B, T, S = 1, 3, 700
    case = _mla_inputs(B, T, S, [700], 12)
    idx = inputs.make_indices(B, T, [700], k, seed=k, device=DEV)
    out, lse = m.sparse_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, idx,
                            case.softmax_scale)
    h = np_case(case)
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale, indices=idx.cpu().numpy())
    assert_out_close(out, lse, o_ref, lse_ref)


@pytest.mark.parametrize("k", [257, 1024])
def test_sparse_mla_one_row_few_splits(k):
    """One query row whose list splits into a handful of parts (the few-row merge
    with fewer than 32 parts), output and lse against the oracle."""
    m = dsa()
    banner(f"sparse_mla one row k={k}")
    case = _mla_inputs(1, 1, 3000, [3000], 31)
    idx = inputs.make_indices(1, 1, [3000], k, seed=k, device=DEV)
    out, lse = m.sparse_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, idx,
                            case.softmax_scale)
    h = np_case(case)
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale, indices=idx.cpu().numpy())
    assert_out_close(out, lse, o_ref, lse_ref)


def test_dense_mla_one_row_short():
    """Dense attention of one row over 1000 positions (few splits), output and lse."""
    m = dsa()
    banner("dense_mla one row S=1000")
    case = _mla_inputs(1, 1, 1000, [1000], 32)
    out, lse = m.dense_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, case.end_pos,
                           case.softmax_scale, max_end_pos=1000)
    h = np_case(case)
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale)
    assert_out_close(out, lse, o_ref, lse_ref)


def test_sparse_mla_single_row_and_empty():
    """One kept row returns that row exactly; a row with no entry gives 0 and lse=-inf."""
    m = dsa()
    banner("sparse_mla single row / empty")
    B, T, S, k = 1, 2, 300, 64
    case = _mla_inputs(B, T, S, [300], 13)
    idx = torch.full((B, T, k), -1, dtype=torch.int32)
    idx[0, 0, 0] = 123
    idx = idx.to(DEV)
    out, lse = m.sparse_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, idx,
                            case.softmax_scale)
    row = case.kv_cache[0, 123].float()
    assert torch.equal(out[0, 0].float(), row.expand(128, -1))
    assert torch.equal(out[0, 1].float(), torch.zeros(128, 512, device=DEV))
    assert torch.isinf(lse[0, 1]).all() and (lse[0, 1] < 0).all()


@pytest.mark.parametrize("B,T,S,ep,k,fill", [
    (2, 2, 5000, [5000, 2500], 2048, "random"),    # 4 rows: the tile form, 32 splits
    (2, 8, 5000, [5000, 2500], 2048, "random"),    # 16 rows: the 8-wave form, 16 splits
    (5, 1, 9000, [9000, 4100, 2048, 700, 9000], 2048, "first"),  # 5 rows: 8-wave, 32 splits
    (2, 60, 5000, [5000, 1500], 2048, "random"),   # 120 rows: the many-row form, 2 splits
    (1, 300, 3000, [3000], 2048, "random"),        # 300 rows: one split, direct output
    (4, 9, 400, [400, 30, 200, 9], 100, "last"),   # splits of 64 + 36, short rows, ragged
])
def test_sparse_mla_many_rows(B, T, S, ep, k, fill):
    """Batches with more than 4 query rows take the 8-wave form (scores per
    16 heads, values per 64 latent dims, probabilities exchanged through LDS),
    up to 4 rows the tile form (32 heads, one 64-row tile per workgroup);
    checked on sampled rows, including the first and last."""
    m = dsa()
    banner(f"sparse_mla many rows B={B} T={T} k={k}")
    case = _mla_inputs(B, T, S, ep, 15)
    idx = inputs.make_indices(B, T, ep, k, seed=9, fill=fill, device=DEV)
    out, lse = m.sparse_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, idx,
                            case.softmax_scale)
    h = np_case(case)
    n = B * T
    rows = sorted({0, 1, T - 1, T, n // 2, n - 2, n - 1} & set(range(n)))
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale, indices=idx.cpu().numpy(),
                                rows=rows)
    assert_out_close(out, lse, o_ref, lse_ref, rows=rows)


@pytest.mark.parametrize("seed", list(range(12)))
def test_mla_random_shapes(seed):
    """dsa_sparse_mla and dsa_dense_mla alone on seeded shapes across their plans:
    query rows on either side of the tile form's 4 (sparse) and 16 (dense) rows,
    list lengths k that end inside a 64-row tile or a split, selections that are
    random, leading or trailing, some of them shuffled and with empty (-1) or
    out-of-range slots; sampled rows against the oracle."""
    m = dsa()
    rng = np.random.default_rng(5000 + seed)
    T = int(rng.choice([1, 1, 2, 3, 5, 9]))
    B = int(rng.integers(1, (6 if T == 1 else 3) + 1))
    S = int(rng.choice([700, 2048, 2500, 5000, 20000]))
    k = int(rng.choice([64, 100, 1000, 2047, 2048]))
    fill = str(rng.choice(["random", "first", "last"]))
    ep = rng.integers(T, S + 1, size=B)
    ep[int(rng.integers(0, B))] = S
    ep = [int(x) for x in ep]
    banner(f"mla random seed={seed}: B={B} T={T} S={S} k={k} fill={fill} end_pos={ep}")
    case = _mla_inputs(B, T, S, ep, 30 + seed)
    idx = inputs.make_indices(B, T, ep, k, seed=40 + seed, fill=fill)
    ref_idx = idx.clone()
    if seed % 3 == 0:  # any order; an empty slot of each row holding S_max + 5 instead of -1
        for b in range(B):
            for t in range(T):
                perm = torch.from_numpy(rng.permutation(k))
                idx[b, t] = idx[b, t, perm]
        ref_idx = idx.clone()  # the selection the library must use: out-of-range = empty
        empty = (idx == -1).nonzero()
        if len(empty):
            idx[tuple(empty[0].tolist())] = S + 5
    idx = idx.to(DEV)
    out, lse = m.sparse_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, idx,
                            case.softmax_scale)
    dout, dlse = m.dense_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, case.end_pos,
                             case.softmax_scale, max_end_pos=S)
    h = np_case(case)
    n = B * T
    rows = sorted({0, n // 2, n - 1})
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale, indices=ref_idx.numpy(),
                                rows=rows)
    assert_out_close(out, lse, o_ref, lse_ref, rows=rows)
    d_ref, dlse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                 h["end_pos"], case.softmax_scale, rows=rows)
    assert_out_close(dout, dlse, d_ref, dlse_ref, rows=rows)


def test_dense_mla_many_rows():
    """Dense attention for 40 query rows over 3000 positions: the many-row form
    with splits of 512 positions (the last one partial)."""
    m = dsa()
    banner("dense_mla many rows")
    B, T, S = 1, 40, 3000
    case = _mla_inputs(B, T, S, [S], 16)
    out, lse = m.dense_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, case.end_pos,
                           case.softmax_scale, max_end_pos=S)
    h = np_case(case)
    rows = [0, 1, 17, 38, 39]
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale, rows=rows)
    assert_out_close(out, lse, o_ref, lse_ref, rows=rows)


@pytest.mark.parametrize("S,ep,T", [(3000, [3000, 1200], 1), (20000, [20000, 9000], 1),
                                    (4000, [4000, 2100], 3)])
def test_dense_mla_vs_oracle(S, ep, T):
    """Two rows and six rows in the tile form (64-position splits), ragged at the end."""
    m = dsa()
    banner(f"dense_mla S={S} T={T}")
    B = 2
    case = _mla_inputs(B, T, S, ep, 14)
    out, lse = m.dense_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, case.end_pos,
                           case.softmax_scale, max_end_pos=max(ep))
    h = np_case(case)
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale)
    assert_out_close(out, lse, o_ref, lse_ref)


# --- whole path ----------------------------------------------------------------------

def _forward_and_oracle(case, rows=None, rows_b=None):
    """Run dsa_forward; oracle scores -> oracle top-k -> oracle attention on the same inputs."""
    m = dsa()
    B, T, k = case.B, case.T, case.topk
    topk_out = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    out, lse, _ = m.forward_case(case, topk_out=topk_out)
    torch.cuda.synchronize()
    h = np_case(case)
    ref_s = oracle_scores(case, h, rows=rows)
    ref_idx = oracle.topk(np.nan_to_num(ref_s, nan=0.0), h["end_pos"], k, rows=rows)
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale, indices=ref_idx, rows=rows)
    return out, lse, topk_out.cpu().numpy(), ref_s, ref_idx, o_ref, lse_ref, h


@pytest.mark.parametrize("variant", ["base", "dup", "equal", "short", "fp8int"])
def test_forward_tiny_exact_indices(variant):
    banner(f"forward tiny_decode {variant}")
    case = inputs.tiny_decode(variant).to(DEV)
    out, lse, idx, ref_s, ref_idx, o_ref, lse_ref, h = _forward_and_oracle(case)
    assert np.array_equal(idx, ref_idx)
    assert_out_close(out, lse, o_ref, lse_ref)


def test_forward_prefill_integer_exact():
    banner("forward integer prefill B=2 T=96")
    case = inputs.make_case("prefill_int", 2, 96, [2500, 96], 2500, index_dist="int", seed=15,
                            device=DEV)
    out, lse, idx, ref_s, ref_idx, o_ref, lse_ref, h = _forward_and_oracle(case)
    assert np.array_equal(idx, ref_idx)
    assert_out_close(out, lse, o_ref, lse_ref)


def test_forward_decode_32k_integer_exact():
    """The 32K decode shape with integer-valued indexer inputs: indices exact end to end."""
    banner("forward decode 32k integer")
    case = inputs.make_case("d32k_int", 1, 1, [32768], 32768, index_dist="int", seed=16,
                            device=DEV)
    out, lse, idx, ref_s, ref_idx, o_ref, lse_ref, h = _forward_and_oracle(case)
    assert np.array_equal(idx, ref_idx)
    assert_out_close(out, lse, o_ref, lse_ref)


def _gpu_scores_like_forward(m, case):
    """The indexer scores dsa_forward computes internally: the same entry point with
    the same arguments (so the same kernel and launch shape) writes them out."""
    return m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale,
                          q_scale=case.q_scale, k_scale=case.k_scale,
                          max_end_pos=case.max_end_pos)


def _check_forward_rows(case, seqs):
    """dsa_forward on the whole batch; for each sampled sequence b (T = 1): the
    GPU's scores within tolerance of the oracle's, the selection bit-exact
    against the oracle's top-k of the GPU's own scores, and the attention
    within tolerance of the oracle's attention over the GPU's selection."""
    m = dsa()
    B, k = case.B, case.topk
    assert case.T == 1
    topk_out = torch.full((B, 1, k), -7, dtype=torch.int32, device=DEV)
    out, lse, _ = m.forward_case(case, topk_out=topk_out)
    gs = _gpu_scores_like_forward(m, case)
    torch.cuda.synchronize()
    idx = topk_out.cpu().numpy()
    ep_all = case.end_pos.cpu().numpy()
    check_topk_invariants(idx, ep_all, 1, k)
    for b in seqs:
        sub = slice(b, b + 1)
        h = np_case(case, rows_b=sub)
        n = int(ep_all[b])
        ref_s = oracle.index_scores(h["q"], h["w"], h["k_cache"], h["end_pos"], case.scale,
                                    q_scale=h["q_scale"], k_scale=h["k_scale"])
        g = gs[b:b + 1, :, :n].cpu().numpy()
        assert_scores_close(g, ref_s[:, :, :n], h["end_pos"], 1, SCORE_TOL[case.dtype])
        ref_idx = oracle.topk(np.ascontiguousarray(g), h["end_pos"], k)
        assert np.array_equal(idx[b:b + 1], ref_idx), f"sequence {b}: selection differs"
        o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                    h["end_pos"], case.softmax_scale, indices=idx[b:b + 1])
        assert_out_close(out[sub], lse[sub], o_ref, lse_ref)


def _random_forward_case(seed):
    """A seeded batch drawn across the plan boundaries: query rows on either side
    of the small-batch attention form (4 rows) and of the prefill indexer form
    (8 queries), contexts on either side of the top-k path limits (4096, 32768),
    ragged end_pos, k below and at 2048, both indexer dtypes."""
    rng = np.random.default_rng(1000 + seed)
    T = int(rng.choice([1, 1, 2, 3, 7, 8, 9, 16]))
    B = int(rng.integers(1, (6 if T == 1 else 3) + 1))
    S = int(rng.choice([2300, 4096, 4097, 8192, 20000, 32768, 32769, 70000]))
    k = int(rng.choice([2048, 2048, 1024, 300]))
    dtype = str(rng.choice(["bf16", "fp8"]))
    ep = rng.integers(T, S + 1, size=B)
    ep[int(rng.integers(0, B))] = S  # one sequence fills the cache
    return inputs.make_case(f"rand{seed}", B, T, [int(x) for x in ep], S, dtype=dtype,
                            seed=2000 + seed, device=DEV, topk=k)


@pytest.mark.parametrize("seed", list(range(24)))
def test_forward_random_shapes(seed):
    """dsa_forward on seeded shapes across the plan boundaries, every query row of
    up to two sequences checked as in the fixed-shape tests: scores within
    tolerance of the oracle's, the selection bit-exact against the oracle's top-k
    of the GPU's own scores, the attention within tolerance of the oracle's over
    that selection."""
    m = dsa()
    case = _random_forward_case(seed)
    B, T, k = case.B, case.T, case.topk
    ep_all = case.end_pos.cpu().numpy()
    banner(f"forward random seed={seed}: B={B} T={T} S_max={case.S_max} k={k} "
           f"dtype={case.dtype} end_pos={ep_all.tolist()}")
    topk_out = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    out, lse, _ = m.forward_case(case, topk_out=topk_out)
    gs = _gpu_scores_like_forward(m, case)
    torch.cuda.synchronize()
    idx = topk_out.cpu().numpy()
    check_topk_invariants(idx, ep_all, T, k)
    for b in sorted({0, B - 1}):
        sub = slice(b, b + 1)
        h = np_case(case, rows_b=sub)
        n = int(ep_all[b])
        ref_s = oracle.index_scores(h["q"], h["w"], h["k_cache"], h["end_pos"], case.scale,
                                    q_scale=h["q_scale"], k_scale=h["k_scale"])
        g = gs[sub, :, :n].cpu().numpy()
        assert_scores_close(g, ref_s[:, :, :n], h["end_pos"], T, SCORE_TOL[case.dtype])
        ref_idx = oracle.topk(np.ascontiguousarray(g), h["end_pos"], k)
        assert np.array_equal(idx[sub], ref_idx), f"sequence {b}: selection differs"
        o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                    h["end_pos"], case.softmax_scale, indices=idx[sub])
        assert_out_close(out[sub], lse[sub], o_ref, lse_ref)


def test_forward_decode_32k_normal():
    """The 32K bf16 decode workload, as timed: scores within tolerance of the
    oracle's, the selection bit-exact against the oracle's top-k of the GPU's
    own scores, the output within tolerance of the oracle's attention over that
    selection."""
    banner("forward decode_32k normal")
    _check_forward_rows(inputs.decode_32k(device=DEV), [0])


@pytest.mark.parametrize("B,T,eps,k", [(2, 640, [640, 3000], 256), (1, 2, [2], 2048),
                                        (1, 40, [40], 64)])
def test_forward_skips_empty_list_tail(B, T, eps, k):
    """dsa_forward bounds each attention list by the query's causal bound
    (the selection fills only the first min(k, bound) slots).  Early prefill
    queries then have short lists, ending inside a tile or a split; the
    result must equal, bit for bit, dsa_sparse_mla over the full k slots of
    the same selection, and match the oracle on sampled rows."""
    m = dsa()
    banner(f"forward list bound B={B} T={T} end_pos={eps} k={k}")
    case = inputs.make_case("list_bound", B, T, eps, max(eps), seed=21, topk=k, device=DEV)
    topk_out = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
    out, lse, _ = m.forward_case(case, topk_out=topk_out)
    out2, lse2 = m.sparse_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, topk_out,
                              case.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(lse, lse2)
    h = np_case(case)
    n = B * T
    rows = sorted({0, 1, 31, 32, 33, k - 1, k, T - 1, n - 1} & set(range(n)))
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                h["end_pos"], case.softmax_scale,
                                indices=topk_out.cpu().numpy(), rows=rows)
    assert_out_close(out, lse, o_ref, lse_ref, rows=rows)


def test_forward_rows_mix():
    """Four decode rows mixing the top-k's forms: candidate-list rows of 20000 and 9000
    positions (split over workgroups, finished by the second launch), one that fits a
    single workgroup (3000) and one with fewer than k positions (1500); the attention
    takes its 4-wave small-batch form.  Integer inputs, indices exact end to end."""
    banner("forward rows mix")
    case = inputs.make_case("fused_mix", 4, 1, [20000, 3000, 9000, 1500], 20000,
                            index_dist="int", seed=17, device=DEV)
    out, lse, idx, ref_s, ref_idx, o_ref, lse_ref, h = _forward_and_oracle(case)
    assert np.array_equal(idx, ref_idx)
    assert_out_close(out, lse, o_ref, lse_ref)


def test_forward_sample_misjudged():
    """A 32768-token row built so that the top-k's sampled cut lets fewer than k
    candidates through.  The sample is 128 evenly spaced runs of 16 consecutive positions
    (run g starts at floor(g (n - 16) / 127)); the even-numbered runs score highest, the
    odd-numbered ones lowest, every other position in between and equal.  The sample's
    cut then admits only the 1024 high positions, and the selection falls back to a pass
    over the whole row; the answer is those 1024 plus the first 1024 of the middle ones
    (ties to the smaller position)."""
    banner("forward, sample misjudged")
    n = 32768
    case = inputs.make_case("fused_fallback", 1, 1, [n], n, seed=18, device=DEV)
    starts = (np.arange(128) * (n - 16)) // 127
    runs = starts[:, None] + np.arange(16)[None, :]
    c = torch.full((n,), 2.0)
    c[torch.from_numpy(runs[0::2].ravel())] = 3.0
    c[torch.from_numpy(runs[1::2].ravel())] = 1.0
    q = torch.zeros(1, 1, 64, 128)
    q[..., 0] = 1.0
    k_cache = torch.zeros(1, n, 128)
    k_cache[0, :, 0] = c
    case.q = q.to(torch.bfloat16).to(DEV)
    case.w = torch.ones(1, 1, 64, device=DEV)
    case.k_cache = k_cache.to(torch.bfloat16).to(DEV)
    out, lse, idx, ref_s, ref_idx, o_ref, lse_ref, h = _forward_and_oracle(case)
    cn = c.numpy()
    expect = np.sort(np.concatenate([np.flatnonzero(cn == 3.0), np.flatnonzero(cn == 2.0)[:1024]]))
    assert np.array_equal(ref_idx[0, 0], expect)
    assert np.array_equal(idx, ref_idx)
    assert_out_close(out, lse, o_ref, lse_ref)


@pytest.mark.parametrize("n,hot", [(32768, [(1000, 1400)]), (32768, [(0, 64), (32700, 32768)]),
                                   (100000, [(5000, 7500)])])
def test_forward_clustered_winners(n, hot):
    """Integer inputs whose highest scores sit in a few runs of consecutive positions:
    the regions holding them keep only their local share of candidates, so the
    selection must read those regions again in full.  Indices exact end to end."""
    banner(f"forward clustered winners n={n} hot={hot}")
    case = inputs.make_case("clustered", 1, 1, [n], n, index_dist="int", seed=41, device=DEV)
    kc = case.k_cache.float()
    for a, b in hot:
        kc[0, a:b] = 4.0  # every dot product at its largest: these score highest
    case.k_cache = kc.to(torch.bfloat16)
    case.q = case.q.abs()
    case.w = case.w.abs()
    out, lse, idx, ref_s, ref_idx, o_ref, lse_ref, h = _forward_and_oracle(case)
    assert np.array_equal(idx, ref_idx)
    assert_out_close(out, lse, o_ref, lse_ref)


def test_forward_b64_varlen_fp8_sampled():
    """The batch-64 fp8 workload at full size, as timed; the oracle checks sampled
    sequences (the shortest, the longest and two others)."""
    banner("forward decode_b64_varlen fp8 (sampled)")
    case = inputs.decode_b64_varlen(device=DEV)
    ep = case.end_pos.cpu().numpy()
    seqs = sorted({0, 37, int(np.argmin(ep)), int(np.argmax(ep))})
    _check_forward_rows(case, seqs)


@pytest.mark.parametrize("n", [131072, 1024])
def test_forward_sweep_b8_fp8_sampled(n):
    """The batch-8 fp8 sweep shape the break-even is timed on, at its longest and
    shortest context; sampled sequences."""
    banner(f"forward sweep b8 fp8 n={n}")
    _check_forward_rows(inputs.sweep(n, device=DEV), [0, 7])


@pytest.mark.parametrize("n,T", [(1024, 1), (2048, 1), (2000, 16)])
def test_forward_short_context_equals_dense(n, T):
    """Every query with at most k valid positions keeps all of them (topk(min(k, end_pos))
    of Indexer.forward), so the full indexer -> top-k -> attention path must give the
    dense attention over each causal prefix (the bypass MLX takes for short contexts):
    the selection is 0..bound then -1 bit for bit, and the two outputs agree within the
    attention tolerance."""
    m = dsa()
    banner(f"forward short context n={n} T={T}")
    B, k = 8 if T == 1 else 2, 2048
    case = inputs.make_case(f"short_{n}_{T}", B, T, [n] * B, n, dtype="fp8", seed=29,
                            device=DEV)
    out, lse, idx = m.forward_case(case, topk_out=torch.empty((B, T, k), dtype=torch.int32,
                                                               device=DEV))
    dout, dlse = m.dense_mla(case.q_nope, case.q_pe, case.kv_cache, case.pe_cache, case.end_pos,
                             case.softmax_scale, max_end_pos=n)
    torch.cuda.synchronize()
    bound = n - T + np.arange(T)  # last valid position of each query row
    want = np.full((T, k), -1, np.int32)
    for t in range(T):
        want[t, :bound[t] + 1] = np.arange(bound[t] + 1)
    got = idx.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got[b], want), b
    diff = (out.float() - dout.float()).abs().max().item()
    assert diff <= OUT_TOL, diff
    assert (lse - dlse).abs().max().item() <= LSE_TOL


def test_forward_deterministic():
    m = dsa()
    banner("forward determinism")
    case = inputs.make_case("det", 4, 1, [9000, 4000, 2048, 12000], 12000, dtype="fp8",
                            seed=17, device=DEV)
    r1 = m.forward_case(case, topk_out=torch.empty((4, 1, 2048), dtype=torch.int32, device=DEV))
    r2 = m.forward_case(case, topk_out=torch.empty((4, 1, 2048), dtype=torch.int32, device=DEV))
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1]) and torch.equal(r1[2], r2[2])


def test_forward_graph_replay_matches_eager():
    """dsa_forward captured in a HIP graph: every replay, with eager work in between,
    gives the eager result bit for bit (no memset nodes, no hidden allocation)."""
    m = dsa()
    banner("forward graph replay")
    case = inputs.make_case("graph", 2, 1, [5000, 3100], 5000, seed=18, device=DEV)
    other = inputs.make_case("graph_other", 2, 1, [5000, 4000], 5000, seed=19, device=DEV)
    B, T, S, k = case.B, case.T, case.S_max, case.topk
    ws = torch.zeros(m.forward_workspace_size(B, T, S, k), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, T, 128, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, T, 128), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)

    def run(c):
        m.forward(c.q, c.w, c.k_cache, c.end_pos, c.q_nope, c.q_pe, c.kv_cache, c.pe_cache,
                  c.scale, c.softmax_scale, k=k, max_end_pos=S, out=out, lse=lse, topk_out=idx,
                  workspace=ws)

    run(case)
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), idx.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run(case)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        run(other)  # eager work that overwrites every output and the workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]) and torch.equal(idx, ref[2]), rep
    # The replayed step against the oracle: its selection equals the oracle's
    # top-k of the GPU's own scores, its attention the oracle's over that selection.
    gs = m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale, max_end_pos=S)
    torch.cuda.synchronize()
    h = np_case(case)
    ep = h["end_pos"]
    ref_s = oracle_scores(case, h)
    g_np = gs.cpu().numpy()
    for b in range(B):
        n = int(ep[b])
        assert_scores_close(g_np[b:b + 1, :, :n], ref_s[b:b + 1, :, :n], ep[b:b + 1], 1,
                            SCORE_TOL[case.dtype])
    g_np = np.where(np.isfinite(g_np), g_np, 0.0).astype(np.float32)
    assert np.array_equal(idx.cpu().numpy(), oracle.topk(g_np, ep, k))
    o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"], ep,
                                case.softmax_scale, indices=idx.cpu().numpy())
    assert_out_close(out, lse, o_ref, lse_ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_forward_graph_api_steps_vs_oracle(dtype):
    """The library's captured decode step (dsa_forward_graph_create / _launch)
    driven like a serving loop: the bound buffers are rewritten in place with a
    new batch before each replay (new queries, caches, end positions under the
    same max_end_pos), and every replay is checked against the oracle on that
    batch.  Integer-valued indexer inputs, so the selection is exact end to end."""
    m = dsa()
    B, S, k = 2, 5000, 2048
    steps = [([5000, 3100], 31), ([4000, 4999], 32), ([2049, 5000], 33)]
    first = inputs.make_case("graph_api", B, 1, steps[0][0], S, dtype=dtype, index_dist="int",
                             seed=steps[0][1], device=DEV)
    buf = inputs.make_case("graph_api_buf", B, 1, steps[0][0], S, dtype=dtype,
                           index_dist="int", seed=30, device=DEV)  # other contents at capture
    ws = torch.empty(m.forward_workspace_size(B, 1, S, k), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, 1, 128, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, 1, 128), dtype=torch.float32, device=DEV)
    idx = torch.full((B, 1, k), -7, dtype=torch.int32, device=DEV)
    graph = m.ForwardGraph(buf.q, buf.w, buf.k_cache, buf.end_pos, buf.q_nope, buf.q_pe,
                           buf.kv_cache, buf.pe_cache, buf.scale, buf.softmax_scale, out, lse,
                           idx, ws, k=k, q_scale=buf.q_scale, k_scale=buf.k_scale,
                           max_end_pos=S)
    names = ("q", "w", "k_cache", "end_pos", "q_nope", "q_pe", "kv_cache", "pe_cache",
             "q_scale", "k_scale")
    try:
        for eps, seed in steps:
            banner(f"forward graph api {dtype} end_pos={eps}")
            case = first if seed == steps[0][1] else inputs.make_case(
                "graph_api", B, 1, eps, S, dtype=dtype, index_dist="int", seed=seed, device=DEV)
            for nm in names:
                src = getattr(case, nm)
                if src is not None:
                    getattr(buf, nm).copy_(src)
            graph.launch()
            torch.cuda.synchronize()
            h = np_case(case)
            ref_s = oracle_scores(case, h)
            ref_idx = oracle.topk(np.nan_to_num(ref_s, nan=0.0), h["end_pos"], k)
            assert np.array_equal(idx.cpu().numpy(), ref_idx), f"end_pos {eps}"
            o_ref, lse_ref = oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"],
                                        h["end_pos"], case.softmax_scale, indices=ref_idx)
            assert_out_close(out, lse, o_ref, lse_ref)
    finally:
        graph.close()


@pytest.mark.parametrize("S", [40000, 140000])
@pytest.mark.parametrize("fill", [0x00, 0xFF, 0x3C, "random"])
def test_topk_any_workspace_content(fill, S):
    """Whatever the top-k workspace holds on entry (region headers, lists and the
    list counters of the split path, which the call clears itself), the
    selection is exact: rows up to 131072 positions take the cut path, longer
    promised bounds the split path."""
    m = dsa()
    banner(f"topk workspace fill={fill} S={S}")
    B, T, k = 3, 1, 2048
    ep = np.array([S if S <= 131072 else 120000, 33000, 9000], np.int32)
    scores = inputs.make_scores(B, T, S, kind="normal", seed=21, device=DEV)
    nbytes = m.lib().dsa_topk_workspace_size(B, T, S, k)
    if fill == "random":
        g = torch.Generator(device=DEV)
        g.manual_seed(5)
        ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV, generator=g)
    else:
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
    ref = oracle.topk(scores.cpu().numpy(), ep, k)
    end_pos = torch.from_numpy(ep).to(DEV)
    for rep in range(3):  # repeated calls over the same workspace
        out = m.topk(scores, end_pos, k, max_end_pos=S, workspace=ws)
        assert np.array_equal(out.cpu().numpy(), ref), rep


def test_prefill_8192_sampled():
    """The T=8192 causal prefill at full size, checked on sampled query rows
    (each recomputed by the oracle as a one-query decode with end_pos = t+1,
    which has the same causal bound): indexer scores within tolerance, top-k
    bit-exact on the GPU's own scores, attention within tolerance given the
    GPU's indices."""
    m = dsa()
    banner("prefill T=8192 sampled rows")
    case = inputs.prefill(8192, device=DEV)
    T, k = case.T, case.topk
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    out, _, _ = m.forward(case.q, case.w, case.k_cache, case.end_pos, case.q_nope, case.q_pe,
                       case.kv_cache, case.pe_cache, case.scale, case.softmax_scale, k=k,
                       max_end_pos=T, topk_out=idx)
    scores = m.index_scores(case.q, case.w, case.k_cache, case.end_pos, case.scale,
                            max_end_pos=T)
    torch.cuda.synchronize()
    kc = inputs.to_numpy(case.k_cache)
    kv = inputs.to_numpy(case.kv_cache)
    pe = inputs.to_numpy(case.pe_cache)
    for t in (0, 15, 16, 2047, 2048, 5001, 8191):
        ep = np.array([t + 1], np.int32)
        qt = inputs.to_numpy(case.q[:, t:t + 1])
        wt = case.w[:, t:t + 1].cpu().numpy()
        ref_s = oracle.index_scores(qt, wt, kc, ep, case.scale)[0, 0, :t + 1]
        g_s = scores[0, t, :t + 1].cpu().numpy()
        err = np.abs(g_s.astype(np.float64) - ref_s).max() / max(np.abs(ref_s).max(), 1e-30)
        assert err <= SCORE_TOL["bf16"], (t, float(err))
        ref_i = oracle.topk(g_s.reshape(1, 1, -1), ep, k)
        assert np.array_equal(idx[0, t].cpu().numpy(), ref_i[0, 0]), t
        o_ref, _ = oracle.mla(inputs.to_numpy(case.q_nope[:, t:t + 1]),
                              inputs.to_numpy(case.q_pe[:, t:t + 1]), kv, pe, ep,
                              case.softmax_scale, indices=ref_i)
        o_gpu = out[0, t].float().cpu().numpy()
        assert np.abs(o_gpu - o_ref[0, 0]).max() < OUT_TOL, t


def test_forward_chunked_prefill_long_cache_fp8():
    """1100 new queries at the end of a 40000-position fp8 cache (a chunk of a long
    prefill): more than 1024 query rows over rows longer than 32768 positions, so the
    forward path's selection is the chunk-by-chunk whole-row form, behind the prefill
    indexer form and the many-row attention.  Sampled rows as in the 8192-token test:
    scores within tolerance, selection bit-exact on the GPU's own scores, attention
    within tolerance over it."""
    m = dsa()
    banner("forward chunked prefill T=1100 over 40000 fp8")
    B, T, S = 1, 1100, 40000
    case = inputs.make_case("chunk", B, T, [S], S, dtype="fp8", seed=61, device=DEV)
    k = case.topk
    idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    out, _, _ = m.forward_case(case, topk_out=idx)
    gs = _gpu_scores_like_forward(m, case)
    torch.cuda.synchronize()
    h = np_case(case)
    for t in (0, 1, 547, 1098, 1099):
        bound = S - T + t
        ep = np.array([bound + 1], np.int32)
        ref_s = oracle.index_scores(h["q"][:, t:t + 1], h["w"][:, t:t + 1], h["k_cache"], ep,
                                    case.scale, q_scale=h["q_scale"][:, t:t + 1],
                                    k_scale=h["k_scale"])[0, 0, :bound + 1]
        g_s = gs[0, t, :bound + 1].cpu().numpy()
        err = np.abs(g_s.astype(np.float64) - ref_s).max() / max(np.abs(ref_s).max(), 1e-30)
        assert err <= SCORE_TOL["fp8"], (t, float(err))
        ref_i = oracle.topk(g_s.reshape(1, 1, -1), ep, k)
        assert np.array_equal(idx[0, t].cpu().numpy(), ref_i[0, 0]), t
        o_ref, _ = oracle.mla(h["q_nope"][:, t:t + 1], h["q_pe"][:, t:t + 1], h["kv_cache"],
                              h["pe_cache"], ep, case.softmax_scale, indices=ref_i)
        assert np.abs(out[0, t].float().cpu().numpy() - o_ref[0, 0]).max() < OUT_TOL, t


# --- query absorption and output up-projection --------------------------------------

@pytest.mark.parametrize("B,T", [(1, 1), (3, 37), (1, 300), (1, 2), (1, 63), (1, 64), (5, 13),
                                 (2, 128), (1, 256), (1, 257), (4, 150)])
def test_q_absorb_and_out_proj(B, T):
    """Both head-batched products against the oracle: one decode row, a ragged
    batch (two 64-row workgroups, the second partial), 300 rows, and row counts
    around the 64-row blocks and the up-projection's switch at 256 rows."""
    m = dsa()
    banner(f"absorb / up-projection B={B} T={T}")
    qn, wkv, x = inputs.make_proj(B, T, seed=B * 100 + T, device=DEV)
    qa = m.q_absorb(qn, wkv)
    y = m.out_proj(x, wkv)
    ref_qa = oracle.q_absorb(inputs.to_numpy(qn), inputs.to_numpy(wkv))
    ref_y = oracle.out_proj(inputs.to_numpy(x), inputs.to_numpy(wkv))
    # bf16 outputs of fp32 sums: within two bf16 half-ulps of the largest value
    for g, r in ((qa, ref_qa), (y, ref_y)):
        g = g.float().cpu().numpy().astype(np.float64)
        assert np.abs(g - r).max() <= 2.0 ** -8 * np.abs(r).max()


# --- indexer input preparation -----------------------------------------------------

E4M3_POISON = 0x7F      # an e4m3fn NaN code: a cache row the call must not touch keeps it
BF16_POISON = 0x7FC1


def _prep_run(m, q_in, k_in, cos, sin, ep, S_max, fp8):
    B = q_in.shape[0]
    if fp8:
        kc = torch.full((B, S_max, 128), E4M3_POISON, dtype=torch.uint8, device=DEV)
        kc = kc.view(torch.float8_e4m3fn)
        ks = torch.full((B, S_max), -1.0, dtype=torch.float32, device=DEV)
    else:
        kc = torch.full((B, S_max, 128), BF16_POISON, dtype=torch.int16, device=DEV)
        kc = kc.view(torch.bfloat16)
        ks = None
    qo, qs = m.indexer_prep(q_in, k_in, cos, sin, ep, kc, ks)
    torch.cuda.synchronize()
    return qo, qs, kc, ks


def _e4m3_step(x):
    """Spacing of e4m3 values around |x| (2^-9 below the normal range)."""
    a = np.maximum(np.abs(x), 2.0 ** -6)
    return 2.0 ** (np.floor(np.log2(a)) - 3)


def _check_untouched(kc, ks, ep, T, fp8):
    """Every cache row outside end_pos-T..end_pos-1 still holds the poison."""
    kcb = inputs.to_numpy(kc).reshape(kc.shape[0], kc.shape[1], -1)
    for b, e in enumerate(ep.tolist()):
        keep = np.ones(kc.shape[1], bool)
        keep[e - T:e] = False
        poison = E4M3_POISON if fp8 else BF16_POISON
        assert np.all(kcb[b][keep] == poison), f"sequence {b}: a row outside the new tokens changed"
        if fp8:
            assert np.all(ks[b].cpu().numpy()[keep] == -1.0)


@pytest.mark.parametrize("fp8", [True, False], ids=["fp8", "bf16"])
def test_indexer_prep_integer_exact(fp8):
    """Integer q, k and the identity RoPE (cos 1, sin 0): every sum of the rotation
    is exact in fp32, so codes and scales (fp8) are bit-exact and bf16 values are
    the correctly rounded rotation; a ragged batch (end_pos 7 and 40, T = 5) and
    cache rows outside the new tokens untouched."""
    m = dsa()
    B, T, S_max = 2, 5, 40
    banner(f"prep int fp8={fp8} B={B} T={T}")
    q_in, k_in, cos, sin, ep = inputs.make_prep(B, T, [7, 40], S_max, kind="int", seed=71,
                                                device=DEV)
    qo, qs, kc, ks = _prep_run(m, q_in, k_in, cos, sin, ep, S_max, fp8)
    rq, rqs, rk, rks, pos = oracle.indexer_prep(inputs.to_numpy(q_in), inputs.to_numpy(k_in),
                                                cos.cpu().numpy(), sin.cpu().numpy(),
                                                ep.cpu().numpy(), fp8=fp8)
    kcn = inputs.to_numpy(kc)
    if fp8:
        assert np.array_equal(inputs.to_numpy(qo), rq)
        assert np.array_equal(qs.cpu().numpy(), rqs)
        for b in range(B):
            assert np.array_equal(kcn[b, pos[b]], rk[b])
            assert np.array_equal(ks[b].cpu().numpy()[pos[b]], rks[b])
    else:
        # bf16 keeps 8 significant bits: rounding moves a value by at most 2^-8 of it
        g = qo.float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g - rq) <= 2.0 ** -8 * np.abs(rq))
        gk = kc.float().cpu().numpy().astype(np.float64)
        for b in range(B):
            assert np.all(np.abs(gk[b, pos[b]] - rk[b]) <= 2.0 ** -8 * np.abs(rk[b]))
    _check_untouched(kc, ks, ep.cpu(), T, fp8)


def _compare_prep_fp8(qo, qs, rq, rqs):
    """Scales within 1e-5 relative; dequantised values within one e4m3 step of
    the oracle's (the code decision can go the other way when fp32 and fp64
    land on opposite sides of a rounding midpoint); such flips are rare."""
    gq = inputs.to_numpy(qo)
    gs = np.asarray(qs, np.float64)
    rs = np.asarray(rqs, np.float64)
    assert np.all(np.abs(gs - rs) <= 1e-5 * np.abs(rs))
    assert np.array_equal(gs == 0, rs == 0)
    gv = torch.from_numpy(gq).view(torch.float8_e4m3fn).double().numpy()
    rv = torch.from_numpy(np.ascontiguousarray(rq)).view(torch.float8_e4m3fn).double().numpy()
    d = np.abs(gv - rv)
    assert np.all(d <= _e4m3_step(np.maximum(np.abs(gv), np.abs(rv))) * 1.0001)
    assert (d > 0).mean() < 0.01


def _compare_prep_bf16(g, r):
    g = np.asarray(g, np.float64)
    assert np.all(np.abs(g - r) <= 2.0 ** -8 * np.abs(r) + 1e-6 * np.abs(r).max())


@pytest.mark.parametrize("fp8", [True, False], ids=["fp8", "bf16"])
@pytest.mark.parametrize("kind", ["normal", "zero"])
def test_indexer_prep_random(fp8, kind):
    """N(0,1) inputs, random RoPE angles, ragged batch of 3 sequences with 37 new
    tokens each (end_pos 37, 100, 300); "zero" adds all-zero query heads and keys
    (scale 0, zero codes)."""
    m = dsa()
    B, T, S_max = 3, 37, 300
    banner(f"prep {kind} fp8={fp8} B={B} T={T}")
    q_in, k_in, cos, sin, ep = inputs.make_prep(B, T, [37, 100, 300], S_max, kind=kind,
                                                seed=72, device=DEV)
    qo, qs, kc, ks = _prep_run(m, q_in, k_in, cos, sin, ep, S_max, fp8)
    rq, rqs, rk, rks, pos = oracle.indexer_prep(inputs.to_numpy(q_in), inputs.to_numpy(k_in),
                                                cos.cpu().numpy(), sin.cpu().numpy(),
                                                ep.cpu().numpy(), fp8=fp8)
    gk = np.stack([inputs.to_numpy(kc[b])[pos[b]] for b in range(B)])
    if fp8:
        gks = np.stack([ks[b].cpu().numpy()[pos[b]] for b in range(B)])
        _compare_prep_fp8(qo, qs.cpu().numpy(), rq, rqs)
        _compare_prep_fp8(torch.from_numpy(gk).view(torch.float8_e4m3fn), gks, rk, rks)
        if kind == "zero":
            assert np.all(rqs[:, :, ::7] == 0) and np.all(qs.cpu().numpy()[:, :, ::7] == 0)
            assert not inputs.to_numpy(qo)[:, :, ::7].any()
    else:
        _compare_prep_bf16(qo.float().cpu().numpy(), rq)
        _compare_prep_bf16(torch.from_numpy(gk).view(torch.bfloat16).float().numpy(), rk)
    _check_untouched(kc, ks, ep.cpu(), T, fp8)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("kind", ["normal", "zero"])
def test_indexer_prep_many_tokens(fp8, kind):
    """More than 512 tokens take the form with 4 lanes and 32 dims per vector (RoPE
    pairs inside a lane, two cross-lane rotation stages): a ragged batch of 3
    sequences with 200 new tokens each, both dtypes; "zero" adds all-zero query
    heads and keys (scale 0, zero codes).  Every written query and key against the
    oracle, the rest of the cache untouched."""
    m = dsa()
    B, T, S_max = 3, 200, 1000
    banner(f"prep many tokens {kind} fp8={fp8} B={B} T={T}")
    q_in, k_in, cos, sin, ep = inputs.make_prep(B, T, [200, 640, 1000], S_max, kind=kind,
                                                seed=73, device=DEV)
    qo, qs, kc, ks = _prep_run(m, q_in, k_in, cos, sin, ep, S_max, fp8)
    rq, rqs, rk, rks, pos = oracle.indexer_prep(inputs.to_numpy(q_in), inputs.to_numpy(k_in),
                                                cos.cpu().numpy(), sin.cpu().numpy(),
                                                ep.cpu().numpy(), fp8=fp8)
    gk = np.stack([inputs.to_numpy(kc[b])[pos[b]] for b in range(B)])
    if fp8:
        gks = np.stack([ks[b].cpu().numpy()[pos[b]] for b in range(B)])
        _compare_prep_fp8(qo, qs.cpu().numpy(), rq, rqs)
        _compare_prep_fp8(torch.from_numpy(gk).view(torch.float8_e4m3fn), gks, rk, rks)
        if kind == "zero":
            assert np.all(rqs[:, :, ::7] == 0) and np.all(qs.cpu().numpy()[:, :, ::7] == 0)
            assert not inputs.to_numpy(qo)[:, :, ::7].any()
    else:
        _compare_prep_bf16(qo.float().cpu().numpy(), rq)
        _compare_prep_bf16(torch.from_numpy(gk).view(torch.bfloat16).float().numpy(), rk)
    _check_untouched(kc, ks, ep.cpu(), T, fp8)


@pytest.mark.parametrize("seed", list(range(8)))
def test_indexer_prep_random_shapes(seed):
    """dsa_indexer_prep on seeded ragged batches: 1 to 5 sequences, 1 to 300 new
    tokens each, caches a little or much longer than the longest sequence, fp8 or
    bf16; every written query and key against the oracle, the rest of the cache
    untouched."""
    m = dsa()
    rng = np.random.default_rng(6000 + seed)
    B = int(rng.integers(1, 6))
    T = int(rng.choice([1, 2, 3, 17, 64, 300]))
    ep = [int(x) for x in rng.integers(T, T + 700, size=B)]
    S_max = max(ep) + int(rng.choice([0, 1, 129, 5000]))
    fp8 = bool(rng.integers(0, 2))
    banner(f"prep random seed={seed}: B={B} T={T} S_max={S_max} fp8={fp8} end_pos={ep}")
    q_in, k_in, cos, sin, ep_t = inputs.make_prep(B, T, ep, S_max, seed=7000 + seed, device=DEV)
    qo, qs, kc, ks = _prep_run(m, q_in, k_in, cos, sin, ep_t, S_max, fp8)
    rq, rqs, rk, rks, pos = oracle.indexer_prep(inputs.to_numpy(q_in), inputs.to_numpy(k_in),
                                                cos.cpu().numpy(), sin.cpu().numpy(),
                                                ep_t.cpu().numpy(), fp8=fp8)
    gk = np.stack([inputs.to_numpy(kc[b])[pos[b]] for b in range(B)])
    if fp8:
        gks = np.stack([ks[b].cpu().numpy()[pos[b]] for b in range(B)])
        _compare_prep_fp8(qo, qs.cpu().numpy(), rq, rqs)
        _compare_prep_fp8(torch.from_numpy(gk).view(torch.float8_e4m3fn), gks, rk, rks)
    else:
        _compare_prep_bf16(qo.float().cpu().numpy(), rq)
        _compare_prep_bf16(torch.from_numpy(gk).view(torch.bfloat16).float().numpy(), rk)
    _check_untouched(kc, ks, ep_t.cpu(), T, fp8)


@pytest.mark.parametrize("shape", ["prefill_8192", "decode_b64"])
def test_indexer_prep_full_size_sampled(shape):
    """The two full-size shapes at which the preparation is timed -- one sequence
    of 8192 new tokens, and 64 sequences decoding one token each at context
    lengths up to 131072 -- checked on sampled tokens, each recomputed by the
    oracle on its own (a one-token batch at that position)."""
    m = dsa()
    if shape == "prefill_8192":
        B, T, S_max, ep_list = 1, 8192, 8192, [8192]
        sample = [(0, t) for t in (0, 1, 15, 16, 2047, 4000, 8190, 8191)]
    else:
        g = torch.Generator().manual_seed(73)
        B, T, S_max = 64, 1, 131072
        ep_list = torch.randint(8192, S_max + 1, (B,), generator=g).tolist()
        ep_list[0], ep_list[1] = 1, S_max
        sample = [(b, 0) for b in (0, 1, 2, 31, 63)]
    banner(f"prep full size {shape}")
    q_in, k_in, cos, sin, ep = inputs.make_prep(B, T, ep_list, S_max, seed=74, device=DEV)
    qo, qs, kc, ks = _prep_run(m, q_in, k_in, cos, sin, ep, S_max, True)
    cn, sn = cos.cpu().numpy(), sin.cpu().numpy()
    for b, t in sample:
        p = ep_list[b] - T + t
        rq, rqs, rk, rks, _ = oracle.indexer_prep(
            inputs.to_numpy(q_in[b:b + 1, t:t + 1]), inputs.to_numpy(k_in[b:b + 1, t:t + 1]),
            cn, sn, np.array([p + 1], np.int32))
        _compare_prep_fp8(qo[b:b + 1, t:t + 1], qs[b:b + 1, t:t + 1].cpu().numpy(), rq, rqs)
        _compare_prep_fp8(kc[b:b + 1, p:p + 1].contiguous().view(1, 1, 128),
                          ks[b:b + 1, p:p + 1].cpu().numpy(), rk, rks)
        if T == 1:      # the neighbouring cache rows keep the poison
            for r in (p - 1, p + 1):
                if 0 <= r < S_max:
                    assert np.all(inputs.to_numpy(kc[b, r]) == E4M3_POISON)


def test_indexer_prep_feeds_index_scores():
    """The preparation's fp8 outputs are the inputs of dsa_index_scores: scoring
    the prepared query against the prepared cache on the GPU matches the oracle's
    scores of the oracle's prepared tensors (ragged prefill batch)."""
    m = dsa()
    B, T, S_max = 2, 20, 64
    banner("prep -> index_scores")
    q_in, k_in, cos, sin, ep = inputs.make_prep(B, T, [20, 64], S_max, seed=75, device=DEV)
    # fill the earlier cache rows by preparing them as a first batch of tokens
    kc = torch.zeros((B, S_max, 128), dtype=torch.float8_e4m3fn, device=DEV)
    ks = torch.zeros((B, S_max), dtype=torch.float32, device=DEV)
    q0, k0, _, _, _ = inputs.make_prep(B, 44, [44, 44], S_max, seed=76, device=DEV)
    ep0 = torch.tensor([44, 44], dtype=torch.int32, device=DEV)
    m.indexer_prep(q0, k0, cos, sin, ep0, kc, ks)
    qo, qs = m.indexer_prep(q_in, k_in, cos, sin, ep, kc, ks)
    w = torch.randn((B, T, 64), generator=torch.Generator(device=DEV).manual_seed(77),
                    device=DEV)
    scale = 128 ** -0.5
    got = m.index_scores(qo, w, kc, ep, scale, q_scale=qs, k_scale=ks).cpu().numpy()
    # The oracle's own preparation of the same inputs (first batch, then this one)
    rk = np.zeros((B, S_max, 128), np.uint8)
    rks = np.zeros((B, S_max), np.float32)
    cn, sn = cos.cpu().numpy(), sin.cpu().numpy()
    _, _, k0c, k0s, p0 = oracle.indexer_prep(inputs.to_numpy(q0), inputs.to_numpy(k0), cn, sn,
                                             np.array([44, 44], np.int32))
    rq, rqs, k1c, k1s, p1 = oracle.indexer_prep(inputs.to_numpy(q_in), inputs.to_numpy(k_in),
                                                cn, sn, ep.cpu().numpy())
    for b in range(B):
        rk[b, p0[b]], rks[b, p0[b]] = k0c[b], k0s[b]
        rk[b, p1[b]], rks[b, p1[b]] = k1c[b], k1s[b]
    ref = oracle.index_scores(rq, w.cpu().numpy(), rk, ep.cpu().numpy(), scale, q_scale=rqs,
                              k_scale=rks)
    for b in range(B):
        for t in range(T):
            bound = int(ep[b]) - T + t
            g, r = got[b, t, :bound + 1], ref[b, t, :bound + 1]
            assert np.abs(g - r).max() <= 2e-2 * np.abs(r).max()



# --- MHA-form prefill attention ------------------------------------------------------

def _mha_indices(B, T, k, kind, seed):
    """Index lists: "random" (any of 0..T+2, -1, ...: duplicates, future and out
    of range entries), or make_indices' causal "random" / "last" selections."""
    if kind == "messy":
        g = torch.Generator().manual_seed(seed)
        return torch.randint(-3, T + 3, (B, T, k), generator=g, dtype=torch.int32).to(DEV)
    return inputs.make_indices(B, T, [T] * B, k, seed=seed, fill=kind, device=DEV)


def _mha_check(B, T, k, kind, seed, rows=None):
    m = dsa()
    q, kn, kp, v = inputs.make_mha(B, T, seed=seed, device=DEV)
    idx = _mha_indices(B, T, k, kind, seed)
    scale = 192 ** -0.5
    out, lse = m.sparse_mha_prefill(q, kn, kp, v, idx, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.sparse_mha_prefill(inputs.to_numpy(q), inputs.to_numpy(kn),
                                               inputs.to_numpy(kp), inputs.to_numpy(v),
                                               idx.cpu().numpy(), scale, rows=rows)
    assert_out_close(out, lse, o_ref, lse_ref, rows=rows)


@pytest.mark.parametrize("B,T,k,kind", [
    (2, 100, 16, "messy"),    # duplicates, future and out-of-range entries; ragged 64-query tail
    (1, 37, 64, "last"),      # fewer tokens than one query block
    (1, 200, 2048, "random"), # k >= T: every causal position selected (dense causal)
    (2, 130, 24, "random"),   # causal random selections, two sequences
    (1, 700, 300, "random"),  # three 256-query blocks, the last one ragged
    (2, 520, 40, "messy"),    # two sequences of just over two query blocks
])
def test_mha_prefill_vs_oracle(B, T, k, kind):
    """MHA-form prefill (selection bitmap + masked tiles) against the oracle on
    every query row."""
    banner(f"mha prefill B={B} T={T} k={k} {kind}")
    _mha_check(B, T, k, kind, seed=B * 1000 + T)


@pytest.mark.parametrize("seed", list(range(8)))
def test_mha_prefill_random_shapes(seed):
    """dsa_sparse_mha_prefill on seeded shapes: 1 or 2 sequences of 1 to 1100
    tokens (query blocks of 256 with ragged tails), k from 1 to 2048, random,
    trailing or messy selections (duplicates, future and out-of-range entries);
    sampled rows against the oracle."""
    rng = np.random.default_rng(8000 + seed)
    B = int(rng.integers(1, 3))
    T = int(rng.choice([1, 5, 63, 64, 255, 257, 600, 1100]))
    k = int(rng.choice([1, 16, 300, 2048]))
    kind = str(rng.choice(["random", "last", "messy"]))
    banner(f"mha random seed={seed}: B={B} T={T} k={k} {kind}")
    n = B * T
    rows = sorted({0, T - 1, n // 2, n - 1} | {int(x) for x in rng.integers(0, n, size=3)})
    _mha_check(B, T, k, kind, seed=9000 + seed, rows=rows)


def test_mha_prefill_8192_sampled():
    """The timed size, one 8192-token sequence with 2048 random causal
    selections per query, on sampled rows (first and last of query blocks, the
    first row with more than k candidates, the last row)."""
    banner("mha prefill T=8192 sampled")
    _mha_check(1, 8192, 2048, "random", seed=91, rows=[0, 1, 63, 64, 2047, 2048, 5000, 8191])
