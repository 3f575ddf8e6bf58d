"""The C ABI on the CPU: exports match the header, validation happens before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


@pytest.fixture(scope="module")
def L():
    import sparse_attention_indexer_amd as dsa
    return dsa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_path():
    names = declared_functions()
    for n in ("dsa_index_scores", "dsa_topk", "dsa_sparse_mla", "dsa_forward", "dsa_dense_mla",
              "dsa_status_string", "dsa_topk_workspace_size", "dsa_sparse_mla_workspace_size",
              "dsa_forward_workspace_size", "dsa_dense_mla_workspace_size"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in dsa.h but not exported"


def test_status_strings(L):
    for st in (0, -1, -2, -3, -4, -5):
        s = L.dsa_status_string(st).decode()
        assert s.startswith("DSA_")
    assert L.dsa_status_string(-99).decode() == "unknown dsa status"


P = ctypes.c_void_p(256)  # an aligned non-null address; never dereferenced on failure paths
ODD = ctypes.c_void_p(258)


def idx_args(**over):
    a = dict(q=P, q_scale=None, w=P, k=P, k_scale=None, end_pos=P, B=1, T=1, S_max=100,
             max_end_pos=100, scale=1.0, dtype=0, out=P, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,expect", [
    (dict(q=None), -1), (dict(w=None), -1), (dict(k=None), -1), (dict(end_pos=None), -1),
    (dict(out=None), -1), (dict(B=0), -1), (dict(T=0), -1), (dict(S_max=0), -1),
    (dict(max_end_pos=101), -1), (dict(T=5, max_end_pos=4), -1), (dict(dtype=2), -2),
    (dict(dtype=1), -1), (dict(q=ODD), -3), (dict(k=ODD), -3),
    (dict(dtype=1, q_scale=P, k_scale=None), -1),
])
def test_index_scores_validation(L, over, expect):
    assert L.dsa_index_scores(*idx_args(**over)) == expect


@pytest.mark.parametrize("k,expect", [(0, -1), (2049, -2), (-3, -1)])
def test_topk_validation(L, k, expect):
    assert L.dsa_topk(P, P, 1, 1, 100, 100, k, P, None, 0, None) == expect


def test_sparse_mla_validation(L):
    args = [P, P, P, P, P, 1, 1, 100, 2048, 1.0, P, None]
    need = L.dsa_sparse_mla_workspace_size(1, 1, 2048)
    assert need > 0  # batch 1 splits the row list
    assert L.dsa_sparse_mla(*args, P, need - 1, None) == -4
    assert L.dsa_sparse_mla(*args, None, need, None) == -1
    assert L.dsa_sparse_mla(*args, ctypes.c_void_p(272), need, None) == -3
    bad = list(args)
    bad[0] = ODD
    assert L.dsa_sparse_mla(*bad, P, need, None) == -3
    bad = list(args)
    bad[8] = 4096
    assert L.dsa_sparse_mla(*bad, P, 1 << 40, None) == -2
    for s in (0.0, -0.1, float("nan"), float("inf")):  # the softmax scale must be > 0, finite
        bad = list(args)
        bad[9] = s
        assert L.dsa_sparse_mla(*bad, P, need, None) == -1


def test_forward_validation(L):
    need = L.dsa_forward_workspace_size(2, 1, 1000, 2048)
    # index_score (2*1000*4 -> 8192 after alignment) + indices (2*2048*4) + attention partials
    assert need >= 8192 + 16384
    base = [P, None, P, P, None, P, P, P, P, P, 2, 1, 1000, 1000, 2048, 1.0, 1.0, 0, P, None,
            None]
    assert L.dsa_forward(*base, P, need - 1, None) == -4
    bad = list(base)
    bad[14] = 4096
    assert L.dsa_forward(*bad, P, need, None) == -2
    bad = list(base)
    bad[6] = None
    assert L.dsa_forward(*bad, P, need, None) == -1


def test_forward_noalloc_validation(L):
    # Same checks as dsa_forward, then the workspace must fit the library's
    # scratch (96 MiB): refused before any HIP call, so this runs without a GPU.
    scratch = 96 << 20
    base = [P, None, P, P, None, P, P, P, P, P, 2, 1, 1000, 1000, 2048, 1.0, 1.0, 0, P, None,
            None]
    bad = list(base)
    bad[14] = 4096
    assert L.dsa_forward_noalloc(*bad, None) == -2
    bad = list(base)
    bad[6] = None
    assert L.dsa_forward_noalloc(*bad, None) == -1
    S = 1 << 24  # batch 2 at 2^24 positions: 64 MiB of scores per row alone
    assert L.dsa_forward_workspace_size(2, 1, S, 2048) > scratch
    big = list(base)
    big[12] = big[13] = S
    assert L.dsa_forward_noalloc(*big, None) == -4
    # A 4096-query prefill fits exactly.
    assert L.dsa_forward_workspace_size(1, 4096, 4096, 2048) <= scratch


def test_forward_graph_validation(L):
    # dsa_forward's checks come first: nothing is created (no stream, no
    # capture) for a call dsa_forward would refuse, and *graph is NULL.
    need = L.dsa_forward_workspace_size(2, 1, 1000, 2048)
    base = [P, None, P, P, None, P, P, P, P, P, 2, 1, 1000, 1000, 2048, 1.0, 1.0, 0, P, None,
            None]
    h = ctypes.c_void_p(1234)
    assert L.dsa_forward_graph_create(*base, P, need - 1, ctypes.byref(h)) == -4
    assert h.value is None
    bad = list(base)
    bad[14] = 4096
    assert L.dsa_forward_graph_create(*bad, P, need, ctypes.byref(h)) == -2
    bad = list(base)
    bad[6] = None
    assert L.dsa_forward_graph_create(*bad, P, need, ctypes.byref(h)) == -1
    assert L.dsa_forward_graph_create(*base, P, need, None) == -1  # nowhere to put the graph
    assert L.dsa_forward_graph_launch(None, None) == -1
    assert L.dsa_forward_graph_destroy(None) == 0


def test_workspace_sizes_monotone(L):
    a = L.dsa_dense_mla_workspace_size(8, 1, 131072)
    b = L.dsa_dense_mla_workspace_size(8, 1, 262144)
    assert b >= a > 0
    # up to 1024 rows: two counters and a list of 8192 (key, position) pairs per row
    assert L.dsa_topk_workspace_size(1, 1, 32768, 2048) >= 8192 * 8
    assert L.dsa_topk_workspace_size(64, 1, 131072, 2048) >= 64 * 8192 * 8
    # the per-row figures dsa.h states: just over 64 KiB up to 4096 positions, just
    # over 384 KiB (16 regions of 3072 pairs) above
    for rows, S in ((1, 4096), (7, 1000), (1, 4097), (3, 32768), (64, 131072)):
        per_row = L.dsa_topk_workspace_size(rows, 1, S, 2048) / rows
        lo = (64 if S <= 4096 else 384) * 1024
        assert lo <= per_row < lo + 1024, (rows, S, per_row)
    # more rows: one workgroup per row, no workspace
    assert L.dsa_topk_workspace_size(2048, 1, 65536, 2048) == 0
    assert L.dsa_topk_workspace_size(8, 1024, 8192, 2048) == 0
    S = 40000
    assert L.dsa_topk(P, P, 1, 1, S, S, 64, P, None, 1 << 20, None) == -1  # null workspace
    need = L.dsa_topk_workspace_size(1, 1, S, 64)
    assert L.dsa_topk(P, P, 1, 1, S, S, 64, P, P, need - 1, None) == -4
    assert L.dsa_topk(P, P, 1, 1, S, S, 64, P, ctypes.c_void_p(272), need, None) == -3


def test_projection_validation(L):
    """Absorption / up-projection: null, empty and misaligned arguments are
    rejected on the host."""
    for fn in (L.dsa_q_absorb, L.dsa_out_proj):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_void_p, ctypes.c_void_p]
        assert fn(None, P, 1, 1, P, None) == -1
        assert fn(P, P, 0, 1, P, None) == -1
        assert fn(P, P, 1, 0, P, None) == -1
        assert fn(P, ctypes.c_void_p(P.value + 8), 1, 1, P, None) == -3


def test_indexer_prep_validation(L):
    """Input preparation: null, empty, inconsistent, unsupported and misaligned
    arguments are rejected on the host before any launch."""
    fn = L.dsa_indexer_prep
    fn.restype = ctypes.c_int
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    fn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]

    def call(**over):
        a = dict(q=P, k=P, cos=P, sin=P, ep=P, B=1, T=1, S=16, dt=1, qo=P, qs=P, kc=P, ks=P)
        a.update(over)
        return fn(a["q"], a["k"], a["cos"], a["sin"], a["ep"], a["B"], a["T"], a["S"], a["dt"],
                  a["qo"], a["qs"], a["kc"], a["ks"], None)

    for name in ("q", "k", "cos", "sin", "ep", "qo", "kc"):
        assert call(**{name: None}) == -1, name
    assert call(qs=None) == -1 and call(ks=None) == -1          # fp8 needs both scales
    assert call(B=0) == -1 and call(T=0) == -1 and call(S=0) == -1
    assert call(T=17, S=16) == -1                                 # T > S_max
    assert call(B=1 << 13, T=1 << 12) == -1                       # B*T > 2^24
    assert call(dt=2) == -2
    for name in ("q", "k", "cos", "sin", "qo", "kc"):
        assert call(**{name: ctypes.c_void_p(P.value + 8)}) == -3, name
    assert call(ep=ODD) == -3 and call(qs=ODD) == -3 and call(ks=ODD) == -3


def test_mha_prefill_validation(L):
    """MHA prefill: null, empty, bad-scale, misaligned and short-workspace
    arguments are rejected on the host."""
    fn = L.dsa_sparse_mha_prefill
    fn.restype = ctypes.c_int
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    fn.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, ctypes.c_float, vp, vp, vp, ctypes.c_size_t, vp]
    L.dsa_sparse_mha_prefill_workspace_size.restype = ctypes.c_size_t
    L.dsa_sparse_mha_prefill_workspace_size.argtypes = [i32, i32]
    need = L.dsa_sparse_mha_prefill_workspace_size(1, 100)
    assert need == 4 * 4 * 256          # ceil(100/32) words x 256 padded queries
    assert L.dsa_sparse_mha_prefill_workspace_size(0, 100) == 0

    def call(**over):
        a = dict(q=P, kn=P, kp=P, v=P, idx=P, B=1, T=100, k=8, s=0.07, out=P, lse=None, ws=P,
                 nb=need)
        a.update(over)
        return fn(a["q"], a["kn"], a["kp"], a["v"], a["idx"], a["B"], a["T"], a["k"], a["s"],
                  a["out"], a["lse"], a["ws"], a["nb"], None)

    for name in ("q", "kn", "kp", "v", "idx", "out"):
        assert call(**{name: None}) == -1, name
    assert call(B=0) == -1 and call(T=0) == -1 and call(k=0) == -1
    assert call(s=0.0) == -1 and call(s=float("nan")) == -1
    assert call(nb=need - 1) == -4 and call(ws=None) == -1
    for name in ("q", "kn", "kp", "v", "out"):
        assert call(**{name: ctypes.c_void_p(P.value + 8)}) == -3, name
    assert call(idx=ODD) == -3 and call(lse=ODD) == -3
