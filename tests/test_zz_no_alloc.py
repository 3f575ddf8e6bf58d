"""dsa_forward_noalloc (workspace in the library's per-device scratch) against
dsa_forward with a caller workspace: identical outputs, on consecutive calls
of decreasing size that reuse the scratch.  (The size limit, checked before
anything is launched, is tested on the CPU with the other ABI checks.)"""
import pytest
import torch

import sparse_attention_indexer_amd as dsa
from sparse_attention_indexer_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(case):
    """(forward with its own workspace, forward_noalloc) on the same inputs."""
    B, T, k = case.B, case.T, case.topk
    mep = case.max_end_pos
    outs = []
    for fn in (dsa.forward, dsa.forward_noalloc):
        out = torch.full((B, T, 128, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((B, T, 128), float("nan"), dtype=torch.float32, device=DEV)
        idx = torch.full((B, T, k), -7, dtype=torch.int32, device=DEV)
        fn(case.q, case.w, case.k_cache, case.end_pos, case.q_nope, case.q_pe, case.kv_cache,
           case.pe_cache, case.scale, case.softmax_scale, k=k, q_scale=case.q_scale,
           k_scale=case.k_scale, max_end_pos=mep, out=out, lse=lse, topk_out=idx)
        torch.cuda.synchronize()
        outs.append((out, lse, idx))
    return outs


def _same(a, b):
    (o1, l1, i1), (o2, l2, i2) = a, b
    assert torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_noalloc_matches_forward_on_shrinking_calls():
    # First call: batch 8 at 65536 positions (fp8 indexer, a 38 MiB workspace);
    # second: one query at 32768 (bf16, 4.4 MiB); third: the short-context
    # case that keeps every position (1001 < k).  Each reuses the scratch the
    # previous call left behind.
    cases = [inputs.sweep(65536, device=DEV), inputs.decode_32k(device=DEV),
             inputs.tiny_decode("short", device=DEV)]
    sizes = [dsa.forward_workspace_size(c.B, c.T, c.S_max, c.topk) for c in cases]
    assert sizes[0] > sizes[1] > sizes[2]
    assert sizes[0] <= dsa.SCRATCH_BYTES
    for c in cases:
        a, b = _both(c)
        assert not torch.isnan(b[0].float()).any()
        _same(a, b)


def test_noalloc_repeat_is_identical():
    # The same call twice in a row on one stream gives the same bits.
    c = inputs.decode_32k(device=DEV, n=20000)
    _, b1 = _both(c)
    _, b2 = _both(c)
    _same(b1, b2)


def test_noalloc_captured_in_a_graph():
    # The callers this entry point is for capture it: each replay, with other
    # no-allocation calls on other inputs in between (which reuse the same
    # scratch), gives the eager result bit for bit.
    case = inputs.make_case("noalloc_graph", 2, 1, [6000, 3500], 6000, seed=31, device=DEV)
    other = inputs.make_case("noalloc_other", 2, 1, [6000, 5200], 6000, seed=32, device=DEV)
    B, T, k = case.B, case.T, case.topk
    out = torch.empty((B, T, 128, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, T, 128), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)

    def run(c):
        dsa.forward_noalloc(c.q, c.w, c.k_cache, c.end_pos, c.q_nope, c.q_pe, c.kv_cache,
                            c.pe_cache, c.scale, c.softmax_scale, k=k, max_end_pos=c.S_max,
                            out=out, lse=lse, topk_out=idx)

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
        run(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(ref, (out, lse, idx))
