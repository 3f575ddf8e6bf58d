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
