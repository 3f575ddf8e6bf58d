"""DeepSeek Sparse Attention (DSA) decode hot path on AMD MI355X (gfx950).

Thin ctypes binding over ``libdsa.so`` (C ABI in ``include/dsa.h``).  The
functions here only check tensor dtype/device/contiguity/shape and pass raw
device pointers plus torch's current HIP stream; every step of the path runs
in the library's HIP kernels.  There is no fallback: if ``libdsa.so`` is
missing or cannot be loaded, every call raises.

Stages (same names as the C ABI, without the ``dsa_`` prefix):
  index_scores  lightning-indexer score, 64 heads x 128 dims, ReLU -> weight -> head sum
  topk          per-query top-k positions (ascending, ties to the smaller position, -1 pad)
  sparse_mla    absorbed MLA (128 heads, 512 latent + 64 rope) over the selected rows
  forward       the three stages on one stream
  forward_noalloc  the same with the workspace in the library's per-device scratch
  ForwardGraph  the forward step captured once into a HIP graph and replayed
  dense_mla     the same attention over every valid position (baseline)

Defaults that matter for capture and latency: without ``max_end_pos`` the
calls use S_max as the bound on end_pos (no device->host sync); without
``workspace`` (or ``out``) they take one from torch's caching allocator on
every call.  Passing both keeps a call free of syncs and allocations, so it
can be captured into a HIP graph.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

BF16 = 0
FP8_E4M3 = 1
INDEX_HEADS, INDEX_DIM = 64, 128
MLA_HEADS, LATENT_DIM, ROPE_DIM = 128, 512, 64
MAX_TOPK = 2048
SCRATCH_BYTES = 96 << 20  # DSA_FORWARD_SCRATCH_BYTES: dsa_forward_noalloc's per-device workspace

_lib = None


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def lib():
    """The loaded libdsa.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python sparse_attention_indexer_amd/_build.py")
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _bind(L):
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sig = {
        "dsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "dsa_index_scores": ([vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp, vp],
                             ctypes.c_int),
        "dsa_topk_workspace_size": ([i32, i32, i32, i32], sz),
        "dsa_topk": ([vp, vp, i32, i32, i32, i32, i32, vp, vp, sz, vp], ctypes.c_int),
        "dsa_sparse_mla_workspace_size": ([i32, i32, i32], sz),
        "dsa_sparse_mla": ([vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, sz, vp],
                           ctypes.c_int),
        "dsa_forward_workspace_size": ([i32, i32, i32, i32], sz),
        "dsa_forward": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                         f32, i32, vp, vp, vp, vp, sz, vp], ctypes.c_int),
        "dsa_forward_noalloc": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                 f32, f32, i32, vp, vp, vp, vp], ctypes.c_int),
        "dsa_dense_mla_workspace_size": ([i32, i32, i32], sz),
        "dsa_dense_mla": ([vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, sz, vp],
                          ctypes.c_int),
        "dsa_q_absorb": ([vp, vp, i32, i32, vp, vp], ctypes.c_int),
        "dsa_out_proj": ([vp, vp, i32, i32, vp, vp], ctypes.c_int),
        "dsa_sparse_mha_prefill_workspace_size": ([i32, i32], sz),
        "dsa_sparse_mha_prefill": ([vp, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp, sz, vp],
                                   ctypes.c_int),
        "dsa_indexer_prep": ([vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp],
                             ctypes.c_int),
        "dsa_forward_graph_create": ([vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                      i32, f32, f32, i32, vp, vp, vp, vp, sz,
                                      ctypes.POINTER(vp)], ctypes.c_int),
        "dsa_forward_graph_launch": ([vp, vp], ctypes.c_int),
        "dsa_forward_graph_destroy": ([vp], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


def status_string(status: int) -> str:
    return lib().dsa_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DsaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _max_end_pos(max_end_pos, S_max):
    # end_pos lives on the device and the grid needs a host bound.  Without the
    # caller's bound S_max serves (always valid, as end_pos <= S_max): no
    # device->host sync, only more workgroups that find nothing to do.
    return int(S_max) if max_end_pos is None else int(max_end_pos)


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        # The kernels need nothing in particular in it on entry.  This comes from
        # torch's caching allocator (a hipMalloc only when its pool is short);
        # pass a workspace to keep allocation out of the call altogether.
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace of {workspace.numel()} bytes < required {nbytes}")
    return workspace, workspace.numel() * workspace.element_size()


def index_scores(q, weights, k_cache, end_pos, scale, q_scale=None, k_scale=None,
                 max_end_pos=None, out=None, stream=None):
    """Indexer scores [B,T,S_max] fp32 (entries past each causal bound untouched)."""
    fp8 = q.dtype == torch.float8_e4m3fn
    B, T, H, D = q.shape
    S_max = k_cache.shape[1]
    dev = q.device
    _need(q, "q", (torch.bfloat16, torch.float8_e4m3fn), (B, T, INDEX_HEADS, INDEX_DIM))
    _need(weights, "weights", torch.float32, (B, T, INDEX_HEADS), dev)
    _need(k_cache, "k_cache", q.dtype, (B, S_max, INDEX_DIM), dev)
    _need(end_pos, "end_pos", torch.int32, (B,), dev)
    if fp8:
        _need(q_scale, "q_scale", torch.float32, (B, T, INDEX_HEADS), dev)
        _need(k_scale, "k_scale", torch.float32, (B, S_max), dev)
    if out is None:
        out = torch.empty((B, T, S_max), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, (B, T, S_max), dev)
    st = lib().dsa_index_scores(_ptr(q), _ptr(q_scale) if fp8 else None, _ptr(weights),
                                _ptr(k_cache), _ptr(k_scale) if fp8 else None, _ptr(end_pos),
                                B, T, S_max, _max_end_pos(max_end_pos, S_max), float(scale),
                                FP8_E4M3 if fp8 else BF16, _ptr(out), _stream(stream))
    _check(st, "dsa_index_scores")
    return out


def topk(index_score, end_pos, k=MAX_TOPK, max_end_pos=None, out=None, workspace=None,
         stream=None):
    """Top-k positions [B,T,k] int32: ascending, ties to the smaller position, -1 padded."""
    B, T, S_max = index_score.shape
    dev = index_score.device
    _need(index_score, "index_score", torch.float32)
    _need(end_pos, "end_pos", torch.int32, (B,), dev)
    if out is None:
        out = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    _need(out, "out", torch.int32, (B, T, k), dev)
    ws, nb = _workspace(lib().dsa_topk_workspace_size(B, T, S_max, k), dev, workspace)
    st = lib().dsa_topk(_ptr(index_score), _ptr(end_pos), B, T, S_max,
                        _max_end_pos(max_end_pos, S_max), int(k), _ptr(out), _ptr(ws), nb,
                        _stream(stream))
    _check(st, "dsa_topk")
    return out


def _mla_checks(q_nope, q_pe, kv_cache, pe_cache):
    B, T = q_nope.shape[:2]
    S_max = kv_cache.shape[1]
    dev = q_nope.device
    _need(q_nope, "q_nope", torch.bfloat16, (B, T, MLA_HEADS, LATENT_DIM))
    _need(q_pe, "q_pe", torch.bfloat16, (B, T, MLA_HEADS, ROPE_DIM), dev)
    _need(kv_cache, "kv_cache", torch.bfloat16, (B, S_max, LATENT_DIM), dev)
    _need(pe_cache, "pe_cache", torch.bfloat16, (B, S_max, ROPE_DIM), dev)
    return B, T, S_max, dev


def _mla_outputs(B, T, dev, out, lse, want_lse):
    if out is None:
        out = torch.empty((B, T, MLA_HEADS, LATENT_DIM), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (B, T, MLA_HEADS, LATENT_DIM), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, T, MLA_HEADS), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, T, MLA_HEADS), dev)
    return out, lse


def sparse_mla(q_nope, q_pe, kv_cache, pe_cache, topk_indices, softmax_scale, out=None,
               lse=None, want_lse=True, workspace=None, stream=None):
    """Absorbed MLA over the selected rows: (out [B,T,128,512] bf16, lse [B,T,128] fp32)."""
    B, T, S_max, dev = _mla_checks(q_nope, q_pe, kv_cache, pe_cache)
    k = topk_indices.shape[-1]
    _need(topk_indices, "topk_indices", torch.int32, (B, T, k), dev)
    out, lse = _mla_outputs(B, T, dev, out, lse, want_lse)
    ws, nb = _workspace(lib().dsa_sparse_mla_workspace_size(B, T, k), dev, workspace)
    st = lib().dsa_sparse_mla(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(pe_cache),
                              _ptr(topk_indices), B, T, S_max, k, float(softmax_scale),
                              _ptr(out), _ptr(lse), _ptr(ws), nb, _stream(stream))
    _check(st, "dsa_sparse_mla")
    return out, lse


def dense_mla(q_nope, q_pe, kv_cache, pe_cache, end_pos, softmax_scale, max_end_pos=None,
              out=None, lse=None, want_lse=True, workspace=None, stream=None):
    """Absorbed MLA over every causally valid position (the dense baseline)."""
    B, T, S_max, dev = _mla_checks(q_nope, q_pe, kv_cache, pe_cache)
    _need(end_pos, "end_pos", torch.int32, (B,), dev)
    out, lse = _mla_outputs(B, T, dev, out, lse, want_lse)
    ws, nb = _workspace(lib().dsa_dense_mla_workspace_size(B, T, S_max), dev, workspace)
    st = lib().dsa_dense_mla(_ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(pe_cache),
                             _ptr(end_pos), B, T, S_max, _max_end_pos(max_end_pos, S_max),
                             float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), nb,
                             _stream(stream))
    _check(st, "dsa_dense_mla")
    return out, lse


def q_absorb(q_nope, wkv_b, out=None, stream=None):
    """q_abs[b,t,h,:] = q_nope[b,t,h,:] @ wkv_b[h,:128,:]  ([B,T,128,128] -> [B,T,128,512])."""
    B, T = q_nope.shape[:2]
    dev = q_nope.device
    _need(q_nope, "q_nope", torch.bfloat16, (B, T, 128, 128), dev)
    _need(wkv_b, "wkv_b", torch.bfloat16, (128, 256, 512), dev)
    if out is None:
        out = torch.empty((B, T, 128, 512), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (B, T, 128, 512), dev)
    _check(lib().dsa_q_absorb(_ptr(q_nope), _ptr(wkv_b), B, T, _ptr(out), _stream(stream)),
           "dsa_q_absorb")
    return out


def out_proj(x, wkv_b, out=None, stream=None):
    """y[b,t,h,:] = x[b,t,h,:] @ wkv_b[h,128:,:]^T  ([B,T,128,512] -> [B,T,128,128])."""
    B, T = x.shape[:2]
    dev = x.device
    _need(x, "x", torch.bfloat16, (B, T, 128, 512), dev)
    _need(wkv_b, "wkv_b", torch.bfloat16, (128, 256, 512), dev)
    if out is None:
        out = torch.empty((B, T, 128, 128), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (B, T, 128, 128), dev)
    _check(lib().dsa_out_proj(_ptr(x), _ptr(wkv_b), B, T, _ptr(out), _stream(stream)),
           "dsa_out_proj")
    return out


def indexer_prep(q_in, k_in, rope_cos, rope_sin, end_pos, k_cache, k_scale=None, q_out=None,
                 q_scale=None, stream=None):
    """RoPE (rope dims first, non-interleaved), Hadamard rotation and, for an fp8
    cache, block-128 e4m3 quantisation of the indexer's query heads
    [B,T,64,128] and keys [B,T,128]; the keys go into k_cache [B,S_max,128]
    (and k_scale [B,S_max]) at rows end_pos[b]-T+t.  The cache's dtype picks
    the mode (bfloat16 or float8_e4m3fn).  Returns (q_out, q_scale); q_scale
    is None for bf16."""
    B, T = q_in.shape[:2]
    dev = q_in.device
    S_max = k_cache.shape[1] if k_cache.dim() == 3 else -1
    _need(q_in, "q_in", torch.bfloat16, (B, T, 64, 128), dev)
    _need(k_in, "k_in", torch.bfloat16, (B, T, 128), dev)
    _need(rope_cos, "rope_cos", torch.float32, (S_max, 32), dev)
    _need(rope_sin, "rope_sin", torch.float32, (S_max, 32), dev)
    _need(end_pos, "end_pos", torch.int32, (B,), dev)
    _need(k_cache, "k_cache", (torch.bfloat16, torch.float8_e4m3fn), (B, S_max, 128), dev)
    fp8 = k_cache.dtype == torch.float8_e4m3fn
    if q_out is None:
        q_out = torch.empty((B, T, 64, 128), dtype=k_cache.dtype, device=dev)
    _need(q_out, "q_out", k_cache.dtype, (B, T, 64, 128), dev)
    if fp8:
        if q_scale is None:
            q_scale = torch.empty((B, T, 64), dtype=torch.float32, device=dev)
        _need(q_scale, "q_scale", torch.float32, (B, T, 64), dev)
        _need(k_scale, "k_scale", torch.float32, (B, S_max), dev)
    else:
        q_scale = None
    _check(lib().dsa_indexer_prep(_ptr(q_in), _ptr(k_in), _ptr(rope_cos), _ptr(rope_sin),
                                  _ptr(end_pos), B, T, S_max, 1 if fp8 else 0, _ptr(q_out),
                                  _ptr(q_scale), _ptr(k_cache),
                                  _ptr(k_scale) if fp8 else None, _stream(stream)),
           "dsa_indexer_prep")
    return q_out, q_scale


def sparse_mha_prefill(q, k_nope, k_pe, v, topk_indices, softmax_scale, out=None, lse=None,
                       want_lse=True, workspace=None, stream=None):
    """MHA-form prefill attention (per-head keys/values, index and causal masks):
    (out [B,T,128,128] bf16, lse [B,T,128] fp32 or None)."""
    B, T = q.shape[:2]
    dev = q.device
    k = topk_indices.shape[-1]
    _need(q, "q", torch.bfloat16, (B, T, 128, 192), dev)
    _need(k_nope, "k_nope", torch.bfloat16, (B, T, 128, 128), dev)
    _need(k_pe, "k_pe", torch.bfloat16, (B, T, 64), dev)
    _need(v, "v", torch.bfloat16, (B, T, 128, 128), dev)
    _need(topk_indices, "topk_indices", torch.int32, (B, T, k), dev)
    if out is None:
        out = torch.empty((B, T, 128, 128), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (B, T, 128, 128), dev)
    if want_lse and lse is None:
        lse = torch.empty((B, T, 128), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, T, 128), dev)
    L = lib()
    workspace, nbytes = _workspace(int(L.dsa_sparse_mha_prefill_workspace_size(B, T)), dev,
                                   workspace)
    _check(L.dsa_sparse_mha_prefill(_ptr(q), _ptr(k_nope), _ptr(k_pe), _ptr(v), _ptr(topk_indices),
                                    B, T, k, float(softmax_scale), _ptr(out), _ptr(lse),
                                    _ptr(workspace), nbytes, _stream(stream)),
           "dsa_sparse_mha_prefill")
    return out, lse


def forward_workspace_size(B, T, S_max, k=MAX_TOPK) -> int:
    return int(lib().dsa_forward_workspace_size(B, T, S_max, k))


def forward(q, weights, k_cache, end_pos, q_nope, q_pe, kv_cache, pe_cache, index_scale,
            softmax_scale, k=MAX_TOPK, q_scale=None, k_scale=None, max_end_pos=None, out=None,
            lse=None, want_lse=True, topk_out=None, workspace=None, stream=None):
    """Indexer -> top-k -> sparse MLA on one stream.  Returns (out, lse, topk_out)."""
    fp8 = q.dtype == torch.float8_e4m3fn
    B, T = q.shape[:2]
    S_max = k_cache.shape[1]
    dev = q.device
    _need(q, "q", (torch.bfloat16, torch.float8_e4m3fn), (B, T, INDEX_HEADS, INDEX_DIM))
    _need(weights, "weights", torch.float32, (B, T, INDEX_HEADS), dev)
    _need(k_cache, "k_cache", q.dtype, (B, S_max, INDEX_DIM), dev)
    _need(end_pos, "end_pos", torch.int32, (B,), dev)
    if fp8:
        _need(q_scale, "q_scale", torch.float32, (B, T, INDEX_HEADS), dev)
        _need(k_scale, "k_scale", torch.float32, (B, S_max), dev)
    Bm, Tm, S_kv, _ = _mla_checks(q_nope, q_pe, kv_cache, pe_cache)
    if (Bm, Tm, S_kv) != (B, T, S_max):
        raise ValueError("indexer and attention tensors disagree on B, T or S_max")
    out, lse = _mla_outputs(B, T, dev, out, lse, want_lse)
    if topk_out is not None:
        _need(topk_out, "topk_out", torch.int32, (B, T, k), dev)
    ws, nb = _workspace(forward_workspace_size(B, T, S_max, k), dev, workspace)
    st = lib().dsa_forward(_ptr(q), _ptr(q_scale) if fp8 else None, _ptr(weights),
                           _ptr(k_cache), _ptr(k_scale) if fp8 else None, _ptr(end_pos),
                           _ptr(q_nope), _ptr(q_pe), _ptr(kv_cache), _ptr(pe_cache), B, T, S_max,
                           _max_end_pos(max_end_pos, S_max), int(k), float(index_scale),
                           float(softmax_scale), FP8_E4M3 if fp8 else BF16, _ptr(out),
                           _ptr(lse), _ptr(topk_out), _ptr(ws), nb, _stream(stream))
    _check(st, "dsa_forward")
    return out, lse, topk_out


def forward_noalloc(q, weights, k_cache, end_pos, q_nope, q_pe, kv_cache, pe_cache, index_scale,
                    softmax_scale, k=MAX_TOPK, q_scale=None, k_scale=None, max_end_pos=None,
                    out=None, lse=None, want_lse=True, topk_out=None, stream=None):
    """forward() through dsa_forward_noalloc: the workspace is the library's
    per-device scratch (at most SCRATCH_BYTES), so with ``out`` (and ``lse``)
    given the call allocates nothing.  Calls that overlap on one GPU race."""
    fp8 = q.dtype == torch.float8_e4m3fn
    B, T = q.shape[:2]
    S_max = k_cache.shape[1]
    dev = q.device
    _need(q, "q", (torch.bfloat16, torch.float8_e4m3fn), (B, T, INDEX_HEADS, INDEX_DIM))
    _need(weights, "weights", torch.float32, (B, T, INDEX_HEADS), dev)
    _need(k_cache, "k_cache", q.dtype, (B, S_max, INDEX_DIM), dev)
    _need(end_pos, "end_pos", torch.int32, (B,), dev)
    if fp8:
        _need(q_scale, "q_scale", torch.float32, (B, T, INDEX_HEADS), dev)
        _need(k_scale, "k_scale", torch.float32, (B, S_max), dev)
    Bm, Tm, S_kv, _ = _mla_checks(q_nope, q_pe, kv_cache, pe_cache)
    if (Bm, Tm, S_kv) != (B, T, S_max):
        raise ValueError("indexer and attention tensors disagree on B, T or S_max")
    out, lse = _mla_outputs(B, T, dev, out, lse, want_lse)
    if topk_out is not None:
        _need(topk_out, "topk_out", torch.int32, (B, T, k), dev)
    with torch.cuda.device(dev):
        st = lib().dsa_forward_noalloc(
            _ptr(q), _ptr(q_scale) if fp8 else None, _ptr(weights), _ptr(k_cache),
            _ptr(k_scale) if fp8 else None, _ptr(end_pos), _ptr(q_nope), _ptr(q_pe),
            _ptr(kv_cache), _ptr(pe_cache), B, T, S_max, _max_end_pos(max_end_pos, S_max),
            int(k), float(index_scale), float(softmax_scale), FP8_E4M3 if fp8 else BF16,
            _ptr(out), _ptr(lse), _ptr(topk_out), _stream(stream))
    _check(st, "dsa_forward_noalloc")
    return out, lse, topk_out


class ForwardGraph:
    """The decode step captured once (dsa_forward_graph_create) and replayed
    with launch(): the tensors are bound at construction, so a serving loop
    rewrites their contents in place between steps.  Keeps references to
    every bound tensor (the graph reads them at each replay)."""

    def __init__(self, q, weights, k_cache, end_pos, q_nope, q_pe, kv_cache, pe_cache,
                 index_scale, softmax_scale, out, lse, topk_out, workspace, k=MAX_TOPK,
                 q_scale=None, k_scale=None, max_end_pos=None):
        fp8 = q.dtype == torch.float8_e4m3fn
        B, T = q.shape[:2]
        S_max = k_cache.shape[1]
        dev = q.device
        _need(q, "q", (torch.bfloat16, torch.float8_e4m3fn), (B, T, INDEX_HEADS, INDEX_DIM))
        _need(weights, "weights", torch.float32, (B, T, INDEX_HEADS), dev)
        _need(k_cache, "k_cache", q.dtype, (B, S_max, INDEX_DIM), dev)
        _need(end_pos, "end_pos", torch.int32, (B,), dev)
        if fp8:
            _need(q_scale, "q_scale", torch.float32, (B, T, INDEX_HEADS), dev)
            _need(k_scale, "k_scale", torch.float32, (B, S_max), dev)
        Bm, Tm, S_kv, _ = _mla_checks(q_nope, q_pe, kv_cache, pe_cache)
        if (Bm, Tm, S_kv) != (B, T, S_max):
            raise ValueError("indexer and attention tensors disagree on B, T or S_max")
        _need(out, "out", torch.bfloat16, (B, T, MLA_HEADS, LATENT_DIM), dev)
        if lse is not None:
            _need(lse, "lse", torch.float32, (B, T, MLA_HEADS), dev)
        if topk_out is not None:
            _need(topk_out, "topk_out", torch.int32, (B, T, k), dev)
        _need(workspace, "workspace", torch.uint8, None, dev)
        nb = workspace.numel()
        if nb < forward_workspace_size(B, T, S_max, k):
            raise ValueError(f"workspace of {nb} bytes < required "
                             f"{forward_workspace_size(B, T, S_max, k)}")
        self._keep = (q, weights, k_cache, end_pos, q_nope, q_pe, kv_cache, pe_cache, out, lse,
                      topk_out, workspace, q_scale, k_scale)
        self._h = ctypes.c_void_p()
        self._lib = lib()
        with torch.cuda.device(dev):
            st = self._lib.dsa_forward_graph_create(
                _ptr(q), _ptr(q_scale) if fp8 else None, _ptr(weights), _ptr(k_cache),
                _ptr(k_scale) if fp8 else None, _ptr(end_pos), _ptr(q_nope), _ptr(q_pe),
                _ptr(kv_cache), _ptr(pe_cache), B, T, S_max, _max_end_pos(max_end_pos, S_max),
                int(k), float(index_scale), float(softmax_scale), FP8_E4M3 if fp8 else BF16,
                _ptr(out), _ptr(lse), _ptr(topk_out), _ptr(workspace), nb,
                ctypes.byref(self._h))
        _check(st, "dsa_forward_graph_create")

    def launch(self, stream=None):
        """Enqueue one replay of the captured step."""
        if not self._h:
            raise RuntimeError("the graph has been destroyed")
        _check(self._lib.dsa_forward_graph_launch(self._h, _stream(stream)),
               "dsa_forward_graph_launch")

    def close(self):
        """Release the graph (no replay may still be pending)."""
        if self._h:
            _check(self._lib.dsa_forward_graph_destroy(self._h), "dsa_forward_graph_destroy")
            self._h = ctypes.c_void_p()
        self._keep = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def forward_case(case, out=None, lse=None, topk_out=None, workspace=None, stream=None):
    """dsa_forward on an inputs.Case already on the device."""
    return forward(case.q, case.w, case.k_cache, case.end_pos, case.q_nope, case.q_pe,
                   case.kv_cache, case.pe_cache, case.scale, case.softmax_scale, k=case.topk,
                   q_scale=case.q_scale, k_scale=case.k_scale, max_end_pos=case.max_end_pos,
                   out=out, lse=lse, topk_out=topk_out, workspace=workspace, stream=stream)
