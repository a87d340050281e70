"""Python binding of the MI355X fused exact-attention library (include/fa.h).

Thin ctypes marshalling only: every step of the computation runs in the HIP
kernels of libfa.so.  The functions keep the C names:

    fa_fwd(q, k, v, ...)                 dense prefill forward
    fa_fwd_varlen(q, k, v, cu_q, cu_k, ...)  packed varlen prefill
    fa_decode_paged(q, k_cache, v_cache, block_table, cache_seqlens, ...)
    fa_decode_paged_workspace_size(...)

Tensors are torch CUDA(HIP) tensors used purely as device memory; work is
enqueued on torch's current stream.  There is no CPU fallback: if libfa.so is
missing or no GPU is present the calls raise.
"""

import ctypes
import math
import os

import numpy as np

from .build import LIB_PATH

FA_OK = 0
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
           3: "decode workspace missing or too small", 4: "HIP kernel launch failed"}

_lib = None

# softcap, alibi_slopes, alibi_batch_stride (prefill entry points)
_MODS = [ctypes.c_float, ctypes.c_void_p, ctypes.c_int]

_EXPORTS = {
    "fa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fa_fwd": (ctypes.c_int, [ctypes.c_void_p] * 4 + [ctypes.c_void_p]
               + [ctypes.c_int] * 6 + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int]
               + _MODS + [ctypes.c_void_p]),
    "fa_fwd_varlen": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_void_p] * 2
                      + [ctypes.c_int] * 8 + [ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int] + _MODS + [ctypes.c_void_p]),
    "fa_varlen_plan": (ctypes.c_int, [ctypes.c_void_p] * 2 + [ctypes.c_int] * 4
                       + [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "fa_fwd_varlen_run": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_void_p] * 3
                          + [ctypes.c_int] * 9 + [ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_int] + _MODS + [ctypes.c_void_p]),
    "fa_decode_paged_workspace_size": (ctypes.c_size_t, [ctypes.c_int] * 6),
    "fa_bwd_workspace_size": (ctypes.c_size_t, [ctypes.c_int] * 3),
    "fa_bwd_varlen_workspace_size": (ctypes.c_size_t, [ctypes.c_int] * 3),
    "fa_bwd_varlen": (ctypes.c_int, [ctypes.c_void_p] * 11 + [ctypes.c_int] * 8
                      + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_bwd": (ctypes.c_int, [ctypes.c_void_p] * 9 + [ctypes.c_int] * 6
               + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_decode_plan": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.c_int] * 5
                       + [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "fa_decode_paged_run": (ctypes.c_int, [ctypes.c_void_p] * 6 + [ctypes.c_int]
                            + [ctypes.c_void_p] * 2 + [ctypes.c_int] * 7
                            + [ctypes.c_float, ctypes.c_int] + _MODS
                            + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_decode_paged": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_void_p] * 2
                        + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int] + _MODS
                        + [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "fa_fwd_kvcache": (ctypes.c_int, [ctypes.c_void_p] * 9 + [ctypes.c_int] * 8
                       + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int]
                       + _MODS + [ctypes.c_void_p]),
}


class FAError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {_STATUS.get(status, 'unknown')} (status {status})")
        self.status = status


def load_library(path=None):
    """Load libfa.so (built by exact_attention_17_amd.build); raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m exact_attention_17_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols():
    return list(_EXPORTS)


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != FA_OK:
        raise FAError(fn, status)


def _need(t, name, dtype=None, ndim=None, device=True):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def cu_seqlens_from_lengths(lengths):
    """Host helper: per-sequence lengths -> cumulative offsets of length B+1
    (lengths [100, 200, 150] -> [0, 100, 300, 450])."""
    lengths = np.asarray(lengths, dtype=np.int64)
    if lengths.ndim != 1 or (lengths < 0).any():
        raise ValueError("lengths must be a 1-D array of non-negative integers")
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    if cu[-1] >= 2 ** 31:
        raise ValueError("total length exceeds int32")
    return cu.astype(np.int32)


def lengths_from_cu_seqlens(cu):
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or len(cu) < 1 or cu[0] != 0 or (np.diff(cu) < 0).any():
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    return np.diff(cu).astype(np.int32)


def _mods(softcap, alibi_slopes, B, Hq):
    """(softcap, slopes pointer, batch stride) for the C call; slopes is a float32
    device tensor of shape (Hq,) or (B, Hq), or None."""
    if alibi_slopes is None:
        return float(softcap), None, 0
    torch = _torch()
    _need(alibi_slopes, "alibi_slopes", torch.float32)
    if tuple(alibi_slopes.shape) == (Hq,):
        return float(softcap), _ptr(alibi_slopes), 0
    if tuple(alibi_slopes.shape) == (B, Hq):
        return float(softcap), _ptr(alibi_slopes), Hq
    raise ValueError("alibi_slopes must be (Hq,) or (B, Hq)")


def fa_fwd(q, k, v, softmax_scale=None, causal=False, window=(-1, -1), out=None,
           lse=None, return_lse=True, stream=None, softcap=0.0, alibi_slopes=None):
    """Dense prefill: q (B, Lq, Hq, d), k/v (B, Lk, Hkv, d) bf16 -> O, LSE (B, Hq, Lq).
    softcap > 0 caps the logits (c*tanh(x/c)); alibi_slopes (Hq,) or (B, Hq)
    float32 adds -slope*|i + Lk - Lq - j|."""
    torch = _torch()
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 4)
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Lk, Hkv, d) or tuple(v.shape) != (B, Lk, Hkv, d):
        raise ValueError("k and v must be (B, Lk, Hkv, d) matching q")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, 4)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
    st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Lq, Lk, Hq, Hkv, d,
                    scale, int(bool(causal)), int(window[0]), int(window[1]),
                    *_mods(softcap, alibi_slopes, B, Hq), _stream(stream))
    _check("fa_fwd", st)
    return out, lse


def _varlen_args(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, out, lse, return_lse):
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 3)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if tuple(v.shape) != (total_k, Hkv, d) or k.shape[2] != d:
        raise ValueError("k and v must be (total_k, Hkv, d)")
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    return out, lse, B, total_q, total_k, Hq, Hkv, d, scale


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  softmax_scale=None, causal=False, window=(-1, -1), out=None, lse=None,
                  return_lse=True, stream=None, softcap=0.0, alibi_slopes=None):
    """Packed varlen prefill: q (total_q, Hq, d), k/v (total_k, Hkv, d), cu_seqlens int32
    device tensors of length B+1 -> O, LSE (Hq, total_q)."""
    lib = load_library()
    out, lse, B, total_q, total_k, Hq, Hkv, d, scale = _varlen_args(
        q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, out, lse, return_lse)
    st = lib.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                           _ptr(cu_seqlens_k), B, int(max_seqlen_q), int(max_seqlen_k), total_q,
                           total_k, Hq, Hkv, d, scale, int(bool(causal)), int(window[0]),
                           int(window[1]), *_mods(softcap, alibi_slopes, B, Hq),
                           _stream(stream))
    _check("fa_fwd_varlen", st)
    return out, lse


def fa_varlen_plan(cu_seqlens_q, cu_seqlens_k, causal=False, window=(-1, -1)):
    """Host plan for fa_fwd_varlen_run from HOST cumulative lengths (lists, numpy arrays or
    CPU tensors of B+1 ints) -> numpy int32 array (num_items, 2) of (sequence, query tile),
    heaviest first.  No GPU is needed."""
    import numpy as np
    lib = load_library()
    cq = np.ascontiguousarray(np.asarray(cu_seqlens_q, dtype=np.int64)).astype(np.int32)
    ck = np.ascontiguousarray(np.asarray(cu_seqlens_k, dtype=np.int64)).astype(np.int32)
    if cq.ndim != 1 or ck.shape != cq.shape or cq.size < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D of the same length >= 2")
    B = cq.size - 1
    n = ctypes.c_int(0)
    args = (cq.ctypes.data_as(ctypes.c_void_p), ck.ctypes.data_as(ctypes.c_void_p), B,
            int(bool(causal)), int(window[0]), int(window[1]))
    _check("fa_varlen_plan", lib.fa_varlen_plan(*args, None, 0, ctypes.byref(n)))
    plan = np.zeros((max(n.value, 1), 2), dtype=np.int32)
    _check("fa_varlen_plan", lib.fa_varlen_plan(*args, plan.ctypes.data_as(ctypes.c_void_p),
                                                 n.value, ctypes.byref(n)))
    return plan[:n.value]


def fa_fwd_varlen_run(q, k, v, cu_seqlens_q, cu_seqlens_k, plan, max_seqlen_q, max_seqlen_k,
                      softmax_scale=None, causal=False, window=(-1, -1), out=None, lse=None,
                      return_lse=True, stream=None, softcap=0.0, alibi_slopes=None):
    """fa_fwd_varlen in the order of a plan from fa_varlen_plan (same lengths, causal flag and
    window), uploaded as a device int32 tensor (num_items, 2)."""
    torch = _torch()
    lib = load_library()
    _need(plan, "plan", torch.int32, 2)
    if plan.shape[1] != 2:
        raise ValueError("plan must be (num_items, 2)")
    out, lse, B, total_q, total_k, Hq, Hkv, d, scale = _varlen_args(
        q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, out, lse, return_lse)
    st = lib.fa_fwd_varlen_run(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                               _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(plan),
                               plan.shape[0], B, int(max_seqlen_q), int(max_seqlen_k), total_q,
                               total_k, Hq, Hkv, d, scale, int(bool(causal)), int(window[0]),
                               int(window[1]), *_mods(softcap, alibi_slopes, B, Hq),
                               _stream(stream))
    _check("fa_fwd_varlen_run", st)
    return out, lse


def fa_decode_paged_workspace_size(B, Hq, d, max_blocks_per_seq, page_size, split_tokens=0):
    return int(load_library().fa_decode_paged_workspace_size(B, Hq, d, max_blocks_per_seq,
                                                              page_size, split_tokens))


def _decode_args(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale, split_tokens,
                 out, lse, workspace, return_lse):
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, one, Hq, d = q.shape
    if one != 1:
        raise ValueError("q must be (B, 1, Hq, d)")
    num_pages, page_size, Hkv, dk = k_cache.shape
    if dk != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [num_pages, page_size, Hkv, d]")
    if block_table.shape[0] != B or cache_seqlens.shape[0] != B:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    max_blocks = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    need = fa_decode_paged_workspace_size(B, Hq, d, max_blocks, page_size, split_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    return out, lse, workspace, B, Hq, Hkv, d, num_pages, page_size, max_blocks, scale


def fa_decode_paged(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale=None,
                    window_left=-1, split_tokens=0, out=None, lse=None, workspace=None,
                    return_lse=True, stream=None, softcap=0.0, alibi_slopes=None):
    """Paged decode: q (B, 1, Hq, d), caches [num_pages, page_size, Hkv, d],
    block_table int32 [B, max_blocks], cache_seqlens int32 [B] -> O, LSE (B, Hq).
    softcap / alibi_slopes ((Hq,) or (B, Hq) float32) as for fa_fwd; the query sits
    at position cache_seqlens[b] - 1."""
    lib = load_library()
    out, lse, workspace, B, Hq, Hkv, d, num_pages, page_size, max_blocks, scale = _decode_args(
        q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale, split_tokens, out, lse,
        workspace, return_lse)
    st = lib.fa_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                             _ptr(cache_seqlens), _ptr(out), _ptr(lse), B, Hq, Hkv, d, num_pages,
                             page_size, max_blocks, scale, int(window_left),
                             *_mods(softcap, alibi_slopes, B, Hq), int(split_tokens),
                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream))
    _check("fa_decode_paged", st)
    return out, lse


def fa_decode_plan(cache_seqlens, page_size, max_blocks_per_seq, window_left=-1, split_tokens=0):
    """Host plan for fa_decode_paged_run from HOST lengths (list, numpy array or CPU tensor of
    B ints) -> numpy int32 array (num_items, 2) of (request, split), heaviest first.  No GPU is
    needed."""
    import numpy as np
    lib = load_library()
    sl = np.ascontiguousarray(np.asarray(cache_seqlens, dtype=np.int64)).astype(np.int32)
    if sl.ndim != 1 or sl.size < 1:
        raise ValueError("cache_seqlens must be 1-D with at least one request")
    n = ctypes.c_int(0)
    args = (sl.ctypes.data_as(ctypes.c_void_p), sl.size, int(page_size), int(max_blocks_per_seq),
            int(window_left), int(split_tokens))
    _check("fa_decode_plan", lib.fa_decode_plan(*args, None, 0, ctypes.byref(n)))
    plan = np.zeros((max(n.value, 1), 2), dtype=np.int32)
    _check("fa_decode_plan", lib.fa_decode_plan(*args, plan.ctypes.data_as(ctypes.c_void_p),
                                                 n.value, ctypes.byref(n)))
    return plan[:n.value]


def fa_decode_paged_run(q, k_cache, v_cache, block_table, cache_seqlens, plan,
                        softmax_scale=None, window_left=-1, split_tokens=0, out=None, lse=None,
                        workspace=None, return_lse=True, stream=None, softcap=0.0,
                        alibi_slopes=None):
    """fa_decode_paged over the items of a plan from fa_decode_plan (same lengths, page size,
    block-table width, window and split size), uploaded as a device int32 tensor
    (num_items, 2)."""
    torch = _torch()
    lib = load_library()
    _need(plan, "plan", torch.int32, 2)
    if plan.shape[1] != 2:
        raise ValueError("plan must be (num_items, 2)")
    out, lse, workspace, B, Hq, Hkv, d, num_pages, page_size, max_blocks, scale = _decode_args(
        q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale, split_tokens, out, lse,
        workspace, return_lse)
    st = lib.fa_decode_paged_run(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                 _ptr(cache_seqlens), _ptr(plan), plan.shape[0], _ptr(out),
                                 _ptr(lse), B, Hq, Hkv, d, num_pages, page_size, max_blocks,
                                 scale, int(window_left), *_mods(softcap, alibi_slopes, B, Hq),
                                 int(split_tokens), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _check("fa_decode_paged_run", st)
    return out, lse


def fa_bwd_workspace_size(B, Hq, Lq):
    return int(load_library().fa_bwd_workspace_size(B, Hq, Lq))


def fa_bwd(q, k, v, out, lse, dout, softmax_scale=None, causal=False, window=(-1, -1),
           dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward of fa_fwd: q, out, dout (B, Lq, Hq, d), k, v (B, Lk, Hkv, d) bf16, lse
    (B, Hq, Lq) float32 from fa_fwd -> dq, dk, dv (bf16, shapes of q, k, v)."""
    torch = _torch()
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, nm, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, Lq, Hq, d = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Lk, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be (B, Lk, Hkv, d)")
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("out and dout must have q's shape")
    if tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("lse must be (B, Hq, Lq)")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        need = fa_bwd_workspace_size(B, Hq, Lq)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                    _ptr(dk), _ptr(dv), B, Lq, Lk, Hq, Hkv, d, scale, int(bool(causal)),
                    int(window[0]), int(window[1]), _ptr(workspace),
                    workspace.numel() * workspace.element_size(), _stream(stream))
    _check("fa_bwd", st)
    return dq, dk, dv


def fa_bwd_varlen_workspace_size(B, Hq, total_q):
    return int(load_library().fa_bwd_varlen_workspace_size(B, Hq, total_q))


def fa_bwd_varlen(q, k, v, out, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                  max_seqlen_k, softmax_scale=None, causal=False, window=(-1, -1), dq=None,
                  dk=None, dv=None, workspace=None, stream=None):
    """Backward of fa_fwd_varlen: q, out, dout (total_q, Hq, d), k, v (total_k, Hkv, d),
    lse (Hq, total_q) from fa_fwd_varlen, cu_seqlens int32 device tensors -> dq, dk, dv."""
    torch = _torch()
    lib = load_library()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, nm, torch.bfloat16, 3)
    _need(lse, "lse", torch.float32, 2)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if tuple(k.shape) != (total_k, Hkv, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be (total_k, Hkv, d)")
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("out and dout must have q's shape")
    if tuple(lse.shape) != (Hq, total_q):
        raise ValueError("lse must be (Hq, total_q)")
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        need = fa_bwd_varlen_workspace_size(B, Hq, total_q)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = lib.fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B,
                           int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, Hq, Hkv, d,
                           scale, int(bool(causal)), int(window[0]), int(window[1]),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream(stream))
    _check("fa_bwd_varlen", st)
    return dq, dk, dv


def fa_fwd_kvcache(q, k_cache, v_cache, block_table, cache_seqlens, k_new=None, v_new=None,
                   softmax_scale=None, causal=True, window=(-1, -1), out=None, lse=None,
                   return_lse=True, stream=None, softcap=0.0, alibi_slopes=None):
    """Chunked prefill over a paged KV cache: q (B, Lq, Hq, d) attends to each
    request's cache_seqlens[b] cached keys, after k_new / v_new (B, Lq, Hkv, d),
    if given, are written into the caches at positions cache_seqlens[b] + i
    (in place; cache_seqlens is not changed).  Caches [num_pages, page_size,
    Hkv, d] with page_size a multiple of 16.  Returns O (B, Lq, Hq, d) and LSE
    (B, Hq, Lq)."""
    torch = _torch()
    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, Lq, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = k_cache.shape
    if dk != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [num_pages, page_size, Hkv, d]")
    if block_table.shape[0] != B or cache_seqlens.shape[0] != B:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        _need(k_new, "k_new", torch.bfloat16, 4)
        _need(v_new, "v_new", torch.bfloat16, 4)
        if tuple(k_new.shape) != (B, Lq, Hkv, d) or tuple(v_new.shape) != (B, Lq, Hkv, d):
            raise ValueError("k_new / v_new must be (B, Lq, Hkv, d)")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    wl, wr = window
    st = lib.fa_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                            _ptr(block_table), _ptr(cache_seqlens), _ptr(out), _ptr(lse),
                            B, Lq, Hq, Hkv, d, num_pages, page_size, block_table.shape[1],
                            scale, int(bool(causal)), int(wl), int(wr),
                            *_mods(softcap, alibi_slopes, B, Hq), _stream(stream))
    _check("fa_fwd_kvcache", st)
    return out, lse


__all__ = ["fa_fwd", "fa_fwd_varlen", "fa_varlen_plan", "fa_fwd_varlen_run",
           "fa_decode_paged", "fa_decode_plan", "fa_decode_paged_run",
           "fa_decode_paged_workspace_size", "fa_fwd_kvcache", "fa_bwd",
           "fa_bwd_workspace_size", "fa_bwd_varlen", "fa_bwd_varlen_workspace_size",
           "load_library", "exported_symbols", "cu_seqlens_from_lengths",
           "lengths_from_cu_seqlens", "FAError", "LIB_PATH"]
