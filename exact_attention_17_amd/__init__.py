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
    "fa_decode_paged_noalloc": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_void_p] * 2
                                + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int] + _MODS
                                + [ctypes.c_int, ctypes.c_void_p]),
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


def _stream_obj(stream):
    return stream if stream is not None else _torch().cuda.current_stream()


def _stream(s):
    """The HIP stream handle of a torch stream object."""
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != FA_OK:
        raise FAError(fn, status)


def _is_device(t):
    return t.is_cuda


def _need(t, name, dtype=None, ndim=None, shape=None, device=None):
    """Validate a tensor handed to the C ABI, which sees only its pointer: it must be
    a contiguous device tensor of the given dtype, rank and exact shape, on the same
    device as the call's other tensors."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not _is_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _output(t, name, shape, dtype, device, s):
    """A caller's output buffer, checked against the exact shape the call writes, or a
    new one.  New buffers are allocated on the launch stream s, so torch's caching
    allocator does not hand their memory to other streams while the kernels run."""
    if t is None:
        torch = _torch()
        with torch.cuda.stream(s):
            return torch.empty(tuple(shape), dtype=dtype, device=device)
    _need(t, name, dtype, shape=shape, device=device)
    return t


def _workspace(t, need, device, s):
    """A caller's workspace (any dtype, contiguous, on the device, at least `need`
    bytes) or a new one on the launch stream; returns (tensor, size in bytes)."""
    torch = _torch()
    if t is None:
        with torch.cuda.stream(s):
            t = torch.empty(max(int(need), 256), dtype=torch.uint8, device=device)
    else:
        _need(t, "workspace", device=device)
        if t.numel() * t.element_size() < need:
            raise ValueError(f"workspace holds {t.numel() * t.element_size()} bytes, "
                             f"the call needs {need}")
    return t, t.numel() * t.element_size()


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


def _mods(softcap, alibi_slopes, B, Hq, device):
    """(softcap, slopes pointer, batch stride) for the C call; slopes is a float32
    device tensor of shape (Hq,) or (B, Hq), or None."""
    if alibi_slopes is None:
        return float(softcap), None, 0
    torch = _torch()
    _need(alibi_slopes, "alibi_slopes", torch.float32, device=device)
    if tuple(alibi_slopes.shape) == (Hq,):
        return float(softcap), _ptr(alibi_slopes), 0
    if tuple(alibi_slopes.shape) == (B, Hq):
        return float(softcap), _ptr(alibi_slopes), Hq
    raise ValueError("alibi_slopes must be (Hq,) or (B, Hq)")


def _scale(softmax_scale, d):
    return 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)


def fa_fwd(q, k, v, softmax_scale=None, causal=False, window=(-1, -1), out=None,
           lse=None, return_lse=True, stream=None, softcap=0.0, alibi_slopes=None):
    """Dense prefill: q (B, Lq, Hq, d), k/v (B, Lk, Hkv, d) bf16 -> O, LSE (B, Hq, Lq).
    softcap > 0 caps the logits (c*tanh(x/c)); alibi_slopes (Hq,) or (B, Hq)
    float32 adds -slope*|i + Lk - Lq - j|.  out / lse, if given, must have exactly
    those shapes (bf16 / float32, contiguous, on q's device)."""
    torch = _torch()
    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    B, Lq, Hq, d = q.shape
    _need(k, "k", torch.bfloat16, 4, device=dev)
    Lk, Hkv = k.shape[1], k.shape[2]
    _need(k, "k", shape=(B, Lk, Hkv, d))
    _need(v, "v", torch.bfloat16, shape=(B, Lk, Hkv, d), device=dev)
    s = _stream_obj(stream)
    mods = _mods(softcap, alibi_slopes, B, Hq, dev)
    out = _output(out, "out", (B, Lq, Hq, d), torch.bfloat16, dev, s)
    if return_lse or lse is not None:
        lse = _output(lse, "lse", (B, Hq, Lq), torch.float32, dev, s)
    st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Lq, Lk, Hq, Hkv, d,
                    _scale(softmax_scale, d), int(bool(causal)), int(window[0]), int(window[1]),
                    *mods, _stream(s))
    _check("fa_fwd", st)
    return out, lse


def _varlen_args(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, return_lse, s):
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    total_q, Hq, d = q.shape
    _need(k, "k", torch.bfloat16, 3, device=dev)
    total_k, Hkv = k.shape[0], k.shape[1]
    _need(k, "k", shape=(total_k, Hkv, d))
    _need(v, "v", torch.bfloat16, shape=(total_k, Hkv, d), device=dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, device=dev)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, device=dev)
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    out = _output(out, "out", (total_q, Hq, d), torch.bfloat16, dev, s)
    if return_lse or lse is not None:
        lse = _output(lse, "lse", (Hq, total_q), torch.float32, dev, s)
    return out, lse, B, total_q, total_k, Hq, Hkv, d


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  softmax_scale=None, causal=False, window=(-1, -1), out=None, lse=None,
                  return_lse=True, stream=None, softcap=0.0, alibi_slopes=None):
    """Packed varlen prefill: q (total_q, Hq, d), k/v (total_k, Hkv, d), cu_seqlens int32
    device tensors of length B+1 -> O (total_q, Hq, d), LSE (Hq, total_q)."""
    lib = load_library()
    s = _stream_obj(stream)
    out, lse, B, total_q, total_k, Hq, Hkv, d = _varlen_args(
        q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, return_lse, s)
    mods = _mods(softcap, alibi_slopes, B, Hq, q.device)
    st = lib.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                           _ptr(cu_seqlens_k), B, int(max_seqlen_q), int(max_seqlen_k), total_q,
                           total_k, Hq, Hkv, d, _scale(softmax_scale, d), int(bool(causal)),
                           int(window[0]), int(window[1]), *mods, _stream(s))
    _check("fa_fwd_varlen", st)
    return out, lse


def fa_varlen_plan(cu_seqlens_q, cu_seqlens_k, causal=False, window=(-1, -1)):
    """Host plan for fa_fwd_varlen_run from HOST cumulative lengths (lists, numpy arrays or
    CPU tensors of B+1 ints) -> numpy int32 array (num_items, 2) of (sequence, query tile),
    heaviest first.  No GPU is needed."""
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
    s = _stream_obj(stream)
    out, lse, B, total_q, total_k, Hq, Hkv, d = _varlen_args(
        q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, return_lse, s)
    _need(plan, "plan", torch.int32, 2, device=q.device)
    if plan.shape[1] != 2:
        raise ValueError("plan must be (num_items, 2)")
    mods = _mods(softcap, alibi_slopes, B, Hq, q.device)
    st = lib.fa_fwd_varlen_run(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                               _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(plan),
                               plan.shape[0], B, int(max_seqlen_q), int(max_seqlen_k), total_q,
                               total_k, Hq, Hkv, d, _scale(softmax_scale, d), int(bool(causal)),
                               int(window[0]), int(window[1]), *mods, _stream(s))
    _check("fa_fwd_varlen_run", st)
    return out, lse


def fa_decode_paged_workspace_size(B, Hq, d, max_blocks_per_seq, page_size, split_tokens=0):
    return int(load_library().fa_decode_paged_workspace_size(B, Hq, d, max_blocks_per_seq,
                                                              page_size, split_tokens))


def _paged_inputs(q, k_cache, v_cache, block_table, cache_seqlens):
    """Checks shared by the calls over a paged cache; returns (num_pages, page_size, Hkv)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    B, _, _, d = q.shape
    _need(k_cache, "k_cache", torch.bfloat16, 4, device=dev)
    num_pages, page_size, Hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError("caches must be [num_pages, page_size, Hkv, d] with q's d")
    _need(v_cache, "v_cache", torch.bfloat16, shape=tuple(k_cache.shape), device=dev)
    _need(block_table, "block_table", torch.int32, 2, device=dev)
    if block_table.shape[0] != B:
        raise ValueError("block_table must be (B, max_blocks_per_seq)")
    _need(cache_seqlens, "cache_seqlens", torch.int32, shape=(B,), device=dev)
    return num_pages, page_size, Hkv


def _decode_args(q, k_cache, v_cache, block_table, cache_seqlens, split_tokens, out, lse,
                 workspace, return_lse, s):
    torch = _torch()
    num_pages, page_size, Hkv = _paged_inputs(q, k_cache, v_cache, block_table, cache_seqlens)
    B, one, Hq, d = q.shape
    if one != 1:
        raise ValueError("q must be (B, 1, Hq, d)")
    dev = q.device
    max_blocks = block_table.shape[1]
    need = fa_decode_paged_workspace_size(B, Hq, d, max_blocks, page_size, split_tokens)
    workspace, ws_bytes = _workspace(workspace, need, dev, s)
    out = _output(out, "out", (B, 1, Hq, d), torch.bfloat16, dev, s)
    if return_lse or lse is not None:
        lse = _output(lse, "lse", (B, Hq), torch.float32, dev, s)
    return out, lse, workspace, ws_bytes, B, Hq, Hkv, d, num_pages, page_size, max_blocks


def fa_decode_paged(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale=None,
                    window_left=-1, split_tokens=0, out=None, lse=None, workspace=None,
                    return_lse=True, stream=None, softcap=0.0, alibi_slopes=None):
    """Paged decode: q (B, 1, Hq, d), caches [num_pages, page_size, Hkv, d],
    block_table int32 [B, max_blocks], cache_seqlens int32 [B] -> O (B, 1, Hq, d),
    LSE (B, Hq).  softcap / alibi_slopes ((Hq,) or (B, Hq) float32) as for fa_fwd; the
    query sits at position cache_seqlens[b] - 1."""
    lib = load_library()
    s = _stream_obj(stream)
    out, lse, ws, ws_bytes, B, Hq, Hkv, d, num_pages, page_size, max_blocks = _decode_args(
        q, k_cache, v_cache, block_table, cache_seqlens, split_tokens, out, lse, workspace,
        return_lse, s)
    mods = _mods(softcap, alibi_slopes, B, Hq, q.device)
    st = lib.fa_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                             _ptr(cache_seqlens), _ptr(out), _ptr(lse), B, Hq, Hkv, d, num_pages,
                             page_size, max_blocks, _scale(softmax_scale, d), int(window_left),
                             *mods, int(split_tokens), _ptr(ws), ws_bytes, _stream(s))
    _check("fa_decode_paged", st)
    return out, lse


DECODE_NOALLOC_MAX_BYTES = 32 << 20


def fa_decode_paged_noalloc(q, k_cache, v_cache, block_table, cache_seqlens, softmax_scale=None,
                            window_left=-1, split_tokens=0, out=None, lse=None, return_lse=True,
                            stream=None, softcap=0.0, alibi_slopes=None):
    """fa_decode_paged without a workspace: the library's per-GPU scratch array
    (DECODE_NOALLOC_MAX_BYTES) holds the split partials.  Pass out (and lse) to make
    the call allocate nothing at all; calls that can overlap on one GPU must be
    ordered by the caller (they share the array)."""
    torch = _torch()
    lib = load_library()
    num_pages, page_size, Hkv = _paged_inputs(q, k_cache, v_cache, block_table, cache_seqlens)
    B, one, Hq, d = q.shape
    if one != 1:
        raise ValueError("q must be (B, 1, Hq, d)")
    dev = q.device
    s = _stream_obj(stream)
    out = _output(out, "out", (B, 1, Hq, d), torch.bfloat16, dev, s)
    if return_lse or lse is not None:
        lse = _output(lse, "lse", (B, Hq), torch.float32, dev, s)
    mods = _mods(softcap, alibi_slopes, B, Hq, dev)
    st = lib.fa_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                     _ptr(cache_seqlens), _ptr(out), _ptr(lse), B, Hq, Hkv, d,
                                     num_pages, page_size, block_table.shape[1],
                                     _scale(softmax_scale, d), int(window_left), *mods,
                                     int(split_tokens), _stream(s))
    _check("fa_decode_paged_noalloc", st)
    return out, lse


def fa_decode_plan(cache_seqlens, page_size, max_blocks_per_seq, window_left=-1, split_tokens=0):
    """Host plan for fa_decode_paged_run from HOST lengths (list, numpy array or CPU tensor of
    B ints) -> numpy int32 array (num_items, 2) of (request, split), heaviest first.  No GPU is
    needed."""
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
    s = _stream_obj(stream)
    out, lse, ws, ws_bytes, B, Hq, Hkv, d, num_pages, page_size, max_blocks = _decode_args(
        q, k_cache, v_cache, block_table, cache_seqlens, split_tokens, out, lse, workspace,
        return_lse, s)
    _need(plan, "plan", torch.int32, 2, device=q.device)
    if plan.shape[1] != 2:
        raise ValueError("plan must be (num_items, 2)")
    mods = _mods(softcap, alibi_slopes, B, Hq, q.device)
    st = lib.fa_decode_paged_run(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                 _ptr(cache_seqlens), _ptr(plan), plan.shape[0], _ptr(out),
                                 _ptr(lse), B, Hq, Hkv, d, num_pages, page_size, max_blocks,
                                 _scale(softmax_scale, d), int(window_left), *mods,
                                 int(split_tokens), _ptr(ws), ws_bytes, _stream(s))
    _check("fa_decode_paged_run", st)
    return out, lse


def fa_bwd_workspace_size(B, Hq, Lq):
    return int(load_library().fa_bwd_workspace_size(B, Hq, Lq))


def _grads(q, k, v, dq, dk, dv, dev, s):
    torch = _torch()
    return (_output(dq, "dq", tuple(q.shape), torch.bfloat16, dev, s),
            _output(dk, "dk", tuple(k.shape), torch.bfloat16, dev, s),
            _output(dv, "dv", tuple(v.shape), torch.bfloat16, dev, s))


def fa_bwd(q, k, v, out, lse, dout, softmax_scale=None, causal=False, window=(-1, -1),
           dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward of fa_fwd: q, out, dout (B, Lq, Hq, d), k, v (B, Lk, Hkv, d) bf16, lse
    (B, Hq, Lq) float32 from fa_fwd -> dq, dk, dv (bf16, shapes of q, k, v)."""
    torch = _torch()
    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    B, Lq, Hq, d = q.shape
    _need(k, "k", torch.bfloat16, 4, device=dev)
    Lk, Hkv = k.shape[1], k.shape[2]
    _need(k, "k", shape=(B, Lk, Hkv, d))
    _need(v, "v", torch.bfloat16, shape=(B, Lk, Hkv, d), device=dev)
    _need(out, "out", torch.bfloat16, shape=tuple(q.shape), device=dev)
    _need(dout, "dout", torch.bfloat16, shape=tuple(q.shape), device=dev)
    _need(lse, "lse", torch.float32, shape=(B, Hq, Lq), device=dev)
    s = _stream_obj(stream)
    dq, dk, dv = _grads(q, k, v, dq, dk, dv, dev, s)
    ws, ws_bytes = _workspace(workspace, fa_bwd_workspace_size(B, Hq, Lq), dev, s)
    st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                    _ptr(dk), _ptr(dv), B, Lq, Lk, Hq, Hkv, d, _scale(softmax_scale, d),
                    int(bool(causal)), int(window[0]), int(window[1]), _ptr(ws), ws_bytes,
                    _stream(s))
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
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    total_q, Hq, d = q.shape
    _need(k, "k", torch.bfloat16, 3, device=dev)
    total_k, Hkv = k.shape[0], k.shape[1]
    _need(k, "k", shape=(total_k, Hkv, d))
    _need(v, "v", torch.bfloat16, shape=(total_k, Hkv, d), device=dev)
    _need(out, "out", torch.bfloat16, shape=tuple(q.shape), device=dev)
    _need(dout, "dout", torch.bfloat16, shape=tuple(q.shape), device=dev)
    _need(lse, "lse", torch.float32, shape=(Hq, total_q), device=dev)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, device=dev)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, device=dev)
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    s = _stream_obj(stream)
    dq, dk, dv = _grads(q, k, v, dq, dk, dv, dev, s)
    ws, ws_bytes = _workspace(workspace, fa_bwd_varlen_workspace_size(B, Hq, total_q), dev, s)
    st = lib.fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B,
                           int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, Hq, Hkv, d,
                           _scale(softmax_scale, d), int(bool(causal)), int(window[0]),
                           int(window[1]), _ptr(ws), ws_bytes, _stream(s))
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
    num_pages, page_size, Hkv = _paged_inputs(q, k_cache, v_cache, block_table, cache_seqlens)
    dev = q.device
    B, Lq, Hq, d = q.shape
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        _need(k_new, "k_new", torch.bfloat16, shape=(B, Lq, Hkv, d), device=dev)
        _need(v_new, "v_new", torch.bfloat16, shape=(B, Lq, Hkv, d), device=dev)
    s = _stream_obj(stream)
    mods = _mods(softcap, alibi_slopes, B, Hq, dev)
    out = _output(out, "out", (B, Lq, Hq, d), torch.bfloat16, dev, s)
    if return_lse or lse is not None:
        lse = _output(lse, "lse", (B, Hq, Lq), torch.float32, dev, s)
    wl, wr = window
    st = lib.fa_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                            _ptr(block_table), _ptr(cache_seqlens), _ptr(out), _ptr(lse),
                            B, Lq, Hq, Hkv, d, num_pages, page_size, block_table.shape[1],
                            _scale(softmax_scale, d), int(bool(causal)), int(wl), int(wr),
                            *mods, _stream(s))
    _check("fa_fwd_kvcache", st)
    return out, lse


__all__ = ["fa_fwd", "fa_fwd_varlen", "fa_varlen_plan", "fa_fwd_varlen_run",
           "fa_decode_paged", "fa_decode_plan", "fa_decode_paged_run", "fa_decode_paged_noalloc",
           "DECODE_NOALLOC_MAX_BYTES",
           "fa_decode_paged_workspace_size", "fa_fwd_kvcache", "fa_bwd",
           "fa_bwd_workspace_size", "fa_bwd_varlen", "fa_bwd_varlen_workspace_size",
           "load_library", "exported_symbols", "cu_seqlens_from_lengths",
           "lengths_from_cu_seqlens", "FAError", "LIB_PATH"]
