"""Shared helpers for the GPU tests (not collected as tests).

Comparison rule, fixed for every GPU test: with O_ref the unrounded float64
oracle output, |O - O_ref| <= 4e-3 + 1e-2 * |O_ref| element-wise for the bf16
output, and |LSE - LSE_ref| <= 1e-4 (absolute) for the fp32 log-sum-exp; rows
with no visible key must give O = 0 and LSE = -inf exactly.
"""

import numpy as np
import torch

O_ATOL, O_RTOL, LSE_TOL = 4e-3, 1e-2, 1e-4


def bits(t):
    """CPU bf16 tensor -> numpy uint16 bit patterns (the oracle reads these exactly)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def dev(t):
    return t.to("cuda", non_blocking=False)


def check(name, o, lse, o_ref, lse_ref):
    """Assert the tolerance; returns (max err/tol for O, max |dLSE|)."""
    o = f64(o) if isinstance(o, torch.Tensor) else o
    assert o.shape == o_ref.shape, (name, o.shape, o_ref.shape)
    assert np.isfinite(o).all(), f"{name}: non-finite output"
    ratio = float((np.abs(o - o_ref) / (O_ATOL + O_RTOL * np.abs(o_ref))).max()) if o.size else 0.0
    dl = 0.0
    if lse is not None:
        lse = f64(lse) if isinstance(lse, torch.Tensor) else lse
        assert lse.shape == lse_ref.shape, (name, lse.shape, lse_ref.shape)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isneginf(lse), ~fin), f"{name}: -inf LSE pattern differs"
        dl = float(np.abs(lse[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    print(f"[parity] {name}: max err/tol {ratio:.3f}, max |dLSE| {dl:.2e}", flush=True)
    assert ratio <= 1.0, f"{name}: O error {ratio:.3f} x tolerance"
    assert dl <= LSE_TOL, f"{name}: LSE error {dl:.3e}"
    return ratio, dl


def oracle_rows_parallel(q, k, v, tasks, scale, causal, window, workers=None):
    """oracle.attention_rows_ref over many (b, h, rows) tasks, run in a thread pool
    (numpy's kernels release the GIL; BLAS is held to one thread per task so the
    pool does not oversubscribe the host).  q, k, v: bf16 bit patterns (uint16)
    of the dense (B, L, H, d) layout.  Returns a list of (O, LSE) per task."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                      # pragma: no cover - installed here
        threadpool_limits = None
    n = workers or max(1, min(16, len(os.sched_getaffinity(0))))

    def one(t):
        b, h, rows = t
        return oracle.attention_rows_ref(q, k, v, b, h, rows, scale, causal, window)

    if threadpool_limits is None:
        with ThreadPoolExecutor(n) as ex:
            return list(ex.map(one, tasks))
    with threadpool_limits(limits=1), ThreadPoolExecutor(n) as ex:
        return list(ex.map(one, tasks))


def nan_like(t):
    """A device tensor of t's shape and dtype filled with NaN: outputs start
    poisoned, so an element the kernels never write fails the finiteness check."""
    return torch.full_like(t, float("nan"))
