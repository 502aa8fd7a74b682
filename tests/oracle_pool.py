"""The float64 backward oracle over every head of a full-size case, in CPU-only
worker processes.

The workers are spawned (fresh interpreters that import NumPy and the oracle
only), so they never touch the GPU.  Each task carries one head's inputs and
the GPU's gradients for that head; the worker runs the oracle on the head and
returns the relative errors, so no float64 gradients travel back.  This module
imports no torch, which is what lets the spawned workers import it.
"""
import multiprocessing as mp
import os
import sys
from concurrent.futures import FIRST_COMPLETED, ProcessPoolExecutor, wait

import numpy as np

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = ("dq", "dk", "dv", "dalpha", "dbeta")


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (inf if anything is not finite)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    denom = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    if not np.isfinite(err):
        return float("inf")
    return err / denom if denom > 0 else err


def _init():
    if _ROOT not in sys.path:
        sys.path.insert(0, _ROOT)


def _head(task):
    import oracle
    q, k, v, alpha, beta, s0, do, dst, got, scale = task
    ref = oracle.backward(q, k, v, alpha, beta, s0, do, dst, scale=scale)
    out = {key: rel_err(got[key], ref[key][0, :, 0]) for key in KEYS}
    out["ds0"] = rel_err(got["ds0"], ref["ds0"][0, 0])
    return out


def backward_errors_every_head(inp, do, dst, got, scale=1.0, workers=None, stall_s=900):
    """Relative errors {(b, h): {key: err}} of the GPU gradients `got`
    (arrays [B, T, H, ...], ds0 [B, H, dk, dv]) against the oracle, head by
    head.  At most 2 x workers tasks are in flight, so only that many heads'
    arrays are held at once; if no head finishes within stall_s seconds the
    call raises instead of waiting on."""
    B, T, H = inp["q"].shape[:3]
    n = workers or min(16, len(os.sched_getaffinity(0)))

    def task(b, h):
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        s0 = None if inp["s0"] is None else np.ascontiguousarray(inp["s0"][b:b + 1, h:h + 1])
        g = {key: np.ascontiguousarray(got[key][b, :, h]) for key in KEYS}
        g["ds0"] = np.ascontiguousarray(got["ds0"][b, h])
        return (sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["alpha"]), sl(inp["beta"]), s0,
                sl(do), np.ascontiguousarray(dst[b:b + 1, h:h + 1]), g, scale)

    heads = [(b, h) for b in range(B) for h in range(H)]
    # one BLAS thread per worker (the children inherit this environment)
    keep = {v: os.environ.get(v) for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for v in keep:
        os.environ[v] = "1"
    try:
        res = {}
        ex = ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=_init)
        try:
            pending = {}
            it = iter(heads)
            for bh in it:
                pending[ex.submit(_head, task(*bh))] = bh
                if len(pending) >= 2 * n:
                    break
            while pending:
                finished, _ = wait(pending, timeout=stall_s, return_when=FIRST_COMPLETED)
                if not finished:
                    raise TimeoutError("no oracle head finished within %d s" % stall_s)
                for f in finished:
                    res[pending.pop(f)] = f.result()
                    nxt = next(it, None)
                    if nxt is not None:
                        pending[ex.submit(_head, task(*nxt))] = nxt
        finally:
            ex.shutdown(wait=not pending, cancel_futures=True)
        return res
    finally:
        for v, old in keep.items():
            if old is None:
                os.environ.pop(v, None)
            else:
                os.environ[v] = old
