"""CPU oracle of the gated delta-rule token mixer (float64).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``, the smoke check
in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import this
package.  It shares no code with the GPU library ``gated_delta_rule_08_amd``.

Three independent forms of the same recurrence (see ``gdr_oracle.c`` for the
definition and the chunked algebra):

* :func:`recurrent`  -- plain C, token by token (the main oracle);
* :func:`chunked`    -- plain C, the exact chunked (WY/UT) refactoring;
* :func:`brute`      -- NumPy, dense per-token transition matrices
  ``M_t = (I - beta_t k_t k_t^T) D_t``, for tiny inputs only;
* :func:`prologue`   -- NumPy, the input steps before the mixer (q/k L2
  normalisation, sigmoid of the gate logits);
* :func:`backward`   -- NumPy, reverse-mode gradients of the token recurrence
  (pinned by central finite differences of :func:`recurrent` and by closed
  forms; see tests/test_oracle.py).

Pins: every function here is checked against facts fixed by the mathematics
(identity and rank-one special cases, the delta rule's exact recall, a scalar
closed form, linearity, column independence, the contraction bound, and the
agreement of the three forms).  The pages print no worked example, formula or
value for the mixer, so no number here is pinned to the pages themselves.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libgdr_oracle.so``."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        args = [ctypes.c_int] * 6 + [ctypes.c_double] + [dp] * 8 + [ctypes.c_int]
        lib.oracle_recurrent.argtypes = args
        lib.oracle_recurrent.restype = ctypes.c_int
        lib.oracle_chunked.argtypes = [ctypes.c_int] * 7 + [ctypes.c_double] + [dp] * 8 + [ctypes.c_int]
        lib.oracle_chunked.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shapes(q, v, alpha):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    kda = alpha.ndim == 4
    return B, T, H, dk, dv, kda


def _run(fn_name, q, k, v, alpha, beta, s0, scale, chunk, nthreads):
    q, k, v, alpha, beta, s0 = (_f64(x) for x in (q, k, v, alpha, beta, s0))
    B, T, H, dk, dv, kda = _shapes(q, v, alpha)
    assert k.shape == q.shape and v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    assert alpha.shape in ((B, T, H), (B, T, H, dk))
    if s0 is not None:
        assert s0.shape == (B, H, dk, dv)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    sT = np.zeros((B, H, dk, dv), dtype=np.float64)
    nt = default_threads() if nthreads is None else int(nthreads)
    lib = _load()
    if fn_name == "recurrent":
        rc = lib.oracle_recurrent(int(kda), B, T, H, dk, dv, float(scale), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0), _ptr(o),
                                  _ptr(sT), nt)
    else:
        rc = lib.oracle_chunked(int(kda), B, T, H, dk, dv, int(chunk), float(scale), _ptr(q),
                                _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(s0), _ptr(o),
                                _ptr(sT), nt)
    if rc != 0:
        raise RuntimeError("oracle %s failed with status %d" % (fn_name, rc))
    return o, sT


def recurrent(q, k, v, alpha, beta, s0=None, scale: float = 1.0,
              nthreads: Optional[int] = None):
    """Token-by-token gated delta rule.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv]).

    ``alpha`` of shape [B,T,H] selects the scalar gate (GDN), [B,T,H,dk] the
    channel gate (KDA).  All arithmetic is float64.
    """
    return _run("recurrent", q, k, v, alpha, beta, s0, scale, 1, nthreads)


def chunked(q, k, v, alpha, beta, s0=None, scale: float = 1.0, chunk: int = 64,
            nthreads: Optional[int] = None):
    """Chunked (WY/UT) form of the same recurrence, float64."""
    return _run("chunked", q, k, v, alpha, beta, s0, scale, chunk, nthreads)


def decode_step(q, k, v, alpha, beta, state, scale: float = 1.0,
                nthreads: Optional[int] = None):
    """One decode step on [B,H,d] inputs.  Returns (o [B,H,dv], new state)."""
    q, k, v, beta = (np.asarray(x)[:, None] for x in (q, k, v, beta))
    alpha = np.asarray(alpha)[:, None]
    o, s = recurrent(q, k, v, alpha, beta, state, scale, nthreads)
    return o[:, 0], s


def prologue(q, k, alpha, beta, norm_qk: bool = True, sigmoid_gates: bool = True,
             eps: float = 1e-12):
    """The input steps on the near side of the mixer, in float64.

    ``norm_qk``: every q and k vector (last axis, length dk) is divided by its
    Euclidean norm, the norm clamped below at ``eps`` (a zero vector stays
    zero).  ``sigmoid_gates``: alpha and beta are logits and become
    1 / (1 + exp(-x)), evaluated without overflow for either sign.
    Returns (q, k, alpha, beta) ready for :func:`recurrent`.
    """
    q, k, alpha, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, alpha, beta))
    if norm_qk:
        q = q / np.maximum(np.sqrt(np.sum(q * q, axis=-1, keepdims=True)), eps)
        k = k / np.maximum(np.sqrt(np.sum(k * k, axis=-1, keepdims=True)), eps)
    if sigmoid_gates:
        def sig(x):
            e = np.exp(-np.abs(x))  # <= 1, never overflows
            return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
        alpha, beta = sig(alpha), sig(beta)
    return q, k, alpha, beta


def brute(q, k, v, alpha, beta, s0=None, scale: float = 1.0):
    """Dense-matrix form for tiny inputs (pure Python loop over tokens).

    For each (b, h) and token t, builds the dk x dk transition
    M_t = (I - beta_t k_t k_t^T) D_t explicitly and applies
    S_t = M_t S_{t-1} + beta_t k_t v_t^T, o_t = scale * S_t^T q_t with full
    matrix products -- a code path separate from the rank-one update above.
    """
    q, k, v, alpha, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert dk <= 8 and dv <= 8 and T <= 64, "brute force is for tiny inputs only"
    o = np.zeros((B, T, H, dv))
    sT = np.zeros((B, H, dk, dv))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if s0 is None else np.array(s0[b, h], dtype=np.float64)
            for t in range(T):
                kt = k[b, t, h][:, None]
                a = alpha[b, t, h]
                D = np.diag(a) if np.ndim(a) == 1 else a * eye
                M = (eye - beta[b, t, h] * (kt @ kt.T)) @ D
                S = M @ S + beta[b, t, h] * (kt @ v[b, t, h][None, :])
                o[b, t, h] = scale * (S.T @ q[b, t, h])
            sT[b, h] = S
    return o, sT


def backward(q, k, v, alpha, beta, s0, do, ds_t=None, scale: float = 1.0):
    """Gradients of L = sum(do * o) + sum(ds_t * S_T) through the token
    recurrence, float64.

    Forward, per (b, h) and token t (D_t = alpha_t I or diag(alpha_t)):
        S'_t = D_t S_{t-1},  u_t = S'_t^T k_t,  e_t = v_t - u_t,
        S_t = S'_t + beta_t k_t e_t^T,  o_t = scale S_t^T q_t.
    Reverse, with G the gradient of L with respect to S_t (starting from
    ds_t) and each forward step undone in the opposite order:
        G += scale q_t do_t^T;           dq_t = scale S_t do_t
        g = G^T k_t (d/d e_t = beta_t g): dv_t = beta_t g,
                                           dbeta_t = e_t . g,
                                           dk_t = beta_t G e_t
        du_t = -beta_t g;  G' = G + k_t du_t^T;  dk_t += S'_t du_t
        dalpha_t = sum_j G'[:, j] * S_{t-1}[:, j]   (summed over i for GDN)
        G = D_t G'
    and dS_0 = G at the end.  Returns a dict with dq, dk, dv, dalpha, dbeta,
    ds0 shaped like the inputs (ds0 like s0, zeros-state when s0 is None).
    """
    q, k, v, alpha, beta, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, alpha, beta, do))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    kda = alpha.ndim == 4
    s = np.zeros((B, H, dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)

    def step(t, s_prev):  # the forward step from S_{t-1}: (S'_t, e_t, S_t)
        a = alpha[:, t][..., None] if kda else alpha[:, t][..., None, None]   # [B,H,dk,1] or [B,H,1,1]
        sp = a * s_prev
        e = v[:, t] - np.einsum("bhij,bhi->bhj", sp, k[:, t])
        return sp, e, sp + beta[:, t][..., None, None] * k[:, t][..., :, None] * e[..., None, :]

    # forward, keeping S_{t-1} only (the rest of a step is recomputed from it)
    prev = []
    for t in range(T):
        prev.append(s)
        s = step(t, s)[2]
    G = np.zeros((B, H, dk, dv)) if ds_t is None else np.array(ds_t, dtype=np.float64)
    dq, dkk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    da, db = np.zeros_like(alpha), np.zeros_like(beta)
    for t in reversed(range(T)):
        sp, e, s_t = step(t, prev[t])
        bt = beta[:, t][..., None]                                  # [B,H,1]
        G = G + scale * q[:, t][..., :, None] * do[:, t][..., None, :]
        dq[:, t] = scale * np.einsum("bhij,bhj->bhi", s_t, do[:, t])
        g = np.einsum("bhij,bhi->bhj", G, k[:, t])                  # G^T k
        dvv[:, t] = bt * g
        db[:, t] = np.sum(e * g, axis=-1)
        dkk[:, t] = bt * np.einsum("bhij,bhj->bhi", G, e)
        du = -bt * g
        Gp = G + k[:, t][..., :, None] * du[..., None, :]
        dkk[:, t] += np.einsum("bhij,bhj->bhi", sp, du)
        row = np.sum(Gp * prev[t], axis=-1)                         # [B,H,dk]
        if kda:
            da[:, t] = row
            G = alpha[:, t][..., None] * Gp
        else:
            da[:, t] = np.sum(row, axis=-1)
            G = alpha[:, t][..., None, None] * Gp
    return {"dq": dq, "dk": dkk, "dv": dvv, "dalpha": da, "dbeta": db, "ds0": G}

