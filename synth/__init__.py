"""Seeded synthetic inputs for the gated delta-rule mixer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
bench.  It holds no arithmetic of the mixer itself: it draws random numbers,
applies the input-side transforms of the workloads (L2-normalisation of q and
k per head, the logistic sigmoid for the gates) and rounds to bfloat16.

The pages ("Super Apriel: One Checkpoint, Many Speeds", §2.A "The Supernet
Architecture") name the two mixers -- GDN with a scalar gate and KDA with a
channel-wise gate -- but give no shapes, dtypes or distributions.  The
workloads below are synthetic stand-ins shaped like one mixer layer of a
48-layer 15B-class decoder.

Recipe (all workloads):
  * generator: numpy PCG64; each tensor gets its own child stream of
    ``SeedSequence([seed, layer])``, spawned in the order q, k, v, alpha,
    beta, s0;
  * q, k ~ N(0, 1) drawn in float32, then divided by their Euclidean norm
    over the key dimension (in float64), per (b, t, h);
  * v ~ N(0, 1);
  * beta = sigmoid(N(0, 1)); alpha = sigmoid(N(2, 0.5)) per (b, t, h) for
    the scalar gate, per (b, t, h, c) for the channel gate (N(mu, sigma),
    sigma a standard deviation);
  * s0 ~ N(0, 0.02) in fp32 where the workload has an initial state;
  * q, k, v are rounded to bfloat16 (round to nearest even) for the bf16
    workloads; alpha, beta and the state are always fp32.

Arrays are returned as float32 numpy arrays whose values are exactly
representable in the workload's dtype, so the oracle can upcast them to
float64 without loss and the device can take them as bf16 without rounding.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "bf16_round",
    "bf16_bits",
    "make_inputs",
    "make_raw_inputs",
    "make_state",
]


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "decode" | "prefill"
    gate: str            # "gdn" | "kda"
    dtype: str           # "f32" | "bf16" -- dtype of q, k, v, o
    B: int
    T: int               # tokens per sequence (1 for decode)
    H: int
    dk: int
    dv: int
    chunk: int = 64
    s0: str = "zero"     # "zero" | "normal" (N(0, 0.02))
    layers: int = 1      # independent layer states (decode timing)
    seed: int = 0
    extra: dict = field(default_factory=dict, compare=False, hash=False)


# The five workloads of the mixer's hot path.  Seeds follow the order in
# which they are listed.
WORKLOADS = {
    "gdn_tiny_f32": Workload("gdn_tiny_f32", "prefill", "gdn", "f32",
                             B=1, T=64, H=2, dk=16, dv=16, s0="zero", seed=0),
    "gdn_decode_b64_h32_d128": Workload("gdn_decode_b64_h32_d128", "decode", "gdn", "bf16",
                                        B=64, T=1, H=32, dk=128, dv=128, s0="normal",
                                        layers=48, seed=1),
    "kda_decode_b256_h32_d128": Workload("kda_decode_b256_h32_d128", "decode", "kda", "bf16",
                                         B=256, T=1, H=32, dk=128, dv=128, s0="normal",
                                         seed=2),
    "gdn_prefill_b4_t8192_h32_d128": Workload("gdn_prefill_b4_t8192_h32_d128", "prefill",
                                              "gdn", "bf16", B=4, T=8192, H=32, dk=128,
                                              dv=128, s0="zero", seed=3),
    "kda_prefill_b1_t32768_h32_d128": Workload("kda_prefill_b1_t32768_h32_d128", "prefill",
                                               "kda", "bf16", B=1, T=32768, H=32, dk=128,
                                               dv=128, s0="normal", seed=4),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    NaN stays NaN; infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    nan = np.isnan(x)
    out = r.view(np.float32).copy()
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values already rounded by :func:`bf16_round`."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    n = np.sqrt((x64 * x64).sum(axis=-1, keepdims=True))
    n[n == 0] = 1.0
    return (x64 / n).astype(np.float32)


def _streams(seed: int, layer: int):
    ss = np.random.SeedSequence([int(seed), int(layer)])
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(6)]


def make_state(rng: np.random.Generator, B: int, H: int, dk: int, dv: int) -> np.ndarray:
    """Initial state S_0 ~ N(0, 0.02) in fp32, layout [B, H, dk, dv]."""
    s = rng.standard_normal((B, H, dk, dv), dtype=np.float32)
    s *= np.float32(0.02)
    return s


def make_inputs(w: Workload, layer: int = 0, *, B: Optional[int] = None,
                T: Optional[int] = None, H: Optional[int] = None,
                seed: Optional[int] = None, s0: Optional[str] = None,
                alpha_mean: float = 2.0) -> dict:
    """Draw one layer's inputs for workload ``w``.

    Token tensors use the layout [B, T, H, d]; decode workloads (T == 1) use
    the same arrays, which are also valid as [B, H, d].  ``B``, ``T``, ``H``,
    ``seed`` and ``s0`` override the workload's values (used to draw smaller
    cases with the same distributions); ``alpha_mean`` moves the mean of the
    gate logits (2.0 for every workload; -2.0 gives fast-forgetting gates).

    Returns a dict with float32 arrays ``q, k`` [B,T,H,dk], ``v`` [B,T,H,dv],
    ``alpha`` [B,T,H] (gdn) or [B,T,H,dk] (kda), ``beta`` [B,T,H], and
    ``s0`` [B,H,dk,dv] or None.
    """
    B = w.B if B is None else B
    T = w.T if T is None else T
    H = w.H if H is None else H
    seed = w.seed if seed is None else seed
    s0_kind = w.s0 if s0 is None else s0
    rq, rk, rv, ra, rb, rs = _streams(seed, layer)
    dk, dv = w.dk, w.dv

    q = _l2_normalise(rq.standard_normal((B, T, H, dk), dtype=np.float32))
    k = _l2_normalise(rk.standard_normal((B, T, H, dk), dtype=np.float32))
    v = rv.standard_normal((B, T, H, dv), dtype=np.float32)
    if w.dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    ashape = (B, T, H) if w.gate == "gdn" else (B, T, H, dk)
    alpha = _sigmoid(np.float32(alpha_mean) + 0.5 * ra.standard_normal(ashape, dtype=np.float32))
    beta = _sigmoid(rb.standard_normal((B, T, H), dtype=np.float32))
    s0 = make_state(rs, B, H, dk, dv) if s0_kind == "normal" else None
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta, "s0": s0}


def make_raw_inputs(w: Workload, layer: int = 0, *, B: Optional[int] = None,
                    T: Optional[int] = None, H: Optional[int] = None,
                    seed: Optional[int] = None, s0: Optional[str] = None,
                    round_bf16: bool = True, alpha_mean: float = 2.0) -> dict:
    """The same draws as :func:`make_inputs` before its two transforms: q and
    k are the raw normal draws (not normalised) and ``alpha``, ``beta`` are the
    logits (before the sigmoid).  With a bf16 workload and ``round_bf16`` the
    raw q, k, v are rounded to bf16 (what a caller would pass)."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    H = w.H if H is None else H
    seed = w.seed if seed is None else seed
    s0_kind = w.s0 if s0 is None else s0
    rq, rk, rv, ra, rb, rs = _streams(seed, layer)
    dk, dv = w.dk, w.dv
    q = rq.standard_normal((B, T, H, dk), dtype=np.float32)
    k = rk.standard_normal((B, T, H, dk), dtype=np.float32)
    v = rv.standard_normal((B, T, H, dv), dtype=np.float32)
    if w.dtype == "bf16" and round_bf16:
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    ashape = (B, T, H) if w.gate == "gdn" else (B, T, H, dk)
    alpha = (np.float32(alpha_mean) + 0.5 * ra.standard_normal(ashape, dtype=np.float32)).astype(np.float32)
    beta = rb.standard_normal((B, T, H), dtype=np.float32)
    s0 = make_state(rs, B, H, dk, dv) if s0_kind == "normal" else None
    return {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta, "s0": s0}

