"""Helpers for the GPU parity tests: device upload, oracle comparison."""
import os
import sys

import numpy as np
import torch

import gated_delta_rule_08_amd as gdr
from oracle_pool import rel_err

TOL = {"f32": 1e-4, "bf16": 2e-2}


def ensure_built():
    if not os.path.exists(gdr.library_path()):
        from gated_delta_rule_08_amd import build
        build.build()
    gdr.load_library()


def announce(msg: str) -> None:
    """Name the case on stdout before a GPU step, so a fault can be attributed."""
    sys.stdout.write("[gpu-case] %s\n" % msg)
    sys.stdout.flush()


def to_dev(x, dtype: str, dev="cuda"):
    """numpy float32 (already representable in `dtype`) -> device tensor."""
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.to(dev)


def to_host64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got, ref, tol, what=""):
    e = rel_err(got, ref)
    assert e <= tol, "%s: max|err| / max|ref| = %.3e > %.1e" % (what, e, tol)
    return e
