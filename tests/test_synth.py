"""The seeded input generator: determinism, bf16 rounding, distributions."""
import numpy as np
import pytest
import torch

import synth


def test_same_seed_same_bytes():
    w = synth.WORKLOADS["kda_decode_b256_h32_d128"]
    a = synth.make_inputs(w, B=2, H=3)
    b = synth.make_inputs(w, B=2, H=3)
    for key in a:
        if a[key] is None:
            assert b[key] is None
        else:
            assert a[key].tobytes() == b[key].tobytes()
    c = synth.make_inputs(w, layer=1, B=2, H=3)
    assert c["q"].tobytes() != a["q"].tobytes()


def test_bf16_round_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(100000).astype(np.float32),
        (r.standard_normal(1000) * 1e30).astype(np.float32),
        (r.standard_normal(1000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8],
                 dtype=np.float32),
    ])
    ours = synth.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    bits = synth.bf16_bits(ours)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(back.view(np.uint32), ours.view(np.uint32))


def test_bf16_round_nan():
    x = np.array([np.nan], dtype=np.float32)
    assert np.isnan(synth.bf16_round(x)[0])


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_distributions(name):
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w, B=1, T=min(w.T, 256), H=min(w.H, 4))
    qn = np.linalg.norm(inp["q"].astype(np.float64), axis=-1)
    kn = np.linalg.norm(inp["k"].astype(np.float64), axis=-1)
    tol = 1e-2 if w.dtype == "bf16" else 1e-6
    assert np.abs(qn - 1).max() < tol and np.abs(kn - 1).max() < tol
    a = inp["alpha"].astype(np.float64)
    assert a.shape[-1] == (w.dk if w.gate == "kda" else 1) or a.ndim == 3
    assert 0 < a.min() and a.max() < 1
    # sigmoid(N(2, 0.5)) has mean ~0.87; sigmoid(N(0, 1)) has mean 0.5.
    assert abs(a.mean() - 0.87) < 0.03
    assert abs(inp["beta"].mean() - 0.5) < 0.08
    if w.dtype == "bf16":
        for key in ("q", "k", "v"):
            assert np.array_equal(synth.bf16_round(inp[key]), inp[key])
    if w.s0 == "normal":
        assert abs(inp["s0"].std() - 0.02) < 0.002
    else:
        assert inp["s0"] is None
