"""GPU parity of the decode step against the float64 oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_08_amd as gdr
import oracle
import synth
from gpu_util import TOL, announce, assert_close, ensure_built, to_dev, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _decode_inputs(w, layer=0, B=None, H=None, s0="normal", seed=None):
    inp = synth.make_inputs(w, layer=layer, B=B, H=H, T=1, s0=s0, seed=seed)
    # decode layout [B, H, d] is the T == 1 slice of [B, T, H, d]
    return {k: (None if v is None else (v[:, 0] if k != "s0" else v)) for k, v in inp.items()}


def _run_decode(gate, dtype, inp, scale=1.0):
    dev = {k: to_dev(v, dtype if k in ("q", "k", "v") else "f32") for k, v in inp.items()}
    B, H, dv = inp["v"].shape
    state = dev["s0"].clone()
    o = torch.empty(B, H, dv, device="cuda", dtype=dev["q"].dtype)
    gdr.gdr_decode_step(gate, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], state, o,
                        scale=scale)
    torch.cuda.synchronize()
    return to_host64(o), to_host64(state)


def _check_step(gate, dtype, inp, scale=1.0):
    o, s = _run_decode(gate, dtype, inp, scale)
    o_ref, s_ref = oracle.decode_step(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                      inp["s0"], scale=scale)
    tol = TOL[dtype]
    return assert_close(o, o_ref, tol, "o"), assert_close(s, s_ref, tol, "state")


@pytest.mark.parametrize("layer", [0, 47])
def test_gdn_decode_b64_h32_d128(layer):
    """GDN decode at its full size; two of the 48 independent layers (first, last)."""
    w = synth.WORKLOADS["gdn_decode_b64_h32_d128"]
    announce("gdn decode B=64 H=32 d=128 layer %d" % layer)
    _check_step("gdn", "bf16", _decode_inputs(w, layer=layer))


def test_kda_decode_b256_h32_d128():
    w = synth.WORKLOADS["kda_decode_b256_h32_d128"]
    announce("kda decode B=256 H=32 d=128")
    _check_step("kda", "bf16", _decode_inputs(w))


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 128), (128, 32), (64, 64), (128, 16),
                                   (16, 128), (128, 128)])
def test_decode_head_sizes(gate, dtype, dk, dv):
    from dataclasses import replace
    base = synth.WORKLOADS["gdn_tiny_f32" if gate == "gdn" else "kda_decode_b256_h32_d128"]
    w = replace(base, dtype=dtype, dk=dk, dv=dv)
    announce("decode %s %s dk=%d dv=%d" % (gate, dtype, dk, dv))
    _check_step(gate, dtype, _decode_inputs(w, B=3, H=5, seed=11), scale=0.5)


def test_tiny_f32_stepped_64_times():
    """The 64-token fp32 GDN case (d = 16) run token by token through decode."""
    w = synth.WORKLOADS["gdn_tiny_f32"]
    inp = synth.make_inputs(w)
    B, T, H, dk = inp["q"].shape
    state = torch.zeros(B, H, dk, w.dv, device="cuda")
    outs = []
    announce("decode gdn f32 stepped 64x")
    for t in range(T):
        dev = {k: to_dev(np.ascontiguousarray(inp[k][:, t]), "f32")
               for k in ("q", "k", "v", "alpha", "beta")}
        o = torch.empty(B, H, w.dv, device="cuda")
        gdr.gdr_decode_step("gdn", dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], state, o)
        outs.append(o)
    torch.cuda.synchronize()
    o = np.stack([to_host64(x) for x in outs], axis=1)
    o_ref, s_ref = oracle.recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    assert_close(o, o_ref, TOL["f32"], "o")
    assert_close(to_host64(state), s_ref, TOL["f32"], "state")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_decode_special_gates(gate):
    """alpha = 0 (rank-one write) and beta = 0, alpha = 1 (identity) on the GPU."""
    w = synth.WORKLOADS["kda_decode_b256_h32_d128"]
    from dataclasses import replace
    w = replace(w, gate=gate)
    inp = _decode_inputs(w, B=4, H=8)
    z = dict(inp)
    z["alpha"] = np.zeros_like(inp["alpha"])
    _check_step(gate, "bf16", z)
    ident = dict(inp)
    ident["alpha"] = np.ones_like(inp["alpha"])
    ident["beta"] = np.zeros_like(inp["beta"])
    o, s = _run_decode(gate, "bf16", ident)
    assert np.array_equal(s, inp["s0"].astype(np.float64))  # state untouched, bitwise


def test_decode_deterministic():
    w = synth.WORKLOADS["kda_decode_b256_h32_d128"]
    inp = _decode_inputs(w, B=16, H=32)
    a = _run_decode("kda", "bf16", inp)
    b = _run_decode("kda", "bf16", inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_decode_graph_replays_match_eager():
    """A decode step captured in a HIP graph, replayed several times with eager
    work and synchronisations in between; every replay matches eager steps."""
    w = synth.WORKLOADS["gdn_decode_b64_h32_d128"]
    inp = _decode_inputs(w, B=8, H=32)
    dev = {k: to_dev(v, "bf16" if k in ("q", "k", "v") else "f32") for k, v in inp.items()}
    B, H, dv = inp["v"].shape
    s_graph = dev["s0"].clone()
    s_eager = dev["s0"].clone()
    o_graph = torch.empty(B, H, dv, device="cuda", dtype=torch.bfloat16)
    o_eager = torch.empty_like(o_graph)
    step = lambda st, o: gdr.gdr_decode_step("gdn", dev["q"], dev["k"], dev["v"], dev["alpha"],
                                             dev["beta"], st, o)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        warm = dev["s0"].clone()
        step(warm, torch.empty_like(o_graph))
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(s_graph, o_graph)
    # capture does not execute: restore the starting state
    s_graph.copy_(dev["s0"])
    announce("decode graph replays")
    for rep in range(4):
        g.replay()
        step(s_eager, o_eager)
        torch.cuda.synchronize()
        assert torch.equal(o_graph, o_eager), rep
        assert torch.equal(s_graph, s_eager), rep
        junk = torch.randn(1024, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        del junk
