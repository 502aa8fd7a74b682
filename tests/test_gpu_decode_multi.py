"""GPU parity of the multi-token decode (speculative verify) step.

The reference for every intermediate state is the float64 token-by-token
oracle run one token at a time from the previous state; the kernel's own
consistency is checked bitwise against T single decode steps (same
arithmetic in the same order), a rollback from a saved state, and a run
without the saved states.
"""
from dataclasses import replace

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


def _workload(gate, dtype, dk=128, dv=128):
    base = synth.WORKLOADS["gdn_decode_b64_h32_d128" if gate == "gdn" else "kda_decode_b256_h32_d128"]
    return replace(base, dtype=dtype, dk=dk, dv=dv)


def _dev(inp, dtype):
    return {k: to_dev(v, dtype if k in ("q", "k", "v") else "f32") for k, v in inp.items()}


def _run_multi(gate, dtype, inp, scale=1.0, save=True):
    dev = _dev(inp, dtype)
    B, T, H, dv = inp["v"].shape
    dk = inp["q"].shape[-1]
    state = dev["s0"].clone()
    o = torch.empty(B, T, H, dv, device="cuda", dtype=dev["q"].dtype)
    states = torch.empty(B, T, H, dk, dv, device="cuda") if save else None
    gdr.gdr_decode_multi(gate, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], state, o,
                         states, scale=scale)
    torch.cuda.synchronize()
    return to_host64(o), to_host64(state), (to_host64(states) if save else None)


def _oracle_stepped(inp, scale=1.0):
    """The float64 recurrence one token at a time: o [B,T,H,dv], S_t for every t."""
    B, T, H, dv = inp["v"].shape
    s = inp["s0"]
    outs, states = [], []
    for t in range(T):
        sl = slice(t, t + 1)
        o, s = oracle.recurrent(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl],
                                inp["alpha"][:, sl], inp["beta"][:, sl], s, scale=scale)
        outs.append(o[:, 0])
        states.append(s)
    return np.stack(outs, axis=1), np.stack(states, axis=1)


def _check(gate, dtype, inp, scale=1.0):
    o, s, states = _run_multi(gate, dtype, inp, scale)
    o_ref, st_ref = _oracle_stepped(inp, scale)
    tol = TOL[dtype]
    assert_close(o, o_ref, tol, "o")
    assert_close(s, st_ref[:, -1], tol, "S_T")
    for t in range(st_ref.shape[1]):
        assert_close(states[:, t], st_ref[:, t], tol, "S_%d" % (t + 1))


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 128), (32, 128)])
@pytest.mark.parametrize("T", [1, 5])
def test_multi_matches_stepped_oracle(gate, dtype, dk, dv, T):
    w = _workload(gate, dtype, dk, dv)
    announce("decode_multi %s %s dk=%d dv=%d T=%d" % (gate, dtype, dk, dv, T))
    inp = synth.make_inputs(w, B=3, H=5, T=T, s0="normal", seed=21)
    _check(gate, dtype, inp, scale=0.5)


def test_multi_gdn_full_size_t4():
    """GDN verify of 4 draft tokens at the decode workload's full size."""
    w = _workload("gdn", "bf16")
    announce("decode_multi gdn B=64 H=32 d=128 T=4")
    _check("gdn", "bf16", synth.make_inputs(w, T=4))


def test_multi_kda_t8():
    w = _workload("kda", "bf16")
    announce("decode_multi kda B=16 H=32 d=128 T=8")
    _check("kda", "bf16", synth.make_inputs(w, B=16, T=8))


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_multi_equals_single_steps_bitwise(gate):
    """T tokens in one call give bitwise the outputs and states of T decode steps."""
    w = _workload(gate, "bf16")
    T = 6
    inp = synth.make_inputs(w, B=4, H=8, T=T)
    announce("decode_multi %s vs %d decode steps" % (gate, T))
    o, s, states = _run_multi(gate, "bf16", inp, scale=0.75)
    dev = _dev(inp, "bf16")
    state = dev["s0"].clone()
    for t in range(T):
        step = {k: dev[k][:, t].contiguous() for k in ("q", "k", "v", "alpha", "beta")}
        ot = torch.empty_like(step["v"])
        gdr.gdr_decode_step(gate, step["q"], step["k"], step["v"], step["alpha"], step["beta"],
                            state, ot, scale=0.75)
        torch.cuda.synchronize()
        assert np.array_equal(to_host64(ot), o[:, t]), t
        assert np.array_equal(to_host64(state), states[:, t]), t
    assert np.array_equal(to_host64(state), s)


def test_multi_rollback_and_no_states():
    """Continue from a saved state after an accepted prefix: the remaining
    tokens give the same outputs and final state; a run without saved states
    gives the same outputs and final state as one with them."""
    w = _workload("gdn", "bf16")
    T, a = 6, 3
    inp = synth.make_inputs(w, B=4, H=8, T=T)
    announce("decode_multi rollback T=%d accept=%d" % (T, a))
    o, s, states = _run_multi("gdn", "bf16", inp)
    o2, s2, _ = _run_multi("gdn", "bf16", inp, save=False)
    assert np.array_equal(o, o2) and np.array_equal(s, s2)
    rest = {k: (np.ascontiguousarray(v[:, a:]) if k != "s0" else states[:, a - 1].astype(np.float32))
            for k, v in inp.items()}
    o3, s3, _ = _run_multi("gdn", "bf16", rest)
    assert np.array_equal(o3, o[:, a:]) and np.array_equal(s3, s)


def test_multi_special_gates():
    """alpha = 1, beta = 0 leaves the state untouched (bitwise) for every t."""
    w = _workload("kda", "bf16")
    inp = synth.make_inputs(w, B=2, H=4, T=3)
    inp["alpha"] = np.ones_like(inp["alpha"])
    inp["beta"] = np.zeros_like(inp["beta"])
    announce("decode_multi identity gates")
    o, s, states = _run_multi("kda", "bf16", inp)
    s0 = inp["s0"].astype(np.float64)
    assert np.array_equal(s, s0)
    for t in range(3):
        assert np.array_equal(states[:, t], s0)


def test_multi_t0_is_noop():
    w = _workload("gdn", "bf16")
    inp = synth.make_inputs(w, B=2, H=4, T=1)
    dev = _dev(inp, "bf16")
    state = dev["s0"].clone()
    empty = {k: dev[k][:, :0].contiguous() for k in ("q", "k", "v", "alpha", "beta")}
    o = torch.empty(2, 0, 4, 128, device="cuda", dtype=torch.bfloat16)
    gdr.gdr_decode_multi("gdn", empty["q"], empty["k"], empty["v"], empty["alpha"], empty["beta"],
                         state, o)
    torch.cuda.synchronize()
    assert torch.equal(state, dev["s0"])
