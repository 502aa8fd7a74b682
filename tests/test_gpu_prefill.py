"""GPU parity of the chunked prefill (fp32 and bf16 matrix-core paths)."""
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


def _dev_inputs(inp, dtype):
    return {k: to_dev(v, dtype if k in ("q", "k", "v") else "f32") for k, v in inp.items()}


def run_prefill(gate, dtype, inp, scale=1.0, state_in=None, in_place=False, flags=0):
    d = _dev_inputs(inp, dtype)
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    s_in = d["s0"] if state_in is None else state_in
    s_out = s_in if (in_place and s_in is not None) else torch.empty(B, H, dk, dv, device="cuda")
    o = torch.empty(B, T, H, dv, device="cuda", dtype=d["q"].dtype)
    gdr.gdr_chunk_prefill_ex(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], s_in, s_out, o,
                             flags=flags, scale=scale)
    torch.cuda.synchronize()
    return o, s_out


def check(gate, dtype, inp, scale=1.0, heads=None, flags=0):
    """Compare against the oracle (one run over every head); `heads` restricts
    the oracle to a sample of (b, h)."""
    o, s = run_prefill(gate, dtype, inp, scale, flags=flags)
    o, s = to_host64(o), to_host64(s)
    tol = TOL[dtype]
    if heads is None:
        o_ref, s_ref = oracle.recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"],
                                        inp["s0"], scale=scale)
        return assert_close(o, o_ref, tol, "o"), assert_close(s, s_ref, tol, "state")
    for (b, h) in heads:
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        s0 = None if inp["s0"] is None else np.ascontiguousarray(inp["s0"][b:b + 1, h:h + 1])
        o_ref, s_ref = oracle.recurrent(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["alpha"]),
                                        sl(inp["beta"]), s0, scale=scale)
        assert_close(o[b:b + 1, :, h:h + 1], o_ref, tol, "o[b=%d,h=%d]" % (b, h))
        assert_close(s[b:b + 1, h:h + 1], s_ref, tol, "state[b=%d,h=%d]" % (b, h))


def test_gdn_tiny_f32():
    """The 64-token fp32 GDN case (B=1, H=2, d=16, zero initial state)."""
    announce("prefill gdn f32 tiny")
    w = synth.WORKLOADS["gdn_tiny_f32"]
    check("gdn", "f32", synth.make_inputs(w))


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_ragged_lengths(gate, dtype, T):
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], gate=gate, dtype=dtype)
    announce("prefill %s %s T=%d d=128" % (gate, dtype, T))
    check(gate, dtype, synth.make_inputs(w, B=2, T=T, H=3, seed=100 + T), scale=0.7)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128),
                                   (64, 128)])
def test_head_sizes(gate, dtype, dk, dv):
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], gate=gate, dtype=dtype,
                dk=dk, dv=dv)
    announce("prefill %s %s dk=%d dv=%d" % (gate, dtype, dk, dv))
    check(gate, dtype, synth.make_inputs(w, B=1, T=150, H=4, seed=7))


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_many_heads_slice_width(gate):
    """Enough heads that each workgroup takes 64 value columns (two slices per head)."""
    w = replace(synth.WORKLOADS["gdn_prefill_b4_t8192_h32_d128"], gate=gate)
    announce("prefill %s bf16 B=8 H=32 T=130" % gate)
    inp = synth.make_inputs(w, B=8, T=130, H=32, seed=5, s0="normal")
    check(gate, "bf16", inp)


def test_gdn_prefill_b4_t8192_h32_d128():
    """Full-size GDN prefill: o and S_T over all 128 heads and the whole
    length against one full oracle run."""
    w = synth.WORKLOADS["gdn_prefill_b4_t8192_h32_d128"]
    inp = synth.make_inputs(w)
    announce("prefill gdn bf16 B=4 T=8192 H=32 d=128")
    check("gdn", "bf16", inp)


def test_kda_prefill_b1_t32768_h32_d128():
    """Full-size KDA prefill (long context): o and S_T over all 32 heads and
    the whole length against one full oracle run."""
    w = synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"]
    inp = synth.make_inputs(w)
    announce("prefill kda bf16 B=1 T=32768 H=32 d=128")
    check("kda", "bf16", inp)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_sequence_consistency(gate, dtype):
    """prefill(T1) then prefill(T2) from its state equals prefill(T1 + T2)."""
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], gate=gate, dtype=dtype)
    inp = synth.make_inputs(w, B=2, T=300, H=4, seed=9)
    announce("prefill split %s %s" % (gate, dtype))
    o_full, s_full = run_prefill(gate, dtype, inp)
    a = {k: (v if k == "s0" else np.ascontiguousarray(v[:, :100])) for k, v in inp.items()}
    bb = {k: (None if k == "s0" else np.ascontiguousarray(v[:, 100:])) for k, v in inp.items()}
    o_a, s_a = run_prefill(gate, dtype, a)
    o_b, s_b = run_prefill(gate, dtype, bb, state_in=s_a)
    tol = TOL[dtype]
    o_cat = torch.cat([o_a, o_b], dim=1)
    assert_close(to_host64(o_cat), to_host64(o_full), tol, "o")
    assert_close(to_host64(s_b), to_host64(s_full), tol, "state")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_decode_steps_match_prefill(gate):
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], gate=gate)
    inp = synth.make_inputs(w, B=2, T=70, H=4, seed=3)
    announce("prefill vs decode steps %s" % gate)
    o_p, s_p = run_prefill(gate, "bf16", inp)
    d = _dev_inputs(inp, "bf16")
    state = d["s0"].clone()
    outs = []
    for t in range(inp["q"].shape[1]):
        o = torch.empty(2, 4, w.dv, device="cuda", dtype=torch.bfloat16)
        gdr.gdr_decode_step(gate, d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                            d["v"][:, t].contiguous(), d["alpha"][:, t].contiguous(),
                            d["beta"][:, t].contiguous(), state, o)
        outs.append(o)
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=1)
    assert_close(to_host64(o_p), to_host64(o_d), TOL["bf16"], "o")
    assert_close(to_host64(s_p), to_host64(state), TOL["bf16"], "state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_in_place_state_and_empty_sequence(dtype):
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], dtype=dtype)
    inp = synth.make_inputs(w, B=1, T=90, H=2, seed=4)
    announce("prefill in place %s" % dtype)
    o1, s1 = run_prefill("kda", dtype, inp)
    s_dev = to_dev(inp["s0"], "f32")
    o2, s2 = run_prefill("kda", dtype, inp, state_in=s_dev, in_place=True)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    # T == 0: state copied (or zeroed) without touching o
    e = {k: (v if k == "s0" else np.ascontiguousarray(v[:, :0])) for k, v in inp.items()}
    _, s3 = run_prefill("kda", dtype, e)
    assert torch.equal(s3, to_dev(inp["s0"], "f32"))
    e["s0"] = None
    _, s4 = run_prefill("kda", dtype, e)
    assert torch.count_nonzero(s4) == 0


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_zero_gate_inside_chunk(gate):
    """alpha == 0 at one token: everything before it is forgotten exactly."""
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], gate=gate)
    inp = synth.make_inputs(w, B=1, T=128, H=2, seed=8)
    inp["alpha"][:, 40] = 0.0
    announce("prefill zero gate %s" % gate)
    check(gate, "bf16", inp)
    inp2 = dict(inp)
    inp2["alpha"] = inp["alpha"].copy()
    w32 = replace(w, dtype="f32")
    check(gate, "f32", synth.make_inputs(w32, B=1, T=128, H=2, seed=8) | {"alpha": inp2["alpha"]})


@pytest.mark.parametrize("dk,dv,T", [(128, 128, 1000), (64, 32, 333), (32, 64, 200), (16, 128, 130),
                                     (128, 16, 65)])
def test_kda_strong_channel_decay(dk, dv, T):
    """Fast-forgetting channel gates, alpha = sigmoid(N(-2, 0.5)): about -3
    in log2 per token, about -200 over a chunk, in every channel."""
    w = replace(synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"], dk=dk, dv=dv)
    inp = synth.make_inputs(w, B=2, T=T, H=3, seed=50 + dk, s0="normal", alpha_mean=-2.0)
    announce("prefill kda strong decay dk=%d dv=%d T=%d" % (dk, dv, T))
    check("kda", "bf16", inp, scale=0.9)


def test_kda_zero_channels():
    """Whole channels at alpha = 0 for whole chunks and across chunk
    boundaries, every channel at one token, and tiny nonzero gates."""
    w = synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"]
    inp = synth.make_inputs(w, B=1, T=400, H=5, seed=51, s0="normal")
    a = inp["alpha"]
    a[0, 64:128, 0, :32] = 0.0        # 32 channels of head 0 over all of chunk 1
    a[0, :, 1, 5] = 0.0               # channel 5 of head 1 at every token
    a[0, 100:300, 2, 64:] = 0.0       # half the channels of head 2 across three chunk boundaries
    a[0, 150, 3, :] = 0.0             # every channel of head 3 at one token
    a[0, 200:216, 4, ::2] = 1e-30     # tiny, nonzero
    announce("prefill kda zero channels")
    check("kda", "bf16", inp)


def test_prefill_deterministic():
    w = synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"]
    inp = synth.make_inputs(w, B=1, T=256, H=8, seed=12)
    a = run_prefill("kda", "bf16", inp)
    b = run_prefill("kda", "bf16", inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
