"""GPU parity of the chunked backward pass (gdr_chunk_backward).

Reference: the float64 token-recurrence backward of the oracle (itself pinned
by central finite differences), on the same seeded inputs, output gradient
and final-state gradient.  Each gradient is compared element by element,
relative to its own largest magnitude.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import gated_delta_rule_08_amd as gdr
import oracle
import synth
from gpu_util import TOL, announce, assert_close, ensure_built, to_dev, to_host64
from oracle_pool import backward_errors_every_head

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _case(gate, dtype, B, T, H, dk, dv, seed, s0=True, dst=True, alpha_mean=2.0):
    base = synth.WORKLOADS["gdn_prefill_b4_t8192_h32_d128" if gate == "gdn" else "kda_prefill_b1_t32768_h32_d128"]
    w = replace(base, dtype=dtype, dk=dk, dv=dv)
    inp = synth.make_inputs(w, B=B, T=T, H=H, seed=seed, s0="normal" if s0 else "zero",
                            alpha_mean=alpha_mean)
    rng = np.random.default_rng(seed + 100)
    do = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    if dtype == "bf16":
        do = synth.bf16_round(do)
    dst_arr = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32) if dst else None
    return inp, do, dst_arr


def _run(gate, dtype, inp, do, dst, scale, want_ds0=True, ws_bytes=None):
    d = {key: to_dev(val, dtype if key in ("q", "k", "v") else "f32") for key, val in inp.items()}
    g_o = to_dev(do, dtype)
    g_st = None if dst is None else to_dev(dst, "f32")
    out = {"dq": torch.full_like(d["q"], 7.0), "dk": torch.full_like(d["k"], 7.0),
           "dv": torch.full_like(d["v"], 7.0), "dalpha": torch.full_like(d["alpha"], 7.0),
           "dbeta": torch.full_like(d["beta"], 7.0)}
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    out["ds0"] = torch.full((B, H, dk, dv), 7.0, device="cuda") if want_ds0 else None
    # an explicit workspace of ws_bytes (a ranged one below the one-pass size),
    # filled with garbage first
    ws = None if ws_bytes is None else torch.full((ws_bytes // 4,), float("nan"), device="cuda")
    gdr.gdr_chunk_backward(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["s0"], g_o, g_st,
                           out["dq"], out["dk"], out["dv"], out["dalpha"], out["dbeta"], out["ds0"],
                           scale=scale, workspace=ws)
    torch.cuda.synchronize()
    return {key: (None if val is None else to_host64(val)) for key, val in out.items()}


def _check(gate, dtype, B, T, H, dk, dv, seed=1, s0=True, dst=True, scale=0.8, alpha_mean=2.0):
    inp, do, dst_arr = _case(gate, dtype, B, T, H, dk, dv, seed, s0, dst, alpha_mean)
    got = _run(gate, dtype, inp, do, dst_arr, scale)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["s0"], do,
                          dst_arr, scale=scale)
    tol = TOL[dtype]
    for key in ("dq", "dk", "dv", "dalpha", "dbeta", "ds0"):
        assert_close(got[key], ref[key], tol, key)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_matches_oracle_ragged(gate, dtype):
    """Three chunks with a ragged tail, from a given state, with dS_T."""
    announce("backward %s %s B=2 T=150 H=2 d=64" % (gate, dtype))
    _check(gate, dtype, B=2, T=150, H=2, dk=64, dv=64)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (16, 32), (32, 16), (128, 64)])
def test_backward_head_sizes(gate, dk, dv):
    announce("backward %s f32 dk=%d dv=%d" % (gate, dk, dv))
    _check(gate, "f32", B=1, T=130, H=2, dk=dk, dv=dv, seed=4)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_backward_without_states(gate):
    """No initial state, no final-state gradient, one partial chunk."""
    announce("backward %s no states T=37" % gate)
    _check(gate, "f32", B=2, T=37, H=3, dk=32, dv=32, seed=6, s0=False, dst=False)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_backward_exact_chunks_bf16_d128(gate):
    announce("backward %s bf16 T=256 d=128" % gate)
    _check(gate, "bf16", B=1, T=256, H=2, dk=128, dv=128, seed=8)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_strong_decay(gate, dtype):
    """Fast-forgetting gates, alpha = sigmoid(N(-2, 0.5)) (per channel for KDA)."""
    announce("backward %s %s strong decay" % (gate, dtype))
    _check(gate, dtype, B=1, T=200, H=2, dk=64, dv=64, seed=12, alpha_mean=-2.0)


def test_backward_t0_copies_the_state_gradient():
    B, H, dk, dv = 2, 3, 32, 32
    dst = torch.randn(B, H, dk, dv, device="cuda")
    e = torch.empty(B, 0, H, dk, device="cuda")
    ev = torch.empty(B, 0, H, dv, device="cuda")
    ea = torch.empty(B, 0, H, device="cuda")
    ds0 = torch.full((B, H, dk, dv), 7.0, device="cuda")
    announce("backward T=0")
    gdr.gdr_chunk_backward("gdn", e, e, ev, ea, ea, None, ev, dst, e.clone(), e.clone(), ev.clone(),
                           ea.clone(), ea.clone(), ds0)
    torch.cuda.synchronize()
    assert torch.equal(ds0, dst)


def _full_size(gate, name, seed=31):
    """The backward at the prefill workload's full shape, in the launch
    configuration the benchmark times, against the oracle on every head over
    the whole length (one head per task in CPU-only worker processes)."""
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    rng = np.random.default_rng(seed)
    do = synth.bf16_round(rng.standard_normal((B, T, H, dv)).astype(np.float32))
    dst = (0.1 * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    announce("backward %s bf16 full size %s, every head" % (gate, name))
    got = _run(gate, "bf16", inp, do, dst, 1.0)
    errs = backward_errors_every_head(inp, do, dst, got)
    assert len(errs) == B * H
    for (b, h), e in sorted(errs.items()):
        for key, val in e.items():
            assert val <= TOL["bf16"], "%s[b=%d,h=%d]: max|err| / max|ref| = %.3e > %.1e" % (key, b, h, val, TOL["bf16"])


def test_backward_gdn_full_size():
    _full_size("gdn", "gdn_prefill_b4_t8192_h32_d128")


def test_backward_kda_full_size():
    _full_size("kda", "kda_prefill_b1_t32768_h32_d128")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_zero_gate_token(gate, dtype):
    """alpha = 0 at one token (the state is reset there).  The kernels take
    log(alpha) floored at -40; the gate's gradient at that token is summed
    from the terms that carry alpha, so it matches the oracle's value at
    alpha = 0 like every other gradient."""
    inp, do, dst = _case(gate, dtype, B=1, T=100, H=2, dk=32, dv=32, seed=12)
    inp["alpha"][:, 70] = 0.0
    announce("backward %s %s alpha=0 at t=70" % (gate, dtype))
    got = _run(gate, dtype, inp, do, dst, 0.9)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["s0"], do, dst, scale=0.9)
    for key in ("dq", "dk", "dv", "dalpha", "dbeta", "ds0"):
        assert_close(got[key], ref[key], TOL[dtype], key)
    assert_close(got["dalpha"][:, 70], ref["dalpha"][:, 70], TOL[dtype], "dalpha at the zero gate")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_backward_many_zero_gates(gate):
    """Several zero gates in one chunk and across chunks (KDA: whole channels
    at every token, a few channels at one token), d = 64."""
    inp, do, dst = _case(gate, "f32", B=1, T=200, H=3, dk=64, dv=64, seed=13)
    a = inp["alpha"]
    if gate == "gdn":
        a[:, [3, 20, 21, 63, 64, 130], 0] = 0.0
        a[:, 100:110, 1] = 0.0
    else:
        a[:, :, 0, 5] = 0.0            # channel 5 of head 0 at every token
        a[:, 40, 1, :16] = 0.0         # 16 channels of head 1 at one token
        a[:, 120:140, 2, 32:] = 0.0    # half the channels of head 2 across a chunk boundary
    announce("backward %s many zero gates" % gate)
    got = _run(gate, "f32", inp, do, dst, 0.8)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["s0"], do, dst, scale=0.8)
    for key in ("dq", "dk", "dv", "dalpha", "dbeta", "ds0"):
        assert_close(got[key], ref[key], TOL["f32"], key)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_backward_deterministic(gate):
    """Two calls on the same inputs give bitwise equal gradients (every sum
    runs in a fixed order), with and without a zero gate."""
    inp, do, dst = _case(gate, "bf16", B=2, T=300, H=4, dk=128, dv=128, seed=14)
    inp["alpha"][:, 77] = 0.0
    announce("backward %s deterministic" % gate)
    first = _run(gate, "bf16", inp, do, dst, 1.0)
    second = _run(gate, "bf16", inp, do, dst, 1.0)
    for key in first:
        assert np.array_equal(first[key], second[key]), key


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_backward_zero_beta_and_single_token(gate):
    """beta = 0 on half the tokens (no write there), and a one-token sequence."""
    inp, do, dst = _case(gate, "f32", B=2, T=90, H=2, dk=16, dv=16, seed=13)
    inp["beta"][:, ::2] = 0.0
    announce("backward %s beta=0 on even tokens" % gate)
    got = _run(gate, "f32", inp, do, dst, 1.0)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["s0"], do, dst)
    for key in ("dq", "dk", "dv", "dalpha", "dbeta", "ds0"):
        assert_close(got[key], ref[key], TOL["f32"], key)
    one, do1, dst1 = _case(gate, "f32", B=1, T=1, H=3, dk=64, dv=32, seed=14)
    announce("backward %s T=1" % gate)
    got = _run(gate, "f32", one, do1, dst1, 0.5)
    ref = oracle.backward(one["q"], one["k"], one["v"], one["alpha"], one["beta"], one["s0"], do1, dst1, scale=0.5)
    for key in ("dq", "dk", "dv", "dalpha", "dbeta", "ds0"):
        assert_close(got[key], ref[key], TOL["f32"], key)


@pytest.mark.parametrize("gate,dk,dv", [("gdn", 64, 32), ("kda", 16, 64)])
def test_backward_many_heads_wide_slices(gate, dk, dv):
    """Enough heads that the forward chain takes wide slices (32 columns for
    dv = 32, 64 for dv = 64; one workgroup per CU still); the oracle on
    every head."""
    inp, do, dst = _case(gate, "f32", B=8, T=70, H=32, dk=dk, dv=dv, seed=15)
    announce("backward %s wide slices B=8 H=32 dk=%d dv=%d" % (gate, dk, dv))
    got = _run(gate, "f32", inp, do, dst, 1.0)
    errs = backward_errors_every_head(inp, do, dst, got)
    assert len(errs) == 8 * 32
    for (b, h), e in sorted(errs.items()):
        for key, val in e.items():
            assert val <= TOL["f32"], "%s[%d,%d]: max|err| / max|ref| = %.3e > %.1e" % (key, b, h, val, TOL["f32"])


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_backward_graph_replays_match_eager(gate):
    """The backward (five launches, workspace passed in) captured in a HIP
    graph and replayed several times with eager work in between: every replay
    matches an eager call (bitwise where the kernels are deterministic; dalpha
    and dbeta sum a few terms with LDS atomics, so to 1e-6 of their scale)."""
    inp, do, dst = _case(gate, "bf16", B=2, T=150, H=4, dk=64, dv=64, seed=16)
    d = {key: to_dev(val, "bf16" if key in ("q", "k", "v") else "f32") for key, val in inp.items()}
    g_o, g_st = to_dev(do, "bf16"), to_dev(dst, "f32")
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    need = gdr.gdr_chunk_backward_workspace_bytes(gate, torch.bfloat16, B, T, H, dk, dv)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def outputs():
        return [torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"]),
                torch.empty_like(d["alpha"]), torch.empty_like(d["beta"]),
                torch.empty(B, H, dk, dv, device="cuda")]

    def call(out):
        gdr.gdr_chunk_backward(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["s0"], g_o, g_st,
                               *out, workspace=ws)

    og, oe = outputs(), outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(outputs())
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(og)
    announce("backward %s graph replays" % gate)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        call(oe)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(og, oe)):
            if i in (3, 4):
                scale = float(y.abs().max())
                assert float((x - y).abs().max()) <= 1e-6 * max(scale, 1e-30), (rep, i)
            else:
                assert torch.equal(x, y), (rep, i)
        junk = torch.randn(4096, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        del junk


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_ranges_bitwise(gate, dtype):
    """A workspace below the one-pass size runs the sequence in chunk ranges
    (a forward pass for each range's start state, then the ranges from the
    last): every gradient is bitwise the one-pass result, for ranges of 1, 2
    and 3 chunks over a ragged 5-chunk sequence with a zero gate, with and
    without S0 and dS_T."""
    B, T, H, dk, dv = 2, 300, 3, 64, 32
    inp, do, dst = _case(gate, dtype, B, T, H, dk, dv, seed=31)
    inp["alpha"][:, 150] = 0.0
    announce("backward %s %s ranges" % (gate, dtype))
    ref = _run(gate, dtype, inp, do, dst, 0.9)
    full = gdr.gdr_chunk_backward_workspace_bytes(gate, torch.float32 if dtype == "f32" else torch.bfloat16,
                                                  B, T, H, dk, dv)
    for rc in (1, 2, 3):
        need = gdr.gdr_chunk_backward_workspace_bytes_ranged(
            gate, torch.float32 if dtype == "f32" else torch.bfloat16, B, T, H, dk, dv, rc)
        assert 0 < need < full
        got = _run(gate, dtype, inp, do, dst, 0.9, ws_bytes=need)
        for key in ref:
            assert np.array_equal(got[key], ref[key]), (rc, key)
    inp0, do0, _ = _case(gate, dtype, B, T, H, dk, dv, seed=32, s0=False, dst=False)
    ref0 = _run(gate, dtype, inp0, do0, None, 0.9, want_ds0=False)
    need = gdr.gdr_chunk_backward_workspace_bytes_ranged(
        gate, torch.float32 if dtype == "f32" else torch.bfloat16, B, T, H, dk, dv, 2)
    got0 = _run(gate, dtype, inp0, do0, None, 0.9, want_ds0=False, ws_bytes=need)
    for key in ref0:
        if ref0[key] is not None:
            assert np.array_equal(got0[key], ref0[key]), key


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_backward_ranges_full_size(gate):
    """At the prefill workload's shape, a workspace of at most 2 GB (GDN: 32
    chunks per range, KDA: 128) gives the one-pass gradients bitwise, every
    head and token."""
    name = "gdn_prefill_b4_t8192_h32_d128" if gate == "gdn" else "kda_prefill_b1_t32768_h32_d128"
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    rng = np.random.default_rng(77)
    do = synth.bf16_round(rng.standard_normal((w.B, w.T, w.H, w.dv)).astype(np.float32))
    dst = (0.1 * rng.standard_normal((w.B, w.H, w.dk, w.dv))).astype(np.float32)
    rc = 32 if gate == "gdn" else 128
    need = gdr.gdr_chunk_backward_workspace_bytes_ranged(gate, torch.bfloat16, w.B, w.T, w.H, w.dk, w.dv, rc)
    assert need <= 2 * 10 ** 9
    announce("backward %s full size, ranged workspace %.2f GB" % (gate, need / 1e9))
    ref = _run(gate, "bf16", inp, do, dst, 1.0)
    got = _run(gate, "bf16", inp, do, dst, 1.0, ws_bytes=need)
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key
