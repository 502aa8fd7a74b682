"""GPU parity of the fused input prologue (L2-normalised q, k; sigmoid gates).

The kernels take raw q, k and gate logits; the reference is the float64
recurrence on the oracle's prologue of the same raw inputs.  flags == 0 must
give bitwise the calls without a prologue.
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

NORM, SIG = gdr.PRO_L2NORM_QK, gdr.PRO_SIGMOID


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _workload(kind, gate, dtype, dk=128, dv=128):
    name = {("decode", "gdn"): "gdn_decode_b64_h32_d128", ("decode", "kda"): "kda_decode_b256_h32_d128",
            ("prefill", "gdn"): "gdn_prefill_b4_t8192_h32_d128",
            ("prefill", "kda"): "kda_prefill_b1_t32768_h32_d128"}[(kind, gate)]
    return replace(synth.WORKLOADS[name], dtype=dtype, dk=dk, dv=dv)


def _reference_inputs(raw, flags):
    """What the kernels should see after the prologue the flags ask for."""
    q, k, a, b = oracle.prologue(raw["q"], raw["k"], raw["alpha"], raw["beta"],
                                 norm_qk=bool(flags & NORM), sigmoid_gates=bool(flags & SIG))
    return q, k, a, b


def _raw(w, flags, B, T, H, seed, zero_rows=False, alpha_mean=2.0):
    raw = synth.make_raw_inputs(w, B=B, T=T, H=H, seed=seed, s0="normal", alpha_mean=alpha_mean)
    if not flags & NORM:  # q, k given normalised (raw ones would make the recurrence diverge)
        normed = synth.make_inputs(w, B=B, T=T, H=H, seed=seed, s0="normal")
        raw["q"], raw["k"] = normed["q"], normed["k"]
    if not flags & SIG:  # gates given as values in (0, 1)
        raw["alpha"] = (1.0 / (1.0 + np.exp(-raw["alpha"].astype(np.float64)))).astype(np.float32)
        raw["beta"] = (1.0 / (1.0 + np.exp(-raw["beta"].astype(np.float64)))).astype(np.float32)
    if zero_rows:  # a zero q row and a zero k row: normalised to zero, not NaN
        raw["q"][0, T // 2, 0] = 0.0
        raw["k"][-1, T - 1, H - 1] = 0.0
    return raw


def _dev(raw, dtype):
    return {key: to_dev(val, dtype if key in ("q", "k", "v") else "f32") for key, val in raw.items()}


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flags", [NORM, SIG, NORM | SIG])
@pytest.mark.parametrize("dk,dv", [(128, 128), (32, 64)])
def test_decode_prologue_matches_oracle(gate, dtype, flags, dk, dv):
    w = _workload("decode", gate, dtype, dk, dv)
    raw = _raw(w, flags, B=3, T=1, H=5, seed=11, zero_rows=True)
    announce("decode prologue %s %s flags=%d dk=%d dv=%d" % (gate, dtype, flags, dk, dv))
    step = {key: (val[:, 0].copy() if key != "s0" else val) for key, val in raw.items()}
    d = _dev(step, dtype)
    state = d["s0"].clone()
    o = torch.empty_like(d["v"])
    gdr.gdr_decode_step_ex(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], state, o,
                           flags=flags, scale=0.5)
    torch.cuda.synchronize()
    q, k, a, b = _reference_inputs(step, flags)
    o_ref, s_ref = oracle.decode_step(q, k, step["v"], a, b, step["s0"], scale=0.5)
    assert_close(to_host64(o), o_ref, TOL[dtype], "o")
    assert_close(to_host64(state), s_ref, TOL[dtype], "state")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_decode_prologue_full_size(gate):
    w = _workload("decode", gate, "bf16")
    raw = _raw(w, NORM | SIG, B=w.B, T=1, H=w.H, seed=3)
    announce("decode prologue %s full size B=%d" % (gate, w.B))
    step = {key: (val[:, 0].copy() if key != "s0" else val) for key, val in raw.items()}
    d = _dev(step, "bf16")
    state = d["s0"].clone()
    o = torch.empty_like(d["v"])
    gdr.gdr_decode_step_ex(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], state, o, flags=NORM | SIG)
    torch.cuda.synchronize()
    q, k, a, b = _reference_inputs(step, NORM | SIG)
    o_ref, s_ref = oracle.decode_step(q, k, step["v"], a, b, step["s0"])
    assert_close(to_host64(o), o_ref, TOL["bf16"], "o")
    assert_close(to_host64(state), s_ref, TOL["bf16"], "state")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_decode_flags_zero_is_the_plain_step_bitwise(gate):
    w = _workload("decode", gate, "bf16")
    inp = synth.make_inputs(w, B=4, H=8)
    d = _dev({key: (val[:, 0].copy() if key != "s0" else val) for key, val in inp.items()}, "bf16")
    announce("decode_ex flags=0 vs decode %s" % gate)
    s1, s2 = d["s0"].clone(), d["s0"].clone()
    o1, o2 = torch.empty_like(d["v"]), torch.empty_like(d["v"])
    gdr.gdr_decode_step(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], s1, o1)
    gdr.gdr_decode_step_ex(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], s2, o2, flags=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def _prefill(gate, dtype, d, flags, B, T, H, dv):
    s_out = torch.empty(B, H, d["q"].shape[-1], dv, device="cuda")
    o = torch.empty(B, T, H, dv, device="cuda", dtype=d["q"].dtype)
    gdr.gdr_chunk_prefill_ex(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["s0"], s_out, o,
                             flags=flags, scale=0.75)
    torch.cuda.synchronize()
    return to_host64(o), to_host64(s_out)


def _check_prefill(gate, dtype, flags, dk, dv, B=2, T=200, H=3, seed=17, zero_rows=True, alpha_mean=2.0):
    w = _workload("prefill", gate, dtype, dk, dv)
    raw = _raw(w, flags, B=B, T=T, H=H, seed=seed, zero_rows=zero_rows, alpha_mean=alpha_mean)
    o, s = _prefill(gate, dtype, _dev(raw, dtype), flags, B, T, H, dv)
    q, k, a, b = _reference_inputs(raw, flags)
    o_ref, s_ref = oracle.recurrent(q, k, raw["v"], a, b, raw["s0"], scale=0.75)
    assert_close(o, o_ref, TOL[dtype], "o")
    assert_close(s, s_ref, TOL[dtype], "S_T")


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("flags", [NORM, SIG, NORM | SIG])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_prefill_bf16_prologue_matches_oracle(gate, flags, dk, dv):
    announce("prefill prologue bf16 %s flags=%d dk=%d dv=%d" % (gate, flags, dk, dv))
    _check_prefill(gate, "bf16", flags, dk, dv)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dk", [16, 32])
def test_prefill_bf16_prologue_small_heads(gate, dk):
    """Rows of 2 and 4 octets (GDN: the smaller lane-group sums; KDA: waves
    without a row share, which still take part in the barrier)."""
    announce("prefill prologue bf16 %s dk=%d" % (gate, dk))
    _check_prefill(gate, "bf16", NORM | SIG, dk, 32)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_prefill_f32_prologue_matches_oracle(gate):
    announce("prefill prologue f32 %s" % gate)
    _check_prefill(gate, "f32", NORM | SIG, 64, 32, T=130)


def test_prefill_sigmoid_in_the_split_gdn_schedule():
    announce("prefill prologue bf16 gdn split sigmoid")
    _check_prefill("gdn", "bf16", SIG | gdr.SCHED_SPLIT, 128, 128)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_prefill_prologue_with_explicit_default_schedule(gate):
    """Naming the default schedule explicitly gives the default call bitwise."""
    sched = gdr.SCHED_FUSED if gate == "gdn" else gdr.SCHED_SPLIT
    w = _workload("prefill", gate, "bf16", 64, 64)
    raw = _raw(w, NORM | SIG, B=2, T=150, H=3, seed=21)
    d = _dev(raw, "bf16")
    announce("prefill prologue bf16 %s explicit schedule" % gate)
    a = _prefill(gate, "bf16", d, NORM | SIG, 2, 150, 3, 64)
    b = _prefill(gate, "bf16", d, NORM | SIG | sched, 2, 150, 3, 64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_prefill_sigmoid_very_negative_logits(gate):
    """Gate logits around -6 (some below -8): the chunked paths take
    log2 sigmoid of the logit directly."""
    announce("prefill prologue bf16 %s negative logits" % gate)
    _check_prefill(gate, "bf16", NORM | SIG, 128, 128, T=300, alpha_mean=-6.0)


def test_prefill_gdn_long_sequence_prologue():
    """Every chunk position of a longer sequence (prep runs two chunks ahead)."""
    announce("prefill prologue bf16 gdn T=1000")
    _check_prefill("gdn", "bf16", NORM | SIG, 128, 128, B=1, T=1000, H=2, zero_rows=False)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_prefill_flags_zero_is_the_plain_call_bitwise(gate):
    w = _workload("prefill", gate, "bf16")
    inp = synth.make_inputs(w, B=2, T=150, H=4, seed=2, s0="normal")
    d = _dev(inp, "bf16")
    announce("prefill_ex flags=0 vs prefill %s" % gate)
    o1 = torch.empty(2, 150, 4, 128, device="cuda", dtype=torch.bfloat16)
    o2 = torch.empty_like(o1)
    s1, s2 = torch.empty_like(d["s0"]), torch.empty_like(d["s0"])
    gdr.gdr_chunk_prefill(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["s0"], s1, o1)
    gdr.gdr_chunk_prefill_ex(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["s0"], s2, o2, flags=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("gate,name", [
    ("gdn", "gdn_prefill_b4_t8192_h32_d128"),
    ("kda", "kda_prefill_b1_t32768_h32_d128"),
])
def test_prefill_prologue_full_size(gate, name):
    """The prologue at the prefill workload's full shape (the benchmark's
    launch configuration); the oracle on every head over the whole length,
    and each head's error checked on its own."""
    w = synth.WORKLOADS[name]
    raw = synth.make_raw_inputs(w)
    B, T, H, dv = w.B, w.T, w.H, w.dv
    announce("prefill prologue full size %s, every head" % name)
    o, s = _prefill(gate, "bf16", _dev(raw, "bf16"), NORM | SIG, B, T, H, dv)
    q, k, a, bt = oracle.prologue(raw["q"], raw["k"], raw["alpha"], raw["beta"])
    o_ref, s_ref = oracle.recurrent(q, k, raw["v"], a, bt, raw["s0"], scale=0.75)
    for b in range(B):
        for h in range(H):
            assert_close(o[b, :, h], o_ref[b, :, h], TOL["bf16"], "o[b=%d,h=%d]" % (b, h))
            assert_close(s[b, h], s_ref[b, h], TOL["bf16"], "S_T[b=%d,h=%d]" % (b, h))


@pytest.mark.parametrize("gate", ["gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_multi_prologue_matches_stepped_oracle(gate, dtype):
    """The verify step on raw inputs: every token's prologue, then the
    float64 recurrence token by token; flags 0 is the plain call bitwise."""
    w = _workload("decode", gate, dtype, 64, 64)
    T = 5
    raw = _raw(w, NORM | SIG, B=3, T=T, H=4, seed=19, zero_rows=True)
    d = _dev(raw, dtype)
    state = d["s0"].clone()
    o = torch.empty(3, T, 4, 64, device="cuda", dtype=d["q"].dtype)
    states = torch.empty(3, T, 4, 64, 64, device="cuda")
    announce("decode_multi prologue %s %s" % (gate, dtype))
    gdr.gdr_decode_multi_ex(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], state, o, states,
                            flags=NORM | SIG, scale=0.5)
    torch.cuda.synchronize()
    q, k, a, b = _reference_inputs(raw, NORM | SIG)
    s = raw["s0"]
    for t in range(T):
        sl = slice(t, t + 1)
        o_ref, s = oracle.recurrent(q[:, sl], k[:, sl], raw["v"][:, sl], a[:, sl], b[:, sl], s, scale=0.5)
        assert_close(to_host64(o)[:, t], o_ref[:, 0], TOL[dtype], "o_%d" % t)
        assert_close(to_host64(states)[:, t], s, TOL[dtype], "S_%d" % (t + 1))
    assert_close(to_host64(state), s, TOL[dtype], "S_T")
    # flags 0: bitwise the plain call
    plain = _dev(synth.make_inputs(w, B=3, T=T, H=4, seed=19, s0="normal"), dtype)
    s1, s2 = plain["s0"].clone(), plain["s0"].clone()
    o1, o2 = torch.empty_like(o), torch.empty_like(o)
    gdr.gdr_decode_multi(gate, plain["q"], plain["k"], plain["v"], plain["alpha"], plain["beta"], s1, o1)
    gdr.gdr_decode_multi_ex(gate, plain["q"], plain["k"], plain["v"], plain["alpha"], plain["beta"], s2, o2,
                            flags=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_prefill_varlen_prologue_matches_oracle(gate):
    """Packed prompts on raw inputs: each sequence against the float64
    recurrence on its own prologue'd inputs, from its pool row."""
    w = _workload("prefill", gate, "bf16", 64, 64)
    lens, slots, has = [1, 70, 0, 130], [2, 0, 3, 1], [1, 0, 1, 1]
    H = 3
    seqs = [_raw(w, NORM | SIG, B=1, T=max(n, 1), H=H, seed=50 + i) for i, n in enumerate(lens)]
    cat = lambda key: np.ascontiguousarray(np.concatenate([sq[key][0, :n] for sq, n in zip(seqs, lens)], axis=0))
    packed = {key: cat(key) for key in ("q", "k", "v", "alpha", "beta")}
    pool0 = (0.02 * np.random.default_rng(3).standard_normal((4, H, 64, 64))).astype(np.float32)
    d = _dev(packed, "bf16")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    pool = torch.from_numpy(pool0.copy()).cuda()
    o = torch.zeros(sum(lens), H, 64, device="cuda", dtype=torch.bfloat16)
    announce("prefill varlen prologue %s" % gate)
    gdr.gdr_chunk_prefill_varlen_ex(gate, d["q"], d["k"], d["v"], d["alpha"], d["beta"], cu,
                                    torch.tensor(slots, dtype=torch.int32, device="cuda"), pool, o,
                                    has_state=torch.tensor(has, dtype=torch.int32, device="cuda"),
                                    flags=NORM | SIG)
    torch.cuda.synchronize()
    o, pool = to_host64(o), to_host64(pool)
    off = np.concatenate([[0], np.cumsum(lens)])
    for i, n in enumerate(lens):
        r = slots[i]
        if n == 0:
            assert np.array_equal(pool[r], pool0[r])
            continue
        sl = slice(off[i], off[i + 1])
        q, k, a, b = oracle.prologue(packed["q"][sl][None], packed["k"][sl][None], packed["alpha"][sl][None],
                                     packed["beta"][sl][None])
        o_ref, s_ref = oracle.recurrent(q, k, packed["v"][sl][None], a, b, pool0[r][None] if has[i] else None)
        assert_close(o[sl], o_ref[0], TOL["bf16"], "o of sequence %d" % i)
        assert_close(pool[r], s_ref[0], TOL["bf16"], "state of sequence %d" % i)
