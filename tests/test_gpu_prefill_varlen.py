"""GPU parity of the packed variable-length prefill with pooled states.

Every sequence is checked against the float64 recurrence run on that
sequence alone (from its pool row, or zeros), on its outputs and on its
final pool row; rows no sequence uses stay untouched bitwise.  Equal-length
sequences with the identity slot map give bitwise the uniform call.
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

LENS = [1, 63, 64, 0, 65, 200, 130]
SLOTS = [4, 0, 7, 2, 5, 1, 3]  # rows of an 9-row pool; rows 6 and 8 are unused
HAS = [1, 0, 1, 1, 1, 0, 1]


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _workload(gate, dtype, dk=64, dv=64):
    base = synth.WORKLOADS["gdn_prefill_b4_t8192_h32_d128" if gate == "gdn" else "kda_prefill_b1_t32768_h32_d128"]
    return replace(base, dtype=dtype, dk=dk, dv=dv)


def _packed_inputs(w, lens, H, seed):
    """Draws each sequence with the workload's distributions and packs them."""
    seqs = [synth.make_inputs(w, B=1, T=max(n, 1), H=H, seed=seed + i, s0="zero") for i, n in enumerate(lens)]
    cat = lambda key: np.ascontiguousarray(np.concatenate([s[key][0, :n] for s, n in zip(seqs, lens)], axis=0))
    return {k: cat(k) for k in ("q", "k", "v", "alpha", "beta")}


def _run(gate, dtype, inp, lens, slots, has, pool0, max_T=None, flags=0):
    dev = {k: to_dev(v, dtype if k in ("q", "k", "v") else "f32") for k, v in inp.items()}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    hs = None if has is None else torch.tensor(has, dtype=torch.int32, device="cuda")
    states = torch.from_numpy(pool0.copy()).cuda()
    total_T, H = inp["beta"].shape
    dv = inp["v"].shape[-1]
    o = torch.full((total_T, H, dv), 7.0, device="cuda", dtype=dev["q"].dtype)
    gdr.gdr_chunk_prefill_varlen_ex(gate, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], cu, sl,
                                    states, o, has_state=hs, max_seqlen=max_T, flags=flags)
    torch.cuda.synchronize()
    return to_host64(o), to_host64(states)


def _check(gate, dtype, H=3, dk=64, dv=64, lens=LENS, slots=SLOTS, has=HAS, flags=0):
    w = _workload(gate, dtype, dk, dv)
    inp = _packed_inputs(w, lens, H, seed=40)
    rng = np.random.default_rng(5)
    pool0 = (0.02 * rng.standard_normal((9, H, dk, dv))).astype(np.float32)
    o, pool = _run(gate, dtype, inp, lens, slots, has, pool0, flags=flags)
    tol = TOL[dtype]
    off = np.concatenate([[0], np.cumsum(lens)])
    for n, L in enumerate(lens):
        r = slots[n]
        if L == 0:
            assert np.array_equal(pool[r], pool0[r]), "empty sequence changed its row"
            continue
        sl = slice(off[n], off[n + 1])
        s0 = pool0[r][None] if has[n] else None
        x = {k: inp[k][sl][None] for k in ("q", "k", "v", "alpha", "beta")}
        o_ref, s_ref = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], s0)
        assert_close(o[sl], o_ref[0], tol, "o of sequence %d" % n)
        assert_close(pool[r], s_ref[0], tol, "state of sequence %d" % n)
    for r in (6, 8):
        assert np.array_equal(pool[r], pool0[r]), "unused row %d changed" % r


@pytest.mark.parametrize("gate,sched", [("gdn", "fused"), ("gdn", "split"), ("kda", "split")])
def test_varlen_bf16_matches_oracle(gate, sched):
    announce("prefill varlen %s bf16 %s" % (gate, sched))
    _check(gate, "bf16", flags={"fused": gdr.SCHED_FUSED, "split": gdr.SCHED_SPLIT}[sched])


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_varlen_f32_matches_oracle(gate):
    announce("prefill varlen %s f32" % gate)
    _check(gate, "f32", dk=32, dv=32)


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_varlen_d128_all_have_state(gate):
    announce("prefill varlen %s bf16 d=128" % gate)
    _check(gate, "bf16", H=2, dk=128, dv=128, has=[1] * len(LENS))


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_varlen_equal_lengths_is_the_uniform_call_bitwise(gate):
    """Equal lengths, slot n = sequence n, all reading their rows: bitwise the
    [B, T, H, .] call (the packed layout is the same memory)."""
    w = _workload(gate, "bf16")
    B, T, H = 3, 130, 4
    inp = synth.make_inputs(w, B=B, T=T, H=H, seed=9, s0="normal")
    announce("prefill varlen vs uniform %s" % gate)
    dev = {k: to_dev(v, "bf16" if k in ("q", "k", "v") else "f32") for k, v in inp.items()}
    s_out = torch.empty_like(dev["s0"])
    o_u = torch.empty(B, T, H, w.dv, device="cuda", dtype=torch.bfloat16)
    gdr.gdr_chunk_prefill(gate, dev["q"], dev["k"], dev["v"], dev["alpha"], dev["beta"], dev["s0"], s_out, o_u)
    packed = {k: np.ascontiguousarray(inp[k].reshape((B * T,) + inp[k].shape[2:]))
              for k in ("q", "k", "v", "alpha", "beta")}
    o_v, pool = _run(gate, "bf16", packed, [T] * B, list(range(B)), None, inp["s0"], max_T=T)
    torch.cuda.synchronize()
    assert np.array_equal(o_v, to_host64(o_u).reshape(B * T, H, w.dv))
    assert np.array_equal(pool, to_host64(s_out))


def test_varlen_bad_slot_is_skipped():
    """A slot outside the pool skips its sequence: its outputs keep their
    previous contents and no pool row changes because of it."""
    w = _workload("gdn", "bf16")
    lens, slots, has = [70, 30], [1, 9], [1, 1]
    inp = _packed_inputs(w, lens, 2, seed=3)
    pool0 = (0.02 * np.random.default_rng(1).standard_normal((9, 2, 64, 64))).astype(np.float32)
    announce("prefill varlen bad slot")
    o, pool = _run("gdn", "bf16", inp, lens, slots, has, pool0)
    assert np.all(o[70:] == 7.0)
    for r in range(9):
        if r != 1:
            assert np.array_equal(pool[r], pool0[r]), r
