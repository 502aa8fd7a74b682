"""The per-head oracle comparison used by the full-size backward tests
(tests/oracle_pool.py), checked on the CPU: gradients equal to the oracle's
give errors at rounding level on every head, and a mistake planted in one
head's gradient shows up in that head and key only."""
import numpy as np

import oracle
import synth
from oracle_pool import KEYS, backward_errors_every_head


def _case():
    w = synth.WORKLOADS["kda_prefill_b1_t32768_h32_d128"]
    inp = synth.make_inputs(w, B=2, T=150, H=3, seed=4)
    rng = np.random.default_rng(5)
    do = rng.standard_normal((2, 150, 3, w.dv)).astype(np.float32)
    dst = (0.1 * rng.standard_normal((2, 3, w.dk, w.dv))).astype(np.float32)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["s0"], do, dst)
    return inp, do, dst, ref


def test_every_head_matches_itself_and_finds_a_planted_mistake():
    inp, do, dst, ref = _case()
    got = {key: ref[key].copy() for key in KEYS + ("ds0",)}
    errs = backward_errors_every_head(inp, do, dst, got, workers=3)
    assert sorted(errs) == [(b, h) for b in range(2) for h in range(3)]
    assert max(max(e.values()) for e in errs.values()) < 1e-12
    got["dalpha"][1, 40:60, 2] *= 1.02
    errs = backward_errors_every_head(inp, do, dst, got, workers=3)
    for (b, h), e in errs.items():
        for key, val in e.items():
            if (b, h, key) == (1, 2, "dalpha"):
                assert val > 1e-3
            else:
                assert val < 1e-12, (b, h, key, val)
