"""Pins for the float64 CPU oracle.

The pages print no formula, worked example or value for the mixer, so the
oracle is pinned to facts fixed by the mathematics of the gated delta rule:
special cases with a closed form, exact (bitwise) reductions, invariants, an
exact rational computation on a tiny case, and the agreement of three
independently written forms (token-by-token C, chunked C, dense NumPy).
Several cases use dk != dv so that a transposed state or an operand applied
on the wrong axis cannot pass.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rand_case(B=2, T=37, H=3, dk=5, dv=7, kda=False, seed=0, s0=True, unit_k=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    if unit_k:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    ashape = (B, T, H, dk) if kda else (B, T, H)
    alpha = 1.0 / (1.0 + np.exp(-(2.0 + 0.5 * r.standard_normal(ashape))))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    S0 = 0.3 * r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, alpha, beta, S0


def _close(a, b, tol):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.abs(b).max()) if b.size else 1.0)
    err = float(np.abs(a - b).max()) if b.size else 0.0
    assert err <= tol * scale, "max abs err %.3e > %.1e * %.3e" % (err, tol, scale)


# --- F1: beta = 0, alpha = 1 leaves the state unchanged --------------------

@pytest.mark.parametrize("kda", [False, True])
def test_identity_when_beta0_alpha1(kda):
    q, k, v, alpha, beta, S0 = _rand_case(kda=kda, seed=1)
    alpha = np.ones_like(alpha)
    beta = np.zeros_like(beta)
    o, sT = oracle.recurrent(q, k, v, alpha, beta, S0)
    assert np.array_equal(sT, S0)  # bitwise
    # o_t = S_0^T q_t, computed with a library contraction.
    expect = np.einsum("bhij,bthi->bthj", S0, q)
    _close(o, expect, 1e-14)
    oc, sc = oracle.chunked(q, k, v, alpha, beta, S0, chunk=8)
    _close(sc, S0, 1e-14)
    _close(oc, expect, 1e-14)


# --- F2: alpha = 1, beta = 1, unit k: the delta rule recalls v exactly -----

@pytest.mark.parametrize("kda", [False, True])
def test_exact_recall(kda):
    q, k, v, alpha, beta, S0 = _rand_case(kda=kda, seed=2, dk=6, dv=4)
    alpha = np.ones_like(alpha)
    beta = np.ones_like(beta)
    # With q_t = k_t the output is S_t^T k_t, which must equal v_t.
    o, _ = oracle.recurrent(k, k, v, alpha, beta, S0)
    _close(o, v, 1e-13)


# --- F3: alpha = 0 reduces every step to a single rank-one write -----------

@pytest.mark.parametrize("kda", [False, True])
def test_zero_gate_is_rank_one(kda):
    q, k, v, alpha, beta, S0 = _rand_case(kda=kda, seed=3, T=1)
    alpha = np.zeros_like(alpha)
    o, sT = oracle.recurrent(q, k, v, alpha, beta, S0)
    expect = (beta[:, 0, :, None] * k[:, 0])[..., None] * v[:, 0][:, :, None, :]
    assert np.array_equal(sT, expect)  # bitwise: a single write of beta k v^T
    kq = (k[:, 0] * q[:, 0]).sum(-1)
    _close(o[:, 0], (beta[:, 0] * kq)[..., None] * v[:, 0], 1e-14)


def test_zero_gate_mid_sequence_forgets_history():
    q, k, v, alpha, beta, S0 = _rand_case(seed=4, T=9)
    alpha[:, 4] = 0.0
    o_full, s_full = oracle.recurrent(q, k, v, alpha, beta, S0)
    # After the zero gate, the state no longer depends on anything before it.
    q2, k2, v2, a2, b2 = (x[:, 4:].copy() for x in (q, k, v, alpha, beta))
    o_tail, s_tail = oracle.recurrent(q2, k2, v2, a2, b2, None)
    _close(o_full[:, 4:], o_tail, 1e-14)
    _close(s_full, s_tail, 1e-14)


# --- F4: the chunked refactoring equals the definition ---------------------

@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("chunk", [1, 2, 4, 8, 16, 64])
@pytest.mark.parametrize("T", [1, 37, 64, 130])
def test_chunked_equals_recurrent(kda, chunk, T):
    q, k, v, alpha, beta, S0 = _rand_case(kda=kda, seed=5 + T, T=T, B=1, H=2)
    if T > 10:
        alpha[:, 10] = 0.0  # a zero gate inside a chunk must be legal
    o1, s1 = oracle.recurrent(q, k, v, alpha, beta, S0, scale=0.7)
    o2, s2 = oracle.chunked(q, k, v, alpha, beta, S0, scale=0.7, chunk=chunk)
    _close(o2, o1, 1e-12)
    _close(s2, s1, 1e-12)


# --- F5: dense brute force equals the rank-one form ------------------------

@pytest.mark.parametrize("kda", [False, True])
def test_brute_force_matches(kda):
    q, k, v, alpha, beta, S0 = _rand_case(kda=kda, seed=6, B=1, T=8, H=2, dk=4, dv=3,
                                          unit_k=False)
    o1, s1 = oracle.recurrent(q, k, v, alpha, beta, S0, scale=1.3)
    o2, s2 = oracle.brute(q, k, v, alpha, beta, S0, scale=1.3)
    _close(o1, o2, 1e-13)
    _close(s1, s2, 1e-13)


def _exact_dense(q, k, v, alpha, beta):
    """Exact rational arithmetic, dense matrices, one (b, h), zero S_0."""
    T, dk = len(q), len(q[0])
    dv = len(v[0])
    S = [[Fraction(0)] * dv for _ in range(dk)]
    outs = []
    for t in range(T):
        D = [[(alpha[t][i] if i == j else Fraction(0)) for j in range(dk)] for i in range(dk)]
        E = [[(Fraction(1) if i == j else Fraction(0)) - beta[t] * k[t][i] * k[t][j]
              for j in range(dk)] for i in range(dk)]
        M = [[sum(E[i][m] * D[m][j] for m in range(dk)) for j in range(dk)] for i in range(dk)]
        S = [[sum(M[i][m] * S[m][j] for m in range(dk)) + beta[t] * k[t][i] * v[t][j]
              for j in range(dv)] for i in range(dk)]
        outs.append([sum(S[i][j] * q[t][i] for i in range(dk)) for j in range(dv)])
    return outs, S


@pytest.mark.parametrize("kda", [False, True])
def test_exact_rational_tiny(kda):
    # Dyadic inputs: exactly representable in float64, exact in Fraction.
    r = np.random.default_rng(7)
    T, dk, dv = 4, 3, 2
    q = r.integers(-4, 5, (T, dk)) / 4.0
    k = r.integers(-4, 5, (T, dk)) / 4.0
    v = r.integers(-8, 9, (T, dv)) / 8.0
    beta = r.integers(1, 8, T) / 8.0
    alpha = (r.integers(1, 16, (T, dk)) / 16.0) if kda else (r.integers(1, 16, T) / 16.0)
    F = lambda a: [[Fraction(x) for x in row] for row in a]
    if kda:
        al = F(alpha)
    else:
        al = [[Fraction(a)] * dk for a in alpha]
    outs, S = _exact_dense(F(q), F(k), F(v), al, [Fraction(b) for b in beta])
    o, sT = oracle.recurrent(q[None, :, None], k[None, :, None], v[None, :, None],
                             alpha[None, :, None], beta[None, :, None])
    _close(o[0, :, 0], np.array([[float(x) for x in row] for row in outs]), 1e-15)
    _close(sT[0, 0], np.array([[float(x) for x in row] for row in S]), 1e-15)


# --- F6: a channel gate that is constant across channels is the scalar gate

def test_kda_with_constant_gate_equals_gdn():
    q, k, v, alpha, beta, S0 = _rand_case(seed=8)
    alpha_kda = np.repeat(alpha[..., None], q.shape[-1], axis=-1)
    o1, s1 = oracle.recurrent(q, k, v, alpha, beta, S0)
    o2, s2 = oracle.recurrent(q, k, v, alpha_kda, beta, S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    o3, s3 = oracle.chunked(q, k, v, alpha_kda, beta, S0, chunk=16)
    _close(o3, o1, 1e-12)
    _close(s3, s1, 1e-12)


# --- F7: splitting the sequence and stepping token by token ----------------

@pytest.mark.parametrize("kda", [False, True])
def test_split_and_decode_steps(kda):
    q, k, v, alpha, beta, S0 = _rand_case(kda=kda, seed=9, T=20)
    o, s = oracle.recurrent(q, k, v, alpha, beta, S0)
    o_a, s_a = oracle.recurrent(q[:, :7], k[:, :7], v[:, :7], alpha[:, :7], beta[:, :7], S0)
    o_b, s_b = oracle.recurrent(q[:, 7:], k[:, 7:], v[:, 7:], alpha[:, 7:], beta[:, 7:], s_a)
    assert np.array_equal(np.concatenate([o_a, o_b], axis=1), o)
    assert np.array_equal(s_b, s)
    st = S0.copy()
    for t in range(q.shape[1]):
        ot, st = oracle.decode_step(q[:, t], k[:, t], v[:, t], alpha[:, t], beta[:, t], st)
        assert np.array_equal(ot, o[:, t])
    assert np.array_equal(st, s)


# --- F8: value columns are independent -------------------------------------

def test_value_columns_independent():
    q, k, v, alpha, beta, S0 = _rand_case(seed=10, dv=9, kda=True)
    o, s = oracle.recurrent(q, k, v, alpha, beta, S0)
    cols = [1, 4, 8]
    o2, s2 = oracle.recurrent(q, k, v[..., cols], alpha, beta, S0[..., cols])
    _close(o2, o[..., cols], 1e-15)
    _close(s2, s[..., cols], 1e-15)


# --- F9: (S_0, v) -> (o, S_T) is linear -------------------------------------

def test_linear_in_state_and_values():
    q, k, v1, alpha, beta, S1 = _rand_case(seed=11, kda=True)
    _, _, v2, _, _, S2 = _rand_case(seed=12, kda=True)
    a, b = 0.75, -1.5
    o1, s1 = oracle.recurrent(q, k, v1, alpha, beta, S1)
    o2, s2 = oracle.recurrent(q, k, v2, alpha, beta, S2)
    o3, s3 = oracle.recurrent(q, k, a * v1 + b * v2, alpha, beta, a * S1 + b * S2)
    _close(o3, a * o1 + b * o2, 1e-13)
    _close(s3, a * s1 + b * s2, 1e-13)


# --- F10: scalar closed form at dk = dv = 1 --------------------------------

def test_scalar_closed_form():
    r = np.random.default_rng(13)
    T = 25
    q = r.standard_normal(T)
    k = r.choice([-1.0, 1.0], T)
    v = r.standard_normal(T)
    alpha = r.uniform(0, 1, T)
    beta = r.uniform(0, 1, T)
    s, outs = 0.4, []
    for t in range(T):
        s = alpha[t] * (1 - beta[t]) * s + beta[t] * k[t] * v[t]
        outs.append(q[t] * s)
    o, sT = oracle.recurrent(q.reshape(1, T, 1, 1), k.reshape(1, T, 1, 1),
                             v.reshape(1, T, 1, 1), alpha.reshape(1, T, 1),
                             beta.reshape(1, T, 1), np.full((1, 1, 1, 1), 0.4))
    _close(o.ravel(), np.array(outs), 1e-14)
    _close(sT.ravel(), [s], 1e-14)


# --- F11: contraction bound --------------------------------------------------

def test_state_norm_bound():
    q, k, v, alpha, beta, S0 = _rand_case(seed=14, kda=True, T=1, B=4, H=4, dk=8, dv=8)
    _, sT = oracle.recurrent(q, k, v, alpha, beta, S0)
    for b in range(4):
        for h in range(4):
            lhs = np.linalg.norm(sT[b, h], 2)
            rhs = np.linalg.norm(S0[b, h], 2) + beta[b, 0, h] * np.linalg.norm(v[b, 0, h])
            assert lhs <= rhs * (1 + 1e-12)


# --- scale and threading -----------------------------------------------------

def test_scale_is_a_pure_output_factor():
    q, k, v, alpha, beta, S0 = _rand_case(seed=15)
    o1, s1 = oracle.recurrent(q, k, v, alpha, beta, S0, scale=1.0)
    o2, s2 = oracle.recurrent(q, k, v, alpha, beta, S0, scale=0.125)
    assert np.array_equal(s1, s2)
    _close(o2, 0.125 * o1, 1e-15)


def test_thread_count_does_not_change_results():
    q, k, v, alpha, beta, S0 = _rand_case(seed=16, B=3, H=5, kda=True)
    a = oracle.recurrent(q, k, v, alpha, beta, S0, nthreads=1)
    b = oracle.recurrent(q, k, v, alpha, beta, S0, nthreads=7)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    c = oracle.chunked(q, k, v, alpha, beta, S0, chunk=4, nthreads=1)
    d = oracle.chunked(q, k, v, alpha, beta, S0, chunk=4, nthreads=6)
    assert all(np.array_equal(x, y) for x, y in zip(c, d))


def test_empty_sequence_copies_state():
    q, k, v, alpha, beta, S0 = _rand_case(seed=17, T=0)
    o, s = oracle.recurrent(q, k, v, alpha, beta, S0)
    assert o.shape[1] == 0 and np.array_equal(s, S0)
    o, s = oracle.chunked(q, k, v, alpha, beta, S0)
    assert np.array_equal(s, S0)


# ---- prologue (q/k L2 normalisation, gate sigmoids) ----

def test_prologue_unit_norm_parallel_and_scale_invariant():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 5, 3, 16))
    k = rng.standard_normal((2, 5, 3, 16)) * 7.0
    qn, kn, _, _ = oracle.prologue(q, k, np.zeros((2, 5, 3)), np.zeros((2, 5, 3)))
    for x, xn in ((q, qn), (k, kn)):
        assert np.allclose(np.linalg.norm(xn, axis=-1), 1.0, atol=1e-14)
        cos = np.sum(x * xn, axis=-1) / np.linalg.norm(x, axis=-1)
        assert np.allclose(cos, 1.0, atol=1e-14)  # same direction, positive factor
    q2, k2, _, _ = oracle.prologue(3.5 * q, 0.25 * k, np.zeros((2, 5, 3)), np.zeros((2, 5, 3)))
    assert np.allclose(q2, qn, atol=1e-15) and np.allclose(k2, kn, atol=1e-15)


def test_prologue_zero_vector_stays_zero():
    q = np.zeros((1, 1, 1, 8))
    q[0, 0, 0, 3] = 0.0
    qn, _, _, _ = oracle.prologue(q, q, np.zeros((1, 1, 1)), np.zeros((1, 1, 1)))
    assert np.all(qn == 0.0) and np.all(np.isfinite(qn))


def test_prologue_sigmoid_values():
    x = np.array([0.0, np.log(3.0), -np.log(3.0), 40.0, -40.0, 1000.0, -1000.0])
    _, _, a, b = oracle.prologue(np.ones((1, 8)), np.ones((1, 8)), x, -x, norm_qk=False)
    assert a[0] == 0.5
    assert abs(a[1] - 0.75) < 1e-15 and abs(a[2] - 0.25) < 1e-15  # 1/(1+1/3), 1/(1+3)
    assert np.allclose(a + b, 1.0, atol=1e-15)  # sigma(x) + sigma(-x) = 1
    assert a[5] == 1.0 and 0.0 <= a[6] < 1e-300 and np.all(np.isfinite(a))
    assert np.all((a >= 0.0) & (a <= 1.0))


def test_prologue_matches_the_input_generator():
    """The generator applies the same two steps to its raw draws (its own code)."""
    import synth
    w = synth.WORKLOADS["gdn_tiny_f32"]
    raw = synth.make_raw_inputs(w)
    qn, kn, a, b = oracle.prologue(raw["q"], raw["k"], raw["alpha"], raw["beta"])
    inp = synth.make_inputs(w)
    assert np.allclose(qn, inp["q"], atol=1e-6) and np.allclose(kn, inp["k"], atol=1e-6)
    assert np.allclose(a, inp["alpha"], atol=1e-6) and np.allclose(b, inp["beta"], atol=1e-6)



# ---------------------------------------------------------------- backward

def _bwd_case(kda, B=1, T=5, H=2, dk=3, dv=4, seed=0, with_s0=True, with_dst=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(0.5, 1.0, (B, T, H, dk) if kda else (B, T, H))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    s0 = rng.standard_normal((B, H, dk, dv)) if with_s0 else None
    do = rng.standard_normal((B, T, H, dv))
    dst = rng.standard_normal((B, H, dk, dv)) if with_dst else None
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, s0=s0, do=do, dst=dst)


def _loss(c, scale, **over):
    x = dict(c, **over)
    o, sT = oracle.recurrent(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["s0"], scale=scale)
    val = float(np.sum(c["do"] * o))
    if c["dst"] is not None:
        val += float(np.sum(c["dst"] * sT))
    return val


@pytest.mark.parametrize("kda", [False, True])
def test_backward_matches_central_differences(kda):
    """Every gradient entry against (L(x + h) - L(x - h)) / 2h of the C
    token recurrence (a code path the backward does not share)."""
    c = _bwd_case(kda, seed=3 + kda)
    scale = 0.7
    g = oracle.backward(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["s0"], c["do"], c["dst"],
                        scale=scale)
    h = 1e-6
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("alpha", "dalpha"),
                      ("beta", "dbeta"), ("s0", "ds0")):
        x = c[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd[idx] = (_loss(c, scale, **{name: xp}) - _loss(c, scale, **{name: xm})) / (2 * h)
        err = np.abs(g[key] - fd).max() / max(np.abs(fd).max(), 1e-12)
        assert err < 1e-6, (name, err)


def test_backward_single_token_closed_form():
    """T = 1 from a zero state: o = scale beta (k.q) v and S_1 = beta k v^T,
    so every gradient has a closed form."""
    c = _bwd_case(False, B=2, T=1, H=3, dk=4, dv=5, seed=9, with_s0=False)
    scale = 1.3
    g = oracle.backward(c["q"], c["k"], c["v"], c["alpha"], c["beta"], None, c["do"], c["dst"], scale=scale)
    q, k, v, b, do, dst = c["q"][:, 0], c["k"][:, 0], c["v"][:, 0], c["beta"][:, 0], c["do"][:, 0], c["dst"]
    kq = np.sum(k * q, -1)
    vdo = np.sum(v * do, -1)
    dstk = np.einsum("bhij,bhi->bhj", dst, k)          # dst^T k
    dstv = np.einsum("bhij,bhj->bhi", dst, v)          # dst v
    np.testing.assert_allclose(g["dv"][:, 0], (scale * b * kq)[..., None] * do + b[..., None] * dstk, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dbeta"][:, 0], scale * kq * vdo + np.sum(k * dstv, -1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dq"][:, 0], (scale * b * vdo)[..., None] * k, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dk"][:, 0], (scale * b * vdo)[..., None] * q + b[..., None] * dstv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dalpha"], 0.0, atol=1e-15)   # the gate multiplies the zero state


@pytest.mark.parametrize("kda", [False, True])
def test_backward_pure_decay_closed_form(kda):
    """beta = 0: S_t = (prod of the gates up to t) S_0, so dS_0 and the gate
    gradients are sums of decayed outer products."""
    c = _bwd_case(kda, B=1, T=4, H=2, dk=3, dv=2, seed=5)
    c["beta"] = np.zeros_like(c["beta"])
    scale = 0.9
    g = oracle.backward(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["s0"], c["do"], c["dst"], scale=scale)
    a = c["alpha"] if kda else c["alpha"][..., None] * np.ones(c["q"].shape)   # [B,T,H,dk]
    cum = np.cumprod(a, axis=1)                                                 # prod_{s<=t}
    want = cum[:, -1][..., None] * c["dst"]
    for t in range(4):
        want += scale * cum[:, t][..., None] * c["q"][:, t][..., :, None] * c["do"][:, t][..., None, :]
    np.testing.assert_allclose(g["ds0"], want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dv"], 0.0, atol=1e-15)
    np.testing.assert_allclose(g["dk"], 0.0, atol=1e-15)


def test_backward_is_linear_in_the_output_gradient():
    c = _bwd_case(True, B=1, T=6, H=1, dk=4, dv=3, seed=8)
    d2 = np.random.default_rng(1).standard_normal(c["do"].shape)
    args = (c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["s0"])
    g1 = oracle.backward(*args, c["do"], None)
    g2 = oracle.backward(*args, d2, None)
    g3 = oracle.backward(*args, c["do"] + 2.0 * d2, None)
    for key in g1:
        np.testing.assert_allclose(g3[key], g1[key] + 2.0 * g2[key], rtol=1e-10, atol=1e-10)
