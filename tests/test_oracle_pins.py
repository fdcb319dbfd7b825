"""Pins of the float64 oracle to facts fixed by the pages and by the mathematics.

Every check below uses code of its own (never the oracle's functions) for
the expected value: hand-derived worked examples, the literal product form of
the matrix memory, the unstabilised recurrence, closed forms of degenerate
gates, invariances of the cell and arbitrary-precision activations. A planted
mistake in the oracle (a dropped term, a wrong sign or index, a transposed
operand, the floor in the wrong units) fails at least one of them; the
mutation tests at the end plant such mistakes in copies of the oracle's step
and show that the pins reject them.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest

from oracle import mlstm_oracle as orc
from linear_recurrent_sequence_fwd_amd.inputs import make_fwd_inputs, make_state

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _num(x):
    if isinstance(x, str):
        return float(x)          # "inf", "-inf"
    if isinstance(x, list):
        return [_num(y) for y in x]
    return float(x)


def _arr(x):
    return np.array(_num(x), dtype=np.float64)


# ---------------------------------------------------------------- independent references

def brute_force(q, k, v, i_pre, f_pre, o_pre):
    """Literal product form, no logs and no stabiliser (one head).

    C_t = sum_{j<=t} (prod_{l=j+1..t} f_l) i_j v_j k_j^T and the same weights
    on k_j for n_t (nareshka notes, "B. mLSTM", parallelisation formula; xLSTM
    guide, dual formulation); h_t = sigmoid(o_t) C_t q_t / max(|n_t . q_t|, 1).
    """
    T = q.shape[0]
    f = 1.0 / (1.0 + np.exp(-f_pre))
    ig = np.exp(i_pre)
    o = 1.0 / (1.0 + np.exp(-o_pre))
    h = np.zeros((T, v.shape[1]))
    for t in range(T):
        num = np.zeros(v.shape[1])
        den = 0.0
        for j in range(t + 1):
            w = ig[j]
            for l in range(j + 1, t + 1):
                w *= f[l]
            s = float(np.dot(k[j], q[t]))
            num += w * s * v[j]
            den += w * s
        h[t] = o[t] * num / max(abs(den), 1.0)
    return h


def unstabilised(q, k, v, i_pre, f_pre, o_pre):
    """The recurrence in true units with plain exp/sigmoid gates (one head or batched)."""
    lead = q.shape[:-2]
    T = q.shape[-2]
    C = np.zeros(lead + (v.shape[-1], q.shape[-1]))
    n = np.zeros(lead + (q.shape[-1],))
    h = np.zeros(lead + (T, v.shape[-1]))
    for t in range(T):
        f = 1.0 / (1.0 + np.exp(-f_pre[..., t]))
        ig = np.exp(i_pre[..., t])
        C = f[..., None, None] * C + ig[..., None, None] * v[..., t, :, None] * k[..., t, None, :]
        n = f[..., None] * n + ig[..., None] * k[..., t, :]
        num = (C @ q[..., t, :, None])[..., 0]
        den = np.maximum(np.abs((n * q[..., t, :]).sum(-1)), 1.0)
        h[..., t, :] = (1.0 / (1.0 + np.exp(-o_pre[..., t, :]))) * num / den[..., None]
    return h, C, n


def _small(T=24, K=5, V=3, seed=0, i_std=1.0, dtype="fp32"):
    x = make_fwd_inputs(1, 1, T, K, V, dtype=dtype, seed=seed, i_std=i_std)
    return {n: (x[n][0, 0].astype(np.float64) if isinstance(x[n], np.ndarray) else x[n]) for n in x}


def _relerr(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- the pins

def test_hand_derived_cases():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q, k, v = _arr(c["q"]), _arr(c["k"]), _arr(c["v"])
        h, (C, n, m) = orc.mlstm_recurrent(q, k, v, _arr(c["i_pre"]), _arr(c["f_pre"]),
                                           _arr(c["o_pre"]))
        np.testing.assert_allclose(h, _arr(c["h"]), rtol=1e-13, atol=1e-13, err_msg=c["name"])
        # final state in true units: C = exp(m) C~
        np.testing.assert_allclose(np.exp(m) * C, _arr(c["C"]), rtol=1e-13, atol=1e-13,
                                   err_msg=c["name"])
        np.testing.assert_allclose(np.exp(m) * n, _arr(c["n"]), rtol=1e-13, atol=1e-13,
                                   err_msg=c["name"])


@pytest.mark.parametrize("seed,T,K,V", [(0, 24, 5, 3), (1, 40, 4, 7), (2, 64, 16, 8)])
def test_brute_force_product_form(seed, T, K, V):
    x = _small(T, K, V, seed)
    ref = brute_force(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    h, _ = orc.mlstm_recurrent(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    assert _relerr(h, ref) < 1e-12
    rows = [0, 1, T // 2, T - 1]
    hr = orc.mlstm_rows(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"], rows)
    assert _relerr(hr, ref[rows]) < 1e-12


def test_brute_force_high_precision():
    """Tiny case against a 50-digit evaluation of the product form."""
    x = _small(T=6, K=3, V=2, seed=7)
    mpmath.mp.dps = 50
    T = 6
    h_ref = np.zeros((T, 2))
    for t in range(T):
        num = [mpmath.mpf(0)] * 2
        den = mpmath.mpf(0)
        for j in range(t + 1):
            w = mpmath.exp(mpmath.mpf(x["i_pre"][j]))
            for l in range(j + 1, t + 1):
                w *= 1 / (1 + mpmath.exp(-mpmath.mpf(x["f_pre"][l])))
            s = mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b) for a, b in zip(x["k"][j], x["q"][t]))
            for c in range(2):
                num[c] += w * s * mpmath.mpf(x["v"][j][c])
            den += w * s
        dd = max(abs(den), mpmath.mpf(1))
        for c in range(2):
            h_ref[t, c] = float(num[c] / dd / (1 + mpmath.exp(-mpmath.mpf(x["o_pre"][t][c]))))
    h, _ = orc.mlstm_recurrent(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    assert _relerr(h, h_ref) < 1e-13


@pytest.mark.parametrize("i_std", [1.0, 6.0])
def test_unstabilised_recurrence_agrees(i_std):
    x = make_fwd_inputs(2, 3, 96, 16, 12, dtype="fp32", seed=3, i_std=i_std)
    args = [x[n].astype(np.float64) for n in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
    h_ref, C_ref, n_ref = unstabilised(*args)
    h, (C, n, m) = orc.mlstm_recurrent(*args)
    assert _relerr(h, h_ref) < 1e-12
    assert _relerr(np.exp(m)[..., None, None] * C, C_ref) < 1e-12
    assert _relerr(np.exp(m)[..., None] * n, n_ref) < 1e-12


def test_no_forgetting_unit_gates_is_linear_attention():
    """f~ = +inf (f = 1), i~ = 0 (i = 1), o~ = +inf (o = 1): cumulative linear attention."""
    x = _small(T=50, K=8, V=6, seed=4)
    T = 50
    f_pre = np.full(T, np.inf)
    i_pre = np.zeros(T)
    o_pre = np.full((T, 6), np.inf)
    h, (C, n, m) = orc.mlstm_recurrent(x["q"], x["k"], x["v"], i_pre, f_pre, o_pre)
    S = np.tril(x["q"] @ x["k"].T)
    ref = (S @ x["v"]) / np.maximum(np.abs(S.sum(1)), 1.0)[:, None]
    assert _relerr(h, ref) < 1e-12
    assert m == 0.0
    np.testing.assert_allclose(C, x["v"].T @ x["k"], rtol=1e-12)


def test_complete_forgetting_closed_form():
    """f~ = -inf (f = 0): each token sees only itself."""
    x = _small(T=30, K=6, V=4, seed=5)
    f_pre = np.full(30, -np.inf)
    h, _ = orc.mlstm_recurrent(x["q"], x["k"], x["v"], x["i_pre"], f_pre, x["o_pre"])
    ig = np.exp(x["i_pre"])
    s = np.einsum("tk,tk->t", x["k"], x["q"])
    ref = (1 / (1 + np.exp(-x["o_pre"]))) * (ig * s)[:, None] * x["v"] / \
        np.maximum(np.abs(ig * s), 1.0)[:, None]
    assert np.all(np.isfinite(h))
    assert _relerr(h, ref) < 1e-13


def test_single_token():
    x = _small(T=1, K=7, V=5, seed=6)
    h, _ = orc.mlstm_recurrent(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    ig = math.exp(x["i_pre"][0])
    s = float(x["k"][0] @ x["q"][0])
    ref = (1 / (1 + np.exp(-x["o_pre"][0]))) * ig * s * x["v"][0] / max(abs(ig * s), 1.0)
    assert _relerr(h[0], ref) < 1e-14


def test_linear_in_values():
    x = _small(T=40, K=6, V=5, seed=8)
    y = _small(T=40, K=6, V=5, seed=9)
    args = lambda vv: (x["q"], x["k"], vv, x["i_pre"], x["f_pre"], x["o_pre"])  # noqa: E731
    h1, _ = orc.mlstm_recurrent(*args(x["v"]))
    h2, _ = orc.mlstm_recurrent(*args(y["v"]))
    h12, _ = orc.mlstm_recurrent(*args(x["v"] + y["v"]))
    h3, _ = orc.mlstm_recurrent(*args(-2.5 * x["v"]))
    assert _relerr(h12, h1 + h2) < 1e-12
    assert _relerr(h3, -2.5 * h1) < 1e-13


def test_batch_and_head_independence():
    x = make_fwd_inputs(3, 4, 33, 8, 6, dtype="fp32", seed=10)
    names = ("q", "k", "v", "i_pre", "f_pre", "o_pre")
    args = [x[n].astype(np.float64) for n in names]
    h, _ = orc.mlstm_recurrent(*args)
    perm_b, perm_h = np.array([2, 0, 1]), np.array([3, 1, 0, 2])
    pargs = [a[perm_b][:, perm_h] for a in args]
    hp, _ = orc.mlstm_recurrent(*pargs)
    np.testing.assert_array_equal(hp, h[perm_b][:, perm_h])
    # one head alone gives the same output as inside the batch
    h1, _ = orc.mlstm_recurrent(*[a[1, 2] for a in args])
    np.testing.assert_allclose(h1, h[1, 2], rtol=1e-14, atol=0)


def test_split_and_resume():
    """Running T1 tokens, handing the state over and running T2 more equals one run."""
    x = make_fwd_inputs(2, 2, 70, 8, 6, dtype="fp32", seed=11, i_std=3.0)
    args = [x[n].astype(np.float64) for n in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
    h, (C, n, m) = orc.mlstm_recurrent(*args)
    for T1 in (1, 29, 69):
        ha, (Ca, na, ma) = orc.mlstm_recurrent(*[a[:, :, :T1] for a in args])
        hb, (Cb, nb, mb) = orc.mlstm_recurrent(*[a[:, :, T1:] for a in args], C0=Ca, n0=na, m0=ma)
        np.testing.assert_allclose(np.concatenate([ha, hb], axis=2), h, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(Cb, C, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(mb, m, rtol=0, atol=0)


def _combine(first, second, g):
    """Compose a state with the summary a stretch reaches from zero state (true units:
    C = exp(g) C_first + C_second), written in stabilised units."""
    Ca, na, ma = first
    Cb, nb, mb = second
    mm = np.maximum(g + ma, mb)
    sa, sb = np.exp(g + ma - mm), np.exp(mb - mm)
    return sa[..., None, None] * Ca + sb[..., None, None] * Cb, sa[..., None] * na + sb[..., None] * nb, mm


def test_chunk_bracketing_is_associative():
    """Summaries of four stretches composed in two bracketings equal the sequential state."""
    x = make_fwd_inputs(1, 2, 64, 6, 5, dtype="fp32", seed=12, i_std=2.0)
    args = [x[n].astype(np.float64) for n in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
    _, (C, n, m) = orc.mlstm_recurrent(*args)
    cuts = [0, 10, 27, 40, 64]
    summ, gs = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        _, s = orc.mlstm_recurrent(*[t[:, :, a:b] for t in args])
        summ.append(s)
        f = 1 / (1 + np.exp(-args[4][:, :, a:b]))
        gs.append(np.log(np.prod(f, axis=-1)))
    left = summ[0]
    for s, g in zip(summ[1:], gs[1:]):
        left = _combine(left, s, g)
    ab = _combine(summ[0], summ[1], gs[1])
    cd = _combine(summ[2], summ[3], gs[3])
    tree = _combine(ab, cd, gs[2] + gs[3])
    for Cx, nx, mx in (left, tree):
        np.testing.assert_allclose(np.exp(mx)[..., None, None] * Cx,
                                   np.exp(m)[..., None, None] * C, rtol=1e-12)
        np.testing.assert_allclose(np.exp(mx)[..., None] * nx, np.exp(m)[..., None] * n, rtol=1e-12)


def test_stabiliser_invariance():
    x = _small(T=45, K=6, V=4, seed=13, i_std=4.0)
    args = (x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    h0, _ = orc.mlstm_recurrent(*args, C0=np.zeros((4, 6)), n0=np.zeros(6), m0=0.0)
    for m0 in (-np.inf, 5.0, -30.0):
        h, _ = orc.mlstm_recurrent(*args, C0=np.zeros((4, 6)), n0=np.zeros(6), m0=m0)
        assert _relerr(h, h0) < 1e-13
    # the same true state written with a shifted stabiliser gives the same outputs
    st = make_state(1, 1, 6, 4, seed=1)
    C0, n0, m0 = st["C"][0, 0].astype(np.float64), st["n"][0, 0].astype(np.float64), 0.7
    ha, _ = orc.mlstm_recurrent(*args, C0=C0, n0=n0, m0=m0)
    for d in (-3.0, 11.0):
        hb, _ = orc.mlstm_recurrent(*args, C0=C0 * np.exp(-d), n0=n0 * np.exp(-d), m0=m0 + d)
        assert _relerr(hb, ha) < 1e-13
    # and the dual form with that initial state agrees
    hr = orc.mlstm_rows(*args, rows=[0, 20, 44], C0=C0, n0=n0, m0=m0)
    assert _relerr(hr, ha[[0, 20, 44]]) < 1e-12


def test_final_state_closed_form_matches_recurrence():
    x = make_fwd_inputs(2, 2, 57, 6, 5, dtype="fp32", seed=16, i_std=3.0)
    args = [x[n].astype(np.float64) for n in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
    args[4][0, 1, 20] = -np.inf          # a zero forget gate in one head
    _, (C, n, m) = orc.mlstm_recurrent(*args)
    C2, n2, m2 = orc.mlstm_final_state(args[1], args[2], args[3], args[4])
    np.testing.assert_allclose(m2, m, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(C2, C, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(n2, n, rtol=1e-12, atol=1e-13)
    st = make_state(2, 2, 6, 5, seed=3)
    C0, n0, m0 = (st[n_].astype(np.float64) for n_ in ("C", "n", "m"))
    _, (C, n, m) = orc.mlstm_recurrent(*args, C0=C0, n0=n0, m0=m0)
    C2, n2, m2 = orc.mlstm_final_state(args[1], args[2], args[3], args[4], C0=C0, n0=n0, m0=m0)
    np.testing.assert_allclose(m2, m, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(C2, C, rtol=1e-12, atol=1e-13)
    # and against the literal product form of C_T in true units (one head)
    f = 1 / (1 + np.exp(-args[4][1, 0]))
    ig = np.exp(args[3][1, 0])
    T = f.shape[0]
    Ct = sum(np.prod(f[j + 1:]) * ig[j] * np.outer(args[2][1, 0, j], args[1][1, 0, j]) for j in range(T))
    Ct = Ct + np.prod(f) * np.exp(m0[1, 0]) * C0[1, 0]
    np.testing.assert_allclose(np.exp(m2[1, 0]) * C2[1, 0], Ct, rtol=1e-12)


def test_extreme_preactivations_finite_and_exact():
    rng = np.random.default_rng(14)
    T, K, V = 48, 6, 5
    x = _small(T, K, V, seed=14)
    i_pre = rng.choice([-100.0, 100.0, 0.0, 2.0], size=T)
    f_pre = rng.choice([-100.0, 100.0, np.inf, -np.inf, 3.0], size=T)
    h, (C, n, m) = orc.mlstm_recurrent(x["q"], x["k"], x["v"], i_pre, f_pre, x["o_pre"])
    assert np.all(np.isfinite(h)) and np.all(np.isfinite(C)) and np.isfinite(m)
    ref = brute_force(x["q"], x["k"], x["v"], i_pre, f_pre, x["o_pre"])
    assert _relerr(h, ref) < 1e-11


def test_activations_against_mpmath():
    mpmath.mp.dps = 40
    grid = [-1000.0, -80.0, -20.0, -3.0, -1e-8, 0.0, 1e-8, 0.5, 3.0, 20.0, 80.0, 1000.0]
    for xv in grid:
        ls = float(-mpmath.log1p(mpmath.exp(-mpmath.mpf(xv))))
        sg = float(1 / (1 + mpmath.exp(-mpmath.mpf(xv))))
        assert abs(orc.logsigmoid(xv) - ls) <= 1e-15 * max(1.0, abs(ls))
        assert abs(orc.sigmoid(xv) - sg) <= 1e-15 * max(1e-300, abs(sg)) + 1e-300
    assert orc.logsigmoid(np.inf) == 0.0 and orc.logsigmoid(-np.inf) == -np.inf
    assert orc.sigmoid(np.inf) == 1.0 and orc.sigmoid(-np.inf) == 0.0


# ---------------------------------------------------------------- planted mistakes

def _mutant_recurrent(q, k, v, i_pre, f_pre, o_pre, mutation):
    T, K = q.shape
    V = v.shape[1]
    C = np.zeros((V, K)); n = np.zeros(K); m = 0.0
    h = np.zeros((T, V))
    for t in range(T):
        lf = float(orc.logsigmoid(f_pre[t]))
        if mutation == "exp_forget":
            lf = f_pre[t]
        if mutation == "index_shift" and t > 0:
            lf = float(orc.logsigmoid(f_pre[t - 1]))
        m_new = max(lf + m, i_pre[t])
        fs, is_ = math.exp(lf + m - m_new), math.exp(i_pre[t] - m_new)
        if mutation == "sign":
            is_ = -is_
        C = fs * C + is_ * np.outer(v[t], k[t])
        n = fs * n + is_ * k[t]
        m = m_new
        num = (C.T if mutation == "transpose" else C) @ q[t]
        den = abs(n @ q[t])
        if mutation == "floor_stabilised":
            den = max(den, 1.0)
        elif mutation == "no_normaliser":
            den = 1.0
        else:
            den = max(den, math.exp(-m))
        h[t] = orc.sigmoid(o_pre[t]) * num / den
    return h


@pytest.mark.parametrize("mutation", ["exp_forget", "index_shift", "sign", "transpose",
                                      "floor_stabilised", "no_normaliser"])
def test_pins_reject_planted_mistakes(mutation):
    x = _small(T=32, K=4, V=4, seed=15, i_std=2.0)   # square, so a transposed C still runs
    args = (x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    ref = brute_force(*args)
    good = _mutant_recurrent(*args, mutation="none")
    assert _relerr(good, ref) < 1e-12
    bad = _mutant_recurrent(*args, mutation=mutation)
    assert _relerr(bad, ref) > 1e-3, mutation
