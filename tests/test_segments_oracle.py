"""Pins of the segment oracle (oracle/mlstm_segments.py) against the recurrence.

The segment summary and its fold with a start state are checked against the
step recurrence of the xLSTM guide run straight through, which computes the
same state by a different route (one token at a time, from whatever state it
is given). Planted mistakes in copies of the two functions must fail the same
checks.
"""
import numpy as np
import pytest

from linear_recurrent_sequence_fwd_amd.inputs import make_fwd_inputs, make_state
from oracle.mlstm_oracle import logsigmoid, mlstm_recurrent
from oracle.mlstm_segments import segment_summary, state_combine

TOL = 1e-12


def rel(a, b):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def true_units(C, n, m):
    """The unstabilised state exp(m) (C~, n~): equal for any two stabilisers."""
    e = np.exp(np.asarray(m, np.float64))
    return e[..., None, None] * C, e[..., None] * n


def seg(x, t0, t1):
    return {key: (val[:, :, t0:t1] if isinstance(val, np.ndarray) else val) for key, val in x.items()}


@pytest.mark.parametrize("start", ["zero", "given"])
def test_fold_of_summary_equals_the_recurrence(start):
    x = make_fwd_inputs(2, 2, 37, 8, 6, seed=11, i_std=2.0)
    st = make_state(2, 2, 8, 6, seed=12, m_scale=3.0)
    C0, n0, m0 = (None, None, None) if start == "zero" else (st["C"], st["n"], st["m"])
    _, (Cr, nr, mr) = mlstm_recurrent(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"],
                                      C0=C0, n0=n0, m0=m0)
    Cs, ns, ms, G = segment_summary(x["k"], x["v"], x["i_pre"], x["f_pre"])
    C, n, m = state_combine(C0, n0, m0, Cs, ns, ms, G)
    # the stabiliser itself must agree: the denominator's floor exp(-m) depends on it
    assert np.max(np.abs(m - mr)) <= TOL * max(1.0, np.max(np.abs(mr)))
    assert rel(C, Cr) <= TOL and rel(n, nr) <= TOL


def test_scan_of_summaries_reproduces_the_whole_sequence():
    x = make_fwd_inputs(1, 3, 90, 8, 4, seed=13, i_std=3.0, f_mean=1.0, f_std=2.0)
    h_ref, (Cr, nr, mr) = mlstm_recurrent(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    cuts = [0, 17, 18, 50, 90]   # uneven segments, one of a single token
    start = (None, None, None)
    hs = []
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        s = seg(x, t0, t1)
        h, _ = mlstm_recurrent(s["q"], s["k"], s["v"], s["i_pre"], s["f_pre"], s["o_pre"],
                               C0=start[0], n0=start[1], m0=start[2])
        hs.append(h)
        start = state_combine(*start, *segment_summary(s["k"], s["v"], s["i_pre"], s["f_pre"]))
    assert rel(np.concatenate(hs, axis=2), h_ref) <= TOL
    assert rel(start[0], Cr) <= TOL and rel(start[1], nr) <= TOL
    assert np.max(np.abs(start[2] - mr)) <= TOL * max(1.0, np.max(np.abs(mr)))


def test_one_token_closed_form():
    # one token from the empty state: log weight i~, so C~ = v k^T, n~ = k, m = i~, G = log f
    rng = np.random.Generator(np.random.PCG64(5))
    k = rng.standard_normal((1, 1, 1, 5)); v = rng.standard_normal((1, 1, 1, 3))
    i = np.array([[[0.7]]]); f = np.array([[[-1.3]]])
    C, n, m, G = segment_summary(k, v, i, f)
    assert rel(C[0, 0], np.outer(v[0, 0, 0], k[0, 0, 0])) <= TOL
    assert rel(n[0, 0], k[0, 0, 0]) <= TOL
    assert m[0, 0] == 0.7
    assert abs(G[0, 0] - (-np.log1p(np.exp(1.3)))) <= 1e-15   # log sigmoid(-1.3)


def test_empty_segment_is_the_identity():
    st = make_state(1, 2, 4, 3, seed=3)
    C, n, m, G = segment_summary(np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0, 3)),
                                 np.zeros((1, 2, 0)), np.zeros((1, 2, 0)))
    assert np.all(C == 0) and np.all(n == 0) and np.all(m == -np.inf) and np.all(G == 0)
    Co, no, mo = state_combine(st["C"], st["n"], st["m"], C, n, m, G)
    assert np.array_equal(Co, st["C"]) and np.array_equal(no, st["n"]) and np.array_equal(mo, st["m"])


def test_reset_inside_a_segment_drops_the_start():
    x = make_fwd_inputs(1, 1, 12, 4, 4, seed=21)
    x["f_pre"][0, 0, 5] = -np.inf   # forget gate 0 at token 5
    st = make_state(1, 1, 4, 4, seed=22)
    Cs, ns, ms, G = segment_summary(x["k"], x["v"], x["i_pre"], x["f_pre"])
    assert G[0, 0] == -np.inf
    a = state_combine(st["C"], st["n"], st["m"], Cs, ns, ms, G)
    b = state_combine(None, None, None, Cs, ns, ms, G)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)
    _, (Cr, nr, mr) = mlstm_recurrent(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"],
                                      C0=st["C"], n0=st["n"], m0=st["m"])
    assert rel(a[0], Cr) <= TOL and rel(a[1], nr) <= TOL


# ---------------------------------------------------------------- planted mistakes
def _summary_suffix_inclusive(k, v, i_pre, f_pre):
    """Token j's weight with its own forget gate included (l >= j instead of l > j)."""
    C, n, m, G = segment_summary(k, v, i_pre, f_pre)
    log_f = logsigmoid(np.asarray(f_pre, np.float64))
    suffix = np.cumsum(log_f[..., ::-1], axis=-1)[..., ::-1]
    log_w = suffix + np.asarray(i_pre, np.float64)
    mm = np.max(log_w, axis=-1)
    w = np.exp(log_w - mm[..., None])
    C = np.matmul(np.swapaxes(w[..., None] * np.asarray(v, np.float64), -1, -2), np.asarray(k, np.float64))
    n = np.matmul(w[..., None, :], np.asarray(k, np.float64))[..., 0, :]
    return C, n, mm, G


def _combine_without_decay(C0, n0, m0, Cs, ns, ms, G):
    """The start state carried over without the segment's forget gates."""
    return state_combine(C0, n0, m0, Cs, ns, ms, np.zeros_like(np.asarray(G, np.float64)))


@pytest.mark.parametrize("mutant", ["suffix", "decay"])
def test_planted_mistakes_fail(mutant):
    x = make_fwd_inputs(1, 2, 20, 6, 5, seed=31, i_std=2.0)
    st = make_state(1, 2, 6, 5, seed=32)
    _, (Cr, nr, mr) = mlstm_recurrent(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"],
                                      C0=st["C"], n0=st["n"], m0=st["m"])
    summ = _summary_suffix_inclusive if mutant == "suffix" else segment_summary
    comb = _combine_without_decay if mutant == "decay" else state_combine
    C, n, m = comb(st["C"], st["n"], st["m"], *summ(x["k"], x["v"], x["i_pre"], x["f_pre"]))
    Ct, _ = true_units(C, n, m)
    Crt, _ = true_units(Cr, nr, mr)
    assert rel(Ct, Crt) > 1e-3
