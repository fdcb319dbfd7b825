"""Pins of the C float64 oracle (oracle/mlstm_ref.c).

It is held to the mathematics directly (the literal product form on tiny
inputs, the unstabilised recurrence, the f = i = 1 reduction to cumulative
linear attention) and to the pinned NumPy oracle at every shape the GPU
tests use it for (d_qk != d_v, given initial states, saturated and infinite
gates, many sequences over several threads), to ~1e-12.
"""
import numpy as np
import pytest

from oracle import mlstm_oracle as orc
from oracle.mlstm_ref import mlstm_recurrent_c, mlstm_step_c
from linear_recurrent_sequence_fwd_amd.inputs import make_fwd_inputs, make_state
from tests.test_oracle_pins import brute_force, unstabilised

NAMES = ("q", "k", "v", "i_pre", "f_pre", "o_pre")


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("seed,T,K,V", [(0, 24, 5, 3), (1, 40, 3, 7), (2, 17, 8, 8)])
def test_c_oracle_brute_force_product_form(seed, T, K, V):
    x = make_fwd_inputs(1, 1, T, K, V, "fp32", seed=seed, i_std=1.5)
    h, _ = mlstm_recurrent_c(*[x[n] for n in NAMES])
    ref = brute_force(*[x[n][0, 0].astype(np.float64) for n in NAMES])
    assert _rel(h[0, 0], ref) < 1e-12


def test_c_oracle_unstabilised_recurrence():
    x = make_fwd_inputs(2, 3, 60, 16, 24, "fp32", seed=3, i_std=4.0)
    h, _ = mlstm_recurrent_c(*[x[n] for n in NAMES])
    ref, _, _ = unstabilised(*[x[n].astype(np.float64) for n in NAMES])
    assert _rel(h, ref) < 1e-11


def test_c_oracle_linear_attention():
    """f~ = +inf (f = 1), i~ = 0 (i = 1), o~ = +inf (o = 1): h = tril(Q K^T) V / max(|rowsum|, 1)."""
    x = make_fwd_inputs(1, 2, 50, 8, 6, "fp32", seed=4)
    x["f_pre"][:] = np.inf
    x["i_pre"][:] = 0.0
    x["o_pre"][:] = np.inf
    h, (_, _, m) = mlstm_recurrent_c(*[x[n] for n in NAMES])
    q, k, v = (x[n].astype(np.float64) for n in ("q", "k", "v"))
    A = np.tril(q @ np.swapaxes(k, -1, -2))
    ref = (A @ v) / np.maximum(np.abs(A.sum(-1)), 1.0)[..., None]
    assert _rel(h, ref) < 1e-12
    assert np.all(m == 0.0)


@pytest.mark.parametrize("dtype,K,V,T,state", [("bf16", 128, 96, 130, False), ("fp32", 64, 160, 77, True),
                                               ("bf16", 256, 512, 40, True)])
def test_c_oracle_matches_numpy_oracle(dtype, K, V, T, state):
    x = make_fwd_inputs(2, 3, T, K, V, dtype, seed=5, i_std=3.0)
    kw = {}
    if state:
        st = make_state(2, 3, K, V, seed=6)
        kw = dict(C0=st["C"], n0=st["n"], m0=st["m"])
    h, (C, n, m) = mlstm_recurrent_c(*[x[n] for n in NAMES], threads=4, **kw)
    hr, (Cr, nr, mr) = orc.mlstm_recurrent(*[x[n] for n in NAMES], **kw)
    assert _rel(h, hr) < 1e-12
    assert _rel(C, Cr) < 1e-12 and _rel(n, nr) < 1e-12 and np.max(np.abs(m - mr)) < 1e-12


def test_c_oracle_extreme_gates_match_numpy():
    rng = np.random.default_rng(7)
    x = make_fwd_inputs(1, 2, 200, 16, 16, "fp32", seed=8)
    x["i_pre"] = rng.choice([-100.0, 100.0, 0.0, 2.0, -3.0], size=(1, 2, 200)).astype(np.float32)
    x["f_pre"] = rng.choice([-100.0, 100.0, np.inf, -np.inf, 3.0], size=(1, 2, 200)).astype(np.float32)
    h, _ = mlstm_recurrent_c(*[x[n] for n in NAMES])
    hr, _ = orc.mlstm_recurrent(*[x[n] for n in NAMES])
    assert np.all(np.isfinite(h))
    assert _rel(h, hr) < 1e-12


def test_c_oracle_steps_equal_sequence():
    x = make_fwd_inputs(3, 2, 9, 32, 48, "fp32", seed=9)
    h_seq, (Cs, ns, ms) = mlstm_recurrent_c(*[x[n] for n in NAMES])
    C = np.zeros((3, 2, 48, 32)); n = np.zeros((3, 2, 32)); m = np.zeros((3, 2))
    for t in range(9):
        h = mlstm_step_c(*[x[a][:, :, t] for a in NAMES], C, n, m)
        assert np.array_equal(h, h_seq[:, :, t])
    assert np.array_equal(C, Cs) and np.array_equal(n, ns) and np.array_equal(m, ms)


def test_c_oracle_thread_count_does_not_change_results():
    x = make_fwd_inputs(2, 5, 33, 16, 32, "bf16", seed=10)
    a, _ = mlstm_recurrent_c(*[x[n] for n in NAMES], threads=1)
    b, _ = mlstm_recurrent_c(*[x[n] for n in NAMES], threads=7)
    assert np.array_equal(a, b)
