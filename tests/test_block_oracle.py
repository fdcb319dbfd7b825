"""Pins of the float64 block oracle (oracle/mlstm_block.py) to facts outside it:
hand-computed values, library routines, invariants, and a closed form of the
whole block for a one-token sequence. No GPU."""
import numpy as np
import pytest
import scipy.linalg

import oracle.mlstm_block as ob
from linear_recurrent_sequence_fwd_amd.inputs import make_block_inputs


def test_layer_norm_hand_values():
    # x = 1, 2, 3, 4: mean 5/2, mean squared deviation 5/4, so the normalised
    # row is (x - 5/2) / sqrt(5/4) = -3/sqrt(5), -1/sqrt(5), 1/sqrt(5), 3/sqrt(5)
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    got = ob.layer_norm(x, np.ones(4), np.zeros(4), 0.0)
    s5 = np.sqrt(5.0)
    np.testing.assert_allclose(got[0], [-3 / s5, -1 / s5, 1 / s5, 3 / s5], rtol=0, atol=1e-15)
    # scale and shift per channel; eps inside the root: var 5/4 + 3/4 = 2
    w, b = np.array([2.0, -1.0, 0.5, 1.0]), np.array([0.0, 1.0, 0.0, -2.0])
    got = ob.layer_norm(x, w, b, 0.75)
    np.testing.assert_allclose(got[0], np.array([-1.5, -0.5, 0.5, 1.5]) / np.sqrt(2.0) * w + b, atol=1e-15)


def test_swish_values():
    # sigmoid(1) = e / (1 + e)
    s1 = np.e / (1.0 + np.e)
    np.testing.assert_allclose(ob.swish(np.array([1.0, -1.0, 0.0])), [s1, -(1.0 - s1), 0.0], atol=1e-15)
    assert ob.swish(np.array([40.0]))[0] == pytest.approx(40.0, rel=1e-15)
    assert abs(ob.swish(np.array([-40.0]))[0]) < 1e-15
    assert ob.sigmoid(np.array([np.inf]))[0] == 1.0


def test_causal_conv_is_numpy_convolve():
    rng = np.random.default_rng(3)
    T, E, KC = 37, 5, 4
    x = rng.standard_normal((T, E))
    w = rng.standard_normal((E, KC))
    b = rng.standard_normal(E)
    got = ob.causal_conv(x, w, b)
    for e in range(E):
        # taps oldest first: the newest input takes w[e, KC - 1]
        ref = np.convolve(x[:, e], w[e, ::-1])[:T] + b[e]
        np.testing.assert_allclose(got[:, e], ref, atol=1e-13)
    # shorter sequence than the kernel
    np.testing.assert_allclose(ob.causal_conv(x[:2], w, b)[1], w[:, 3] * x[1] + w[:, 2] * x[0] + b, atol=1e-14)


def test_causal_conv_is_causal():
    rng = np.random.default_rng(4)
    T, E, KC = 20, 3, 4
    x = rng.standard_normal((T, E))
    w = rng.standard_normal((E, KC))
    b = np.zeros(E)
    y0 = ob.causal_conv(x, w, b)
    x2 = x.copy()
    x2[9] += 1.0
    d = np.abs(ob.causal_conv(x2, w, b) - y0).max(axis=1)
    assert np.all(d[:9] == 0) and np.all(d[13:] == 0) and np.all(d[9:13] > 0)


def test_block_diag_proj_is_dense_block_diagonal():
    rng = np.random.default_rng(5)
    H, n_out, n_in, T = 3, 4, 6, 7
    W = rng.standard_normal((H, n_out, n_in))
    x = rng.standard_normal((T, H * n_in))
    bias = rng.standard_normal(H * n_out)
    dense = scipy.linalg.block_diag(*W)          # [H n_out, H n_in]
    np.testing.assert_allclose(ob.block_diag_proj(x, W, bias, scale=0.5), 0.5 * x @ dense.T + bias, atol=1e-13)


def test_group_norm_moments_per_head():
    rng = np.random.default_rng(6)
    T, H, dv = 5, 3, 16
    h = rng.standard_normal((T, H, dv)) * 3.0 + 1.0
    g = ob.group_norm(h, np.ones(H * dv), np.zeros(H * dv), 0.0).reshape(T, H, dv)
    np.testing.assert_allclose(g.mean(axis=-1), 0.0, atol=1e-14)
    np.testing.assert_allclose((g ** 2).mean(axis=-1), 1.0, atol=1e-13)
    # one group per head: scaling one head leaves the others and itself unchanged
    h2 = h.copy()
    h2[:, 1] *= 7.0
    np.testing.assert_allclose(ob.group_norm(h2, np.ones(H * dv), np.zeros(H * dv), 0.0).reshape(T, H, dv), g,
                               atol=1e-13)


def _one_token_closed_form(x, p):
    """The block for T = 1 from closed forms: the conv sees only its newest tap,
    and from the zero state the ungated cell gives h~ = v s with
    s = e^i (k . q) / max(e^i |k . q|, 1) per head, which a group norm with
    eps = 0 turns into sign(k . q) times the group norm of v."""
    B, T, D = x.shape
    assert T == 1
    E = p["conv_w"].shape[0]
    H, dqk, dv = p["W_q"].shape[0], p["W_q"].shape[1], p["W_v"].shape[1]
    n_in = E // H
    out = np.empty_like(x, dtype=np.float64)
    for b in range(B):
        xt = x[b, 0].astype(np.float64)
        mu = xt.sum() / D
        xn = (xt - mu) / np.sqrt(((xt - mu) ** 2).sum() / D) * p["ln_w"] + p["ln_b"]
        up = p["W_up"].astype(np.float64) @ xn + p["b_up"]
        xm, z = up[:E], up[E:]
        c = p["conv_w"][:, -1] * xm + p["conv_b"]
        xc = c / (1.0 + np.exp(-c))
        y = np.empty(E)
        for h in range(H):
            seg = slice(h * n_in, (h + 1) * n_in)
            q = p["W_q"][h] @ xc[seg] + p["b_q"][h * dqk:(h + 1) * dqk]
            k = p["W_k"][h] @ xc[seg] / np.sqrt(dqk) + p["b_k"][h * dqk:(h + 1) * dqk]
            v = p["W_v"][h] @ xm[seg] + p["b_v"][h * dv:(h + 1) * dv]
            vn = (v - v.mean()) / v.std()
            cols = slice(h * dv, (h + 1) * dv)
            y[cols] = np.sign(k @ q) * vn * p["gn_w"][cols] + p["gn_b"][cols]
        y = (y + p["skip"] * xc) / (1.0 + np.exp(-z))
        out[b, 0] = xt + p["W_down"].astype(np.float64) @ y + p["b_down"]
    return out


def _one_token_case():
    x, p = make_block_inputs(3, 1, 32, 4, 8, 16, seed=11)
    p = dict(p, eps_gn=0.0, eps_ln=0.0)
    return x, p


def test_block_one_token_closed_form():
    x, p = _one_token_case()
    np.testing.assert_allclose(ob.mlstm_block(x, p), _one_token_closed_form(x, p), rtol=0, atol=1e-11)


@pytest.mark.parametrize("mutation", ["v_from_conv", "gn_all_channels", "gate_first_half"])
def test_planted_mistakes_fail_the_closed_form(monkeypatch, mutation):
    """Mistakes planted in the oracle's composition are caught by the pin above."""
    x, p = _one_token_case()
    if mutation == "v_from_conv":
        real = ob.block_diag_proj
        calls = []

        def proj(xx, W, bias, scale=1.0):
            calls.append(xx)
            if len(calls) % 3 == 0:        # the value projection: feed it the conv output
                xx = calls[-2]
            return real(xx, W, bias, scale)
        monkeypatch.setattr(ob, "block_diag_proj", proj)
    elif mutation == "gn_all_channels":
        real = ob.group_norm

        def gn(h, w, b, eps):
            T, H, dv = h.shape
            return real(h.reshape(T, 1, H * dv), w, b, eps)
        monkeypatch.setattr(ob, "group_norm", gn)
    else:   # the oracle reading the gate from the first half of the up-projection
        orig = ob.mlstm_block

        def block(xx, pp, stages=False):
            E = pp["conv_w"].shape[0]
            q = dict(pp)
            q["b_up"] = np.concatenate([pp["b_up"][E:], pp["b_up"][:E]])
            q["W_up"] = np.concatenate([pp["W_up"][E:], pp["W_up"][:E]])
            return orig(xx, q, stages)
        monkeypatch.setattr(ob, "mlstm_block", block)
    err = np.abs(ob.mlstm_block(x, p) - _one_token_closed_form(x, p)).max()
    assert err > 1e-3


def test_block_batch_entries_independent():
    x, p = make_block_inputs(2, 9, 32, 4, 8, 16, seed=12)
    full = ob.mlstm_block(x, p)
    np.testing.assert_array_equal(full[1:], ob.mlstm_block(x[1:], p))


def test_block_stages_consistent_with_steps():
    """The stages the oracle returns are its own steps' outputs, in the order the page gives."""
    x, p = make_block_inputs(1, 12, 32, 4, 8, 16, seed=13)
    out, st = ob.mlstm_block(x, p, stages=True)
    E = p["conv_w"].shape[0]
    np.testing.assert_allclose(st["xc"][0], ob.swish(ob.causal_conv(st["xup"][0][:, :E], p["conv_w"], p["conv_b"])))
    y = (ob.group_norm(st["h"][0], p["gn_w"], p["gn_b"], p["eps_gn"]) + p["skip"] * st["xc"][0]) \
        * ob.sigmoid(st["xup"][0][:, E:])
    np.testing.assert_allclose(st["y"][0], y)
    np.testing.assert_allclose(out[0], x[0] + y @ p["W_down"].T.astype(np.float64) + p["b_down"], atol=1e-12)
