"""Plain float64 CPU oracle for the mLSTM layer around the cell: the residual
block with pre-up-projection.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or runs
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table or
helper with the HIP library; both sides receive the same arrays from the
seeded input generator and nothing else.

What the block computes, in the order of the hu-po page "Introduction to
xLSTM architecture", section "Residual Block with Pre-Up Projection"
(primarily for the mLSTM), with the cell's projections and gates from the
xLSTM guide (aifetchly), "mLSTM: Matrix Key-Value Memory and Covariance
Updates", recurrent formulation. Per batch entry, x is [T, D]:

  1. pre-layer norm:          xn = LayerNorm(x)                    (per token over D)
  2. up-projection by two:    [xm | z] = xn W_up^T + b_up           (E = 2 D columns each)
  3. causal conv + Swish:     xc = swish(conv_t(xm) + b_conv)       (per channel, KC taps,
                              taps ordered oldest first, zero before t = 0)
  4. queries and keys:        q = BlockDiag(W_q) xc + b_q           (one block per head)
                              k = BlockDiag(W_k) xc / sqrt(d_qk) + b_k
     values skip the conv:    v = BlockDiag(W_v) xm + b_v
     gates from the cell input:  i~ = xc w_i^T + b_i,  f~ = xc w_f^T + b_f  (one per head)
  5. the mLSTM cell with no output gate of its own (sigma(o~) = 1): h~ [T, H, d_v]
  6. group norm per head:     g = GroupNorm(h~)                     (over d_v, per token)
  7. learnable skip:          s = g + skip * xc
  8. external output gate:    y = s * sigmoid(z)
  9. down-projection, residual: out = x + y W_down^T + b_down

Readings (the pages name the parts, not every operand):
  * the external output gate is sigmoid(z) with z the second half of the
    up-projection: the page places it outside the cell, depending only on
    the input, and the guide's output gate is a sigmoid of a linear function
    of the input; the cell therefore runs ungated;
  * "block-diagonal" means one block per head: head h's q, k and v read the
    head's own E/H channels;
  * the key scaling 1/sqrt(d_qk) sits in the key projection, as in the
    guide's recurrent formulation;
  * the value projection is block-diagonal like q and k and reads the
    up-projection before the conv ("values skip the convolution part");
  * the learnable skip adds skip * xc (the cell's input, the conv output);
  * the cell's value width fills the inner width: H d_v = E;
  * layer norm and group norm use the biased variance with eps inside the
    square root, and learnable per-channel scale and shift.

Functions:
  layer_norm, causal_conv, swish, block_diag_proj, group_norm, sigmoid
  cell_ungated      the cell of mlstm_oracle with the output gate set to one
  mlstm_block       the whole block; ``stages=True`` also returns the
                    intermediates xn, xup, xc, q, k, v, i_pre, f_pre, h, y
"""
from __future__ import annotations

import numpy as np

from .mlstm_oracle import mlstm_recurrent

__all__ = ["layer_norm", "causal_conv", "swish", "sigmoid", "block_diag_proj", "group_norm",
           "cell_ungated", "mlstm_block"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def sigmoid(x):
    """1 / (1 + exp(-x)) without overflow for either sign."""
    x = _f64(x)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def swish(x):
    """Swish (SiLU): x * sigmoid(x)."""
    x = _f64(x)
    return x * sigmoid(x)


def layer_norm(x, w, b, eps):
    """Normalise each row over its last axis: (x - mean) / sqrt(var + eps) * w + b,
    var the mean squared deviation (hu-po page: the pre-layer norm of the block)."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f64(w) + _f64(b)


def causal_conv(x, w, b):
    """Channel-wise causal convolution over time (hu-po page: "dimension-wise
    causally convolved"): x [T, E], w [E, KC], b [E];
    y[t, e] = b[e] + sum_j w[e, j] x[t - (KC - 1) + j, e], terms before t = 0 absent."""
    x, w = _f64(x), _f64(w)
    T, E = x.shape
    KC = w.shape[1]
    y = np.tile(_f64(b), (T, 1))
    for j in range(KC):
        lag = KC - 1 - j
        if lag >= T:
            continue
        y[lag:] += w[:, j] * x[:T - lag]
    return y


def block_diag_proj(x, W, bias, scale=1.0):
    """Block-diagonal projection, one block per head: x [T, H * n_in], W [H, n_out, n_in];
    head h's outputs are scale * W[h] x[:, h n_in:(h + 1) n_in] + bias[h n_out:(h + 1) n_out]."""
    x, W = _f64(x), _f64(W)
    H, n_out, n_in = W.shape
    T = x.shape[0]
    out = np.empty((T, H * n_out))
    for h in range(H):
        out[:, h * n_out:(h + 1) * n_out] = scale * (x[:, h * n_in:(h + 1) * n_in] @ W[h].T)
    return out + _f64(bias)


def group_norm(h, w, b, eps):
    """Group norm with one group per head (hu-po page: outputs normalised by
    group normalisation after sequence mixing): h [T, H, d_v], w, b [H * d_v];
    each (token, head) row normalised over d_v, then scaled and shifted."""
    h = _f64(h)
    T, H, dv = h.shape
    mu = h.mean(axis=-1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=-1, keepdims=True)
    return ((h - mu) / np.sqrt(var + eps)).reshape(T, H * dv) * _f64(w) + _f64(b)


def cell_ungated(q, k, v, i_pre, f_pre):
    """The mLSTM cell of one batch entry with sigma(o~) = 1: q, k [T, H, d_qk],
    v [T, H, d_v], gates [T, H]; returns h~ [T, H, d_v] from the float64 step
    recurrence (mlstm_oracle.mlstm_recurrent) fed with an output-gate
    preactivation of +inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, dqk = q.shape
    dv = v.shape[2]
    tr = lambda a: np.ascontiguousarray(np.moveaxis(a, 1, 0))[None]   # [T, H, d] -> [1, H, T, d]
    o_pre = np.full((1, H, T, dv), np.inf)
    h, _ = mlstm_recurrent(tr(q), tr(k), tr(v), tr(_f64(i_pre)[..., None])[..., 0],
                           tr(_f64(f_pre)[..., None])[..., 0], o_pre)
    return np.moveaxis(h[0], 0, 1)


def mlstm_block(x, p, stages=False):
    """The pre-up-projection block on x [B, T, D] with parameters ``p`` (a dict:
    ln_w, ln_b [D]; W_up [2E, D], b_up [2E]; conv_w [E, KC], conv_b [E];
    W_q, W_k [H, d_qk, E/H], b_q, b_k [H d_qk]; W_v [H, d_v, E/H], b_v [E];
    w_i, w_f [H, E], b_i, b_f [H]; gn_w, gn_b, skip [E]; W_down [D, E],
    b_down [D]; eps_ln, eps_gn). Returns out [B, T, D] (and the stages)."""
    x = _f64(x)
    B, T, D = x.shape
    E = p["conv_w"].shape[0]
    H, dqk = p["W_q"].shape[0], p["W_q"].shape[1]
    dv = p["W_v"].shape[1]
    assert H * dv == E, "the value width fills the inner width"
    outs, keep = [], {n: [] for n in ("xn", "xup", "xc", "q", "k", "v", "i_pre", "f_pre", "h", "y")}
    for bi in range(B):
        xn = layer_norm(x[bi], p["ln_w"], p["ln_b"], p["eps_ln"])
        xup = xn @ _f64(p["W_up"]).T + _f64(p["b_up"])
        xm, z = xup[:, :E], xup[:, E:]
        xc = swish(causal_conv(xm, p["conv_w"], p["conv_b"]))
        q = block_diag_proj(xc, p["W_q"], p["b_q"])
        k = block_diag_proj(xc, p["W_k"], p["b_k"], scale=1.0 / np.sqrt(dqk))
        v = block_diag_proj(xm, p["W_v"], p["b_v"])
        i_pre = xc @ _f64(p["w_i"]).T + _f64(p["b_i"])
        f_pre = xc @ _f64(p["w_f"]).T + _f64(p["b_f"])
        h = cell_ungated(q.reshape(T, H, dqk), k.reshape(T, H, dqk), v.reshape(T, H, dv), i_pre, f_pre)
        y = (group_norm(h, p["gn_w"], p["gn_b"], p["eps_gn"]) + _f64(p["skip"]) * xc) * sigmoid(z)
        outs.append(x[bi] + y @ _f64(p["W_down"]).T + _f64(p["b_down"]))
        if stages:
            for n, val in (("xn", xn), ("xup", xup), ("xc", xc), ("q", q), ("k", k), ("v", v),
                           ("i_pre", i_pre), ("f_pre", f_pre), ("h", h), ("y", y)):
                keep[n].append(val)
    out = np.stack(outs)
    if stages:
        return out, {n: np.stack(vals) for n, vals in keep.items()}
    return out
