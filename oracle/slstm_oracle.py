"""Plain float64 CPU oracle for the sLSTM scalar-memory cell forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or runs
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table or
helper with the HIP library; both sides receive the same arrays from the
seeded input generator and nothing else.

What it computes, per batch entry b and head h (xLSTM guide, "The Twin
Cells: sLSTM and mLSTM Mathematical Formulations", sLSTM step-by-step
recurrent equations):

    g~_t = P_t + R h_{t-1}            for the four gates g = i, f, z, o
    m_t  = max(m_{t-1} + f~_t, i~_t)
    c_t  = exp(f~_t + m_{t-1} - m_t) c_{t-1} + exp(i~_t - m_t) tanh(z~_t)
    n_t  = exp(f~_t + m_{t-1} - m_t) n_{t-1} + exp(i~_t - m_t)
    h_t  = sigmoid(o~_t) * c_t / n_t

P_t = W x_t + b is the input projection, computed outside the cell and given
as the input (the cell's own work is the recurrence). R mixes the hidden
state within a head only: head h's gates see h_{t-1} of head h alone (xLSTM
paper, section 2: multiple heads with memory mixing across the cells of a
head but not across heads; the introduction video's block-diagonal layer with
one block per head). One head is the full recurrent matrix of the guide's
listing.

Readings (listed with their reasons in the design notes): the forget gate
enters the exponent as is (exponential activation, as the equations write
it); no epsilon in c/n (the equations' form; after the first step n > 0);
zero initial state with m_0 = 0, as the listing initialises it.

Functions:
  slstm_step       one recurrent step (the body of the recurrence)
  slstm_recurrent  the step applied over a whole sequence
"""
from __future__ import annotations

import numpy as np

from .mlstm_oracle import sigmoid

__all__ = ["slstm_step", "slstm_recurrent"]


def slstm_step(pre_t, R, c, n, m, h):
    """One stabilised sLSTM step (xLSTM guide, sLSTM recurrent equations).

    pre_t [B, 4, H, D]: input-projected preactivations of i, f, z, o;
    R [H, 4, D, D]: per head and gate, row d' maps h_{t-1} of the head to the
    gate preactivation of cell d'; c, n, m, h [B, H, D]: the state.
    Returns the new (c, n, m, h), in the arrays' precision (float64 as
    slstm_recurrent calls it by default).
    """
    dt = np.asarray(c).dtype
    pre_t = np.asarray(pre_t, dtype=dt)
    R = np.asarray(R, dtype=dt)
    rec = np.einsum("hgij,bhj->bghi", R, h)          # R h_{t-1}, per head and gate
    g = pre_t + rec
    it, ft, zt, ot = g[:, 0], g[:, 1], g[:, 2], g[:, 3]
    m_new = np.maximum(m + ft, it)
    fa = np.exp(ft + m - m_new)
    ia = np.exp(it - m_new)
    c_new = fa * c + ia * np.tanh(zt)
    n_new = fa * n + ia
    h_new = sigmoid(ot).astype(dt) * c_new / n_new
    return c_new, n_new, m_new, h_new


def slstm_recurrent(pre, R, state=None, dtype=np.float64):
    """The step over a whole sequence.

    pre [B, T, 4, H, D], R [H, 4, D, D]; state = (c0, n0, m0, h0) [B, H, D] or
    None for the zero state with m_0 = 0. Returns h [B, T, H, D] and the final
    (c, n, m, h).

    dtype=np.float32 evaluates the same equations in float32 arithmetic
    instead of float64. Tests use it to measure the rounding error that any
    float32 evaluation of the recurrence carries: with the exponential forget
    gate the stabiliser m grows without bound over long sequences, and its
    float32 resolution then sets the error of h.
    """
    pre = np.asarray(pre, dtype=dtype)
    R = np.asarray(R, dtype=dtype)
    B, T, _, H, D = pre.shape
    if state is None:
        c, n, m, h = (np.zeros((B, H, D), dtype=dtype) for _ in range(4))
    else:
        c, n, m, h = (np.asarray(s, dtype=dtype).copy() for s in state)
    out = np.zeros((B, T, H, D), dtype=dtype)
    for t in range(T):
        c, n, m, h = slstm_step(pre[:, t], R, c, n, m, h)
        out[:, t] = h
    return out, (c, n, m, h)
