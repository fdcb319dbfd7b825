"""Plain float64 CPU oracle for the mLSTM matrix-memory cell forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or runs
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table or
helper with the HIP library; both sides receive the same arrays from the
seeded input generator and nothing else.

What it computes (per batch entry b and head h, independently):

* gates (xLSTM guide, "The Innovation: Exponential Gating and Dynamic
  Normalization"): input gate i = exp(i~); the forget gate is the sigmoid of
  its preactivation, carried in log space as log f = logsigmoid(f~); output
  gate o = sigmoid(o~), applied elementwise over d_v;
* matrix memory and normaliser (xLSTM guide, "mLSTM: Matrix Key-Value Memory
  and Covariance Updates", recurrent formulation):
      C_t = f_t C_{t-1} + i_t v_t k_t^T        (d_v x d_qk)
      n_t = f_t n_{t-1} + i_t k_t
      h_t = o_t * (C_t q_t) / max(|n_t^T q_t|, 1)
* the running-max stabiliser m_t = max(log f_t + m_{t-1}, i~_t) of the same
  guide ("The Stabilizer State"), under which C~ = exp(-m) C and
  n~ = exp(-m) n are stored. The floor of 1 in the denominator belongs to the
  true (unstabilised) quantities, so in stabilised units it reads
  max(|n~^T q|, exp(-m)).

Readings taken where the pages are silent or disagree (each is listed with
its reason in the design notes): logsigmoid forget gate; exp input gate with
no normalisation over time; the floor of 1 in true units; C oriented d_v x
d_qk with h = C q; no 1/sqrt(d) scaling inside the cell (the inputs carry
it); zero initial state with m_0 = 0; no epsilon in the denominator.

Functions:
  logsigmoid, sigmoid      stable scalar activations
  mlstm_step               one recurrent step (the body of the recurrence)
  mlstm_recurrent          the step applied over a whole sequence
  mlstm_rows               h at chosen time indices from the parallel (dual)
                           closed form of the same cell, for sampled checks
                           at sizes where the full recurrence is too slow
  mlstm_final_state        the state after a whole sequence from the
                           sum-of-products form of C_T (one matrix product)
"""
from __future__ import annotations

import numpy as np

__all__ = ["logsigmoid", "sigmoid", "mlstm_step", "mlstm_recurrent", "mlstm_rows",
           "mlstm_final_state"]


def logsigmoid(x):
    """log(1 / (1 + exp(-x))) = min(x, 0) - log1p(exp(-|x|)), exact at +-inf."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + exp(-x)), evaluated without overflow for either sign."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def mlstm_step(q, k, v, i_pre, f_pre, o_pre, C, n, m):
    """One step of the stabilised mLSTM recurrence (xLSTM guide, recurrent formulation).

    Shapes (any leading dims ``...`` shared by all arguments):
      q, k [..., d_qk]; v, o_pre [..., d_v]; i_pre, f_pre, m [...];
      C [..., d_v, d_qk] (stabilised C~); n [..., d_qk] (stabilised n~).
    Returns (h [..., d_v], C', n', m').
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); o_pre = np.asarray(o_pre, np.float64)
    i_pre = np.asarray(i_pre, np.float64); m = np.asarray(m, np.float64)
    log_f = logsigmoid(f_pre)
    with np.errstate(over="ignore", invalid="ignore"):
        # stabiliser: m_t = max(log f_t + m_{t-1}, i~_t)
        m_new = np.maximum(log_f + m, i_pre)
        # stabilised gates: f' = exp(log f + m_{t-1} - m_t), i' = exp(i~ - m_t)
        f_s = np.exp(log_f + m - m_new)
        i_s = np.exp(i_pre - m_new)
        # covariance update of the matrix memory, C = v k^T orientation
        C_new = f_s[..., None, None] * C + i_s[..., None, None] * (v[..., :, None] * k[..., None, :])
        n_new = f_s[..., None] * n + i_s[..., None] * k
        num = np.einsum("...vk,...k->...v", C_new, q)
        # floor of 1 in true units is exp(-m) in stabilised units
        den = np.maximum(np.abs(np.einsum("...k,...k->...", n_new, q)), np.exp(-m_new))
        h = sigmoid(o_pre) * num / den[..., None]
    return h, C_new, n_new, m_new


def mlstm_recurrent(q, k, v, i_pre, f_pre, o_pre, C0=None, n0=None, m0=None):
    """The stabilised recurrence over t = 1..T.

    q, k [..., T, d_qk]; v, o_pre [..., T, d_v]; i_pre, f_pre [..., T].
    Optional initial state C0 [..., d_v, d_qk], n0 [..., d_qk], m0 [...]
    (stabilised units); absent, the state starts at zero with m_0 = 0.
    Returns h [..., T, d_v] and the final state (C~, n~, m), all float64.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); o_pre = np.asarray(o_pre, np.float64)
    i_pre = np.asarray(i_pre, np.float64); f_pre = np.asarray(f_pre, np.float64)
    lead = q.shape[:-2]
    T, d_qk = q.shape[-2], q.shape[-1]
    d_v = v.shape[-1]
    C = np.zeros(lead + (d_v, d_qk)) if C0 is None else np.array(C0, np.float64)
    n = np.zeros(lead + (d_qk,)) if n0 is None else np.array(n0, np.float64)
    m = np.zeros(lead) if m0 is None else np.array(m0, np.float64)
    h = np.empty(lead + (T, d_v))
    for t in range(T):
        h[..., t, :], C, n, m = mlstm_step(q[..., t, :], k[..., t, :], v[..., t, :],
                                           i_pre[..., t], f_pre[..., t], o_pre[..., t, :],
                                           C, n, m)
    return h, (C, n, m)


def mlstm_rows(q, k, v, i_pre, f_pre, o_pre, rows, C0=None, n0=None, m0=None):
    """h at the time indices ``rows`` from the parallel (dual) form, float64.

    xLSTM guide, "The Dual Formulation": with the decay matrix
        log D_tj = sum_{l=j+1..t} log f_l + i~_j      (j <= t)
    the output is h~_t = sum_j D_tj (q_t . k_j) v_j divided by the same sum
    with v_j replaced by 1, floored at 1 in absolute value. An initial state
    (C0, n0, m0) enters as one more term of log weight sum_{l=1..t} log f_l + m0.
    The log weights of each row are shifted by their maximum before the exp.
    The sum over l is a suffix sum per row, so no difference of two large
    prefix sums is ever taken.

    q, k [..., T, d_qk]; v, o_pre [..., T, d_v]; i_pre, f_pre [..., T].
    Returns h [..., len(rows), d_v].
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); o_pre = np.asarray(o_pre, np.float64)
    i_pre = np.asarray(i_pre, np.float64)
    log_f = logsigmoid(f_pre)
    lead = q.shape[:-2]
    d_v = v.shape[-1]
    out = np.empty(lead + (len(rows), d_v))
    for r, t in enumerate(rows):
        # suffix[..., j] = sum_{l=j+1..t} log f_l for j = 0..t; suffix[..., t] = 0
        rev = np.cumsum(log_f[..., t:0:-1], axis=-1)          # sums over l = t, t..t-1, ...
        suffix = np.concatenate([rev[..., ::-1], np.zeros(lead + (1,))], axis=-1)
        with np.errstate(invalid="ignore"):
            log_w = suffix + i_pre[..., :t + 1]
        s = np.einsum("...jk,...k->...j", k[..., :t + 1, :], q[..., t, :])
        if C0 is not None:
            log_w0 = np.sum(log_f[..., :t + 1], axis=-1) + np.asarray(m0, np.float64)
            mrow = np.maximum(np.max(log_w, axis=-1), log_w0)
        else:
            mrow = np.max(log_w, axis=-1)
        with np.errstate(over="ignore", invalid="ignore"):
            w = np.exp(log_w - mrow[..., None])
            num = np.einsum("...j,...jv->...v", w * s, v[..., :t + 1, :])
            den_raw = np.sum(w * s, axis=-1)
            if C0 is not None:
                w0 = np.exp(log_w0 - mrow)
                num = num + w0[..., None] * np.einsum("...vk,...k->...v",
                                                      np.asarray(C0, np.float64), q[..., t, :])
                den_raw = den_raw + w0 * np.einsum("...k,...k->...", np.asarray(n0, np.float64),
                                                   q[..., t, :])
            den = np.maximum(np.abs(den_raw), np.exp(-mrow))
            out[..., r, :] = sigmoid(o_pre[..., t, :]) * num / den[..., None]
    return out



def mlstm_final_state(k, v, i_pre, f_pre, C0=None, n0=None, m0=None):
    """State (C~_T, n~_T, m_T) after the whole sequence, float64.

    Sum-of-products form of the matrix memory (nareshka notes, "B. mLSTM",
    parallelisation formula; xLSTM guide, dual formulation):
        C_T = sum_j (prod_{l=j+1..T} f_l) i_j v_j k_j^T + (prod_{l=1..T} f_l) C_0
    and the same weights on k_j for n_T. The log weight of token j is
    sum_{l=j+1..T} log f_l + i~_j and that of the initial state
    sum_{l=1..T} log f_l + m_0 (m_0 = 0 without an initial state, as in the
    recurrence); m_T is the largest of them, which is the recurrence's
    running max, and C~ = exp(-m_T) C.

    k [..., T, d_qk]; v [..., T, d_v]; i_pre, f_pre [..., T].
    """
    k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    i_pre = np.asarray(i_pre, np.float64)
    log_f = logsigmoid(f_pre)
    lead = k.shape[:-2]
    rev = np.cumsum(log_f[..., :0:-1], axis=-1)      # sums over l = T-1, T-1..T-2, ...
    suffix = np.concatenate([rev[..., ::-1], np.zeros(lead + (1,))], axis=-1)
    with np.errstate(invalid="ignore"):
        log_w = suffix + i_pre
    m_init = np.zeros(lead) if m0 is None else np.asarray(m0, np.float64)
    log_w0 = np.sum(log_f, axis=-1) + m_init
    m = np.maximum(np.max(log_w, axis=-1), log_w0)
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.exp(log_w - m[..., None])
        w0 = np.exp(log_w0 - m)
    C = np.matmul(np.swapaxes(w[..., None] * v, -1, -2), k)
    n = np.matmul(w[..., None, :], k)[..., 0, :]
    if C0 is not None:
        C = C + w0[..., None, None] * np.asarray(C0, np.float64)
        n = n + w0[..., None] * np.asarray(n0, np.float64)
    return C, n, m
