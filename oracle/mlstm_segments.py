"""Plain float64 CPU oracle for splitting a sequence into segments.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or runs
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library.

The chunkwise form carries a state from chunk to chunk (xLSTM guide,
"Exploit Chunkwise Hardware Kernels for Production Training": dense products
inside a chunk, a recurrent state between chunks). The nareshka notes
("B. mLSTM", the parallelisation formula) write the matrix memory after a
stretch of tokens as a sum of products,

    C_T = (prod_{l=1..T} f_l) C_0 + sum_j (prod_{l=j+1..T} f_l) i_j v_j k_j^T,

so a segment acts on any state it starts from through two things only: the
product of its forget gates and the sum it adds. With G = sum_l log f_l and
the segment's own contribution held in stabilised units (C~_s, n~_s, m_s),
the state after the segment, started from (C~_0, n~_0, m_0), is

    m'  = max(m_0 + G, m_s)
    C~' = exp(m_0 + G - m') C~_0 + exp(m_s - m') C~_s      (n~ alike),

the fold the chunkwise form applies between its chunks. A sequence split
across devices therefore needs from each segment only its summary
(C~_s, n~_s, m_s, G), and an exclusive scan of the summaries with this fold
gives every segment its start state.

Functions:
  segment_summary   the summary of one segment, from its definition
  state_combine     the fold of a start state with a summary
"""
from __future__ import annotations

import numpy as np

from .mlstm_oracle import logsigmoid

__all__ = ["segment_summary", "state_combine"]


def segment_summary(k, v, i_pre, f_pre):
    """(C~_s, n~_s, m_s, G) of a segment, float64.

    The segment's own terms of the sum of products, with no initial state:
    token j enters with log weight sum_{l=j+1..T} log f_l + i~_j; m_s is the
    largest of them (-inf for an empty segment), C~_s = sum_j
    exp(log w_j - m_s) v_j k_j^T and n~_s = sum_j exp(log w_j - m_s) k_j.
    G = sum_{l=1..T} log f_l (0 for an empty segment, -inf after f~ = -inf).

    k [..., T, d_qk]; v [..., T, d_v]; i_pre, f_pre [..., T].
    Returns C~_s [..., d_v, d_qk], n~_s [..., d_qk], m_s [...], G [...].
    """
    k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    i_pre = np.asarray(i_pre, np.float64)
    log_f = logsigmoid(np.asarray(f_pre, np.float64))
    lead = k.shape[:-2]
    T, d_qk, d_v = k.shape[-2], k.shape[-1], v.shape[-1]
    G = np.sum(log_f, axis=-1) if T else np.zeros(lead)
    if T == 0:
        return np.zeros(lead + (d_v, d_qk)), np.zeros(lead + (d_qk,)), np.full(lead, -np.inf), G
    # suffix[..., j] = sum_{l=j+1..T-1} log f_l (0-based), 0 for the last token
    rev = np.cumsum(log_f[..., :0:-1], axis=-1)
    suffix = np.concatenate([rev[..., ::-1], np.zeros(lead + (1,))], axis=-1)
    with np.errstate(invalid="ignore"):
        log_w = suffix + i_pre
    m = np.max(log_w, axis=-1)
    with np.errstate(over="ignore", invalid="ignore"):
        w = np.where(np.isneginf(log_w), 0.0, np.exp(log_w - m[..., None]))
    C = np.matmul(np.swapaxes(w[..., None] * v, -1, -2), k)
    n = np.matmul(w[..., None, :], k)[..., 0, :]
    return C, n, m, G


def state_combine(C0, n0, m0, Cs, ns, ms, G):
    """The state after a segment with summary (Cs, ns, ms, G), started from
    (C0, n0, m0), float64. C0 = None is the zero state with m_0 = 0, the
    recurrence's own start. Returns (C~', n~', m')."""
    Cs = np.asarray(Cs, np.float64); ns = np.asarray(ns, np.float64)
    ms = np.asarray(ms, np.float64); G = np.asarray(G, np.float64)
    lead = ms.shape
    if C0 is None:
        C0 = np.zeros(Cs.shape); n0 = np.zeros(ns.shape); m0 = np.zeros(lead)
    C0 = np.asarray(C0, np.float64); n0 = np.asarray(n0, np.float64)
    m0 = np.asarray(m0, np.float64)
    with np.errstate(invalid="ignore"):
        carried = m0 + G                     # log weight of the start state after the segment
    m = np.maximum(carried, ms)
    m = np.where(np.isneginf(m), 0.0, m)     # nothing at all: an all-zero state
    with np.errstate(over="ignore", invalid="ignore"):
        a = np.where(np.isneginf(carried), 0.0, np.exp(carried - m))
        b = np.where(np.isneginf(ms), 0.0, np.exp(ms - m))
    C = a[..., None, None] * C0 + b[..., None, None] * Cs
    n = a[..., None] * n0 + b[..., None] * ns
    return C, n, m
