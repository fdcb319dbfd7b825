"""Plain float64 CPU oracle of the mLSTM cell's gradients (reverse mode).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or runs
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, table or
helper with the HIP library.

The pages present the parallel and chunkwise forms of the mLSTM as what
makes it trainable (xLSTM guide, aifetchly blog, "The Dual Formulation: How
mLSTM Enables Parallel GPU Training", training mode; "Exploit Chunkwise
Hardware Kernels for Production Training"). Training needs the gradient of a
loss through the cell. This module gives it for a loss L that depends on the
outputs h_t: given dh_t = dL/dh_t it returns dL/d of every input of the
forward (q, k, v, the three gate preactivations, and the initial state).

Forward, per (batch, head), in true units (the same cell as mlstm_oracle;
xLSTM guide, "mLSTM: Matrix Key-Value Memory and Covariance Updates"):
    C_t = f_t C_{t-1} + i_t v_t k_t^T,  n_t = f_t n_{t-1} + i_t k_t
    h_t = o_t * (C_t q_t) / max(|n_t . q_t|, 1)
with f_t = sigmoid(f~_t), i_t = exp(i~_t), o_t = sigmoid(o~_t).

Reverse mode of that recurrence (the chain rule, step by step). With
g_t = dh_t o_t / den_t and dz_t = -sign(z_t) [|z_t| > 1] (g_t . num_t) / den_t
(z_t = n_t . q_t, num_t = C_t q_t, den_t = max(|z_t|, 1)), the adjoints of the
state obey
    E_t = g_t q_t^T + f_{t+1} E_{t+1},    e_t = dz_t q_t + f_{t+1} e_{t+1}
and
    dq_t = C_t^T g_t + dz_t n_t
    dv_t = i_t E_t k_t,   dk_t = i_t (E_t^T v_t + e_t),   di~_t = i_t dL/di_t = k_t . dk_t
    dlog f_t = f_t (<E_t, C_{t-1}> + e_t . n_{t-1}),   df~_t = dlog f_t * sigmoid(-f~_t)
    do~_t = dh_t * (num_t / den_t) * o_t (1 - o_t)
    dC_0 = f_1 E_1,   dn_0 = f_1 e_1.

Stabilised evaluation. True units overflow (i_t = exp(i~_t)), so the forward
runs in the stabilised units of "The Stabilizer State" (C~ = exp(-m) C,
n~ = exp(-m) n) and the adjoints are carried as E^_t = exp(m_t) E_t,
e^_t = exp(m_t) e_t. Substituting gives the same recurrences with the
stabilised factors f'_t = exp(log f_t + m_{t-1} - m_t) and
i'_t = exp(i~_t - m_t), both at most 1:
    g~_t = dh_t o_t / den~_t,  den~_t = max(|z~_t|, exp(-m_t))
    dz~_t = -sign(z~_t) [|z~_t| > exp(-m_t)] (g~_t . num~_t) / den~_t
    E^_t = g~_t q_t^T + f'_{t+1} E^_{t+1}   (and e^_t with dz~_t)
    dq_t = C~_t^T g~_t + dz~_t n~_t
    dv_t = i'_t E^_t k_t,  dk_t = i'_t (E^_t^T v_t + e^_t)
    dlog f_t = f'_t (<E^_t, C~_{t-1}> + e^_t . n~_{t-1})
The initial state is given in stabilised units (C~_0, n~_0, m_0), so
C_0 = exp(m_0) C~_0 and
    dL/dC~_0 = f'_1 E^_1,  dL/dn~_0 = f'_1 e^_1,
    dL/dm_0 = <dL/dC~_0, C~_0> + dL/dn~_0 . n~_0.
Without an initial state these are the gradients at the zero state, m_0 = 0.

The stabiliser m_t itself carries no gradient: h does not depend on it.

Readings (listed with the forward's in the design notes): the loss reaches
the cell only through h (no gradient of the final state is taken in); at the
two kinks of the forward, |z_t| = 1 and z_t = 0, the one-sided derivative
with the floor inactive at equality is used (they have measure zero).

Function:
  mlstm_backward   all gradients of sum(dh * h), float64
"""
from __future__ import annotations

import numpy as np

from .mlstm_oracle import logsigmoid, sigmoid

__all__ = ["mlstm_backward"]


def mlstm_backward(q, k, v, i_pre, f_pre, o_pre, dh, C0=None, n0=None, m0=None):
    """Gradients of L = sum(dh * h) through the stabilised mLSTM recurrence.

    q, k [..., T, d_qk]; v, o_pre, dh [..., T, d_v]; i_pre, f_pre [..., T];
    optional initial state C0 [..., d_v, d_qk], n0 [..., d_qk], m0 [...] in
    stabilised units. Returns a dict of float64 arrays shaped like the
    inputs: dq, dk, dv, di (of i~), df (of f~), do (of o~), dC0, dn0, dm0.
    Stores every step's state: meant for small sequences.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); o_pre = np.asarray(o_pre, np.float64)
    dh = np.asarray(dh, np.float64)
    i_pre = np.asarray(i_pre, np.float64); f_pre = np.asarray(f_pre, np.float64)
    lead = q.shape[:-2]
    T, d_qk = q.shape[-2], q.shape[-1]
    d_v = v.shape[-1]
    Cs = np.zeros(lead + (T + 1, d_v, d_qk))      # Cs[..., t] = C~ after t tokens
    ns = np.zeros(lead + (T + 1, d_qk))
    if C0 is not None:
        Cs[..., 0, :, :] = np.asarray(C0, np.float64)
        ns[..., 0, :] = np.asarray(n0, np.float64)
    m = np.zeros(lead) if m0 is None else np.array(m0, np.float64)
    fp = np.empty(lead + (T,))     # f'_t
    ip = np.empty(lead + (T,))     # i'_t
    gt = np.empty(lead + (T, d_v))  # g~_t
    dz = np.empty(lead + (T,))     # dz~_t
    out = {"dq": np.empty(lead + (T, d_qk)), "dk": np.empty(lead + (T, d_qk)),
           "dv": np.empty(lead + (T, d_v)), "di": np.empty(lead + (T,)),
           "df": np.empty(lead + (T,)), "do": np.empty(lead + (T, d_v))}

    # forward sweep: states, then the per-step quantities that need only them
    for t in range(T):
        log_f = logsigmoid(f_pre[..., t])
        with np.errstate(over="ignore", invalid="ignore"):
            m_new = np.maximum(log_f + m, i_pre[..., t])
            fp[..., t] = np.exp(log_f + m - m_new)
            ip[..., t] = np.exp(i_pre[..., t] - m_new)
        C = (fp[..., t, None, None] * Cs[..., t, :, :]
             + ip[..., t, None, None] * (v[..., t, :, None] * k[..., t, None, :]))
        n = fp[..., t, None] * ns[..., t, :] + ip[..., t, None] * k[..., t, :]
        Cs[..., t + 1, :, :] = C
        ns[..., t + 1, :] = n
        num = np.einsum("...vk,...k->...v", C, q[..., t, :])
        z = np.einsum("...k,...k->...", n, q[..., t, :])
        floor = np.exp(-m_new)
        den = np.maximum(np.abs(z), floor)
        og = sigmoid(o_pre[..., t, :])
        g = dh[..., t, :] * og / den[..., None]
        active = np.abs(z) > floor
        dz_t = np.where(active, -np.sign(z) * np.einsum("...v,...v->...", g, num) / den, 0.0)
        gt[..., t, :] = g
        dz[..., t] = dz_t
        out["dq"][..., t, :] = np.einsum("...vk,...v->...k", C, g) + dz_t[..., None] * n
        out["do"][..., t, :] = dh[..., t, :] * (num / den[..., None]) * og * (1.0 - og)
        m = m_new

    # reverse sweep: adjoints of the state
    E = np.zeros(lead + (d_v, d_qk))
    e = np.zeros(lead + (d_qk,))
    f_next = np.zeros(lead)        # f'_{t+1}; no step after the last
    for t in range(T - 1, -1, -1):
        E = gt[..., t, :, None] * q[..., t, None, :] + f_next[..., None, None] * E
        e = dz[..., t, None] * q[..., t, :] + f_next[..., None] * e
        dv = ip[..., t, None] * np.einsum("...vk,...k->...v", E, k[..., t, :])
        dk = ip[..., t, None] * (np.einsum("...vk,...v->...k", E, v[..., t, :]) + e)
        out["dv"][..., t, :] = dv
        out["dk"][..., t, :] = dk
        out["di"][..., t] = np.einsum("...k,...k->...", k[..., t, :], dk)
        dlogf = fp[..., t] * (np.einsum("...vk,...vk->...", E, Cs[..., t, :, :])
                              + np.einsum("...k,...k->...", e, ns[..., t, :]))
        out["df"][..., t] = dlogf * sigmoid(-f_pre[..., t])
        f_next = fp[..., t]
    out["dC0"] = f_next[..., None, None] * E
    out["dn0"] = f_next[..., None] * e
    out["dm0"] = (np.einsum("...vk,...vk->...", out["dC0"], Cs[..., 0, :, :])
                  + np.einsum("...k,...k->...", out["dn0"], ns[..., 0, :]))
    return out
