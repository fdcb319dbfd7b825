"""Seeded synthetic inputs for the mLSTM cell forward and decode step, for
the sLSTM cell forward (make_slstm_inputs, make_slstm_state) and for the
mLSTM block around the cell (make_block_inputs).

This module draws random numbers and nothing else of the method: it holds no
gate activation, no recurrence and no normalisation. The same arrays feed the
HIP path and the CPU oracle.

Recipe (the workloads described for the mLSTM cell; no dataset is involved):
  * one ``numpy.random.Generator(PCG64(seed))`` per call, draws in the fixed
    order q, k, v, input-gate preactivation, forget-gate preactivation,
    output-gate preactivation;
  * q, k, v ~ N(0, 1); k is multiplied by 1/sqrt(d_qk), the key scaling that
    the xLSTM guide places inside the key projection (aifetchly guide,
    "mLSTM: Matrix Key-Value Memory", recurrent formulation);
  * input-gate preactivation ~ N(i_mean, i_std), forget-gate preactivation
    ~ N(f_mean, f_std), output-gate preactivation ~ N(0, 1);
  * values are drawn in float32; for ``dtype="bf16"`` the q/k/v/output-gate
    arrays are rounded to bfloat16 (round to nearest even on the bit pattern)
    and kept as float32 arrays holding bf16-representable values, so the
    device copy and the oracle's float64 copy hold exactly the same numbers.
    Gate preactivations stay float32.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits",
    "bf16_round",
    "make_fwd_inputs",
    "make_grad_output",
    "make_step_inputs",
    "make_state",
    "make_slstm_inputs",
    "make_slstm_state",
    "make_block_inputs",
]


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns.

    Works on the 32-bit patterns: adding 0x7FFF plus the lowest kept bit and
    dropping the low half rounds to nearest even; no finite value or infinity
    carries out of 32 bits. NaNs become the quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    rounded = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 value; the result is float32."""
    bits = bf16_bits(x).astype(np.uint32) << 16
    return bits.view(np.float32)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "fp32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(f"dtype must be 'fp32' or 'bf16', got {dtype!r}")


def make_fwd_inputs(B: int, H: int, T: int, d_qk: int, d_v: int, dtype: str = "fp32",
                    seed: int = 0, i_mean: float = 0.0, i_std: float = 1.0,
                    f_mean: float = 3.0, f_std: float = 1.0) -> dict:
    """Inputs of one full-sequence forward, laid out [B, H, T, d] / [B, H, T].

    Returns a dict with float32 arrays ``q, k, v, o_pre`` (bf16-representable
    when ``dtype == "bf16"``) and float32 ``i_pre, f_pre``.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, T, d_qk), dtype=np.float32)
    k = rng.standard_normal((B, H, T, d_qk), dtype=np.float32) * np.float32(1.0 / np.sqrt(d_qk))
    v = rng.standard_normal((B, H, T, d_v), dtype=np.float32)
    i_pre = (rng.standard_normal((B, H, T), dtype=np.float32) * np.float32(i_std)
             + np.float32(i_mean))
    f_pre = (rng.standard_normal((B, H, T), dtype=np.float32) * np.float32(f_std)
             + np.float32(f_mean))
    o_pre = rng.standard_normal((B, H, T, d_v), dtype=np.float32)
    return {
        "q": _cast(q, dtype), "k": _cast(k, dtype), "v": _cast(v, dtype),
        "i_pre": i_pre.astype(np.float32), "f_pre": f_pre.astype(np.float32),
        "o_pre": _cast(o_pre, dtype), "dtype": dtype,
    }


def make_grad_output(B: int, H: int, T: int, d_v: int, dtype: str = "fp32", seed: int = 0,
                     scale: float = 1.0) -> np.ndarray:
    """Upstream gradient dL/dh of a full-sequence forward, [B, H, T, d_v].

    Drawn from its own stream ``PCG64([seed, 0xD0])`` so that it does not
    shift the forward's draws: N(0, 1) times ``scale``, in float32, rounded to
    bfloat16 for ``dtype == "bf16"`` like the forward's activations.
    """
    rng = np.random.Generator(np.random.PCG64([seed, 0xD0]))
    dh = rng.standard_normal((B, H, T, d_v), dtype=np.float32) * np.float32(scale)
    return _cast(dh, dtype)


def make_step_inputs(B: int, H: int, d_qk: int, d_v: int, step: int, dtype: str = "fp32",
                     seed: int = 0) -> dict:
    """Inputs of one decode step, laid out [B, H, d] / [B, H].

    Each step draws from its own stream ``PCG64([seed, step])`` so that steps
    can be generated one at a time, in the same order of draws as above.
    """
    rng = np.random.Generator(np.random.PCG64([seed, step]))
    q = rng.standard_normal((B, H, d_qk), dtype=np.float32)
    k = rng.standard_normal((B, H, d_qk), dtype=np.float32) * np.float32(1.0 / np.sqrt(d_qk))
    v = rng.standard_normal((B, H, d_v), dtype=np.float32)
    i_pre = rng.standard_normal((B, H), dtype=np.float32)
    f_pre = rng.standard_normal((B, H), dtype=np.float32) + np.float32(3.0)
    o_pre = rng.standard_normal((B, H, d_v), dtype=np.float32)
    return {
        "q": _cast(q, dtype), "k": _cast(k, dtype), "v": _cast(v, dtype),
        "i_pre": i_pre, "f_pre": f_pre, "o_pre": _cast(o_pre, dtype), "dtype": dtype,
    }


def make_state(B: int, H: int, d_qk: int, d_v: int, seed: int = 0, m_scale: float = 1.0) -> dict:
    """A random, well-scaled recurrent state (C [B,H,d_v,d_qk], n [B,H,d_qk], m [B,H]), float32.

    Used where a test needs a non-zero initial state that no prefill produced.
    """
    rng = np.random.Generator(np.random.PCG64([seed, 0x5EED]))
    C = rng.standard_normal((B, H, d_v, d_qk), dtype=np.float32) * np.float32(0.5)
    n = rng.standard_normal((B, H, d_qk), dtype=np.float32) * np.float32(0.5)
    m = rng.standard_normal((B, H), dtype=np.float32) * np.float32(m_scale)
    return {"C": C, "n": n, "m": m.astype(np.float32)}


def make_slstm_inputs(B: int, H: int, T: int, D: int, seed: int = 0, f_mean: float = 0.0,
                      r_scale: float = 0.5):
    """Seeded sLSTM inputs: input-projected gate preactivations and the
    recurrent matrices.

    Draws, in this order, from ``Generator(PCG64(seed))`` in float32:
    ``pre`` [B, T, 4, H, D] ~ N(0, 1) (gates i, f, z, o; the forget gate's
    draws shifted by ``f_mean``), then ``R`` [H, 4, D, D] ~ N(0, 1) scaled by
    r_scale / sqrt(D), so that R h keeps the size of one preactivation.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    pre = rng.standard_normal((B, T, 4, H, D), dtype=np.float32)
    pre[:, :, 1] += np.float32(f_mean)
    R = rng.standard_normal((H, 4, D, D), dtype=np.float32) * np.float32(r_scale / np.sqrt(D))
    return np.ascontiguousarray(pre), np.ascontiguousarray(R, dtype=np.float32)


def make_slstm_state(B: int, H: int, D: int, seed: int = 0):
    """A seeded non-zero sLSTM state (c, n, m, h) [B, H, D], float32: n in
    [0.5, 2), c = n * U(-1, 1), m ~ N(0, 1), h ~ U(-1, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n = rng.uniform(0.5, 2.0, (B, H, D)).astype(np.float32)
    c = (n * rng.uniform(-1.0, 1.0, (B, H, D))).astype(np.float32)
    m = rng.standard_normal((B, H, D), dtype=np.float32)
    h = rng.uniform(-1.0, 1.0, (B, H, D)).astype(np.float32)
    return c, n, m, h


def make_block_inputs(B: int, T: int, D: int, H: int, d_qk: int, d_v: int, KC: int = 4,
                      seed: int = 0, f_mean: float = 3.0) -> tuple:
    """Seeded input and parameters of the mLSTM block around the cell
    (pre-up-projection residual block; inner width E = 2 D = H d_v).

    Returns ``(x, p)``: x [B, T, D] and a dict of parameters. Matrices are
    rounded to bfloat16 (kept as float32 arrays holding bf16 values, like the
    activations above); vectors stay float32. Draws from
    ``Generator(PCG64([seed, 0xB10C]))`` in this order, each N(0, 1) times the
    scale given:

    =========  ==============  ========================================
    name       shape           scale
    =========  ==============  ========================================
    x          [B, T, D]       1
    ln_w       [D]             0.1, plus 1
    ln_b       [D]             0.1
    W_up       [2E, D]         1 / sqrt(D)
    b_up       [2E]            0.1
    conv_w     [E, KC]         1 / sqrt(KC)
    conv_b     [E]             0.1
    W_q, W_k   [H, d_qk, E/H]  1 / sqrt(E/H)
    b_q, b_k   [H d_qk]        0.1
    W_v        [H, d_v, E/H]   1 / sqrt(E/H)
    b_v        [E]             0.1
    w_i, w_f   [H, E]          1.7 / sqrt(E)
    b_i        [H]             0
    b_f        [H]             0, plus f_mean
    gn_w       [E]             0.1, plus 1
    gn_b       [E]             0.1
    skip       [E]             0.1, plus 1
    W_down     [D, E]          1 / sqrt(E)
    b_down     [D]             0.1
    =========  ==============  ========================================

    The 1.7 / sqrt(E) gate weights give gate preactivations of about unit
    spread over the block's conv outputs (whose mean square is about 0.35),
    so that the forget gate's preactivation is near N(f_mean, 1) and the
    input gate's near N(0, 1), the spreads of the cell workloads.
    eps_ln = eps_gn = 1e-5.
    """
    E = 2 * D
    if H * d_v != E or E % H:
        raise ValueError("need H * d_v == 2 * D")
    rng = np.random.Generator(np.random.PCG64([seed, 0xB10C]))
    n = lambda shape, s: rng.standard_normal(shape, dtype=np.float32) * np.float32(s)
    x = bf16_round(n((B, T, D), 1.0))
    p = {}
    p["ln_w"] = n((D,), 0.1) + np.float32(1.0)
    p["ln_b"] = n((D,), 0.1)
    p["W_up"] = bf16_round(n((2 * E, D), 1.0 / np.sqrt(D)))
    p["b_up"] = n((2 * E,), 0.1)
    p["conv_w"] = n((E, KC), 1.0 / np.sqrt(KC))
    p["conv_b"] = n((E,), 0.1)
    p["W_q"] = bf16_round(n((H, d_qk, E // H), 1.0 / np.sqrt(E // H)))
    p["b_q"] = n((H * d_qk,), 0.1)
    p["W_k"] = bf16_round(n((H, d_qk, E // H), 1.0 / np.sqrt(E // H)))
    p["b_k"] = n((H * d_qk,), 0.1)
    p["W_v"] = bf16_round(n((H, d_v, E // H), 1.0 / np.sqrt(E // H)))
    p["b_v"] = n((E,), 0.1)
    p["w_i"] = bf16_round(n((H, E), 1.7 / np.sqrt(E)))
    p["w_f"] = bf16_round(n((H, E), 1.7 / np.sqrt(E)))
    p["b_i"] = np.zeros(H, np.float32)
    p["b_f"] = np.full(H, f_mean, np.float32)
    p["gn_w"] = n((E,), 0.1) + np.float32(1.0)
    p["gn_b"] = n((E,), 0.1)
    p["skip"] = n((E,), 0.1) + np.float32(1.0)
    p["W_down"] = bf16_round(n((D, E), 1.0 / np.sqrt(E)))
    p["b_down"] = n((D,), 0.1)
    p["eps_ln"] = 1e-5
    p["eps_gn"] = 1e-5
    return x, p
