"""Seeded synthetic inputs for the mLSTM cell forward and decode step, and
for the sLSTM cell forward (make_slstm_inputs, make_slstm_state).

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
