"""ctypes front of the C float64 oracle (oracle/mlstm_ref.c).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the bench's CPU
baseline, never by the product path. The C file is the same stabilised step
recurrence as ``mlstm_oracle.mlstm_recurrent`` and the same reverse mode as
``mlstm_grad.mlstm_backward``, one sequence per host thread, so that whole
outputs of the large workloads can be compared.
``build()`` compiles it with gcc into oracle/libmlstm_ref.so; ``lib()`` builds
it first when the library is missing or older than its source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mlstm_ref.c")
LIB = os.path.join(HERE, "libmlstm_ref.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle (plain -O2, no vector extensions beyond the base ISA)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        L.mlstm_ref_run.argtypes = [ctypes.c_int64] * 4 + [P] * 6 + [P] * 4 + [ctypes.c_int]
        L.mlstm_ref_run.restype = ctypes.c_int
        L.mlstm_ref_bwd.argtypes = ([ctypes.c_int64] * 4 + [P] * 7 + [P] * 3 + [P] * 9
                                    + [ctypes.c_int64, ctypes.c_int])
        L.mlstm_ref_bwd.restype = ctypes.c_int
        _lib = L
    return _lib


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def mlstm_recurrent_c(q, k, v, i_pre, f_pre, o_pre, C0=None, n0=None, m0=None, threads=None):
    """Same contract as mlstm_oracle.mlstm_recurrent for float32-representable
    inputs (every input the generator makes is): q, k [..., T, d_qk];
    v, o_pre [..., T, d_v]; i_pre, f_pre [..., T]; optional initial state in
    stabilised units. Returns h [..., T, d_v] float64 and (C~, n~, m)."""
    q = _f32(q)
    lead = q.shape[:-2]
    T, K = q.shape[-2], q.shape[-1]
    V = np.shape(v)[-1]
    BH = int(np.prod(lead)) if lead else 1
    a = [_f32(x).reshape(BH, T, -1) for x in (q, k, v)]
    g = [_f32(x).reshape(BH, T) for x in (i_pre, f_pre)]
    o = _f32(o_pre).reshape(BH, T, V)
    C = np.zeros((BH, V, K)) if C0 is None else np.array(C0, np.float64).reshape(BH, V, K).copy()
    n = np.zeros((BH, K)) if n0 is None else np.array(n0, np.float64).reshape(BH, K).copy()
    m = np.zeros(BH) if m0 is None else np.array(m0, np.float64).reshape(BH).copy()
    h = np.empty((BH, T, V))
    rc = lib().mlstm_ref_run(BH, T, K, V, a[0].ctypes.data, a[1].ctypes.data, a[2].ctypes.data,
                             g[0].ctypes.data, g[1].ctypes.data, o.ctypes.data, C.ctypes.data,
                             n.ctypes.data, m.ctypes.data, h.ctypes.data,
                             threads or default_threads())
    if rc != 0:
        raise RuntimeError("mlstm_ref_run could not start its threads")
    return h.reshape(lead + (T, V)), (C.reshape(lead + (V, K)), n.reshape(lead + (K,)), m.reshape(lead))


def mlstm_step_c(q, k, v, i_pre, f_pre, o_pre, C, n, m, threads=None):
    """One step for every (b, h); C [..., d_v, d_qk], n [..., d_qk], m [...] are
    float64 arrays updated IN PLACE (C-contiguous). Returns h [..., d_v]."""
    lead = np.shape(q)[:-1]
    K = np.shape(q)[-1]
    V = np.shape(v)[-1]
    BH = int(np.prod(lead)) if lead else 1
    for arr in (C, n, m):
        assert arr.dtype == np.float64 and arr.flags.c_contiguous
    a = [_f32(x).reshape(BH, 1, -1) for x in (q, k, v, o_pre)]
    g = [_f32(x).reshape(BH, 1) for x in (i_pre, f_pre)]
    h = np.empty((BH, 1, V))
    rc = lib().mlstm_ref_run(BH, 1, K, V, a[0].ctypes.data, a[1].ctypes.data, a[2].ctypes.data,
                             g[0].ctypes.data, g[1].ctypes.data, a[3].ctypes.data, C.ctypes.data,
                             n.ctypes.data, m.ctypes.data, h.ctypes.data,
                             threads or default_threads())
    if rc != 0:
        raise RuntimeError("mlstm_ref_run could not start its threads")
    return h.reshape(lead + (V,))


def mlstm_backward_c(q, k, v, i_pre, f_pre, o_pre, dh, C0=None, n0=None, m0=None, threads=None,
                     seg=0):
    """Same contract as mlstm_grad.mlstm_backward for float32-representable
    inputs: returns a dict of float64 arrays dq, dk, dv, di, df, do, dC0,
    dn0, dm0. ``seg`` is the checkpoint interval of the reverse sweep (0:
    about sqrt(T)); it changes memory, not results."""
    q = _f32(q)
    lead = q.shape[:-2]
    T, K = q.shape[-2], q.shape[-1]
    V = np.shape(v)[-1]
    BH = int(np.prod(lead)) if lead else 1
    a = [_f32(x).reshape(BH, T, -1) for x in (q, k, v)]
    g = [_f32(x).reshape(BH, T) for x in (i_pre, f_pre)]
    o = _f32(o_pre).reshape(BH, T, V)
    d = _f32(dh).reshape(BH, T, V)
    st = [None, None, None]
    if C0 is not None:
        st = [np.ascontiguousarray(np.asarray(C0, np.float64).reshape(BH, V, K)),
              np.ascontiguousarray(np.asarray(n0, np.float64).reshape(BH, K)),
              np.ascontiguousarray(np.asarray(m0, np.float64).reshape(BH))]
    out = {"dq": np.empty((BH, T, K)), "dk": np.empty((BH, T, K)), "dv": np.empty((BH, T, V)),
           "di": np.empty((BH, T)), "df": np.empty((BH, T)), "do": np.empty((BH, T, V)),
           "dC0": np.empty((BH, V, K)), "dn0": np.empty((BH, K)), "dm0": np.empty(BH)}
    ptr = lambda x: None if x is None else x.ctypes.data  # noqa: E731
    rc = lib().mlstm_ref_bwd(BH, T, K, V, a[0].ctypes.data, a[1].ctypes.data, a[2].ctypes.data,
                             g[0].ctypes.data, g[1].ctypes.data, o.ctypes.data, d.ctypes.data,
                             ptr(st[0]), ptr(st[1]), ptr(st[2]),
                             *(out[n].ctypes.data for n in ("dq", "dk", "dv", "di", "df", "do",
                                                            "dC0", "dn0", "dm0")),
                             int(seg), threads or default_threads())
    if rc != 0:
        raise RuntimeError("mlstm_ref_bwd could not allocate its buffers or start its threads")
    shapes = {"dq": (T, K), "dk": (T, K), "dv": (T, V), "di": (T,), "df": (T,), "do": (T, V),
              "dC0": (V, K), "dn0": (K,), "dm0": ()}
    return {n: out[n].reshape(lead + shapes[n]) for n in out}
