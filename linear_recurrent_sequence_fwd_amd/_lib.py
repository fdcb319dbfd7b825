"""ctypes binding of libmlstm.so: the C ABI declared in include/mlstm.h,
include/slstm.h and (measurement entry points) include/mlstm_prof.h.

Argument marshalling only. Tensors supply device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
If the library is missing the calls raise; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_int, c_int32, c_int64, c_size_t, c_void_p, c_char_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmlstm.so")

MLSTM_FP32, MLSTM_BF16 = 0, 1
STATUS = {
    0: "MLSTM_OK", -1: "MLSTM_ERR_NULLPTR", -2: "MLSTM_ERR_BAD_SHAPE", -3: "MLSTM_ERR_BAD_DTYPE",
    -4: "MLSTM_ERR_MISALIGNED", -5: "MLSTM_ERR_ALIAS", -6: "MLSTM_ERR_WORKSPACE",
    -7: "MLSTM_ERR_UNSUPPORTED", -8: "MLSTM_ERR_HIP",
}
PROF_GROUPS = ("gate", "state", "out")   # kernel groups of mlstm_prof_fwd_chunkwise, in order
# kernel groups of mlstm_prof_bwd_chunkwise, in order
BWD_PROF_GROUPS = ("fwd_gate", "fwd_state", "dq", "adjoint", "dkv", "dgate")


class FwdArgs(ctypes.Structure):
    _fields_ = [
        ("B", c_int64), ("H", c_int64), ("T", c_int64), ("d_qk", c_int64), ("d_v", c_int64),
        ("dtype", c_int32),
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("o_pre", c_void_p),
        ("i_pre", c_void_p), ("f_pre", c_void_p), ("h", c_void_p),
        ("C0", c_void_p), ("n0", c_void_p), ("m0", c_void_p),
        ("C_out", c_void_p), ("n_out", c_void_p), ("m_out", c_void_p),
    ]


class StepArgs(ctypes.Structure):
    _fields_ = [
        ("B", c_int64), ("H", c_int64), ("d_qk", c_int64), ("d_v", c_int64), ("dtype", c_int32),
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("o_pre", c_void_p),
        ("i_pre", c_void_p), ("f_pre", c_void_p),
        ("C", c_void_p), ("n_in", c_void_p), ("m_in", c_void_p),
        ("n_out", c_void_p), ("m_out", c_void_p), ("h", c_void_p),
    ]


class BwdArgs(ctypes.Structure):
    _fields_ = [
        ("B", c_int64), ("H", c_int64), ("T", c_int64), ("d_qk", c_int64), ("d_v", c_int64),
        ("dtype", c_int32),
        ("q", c_void_p), ("k", c_void_p), ("v", c_void_p), ("o_pre", c_void_p),
        ("i_pre", c_void_p), ("f_pre", c_void_p), ("h", c_void_p), ("dh", c_void_p),
        ("C0", c_void_p), ("n0", c_void_p), ("m0", c_void_p),
        ("dq", c_void_p), ("dk", c_void_p), ("dv", c_void_p), ("do_pre", c_void_p),
        ("di_pre", c_void_p), ("df_pre", c_void_p),
        ("dC0", c_void_p), ("dn0", c_void_p), ("dm0", c_void_p),
    ]


class SlstmArgs(ctypes.Structure):
    _fields_ = [
        ("B", c_int64), ("H", c_int64), ("T", c_int64), ("D", c_int64),
        ("pre", c_void_p), ("R", c_void_p), ("h", c_void_p),
        ("c0", c_void_p), ("n0", c_void_p), ("m0", c_void_p), ("h0", c_void_p),
        ("c_out", c_void_p), ("n_out", c_void_p), ("m_out", c_void_p), ("h_out", c_void_p),
    ]


class MlstmError(RuntimeError):
    def __init__(self, code: int, what: str, detail: str):
        super().__init__(f"{what} failed: {STATUS.get(code, code)}: {detail}")
        self.code = code


_lib = None

# MLSTM_ABI_VERSION of include/mlstm.h that the argument structs here follow
ABI_VERSION = 2


def lib() -> ctypes.CDLL:
    """The loaded library with argument types set (loaded once)."""
    global _lib
    if _lib is None:
        # torch's HIP runtime carries the same soname; loading torch first
        # makes the library bind to it, so torch streams and events are valid.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_recurrent_sequence_fwd_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.mlstm_fwd_chunkwise_workspace_size.argtypes = [P(FwdArgs), c_int]
        L.mlstm_fwd_chunkwise_workspace_size.restype = c_size_t
        L.mlstm_fwd_chunkwise.argtypes = [P(FwdArgs), c_int, c_void_p, c_size_t, c_void_p]
        L.mlstm_fwd_chunkwise.restype = c_int
        L.mlstm_fwd_chunkwise_noalloc_limit.argtypes = []
        L.mlstm_fwd_chunkwise_noalloc_limit.restype = c_size_t
        L.mlstm_fwd_chunkwise_noalloc.argtypes = [P(FwdArgs), c_int, c_void_p]
        L.mlstm_fwd_chunkwise_noalloc.restype = c_int
        L.mlstm_fwd_parallel_workspace_size.argtypes = [P(FwdArgs)]
        L.mlstm_fwd_parallel_workspace_size.restype = c_size_t
        L.mlstm_fwd_parallel.argtypes = [P(FwdArgs), c_void_p, c_size_t, c_void_p]
        L.mlstm_fwd_parallel.restype = c_int
        L.mlstm_bwd_chunkwise_workspace_size.argtypes = [P(BwdArgs), c_int]
        L.mlstm_bwd_chunkwise_workspace_size.restype = c_size_t
        L.mlstm_bwd_chunkwise.argtypes = [P(BwdArgs), c_int, c_void_p, c_size_t, c_void_p]
        L.mlstm_bwd_chunkwise.restype = c_int
        L.mlstm_prof_bwd_chunkwise.argtypes = [P(BwdArgs), c_int, c_void_p, c_size_t, c_void_p,
                                               P(c_void_p)]
        L.mlstm_prof_bwd_chunkwise.restype = c_int
        L.mlstm_step.argtypes = [P(StepArgs), c_void_p]
        L.mlstm_step.restype = c_int
        L.mlstm_status_string.argtypes = [c_int]
        L.mlstm_status_string.restype = c_char_p
        L.mlstm_last_error.argtypes = []
        L.mlstm_last_error.restype = c_char_p
        L.mlstm_abi_version.argtypes = []
        L.mlstm_abi_version.restype = c_int
        if L.mlstm_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.mlstm_abi_version()}, the binding "
                               f"follows version {ABI_VERSION}: rebuild the library")
        L.mlstm_prof_fwd_chunkwise.argtypes = [P(FwdArgs), c_int, c_void_p, c_size_t, c_void_p,
                                               P(c_void_p)]
        L.mlstm_prof_fwd_chunkwise.restype = c_int
        L.mlstm_prof_step.argtypes = [P(StepArgs), c_void_p, c_void_p, c_void_p]
        L.mlstm_prof_step.restype = c_int
        L.mlstm_prof_copy_lds.argtypes = [c_void_p, c_void_p, c_size_t, c_void_p]
        L.mlstm_prof_copy_lds.restype = c_int
        L.mlstm_clock_probe.argtypes = [c_void_p, c_int, c_void_p]
        L.mlstm_clock_probe.restype = c_int
        L.slstm_fwd.argtypes = [P(SlstmArgs), c_void_p]
        L.slstm_fwd.restype = c_int
        _lib = L
    return _lib


def _check(code: int, what: str) -> None:
    if code != 0:
        raise MlstmError(code, what, lib().mlstm_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MLSTM_BF16
    if t.dtype == torch.float32:
        return MLSTM_FP32
    raise TypeError(f"q/k/v/o_pre must be float32 or bfloat16, got {t.dtype}")


def _require(t, name, shape, dtype):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd_args(q, k, v, o_pre, i_pre, f_pre, h, C0=None, n0=None, m0=None,
             C_out=None, n_out=None, m_out=None) -> FwdArgs:
    """Fill the argument struct of a forward call from tensors (shapes checked)."""
    import torch
    B, H, T, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    for name, t, shp in (("q", q, (B, H, T, K)), ("k", k, (B, H, T, K)), ("v", v, (B, H, T, V)),
                         ("o_pre", o_pre, (B, H, T, V)), ("h", h, (B, H, T, V))):
        _require(t, name, shp, dt)
    _require(i_pre, "i_pre", (B, H, T), torch.float32)
    _require(f_pre, "f_pre", (B, H, T), torch.float32)
    if C0 is not None:
        _require(C0, "C0", (B, H, V, K), torch.float32)
        _require(n0, "n0", (B, H, K), torch.float32)
        _require(m0, "m0", (B, H), torch.float32)
    if C_out is not None:
        _require(C_out, "C_out", (B, H, V, K), torch.float32)
        _require(n_out, "n_out", (B, H, K), torch.float32)
        _require(m_out, "m_out", (B, H), torch.float32)
    return FwdArgs(B, H, T, K, V, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o_pre),
                   _ptr(i_pre), _ptr(f_pre), _ptr(h), _ptr(C0), _ptr(n0), _ptr(m0),
                   _ptr(C_out), _ptr(n_out), _ptr(m_out))


def chunkwise_workspace_bytes(args: FwdArgs, chunk: int) -> int:
    return int(lib().mlstm_fwd_chunkwise_workspace_size(ctypes.byref(args), chunk))


def parallel_workspace_bytes(args: FwdArgs) -> int:
    return int(lib().mlstm_fwd_parallel_workspace_size(ctypes.byref(args)))


def _workspace(nbytes, device, workspace):
    import torch
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace smaller than {nbytes} bytes")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _state_out(q, v, want):
    import torch
    if not want:
        return None, None, None
    B, H, _, K = q.shape
    V = v.shape[-1]
    dev = q.device
    return (torch.empty((B, H, V, K), dtype=torch.float32, device=dev),
            torch.empty((B, H, K), dtype=torch.float32, device=dev),
            torch.empty((B, H), dtype=torch.float32, device=dev))


def mlstm_fwd_chunkwise(q, k, v, o_pre, i_pre, f_pre, chunk=64, C0=None, n0=None, m0=None,
                        return_state=False, h=None, workspace=None, stream=None):
    """Chunkwise forward. Returns h, or (h, (C, n, m)) when return_state."""
    import torch
    if h is None:
        h = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    C_out, n_out, m_out = _state_out(q, v, return_state)
    args = fwd_args(q, k, v, o_pre, i_pre, f_pre, h, C0, n0, m0, C_out, n_out, m_out)
    nbytes = chunkwise_workspace_bytes(args, chunk)
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib().mlstm_fwd_chunkwise(ctypes.byref(args), int(chunk), _ptr(ws), nbytes, _stream(stream)),
           "mlstm_fwd_chunkwise")
    return (h, (C_out, n_out, m_out)) if return_state else h


def mlstm_fwd_chunkwise_noalloc(q, k, v, o_pre, i_pre, f_pre, chunk=64, C0=None, n0=None, m0=None,
                                return_state=False, h=None, stream=None):
    """Chunkwise forward through the no-allocation entry point (the library's
    fixed per-device scratch instead of a workspace). Returns h, or
    (h, (C, n, m)) when return_state. Outputs are allocated here unless given."""
    import torch
    if h is None:
        h = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    C_out, n_out, m_out = _state_out(q, v, return_state)
    args = fwd_args(q, k, v, o_pre, i_pre, f_pre, h, C0, n0, m0, C_out, n_out, m_out)
    _check(lib().mlstm_fwd_chunkwise_noalloc(ctypes.byref(args), int(chunk), _stream(stream)),
           "mlstm_fwd_chunkwise_noalloc")
    return (h, (C_out, n_out, m_out)) if return_state else h


def mlstm_fwd_parallel(q, k, v, o_pre, i_pre, f_pre, C0=None, n0=None, m0=None,
                       return_state=False, h=None, workspace=None, stream=None):
    """Parallel (dual) form for T <= 8192. Returns h, or (h, (C, n, m))."""
    import torch
    if h is None:
        h = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    C_out, n_out, m_out = _state_out(q, v, return_state)
    args = fwd_args(q, k, v, o_pre, i_pre, f_pre, h, C0, n0, m0, C_out, n_out, m_out)
    nbytes = parallel_workspace_bytes(args)
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib().mlstm_fwd_parallel(ctypes.byref(args), _ptr(ws), nbytes, _stream(stream)),
           "mlstm_fwd_parallel")
    return (h, (C_out, n_out, m_out)) if return_state else h


def bwd_args(q, k, v, o_pre, i_pre, f_pre, h, dh, grads, C0=None, n0=None, m0=None) -> BwdArgs:
    """Fill the argument struct of a backward call from tensors (shapes
    checked). `grads` maps dq, dk, dv, do, di, df (and optionally dC0, dn0,
    dm0) to output tensors."""
    import torch
    B, H, T, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    for name, t, shp in (("q", q, (B, H, T, K)), ("k", k, (B, H, T, K)), ("v", v, (B, H, T, V)),
                         ("o_pre", o_pre, (B, H, T, V)), ("h", h, (B, H, T, V)),
                         ("dh", dh, (B, H, T, V)), ("dq", grads["dq"], (B, H, T, K)),
                         ("dk", grads["dk"], (B, H, T, K)), ("dv", grads["dv"], (B, H, T, V)),
                         ("do", grads["do"], (B, H, T, V))):
        _require(t, name, shp, dt)
    for name, t in (("i_pre", i_pre), ("f_pre", f_pre), ("di", grads["di"]), ("df", grads["df"])):
        _require(t, name, (B, H, T), torch.float32)
    if C0 is not None:
        _require(C0, "C0", (B, H, V, K), torch.float32)
        _require(n0, "n0", (B, H, K), torch.float32)
        _require(m0, "m0", (B, H), torch.float32)
    dC0, dn0, dm0 = grads.get("dC0"), grads.get("dn0"), grads.get("dm0")
    if dC0 is not None:
        _require(dC0, "dC0", (B, H, V, K), torch.float32)
        _require(dn0, "dn0", (B, H, K), torch.float32)
        _require(dm0, "dm0", (B, H), torch.float32)
    return BwdArgs(B, H, T, K, V, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o_pre),
                   _ptr(i_pre), _ptr(f_pre), _ptr(h), _ptr(dh), _ptr(C0), _ptr(n0), _ptr(m0),
                   _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]), _ptr(grads["do"]),
                   _ptr(grads["di"]), _ptr(grads["df"]), _ptr(dC0), _ptr(dn0), _ptr(dm0))


def bwd_workspace_bytes(args: BwdArgs, chunk: int) -> int:
    return int(lib().mlstm_bwd_chunkwise_workspace_size(ctypes.byref(args), chunk))


def bwd_outputs(q, v, init_grad=False) -> dict:
    """Freshly allocated gradient outputs for a backward call."""
    import torch
    B, H, T, K = q.shape
    V = v.shape[-1]
    dev, dt = q.device, q.dtype
    g = {"dq": torch.empty((B, H, T, K), dtype=dt, device=dev),
         "dk": torch.empty((B, H, T, K), dtype=dt, device=dev),
         "dv": torch.empty((B, H, T, V), dtype=dt, device=dev),
         "do": torch.empty((B, H, T, V), dtype=dt, device=dev),
         "di": torch.empty((B, H, T), dtype=torch.float32, device=dev),
         "df": torch.empty((B, H, T), dtype=torch.float32, device=dev)}
    if init_grad:
        g["dC0"] = torch.empty((B, H, V, K), dtype=torch.float32, device=dev)
        g["dn0"] = torch.empty((B, H, K), dtype=torch.float32, device=dev)
        g["dm0"] = torch.empty((B, H), dtype=torch.float32, device=dev)
    return g


def mlstm_bwd_chunkwise(q, k, v, o_pre, i_pre, f_pre, h, dh, chunk=64, C0=None, n0=None, m0=None,
                        init_grad=False, grads=None, workspace=None, stream=None):
    """Chunkwise backward pass: gradients of a loss through h (dh = dL/dh).
    Returns a dict with dq, dk, dv, do (of o_pre), di (of i_pre), df (of
    f_pre) and, when init_grad, dC0, dn0, dm0. `h` is the forward's output."""
    if grads is None:
        grads = bwd_outputs(q, v, init_grad)
    args = bwd_args(q, k, v, o_pre, i_pre, f_pre, h, dh, grads, C0, n0, m0)
    nbytes = bwd_workspace_bytes(args, chunk)
    ws = _workspace(nbytes, q.device, workspace)
    _check(lib().mlstm_bwd_chunkwise(ctypes.byref(args), int(chunk), _ptr(ws), nbytes, _stream(stream)),
           "mlstm_bwd_chunkwise")
    return grads


def step_args(q, k, v, o_pre, i_pre, f_pre, C, n_in, m_in, n_out, m_out, h) -> StepArgs:
    import torch
    B, H, K = q.shape
    V = v.shape[-1]
    dt = q.dtype
    for name, t, shp in (("q", q, (B, H, K)), ("k", k, (B, H, K)), ("v", v, (B, H, V)),
                         ("o_pre", o_pre, (B, H, V)), ("h", h, (B, H, V))):
        _require(t, name, shp, dt)
    for name, t, shp in (("i_pre", i_pre, (B, H)), ("f_pre", f_pre, (B, H)), ("C", C, (B, H, V, K)),
                         ("n_in", n_in, (B, H, K)), ("m_in", m_in, (B, H)),
                         ("n_out", n_out, (B, H, K)), ("m_out", m_out, (B, H))):
        _require(t, name, shp, torch.float32)
    return StepArgs(B, H, K, V, _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o_pre),
                    _ptr(i_pre), _ptr(f_pre), _ptr(C), _ptr(n_in), _ptr(m_in), _ptr(n_out),
                    _ptr(m_out), _ptr(h))


def mlstm_step(q, k, v, o_pre, i_pre, f_pre, C, n_in, m_in, n_out=None, m_out=None, h=None,
               stream=None):
    """One decode step; C is updated in place. Returns (h, n_out, m_out)."""
    import torch
    if h is None:
        h = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    if n_out is None:
        n_out = torch.empty_like(n_in)
    if m_out is None:
        m_out = torch.empty_like(m_in)
    args = step_args(q, k, v, o_pre, i_pre, f_pre, C, n_in, m_in, n_out, m_out, h)
    _check(lib().mlstm_step(ctypes.byref(args), _stream(stream)), "mlstm_step")
    return h, n_out, m_out


def event_array(events):
    """A ctypes array of hipEvent_t handles (ints or None): six for
    mlstm_prof_fwd_chunkwise (before/after of each group in PROF_GROUPS),
    twelve for mlstm_prof_bwd_chunkwise (BWD_PROF_GROUPS)."""
    if len(events) not in (2 * len(PROF_GROUPS), 2 * len(BWD_PROF_GROUPS)):
        raise ValueError("six or twelve event handles are needed")
    return (c_void_p * len(events))(*events)


def clock_probe(ticks, iters: int, stream=None) -> None:
    """Launch the clock probe; `ticks` is a 4-element int64 CUDA tensor that receives
    the shader-clock counter (start, end) and the constant-rate counter (start, end)."""
    import torch
    _require(ticks, "ticks", (4,), torch.int64)
    _check(lib().mlstm_clock_probe(_ptr(ticks), int(iters), _stream(stream)), "mlstm_clock_probe")


def copy_lds(src, dst, stream=None) -> None:
    """Direct-to-LDS copy of src into dst (device tensors of equal byte size,
    a multiple of 16 KiB): the counter-calibration kernel of mlstm_prof.h."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _check(lib().mlstm_prof_copy_lds(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "mlstm_prof_copy_lds")


def slstm_fwd(pre, R, state=None, want_state=False, h=None, stream=None):
    """sLSTM forward over a sequence. pre [B, T, 4, H, D], R [H, 4, D, D] float32
    device tensors; state = (c0, n0, m0, h0) [B, H, D] each or None. Returns h
    [B, T, H, D], and the final (c, n, m, h) when want_state."""
    import torch
    if pre is None or R is None:
        raise ValueError("pre and R are required")
    B, T, four, H, D = pre.shape
    if four != 4:
        raise ValueError(f"pre must be [B, T, 4, H, D], got {tuple(pre.shape)}")
    _require(pre, "pre", (B, T, 4, H, D), torch.float32)
    _require(R, "R", (H, 4, D, D), torch.float32)
    if h is None:
        h = torch.empty((B, T, H, D), dtype=torch.float32, device=pre.device)
    _require(h, "h", (B, T, H, D), torch.float32)
    st_in = (None,) * 4 if state is None else tuple(state)
    if state is not None:
        for name, t in zip(("c0", "n0", "m0", "h0"), st_in):
            _require(t, name, (B, H, D), torch.float32)
    st_out = tuple(torch.empty((B, H, D), dtype=torch.float32, device=pre.device) for _ in range(4)) \
        if want_state else (None,) * 4
    args = SlstmArgs(B, H, T, D, _ptr(pre), _ptr(R), _ptr(h), *[_ptr(t) for t in st_in],
                     *[_ptr(t) for t in st_out])
    _check(lib().slstm_fwd(ctypes.byref(args), _stream(stream)), "slstm_fwd")
    return (h, st_out) if want_state else h
