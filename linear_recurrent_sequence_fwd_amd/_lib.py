"""ctypes binding of libmlstm.so: the C ABI declared in include/mlstm.h,
include/mlstm_block.h, include/mlstm_segments.h, include/slstm.h and
(measurement entry points) include/mlstm_prof.h.

Argument marshalling only. Tensors supply device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
If the library is missing the calls raise; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_int32, c_int64, c_size_t, c_void_p, c_char_p

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


class GemmArgs(ctypes.Structure):
    _fields_ = [
        ("M", c_int64), ("N", c_int64), ("K", c_int64), ("batch1", c_int64), ("batch2", c_int64),
        ("A", c_void_p), ("lda", c_int64), ("strideA1", c_int64), ("strideA2", c_int64),
        ("B", c_void_p), ("ldb", c_int64), ("strideB1", c_int64), ("strideB2", c_int64),
        ("C", c_void_p), ("ldc", c_int64), ("strideC1", c_int64), ("strideC2", c_int64),
        ("c_dtype", c_int32), ("c_trans", c_int32), ("alpha", c_float),
        ("bias", c_void_p), ("stride_bias2", c_int64),
        ("R", c_void_p), ("ldr", c_int64), ("strideR1", c_int64), ("strideR2", c_int64),
    ]


# parameter arrays of mlstm_block_params, in struct order: (name, bf16 matrix?)
BLOCK_ARRAYS = (("ln_w", False), ("ln_b", False), ("W_up", True), ("b_up", False), ("conv_w", False),
                ("conv_b", False), ("W_q", True), ("W_k", True), ("b_q", False), ("b_k", False),
                ("W_v", True), ("b_v", False), ("w_i", True), ("w_f", True), ("b_i", False), ("b_f", False),
                ("gn_w", False), ("gn_b", False), ("skip", False), ("W_down", True), ("b_down", False))
BLOCK_STAGES = ("xn", "xup", "xc", "q", "k", "v", "i_pre", "f_pre", "h", "y")


class BlockParams(ctypes.Structure):
    _fields_ = ([("D", c_int64), ("H", c_int64), ("d_qk", c_int64), ("d_v", c_int64), ("KC", c_int64),
                 ("eps_ln", c_float), ("eps_gn", c_float)]
                + [(name, c_void_p) for name, _ in BLOCK_ARRAYS])


class SummaryArgs(ctypes.Structure):
    _fields_ = [
        ("B", c_int64), ("H", c_int64), ("T", c_int64), ("d_qk", c_int64), ("d_v", c_int64),
        ("dtype", c_int32),
        ("k", c_void_p), ("v", c_void_p), ("i_pre", c_void_p), ("f_pre", c_void_p),
        ("C_out", c_void_p), ("n_out", c_void_p), ("m_out", c_void_p), ("G_out", c_void_p),
    ]


class CombineArgs(ctypes.Structure):
    _fields_ = [
        ("B", c_int64), ("H", c_int64), ("d_qk", c_int64), ("d_v", c_int64), ("count", c_int64),
        ("C0", c_void_p), ("n0", c_void_p), ("m0", c_void_p),
        ("Cs", c_void_p), ("ns", c_void_p), ("ms", c_void_p), ("Gs", c_void_p),
        ("C_out", c_void_p), ("n_out", c_void_p), ("m_out", c_void_p),
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
ABI_VERSION = 4


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
        L.mlstm_segment_summary_workspace_size.argtypes = [P(SummaryArgs), c_int]
        L.mlstm_segment_summary_workspace_size.restype = c_size_t
        L.mlstm_segment_summary.argtypes = [P(SummaryArgs), c_int, c_void_p, c_size_t, c_void_p]
        L.mlstm_segment_summary.restype = c_int
        L.mlstm_state_combine.argtypes = [P(CombineArgs), c_void_p]
        L.mlstm_state_combine.restype = c_int
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
        L.mlstm_gemm_bf16.argtypes = [P(GemmArgs), c_void_p]
        L.mlstm_gemm_bf16.restype = c_int
        L.mlstm_layernorm_bf16.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_float,
                                           c_void_p]
        L.mlstm_layernorm_bf16.restype = c_int
        L.mlstm_block_conv_gates.argtypes = [P(BlockParams), c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p]
        L.mlstm_block_conv_gates.restype = c_int
        L.mlstm_block_groupnorm_gate.argtypes = [P(BlockParams), c_int64, c_int64, c_void_p, c_void_p,
                                                 c_void_p, c_void_p, c_void_p]
        L.mlstm_block_groupnorm_gate.restype = c_int
        L.mlstm_block_fwd_workspace_size.argtypes = [P(BlockParams), c_int64, c_int64, c_int]
        L.mlstm_block_fwd_workspace_size.restype = c_size_t
        L.mlstm_block_fwd.argtypes = [P(BlockParams), c_int64, c_int64, c_void_p, c_void_p, c_int, c_void_p,
                                      c_size_t, c_void_p]
        L.mlstm_block_fwd.restype = c_int
        L.mlstm_block_workspace_offsets.argtypes = [P(BlockParams), c_int64, c_int64, c_int, P(c_size_t)]
        L.mlstm_block_workspace_offsets.restype = c_int
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
                         ("h", h, (B, H, T, V))):
        _require(t, name, shp, dt)
    if o_pre is not None:   # None: no output gate (chunkwise form, bf16, d_v a multiple of 128)
        _require(o_pre, "o_pre", (B, H, T, V), dt)
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


def summary_args(k, v, i_pre, f_pre, C_out, n_out, m_out, G_out) -> SummaryArgs:
    """Fill the argument struct of a segment summary from tensors (shapes checked)."""
    import torch
    B, H, T, K = k.shape
    V = v.shape[-1]
    _require(k, "k", (B, H, T, K), k.dtype)
    _require(v, "v", (B, H, T, V), k.dtype)
    _require(i_pre, "i_pre", (B, H, T), torch.float32)
    _require(f_pre, "f_pre", (B, H, T), torch.float32)
    _require(C_out, "C_out", (B, H, V, K), torch.float32)
    _require(n_out, "n_out", (B, H, K), torch.float32)
    _require(m_out, "m_out", (B, H), torch.float32)
    _require(G_out, "G_out", (B, H), torch.float64)
    return SummaryArgs(B, H, T, K, V, _dtype_code(k), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre),
                       _ptr(C_out), _ptr(n_out), _ptr(m_out), _ptr(G_out))


def summary_workspace_bytes(args: SummaryArgs, chunk: int) -> int:
    return int(lib().mlstm_segment_summary_workspace_size(ctypes.byref(args), chunk))


def mlstm_segment_summary(k, v, i_pre, f_pre, chunk=256, out=None, workspace=None, stream=None):
    """The summary (C~s, n~s, ms, G) of a segment: its end state from the
    empty state and the sum of its log forget gates. T must be a multiple of
    chunk. `out` may supply the four output tensors."""
    import torch
    B, H, _, K = k.shape
    V = v.shape[-1]
    dev = k.device
    if out is None:
        out = (torch.empty((B, H, V, K), dtype=torch.float32, device=dev),
               torch.empty((B, H, K), dtype=torch.float32, device=dev),
               torch.empty((B, H), dtype=torch.float32, device=dev),
               torch.empty((B, H), dtype=torch.float64, device=dev))
    args = summary_args(k, v, i_pre, f_pre, *out)
    nbytes = summary_workspace_bytes(args, chunk)
    ws = _workspace(nbytes, dev, workspace)
    _check(lib().mlstm_segment_summary(ctypes.byref(args), int(chunk), _ptr(ws), nbytes, _stream(stream)),
           "mlstm_segment_summary")
    return out


def mlstm_state_combine(Cs, ns, ms, Gs, C0=None, n0=None, m0=None, out=None, stream=None):
    """The state after the segments with summaries (Cs, ns, ms, Gs), folded in
    order into (C0, n0, m0), or into the zero state (m0 = 0) when C0 is None.
    One summary has the shapes of a state ([B,H,d_v,d_qk], [B,H,d_qk], [B,H],
    [B,H]); a stack of P summaries has a leading dimension P. Returns (C, n, m)."""
    import torch
    stacked = Cs.dim() == 5
    P = Cs.shape[0] if stacked else 1
    B, H, V, K = Cs.shape[-4:]
    lead = (P,) if stacked else ()
    _require(Cs, "Cs", lead + (B, H, V, K), torch.float32)
    _require(ns, "ns", lead + (B, H, K), torch.float32)
    _require(ms, "ms", lead + (B, H), torch.float32)
    _require(Gs, "Gs", lead + (B, H), torch.float64)
    if C0 is not None:
        _require(C0, "C0", (B, H, V, K), torch.float32)
        _require(n0, "n0", (B, H, K), torch.float32)
        _require(m0, "m0", (B, H), torch.float32)
    if out is None:
        f32 = dict(dtype=torch.float32, device=Cs.device)
        out = (torch.empty((B, H, V, K), **f32), torch.empty((B, H, K), **f32), torch.empty((B, H), **f32))
    args = CombineArgs(B, H, K, V, P, _ptr(C0), _ptr(n0), _ptr(m0), _ptr(Cs), _ptr(ns), _ptr(ms), _ptr(Gs),
                       _ptr(out[0]), _ptr(out[1]), _ptr(out[2]))
    _check(lib().mlstm_state_combine(ctypes.byref(args), _stream(stream)), "mlstm_state_combine")
    return out


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


# ------------------------------------------------------------------ mLSTM block (include/mlstm_block.h)

def gemm_bf16(A, B, bias=None, R=None, alpha=1.0, out_dtype=None, c_trans=False, C=None, stream=None):
    """C = alpha A B^T + bias (+ R) for 2-D bf16 tensors A [M, K], B [N, K]
    (row pitches from their strides); C [M, N] (or [N, M] with c_trans) of
    out_dtype (bfloat16 or float32). Returns C."""
    import torch
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    M, K = A.shape
    N = B.shape[0]
    if C is None:
        C = torch.empty((N, M) if c_trans else (M, N), dtype=out_dtype, device=A.device)
    return gemm_bf16_strided(M, N, K, 1, 1, A, A.stride(0), 0, 0, B, B.stride(0), 0, 0, C, C.stride(0), 0, 0,
                             alpha=alpha, bias=bias, R=R, ldr=R.stride(0) if R is not None else 0,
                             c_trans=c_trans, stream=stream)


def gemm_bf16_strided(M, N, K, batch1, batch2, A, lda, sA1, sA2, B, ldb, sB1, sB2, C, ldc, sC1, sC2,
                      alpha=1.0, bias=None, stride_bias2=0, R=None, ldr=0, sR1=0, sR2=0, c_trans=False,
                      stream=None):
    """The strided-batched form of mlstm_gemm_bf16: A, B, C, bias, R are
    tensors (their data pointers are the bases; strides count elements)."""
    import torch
    for name, t in (("A", A), ("B", B), ("R", R)):
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
    if bias is not None and bias.dtype != torch.float32:
        raise ValueError("bias must be float32")
    if C.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("C must be bfloat16 or float32")
    args = GemmArgs(M, N, K, batch1, batch2, _ptr(A), lda, sA1, sA2, _ptr(B), ldb, sB1, sB2,
                    _ptr(C), ldc, sC1, sC2, MLSTM_BF16 if C.dtype == torch.bfloat16 else MLSTM_FP32,
                    1 if c_trans else 0, float(alpha), _ptr(bias), stride_bias2, _ptr(R), ldr, sR1, sR2)
    _check(lib().mlstm_gemm_bf16(ctypes.byref(args), _stream(stream)), "mlstm_gemm_bf16")
    return C


def layernorm_bf16(x, w, b, eps, y=None, stream=None):
    """Layer norm of the rows of a bf16 tensor [..., D]; w, b float32 [D]."""
    import torch
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    if y is None:
        y = torch.empty_like(x)
    _require(x, "x", tuple(x.shape), torch.bfloat16)
    _require(y, "y", tuple(x.shape), torch.bfloat16)
    _check(lib().mlstm_layernorm_bf16(_ptr(x), _ptr(w), _ptr(b), _ptr(y), rows, D, float(eps), _stream(stream)),
           "mlstm_layernorm_bf16")
    return y


def block_params(p, D, H, d_qk, d_v, KC=4, eps_ln=1e-5, eps_gn=1e-5) -> BlockParams:
    """mlstm_block_params from a dict of device tensors named as in
    BLOCK_ARRAYS (bfloat16 matrices, float32 vectors; shapes checked)."""
    import torch
    E = 2 * D
    shapes = {"ln_w": (D,), "ln_b": (D,), "W_up": (2 * E, D), "b_up": (2 * E,), "conv_w": (E, KC),
              "conv_b": (E,), "W_q": (H, d_qk, E // H), "W_k": (H, d_qk, E // H), "b_q": (H * d_qk,),
              "b_k": (H * d_qk,), "W_v": (H, d_v, E // H), "b_v": (E,), "w_i": (H, E), "w_f": (H, E),
              "b_i": (H,), "b_f": (H,), "gn_w": (E,), "gn_b": (E,), "skip": (E,), "W_down": (D, E),
              "b_down": (D,)}
    ptrs = []
    for name, is_mat in BLOCK_ARRAYS:
        _require(p[name], name, shapes[name], torch.bfloat16 if is_mat else torch.float32)
        ptrs.append(_ptr(p[name]))
    return BlockParams(D, H, d_qk, d_v, KC, float(eps_ln), float(eps_gn), *ptrs)


def block_workspace_bytes(bp: BlockParams, B: int, T: int, chunk: int) -> int:
    return int(lib().mlstm_block_fwd_workspace_size(ctypes.byref(bp), B, T, int(chunk)))


def mlstm_block_fwd(x, bp: BlockParams, chunk=256, out=None, workspace=None, return_stages=False, stream=None):
    """The whole block on x [B, T, D] (bf16). Returns out, or (out, stages)
    with the intermediates as views of the workspace (names BLOCK_STAGES)."""
    import torch
    B, T, D = x.shape
    _require(x, "x", (B, T, D), torch.bfloat16)
    if out is None:
        out = torch.empty_like(x)
    nbytes = block_workspace_bytes(bp, B, T, chunk)
    ws = _workspace(nbytes, x.device, workspace)
    _check(lib().mlstm_block_fwd(ctypes.byref(bp), B, T, _ptr(x), _ptr(out), int(chunk), _ptr(ws), nbytes,
                                 _stream(stream)), "mlstm_block_fwd")
    if not return_stages:
        return out
    offs = (c_size_t * 10)()
    _check(lib().mlstm_block_workspace_offsets(ctypes.byref(bp), B, T, int(chunk), offs),
           "mlstm_block_workspace_offsets")
    E, H = 2 * D, bp.H
    shapes = {"xn": ((B, T, D), torch.bfloat16), "xup": ((B, T, 2 * E), torch.bfloat16),
              "xc": ((B, T, E), torch.bfloat16), "q": ((B, H, T, bp.d_qk), torch.bfloat16),
              "k": ((B, H, T, bp.d_qk), torch.bfloat16), "v": ((B, H, T, bp.d_v), torch.bfloat16),
              "i_pre": ((B, H, T), torch.float32), "f_pre": ((B, H, T), torch.float32),
              "h": ((B, H, T, bp.d_v), torch.bfloat16), "y": ((B, T, E), torch.bfloat16)}
    stages = {}
    for j, name in enumerate(BLOCK_STAGES):
        shape, dt = shapes[name]
        n = 1
        for d in shape:
            n *= d
        es = 2 if dt == torch.bfloat16 else 4
        stages[name] = ws[offs[j]:offs[j] + n * es].view(dt).view(shape)
    return out, stages


def block_conv_gates(bp: BlockParams, xup, stream=None):
    """The block's conv step from xup [B, T, 2E]: returns xc [B, T, E] (bf16)
    and i_pre, f_pre [B, H, T] (float32)."""
    import torch
    B, T, E2 = xup.shape
    _require(xup, "xup", (B, T, E2), torch.bfloat16)
    xc = torch.empty((B, T, E2 // 2), dtype=torch.bfloat16, device=xup.device)
    ip = torch.empty((B, bp.H, T), dtype=torch.float32, device=xup.device)
    fp = torch.empty_like(ip)
    _check(lib().mlstm_block_conv_gates(ctypes.byref(bp), B, T, _ptr(xup), _ptr(xc), _ptr(ip), _ptr(fp),
                                        _stream(stream)), "mlstm_block_conv_gates")
    return xc, ip, fp


def block_groupnorm_gate(bp: BlockParams, h, xc, xup, stream=None):
    """The block's step after the cell: y [B, T, E] from the cell output h
    [B, H, T, d_v], xc [B, T, E] and xup [B, T, 2E]."""
    import torch
    B, T, E = xc.shape
    _require(h, "h", (B, bp.H, T, bp.d_v), torch.bfloat16)
    _require(xc, "xc", (B, T, E), torch.bfloat16)
    _require(xup, "xup", (B, T, 2 * E), torch.bfloat16)
    y = torch.empty_like(xc)
    _check(lib().mlstm_block_groupnorm_gate(ctypes.byref(bp), B, T, _ptr(h), _ptr(xc), _ptr(xup), _ptr(y),
                                            _stream(stream)), "mlstm_block_groupnorm_gate")
    return y
