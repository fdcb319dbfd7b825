"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects invalid arguments before any HIP call (no GPU needed).

Pointers below are fabricated addresses that are never dereferenced: every
call here fails argument validation, which runs before anything is enqueued.
"""
import ctypes
import os
import re

import pytest

from linear_recurrent_sequence_fwd_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlstm.h")
PROF_HEADER = os.path.join(ROOT, "include", "mlstm_prof.h")

OK, NULLPTR, BAD_SHAPE, BAD_DTYPE, MISALIGNED, ALIAS, WORKSPACE, UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6, -7

GB = 1 << 30


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlstm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mlstm_abi_version() == L.ABI_VERSION == 4
    assert "mlstm_bwd_chunkwise" in names and "mlstm_bwd_chunkwise_workspace_size" in names
    prof = declared_functions(PROF_HEADER)
    assert prof == ["mlstm_clock_probe", "mlstm_prof_bwd_chunkwise", "mlstm_prof_copy_lds",
                    "mlstm_prof_fwd_chunkwise", "mlstm_prof_step"]
    for n in prof:
        assert hasattr(lib, n), n
    # the product header declares only the method's calls and the status/version helpers
    assert not set(prof) & set(names)


def test_status_strings():
    lib = L.lib()
    for code, name in L.STATUS.items():
        assert lib.mlstm_status_string(code).decode() == name
    assert lib.mlstm_status_string(12345).decode() == "MLSTM_ERR_UNKNOWN"


def fake_fwd(B=1, H=2, T=100, K=64, V=128, dtype=L.MLSTM_BF16, state_in=False, state_out=False):
    """Argument struct with distinct, non-overlapping, aligned fake device addresses."""
    es = 2 if dtype == L.MLSTM_BF16 else 4
    base = [0x7F0000000000]

    def take(nbytes):
        p = base[0]
        base[0] += (nbytes + 4095) // 4096 * 4096 + 4096
        return p

    BH = B * H
    a = L.FwdArgs(B, H, T, K, V, dtype,
                  take(BH * T * K * es), take(BH * T * K * es), take(BH * T * V * es),
                  take(BH * T * V * es), take(BH * T * 4), take(BH * T * 4), take(BH * T * V * es),
                  None, None, None, None, None, None)
    if state_in:
        a.C0, a.n0, a.m0 = take(BH * V * K * 4), take(BH * K * 4), take(BH * 4)
    if state_out:
        a.C_out, a.n_out, a.m_out = take(BH * V * K * 4), take(BH * K * 4), take(BH * 4)
    a._next = take
    return a


_AUTO = object()


def chunkwise(a, chunk=64, ws=_AUTO, ws_bytes=None):
    """Call with a fake workspace; every case here must fail validation."""
    lib = L.lib()
    need = lib.mlstm_fwd_chunkwise_workspace_size(ctypes.byref(a), chunk)
    if ws is _AUTO:
        ws = a._next(need) if need else None
    if ws_bytes is None:
        ws_bytes = need
    code = lib.mlstm_fwd_chunkwise(ctypes.byref(a), chunk, ws, ws_bytes, None)
    assert code != OK, "a fabricated-pointer call passed validation"
    return code


def test_null_and_dtype():
    lib = L.lib()
    assert lib.mlstm_fwd_chunkwise(None, 64, None, 0, None) == NULLPTR
    assert lib.mlstm_fwd_parallel(None, None, 0, None) == NULLPTR
    assert lib.mlstm_step(None, None) == NULLPTR
    a = fake_fwd()
    a.dtype = 7
    assert chunkwise(a) == BAD_DTYPE
    a = fake_fwd()
    a.q = None
    assert chunkwise(a) == NULLPTR
    assert "required" in lib.mlstm_last_error().decode()


@pytest.mark.parametrize("field,value,code", [
    ("B", 0, BAD_SHAPE), ("H", -1, BAD_SHAPE), ("T", -5, BAD_SHAPE),
    ("d_v", 96, BAD_SHAPE), ("d_qk", 80, BAD_SHAPE), ("d_qk", 192, UNSUPPORTED),
    ("d_qk", 512, UNSUPPORTED),
])
def test_bad_shapes(field, value, code):
    a = fake_fwd()
    setattr(a, field, value)
    assert chunkwise(a) == code


def test_fp32_dqk256_unsupported_for_forward():
    a = fake_fwd(K=256, dtype=L.MLSTM_FP32)
    assert chunkwise(a) == UNSUPPORTED


@pytest.mark.parametrize("chunk", [0, 32, 100, 8256])
def test_bad_chunk(chunk):
    a = fake_fwd()
    assert L.lib().mlstm_fwd_chunkwise(ctypes.byref(a), chunk, a._next(GB), GB, None) == BAD_SHAPE


def test_half_given_states():
    a = fake_fwd(state_in=True)
    a.n0 = None
    assert chunkwise(a) == NULLPTR
    a = fake_fwd(state_out=True)
    a.m_out = None
    assert chunkwise(a) == NULLPTR


def test_misaligned():
    a = fake_fwd()
    a.v = a.v + 2
    assert chunkwise(a) == MISALIGNED
    a = fake_fwd()
    a.f_pre = a.f_pre + 1
    assert chunkwise(a) == MISALIGNED
    a = fake_fwd()
    need = L.lib().mlstm_fwd_chunkwise_workspace_size(ctypes.byref(a), 64)
    assert chunkwise(a, ws=a._next(need) + 16, ws_bytes=need) == MISALIGNED


def test_aliasing_rejected():
    a = fake_fwd()
    a.h = a.v
    assert chunkwise(a) == ALIAS
    a = fake_fwd(state_in=True, state_out=True)
    a.C_out = a.C0
    assert chunkwise(a) == ALIAS
    a = fake_fwd(state_out=True)
    a.n_out = a.C_out + 64          # inside C_out
    assert chunkwise(a) == ALIAS
    a = fake_fwd()
    assert chunkwise(a, ws=a.q, ws_bytes=GB) == ALIAS


def test_workspace_checks_and_size():
    lib = L.lib()
    a = fake_fwd(B=2, H=3, T=1000, K=128, V=192, dtype=L.MLSTM_BF16)
    need = lib.mlstm_fwd_chunkwise_workspace_size(ctypes.byref(a), 128)
    BH, T, Nc, K, V = 6, 1000, 8, 128, 192
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    expect = 3 * al(BH * T * 8) + 2 * al(BH * T * 4) + 2 * al(BH * Nc * 8) + al(BH * Nc * 4) \
        + al(BH * Nc * V * K * 4) + al(BH * Nc * K * 4) + al(BH * Nc * 8)
    assert need == expect   # float32 chunk-start states for both dtypes
    assert chunkwise(a, chunk=128, ws=None, ws_bytes=need) == WORKSPACE
    assert chunkwise(a, chunk=128, ws=a._next(need), ws_bytes=need - 1) == WORKSPACE
    p = lib.mlstm_fwd_parallel_workspace_size(ctypes.byref(a))
    assert p == 3 * al(BH * T * 8) + 2 * al(BH * T * 4) + 2 * al(BH * 8) + al(BH * 4)
    # fp32 stores float32 chunk states
    b = fake_fwd(B=1, H=1, T=256, K=64, V=64, dtype=L.MLSTM_FP32)
    nb = lib.mlstm_fwd_chunkwise_workspace_size(ctypes.byref(b), 64)
    assert nb == 3 * al(256 * 8) + 2 * al(256 * 4) + 2 * al(4 * 8) + al(4 * 4) + al(4 * 64 * 64 * 4) \
        + al(4 * 64 * 4) + al(4 * 8)


def test_fused_workspace_size():
    """bf16 with d_v a multiple of 128: per-token gate data, per-tile scalars and
    split weights, and one float32 state per chunk boundary."""
    lib = L.lib()
    a = fake_fwd(B=2, H=3, T=1000, K=128, V=256, dtype=L.MLSTM_BF16)
    need = lib.mlstm_fwd_chunkwise_workspace_size(ctypes.byref(a), 256)
    BH, T, K, V = 6, 1000, 128, 256
    Nt = -(-T // 64)
    S = -(-Nt // 4)
    ns = S - 1
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    expect = 3 * al(BH * T * 8) + 2 * al(BH * T * 4) + 2 * al(BH * Nt * 8) + al(BH * Nt * 4) \
        + al(BH * ns * V * K * 4) + al(BH * ns * K * 4) + 3 * al(BH * ns * 8) + al(BH * Nt * 3 * 64 * 2)
    assert need == expect


def test_parallel_limits():
    lib = L.lib()
    a = fake_fwd(T=8193)
    need = lib.mlstm_fwd_parallel_workspace_size(ctypes.byref(a))
    assert lib.mlstm_fwd_parallel(ctypes.byref(a), a._next(need), need, None) == UNSUPPORTED


def test_empty_sequence_without_state_is_a_noop():
    """T = 0 with no state output enqueues nothing and succeeds (no device touched)."""
    lib = L.lib()
    a = fake_fwd(T=0)
    assert lib.mlstm_fwd_chunkwise_workspace_size(ctypes.byref(a), 64) == 0
    assert lib.mlstm_fwd_chunkwise(ctypes.byref(a), 64, None, 0, None) == OK
    assert lib.mlstm_fwd_parallel(ctypes.byref(a), None, 0, None) == OK


def fake_step(B=2, H=2, K=128, V=96, dtype=L.MLSTM_FP32):
    es = 2 if dtype == L.MLSTM_BF16 else 4
    base = [0x7E0000000000]

    def take(nbytes):
        p = base[0]
        base[0] += (nbytes + 4095) // 4096 * 4096 + 4096
        return p

    BH = B * H
    return L.StepArgs(B, H, K, V, dtype, take(BH * K * es), take(BH * K * es), take(BH * V * es),
                      take(BH * V * es), take(BH * 4), take(BH * 4), take(BH * V * K * 4),
                      take(BH * K * 4), take(BH * 4), take(BH * K * 4), take(BH * 4),
                      take(BH * V * es))


def test_step_validation():
    lib = L.lib()
    a = fake_step()
    a.n_out = a.n_in
    assert lib.mlstm_step(ctypes.byref(a), None) == ALIAS
    a = fake_step()
    a.m_out = a.m_in
    assert lib.mlstm_step(ctypes.byref(a), None) == ALIAS
    a = fake_step()
    a.h = a.q
    assert lib.mlstm_step(ctypes.byref(a), None) == ALIAS
    a = fake_step(K=96)
    assert lib.mlstm_step(ctypes.byref(a), None) == BAD_SHAPE
    a = fake_step(K=576)
    assert lib.mlstm_step(ctypes.byref(a), None) == UNSUPPORTED
    a = fake_step()
    a.C = a.C + 4
    assert lib.mlstm_step(ctypes.byref(a), None) == MISALIGNED
    a = fake_step()
    a.dtype = 2
    assert lib.mlstm_step(ctypes.byref(a), None) == BAD_DTYPE
    a = fake_step()
    a.k = None
    assert lib.mlstm_step(ctypes.byref(a), None) == NULLPTR


def test_noalloc_entry_point_limits():
    """The no-allocation call validates like the workspace one and rejects a
    problem whose workspace exceeds its fixed scratch before touching a device."""
    lib = L.lib()
    limit = lib.mlstm_fwd_chunkwise_noalloc_limit()
    assert limit == 64 << 20
    assert lib.mlstm_fwd_chunkwise_noalloc(None, 64, None) == NULLPTR
    a = fake_fwd()
    assert lib.mlstm_fwd_chunkwise_noalloc(ctypes.byref(a), 100, None) == BAD_SHAPE
    big = fake_fwd(B=1, H=8, T=131072, K=256, V=512)
    need = lib.mlstm_fwd_chunkwise_workspace_size(ctypes.byref(big), 64)
    assert need > limit
    assert lib.mlstm_fwd_chunkwise_noalloc(ctypes.byref(big), 64, None) == UNSUPPORTED
    assert b"64 MiB" in lib.mlstm_last_error()


def test_profiling_entry_points_validate_like_the_plain_ones():
    """The measurement calls run the same argument checks before anything is
    enqueued, and the chunkwise one needs its event array."""
    lib = L.lib()
    a = fake_fwd()
    ev = L.event_array([None] * 6)
    assert lib.mlstm_prof_fwd_chunkwise(ctypes.byref(a), 64, None, 0, None, None) == NULLPTR
    a.dtype = 7
    assert lib.mlstm_prof_fwd_chunkwise(ctypes.byref(a), 64, None, 0, None, ev) == BAD_DTYPE
    a = fake_fwd()
    assert lib.mlstm_prof_fwd_chunkwise(ctypes.byref(a), 65, None, 0, None, ev) == BAD_SHAPE
    assert lib.mlstm_prof_fwd_chunkwise(ctypes.byref(a), 64, None, 0, None, ev) == WORKSPACE
    s = fake_step()
    s.k = None
    assert lib.mlstm_prof_step(ctypes.byref(s), None, None, None) == NULLPTR


def test_clock_probe_validation():
    lib = L.lib()
    assert lib.mlstm_clock_probe(None, 100, None) == NULLPTR
    assert lib.mlstm_clock_probe(0x7D0000000000, 0, None) == BAD_SHAPE
    assert lib.mlstm_clock_probe(0x7D0000000000, 1 << 25, None) == BAD_SHAPE
    assert lib.mlstm_clock_probe(0x7D0000000004, 100, None) == MISALIGNED


SLSTM_HEADER = os.path.join(ROOT, "include", "slstm.h")


def test_library_exports_every_slstm_symbol():
    text = re.sub(r"/\*.*?\*/", "", open(SLSTM_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(slstm_[a-z_]+)\s*\(", text)))
    assert names == ["slstm_fwd"]
    for n in names:
        assert hasattr(L.lib(), n), n


def fake_slstm(B=2, H=3, T=10, D=64, state_in=True, state_out=True):
    base = [0x7C0000000000]

    def take(nbytes):
        p = base[0]
        base[0] += (nbytes + 4095) // 4096 * 4096 + 4096
        return p

    BH = B * H
    ns = BH * D * 4
    sin = [take(ns) for _ in range(4)] if state_in else [None] * 4
    sout = [take(ns) for _ in range(4)] if state_out else [None] * 4
    return L.SlstmArgs(B, H, T, D, take(BH * T * 4 * D * 4), take(H * 4 * D * D * 4), take(BH * T * D * 4),
                       *sin, *sout)


def test_slstm_validation():
    lib = L.lib()
    assert lib.slstm_fwd(None, None) == NULLPTR
    for field, value, code in (("B", 0, BAD_SHAPE), ("H", 0, BAD_SHAPE), ("T", -1, BAD_SHAPE),
                               ("D", 0, BAD_SHAPE), ("D", 48, UNSUPPORTED), ("D", 256, UNSUPPORTED)):
        a = fake_slstm()
        setattr(a, field, value)
        assert lib.slstm_fwd(ctypes.byref(a), None) == code, (field, value)
    a = fake_slstm()
    a.n0 = None
    assert lib.slstm_fwd(ctypes.byref(a), None) == NULLPTR
    a = fake_slstm()
    a.h_out = None
    assert lib.slstm_fwd(ctypes.byref(a), None) == NULLPTR
    a = fake_slstm()
    a.R = None
    assert lib.slstm_fwd(ctypes.byref(a), None) == NULLPTR
    a = fake_slstm()
    a.pre = None
    assert lib.slstm_fwd(ctypes.byref(a), None) == NULLPTR
    a = fake_slstm()
    a.h = a.h + 8
    assert lib.slstm_fwd(ctypes.byref(a), None) == MISALIGNED
    a = fake_slstm()
    a.h = a.pre
    assert lib.slstm_fwd(ctypes.byref(a), None) == ALIAS
    a = fake_slstm()
    a.c_out = a.c0
    assert lib.slstm_fwd(ctypes.byref(a), None) == ALIAS
    a = fake_slstm()
    a.m_out = a.n_out
    assert lib.slstm_fwd(ctypes.byref(a), None) == ALIAS


def test_slstm_empty_sequence_without_state_is_a_noop():
    a = fake_slstm(T=0, state_in=False, state_out=False)
    a.pre = None
    a.h = None
    assert L.lib().slstm_fwd(ctypes.byref(a), None) == OK


# ---------------------------------------------------------------- backward pass

def fake_bwd(B=1, H=2, T=100, K=64, V=128, dtype=L.MLSTM_BF16, state_in=False, init_grad=False):
    es = 2 if dtype == L.MLSTM_BF16 else 4
    base = [0x7E0000000000]

    def take(nbytes):
        p = base[0]
        base[0] += (nbytes + 4095) // 4096 * 4096 + 4096
        return p

    BH = B * H
    nqk, nv, ng = BH * T * K * es, BH * T * V * es, BH * T * 4
    a = L.BwdArgs(B, H, T, K, V, dtype, take(nqk), take(nqk), take(nv), take(nv), take(ng), take(ng),
                  take(nv), take(nv), None, None, None,
                  take(nqk), take(nqk), take(nv), take(nv), take(ng), take(ng), None, None, None)
    if state_in:
        a.C0, a.n0, a.m0 = take(BH * V * K * 4), take(BH * K * 4), take(BH * 4)
    if init_grad:
        a.dC0, a.dn0, a.dm0 = take(BH * V * K * 4), take(BH * K * 4), take(BH * 4)
    a._next = take
    return a


def backward(a, chunk=64, ws=_AUTO, ws_bytes=None):
    lib = L.lib()
    need = lib.mlstm_bwd_chunkwise_workspace_size(ctypes.byref(a), chunk)
    if ws is _AUTO:
        ws = a._next(need) if need else None
    if ws_bytes is None:
        ws_bytes = need
    code = lib.mlstm_bwd_chunkwise(ctypes.byref(a), chunk, ws, ws_bytes, None)
    assert code != OK, "a fabricated-pointer call passed validation"
    return code


def test_backward_validation():
    lib = L.lib()
    assert lib.mlstm_bwd_chunkwise(None, 64, None, 0, None) == NULLPTR
    a = fake_bwd(); a.dtype = 5
    assert backward(a) == BAD_DTYPE
    a = fake_bwd(); a.dh = None
    assert backward(a) == NULLPTR
    a = fake_bwd(); a.df_pre = None
    assert backward(a) == NULLPTR
    for chunk in (0, 32, 100, 8256):
        assert backward(fake_bwd(), chunk=chunk) == BAD_SHAPE
    a = fake_bwd(K=96)
    assert backward(a) == BAD_SHAPE
    # shapes the backward does not implement
    assert backward(fake_bwd(K=256, V=1024)) == UNSUPPORTED
    assert backward(fake_bwd(K=256, V=128, dtype=L.MLSTM_FP32)) == UNSUPPORTED
    assert backward(fake_bwd(K=128, V=512, dtype=L.MLSTM_FP32)) == UNSUPPORTED
    a = fake_bwd(state_in=True); a.m0 = None
    assert backward(a) == NULLPTR
    a = fake_bwd(init_grad=True); a.dn0 = None
    assert backward(a) == NULLPTR
    a = fake_bwd(); a.dq = a.q
    assert backward(a) == ALIAS
    a = fake_bwd(); a.dv = a.dk
    assert backward(a) == ALIAS
    a = fake_bwd(); a.dq += 2
    assert backward(a) == MISALIGNED
    a = fake_bwd()
    assert backward(a, ws=None) == WORKSPACE
    a = fake_bwd()
    need = lib.mlstm_bwd_chunkwise_workspace_size(ctypes.byref(a), 64)
    assert backward(a, ws_bytes=need - 1) == WORKSPACE
    a = fake_bwd()
    assert backward(a, ws=a.q) == ALIAS
    # profiling variant: same checks, plus the event array
    a = fake_bwd(); a.dh = None
    ev = (ctypes.c_void_p * 12)()
    assert lib.mlstm_prof_bwd_chunkwise(ctypes.byref(a), 64, None, 0, None, ev) == NULLPTR
    assert lib.mlstm_prof_bwd_chunkwise(ctypes.byref(fake_bwd()), 64, None, 0, None, None) == NULLPTR


def test_backward_workspace_size():
    lib = L.lib()
    a = fake_bwd(B=1, H=8, T=8192, K=256, V=512)
    BH, T, K, V, es = 8, 8192, 256, 512, 2
    for chunk in (64, 256, 1024):
        Nc = -(-T // chunk)
        need = lib.mlstm_bwd_chunkwise_workspace_size(ctypes.byref(a), chunk)
        # gate data, forward chunk states, g per token, dz and q.dq, the end adjoints
        # (the forward chunk states in the input dtype, the adjoints float32)
        floor = (BH * T * (8 * 3 + 4 * 2) + BH * Nc * (8 * 2 + 4) + BH * Nc * (V * K * es + K * 4 + 8)
                 + BH * T * V * es + BH * T * 8 + BH * Nc * (V * K * 4 + K * 4 + 8) + BH * (V * K + K) * 4)
        assert floor <= need <= floor + 64 * 256
    a.T = 0
    assert lib.mlstm_bwd_chunkwise_workspace_size(ctypes.byref(a), 64) == 0


def test_backward_empty_sequence_without_init_grad_is_a_noop():
    lib = L.lib()
    a = fake_bwd(T=0)
    assert lib.mlstm_bwd_chunkwise(ctypes.byref(a), 64, None, 0, None) == OK


def test_lds_copy_validation():
    lib = L.lib()
    A, B = 0x7D0000000000, 0x7D0010000000
    assert lib.mlstm_prof_copy_lds(None, B, 16384, None) == NULLPTR
    assert lib.mlstm_prof_copy_lds(A, B, 0, None) == BAD_SHAPE
    assert lib.mlstm_prof_copy_lds(A, B, 16384 + 16, None) == BAD_SHAPE
    assert lib.mlstm_prof_copy_lds(A + 4, B, 16384, None) == MISALIGNED
    assert lib.mlstm_prof_copy_lds(A, A + 16384, 32768, None) == ALIAS


BLOCK_HEADER = os.path.join(ROOT, "include", "mlstm_block.h")


def test_library_exports_every_block_symbol():
    lib = L.lib()
    names = declared_functions(BLOCK_HEADER)
    assert names == ["mlstm_block_conv_gates", "mlstm_block_fwd", "mlstm_block_fwd_workspace_size",
                     "mlstm_block_groupnorm_gate", "mlstm_block_workspace_offsets", "mlstm_gemm_bf16",
                     "mlstm_layernorm_bf16"]
    for n in names:
        assert hasattr(lib, n), n


def fake_block(D=256, H=4, dqk=64, dv=128, KC=4):
    base = [0x7E0000000000]

    def take(nbytes):
        p = base[0]
        base[0] += (nbytes + 4095) // 4096 * 4096 + 4096
        return p

    E = 2 * D
    sizes = {"ln_w": D * 4, "ln_b": D * 4, "W_up": 2 * E * D * 2, "b_up": 2 * E * 4, "conv_w": E * KC * 4,
             "conv_b": E * 4, "W_q": H * dqk * (E // H) * 2, "W_k": H * dqk * (E // H) * 2, "b_q": H * dqk * 4,
             "b_k": H * dqk * 4, "W_v": H * dv * (E // H) * 2, "b_v": E * 4, "w_i": H * E * 2, "w_f": H * E * 2,
             "b_i": H * 4, "b_f": H * 4, "gn_w": E * 4, "gn_b": E * 4, "skip": E * 4, "W_down": D * E * 2,
             "b_down": D * 4}
    p = L.BlockParams(D, H, dqk, dv, KC, 1e-5, 1e-5, *[take(sizes[n]) for n, _ in L.BLOCK_ARRAYS])
    return p, take


@pytest.mark.parametrize("field,value,code", [
    ("D", 100, BAD_SHAPE), ("D", 0, BAD_SHAPE), ("d_v", 64, BAD_SHAPE), ("H", 0, BAD_SHAPE),
    ("d_qk", 96, UNSUPPORTED), ("KC", 0, UNSUPPORTED), ("KC", 5, UNSUPPORTED), ("eps_gn", -1.0, BAD_SHAPE),
])
def test_block_validation(field, value, code):
    lib = L.lib()
    p, take = fake_block()
    B, T = 2, 100
    need = lib.mlstm_block_fwd_workspace_size(ctypes.byref(p), B, T, 64)
    assert need > 0
    x, out, ws = take(B * T * 256 * 2), take(B * T * 256 * 2), take(need)
    setattr(p, field, value)
    assert lib.mlstm_block_fwd(ctypes.byref(p), B, T, x, out, 64, ws, need, None) == code


def test_block_pointer_and_workspace_checks():
    lib = L.lib()
    p, take = fake_block()
    B, T = 1, 70
    need = lib.mlstm_block_fwd_workspace_size(ctypes.byref(p), B, T, 64)
    x, out, ws = take(B * T * 256 * 2), take(B * T * 256 * 2), take(need)
    assert lib.mlstm_block_fwd(None, B, T, x, out, 64, ws, need, None) == NULLPTR
    assert lib.mlstm_block_fwd(ctypes.byref(p), B, T, None, out, 64, ws, need, None) == NULLPTR
    assert lib.mlstm_block_fwd(ctypes.byref(p), B, T, x, out, 64, ws, need - 256, None) == WORKSPACE
    assert lib.mlstm_block_fwd(ctypes.byref(p), B, T, x, out, 64, ws + 16, need, None) == MISALIGNED
    assert lib.mlstm_block_fwd(ctypes.byref(p), B, T, x, x, 64, ws, need, None) == ALIAS
    assert lib.mlstm_block_fwd(ctypes.byref(p), B, T, x, out, 96, ws, need, None) == BAD_SHAPE
    assert lib.mlstm_block_fwd(ctypes.byref(p), B, 0, x, out, 64, None, 0, None) == OK   # empty: nothing to do
    p.W_q = None
    assert lib.mlstm_block_fwd(ctypes.byref(p), B, T, x, out, 64, ws, need, None) == NULLPTR
    assert lib.mlstm_block_fwd_workspace_size(None, B, T, 64) == 0
    offs = (ctypes.c_size_t * 10)()
    assert lib.mlstm_block_workspace_offsets(ctypes.byref(p), B, 0, 64, offs) == BAD_SHAPE
    # batch entries index the group norm's grid in its third dimension (at most 65535)
    h, xc, xup, y = take(8), take(8), take(8), take(8)
    assert lib.mlstm_block_groupnorm_gate(ctypes.byref(p), 65536, 1, h, xc, xup, y, None) == UNSUPPORTED


def test_gemm_and_layernorm_validation():
    lib = L.lib()
    _, take = fake_block()
    A, Bm, C = take(300 * 128 * 2), take(96 * 128 * 2), take(300 * 96 * 2)
    g = L.GemmArgs(300, 96, 128, 1, 1, A, 128, 0, 0, Bm, 128, 0, 0, C, 96, 0, 0, L.MLSTM_BF16, 0, 1.0,
                   None, 0, None, 0, 0, 0)
    bad = [("K", 96, BAD_SHAPE), ("N", 98, BAD_SHAPE), ("M", 0, BAD_SHAPE), ("c_dtype", 3, BAD_DTYPE),
           ("lda", (1 << 21) + 8, UNSUPPORTED),
           ("ldb", 120, BAD_SHAPE), ("ldc", 100, MISALIGNED), ("A", None, NULLPTR), ("C", A + 256, ALIAS)]
    for field, value, code in bad:
        h = L.GemmArgs.from_buffer_copy(g)
        setattr(h, field, value)
        assert lib.mlstm_gemm_bf16(ctypes.byref(h), None) == code, field
    assert lib.mlstm_gemm_bf16(None, None) == NULLPTR
    x, w, b, y = take(10 * 256 * 2), take(256 * 4), take(256 * 4), take(10 * 256 * 2)
    assert lib.mlstm_layernorm_bf16(x, w, b, y, 10, 250, 1e-5, None) == BAD_SHAPE
    assert lib.mlstm_layernorm_bf16(x, w, b, y, 10, 16384, 1e-5, None) == UNSUPPORTED
    assert lib.mlstm_layernorm_bf16(x, w, b, x, 10, 256, 1e-5, None) == ALIAS
    assert lib.mlstm_layernorm_bf16(None, w, b, y, 10, 256, 1e-5, None) == NULLPTR
    assert lib.mlstm_layernorm_bf16(x, w, b, y, 0, 256, 1e-5, None) == OK   # no rows: nothing to do


def test_ungated_cell_only_on_the_fused_chunkwise_path():
    lib = L.lib()
    a = fake_fwd(dtype=L.MLSTM_FP32)
    a.o_pre = None
    assert chunkwise(a) == NULLPTR
    a = fake_fwd(V=64)        # bf16 but d_v not a multiple of 128: not the fused kernels
    a.o_pre = None
    assert chunkwise(a) == NULLPTR
    a = fake_fwd()
    a.o_pre = None
    need = lib.mlstm_fwd_parallel_workspace_size(ctypes.byref(a))
    assert lib.mlstm_fwd_parallel(ctypes.byref(a), a._next(need), need, None) == NULLPTR


SEGMENTS_HEADER = os.path.join(ROOT, "include", "mlstm_segments.h")


def test_library_exports_every_segment_symbol():
    lib = L.lib()
    names = declared_functions(SEGMENTS_HEADER)
    assert names == ["mlstm_segment_summary", "mlstm_segment_summary_workspace_size", "mlstm_state_combine"]
    for n in names:
        assert hasattr(lib, n), n


def _fake_addresses(start):
    base = [start]

    def take(nbytes):
        p = base[0]
        base[0] += (nbytes + 4095) // 4096 * 4096 + 4096
        return p
    return take


def test_segment_summary_validation():
    lib = L.lib()
    take = _fake_addresses(0x7D0000000000)
    B, H, T, K, V = 1, 2, 512, 128, 256
    BH = B * H
    a = L.SummaryArgs(B, H, T, K, V, L.MLSTM_BF16, take(BH * T * K * 2), take(BH * T * V * 2),
                      take(BH * T * 4), take(BH * T * 4), take(BH * V * K * 4), take(BH * K * 4),
                      take(BH * 4), take(BH * 8))
    need = lib.mlstm_segment_summary_workspace_size(ctypes.byref(a), 128)
    # the forward's fused layout with a local state for every chunk (4 here, not 3)
    fwd = L.FwdArgs(B, H, T, K, V, L.MLSTM_BF16, *([0x1000] * 13))
    assert need > L.chunkwise_workspace_bytes(fwd, 128)
    ws = take(need)

    def call(args, chunk=128, w=ws, nb=need):
        return lib.mlstm_segment_summary(ctypes.byref(args), chunk, w, nb, None)

    assert call(a, nb=need - 1) == WORKSPACE
    assert call(a, w=None) == WORKSPACE
    assert call(a, w=ws + 128) == MISALIGNED
    assert call(a, chunk=192) == BAD_SHAPE           # 512 is not a multiple of 192
    assert lib.mlstm_segment_summary_workspace_size(ctypes.byref(a), 192) == 0
    assert call(a, chunk=100) == BAD_SHAPE
    assert call(a, chunk=16384) == BAD_SHAPE
    bad = [("dtype", L.MLSTM_FP32, UNSUPPORTED), ("dtype", 7, BAD_DTYPE), ("d_v", 192, UNSUPPORTED),
           ("d_qk", 96, UNSUPPORTED), ("H", 0, BAD_SHAPE), ("T", -64, BAD_SHAPE),
           ("G_out", None, NULLPTR), ("k", None, NULLPTR), ("G_out", a.G_out + 4, MISALIGNED),
           ("C_out", a.C_out + 8, MISALIGNED), ("n_out", a.C_out, ALIAS), ("C_out", a.k, ALIAS)]
    for field, value, code in bad:
        b = L.SummaryArgs.from_buffer_copy(a)
        setattr(b, field, value)
        assert call(b) == code, field
    assert call(a, w=a.v) == ALIAS                    # workspace over an input
    assert lib.mlstm_segment_summary(None, 128, ws, need, None) == NULLPTR
    e = L.SummaryArgs.from_buffer_copy(a)
    e.T = 0
    assert lib.mlstm_segment_summary_workspace_size(ctypes.byref(e), 128) == 0


def test_state_combine_validation():
    lib = L.lib()
    take = _fake_addresses(0x7C8000000000)
    B, H, K, V = 2, 3, 64, 128
    BH = B * H
    P = 3
    c = L.CombineArgs(B, H, K, V, P, take(BH * V * K * 4), take(BH * K * 4), take(BH * 4),
                      take(P * BH * V * K * 4), take(P * BH * K * 4), take(P * BH * 4), take(P * BH * 8),
                      take(BH * V * K * 4), take(BH * K * 4), take(BH * 4))
    bad = [("m0", None, NULLPTR), ("Gs", None, NULLPTR), ("C_out", None, NULLPTR),
           ("Gs", c.Gs + 4, MISALIGNED), ("ms", c.ms + 2, MISALIGNED), ("Cs", c.Cs + 4, MISALIGNED),
           ("n_out", c.n_out + 8, MISALIGNED), ("d_v", 0, BAD_SHAPE), ("d_qk", 66, BAD_SHAPE),
           ("count", -1, BAD_SHAPE), ("B", -1, BAD_SHAPE), ("C_out", c.C0, ALIAS),
           ("C_out", c.Cs + 64, ALIAS), ("m_out", c.n_out, ALIAS), ("n_out", c.Gs, ALIAS),
           # the third summary of the stack lies over C_out
           ("C_out", c.Cs + 2 * BH * V * K * 4, ALIAS)]
    for field, value, code in bad:
        d = L.CombineArgs.from_buffer_copy(c)
        setattr(d, field, value)
        assert lib.mlstm_state_combine(ctypes.byref(d), None) == code, field
    d = L.CombineArgs.from_buffer_copy(c)
    d.C0 = None                                       # n0, m0 still given: all three or none
    assert lib.mlstm_state_combine(ctypes.byref(d), None) == NULLPTR
    d = L.CombineArgs.from_buffer_copy(c)
    d.count, d.Cs, d.ns = 1, None, None               # summaries are required when count > 0
    assert lib.mlstm_state_combine(ctypes.byref(d), None) == NULLPTR
    assert lib.mlstm_state_combine(None, None) == NULLPTR
