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

OK, NULLPTR, BAD_SHAPE, BAD_DTYPE, MISALIGNED, ALIAS, WORKSPACE, UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6, -7

GB = 1 << 30


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlstm_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mlstm_abi_version() == 1


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
        + al(BH * Nc * V * K * 2) + al(BH * Nc * K * 4) + al(BH * Nc * 8)
    assert need == expect
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
        + al(BH * ns * V * K * 4) + al(BH * ns * K * 4) + 3 * al(BH * ns * 8) + al(BH * Nt * 2 * 64 * 2)
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


def test_launch_event_hook_validation():
    lib = L.lib()
    assert lib.mlstm_set_launch_events(9, None, None) == BAD_SHAPE
    assert lib.mlstm_set_launch_events(2, None, None) == OK


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
