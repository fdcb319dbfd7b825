"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bar: max|h_gpu - h_ref| <= tol * max|h_ref| with tol = 1e-4 for float32
inputs and 2e-2 for bfloat16 inputs; every output finite. States are
compared in true units (exp(m) C~), relative to the oracle's largest entry.
Outputs are pre-filled with NaN so that an unwritten element fails.
"""
import ctypes
import sys

import numpy as np
import pytest

from linear_recurrent_sequence_fwd_amd.configs import CONFIGS
from linear_recurrent_sequence_fwd_amd.inputs import make_fwd_inputs, make_state, make_step_inputs
from oracle import mlstm_oracle as orc
from oracle.mlstm_ref import mlstm_recurrent_c, mlstm_step_c

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}
NAMES = ("q", "k", "v", "i_pre", "f_pre", "o_pre")


def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_recurrent_sequence_fwd_amd as M
    return M


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def dev_inputs(x):
    d = x["dtype"]
    return {"q": dev(x["q"], d), "k": dev(x["k"], d), "v": dev(x["v"], d),
            "o_pre": dev(x["o_pre"], d), "i_pre": dev(x["i_pre"], "fp32"),
            "f_pre": dev(x["f_pre"], "fp32")}


def nan_like(t):
    return torch.full_like(t, float("nan"))


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def state_err(gpu_state, ref_state):
    C, n, m = (host(t) for t in gpu_state)
    Cr, nr, mr = ref_state
    sc = np.exp(m - mr)
    return (rel_err(sc[..., None, None] * C, Cr), rel_err(sc[..., None] * n, nr))


def oracle(x, **state):
    return orc.mlstm_recurrent(*[x[n] for n in NAMES], **state)


def run_chunkwise(M, d, chunk, **kw):
    h = nan_like(d["v"])
    out = M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"],
                                chunk=chunk, h=h, **kw)
    torch.cuda.synchronize()
    return out


def run_parallel(M, d, **kw):
    h = nan_like(d["v"])
    out = M.mlstm_fwd_parallel(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], h=h, **kw)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------ decode step

def test_step_tiny_fp32_matches_recurrence():
    M = _lib()
    cfg = CONFIGS["tiny"]
    x = make_fwd_inputs(1, 1, cfg["T"], cfg["d_qk"], cfg["d_v"], "fp32", seed=0)
    say("step tiny fp32, 256 steps")
    h_ref, st_ref = oracle(x)
    d = dev_inputs(x)
    C = torch.zeros((1, 1, 64, 64), device="cuda")
    n = torch.zeros((1, 1, 64), device="cuda")
    m = torch.zeros((1, 1), device="cuda")
    n2, m2 = torch.empty_like(n), torch.empty_like(m)
    hs = []
    for t in range(cfg["T"]):
        h = torch.full((1, 1, 64), float("nan"), device="cuda")
        M.mlstm_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                     d["v"][:, :, t].contiguous(), d["o_pre"][:, :, t].contiguous(),
                     d["i_pre"][:, :, t].contiguous(), d["f_pre"][:, :, t].contiguous(),
                     C, n, m, n2, m2, h)
        hs.append(h)
        n, n2, m, m2 = n2, n, m2, m
    torch.cuda.synchronize()
    h = np.stack([host(t) for t in hs], axis=2)
    assert rel_err(h, h_ref) <= TOL["fp32"]
    ec, en = state_err((C, n, m), st_ref)
    assert ec <= TOL["fp32"] and en <= TOL["fp32"]


@pytest.mark.parametrize("dtype,K,V", [("bf16", 128, 96), ("fp32", 192, 40), ("bf16", 512, 64)])
def test_step_from_random_state(dtype, K, V):
    M = _lib()
    B, H, steps = 2, 3, 12
    say(f"step {dtype} K={K} V={V}")
    st = make_state(B, H, K, V, seed=4, m_scale=2.0)
    C = torch.from_numpy(st["C"]).cuda()
    n = torch.from_numpy(st["n"]).cuda()
    m = torch.from_numpy(st["m"]).cuda()
    Cr, nr, mr = (st[a].astype(np.float64) for a in ("C", "n", "m"))
    n2, m2 = torch.empty_like(n), torch.empty_like(m)
    for s in range(steps):
        x = make_step_inputs(B, H, K, V, step=s, dtype=dtype, seed=5)
        if s == 3:
            x["f_pre"][0, 1] = -np.inf     # complete forgetting in one head
            x["i_pre"][1, 2] = 40.0        # a strong write
        h_ref, Cr, nr, mr = orc.mlstm_step(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"],
                                           x["o_pre"], Cr, nr, mr)
        d = {a: dev(x[a], dtype if a in ("q", "k", "v", "o_pre") else "fp32") for a in NAMES}
        h = torch.full((B, H, V), float("nan"), device="cuda",
                       dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
        M.mlstm_step(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], C, n, m, n2, m2, h)
        torch.cuda.synchronize()
        assert rel_err(host(h), h_ref) <= TOL[dtype], f"step {s}"
        n, n2, m, m2 = n2, n, m2, m
    ec, en = state_err((C, n, m), (Cr, nr, mr))
    assert ec <= 1e-4 and en <= 1e-4


# ------------------------------------------------------------------ small forwards

@pytest.mark.parametrize("T,chunk", [(256, 64), (256, 128), (200, 64), (130, 192), (1, 64), (64, 64)])
def test_chunkwise_tiny_fp32(T, chunk):
    M = _lib()
    say(f"chunkwise fp32 T={T} chunk={chunk}")
    x = make_fwd_inputs(1, 1, T, 64, 64, "fp32", seed=0)
    h_ref, st_ref = oracle(x)
    h, st = run_chunkwise(M, dev_inputs(x), chunk, return_state=True)
    assert rel_err(host(h), h_ref) <= TOL["fp32"]
    ec, en = state_err(st, st_ref)
    assert ec <= TOL["fp32"] and en <= TOL["fp32"]


@pytest.mark.parametrize("T", [256, 1, 77])
def test_parallel_tiny_fp32(T):
    M = _lib()
    say(f"parallel fp32 T={T}")
    x = make_fwd_inputs(1, 1, T, 64, 64, "fp32", seed=0)
    h_ref, st_ref = oracle(x)
    h, st = run_parallel(M, dev_inputs(x), return_state=True)
    assert rel_err(host(h), h_ref) <= TOL["fp32"]
    ec, en = state_err(st, st_ref)
    assert ec <= TOL["fp32"] and en <= TOL["fp32"]


@pytest.mark.parametrize("dtype,K,V,T,chunk", [
    ("bf16", 128, 192, 333, 64), ("bf16", 128, 192, 333, 128), ("bf16", 64, 128, 500, 256),
    ("bf16", 256, 512, 300, 128), ("fp32", 128, 128, 321, 64), ("fp32", 64, 192, 150, 128),
])
def test_chunkwise_with_initial_state(dtype, K, V, T, chunk):
    M = _lib()
    B, H = 2, 2
    say(f"chunkwise {dtype} K={K} V={V} T={T} chunk={chunk} with state")
    x = make_fwd_inputs(B, H, T, K, V, dtype, seed=1, i_std=2.0)
    st = make_state(B, H, K, V, seed=2)
    h_ref, st_ref = oracle(x, C0=st["C"], n0=st["n"], m0=st["m"])
    d = dev_inputs(x)
    h, sto = run_chunkwise(M, d, chunk, C0=torch.from_numpy(st["C"]).cuda(),
                           n0=torch.from_numpy(st["n"]).cuda(), m0=torch.from_numpy(st["m"]).cuda(),
                           return_state=True)
    assert rel_err(host(h), h_ref) <= TOL[dtype]
    ec, en = state_err(sto, st_ref)
    assert ec <= TOL[dtype] and en <= TOL[dtype]


@pytest.mark.parametrize("dtype,K,V,T", [("bf16", 128, 192, 333), ("fp32", 64, 64, 256),
                                         ("bf16", 256, 512, 200)])
def test_parallel_with_initial_state(dtype, K, V, T):
    M = _lib()
    B, H = 2, 2
    say(f"parallel {dtype} K={K} V={V} T={T} with state")
    x = make_fwd_inputs(B, H, T, K, V, dtype, seed=3, i_std=2.0)
    st = make_state(B, H, K, V, seed=4)
    h_ref, st_ref = oracle(x, C0=st["C"], n0=st["n"], m0=st["m"])
    h, sto = run_parallel(M, dev_inputs(x), C0=torch.from_numpy(st["C"]).cuda(),
                          n0=torch.from_numpy(st["n"]).cuda(), m0=torch.from_numpy(st["m"]).cuda(),
                          return_state=True)
    assert rel_err(host(h), h_ref) <= TOL[dtype]
    ec, en = state_err(sto, st_ref)
    assert ec <= TOL[dtype] and en <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_extreme_preactivations(dtype):
    M = _lib()
    say(f"extreme preactivations {dtype}")
    rng = np.random.default_rng(7)
    B, H, T, K, V = 1, 2, 300, 64, 64
    x = make_fwd_inputs(B, H, T, K, V, dtype, seed=8)
    x["i_pre"] = rng.choice([-100.0, 100.0, 0.0, 2.0, -3.0], size=(B, H, T)).astype(np.float32)
    x["f_pre"] = rng.choice([-100.0, 100.0, np.inf, -np.inf, 3.0, 3.0, 3.0],
                            size=(B, H, T)).astype(np.float32)
    h_ref, _ = oracle(x)
    d = dev_inputs(x)
    for chunk in (64, 128):
        h = run_chunkwise(M, d, chunk)
        assert rel_err(host(h), h_ref) <= TOL[dtype], f"chunk {chunk}"
    h = run_parallel(M, d)
    assert rel_err(host(h), h_ref) <= TOL[dtype], "parallel"


@pytest.mark.parametrize("K,V,T", [(128, 256, 700), (256, 128, 330)])
def test_extreme_preactivations_fused(K, V, T):
    """bf16 with d_v a multiple of 128 (the fused path): zero and saturated
    forget gates, input gates jumping by 200, so that tiles reset, deferred
    decays cross the deferral limit (accumulator rescales in the output pass
    and the step-by-step fallback of the chunk-local scan), over several
    chunks and a ragged last tile."""
    M = _lib()
    say(f"extreme preactivations fused K={K} V={V} T={T}")
    rng = np.random.default_rng(11)
    B, H = 1, 2
    x = make_fwd_inputs(B, H, T, K, V, "bf16", seed=12)
    x["i_pre"] = rng.choice([-100.0, 100.0, 0.0, 2.0, -3.0], size=(B, H, T)).astype(np.float32)
    x["f_pre"] = rng.choice([-100.0, 100.0, np.inf, -np.inf, 3.0, 3.0, 3.0],
                            size=(B, H, T)).astype(np.float32)
    h_ref, st_ref = oracle(x)
    d = dev_inputs(x)
    for chunk in (64, 128, 192):
        h, st = run_chunkwise(M, d, chunk, return_state=True)
        assert bool(torch.isfinite(h.float()).all()), f"chunk {chunk}"
        assert rel_err(host(h), h_ref) <= TOL["bf16"], f"chunk {chunk}"
        ec, en = state_err(st, st_ref)
        assert ec <= TOL["bf16"] and en <= TOL["bf16"], f"chunk {chunk}"


@pytest.mark.parametrize("K,V", [(64, 128), (128, 256), (256, 128)])
@pytest.mark.parametrize("chunk", [64, 512, 1024])
def test_extreme_preactivations_fused_with_state(K, V, chunk):
    """The fused path from a given initial state under resetting and
    saturating gates, for each d_qk the fused kernels are built for: at
    chunk 64 the fold kernel writes the chunk start states (62 local
    states), at 512 (seven, the most, of eight tiles each) and 1024 (three)
    each output workgroup folds its own start state from the local states
    and the initial state."""
    M = _lib()
    T = 4000
    say(f"extreme preactivations fused K={K} V={V} T={T} chunk={chunk} with state")
    rng = np.random.default_rng(21)
    B, H = 1, 2
    x = make_fwd_inputs(B, H, T, K, V, "bf16", seed=22)
    x["i_pre"] = rng.choice([-100.0, 100.0, 0.0, 2.0, -3.0], size=(B, H, T)).astype(np.float32)
    x["f_pre"] = rng.choice([-100.0, 100.0, np.inf, -np.inf, 3.0, 3.0, 3.0],
                            size=(B, H, T)).astype(np.float32)
    st = make_state(B, H, K, V, seed=23)
    h_ref, st_ref = oracle(x, C0=st["C"], n0=st["n"], m0=st["m"])
    d = dev_inputs(x)
    h, sto = run_chunkwise(M, d, chunk, C0=torch.from_numpy(st["C"]).cuda(),
                           n0=torch.from_numpy(st["n"]).cuda(), m0=torch.from_numpy(st["m"]).cuda(),
                           return_state=True)
    assert bool(torch.isfinite(h.float()).all())
    assert rel_err(host(h), h_ref) <= TOL["bf16"]
    ec, en = state_err(sto, st_ref)
    assert ec <= TOL["bf16"] and en <= TOL["bf16"]


def test_empty_sequence_copies_state():
    M = _lib()
    say("T=0")
    st = make_state(1, 2, 64, 64, seed=9)
    x = make_fwd_inputs(1, 2, 0, 64, 64, "fp32", seed=9)
    d = dev_inputs(x)
    C0, n0, m0 = (torch.from_numpy(st[a]).cuda() for a in ("C", "n", "m"))
    for fn in (run_chunkwise, run_parallel):
        kw = {"chunk": 64} if fn is run_chunkwise else {}
        h, (C, n, m) = fn(M, d, C0=C0, n0=n0, m0=m0, return_state=True, **kw)
        assert h.numel() == 0
        assert torch.equal(C, C0) and torch.equal(n, n0) and torch.equal(m, m0)


def test_run_twice_bitwise_identical():
    M = _lib()
    say("determinism")
    x = make_fwd_inputs(2, 4, 700, 128, 256, "bf16", seed=10)
    d = dev_inputs(x)
    a = run_chunkwise(M, d, 128)
    b = run_chunkwise(M, d, 128)
    assert torch.equal(a, b)


# ------------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("entry", ["chunkwise", "parallel"])
def test_config_tiny(entry):
    M = _lib()
    cfg = CONFIGS["tiny"]
    say(f"config tiny {entry}")
    x = make_fwd_inputs(cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], "fp32", seed=0)
    h_ref, _ = oracle(x)
    d = dev_inputs(x)
    h = run_chunkwise(M, d, 64) if entry == "chunkwise" else run_parallel(M, d)
    assert rel_err(host(h), h_ref) <= TOL["fp32"]


_MID = {}


@pytest.mark.parametrize("chunk", [64, 256, 1024])
@pytest.mark.parametrize("seed,i_std", [(0, 1.0), (1, 6.0), (11, 6.0)])
def test_config_mid(seed, i_std, chunk):
    """The mid workload and its stress seeds (input-gate preactivations of
    standard deviation 6, which make single keys dominate the state) at
    several chunk lengths, whole output and final state."""
    M = _lib()
    cfg = CONFIGS["mid"]
    say(f"config mid seed={seed} i_std={i_std} chunk={chunk}")
    x = make_fwd_inputs(cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], "bf16", seed=seed,
                        i_std=i_std)
    if (seed, i_std) not in _MID:
        _MID[(seed, i_std)] = mlstm_recurrent_c(*[x[n] for n in NAMES])
    h_ref, st_ref = _MID[(seed, i_std)]
    d = dev_inputs(x)
    h, st = run_chunkwise(M, d, chunk, return_state=True)
    err = rel_err(host(h), h_ref)
    say(f"  h err {err:.2e}")
    assert err <= TOL["bf16"]
    ec, en = state_err(st, st_ref)
    assert ec <= TOL["bf16"] and en <= TOL["bf16"]
    if chunk == 64:
        hp = run_parallel(M, d)
        assert rel_err(host(hp), h_ref) <= TOL["bf16"]


# Full-size references are computed once per session by the C float64 oracle
# (the same step recurrence as mlstm_oracle, one sequence per host thread).
_REF = {}


def _full_reference(name):
    if name not in _REF:
        cfg = CONFIGS[name]
        x = make_fwd_inputs(cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], "bf16", seed=0)
        say(f"oracle {name}: full float64 recurrence")
        h_ref, st_ref = mlstm_recurrent_c(*[x[n] for n in NAMES])
        _REF[name] = (x, h_ref, st_ref)
    return _REF[name]


def _max_rel_err_by_head(h, h_ref):
    """max|h - h_ref| / max|h_ref| over the whole output, one head at a time
    (keeps the host copies of a long sequence small); also checks finiteness."""
    num, den = 0.0, 0.0
    for b in range(h.shape[0]):
        for hd in range(h.shape[1]):
            got = host(h[b, hd])
            assert np.all(np.isfinite(got)), f"non-finite output in head ({b}, {hd})"
            num = max(num, float(np.max(np.abs(got - h_ref[b, hd]))))
            den = max(den, float(np.max(np.abs(h_ref[b, hd]))))
    return num / den


# chunk lengths of the timed configuration and the sweep around it
BENCH_CHUNKS = [64, 256, 512, 1024, 2048]


@pytest.mark.parametrize("chunk", BENCH_CHUNKS)
def test_config_7b_layer(chunk):
    """The 7B-layer workload in the launch configurations the benchmark times:
    every element of h and the final state against the float64 recurrence."""
    M = _lib()
    x, h_ref, st_ref = _full_reference("7b_layer")
    say(f"config 7b_layer chunk={chunk}")
    d = dev_inputs(x)
    h, st = run_chunkwise(M, d, chunk, return_state=True)
    assert bool(torch.isfinite(h.float()).all())
    err = _max_rel_err_by_head(h, h_ref)
    say(f"7b_layer chunk={chunk}: max rel err {err:.3e}")
    assert err <= TOL["bf16"]
    ec, en = state_err(st, st_ref)
    assert ec <= TOL["bf16"] and en <= TOL["bf16"]


@pytest.mark.parametrize("chunk", [64, 256, 1024])
def test_config_long_context(chunk):
    """T = 131072: every element of h of all eight heads, and the final state."""
    M = _lib()
    x, h_ref, st_ref = _full_reference("long_context")
    say(f"config long_context chunk={chunk}")
    d = dev_inputs(x)
    h, st = run_chunkwise(M, d, chunk, return_state=True)
    del d
    err = _max_rel_err_by_head(h, h_ref)
    say(f"long_context chunk={chunk}: max rel err {err:.3e}")
    assert err <= TOL["bf16"]
    ec, en = state_err(st, st_ref)
    assert ec <= TOL["bf16"] and en <= TOL["bf16"]


def test_config_decode():
    """512-token prefill (state from the oracle's closed form), then 1000 steps:
    h of all 64 x 8 heads at every step and the final state, against the
    float64 recurrence stepped over every head."""
    M = _lib()
    cfg = CONFIGS["decode"]
    B, H, K, V = cfg["B"], cfg["H"], cfg["d_qk"], cfg["d_v"]
    say("config decode prefill")
    pre = make_fwd_inputs(B, H, cfg["prefill"], K, V, "fp32", seed=0)
    Cr, nr, mr = orc.mlstm_final_state(pre["k"], pre["v"], pre["i_pre"], pre["f_pre"])
    C = torch.from_numpy(Cr.astype(np.float32)).cuda()
    n = torch.from_numpy(nr.astype(np.float32)).cuda()
    m = torch.from_numpy(mr.astype(np.float32)).cuda()
    # the oracle starts from the same float32 state the GPU gets
    Cs = np.ascontiguousarray(C.cpu().numpy(), dtype=np.float64)
    ns = np.ascontiguousarray(n.cpu().numpy(), dtype=np.float64)
    ms = np.ascontiguousarray(m.cpu().numpy(), dtype=np.float64)
    n2, m2 = torch.empty_like(n), torch.empty_like(m)
    worst = 0.0
    say("config decode steps")
    for s in range(cfg["steps"]):
        x = make_step_inputs(B, H, K, V, step=s, dtype="fp32", seed=1)
        d = {a: torch.from_numpy(x[a]).cuda() for a in NAMES}
        h = torch.full((B, H, V), float("nan"), device="cuda")
        M.mlstm_step(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], C, n, m, n2, m2, h)
        n, n2, m, m2 = n2, n, m2, m
        hr = mlstm_step_c(*[x[a] for a in NAMES], Cs, ns, ms)
        worst = max(worst, rel_err(host(h), hr))
        if s % 250 == 0 or s == cfg["steps"] - 1:
            say(f"decode step {s} worst so far {worst:.2e}")
    assert worst <= TOL["fp32"]
    ec, en = state_err((C, n, m), (Cs, ns, ms))
    assert ec <= TOL["fp32"] and en <= TOL["fp32"]


def test_chunkwise_prefill_then_steps():
    """State hand-off: bf16 chunkwise prefill on the GPU, then float32 decode steps."""
    M = _lib()
    B, H, K, V, T1, T2 = 2, 4, 256, 512, 512, 40
    say("prefill -> steps hand-off")
    x = make_fwd_inputs(B, H, T1 + T2, K, V, "bf16", seed=11)
    h_ref, st_ref = oracle(x)
    d = dev_inputs(x)
    pre = {a: t[:, :, :T1].contiguous() for a, t in d.items()}
    h1, (C, n, m) = M.mlstm_fwd_chunkwise(pre["q"], pre["k"], pre["v"], pre["o_pre"], pre["i_pre"],
                                          pre["f_pre"], chunk=128, return_state=True)
    n2, m2 = torch.empty_like(n), torch.empty_like(m)
    hs = [h1.float()]
    for t in range(T1, T1 + T2):
        step = {a: d[a][:, :, t].contiguous() for a in d}
        h, _, _ = M.mlstm_step(step["q"], step["k"], step["v"], step["o_pre"], step["i_pre"],
                               step["f_pre"], C, n, m, n2, m2)
        hs.append(h.float()[:, :, None])
        n, n2, m, m2 = n2, n, m2, m
    torch.cuda.synchronize()
    h = torch.cat(hs, dim=2).cpu().numpy().astype(np.float64)
    assert rel_err(h, h_ref) <= TOL["bf16"]
    ec, en = state_err((C, n, m), st_ref)
    assert ec <= TOL["bf16"] and en <= TOL["bf16"]


def test_chunkwise_graph_replays_match_eager():
    """The fused forward captured in a HIP graph (no memsets or host syncs in the
    path): three replays, with eager launches and synchronisations between them,
    each equal bit for bit to the eager result."""
    M = _lib()
    say("graph replay")
    from linear_recurrent_sequence_fwd_amd import _lib as L
    x = make_fwd_inputs(1, 2, 1000, 128, 256, "bf16", seed=21)
    d = dev_inputs(x)
    ref = run_chunkwise(M, d, 128)
    h = torch.empty_like(d["v"])
    args = L.fwd_args(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], h)
    nbytes = L.chunkwise_workspace_bytes(args, 128)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    lib = L.lib()

    def one():
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert lib.mlstm_fwd_chunkwise(ctypes.byref(args), 128, ws.data_ptr(), nbytes, stream) == 0

    one()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one()
    torch.cuda.synchronize()
    for rep in range(3):
        h.zero_()
        other = run_chunkwise(M, d, 64)        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, ref), f"replay {rep}"
        assert other.shape == ref.shape


def test_clock_probe_reads_a_plausible_clock():
    """The measurement helper: both counters advance, the constant-rate counter
    runs at about its nominal 100 MHz against HIP events, and the shader clock
    it implies lies between 0.5 and 3 GHz."""
    from linear_recurrent_sequence_fwd_amd import _lib as L
    ticks = torch.zeros(4, dtype=torch.int64, device="cuda")
    L.clock_probe(ticks, 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    L.clock_probe(ticks, 250)
    e1.record()
    torch.cuda.synchronize()
    t = ticks.cpu().tolist()
    assert t[1] > t[0] and t[3] > t[2]
    rt_mhz = (t[3] - t[2]) / (e0.elapsed_time(e1) * 1e3)
    assert 80.0 < rt_mhz < 120.0, rt_mhz
    mhz = (t[1] - t[0]) / (t[3] - t[2]) * rt_mhz
    assert 500.0 < mhz < 3000.0, mhz
