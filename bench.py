"""Benchmark of the mLSTM cell forward on one MI355X.

One step = one full chunkwise forward (gate prefix sums per 64-token tile,
the chunks' end states and their in-order fold, the fused tile kernel that
produces h) over the 7B-layer-shaped workload
(B=1, H=8, T=8192, d_qk=256, d_v=512, bf16 q/k/v/o and h, float32 gates),
inputs resident in HBM. Prints ONE JSON line on stdout; progress goes to
stderr.

Extra keys: per-kernel average durations from HIP events recorded around
every launch inside the timed region, the roofline of the dominant kernel,
the chunk sweep, the decode step (B=64, H=8, float32 state) in % of HBM
bandwidth, and the oracle timed on the host cores (a baseline, not a target).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12            # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5166e15   # flop/s dense bf16: 256 CU x 2.4 GHz x 4096 flop/clk
METRIC = "mLSTM fwd tokens/s at 7B-layer shape, % bf16 MFMA peak; decode step % HBM BW"
WORKLOAD = dict(B=1, H=8, T=8192, d_qk=256, d_v=512)
DECODE = dict(B=64, H=8, d_qk=256, d_v=512, prefill=512)
SLSTM = dict(B=16, H=8, D=128, T=2048)   # sLSTM recurrence: 128 sequence-heads of 128 cells
FP32_PEAK = 157.3e12          # flop/s float32 vector (FMA = 2 flops), 256 CUs
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_kernel_7b_layer_traffic.md")
KERNEL_SRC = os.path.join(ROOT, "linear_recurrent_sequence_fwd_amd", "csrc", "mlstm_fused.hip")
TILE = 64                    # tokens per tile: the length of the quadratic (intra-tile) form
LABELS = {"gate": "gate", "state": "chunk_states", "out": "fused"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime already loaded by torch."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


# ---------------------------------------------------------------- algorithmic work

def fwd_bytes(B, H, T, K, V, chunk):
    """Algorithmic HBM bytes of the whole forward as timed (no final state
    requested): q, k, v, o read once and h written once (bf16), float32 gates
    read once."""
    return B * H * T * (2 * K + 2 * K + 2 * V + 2 * V + 2 * V + 4 + 4)


def fwd_flops(B, H, T, K, V):
    """Flops of the method as computed: per token-head 2KV (state readout
    q C~^T) + 2KV (state update) + TILE K (causal half of Q K^T over a tile)
    + TILE V (causal half of P V)."""
    return B * H * T * (4 * K * V + TILE * (K + V))


def kernel_bytes(name, B, H, T, K, V, chunk):
    """Algorithmic bytes one launch of a kernel must move (inputs read once,
    outputs written once), at the 7B-layer shape with bf16 data."""
    BH = B * H
    Nt = -(-T // TILE)
    S = -(-Nt // (chunk // TILE))
    state = 4 * (V * K + K) + 8                    # one float32 chunk state C~, n~ and its stabiliser
    gate_tok = 3 * 8 + 4                           # u, b, mp (float64) and rs (int32)
    if name == "gate":
        return BH * T * (4 + 4 + gate_tok + 4) + BH * Nt * (8 + 8 + 4)
    if name == "state":                            # chunks' end states: K, V of chunks 0..S-2; fold
        t_loc = min(T, (S - 1) * chunk)
        return BH * t_loc * (2 * K + 2 * V + 8) + BH * (S - 1) * (3 * state + 8)
    if name == "out":                              # fused tiles: q, k, v, o in, h out, chunk start states
        return BH * T * (2 * K + 2 * K + 2 * V + 2 * V + 2 * V + gate_tok) + BH * Nt * 20 \
            + BH * (S - 1) * state
    raise KeyError(name)


def decode_bytes(B, H, K, V):
    """Algorithmic bytes of one decode step: read and write the float32 state
    (C, n, m), read q, k, v, o and the gates, write h (all float32)."""
    BH = B * H
    return BH * (2 * (V * K + K + 1) * 4 + (2 * K + 2 * V) * 4 + 8 + V * 4)


# ---------------------------------------------------------------- the runs

def make_device_inputs(torch, cfg, dtype="bf16", seed=0):
    from linear_recurrent_sequence_fwd_amd.inputs import make_fwd_inputs
    x = make_fwd_inputs(cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], dtype, seed=seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(x[n]).to("cuda").to(tdt) for n in ("q", "k", "v", "o_pre")}
    for n in ("i_pre", "f_pre"):
        d[n] = torch.from_numpy(x[n]).to("cuda")
    return x, d


def time_chunkwise(torch, M, L, ev, d, chunk, steps, warmup, kernels=("gate", "state", "out")):
    """Wall time of `steps` forward calls with no profiling hooks, then the
    average duration of each kernel group from HIP events recorded around its
    launches in a second, separate pass of the same number of calls."""
    from linear_recurrent_sequence_fwd_amd import _lib
    h = torch.empty_like(d["v"])
    args = _lib.fwd_args(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], h)
    nbytes = _lib.chunkwise_workspace_bytes(args, chunk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib, pargs, wsp = _lib.lib(), ctypes.byref(args), ws.data_ptr()

    def one():     # arguments marshalled once; the loop only enqueues
        code = lib.mlstm_fwd_chunkwise(pargs, chunk, wsp, nbytes, stream)
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    pairs = {k: ev.create(2 * steps) for k in kernels}
    arrays = [_lib.event_array([pairs[g][2 * i + e] if g in kernels else None
                                for g in _lib.PROF_GROUPS for e in (0, 1)]) for i in range(steps)]
    for i in range(steps):
        code = lib.mlstm_prof_fwd_chunkwise(pargs, chunk, wsp, nbytes, stream, arrays[i])
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())
    torch.cuda.synchronize()
    per_kernel = {}
    for k in kernels:
        ms = [ev.elapsed_ms(pairs[k][2 * i], pairs[k][2 * i + 1]) for i in range(steps)]
        per_kernel[k] = sum(ms) / len(ms) * 1e3      # us
        ev.destroy(pairs[k])
    return elapsed, per_kernel


def time_chunkwise_graph(torch, d, chunk, steps, warmup):
    """Wall time of `steps` replays of a HIP graph holding one forward call (its
    four kernel launches), captured on torch's capture stream."""
    from linear_recurrent_sequence_fwd_amd import _lib
    h = torch.empty_like(d["v"])
    args = _lib.fwd_args(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], h)
    nbytes = _lib.chunkwise_workspace_bytes(args, chunk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    lib, pargs, wsp = _lib.lib(), ctypes.byref(args), ws.data_ptr()

    def one():
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        code = lib.mlstm_fwd_chunkwise(pargs, chunk, wsp, nbytes, stream)
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())

    one()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    del g
    return elapsed


def time_decode(torch, M, ev, steps, warmup):
    from linear_recurrent_sequence_fwd_amd.inputs import make_step_inputs
    cfg = DECODE
    B, H, K, V = cfg["B"], cfg["H"], cfg["d_qk"], cfg["d_v"]
    # state from a 512-token chunkwise prefill of the 7B-layer distributions
    _, pre = make_device_inputs(torch, dict(B=B, H=H, T=cfg["prefill"], d_qk=K, d_v=V), "bf16", seed=3)
    _, (C, n, m) = M.mlstm_fwd_chunkwise(pre["q"], pre["k"], pre["v"], pre["o_pre"], pre["i_pre"],
                                         pre["f_pre"], chunk=128, return_state=True)
    del pre
    pool = []
    for s in range(8):
        x = make_step_inputs(B, H, K, V, step=s, dtype="fp32", seed=4)
        pool.append({a: torch.from_numpy(x[a]).to("cuda") for a in ("q", "k", "v", "o_pre", "i_pre", "f_pre")})
    from linear_recurrent_sequence_fwd_amd import _lib
    n2, m2 = torch.empty_like(n), torch.empty_like(m)
    h = torch.empty((B, H, V), device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    bufs = [(n, m, n2, m2), (n2, m2, n, m)]
    lib = _lib.lib()
    # arguments marshalled once per (input set, ping-pong parity); the loop only enqueues
    structs = [[_lib.step_args(x["q"], x["k"], x["v"], x["o_pre"], x["i_pre"], x["f_pre"], C, *bufs[p], h)
                for p in range(2)] for x in pool]

    def one(i):
        code = lib.mlstm_step(ctypes.byref(structs[i % len(pool)][i % 2]), stream)
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    evs = ev.create(2 * steps)     # per-launch durations: a second pass through the profiling call
    for i in range(steps):
        j = warmup + steps + i
        code = lib.mlstm_prof_step(ctypes.byref(structs[j % len(pool)][j % 2]), stream, evs[2 * i],
                                   evs[2 * i + 1])
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())
    torch.cuda.synchronize()
    k_us = sum(ev.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)) / steps * 1e3
    ev.destroy(evs)
    assert bool(torch.isfinite(h).all())
    return elapsed, k_us


def slstm_flops(B, H, T, D):
    """Flops of the sLSTM recurrence as computed: per step and cell the four
    recurrent dot products (2 * 4 * D) plus about 24 for the gates, the
    stabiliser and the cell update."""
    return B * H * T * D * (8 * D + 24)


def time_slstm(torch, reps, warmup):
    """Event-timed sLSTM forward calls (one kernel each) on the current stream."""
    from linear_recurrent_sequence_fwd_amd import _lib
    from linear_recurrent_sequence_fwd_amd.inputs import make_slstm_inputs
    B, H, T, D = SLSTM["B"], SLSTM["H"], SLSTM["T"], SLSTM["D"]
    pre, R = make_slstm_inputs(B, H, T, D, seed=5)
    pre_d, R_d = torch.from_numpy(pre).cuda(), torch.from_numpy(R).cuda()
    h = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        _lib.slstm_fwd(pre_d, R_d, h=h)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        _lib.slstm_fwd(pre_d, R_d, h=h)
    e1.record()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(h).all())
    return e0.elapsed_time(e1) / reps * 1e-3, pre, R


def slstm_cpu_baseline(pre, R, budget_s=8.0):
    """The sLSTM oracle recurrence on one host thread over all sequences and
    heads, as many leading steps as fit the budget."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle.slstm_oracle import slstm_step
    B, T, _, H, D = pre.shape
    c = np.zeros((B, H, D)); n = np.zeros((B, H, D)); m = np.zeros((B, H, D)); h = np.zeros((B, H, D))
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while done < T and time.perf_counter() - t0 < budget_s:
            c, n, m, h = slstm_step(pre[:, done], R, c, n, m, h)
            done += 1
        el = time.perf_counter() - t0
    return {"value": B * done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 NumPy sLSTM step recurrence, B={B} H={H} D={D}, first {done} of {T} "
                      f"steps ({el:.1f} s, one thread)"}


def cpu_baseline(x, budget_s=15.0):
    """The oracle recurrence on the host, all heads, as many leading tokens as fit the budget."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle.mlstm_oracle import mlstm_step
    names = ("q", "k", "v", "i_pre", "f_pre", "o_pre")
    a = {n: x[n][0].astype(np.float64) for n in names}     # [H, T, ...]
    H, T, K = a["q"].shape
    V = a["v"].shape[-1]
    C = np.zeros((H, V, K)); n = np.zeros((H, K)); m = np.zeros(H)
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while done < T and time.perf_counter() - t0 < budget_s:
            t = done
            _, C, n, m = mlstm_step(a["q"][:, t], a["k"][:, t], a["v"][:, t], a["i_pre"][:, t],
                                    a["f_pre"][:, t], a["o_pre"][:, t], C, n, m)
            done += 1
        el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 NumPy step recurrence, B=1 H={H} d_qk={K} d_v={V}, first {done} of "
                      f"{T} tokens ({el:.1f} s, one thread)"}


def traffic_from_profile():
    """HBM bytes per launch of the output kernel from the committed counter
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sha:
        return None
    return float(m_b.group(1))


def measure_clock(torch, d, chunk, steps=20, iters=250):
    """Shader clock (MHz) while the chunkwise forward runs. The probe wave sleeps
    on a side stream (default priority) while `steps` forward calls run on the
    current stream; its shader-clock ticks over its constant-rate ticks, times
    that counter's rate, give the clock. The rate itself (nominally 100 MHz) is
    taken from an event-timed probe run alone, whose own clock is reported as
    the idle figure. iters = 250 sleeps last about 1 ms, well inside the
    forward calls."""
    from linear_recurrent_sequence_fwd_amd import _lib
    ticks = torch.zeros(4, dtype=torch.int64, device="cuda")
    # rate of the constant counter, and the clock with nothing else running
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _lib.clock_probe(ticks, iters)
    e0.record()
    _lib.clock_probe(ticks, iters)
    e1.record()
    torch.cuda.synchronize()
    t = ticks.cpu().tolist()
    rt_mhz = (t[3] - t[2]) / (e0.elapsed_time(e1) * 1e3)
    idle_mhz = (t[1] - t[0]) / (t[3] - t[2]) * rt_mhz
    # the clock under the forward pass
    h = torch.empty_like(d["v"])
    args = _lib.fwd_args(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], h)
    nbytes = _lib.chunkwise_workspace_bytes(args, chunk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    main_stream = torch.cuda.current_stream()
    stream = ctypes.c_void_p(main_stream.cuda_stream)
    lib, pargs, wsp = _lib.lib(), ctypes.byref(args), ws.data_ptr()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _lib.clock_probe(ticks, iters)
    for _ in range(steps):
        code = lib.mlstm_fwd_chunkwise(pargs, chunk, wsp, nbytes, stream)
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())
    torch.cuda.synchronize()
    t = ticks.cpu().tolist()
    load_mhz = (t[1] - t[0]) / (t[3] - t[2]) * rt_mhz
    return {"under_load_mhz": load_mhz, "idle_mhz": idle_mhz, "realtime_counter_mhz": rt_mhz,
            "method": "s_memtime over s_memrealtime of one sleeping wave beside the forward calls"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--chunk", type=int, default=1024,
                    help="chunk length: the state is materialised at chunk starts (multiple of 64)")
    ap.add_argument("--sweep", type=str, default="512,2048", help="chunk sizes reported besides --chunk")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the replayed-graph timing")
    ap.add_argument("--no-clock", action="store_true", help="skip the shader clock measurement")
    ap.add_argument("--no-slstm", action="store_true", help="skip the sLSTM recurrence measurement")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only: the mLSTM path here is a single-GPU build "
              f"(--gpus {args.gpus} requested). Heads and batch shard with no exchange; see the "
              f"design notes for the multi-GPU plan.", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_recurrent_sequence_fwd_amd as M
    from linear_recurrent_sequence_fwd_amd import _lib
    _lib.lib()
    ev = HipEvents()
    cfg = WORKLOAD
    B, H, T, K, V = cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"]

    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {n} bytes read and written per launch, 3 launches")
        del src, dst

    log(f"[bench] inputs 7B-layer B={B} H={H} T={T} d_qk={K} d_v={V} bf16")
    x, d = make_device_inputs(torch, cfg, "bf16", seed=0)

    log(f"[bench] chunkwise chunk={args.chunk}: warmup {args.warmup}, steps {args.steps}")
    elapsed, per_k = time_chunkwise(torch, M, _lib, ev, d, args.chunk, args.steps, args.warmup)
    ms_step = elapsed / args.steps * 1e3
    tok_s = B * T * args.steps / elapsed
    flops = fwd_flops(B, H, T, K, V)
    flops_ci = B * H * T * 4 * K * V
    path_bytes = fwd_bytes(B, H, T, K, V, args.chunk)
    dom = max(per_k, key=per_k.get)
    t_dom = per_k[dom] * 1e-6
    kb = kernel_bytes(dom, B, H, T, K, V, args.chunk)
    # the fused kernel carries all of the method's flops; the others are bandwidth work
    kf = flops if dom == "out" else 0.0
    hbm_f, mfma_f = kb / t_dom / HBM_PEAK, kf / t_dom / MFMA_BF16_PEAK
    if mfma_f > hbm_f:
        roof = {"bound": "mfma", "achieved": kf / t_dom / 1e12, "peak": MFMA_BF16_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": mfma_f}
    else:
        roof = {"bound": "hbm", "achieved": kb / t_dom / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": hbm_f}
    roof = {"kernel": LABELS[dom], **roof, "hbm_frac": hbm_f, "mfma_frac": mfma_f,
            "algorithmic_bytes": kb, "algorithmic_flops": kf,
            "traffic": traffic_from_profile() if dom == "out" else None}
    per_k = {LABELS[k]: v for k, v in per_k.items()}
    log(f"[bench] {ms_step:.3f} ms/step, {tok_s:.3e} tokens/s, kernels us {per_k}")

    sweep = {}
    for L in [int(s) for s in args.sweep.split(",") if s]:
        if L == args.chunk:
            continue
        el, pk = time_chunkwise(torch, M, _lib, ev, d, L, max(5, args.steps // 2), 2)
        st = max(5, args.steps // 2)
        sweep[str(L)] = {"ms_per_step": el / st * 1e3, "tokens_per_s": B * T * st / el,
                         "mfma_frac": flops / (el / st) / MFMA_BF16_PEAK,
                         "kernel_us": {LABELS[k]: v for k, v in pk.items()}}
        log(f"[bench] sweep chunk={L}: {el / st * 1e3:.3f} ms/step")

    graph_ms = None
    if not args.no_graph:
        g_el = time_chunkwise_graph(torch, d, args.chunk, args.steps, args.warmup)
        graph_ms = g_el / args.steps * 1e3
        log(f"[bench] chunkwise as a replayed HIP graph: {graph_ms:.3f} ms/step")

    clock = None
    if not args.no_clock:
        clock = measure_clock(torch, d, args.chunk)
        log(f"[bench] shader clock during the forward: {clock['under_load_mhz']:.0f} MHz "
            f"(idle {clock['idle_mhz']:.0f} MHz, constant counter {clock['realtime_counter_mhz']:.1f} MHz)")

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded PCG64 draws with the 7B-layer distributions)",
        "config": {"workload": "mLSTM chunkwise forward, 7B-layer shape", "B": B, "H": H, "T": T,
                   "d_qk": K, "d_v": V, "chunk": args.chunk, "tile": TILE,
                   "inputs": "bf16 q/k/v/o, fp32 gates",
                   "parallelism": "single GPU"},
        "mfma_frac": flops / (ms_step * 1e-3) / MFMA_BF16_PEAK,
        "mfma_frac_chunk_independent": flops_ci / (ms_step * 1e-3) / MFMA_BF16_PEAK,
        "hbm_frac_path": path_bytes / (ms_step * 1e-3) / HBM_PEAK,
        "kernel_us": per_k,
        "roofline": roof,
        "sweep": sweep,
        "clock": clock,
        "graph_ms_per_step": graph_ms,
    }
    del d
    torch.cuda.empty_cache()

    if not args.no_decode:
        log(f"[bench] decode B={DECODE['B']} H={DECODE['H']} steps {args.decode_steps}")
        el, k_us = time_decode(torch, M, ev, args.decode_steps, 20)
        us_step = el / args.decode_steps * 1e6
        db = decode_bytes(DECODE["B"], DECODE["H"], DECODE["d_qk"], DECODE["d_v"])
        out["decode"] = {"workload": "mlstm_step B=64 H=8 d_qk=256 d_v=512 fp32 state",
                         "us_per_step": us_step, "kernel_us": k_us,
                         "tokens_per_s": DECODE["B"] / (us_step * 1e-6),
                         "achieved_GBps": db / (k_us * 1e-6) / 1e9,
                         "hbm_frac": db / (k_us * 1e-6) / HBM_PEAK,
                         "hbm_frac_wall": db / (us_step * 1e-6) / HBM_PEAK}
        log(f"[bench] decode {us_step:.1f} us/step wall, kernel {k_us:.1f} us")

    if not args.no_slstm:
        B, H, T, D = SLSTM["B"], SLSTM["H"], SLSTM["T"], SLSTM["D"]
        log(f"[bench] sLSTM B={B} H={H} T={T} D={D}")
        sec, pre, R = time_slstm(torch, 10, 2)
        fl = slstm_flops(B, H, T, D)
        # one workgroup per sequence-head runs on one CU: the launch can use at
        # most B * H of the 256 CUs' float32 peak
        peak = FP32_PEAK * min(1.0, B * H / 256)
        out["slstm"] = {"workload": f"slstm_fwd B={B} H={H} D={D} T={T} float32",
                        "ms_per_call": sec * 1e3, "us_per_step": sec / T * 1e6,
                        "tokens_per_s": B * T / sec,
                        "roofline": {"bound": "alu", "achieved": fl / sec / 1e12, "peak": peak / 1e12,
                                     "unit": "TFLOP/s", "frac": fl / sec / peak,
                                     "note": "float32 vector peak of the B*H CUs the launch occupies"}}
        log(f"[bench] sLSTM {sec * 1e3:.3f} ms per call, {sec / T * 1e6:.3f} us per step")
        if not args.no_cpu_baseline:
            out["slstm"]["cpu_baseline"] = slstm_cpu_baseline(pre, R)

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(x, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
