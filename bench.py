"""Benchmark of the mLSTM cell on one MI355X.

One step = one full chunkwise forward over the 7B-layer-shaped workload
(B=1, H=8, T=8192, d_qk=256, d_v=512; bf16 q/k/v/o and h, float32 gates):
gate prefix sums per 64-token tile, the chunks' end states and their
in-order fold, and the fused tile kernel that produces h. Inputs are
resident in HBM when a timed step starts. Prints ONE JSON line on stdout;
progress goes to stderr.

Timing protocol (every figure is a median over reps unless said otherwise):
  * cold (the primary figure): before each rep a 512 MiB scratch buffer is
    overwritten, which evicts the 256 MiB MALL and the L2s, so the step
    reads its inputs from HBM; HIP events on the launch stream bracket the
    step (and, in a second pass through the profiling entry point, each
    kernel group);
  * warm: the same steps back to back, timed on the host clock between two
    synchronisations and with events.
`value` and `ms_per_step` are the cold median step.

Roofline: the method's algorithmic bytes (4,104 B per token-head: q, k, v,
o, h in bf16 and the two float32 gates; workspace traffic is not counted)
over the cold median duration of the dominant kernel, against 8 TB/s, and
the step's flops against the dense bf16 MFMA peak (2.5 PFLOP/s). When a
committed rocprofv3 summary of the same kernel sources exists under
profiles/, its kernel-trace duration and HBM traffic are reported beside.

Other keys: the chunk sweep, the mid workload (chunkwise and parallel
forms), the long-context workload (T = 131072), the chunkwise backward pass,
the decode step, the sLSTM recurrence, the mLSTM block around the cell (its
steps timed one by one, its projections beside the same products in the
vendor library), and the float64 oracles timed on the host's cores
(baselines, not targets).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12            # B/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15      # flop/s, dense bf16 MFMA
FP32_PEAK = 157.3e12         # flop/s, float32 vector (FMA = 2 flops), 256 CUs
METRIC = "mLSTM fwd tokens/s at 7B-layer shape, % bf16 MFMA peak; decode step % HBM BW"
WORKLOAD = dict(B=1, H=8, T=8192, d_qk=256, d_v=512)
MID = dict(B=4, H=8, T=2048, d_qk=128, d_v=128)
LONG = dict(B=1, H=8, T=131072, d_qk=256, d_v=512)
DECODE = dict(B=64, H=8, d_qk=256, d_v=512, prefill=512)
SLSTM = dict(B=16, H=8, D=128, T=2048)   # sLSTM recurrence: 128 sequence-heads of 128 cells
# the block around the cell at the 7B-layer cell shape: inner width E = 2 D = H d_v = 4096
BLOCK = dict(B=1, T=8192, D=2048, H=8, d_qk=256, d_v=512, KC=4, chunk=1024)
# one device's share of the long-context sequence split over eight devices
SEGMENTS = dict(B=1, H=8, T=16384, d_qk=256, d_v=512, chunk=1024, parts=8)
TILE = 64                    # tokens per tile: the length of the quadratic (intra-tile) form
FLUSH_BYTES = 512 << 20
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_recurrent_sequence_fwd_amd", "csrc")
LABELS = {"gate": "gate", "state": "chunk_states", "out": "fused"}
BWD_LABELS = {"fwd_gate": "fwd_gate", "fwd_state": "fwd_chunk_states", "dq": "dq", "adjoint": "adjoint",
              "dkv": "dkv", "dgate": "dgate"}


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
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def record(self, e, stream):
        assert self.hip.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, evs):
        for e in evs:
            if e:
                self.hip.hipEventDestroy(e)


# ---------------------------------------------------------------- algorithmic work

def fwd_bytes(B, H, T, K, V):
    """The forward's algorithmic HBM bytes (no final state requested): q, k,
    v, o read once and h written once in bf16, the two float32 gates read
    once; 4,104 B per token-head at d_qk = 256, d_v = 512."""
    return B * H * T * (2 * K + 2 * K + 2 * V + 2 * V + 2 * V + 4 + 4)


def fwd_flops(B, H, T, K, V):
    """Flops of the forward as computed: per token-head 2KV (readout of the
    carried state, C~ q) + 2KV (state update) + TILE K (causal half of Q K^T
    over a tile) + TILE V (causal half of P V)."""
    return B * H * T * (4 * K * V + TILE * (K + V))


def bwd_bytes(B, H, T, K, V):
    """The backward's algorithmic HBM bytes: q, k, v, o, h and dh read once
    (bf16), the two gates read once, dq, dk, dv, do written once (bf16) and
    di, df written once (float32); 8,208 B per token-head at 256 / 512."""
    return B * H * T * (4 * K + 8 * V + 8 + 4 * K + 4 * V + 8)


def bwd_flops(B, H, T, K, V):
    """Flops of the backward as computed: per token-head 8KV (dq's carried
    term, the adjoint update, and the adjoint's terms of dk and dv) plus
    2 TILE (K + V) for the intra-tile products (Q K^T and G V^T, then their
    products with Q, K and G), causal halves."""
    return B * H * T * (8 * K * V + 2 * TILE * (K + V))


def decode_bytes(B, H, K, V):
    """Algorithmic bytes of one decode step: read and write the float32 state
    (C, n, m), read q, k, v, o and the gates, write h (all float32)."""
    BH = B * H
    return BH * (2 * (V * K + K + 1) * 4 + (2 * K + 2 * V) * 4 + 8 + V * 4)


def slstm_flops(B, H, T, D):
    """Flops of the sLSTM recurrence as computed: per step and cell the four
    recurrent dot products (2 * 4 * D) plus about 24 for the gates, the
    stabiliser and the cell update."""
    return B * H * T * D * (8 * D + 24)


def block_work(c):
    """Algorithmic flops and HBM bytes of each step of the block (bf16
    activations and weights, float32 vectors and gates): a step's bytes are
    its inputs read once and its outputs written once."""
    B, T, D, H, K, V, KC = c["B"], c["T"], c["D"], c["H"], c["d_qk"], c["d_v"], c["KC"]
    E, BT, n_in = 2 * D, c["B"] * c["T"], 2 * c["D"] // c["H"]
    w = {
        "layernorm": (8 * BT * D, BT * D * 2 * 2),
        "up_proj": (2 * BT * D * 2 * E, BT * D * 2 + 2 * E * D * 2 + BT * 2 * E * 2),
        "conv_gates": (BT * E * (2 * KC + 4) + 2 * BT * E * 2 * H,
                       BT * E * 2 * 2 + E * (KC + 1) * 4 + 2 * H * E * 2 + 2 * B * H * T * 4),
        "q_proj": (2 * BT * n_in * K * H, BT * E * 2 + H * K * n_in * 2 + B * H * T * K * 2),
        "k_proj": (2 * BT * n_in * K * H, BT * E * 2 + H * K * n_in * 2 + B * H * T * K * 2),
        "v_proj": (2 * BT * n_in * V * H, BT * E * 2 + H * V * n_in * 2 + B * H * T * V * 2),
        "cell": (fwd_flops(B, H, T, K, V), B * H * T * (2 * K * 2 + 2 * V * 2 + 2 * 4)),
        "groupnorm_gate": (BT * E * 12, BT * E * 2 * 4),
        "down_proj": (2 * BT * E * D, BT * E * 2 + D * E * 2 + 2 * BT * D * 2),
    }
    return w


# ---------------------------------------------------------------- timing

class Timer:
    """Cold and warm step timing on the current stream."""

    def __init__(self, torch, ev):
        self.torch = torch
        self.ev = ev
        self.scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def flush(self, i):
        self.scratch.fill_(i & 0xFF)

    def cold(self, fn, reps, warmup=2):
        """Median, mean and min (ms) of `reps` steps, each after a flush."""
        for i in range(warmup):
            self.flush(i)
            fn()
        evs = self.ev.create(2 * reps)
        for i in range(reps):
            self.flush(i)
            self.ev.record(evs[2 * i], self.stream)
            fn()
            self.ev.record(evs[2 * i + 1], self.stream)
        self.torch.cuda.synchronize()
        ms = [self.ev.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(reps)]
        self.ev.destroy(evs)
        return {"median_ms": statistics.median(ms), "mean_ms": statistics.fmean(ms), "min_ms": min(ms),
                "reps": reps}

    def warm(self, fn, reps, warmup=3):
        """Back-to-back steps: host-clock time per step between two
        synchronisations, and the median of per-step events."""
        for _ in range(warmup):
            fn()
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        self.torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / reps * 1e3
        evs = self.ev.create(2 * reps)
        for i in range(reps):
            self.ev.record(evs[2 * i], self.stream)
            fn()
            self.ev.record(evs[2 * i + 1], self.stream)
        self.torch.cuda.synchronize()
        ms = [self.ev.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(reps)]
        self.ev.destroy(evs)
        return {"wall_ms": wall, "median_ms": statistics.median(ms), "reps": reps}

    def groups(self, fn_prof, groups, reps, cold=True):
        """Median duration (us) of each kernel group, from the events the
        profiling entry point records around the groups."""
        from linear_recurrent_sequence_fwd_amd import _lib
        per = {g: [] for g in groups}
        for i in range(reps):
            evs = self.ev.create(2 * len(groups))
            if cold:
                self.flush(i)
            fn_prof(_lib.event_array(evs))
            self.torch.cuda.synchronize()
            for k, g in enumerate(groups):
                per[g].append(self.ev.elapsed_ms(evs[2 * k], evs[2 * k + 1]) * 1e3)
            self.ev.destroy(evs)
        return {g: statistics.median(v) for g, v in per.items()}


def make_device_inputs(torch, cfg, dtype="bf16", seed=0):
    from linear_recurrent_sequence_fwd_amd.inputs import make_fwd_inputs
    x = make_fwd_inputs(cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"], dtype, seed=seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(x[n]).to("cuda").to(tdt) for n in ("q", "k", "v", "o_pre")}
    for n in ("i_pre", "f_pre"):
        d[n] = torch.from_numpy(x[n]).to("cuda")
    return x, d


def chunkwise_callables(torch, d, chunk):
    """(plain call, profiling call taking an event array) of one chunkwise
    forward on the current stream; arguments are marshalled once, the calls
    only enqueue."""
    from linear_recurrent_sequence_fwd_amd import _lib
    h = torch.empty_like(d["v"])
    args = _lib.fwd_args(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], h)
    nbytes = _lib.chunkwise_workspace_bytes(args, chunk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib, pargs, wsp = _lib.lib(), ctypes.byref(args), ws.data_ptr()

    def one():
        code = lib.mlstm_fwd_chunkwise(pargs, chunk, wsp, nbytes, stream)
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())

    def prof(events):
        code = lib.mlstm_prof_fwd_chunkwise(pargs, chunk, wsp, nbytes, stream, events)
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())

    one.keep = prof.keep = (h, ws, args)
    return one, prof


def segment_callables(torch, d, chunk, parts):
    """Calls of one device's part in a sequence split into `parts` segments:
    its summary, the fold of the other devices' summaries into its start
    state (the last device's: parts - 1 of them), and its forward from the
    folded start state; arguments marshalled once, the calls only enqueue."""
    from linear_recurrent_sequence_fwd_amd import _lib
    B, H, T, K = d["k"].shape
    V = d["v"].shape[-1]
    f32 = dict(dtype=torch.float32, device="cuda")
    summ = (torch.empty((B, H, V, K), **f32), torch.empty((B, H, K), **f32), torch.empty((B, H), **f32),
            torch.empty((B, H), dtype=torch.float64, device="cuda"))
    sargs = _lib.summary_args(d["k"], d["v"], d["i_pre"], d["f_pre"], *summ)
    sbytes = _lib.summary_workspace_bytes(sargs, chunk)
    sws = torch.empty(sbytes, dtype=torch.uint8, device="cuda")
    start = (torch.zeros((B, H, V, K), **f32), torch.zeros((B, H, K), **f32), torch.zeros((B, H), **f32))
    folded = (torch.empty((B, H, V, K), **f32), torch.empty((B, H, K), **f32), torch.empty((B, H), **f32))
    # the last device's start: the fold of the P - 1 summaries before it, stacked as an all-gather
    # leaves them
    stack = tuple(torch.zeros((parts - 1,) + tuple(t.shape), dtype=t.dtype, device="cuda") for t in summ)
    cargs = _lib.CombineArgs(B, H, K, V, parts - 1, *[t.data_ptr() for t in start],
                             *[t.data_ptr() for t in stack], *[t.data_ptr() for t in folded])
    h = torch.empty_like(d["v"])
    fargs = _lib.fwd_args(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], h, *folded)
    fbytes = _lib.chunkwise_workspace_bytes(fargs, chunk)
    fws = torch.empty(fbytes, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = _lib.lib()

    def check(code):
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())

    def summary():
        check(lib.mlstm_segment_summary(ctypes.byref(sargs), chunk, sws.data_ptr(), sbytes, stream))

    def combine():
        check(lib.mlstm_state_combine(ctypes.byref(cargs), stream))

    def forward():
        check(lib.mlstm_fwd_chunkwise(ctypes.byref(fargs), chunk, fws.data_ptr(), fbytes, stream))

    keep = (summ, sargs, sws, start, stack, folded, cargs, h, fargs, fws)
    summary.keep = combine.keep = forward.keep = keep
    return summary, combine, forward


def parallel_callable(torch, d):
    from linear_recurrent_sequence_fwd_amd import _lib
    h = torch.empty_like(d["v"])
    args = _lib.fwd_args(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], h)
    nbytes = _lib.parallel_workspace_bytes(args)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib, pargs, wsp = _lib.lib(), ctypes.byref(args), ws.data_ptr()

    def one():
        code = lib.mlstm_fwd_parallel(pargs, wsp, nbytes, stream)
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())

    one.keep = (h, ws, args)
    return one


def backward_callables(torch, d, chunk, seed=0):
    """(plain call, profiling call) of one chunkwise backward pass given the
    forward's h and a seeded upstream gradient dh."""
    import linear_recurrent_sequence_fwd_amd as M
    from linear_recurrent_sequence_fwd_amd import _lib
    from linear_recurrent_sequence_fwd_amd.inputs import make_grad_output
    B, H, T, K = d["q"].shape
    V = d["v"].shape[-1]
    h = M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], chunk=chunk)
    dh = torch.from_numpy(make_grad_output(B, H, T, V, "bf16", seed=seed)).cuda().to(torch.bfloat16)
    grads = _lib.bwd_outputs(d["q"], d["v"])
    args = _lib.bwd_args(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"], h, dh, grads)
    nbytes = _lib.bwd_workspace_bytes(args, chunk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib, pargs, wsp = _lib.lib(), ctypes.byref(args), ws.data_ptr()

    def one():
        code = lib.mlstm_bwd_chunkwise(pargs, chunk, wsp, nbytes, stream)
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())

    def prof(events):
        code = lib.mlstm_prof_bwd_chunkwise(pargs, chunk, wsp, nbytes, stream, events)
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())

    one.keep = prof.keep = (h, dh, grads, ws, args)
    return one, prof


def graph_ms(torch, d, chunk, steps, warmup):
    """Host-clock time per replay of a HIP graph holding one chunkwise forward
    (captured on torch's capture stream, its buffers from the graph's pool)."""
    one, _ = chunkwise_callables(torch, d, chunk)
    one()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cap, _ = chunkwise_callables(torch, d, chunk)
        cap()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    del g, cap
    return el / steps * 1e3


def time_decode(torch, M, timer, steps, warmup):
    """Host-clock time per step of `steps` back-to-back decode steps
    (ping-ponged n, m), and the median kernel duration from events around
    each launch."""
    from linear_recurrent_sequence_fwd_amd import _lib
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
    n2, m2 = torch.empty_like(n), torch.empty_like(m)
    h = torch.empty((B, H, V), device="cuda")
    stream = timer.stream
    bufs = [(n, m, n2, m2), (n2, m2, n, m)]
    lib = _lib.lib()
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
    wall_us = (time.perf_counter() - t0) / steps * 1e6
    evs = timer.ev.create(2 * steps)
    for i in range(steps):
        j = warmup + steps + i
        code = lib.mlstm_prof_step(ctypes.byref(structs[j % len(pool)][j % 2]), stream, evs[2 * i],
                                   evs[2 * i + 1])
        if code:
            raise RuntimeError(lib.mlstm_last_error().decode())
    torch.cuda.synchronize()
    k_us = statistics.median(timer.ev.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)) * 1e3
    timer.ev.destroy(evs)
    assert bool(torch.isfinite(h).all())
    return wall_us, k_us


def time_slstm(torch, timer, reps):
    from linear_recurrent_sequence_fwd_amd import _lib
    from linear_recurrent_sequence_fwd_amd.inputs import make_slstm_inputs
    B, H, T, D = SLSTM["B"], SLSTM["H"], SLSTM["T"], SLSTM["D"]
    pre, R = make_slstm_inputs(B, H, T, D, seed=5)
    pre_d, R_d = torch.from_numpy(pre).cuda(), torch.from_numpy(R).cuda()
    h = torch.empty((B, T, H, D), dtype=torch.float32, device="cuda")

    def one():
        _lib.slstm_fwd(pre_d, R_d, h=h)

    r = timer.warm(one, reps, warmup=2)
    assert bool(torch.isfinite(h).all())
    return r["median_ms"] * 1e-3, pre, R


def block_setup(torch, c, seed=0):
    import numpy as np
    from linear_recurrent_sequence_fwd_amd import _lib
    from linear_recurrent_sequence_fwd_amd.inputs import make_block_inputs
    x, p = make_block_inputs(c["B"], c["T"], c["D"], c["H"], c["d_qk"], c["d_v"], KC=c["KC"], seed=seed)
    dp = {}
    for name, is_mat in _lib.BLOCK_ARRAYS:
        a = torch.from_numpy(np.ascontiguousarray(p[name], dtype=np.float32))
        dp[name] = a.to("cuda", torch.bfloat16) if is_mat else a.to("cuda")
    bp = _lib.block_params(dp, c["D"], c["H"], c["d_qk"], c["d_v"], c["KC"], p["eps_ln"], p["eps_gn"])
    return x, p, dp, bp, torch.from_numpy(x).to("cuda", torch.bfloat16)


def block_callables(torch, c, p, dp, bp, xd):
    """The whole block, each of its steps alone (the same kernels and launch
    configurations, on the intermediates of a first full run), and the same
    projections in the vendor library (torch.addmm: hipBLASLt) for reference."""
    from linear_recurrent_sequence_fwd_amd import _lib
    B, T, D, H, K, V, chunk = c["B"], c["T"], c["D"], c["H"], c["d_qk"], c["d_v"], c["chunk"]
    E, BT, n_in = 2 * D, B * T, 2 * D // H
    out = torch.empty_like(xd)
    ws = torch.empty(_lib.block_workspace_bytes(bp, B, T, chunk), dtype=torch.uint8, device="cuda")
    _, st = _lib.mlstm_block_fwd(xd, bp, chunk=chunk, out=out, workspace=ws, return_stages=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    cell_args = _lib.fwd_args(st["q"], st["k"], st["v"], None, st["i_pre"], st["f_pre"], st["h"])
    cell_ws = torch.empty(max(1, _lib.chunkwise_workspace_bytes(cell_args, chunk)), dtype=torch.uint8,
                          device="cuda")

    def proj(src, ld, W, n_out, bias, alpha, C):
        return _lib.gemm_bf16_strided(T, n_out, n_in, B, H, src, ld, T * ld, n_in, W, n_in, 0, n_out * n_in,
                                      C, n_out, H * T * n_out, T * n_out, alpha=alpha, bias=bias,
                                      stride_bias2=n_out)

    xn2, xup2, y2, out2, x2 = (st["xn"].view(BT, D), st["xup"].view(BT, 2 * E), st["y"].view(BT, E),
                               out.view(BT, D), xd.view(BT, D))
    steps = {
        "layernorm": lambda: _lib.layernorm_bf16(xd, dp["ln_w"], dp["ln_b"], p["eps_ln"], y=st["xn"]),
        "up_proj": lambda: _lib.gemm_bf16(xn2, dp["W_up"], dp["b_up"], C=xup2),
        "conv_gates": lambda: _lib.block_conv_gates(bp, st["xup"]),
        "q_proj": lambda: proj(st["xc"], E, dp["W_q"], K, dp["b_q"], 1.0, st["q"]),
        "k_proj": lambda: proj(st["xc"], E, dp["W_k"], K, dp["b_k"], K ** -0.5, st["k"]),
        "v_proj": lambda: proj(st["xup"], 2 * E, dp["W_v"], V, dp["b_v"], 1.0, st["v"]),
        "cell": lambda: _lib.mlstm_fwd_chunkwise(st["q"], st["k"], st["v"], None, st["i_pre"], st["f_pre"],
                                                 chunk=chunk, h=st["h"], workspace=cell_ws),
        "groupnorm_gate": lambda: _lib.block_groupnorm_gate(bp, st["h"], st["xc"], st["xup"]),
        "down_proj": lambda: _lib.gemm_bf16(y2, dp["W_down"], dp["b_down"], R=x2, C=out2),
    }
    lib_out = {"up_proj": torch.empty_like(xup2), "down_proj": torch.empty_like(out2)}
    b_up16, b_down16 = dp["b_up"].to(torch.bfloat16), dp["b_down"].to(torch.bfloat16)
    library = {
        "up_proj": lambda: torch.addmm(b_up16, xn2, dp["W_up"].t(), out=lib_out["up_proj"]),
        "down_proj": lambda: torch.addmm(b_down16, y2, dp["W_down"].t(), out=lib_out["down_proj"]),
    }

    def full():
        _lib.mlstm_block_fwd(xd, bp, chunk=chunk, out=out, workspace=ws)

    return full, steps, library


def block_cpu_baseline(x, p, budget_tokens=512):
    """The float64 block oracle on the first tokens of the block workload,
    with the host's BLAS threads."""
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle.mlstm_block as ob
    n = host_threads()
    xs = x[:, :budget_tokens]
    with threadpool_limits(limits=n):
        t0 = time.perf_counter()
        ob.mlstm_block(xs, p)
        el = time.perf_counter() - t0
    used = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    return {"value": xs.shape[0] * xs.shape[1] / el, "unit": "tokens/s", "cores": min(n, used), "kind": "oracle",
            "sample": f"float64 NumPy block oracle (oracle/mlstm_block.py) on the first {xs.shape[1]} of "
                      f"{x.shape[1]} tokens at the full widths: {el:.2f} s",
            "cpu_model": cpu_model()}


# ---------------------------------------------------------------- host baseline

def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(x):
    """The float64 C oracle (one sequence per host thread) on the 7B-layer
    workload: all heads on as many threads as there are heads and host
    cores, and one head on one thread."""
    from oracle.mlstm_ref import mlstm_recurrent_c
    names = ("q", "k", "v", "i_pre", "f_pre", "o_pre")
    H, T = x["q"].shape[1], x["q"].shape[2]
    n = min(host_threads(), H)
    t0 = time.perf_counter()
    mlstm_recurrent_c(*[x[k] for k in names], threads=n)
    el_n = time.perf_counter() - t0
    one = {k: x[k][:, :1] for k in names}
    t0 = time.perf_counter()
    mlstm_recurrent_c(*[one[k] for k in names], threads=1)
    el_1 = time.perf_counter() - t0
    return {"value": T / el_n, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"float64 C step recurrence (oracle/mlstm_ref.c) over the whole 7B-layer workload "
                      f"(B=1 H={H} T={T}), one head per thread, {n} threads: {el_n:.2f} s",
            "one_core": {"value": T / H / el_1, "unit": "tokens/s", "cores": 1,
                         "sample": f"one of the {H} heads on one thread: {el_1:.2f} s"},
            "cpu_model": cpu_model(), "host_threads_available": host_threads()}


def slstm_cpu_baseline(pre, R, budget_s=6.0):
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


# ---------------------------------------------------------------- committed profiles

def sources_sha256():
    """sha256 over the HIP library's sources (sorted file names, contents)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def profile_figures(name):
    """Figures of a committed rocprofv3 summary under profiles/ (`key: value`
    lines), if it names the sha256 of the current library sources."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(1) != sources_sha256():
        return None
    out = {}
    for key in ("trace_avg_us", "traffic_bytes_per_launch"):
        mm = re.search(rf"{key}:\s*([0-9.eE+]+)", text)
        if mm:
            out[key] = float(mm.group(1))
    return out


def roofline(nbytes, flops, seconds, label):
    hbm = nbytes / seconds / HBM_PEAK
    mf = flops / seconds / MFMA_BF16_PEAK
    if mf > hbm:
        r = {"bound": "mfma", "achieved": flops / seconds / 1e12, "peak": MFMA_BF16_PEAK / 1e12,
             "unit": "TFLOP/s", "frac": mf}
    else:
        r = {"bound": "hbm", "achieved": nbytes / seconds / 1e9, "peak": HBM_PEAK / 1e9,
             "unit": "GB/s", "frac": hbm}
    return {"kernel": label, **r, "hbm_frac": hbm, "mfma_frac": mf,
            "algorithmic_bytes": nbytes, "algorithmic_flops": flops}


def measure_clock(torch, one, steps=20, iters=250):
    """Shader clock (MHz) while the chunkwise forward runs: a sleeping probe
    wave on a side stream (default priority) counts shader-clock ticks
    against constant-rate ticks; the constant counter's rate comes from an
    event-timed probe run alone, whose own clock is the idle figure."""
    from linear_recurrent_sequence_fwd_amd import _lib
    ticks = torch.zeros(4, dtype=torch.int64, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _lib.clock_probe(ticks, iters)
    e0.record()
    _lib.clock_probe(ticks, iters)
    e1.record()
    torch.cuda.synchronize()
    t = ticks.cpu().tolist()
    rt_mhz = (t[3] - t[2]) / (e0.elapsed_time(e1) * 1e3)
    idle_mhz = (t[1] - t[0]) / (t[3] - t[2]) * rt_mhz
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        _lib.clock_probe(ticks, iters)
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    t = ticks.cpu().tolist()
    return {"under_load_mhz": (t[1] - t[0]) / (t[3] - t[2]) * rt_mhz, "idle_mhz": idle_mhz,
            "realtime_counter_mhz": rt_mhz,
            "method": "s_memtime over s_memrealtime of one sleeping wave beside the forward calls"}


# ---------------------------------------------------------------- main

SECTIONS = ("sweep", "graph", "clock", "bwd", "block", "mid", "long", "segments", "decode", "slstm", "cpu")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="reps of the headline step")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--chunk", type=int, default=1024,
                    help="chunk length: the state is materialised at chunk starts (multiple of 64)")
    ap.add_argument("--sweep", type=str, default="64,256,512,2048", help="chunk sizes reported besides --chunk")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--bwd-chunk", type=int, default=256)
    ap.add_argument("--only", type=str, default="",
                    help="comma list of sections to run after the headline (" + ", ".join(SECTIONS) +
                         "); empty = all, 'none' = the headline alone")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only: this build of the mLSTM path is single-GPU "
              f"(--gpus {args.gpus} requested). Heads and batch shard with no exchange; the design "
              f"notes describe the multi-GPU plan.", file=sys.stderr)
        sys.exit(2)
    want = set(s for s in args.only.split(",") if s) or set(SECTIONS)

    import torch
    import linear_recurrent_sequence_fwd_amd as M
    from linear_recurrent_sequence_fwd_amd import _lib
    _lib.lib()
    ev = HipEvents()
    timer = Timer(torch, ev)
    cfg = WORKLOAD
    B, H, T, K, V = cfg["B"], cfg["H"], cfg["T"], cfg["d_qk"], cfg["d_v"]

    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        for _ in range(3):
            _lib.copy_lds(src, dst)
        torch.cuda.synchronize()
        assert bool(torch.equal(src, dst))
        log(f"[bench] calibration copies: {n} bytes read and written per launch, 3 plain copies and "
            f"3 direct-to-LDS copies")
        del src, dst

    log(f"[bench] inputs 7B-layer B={B} H={H} T={T} d_qk={K} d_v={V} bf16")
    x, d = make_device_inputs(torch, cfg, "bf16", seed=0)
    nbytes, flops = fwd_bytes(B, H, T, K, V), fwd_flops(B, H, T, K, V)

    # ---- headline: cold step, warm beside it, per-kernel groups
    log(f"[bench] chunkwise chunk={args.chunk}: {args.warmup} warmup, {args.steps} cold reps")
    one, prof = chunkwise_callables(torch, d, args.chunk)
    cold = timer.cold(one, args.steps, args.warmup)
    warm = timer.warm(one, args.steps, args.warmup)
    groups = timer.groups(prof, _lib.PROF_GROUPS, max(10, args.steps // 2), cold=True)
    groups_warm = timer.groups(prof, _lib.PROF_GROUPS, max(10, args.steps // 2), cold=False)
    ms_step = cold["median_ms"]
    tok_s = B * T / (ms_step * 1e-3)
    roof = roofline(nbytes, flops, groups["out"] * 1e-6, "out_kernel_fused")
    roof["timing"] = "median cold kernel duration from events around the launch"
    roof["kernel_us"] = groups["out"]
    roof["kernel_us_warm"] = groups_warm["out"]
    roof["frac_warm"] = nbytes / (groups_warm["out"] * 1e-6) / HBM_PEAK
    pf = profile_figures("fused_kernel_7b_layer.md") or {}
    roof["trace_us"] = pf.get("trace_avg_us")
    roof["frac_trace"] = nbytes / (pf["trace_avg_us"] * 1e-6) / HBM_PEAK if "trace_avg_us" in pf else None
    roof["traffic"] = pf.get("traffic_bytes_per_launch")
    log(f"[bench] cold {ms_step:.3f} ms/step (warm {warm['wall_ms']:.3f}), {tok_s:.3e} tokens/s, "
        f"kernels us cold {groups} warm {groups_warm}")

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
                   "inputs": "bf16 q/k/v/o, fp32 gates", "parallelism": "single GPU"},
        "timing": {"cold": cold, "warm": warm,
                   "protocol": "cold: 512 MiB scratch overwrite before each rep, events around the step; "
                               "warm: back-to-back steps"},
        "mfma_frac": flops / (ms_step * 1e-3) / MFMA_BF16_PEAK,
        "hbm_frac_step": nbytes / (ms_step * 1e-3) / HBM_PEAK,
        "kernel_us": {LABELS[k]: v for k, v in groups.items()},
        "kernel_us_warm": {LABELS[k]: v for k, v in groups_warm.items()},
        "roofline": roof,
    }

    if "sweep" in want:
        sweep = {}
        for L in [int(s) for s in args.sweep.split(",") if s]:
            if L == args.chunk:
                continue
            o, p = chunkwise_callables(torch, d, L)
            c = timer.cold(o, max(10, args.steps // 3), 2)
            g = timer.groups(p, _lib.PROF_GROUPS, 10, cold=True)
            sweep[str(L)] = {"ms_per_step": c["median_ms"], "tokens_per_s": B * T / (c["median_ms"] * 1e-3),
                             "mfma_frac": flops / (c["median_ms"] * 1e-3) / MFMA_BF16_PEAK,
                             "kernel_us": {LABELS[k]: v for k, v in g.items()}}
            log(f"[bench] sweep chunk={L}: {c['median_ms']:.3f} ms/step cold")
        out["sweep"] = sweep

    if "graph" in want:
        out["graph_ms_per_step"] = graph_ms(torch, d, args.chunk, args.steps, args.warmup)
        log(f"[bench] chunkwise as a replayed HIP graph: {out['graph_ms_per_step']:.3f} ms/step (warm)")

    if "clock" in want:
        out["clock"] = measure_clock(torch, one)
        log(f"[bench] shader clock during the forward: {out['clock']['under_load_mhz']:.0f} MHz")

    if "bwd" in want:
        log(f"[bench] backward chunk={args.bwd_chunk}")
        o, p = backward_callables(torch, d, args.bwd_chunk)
        c = timer.cold(o, max(10, args.steps // 3), 2)
        g = timer.groups(p, _lib.BWD_PROF_GROUPS, 10, cold=True)
        bb, bf = bwd_bytes(B, H, T, K, V), bwd_flops(B, H, T, K, V)
        dom = max(g, key=g.get)
        out["backward"] = {
            "workload": f"mlstm_bwd_chunkwise, 7B-layer shape, chunk {args.bwd_chunk}, bf16",
            "ms_per_step": c["median_ms"], "tokens_per_s": B * T / (c["median_ms"] * 1e-3),
            "kernel_us": {BWD_LABELS[k]: v for k, v in g.items()},
            "dominant_kernel": BWD_LABELS[dom],
            "roofline": roofline(bb, bf, c["median_ms"] * 1e-3, "whole backward pass")}
        log(f"[bench] backward {c['median_ms']:.3f} ms cold, kernels {g}")
        del o, p

    del d, one, prof
    torch.cuda.empty_cache()

    if "block" in want:
        bc = BLOCK
        log(f"[bench] block B={bc['B']} T={bc['T']} D={bc['D']} H={bc['H']} d_qk={bc['d_qk']} d_v={bc['d_v']} "
            f"chunk={bc['chunk']}")
        bx, bpar, bdp, bbp, bxd = block_setup(torch, bc, seed=1)
        full, bsteps, blib = block_callables(torch, bc, bpar, bdp, bbp, bxd)
        c = timer.cold(full, max(10, args.steps // 3), 2)
        w = timer.warm(full, max(10, args.steps // 3), 2)
        work = block_work(bc)
        per = {}
        for name, fn in bsteps.items():
            r = timer.cold(fn, 10, 2)
            fl, by = work[name]
            sec = r["median_ms"] * 1e-3
            per[name] = {"us": r["median_ms"] * 1e3, "tflops": fl / sec / 1e12, "GBps": by / sec / 1e9,
                         "mfma_frac": fl / sec / MFMA_BF16_PEAK, "hbm_frac": by / sec / HBM_PEAK}
        ref = {}
        for name, fn in blib.items():
            r = timer.cold(fn, 10, 2)
            fl, _ = work[name]
            ref[name] = {"us": r["median_ms"] * 1e3, "mfma_frac": fl / (r["median_ms"] * 1e-3) / MFMA_BF16_PEAK}
        tot_fl = sum(v[0] for v in work.values())
        dom = max(per, key=lambda k: per[k]["us"])
        fl, by = work[dom]
        sec = per[dom]["us"] * 1e-6
        gemm = dom.endswith("_proj")
        out["block"] = {
            "workload": f"mLSTM pre-up-projection block B={bc['B']} T={bc['T']} D={bc['D']} (E={2 * bc['D']}) "
                        f"H={bc['H']} d_qk={bc['d_qk']} d_v={bc['d_v']} KC={bc['KC']}, cell chunk {bc['chunk']}, bf16",
            "ms_per_step": c["median_ms"], "ms_per_step_warm": w["median_ms"],
            "tokens_per_s": bc["B"] * bc["T"] / (c["median_ms"] * 1e-3),
            "mfma_frac": tot_fl / (c["median_ms"] * 1e-3) / MFMA_BF16_PEAK,
            "steps_us": per, "library_reference_us": ref, "dominant_step": dom,
            "roofline": {"kernel": dom, "bound": "mfma" if gemm else "hbm",
                         "achieved": fl / sec / 1e12 if gemm else by / sec / 1e9,
                         "peak": MFMA_BF16_PEAK / 1e12 if gemm else HBM_PEAK / 1e9,
                         "unit": "TFLOP/s" if gemm else "GB/s",
                         "frac": fl / sec / MFMA_BF16_PEAK if gemm else by / sec / HBM_PEAK,
                         "traffic": None},
        }
        log(f"[bench] block {c['median_ms']:.3f} ms cold ({w['median_ms']:.3f} warm); steps us "
            + ", ".join(f"{k} {v['us']:.1f}" for k, v in per.items())
            + "; library " + ", ".join(f"{k} {v['us']:.1f}" for k, v in ref.items()))
        if "cpu" in want:
            out["block"]["cpu_baseline"] = block_cpu_baseline(bx, bpar)
        del full, bsteps, blib, bdp, bbp, bxd
        torch.cuda.empty_cache()

    if "mid" in want:
        log("[bench] mid workload")
        mc = MID
        _, dm = make_device_inputs(torch, mc, "bf16", seed=0)
        mb, mf = fwd_bytes(mc["B"], mc["H"], mc["T"], mc["d_qk"], mc["d_v"]), \
            fwd_flops(mc["B"], mc["H"], mc["T"], mc["d_qk"], mc["d_v"])
        res = {"workload": "mLSTM fwd B=4 H=8 T=2048 d_qk=d_v=128 bf16"}
        for L in (64, 256):
            o, _ = chunkwise_callables(torch, dm, L)
            c = timer.cold(o, 20, 2)
            res[f"chunkwise_{L}"] = {"ms_per_step": c["median_ms"],
                                     "tokens_per_s": mc["B"] * mc["T"] / (c["median_ms"] * 1e-3),
                                     "hbm_frac": mb / (c["median_ms"] * 1e-3) / HBM_PEAK,
                                     "mfma_frac": mf / (c["median_ms"] * 1e-3) / MFMA_BF16_PEAK}
        o = parallel_callable(torch, dm)
        c = timer.cold(o, 20, 2)
        res["parallel"] = {"ms_per_step": c["median_ms"],
                           "tokens_per_s": mc["B"] * mc["T"] / (c["median_ms"] * 1e-3),
                           "hbm_frac": mb / (c["median_ms"] * 1e-3) / HBM_PEAK}
        out["mid"] = res
        log(f"[bench] mid {res}")
        del dm, o
        torch.cuda.empty_cache()

    if "long" in want:
        log("[bench] long-context workload")
        lc = LONG
        _, dl = make_device_inputs(torch, lc, "bf16", seed=0)
        lb, lf = fwd_bytes(lc["B"], lc["H"], lc["T"], lc["d_qk"], lc["d_v"]), \
            fwd_flops(lc["B"], lc["H"], lc["T"], lc["d_qk"], lc["d_v"])
        res = {"workload": "mLSTM fwd B=1 H=8 T=131072 d_qk=256 d_v=512 bf16", "algorithmic_bytes": lb}
        for L in (64, 256, 1024):
            o, p = chunkwise_callables(torch, dl, L)
            c = timer.cold(o, 10, 2)
            g = timer.groups(p, _lib.PROF_GROUPS, 5, cold=True)
            res[f"chunk_{L}"] = {"ms_per_step": c["median_ms"],
                                 "tokens_per_s": lc["B"] * lc["T"] / (c["median_ms"] * 1e-3),
                                 "hbm_frac": lb / (c["median_ms"] * 1e-3) / HBM_PEAK,
                                 "mfma_frac": lf / (c["median_ms"] * 1e-3) / MFMA_BF16_PEAK,
                                 "kernel_us": {LABELS[k]: v for k, v in g.items()}}
            log(f"[bench] long context chunk={L}: {c['median_ms']:.3f} ms cold")
            del o, p
        out["long_context"] = res
        del dl
        torch.cuda.empty_cache()

    if "segments" in want:
        sc = SEGMENTS
        P, L = sc["parts"], sc["chunk"]
        log(f"[bench] segments: one device's share of T={sc['T'] * P} over {P} devices, "
            f"B={sc['B']} H={sc['H']} T={sc['T']} chunk={L}")
        _, ds = make_device_inputs(torch, sc, seed=7)
        summary, combine, forward = segment_callables(torch, ds, L, P)
        Bq, Hq, Tq, Kq, Vq = sc["B"], sc["H"], sc["T"], sc["d_qk"], sc["d_v"]
        t_sum = timer.cold(summary, 20, 2)["median_ms"]
        t_comb = timer.cold(combine, 20, 2)["median_ms"]
        t_fwd = timer.cold(forward, 20, 2)["median_ms"]
        state_bytes = Bq * Hq * (Vq * Kq + Kq + 1) * 4 + Bq * Hq * 8
        sum_bytes = Bq * Hq * Tq * ((Kq + Vq) * 2 + 8) + state_bytes   # k, v, two gates in; the summary out
        total = t_sum + t_comb + t_fwd
        out["segments"] = {
            "workload": f"one of {P} segments of the long-context sequence: B={Bq} H={Hq} T={Tq} d_qk={Kq} "
                        f"d_v={Vq} bf16, chunk {L}",
            "summary_ms": t_sum, "fold_ms": t_comb, "forward_from_start_ms": t_fwd,
            "device_ms": total, "summaries_folded": P - 1,
            "overhead_vs_forward": (total - t_fwd) / t_fwd,
            "summary_bytes": state_bytes,
            "summary_hbm_frac": sum_bytes / (t_sum * 1e-3) / HBM_PEAK,
            "fold_GBps": (P + 1) * state_bytes / (t_comb * 1e-3) / 1e9,
            "tokens_per_s_per_device": Bq * Tq / (total * 1e-3),
            "timing": "cold medians; the exchange of summaries between devices is not measured (one GPU)",
        }
        log(f"[bench] segments: summary {t_sum:.3f} ms, fold of {P - 1} summaries {t_comb * 1e3:.1f} us, "
            f"forward from the start state {t_fwd:.3f} ms")
        del summary, combine, forward, ds
        torch.cuda.empty_cache()

    if "decode" in want:
        log(f"[bench] decode B={DECODE['B']} H={DECODE['H']} steps {args.decode_steps}")
        wall_us, k_us = time_decode(torch, M, timer, args.decode_steps, 20)
        db = decode_bytes(DECODE["B"], DECODE["H"], DECODE["d_qk"], DECODE["d_v"])
        out["decode"] = {"workload": "mlstm_step B=64 H=8 d_qk=256 d_v=512 fp32 state",
                         "steps": args.decode_steps, "us_per_step": wall_us, "kernel_us": k_us,
                         "tokens_per_s": DECODE["B"] / (wall_us * 1e-6),
                         "achieved_GBps": db / (k_us * 1e-6) / 1e9,
                         "hbm_frac": db / (k_us * 1e-6) / HBM_PEAK,
                         "hbm_frac_wall": db / (wall_us * 1e-6) / HBM_PEAK}
        log(f"[bench] decode {wall_us:.1f} us/step wall, kernel {k_us:.1f} us")

    if "slstm" in want:
        Bs, Hs, Ts, Ds = SLSTM["B"], SLSTM["H"], SLSTM["T"], SLSTM["D"]
        log(f"[bench] sLSTM B={Bs} H={Hs} T={Ts} D={Ds}")
        sec, pre, R = time_slstm(torch, timer, 10)
        fl = slstm_flops(Bs, Hs, Ts, Ds)
        out["slstm"] = {"workload": f"slstm_fwd B={Bs} H={Hs} D={Ds} T={Ts} float32",
                        "ms_per_call": sec * 1e3, "us_per_step": sec / Ts * 1e6,
                        "tokens_per_s": Bs * Ts / sec,
                        "roofline": {"bound": "alu", "achieved": fl / sec / 1e12, "peak": FP32_PEAK / 1e12,
                                     "unit": "TFLOP/s", "frac": fl / sec / FP32_PEAK,
                                     "note": "whole-chip float32 vector peak; the launch occupies "
                                             f"{Bs * Hs} of 256 CUs"}}
        if "cpu" in want:
            out["slstm"]["cpu_baseline"] = slstm_cpu_baseline(pre, R)

    if "cpu" in want:
        log("[bench] cpu baseline (C oracle)")
        out["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
