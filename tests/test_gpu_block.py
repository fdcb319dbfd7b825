"""Parity of the mLSTM block's HIP path (include/mlstm_block.h) with the
float64 oracle (oracle/mlstm_block.py), through the C ABI.

Each step is compared with the oracle's step applied to the GPU's own input
to that step (the intermediates the block returns), element by element,
under a bound derived from the step's arithmetic:
  * bf16 outputs carry one rounding, at most 2^-8 of the value (U below);
  * float32 dot products of length K differ from exact by at most
    K 2^-24 sum |a_k b_k| (the float32 accumulation bound);
  * float32 statistics and the hardware exponential add about 1e-5 of the
    terms' size.
The whole block is also compared with the pure float64 oracle (no
intermediate rounding) at 2e-2 of the largest change the block makes to its
input, the bf16 bar of the cell applied to the block's increment; and the
fused entry point is checked bit for bit against its steps run one by one.
"""
import math

import numpy as np
import pytest
import torch

import linear_recurrent_sequence_fwd_amd as M
from linear_recurrent_sequence_fwd_amd import _lib as L
from linear_recurrent_sequence_fwd_amd.inputs import make_block_inputs, make_fwd_inputs
import oracle.mlstm_block as ob
from oracle.mlstm_oracle import mlstm_rows

pytestmark = pytest.mark.gpu

U = 2.0 ** -8        # bf16 unit roundoff
U32 = 2.0 ** -24     # float32 unit roundoff
DEV = "cuda:0"


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def within(got, ref, bound, what):
    err = np.abs(got - ref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements outside the bound; "
                           f"worst error {float(err.max()):.3e}, worst excess {float(np.max(err - bound)):.3e}")
    return float(err.max())


def dev_params(p):
    out = {}
    for name, is_mat in L.BLOCK_ARRAYS:
        a = torch.from_numpy(np.ascontiguousarray(p[name], dtype=np.float32))
        out[name] = a.to(DEV, torch.bfloat16) if is_mat else a.to(DEV)
    return out


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV, torch.bfloat16)


# ------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("Mm,N,K,out,trans,resid", [
    (300, 200, 192, "bf16", False, True),     # ragged rows and columns, residual
    (257, 260, 64, "fp32", False, False),     # one row past a tile, a column tile of 4
    (512, 96, 128, "fp32", True, False),      # transposed store
    (64, 1024, 1024, "bf16", False, False),
])
def test_gemm_parity(Mm, N, K, out, trans, resid):
    rng = np.random.default_rng(Mm * 7 + N)
    A = L_round(rng.standard_normal((Mm, K)))
    B = L_round(rng.standard_normal((N, K)) / math.sqrt(K))
    bias = rng.standard_normal(N).astype(np.float32)
    R = L_round(rng.standard_normal((Mm, N))) if resid else None
    alpha = 0.7
    C = M.gemm_bf16(bf16_dev(A), bf16_dev(B), torch.from_numpy(bias).to(DEV),
                    bf16_dev(R) if resid else None, alpha=alpha,
                    out_dtype=torch.bfloat16 if out == "bf16" else torch.float32, c_trans=trans)
    torch.cuda.synchronize()
    ref = alpha * (A.astype(np.float64) @ B.astype(np.float64).T) + bias
    if resid:
        ref = ref + R
    absdot = alpha * (np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)).T)
    bound = K * U32 * absdot + 4 * U32 * (np.abs(ref) + np.abs(bias) + (np.abs(R) if resid else 0))
    if out == "bf16":
        bound = bound + U * np.abs(ref) * 1.0001
    got = f64(C)
    within(got.T if trans else got, ref, bound, "gemm")


def L_round(x):
    from linear_recurrent_sequence_fwd_amd.inputs import bf16_round
    return bf16_round(np.asarray(x, dtype=np.float32))


def test_gemm_strided_batch_is_per_head_projection():
    """Batched over (batch entry, head): head h of entry b reads columns
    [h n_in, (h + 1) n_in) of its rows and writes [b][h][T][n_out]."""
    rng = np.random.default_rng(21)
    Bn, H, T, n_in, n_out = 2, 3, 200, 128, 64
    x = L_round(rng.standard_normal((Bn, T, H * n_in)))
    W = L_round(rng.standard_normal((H, n_out, n_in)) / math.sqrt(n_in))
    bias = rng.standard_normal(H * n_out).astype(np.float32)
    xd, Wd = bf16_dev(x), bf16_dev(W)
    C = torch.empty((Bn, H, T, n_out), dtype=torch.bfloat16, device=DEV)
    M.gemm_bf16_strided(T, n_out, n_in, Bn, H, xd, H * n_in, T * H * n_in, n_in, Wd, n_in, 0, n_out * n_in,
                        C, n_out, H * T * n_out, T * n_out, alpha=0.5, bias=torch.from_numpy(bias).to(DEV),
                        stride_bias2=n_out)
    torch.cuda.synchronize()
    got = f64(C)
    for b in range(Bn):
        ref = ob.block_diag_proj(x[b], W, bias, scale=0.5)            # [T, H n_out]
        absdot = 0.5 * np.concatenate([np.abs(x[b][:, h * n_in:(h + 1) * n_in].astype(np.float64))
                                       @ np.abs(W[h].astype(np.float64)).T for h in range(H)], axis=1)
        bound = U * np.abs(ref) * 1.0001 + n_in * U32 * absdot + 4 * U32 * (np.abs(ref) + np.abs(bias))
        within(got[b].transpose(1, 0, 2).reshape(T, H * n_out), ref, bound, f"batch entry {b}")


def test_gemm_full_size_up_projection_sampled_rows():
    """The block workload's up-projection (8192 x 8192 x 2048) in the launch
    configuration the block uses; 96 sampled rows (every column) against float64."""
    rng = np.random.default_rng(22)
    Mm, N, K = 8192, 8192, 2048
    A = L_round(rng.standard_normal((Mm, K), dtype=np.float32))
    B = L_round(rng.standard_normal((N, K), dtype=np.float32) / np.float32(math.sqrt(K)))
    bias = (0.1 * rng.standard_normal(N)).astype(np.float32)
    C = M.gemm_bf16(bf16_dev(A), bf16_dev(B), torch.from_numpy(bias).to(DEV))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([rng.integers(0, Mm, 90), [0, 255, 256, 4095, 8190, 8191]]))
    Ar = A[rows].astype(np.float64)
    ref = Ar @ B.astype(np.float64).T + bias
    bound = U * np.abs(ref) * 1.0001 + K * U32 * (np.abs(Ar) @ np.abs(B.astype(np.float64)).T) \
        + 4 * U32 * (np.abs(ref) + np.abs(bias))
    within(f64(C[torch.from_numpy(rows).to(DEV)]), ref, bound, "up-projection rows")
    assert torch.isfinite(C).all()


# ------------------------------------------------------------------ layer norm

@pytest.mark.parametrize("rows,D", [(37, 256), (300, 2048), (5, 8), (64, 8192)])
def test_layernorm_parity(rows, D):
    rng = np.random.default_rng(rows + D)
    x = L_round(rng.standard_normal((rows, D)) * 2.0 + 0.5)
    w = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    b = (0.1 * rng.standard_normal(D)).astype(np.float32)
    y = M.layernorm_bf16(bf16_dev(x), torch.from_numpy(w).to(DEV), torch.from_numpy(b).to(DEV), 1e-5)
    torch.cuda.synchronize()
    ref = ob.layer_norm(x, w, b, 1e-5)
    norm = np.abs(ob.layer_norm(x, np.ones(D), np.zeros(D), 1e-5)) * np.abs(w)
    within(f64(y), ref, U * np.abs(ref) * 1.0001 + 1e-5 * (norm + np.abs(b)) + 1e-6, "layer norm")


# ------------------------------------------------------------------ the ungated cell

@pytest.mark.parametrize("T,dqk,dv,chunk", [(300, 64, 128, 128), (1000, 128, 256, 256), (1, 64, 128, 64)])
def test_ungated_cell_parity(T, dqk, dv, chunk):
    x = make_fwd_inputs(1, 2, T, dqk, dv, "bf16", seed=T)
    d = {n: torch.from_numpy(x[n]).to(DEV, torch.bfloat16) for n in ("q", "k", "v")}
    ip = torch.from_numpy(x["i_pre"]).to(DEV)
    fp = torch.from_numpy(x["f_pre"]).to(DEV)
    h = M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], None, ip, fp, chunk=chunk)
    torch.cuda.synchronize()
    tr = lambda a: np.moveaxis(a[0], 0, 1)   # [1, H, T, d] -> [T, H, d]
    ref = ob.cell_ungated(tr(x["q"]), tr(x["k"]), tr(x["v"]), x["i_pre"][0].T, x["f_pre"][0].T)
    got = np.moveaxis(f64(h)[0], 0, 1)
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err <= 2e-2, err


# ------------------------------------------------------------------ the block

CONFIGS = {
    # B, T, D, H, d_qk, d_v, KC, chunk
    "tiny": (2, 300, 256, 4, 64, 128, 4, 64),
    "mid": (2, 1000, 512, 8, 64, 128, 4, 256),
    "one_token": (3, 1, 256, 4, 64, 128, 4, 64),
    "short_conv": (1, 77, 256, 2, 128, 256, 2, 128),
    "many_heads": (1, 100, 1024, 16, 64, 128, 3, 64),    # 32 gates: two 16-gate MFMA blocks
}


def run_block(cfg, seed=0):
    B, T, D, H, dqk, dv, KC, chunk = cfg
    x, p = make_block_inputs(B, T, D, H, dqk, dv, KC=KC, seed=seed)
    dp = dev_params(p)
    bp = M.block_params(dp, D, H, dqk, dv, KC, p["eps_ln"], p["eps_gn"])
    xd = bf16_dev(x)
    out, st = M.mlstm_block_fwd(xd, bp, chunk=chunk, return_stages=True)
    torch.cuda.synchronize()
    return x, p, dp, bp, xd, out, st


def check_stages(x, p, st, cfg, what):
    """Every step against the oracle's step on the GPU's input to it."""
    B, T, D, H, dqk, dv, KC, chunk = cfg
    E = 2 * D
    g = {n: f64(t) for n, t in st.items()}
    for b in range(B):
        # layer norm
        ref = ob.layer_norm(x[b], p["ln_w"], p["ln_b"], p["eps_ln"])
        norm = np.abs(ob.layer_norm(x[b], np.ones(D), np.zeros(D), p["eps_ln"])) * np.abs(p["ln_w"])
        within(g["xn"][b], ref, U * np.abs(ref) * 1.0001 + 1e-5 * (norm + np.abs(p["ln_b"])) + 1e-6, f"{what} xn")
        # up-projection from the GPU's xn
        xn = g["xn"][b]
        Wup = p["W_up"].astype(np.float64)
        ref = xn @ Wup.T + p["b_up"]
        bound = U * np.abs(ref) * 1.0001 + D * U32 * (np.abs(xn) @ np.abs(Wup).T) + 4 * U32 * np.abs(p["b_up"])
        within(g["xup"][b], ref, bound, f"{what} xup")
        # conv + Swish from the GPU's xm; the gates from the GPU's xc
        xm, z = g["xup"][b][:, :E], g["xup"][b][:, E:]
        conv = ob.causal_conv(xm, p["conv_w"], p["conv_b"])
        ref = ob.swish(conv)
        aconv = ob.causal_conv(np.abs(xm), np.abs(p["conv_w"]), np.abs(p["conv_b"]))
        within(g["xc"][b], ref, U * np.abs(ref) * 1.0001 + 1e-5 * aconv + 1e-6, f"{what} xc")
        xc = g["xc"][b]
        for name, w, bias in (("i_pre", p["w_i"], p["b_i"]), ("f_pre", p["w_f"], p["b_f"])):
            ref = xc @ w.astype(np.float64).T + bias
            bound = E * U32 * (np.abs(xc) @ np.abs(w.astype(np.float64)).T) + 4 * U32 * np.abs(ref) + 1e-6
            within(g[name][b].T, ref, bound, f"{what} {name}")
        # per-head projections from the GPU's xc / xm
        n_in = E // H
        for name, src, W, bias, scale, n_out in (("q", xc, p["W_q"], p["b_q"], 1.0, dqk),
                                                 ("k", xc, p["W_k"], p["b_k"], 1 / math.sqrt(dqk), dqk),
                                                 ("v", xm, p["W_v"], p["b_v"], 1.0, dv)):
            ref = ob.block_diag_proj(src, W, bias, scale=scale).reshape(T, H, n_out)
            absd = np.stack([np.abs(src[:, h * n_in:(h + 1) * n_in]) @ np.abs(W[h].astype(np.float64)).T
                             for h in range(H)], axis=1) * scale
            bound = U * np.abs(ref) * 1.0001 + n_in * U32 * absd + 4 * U32 * np.abs(bias).reshape(H, n_out)
            within(g[name][b].transpose(1, 0, 2), ref, bound, f"{what} {name}")
        # the cell from the GPU's q, k, v, gates (the cell's own bf16 bar)
        tq = lambda a: a.transpose(1, 0, 2)
        ref = ob.cell_ungated(tq(g["q"][b]), tq(g["k"][b]), tq(g["v"][b]), g["i_pre"][b].T, g["f_pre"][b].T)
        got = tq(g["h"][b])
        assert np.isfinite(got).all()
        err = np.abs(got - ref).max() / np.abs(ref).max()
        assert err <= 2e-2, f"{what} cell {err}"
        # group norm + skip + gate from the GPU's h, xc, z
        hh = g["h"][b].transpose(1, 0, 2)
        gn = ob.group_norm(hh, p["gn_w"], p["gn_b"], p["eps_gn"])
        sg = ob.sigmoid(z)
        ref = (gn + p["skip"] * xc) * sg
        size = (np.abs(gn) + np.abs(p["gn_b"]) + np.abs(p["skip"] * xc)) * sg
        within(g["y"][b], ref, U * np.abs(ref) * 1.0001 + 2e-5 * size + 1e-6, f"{what} y")


@pytest.mark.parametrize("name", list(CONFIGS))
def test_block_steps_against_the_oracle(name):
    cfg = CONFIGS[name]
    x, p, dp, bp, xd, out, st = run_block(cfg, seed=3)
    check_stages(x, p, st, cfg, name)
    # the down-projection and residual from the GPU's y
    B, T, D = x.shape
    E = 2 * D
    got = f64(out)
    Wd = p["W_down"].astype(np.float64)
    for b in range(B):
        y = f64(st["y"])[b]
        ref = x[b] + y @ Wd.T + p["b_down"]
        bound = U * np.abs(ref) * 1.0001 + E * U32 * (np.abs(y) @ np.abs(Wd).T) \
            + 4 * U32 * (np.abs(x[b]) + np.abs(p["b_down"]))
        within(got[b], ref, bound, f"{name} out")


@pytest.mark.parametrize("name", ["tiny", "mid", "one_token"])
def test_block_against_the_float64_oracle(name):
    """End to end, no intermediate rounding on the oracle's side: within 2e-2
    of the largest change the block makes to its input."""
    cfg = CONFIGS[name]
    x, p, dp, bp, xd, out, st = run_block(cfg, seed=4)
    ref = ob.mlstm_block(x, p)
    got = f64(out)
    assert np.isfinite(got).all()
    scale = np.abs(ref - x).max()
    err = np.abs(got - ref).max() / scale
    assert err <= 2e-2, err


def test_block_is_its_steps_in_order():
    """mlstm_block_fwd gives bit for bit what its steps give when called one by one."""
    cfg = CONFIGS["tiny"]
    B, T, D, H, dqk, dv, KC, chunk = cfg
    E, n_in = 2 * D, 2 * D // H
    x, p, dp, bp, xd, out, st = run_block(cfg, seed=5)
    xn = M.layernorm_bf16(xd, dp["ln_w"], dp["ln_b"], p["eps_ln"])
    xup = M.gemm_bf16(xn.view(B * T, D), dp["W_up"].view(2 * E, D), dp["b_up"]).view(B, T, 2 * E)
    xc, ip, fp = M.block_conv_gates(bp, xup)

    def proj(src, ld, W, n_out, bias, alpha):
        C = torch.empty((B, H, T, n_out), dtype=torch.bfloat16, device=DEV)
        return M.gemm_bf16_strided(T, n_out, n_in, B, H, src, ld, T * ld, n_in, W, n_in, 0, n_out * n_in,
                                   C, n_out, H * T * n_out, T * n_out, alpha=alpha, bias=bias, stride_bias2=n_out)
    q = proj(xc, E, dp["W_q"], dqk, dp["b_q"], 1.0)
    k = proj(xc, E, dp["W_k"], dqk, dp["b_k"], float(np.float32(1.0 / math.sqrt(dqk))))
    v = proj(xup, 2 * E, dp["W_v"], dv, dp["b_v"], 1.0)
    h = M.mlstm_fwd_chunkwise(q, k, v, None, ip, fp, chunk=chunk)
    y = M.block_groupnorm_gate(bp, h, xc, xup)
    o = M.gemm_bf16(y.view(B * T, E), dp["W_down"], dp["b_down"], R=xd.view(B * T, D)).view(B, T, D)
    torch.cuda.synchronize()
    for name, t in (("xn", xn), ("xup", xup), ("xc", xc), ("i_pre", ip), ("f_pre", fp), ("q", q), ("k", k),
                    ("v", v), ("h", h), ("y", y)):
        assert torch.equal(t, st[name]), name
    assert torch.equal(o, out)


def test_block_batch_entries_do_not_mix():
    """The conv's first taps of entry b read zeros, not entry b - 1's last rows."""
    cfg = CONFIGS["tiny"]
    x, p, dp, bp, xd, out, st = run_block(cfg, seed=6)
    B, T, D, H, dqk, dv, KC, chunk = cfg
    bp1 = M.block_params(dp, D, H, dqk, dv, KC, p["eps_ln"], p["eps_gn"])
    out1 = M.mlstm_block_fwd(xd[1:].contiguous(), bp1, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(out1, out[1:])


def test_block_full_size_sampled():
    """The block workload (B = 1, T = 8192, D = 2048, H = 8, d_qk = 256,
    d_v = 512, chunk 256) in the launch configuration the bench times: every
    step on sampled tokens against the oracle's step on the GPU's inputs, the
    cell's rows from the parallel form."""
    B, T, D, H, dqk, dv, KC, chunk = 1, 8192, 2048, 8, 256, 512, 4, 256
    E, n_in = 2 * D, 2 * D // H
    x, p, dp, bp, xd, out, st = run_block((B, T, D, H, dqk, dv, KC, chunk), seed=7)
    rng = np.random.default_rng(8)
    rows = np.unique(np.concatenate([rng.integers(0, T, 20), [0, 1, 2, 3, 63, 64, 255, 256, 4096, T - 1]]))
    R = torch.from_numpy(rows).to(DEV)
    sel = lambda t, axis=1: f64(t.index_select(axis, R))
    xn = sel(st["xn"])[0]
    ref = ob.layer_norm(x[0][rows], p["ln_w"], p["ln_b"], p["eps_ln"])
    within(xn, ref, U * np.abs(ref) * 1.0001 + 1e-5 * (np.abs(ref) + 1) + 1e-6, "xn")
    xup = sel(st["xup"])[0]
    Wup = p["W_up"].astype(np.float64)
    ref = xn @ Wup.T + p["b_up"]
    within(xup, ref, U * np.abs(ref) * 1.0001 + D * U32 * (np.abs(xn) @ np.abs(Wup).T) + 1e-6, "xup")
    # conv: rows t - KC + 1 .. t of the GPU's xm
    xm_all = st["xup"][0, :, :E]
    xc = sel(st["xc"])[0]
    for j, t in enumerate(rows):
        lo = max(0, t - KC + 1)
        xm = f64(xm_all[lo:t + 1])
        conv = ob.causal_conv(xm, p["conv_w"], p["conv_b"])[-1]
        ref = ob.swish(conv)
        within(xc[j], ref, U * np.abs(ref) * 1.0001 + 1e-5 * (np.abs(conv) + 1) + 1e-6, f"xc row {t}")
    for name, w, bias in (("i_pre", p["w_i"], p["b_i"]), ("f_pre", p["w_f"], p["b_f"])):
        ref = xc @ w.astype(np.float64).T + bias
        got = f64(st[name][0][:, R]).T
        within(got, ref, E * U32 * (np.abs(xc) @ np.abs(w.astype(np.float64)).T) + 1e-5, name)
    # the cell at the sampled rows, from the GPU's full q, k, v and gates (parallel form)
    q, k, v = (f64(st[n])[0] for n in ("q", "k", "v"))
    ip, fp = f64(st["i_pre"])[0], f64(st["f_pre"])[0]
    ref = mlstm_rows(q, k, v, ip, fp, np.broadcast_to(np.inf, (H, T, dv)), rows)   # [H, rows, dv]
    got = f64(st["h"][0][:, R])
    assert np.isfinite(got).all()
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err <= 2e-2, err
    # group norm + gate and the down-projection at the rows
    z = xup[:, E:]
    gn = ob.group_norm(got.transpose(1, 0, 2), p["gn_w"], p["gn_b"], p["eps_gn"])
    ref = (gn + p["skip"] * xc) * ob.sigmoid(z)
    y = sel(st["y"])[0]
    size = (np.abs(gn) + np.abs(p["gn_b"]) + np.abs(p["skip"] * xc)) * ob.sigmoid(z)
    within(y, ref, U * np.abs(ref) * 1.0001 + 2e-5 * size + 1e-6, "y")
    Wd = p["W_down"].astype(np.float64)
    ref = x[0][rows] + y @ Wd.T + p["b_down"]
    got = sel(out)[0]
    within(got, ref, U * np.abs(ref) * 1.0001 + E * U32 * (np.abs(y) @ np.abs(Wd).T) + 1e-6, "out")
    assert torch.isfinite(out).all()


def test_block_empty_sequence():
    cfg = CONFIGS["tiny"]
    B, T, D, H, dqk, dv, KC, chunk = cfg
    x, p = make_block_inputs(B, 1, D, H, dqk, dv, KC=KC, seed=9)
    dp = dev_params(p)
    bp = M.block_params(dp, D, H, dqk, dv, KC, p["eps_ln"], p["eps_gn"])
    xd = torch.empty((B, 0, D), dtype=torch.bfloat16, device=DEV)
    out = torch.empty_like(xd)
    assert L.lib().mlstm_block_fwd(L.ctypes.byref(bp), B, 0, None, None, chunk, None, 0, None) == 0
    assert out.numel() == 0
