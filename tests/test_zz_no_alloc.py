"""The no-allocation chunkwise entry point against the workspace one.

mlstm_fwd_chunkwise_noalloc runs the same kernels as mlstm_fwd_chunkwise on
the library's fixed per-device scratch instead of a caller workspace, so its
outputs must equal the workspace call's bit for bit. Two calls in a row, the
second on a smaller problem (the scratch keeps the first call's contents),
each also checked against the float64 oracle at the bf16 bar.
"""
import sys

import numpy as np
import pytest

from linear_recurrent_sequence_fwd_amd.inputs import make_fwd_inputs
from oracle.mlstm_ref import mlstm_recurrent_c

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "i_pre", "f_pre", "o_pre")


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _dev(x):
    d = {n: torch.from_numpy(np.ascontiguousarray(x[n])).cuda().to(torch.bfloat16)
         for n in ("q", "k", "v", "o_pre")}
    for n in ("i_pre", "f_pre"):
        d[n] = torch.from_numpy(np.ascontiguousarray(x[n])).cuda()
    return d


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("shape", [[(1, 4, 1500, 256, 512, 256), (2, 1, 300, 128, 256, 128)]])
def test_noalloc_matches_workspace_entry_point(shape):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_recurrent_sequence_fwd_amd as M
    for call, (B, H, T, K, V, chunk) in enumerate(shape):
        say(f"no-alloc call {call}: B={B} H={H} T={T} d_qk={K} d_v={V} chunk={chunk}")
        x = make_fwd_inputs(B, H, T, K, V, "bf16", seed=40 + call)
        d = _dev(x)
        h_ws, st_ws = M.mlstm_fwd_chunkwise(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"], d["f_pre"],
                                            chunk=chunk, return_state=True)
        h0 = torch.full_like(d["v"], float("nan"))
        h_na, st_na = M.mlstm_fwd_chunkwise_noalloc(d["q"], d["k"], d["v"], d["o_pre"], d["i_pre"],
                                                    d["f_pre"], chunk=chunk, return_state=True, h=h0)
        torch.cuda.synchronize()
        assert torch.equal(h_na, h_ws), f"call {call}: h differs from the workspace entry point"
        for a, b in zip(st_na, st_ws):
            assert torch.equal(a, b), f"call {call}: final state differs"
        ref, _ = mlstm_recurrent_c(*[x[n] for n in NAMES])
        got = _host(h_na)
        assert np.all(np.isfinite(got))
        assert np.max(np.abs(got - ref)) <= 2e-2 * np.max(np.abs(ref))
