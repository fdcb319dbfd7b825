"""The five mLSTM workloads: shapes, dtypes and input distributions.

Each entry names the workload by what it is. ``chunk`` lists the chunk sizes
the chunkwise form runs at; ``entry`` lists the entry points that apply.
"""
from __future__ import annotations

CONFIGS = {
    "tiny": dict(B=1, H=1, T=256, d_qk=64, d_v=64, dtype="fp32", chunk=(64,),
                 entry=("chunkwise", "parallel", "step"), i_std=1.0),
    "mid": dict(B=4, H=8, T=2048, d_qk=128, d_v=128, dtype="bf16", chunk=(64,),
                entry=("chunkwise", "parallel"), i_std=1.0, stress_i_std=6.0),
    "7b_layer": dict(B=1, H=8, T=8192, d_qk=256, d_v=512, dtype="bf16", chunk=(64, 128, 256),
                     entry=("chunkwise",), i_std=1.0),
    "long_context": dict(B=1, H=8, T=131072, d_qk=256, d_v=512, dtype="bf16",
                         chunk=(64, 128, 256), entry=("chunkwise",), i_std=1.0),
    "decode": dict(B=64, H=8, d_qk=256, d_v=512, prefill=512, steps=1000, dtype="fp32",
                   entry=("step",)),
}

ORDER = ("tiny", "mid", "7b_layer", "long_context", "decode")
