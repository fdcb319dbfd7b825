"""mLSTM matrix-memory cell forward on MI355X (gfx950): HIP kernels behind a C ABI.

The entry points mirror include/mlstm.h: mlstm_fwd_chunkwise (full
sequences), mlstm_fwd_parallel (short sequences), mlstm_step (recurrent
decode) and mlstm_bwd_chunkwise (the gradients for training);
include/mlstm_block.h: mlstm_block_fwd (the residual block with
pre-up-projection around the cell) and its steps (gemm_bf16,
layernorm_bf16, block_conv_gates, block_groupnorm_gate);
include/mlstm_segments.h: mlstm_segment_summary and mlstm_state_combine (one
sequence run as segments, each from the fold of the summaries before it); and
include/slstm.h: slstm_fwd (the sLSTM scalar-memory cell's
recurrence over a sequence). They take torch tensors for device memory and
run only the HIP library; a missing library raises.
"""
from ._lib import (  # noqa: F401
    MlstmError,
    block_conv_gates,
    block_groupnorm_gate,
    block_params,
    gemm_bf16,
    gemm_bf16_strided,
    layernorm_bf16,
    mlstm_block_fwd,
    mlstm_bwd_chunkwise,
    mlstm_fwd_chunkwise,
    mlstm_fwd_chunkwise_noalloc,
    mlstm_fwd_parallel,
    mlstm_segment_summary,
    mlstm_state_combine,
    mlstm_step,
    slstm_fwd,
)
