"""mLSTM matrix-memory cell forward on MI355X (gfx950): HIP kernels behind a C ABI.

The entry points mirror include/mlstm.h: mlstm_fwd_chunkwise (full
sequences), mlstm_fwd_parallel (short sequences), mlstm_step (recurrent
decode) and mlstm_bwd_chunkwise (the gradients for training); and
include/slstm.h: slstm_fwd (the sLSTM scalar-memory cell's
recurrence over a sequence). They take torch tensors for device memory and
run only the HIP library; a missing library raises.
"""
from ._lib import (  # noqa: F401
    MlstmError,
    mlstm_bwd_chunkwise,
    mlstm_fwd_chunkwise,
    mlstm_fwd_chunkwise_noalloc,
    mlstm_fwd_parallel,
    mlstm_step,
    slstm_fwd,
)
