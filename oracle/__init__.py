"""CPU oracles for the mLSTM and sLSTM cells (test infrastructure; see
mlstm_oracle, mlstm_grad, mlstm_segments, mlstm_block and slstm_oracle)."""
from .mlstm_oracle import logsigmoid, sigmoid, mlstm_step, mlstm_recurrent, mlstm_rows  # noqa: F401
from .mlstm_grad import mlstm_backward  # noqa: F401
from .mlstm_segments import segment_summary, state_combine  # noqa: F401
from .slstm_oracle import slstm_step, slstm_recurrent  # noqa: F401
