"""CPU oracles for the mLSTM and sLSTM cells (test infrastructure; see
mlstm_oracle and slstm_oracle)."""
from .mlstm_oracle import logsigmoid, sigmoid, mlstm_step, mlstm_recurrent, mlstm_rows  # noqa: F401
from .slstm_oracle import slstm_step, slstm_recurrent  # noqa: F401
