"""CPU oracle for the mLSTM cell (test infrastructure; see mlstm_oracle)."""
from .mlstm_oracle import logsigmoid, sigmoid, mlstm_step, mlstm_recurrent, mlstm_rows  # noqa: F401
