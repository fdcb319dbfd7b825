"""mLSTM matrix-memory cell forward on MI355X (gfx950): HIP kernels behind a C ABI."""
