/*
 * mlstm_block.h — C ABI of the mLSTM block around the cell, for gfx950.
 *
 * The residual block with pre-up-projection of the hu-po page "Introduction
 * to xLSTM architecture", section "Residual Block with Pre-Up Projection"
 * (primarily for the mLSTM), with the cell's projections and gates of the
 * xLSTM guide (aifetchly), "mLSTM: Matrix Key-Value Memory and Covariance
 * Updates", recurrent formulation. Per batch entry, x [T, D], inner width
 * E = 2 D = H d_v:
 *
 *   xn = LayerNorm(x)                               pre-layer norm
 *   [xm | z] = xn W_up^T + b_up                     up-projection by two
 *   xc = swish(causal conv(xm) + b_conv)            channel-wise, KC taps
 *   q = BlockDiag(W_q) xc + b_q                     one block per head
 *   k = BlockDiag(W_k) xc / sqrt(d_qk) + b_k
 *   v = BlockDiag(W_v) xm + b_v                     values skip the conv
 *   i~ = xc w_i^T + b_i, f~ = xc w_f^T + b_f        one preactivation per head
 *   h~ = mLSTM cell (mlstm.h) with no output gate of its own
 *   y = (GroupNorm(h~) + skip * xc) * sigmoid(z)    group norm per head over d_v,
 *                                                   learnable skip, external gate
 *   out = x + y W_down^T + b_down                   down-projection, residual
 *
 * Conventions (as in mlstm.h): all pointers are device pointers owned by the
 * caller; nothing is allocated or freed; every call enqueues work on `stream`
 * (a hipStream_t, NULL = default stream) and returns without synchronising.
 * Activations and weight matrices are bfloat16, vectors float32, all
 * row-major; arrays are 16-byte aligned. Arguments are checked on the host
 * before anything is enqueued; the status codes are mlstm_status of mlstm.h.
 */
#ifndef MLSTM_BLOCK_H
#define MLSTM_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#include "mlstm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Strided-batched bf16 matrix product on MFMA with float32 accumulation:
 * for every batch index (b1, b2) in [0, batch1) x [0, batch2),
 *   C = alpha A B^T + bias (+ R)
 * with A [M][K] at A + b1 strideA1 + b2 strideA2 (row pitch lda) and B [N][K]
 * likewise (weights stored output-major, k contiguous). C is bf16 or float32
 * (c_dtype), element (m, n) at C + m ldc + n, or at C + n ldc + m when
 * c_trans; bias [N] float32 at bias + b2 stride_bias2 (NULL: none); R bf16
 * [M][N] (NULL: none; not with c_trans). Strides count elements. The block's
 * projections are this call: the up- and down-projections with one batch
 * entry, the per-head q, k, v projections batched over (batch entry, head).
 * Needs M, N, K >= 1, K % 64 == 0, N % 4 == 0 (M % 4 == 0 with c_trans),
 * lda, ldb <= 2^21 (MLSTM_ERR_UNSUPPORTED beyond),
 * 16-byte aligned arrays and rows (lda, ldb, ldr and the strides of A, B, R
 * multiples of 8 elements; ldc and C's strides multiples of 16 bytes);
 * C must not overlap A, B, bias or R.
 */
typedef struct mlstm_gemm_args {
  int64_t M, N, K;
  int64_t batch1, batch2;
  const void* A;
  int64_t lda, strideA1, strideA2;
  const void* B;
  int64_t ldb, strideB1, strideB2;
  void* C;
  int64_t ldc, strideC1, strideC2;
  int32_t c_dtype;        /* MLSTM_BF16 or MLSTM_FP32 */
  int32_t c_trans;
  float alpha;
  const float* bias;
  int64_t stride_bias2;
  const void* R;
  int64_t ldr, strideR1, strideR2;
} mlstm_gemm_args;

int mlstm_gemm_bf16(const mlstm_gemm_args* g, void* stream);

/*
 * Layer norm of each row (hu-po page, the block's pre-layer norm):
 * y = (x - mean) / sqrt(var + eps) * w + b, var the mean squared deviation,
 * statistics in float32. x, y bf16 [rows][D]; w, b float32 [D].
 * Needs rows >= 0, D % 8 == 0, 8 <= D <= 8192; y must not overlap x.
 */
int mlstm_layernorm_bf16(const void* x, const float* w, const float* b, void* y, int64_t rows, int64_t D,
                         float eps, void* stream);

/* Parameters of one block. Shapes: E = 2 D = H d_v. */
typedef struct mlstm_block_params {
  int64_t D;              /* model width; D % 64 == 0 */
  int64_t H, d_qk, d_v;   /* heads (H <= 32), head dims of the cell (d_qk in {64, 128, 256}, d_v % 128 == 0,
                             d_v <= 2048), H d_v == 2 D, (2 D / H) % 64 == 0 */
  int64_t KC;             /* causal conv taps, 1..4 */
  float eps_ln, eps_gn;   /* layer norm and group norm epsilons */
  const float *ln_w, *ln_b;            /* [D] */
  const void* W_up;                    /* [2E][D] bf16: rows 0..E-1 give xm, rows E..2E-1 give z */
  const float* b_up;                   /* [2E] */
  const float *conv_w, *conv_b;        /* [E][KC] taps oldest first (conv_w[e][KC-1] takes the current token), [E] */
  const void *W_q, *W_k;               /* [H][d_qk][E/H] bf16 */
  const float *b_q, *b_k;              /* [H d_qk] */
  const void* W_v;                     /* [H][d_v][E/H] bf16 */
  const float* b_v;                    /* [E] */
  const void *w_i, *w_f;               /* [H][E] bf16: gate projections from xc */
  const float *b_i, *b_f;              /* [H] */
  const float *gn_w, *gn_b, *skip;     /* [E] */
  const void* W_down;                  /* [D][E] bf16 */
  const float* b_down;                 /* [D] */
} mlstm_block_params;

/*
 * The conv step of the block: xc = swish(causal conv(xm) + conv_b) from the
 * first E columns of xup [B][T][2E] (bf16), and from the bf16-rounded xc the
 * gate preactivations i_pre = xc w_i^T + b_i, f_pre = xc w_f^T + b_f written
 * [B][H][T] float32, the cell's layout. xc bf16 [B][T][E]. Outputs must not
 * overlap xup or each other.
 */
int mlstm_block_conv_gates(const mlstm_block_params* p, int64_t B, int64_t T, const void* xup, void* xc,
                           float* i_pre, float* f_pre, void* stream);

/*
 * The step after the cell: y = (GroupNorm(h) + skip * xc) * sigmoid(z), h
 * the cell output bf16 [B][H][T][d_v] (the cell's layout), each (token,
 * head) normalised over d_v; xc bf16 [B][T][E]; z the last E columns of xup
 * [B][T][2E]; y bf16 [B][T][E]. y must not overlap the inputs.
 */
int mlstm_block_groupnorm_gate(const mlstm_block_params* p, int64_t B, int64_t T, const void* h, const void* xc,
                               const void* xup, void* y, void* stream);

/*
 * The whole block: out = block(x), x and out bf16 [B][T][D] (out must not
 * overlap x, the parameters or the workspace). The cell runs the chunkwise
 * path of mlstm_fwd_chunkwise with `chunk` tokens between stored states
 * (a multiple of 64 in [64, 8192]) and zero initial state. The workspace
 * (256-byte aligned, at least mlstm_block_fwd_workspace_size bytes) holds
 * the intermediates; after the call it holds, at the offsets
 * mlstm_block_workspace_offsets reports: xn [B][T][D], xup [B][T][2E],
 * xc [B][T][E], q, k [B][H][T][d_qk], v [B][H][T][d_v], i_pre, f_pre
 * [B][H][T] float32, h [B][H][T][d_v], y [B][T][E]. T == 0 does nothing.
 */
size_t mlstm_block_fwd_workspace_size(const mlstm_block_params* p, int64_t B, int64_t T, int chunk);
int mlstm_block_fwd(const mlstm_block_params* p, int64_t B, int64_t T, const void* x, void* out, int chunk,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Byte offsets of the intermediates in the block's workspace, in the order
 * xn, xup, xc, q, k, v, i_pre, f_pre, h, y (offsets[0..9]); returns
 * MLSTM_OK or MLSTM_ERR_BAD_SHAPE for invalid sizes. */
int mlstm_block_workspace_offsets(const mlstm_block_params* p, int64_t B, int64_t T, int chunk,
                                  size_t offsets[10]);

#ifdef __cplusplus
}
#endif

#endif /* MLSTM_BLOCK_H */
