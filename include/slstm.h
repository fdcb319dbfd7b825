/*
 * slstm.h -- C ABI of the MI355X (gfx950) sLSTM scalar-memory cell forward.
 *
 * The cell (xLSTM guide, aifetchly blog, "The Twin Cells: sLSTM and mLSTM
 * Mathematical Formulations", sLSTM step-by-step recurrent equations), per
 * batch entry b, head h and cell d of the head:
 *
 *   g~_t = P_t + R h_{t-1}                 g = i, f, z, o
 *   m_t  = max(m_{t-1} + f~_t, i~_t)
 *   c_t  = exp(f~_t + m_{t-1} - m_t) c_{t-1} + exp(i~_t - m_t) tanh(z~_t)
 *   n_t  = exp(f~_t + m_{t-1} - m_t) n_{t-1} + exp(i~_t - m_t)
 *   h_t  = sigmoid(o~_t) c_t / n_t
 *
 * P_t = W x_t + b is the input projection, computed by the caller; the
 * library runs the recurrence. R mixes the cells of one head only (the xLSTM
 * paper's heads without memory mixing across heads); one head of width D is
 * a full recurrent matrix. The forget gate is exponential, as the equations
 * write it. Without a given state the recurrence starts from zero c, n, h;
 * its stabiliser starts at -inf rather than the listing's 0, which changes
 * neither h nor the true-unit state (exp(m) c, exp(m) n) and keeps n >= 1 at
 * every step, so that c / n cannot underflow in float32 (a requested final
 * state after T = 0 reports m = 0). Preactivations must be finite.
 *
 * Conventions are those of mlstm.h: DEVICE pointers, contiguous row-major
 * arrays, caller-owned buffers and stream, no allocation or synchronisation
 * by the library, mlstm_status return codes and mlstm_last_error().
 */
#ifndef SLSTM_H_
#define SLSTM_H_

#include <stdint.h>

#include "mlstm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Arguments of a full-sequence sLSTM forward (float32 throughout). */
typedef struct slstm_fwd_args {
  int64_t B, H, T;        /* batch, heads, steps; B, H >= 1, T >= 0 */
  int64_t D;              /* cells per head: 16, 32, 64 or 128 */
  const float* pre;       /* [B,T,4,H,D] gate preactivations P_t, gates in the order i, f, z, o */
  const float* R;         /* [H,4,D,D] recurrent matrices: gate g of cell e gets sum_d R[h][g][e][d] h_{t-1}[d] */
  float* h;               /* [B,T,H,D] output (written) */
  const float* c0;        /* optional initial state [B,H,D] each; all four NULL = zero c, n, h (stabiliser as above) */
  const float* n0;
  const float* m0;
  const float* h0;
  float* c_out;           /* optional final state [B,H,D] each; all four NULL = not written */
  float* n_out;
  float* m_out;
  float* h_out;
} slstm_fwd_args;

/*
 * sLSTM forward over a whole sequence: one workgroup per (batch entry, head)
 * walks the T steps; each step is a matrix-vector product with the head's
 * recurrent matrix (held in registers) followed by the elementwise cell
 * update. pre, R, h and the state arrays must be 16-byte aligned; outputs
 * must not overlap inputs or each other. Errors: MLSTM_ERR_NULLPTR (args,
 * pre, R or h when T > 0; a partial initial or final state),
 * MLSTM_ERR_BAD_SHAPE (B, H < 1, T < 0, D < 1), MLSTM_ERR_UNSUPPORTED (D not
 * 16, 32, 64 or 128, or B * H above 2^31 - 1), MLSTM_ERR_MISALIGNED,
 * MLSTM_ERR_ALIAS, MLSTM_ERR_HIP (launch). T = 0 copies the initial state
 * (or zeros) to the final state if one is requested.
 */
int slstm_fwd(const slstm_fwd_args* args, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* SLSTM_H_ */
