/*
 * mlstm_segments.h -- C ABI for running one sequence as several segments on
 * gfx950 (segments on several devices, or one after another).
 *
 * The matrix memory after a stretch of tokens is its start state decayed by
 * the stretch's forget gates plus the stretch's own sum of products
 * (nareshka notes, "B. mLSTM", the parallelisation formula:
 * C_T = (prod f) C_0 + sum_j (prod_{l>j} f_l) i_j v_j k_j^T, the same for n),
 * which is also how the chunkwise form passes its state from chunk to chunk
 * (xLSTM guide, aifetchly blog, "Exploit Chunkwise Hardware Kernels for
 * Production Training"). A segment therefore acts on any start state through
 * its summary alone:
 *
 *   C~s, n~s, ms   the segment's own end state from the EMPTY state (no start
 *                  state term; ms = -inf for an empty segment), stabilised
 *                  units as in mlstm.h
 *   G              the sum of the segment's log forget gates (float64;
 *                  -inf when one of them is zero, i.e. f~ = -inf)
 *
 * and the state after it, from (C~0, n~0, m0), is
 *
 *   m' = max(m0 + G, ms),  C~' = exp(m0 + G - m') C~0 + exp(ms - m') C~s.
 *
 * To split a sequence over P segments: every segment's summary
 * (mlstm_segment_summary; independent, so on P devices at once), an
 * exclusive scan of the summaries with mlstm_state_combine (start_0 = the
 * sequence's initial state, start_p = the fold of summaries 0..p-1 into
 * start_0: one call with count = p over the summaries stacked as an
 * all-gather leaves them), then every segment's outputs from its start state
 * (mlstm_fwd_chunkwise with C0/n0/m0 = start_p). The outputs equal those of
 * one call over the whole sequence, and the fold of all P summaries is its
 * final state.
 *
 * Conventions as in mlstm.h: device pointers owned by the caller, nothing
 * allocated or freed, work enqueued on `stream` without synchronising,
 * arguments checked on the host before anything is enqueued, status codes
 * of mlstm_status.
 */
#ifndef MLSTM_SEGMENTS_H_
#define MLSTM_SEGMENTS_H_

#include <stddef.h>
#include <stdint.h>

#include "mlstm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Arguments of a segment summary. */
typedef struct mlstm_summary_args {
  int64_t B, H, T;        /* batch, heads, tokens of the segment; B, H >= 1, T >= 0 */
  int64_t d_qk, d_v;      /* d_qk in {64, 128, 256}, d_v a multiple of 128 */
  int32_t dtype;          /* MLSTM_BF16 (k, v) */
  const void* k;          /* [B,H,T,d_qk] */
  const void* v;          /* [B,H,T,d_v]  */
  const float* i_pre;     /* [B,H,T] input-gate preactivation */
  const float* f_pre;     /* [B,H,T] forget-gate preactivation */
  float* C_out;           /* [B,H,d_v,d_qk] C~s (written) */
  float* n_out;           /* [B,H,d_qk]     n~s */
  float* m_out;           /* [B,H]          ms */
  double* G_out;          /* [B,H]          G, 8-byte aligned */
} mlstm_summary_args;

/*
 * The summary of a segment: the chunk-local end states of its chunks of
 * `chunk` tokens (the chunkwise forward's state kernel) folded in order from
 * the empty state, and the sum of their log-forget totals. No output h is
 * computed. `chunk` is a multiple of 64 in [64, 8192] and must divide T
 * (every chunk full; MLSTM_ERR_BAD_SHAPE otherwise); T = 0 gives the empty
 * summary (0, 0, -inf, 0). Other dtypes and shapes return
 * MLSTM_ERR_UNSUPPORTED. The workspace holds the chunks' local states and the
 * gate prefix sums (size from mlstm_segment_summary_workspace_size, 256-byte
 * aligned). Outputs must not overlap the inputs, each other or the workspace.
 */
size_t mlstm_segment_summary_workspace_size(const mlstm_summary_args* args, int chunk);
int mlstm_segment_summary(const mlstm_summary_args* args, int chunk, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Arguments of a state fold. */
typedef struct mlstm_combine_args {
  int64_t B, H, d_qk, d_v;  /* >= 1; d_qk a multiple of 4 */
  int64_t count;          /* summaries to fold in order, >= 0 (0: the start state itself) */
  const float* C0;        /* start state [B,H,d_v,d_qk]; NULL = the zero state with m0 = 0 (the
                             recurrence's own start; then n0 and m0 are NULL too) */
  const float* n0;        /* [B,H,d_qk] */
  const float* m0;        /* [B,H] (may hold -inf: a summary used as a start state) */
  const float* Cs;        /* the segments' summaries, stacked: [count][B,H,d_v,d_qk] */
  const float* ns;        /* [count][B,H,d_qk] */
  const float* ms;        /* [count][B,H] */
  const double* Gs;       /* [count][B,H], 8-byte aligned */
  float* C_out;           /* the state after the segments: [B,H,d_v,d_qk] (written) */
  float* n_out;           /* [B,H,d_qk] */
  float* m_out;           /* [B,H]; m_out = 0 where every term is empty */
} mlstm_combine_args;

/*
 * The state after `count` segments with the stacked summaries (Cs, ns, ms,
 * Gs), started from (C0, n0, m0): summary 0 folded in first. Elementwise and
 * bandwidth-bound (one pass over the summaries), float32 state with the
 * per-head exponents in float64. State arrays 16-byte aligned (Gs 8-byte, m
 * arrays 4-byte); outputs must not overlap the inputs or each other.
 */
int mlstm_state_combine(const mlstm_combine_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLSTM_SEGMENTS_H_ */
