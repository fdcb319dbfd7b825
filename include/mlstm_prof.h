/*
 * mlstm_prof.h -- measurement entry points of the mLSTM library.
 *
 * Not needed for computing: the calls here do what the entry points of
 * mlstm.h do and, in addition, record caller-owned HIP events on the launch
 * stream around each group of kernels, so that a benchmark can time the
 * kernels of one call. The events belong to that one call only; nothing is
 * remembered between calls and nothing changes for any other call, stream or
 * thread. Conventions, argument checks and status codes are those of mlstm.h.
 */
#ifndef MLSTM_PROF_H_
#define MLSTM_PROF_H_

#include <stddef.h>

#include "mlstm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel groups of a chunkwise forward, in launch order. */
#define MLSTM_PROF_GATE 0   /* gate prefix sums */
#define MLSTM_PROF_STATE 1  /* inter-chunk state pass */
#define MLSTM_PROF_OUT 2    /* intra-chunk output kernel */

/*
 * mlstm_fwd_chunkwise (same arguments, same result) that records
 * events[2 g] before and events[2 g + 1] after kernel group g on `stream`,
 * g = MLSTM_PROF_GATE, MLSTM_PROF_STATE, MLSTM_PROF_OUT. `events` points to
 * six hipEvent_t handles created by the caller; a NULL handle is skipped. A
 * group that a call does not launch records nothing. Returns
 * MLSTM_ERR_NULLPTR for a NULL `events`.
 */
int mlstm_prof_fwd_chunkwise(const mlstm_fwd_args* args, int chunk, void* workspace,
                             size_t workspace_bytes, void* stream, void* const* events);

/* Kernel groups of a chunkwise backward pass, in launch order. */
#define MLSTM_PROF_BWD_FWD_GATE 0   /* the forward's gate prefix sums */
#define MLSTM_PROF_BWD_FWD_STATE 1  /* the forward's inter-chunk state pass */
#define MLSTM_PROF_BWD_DQ 2         /* dq, do~ and g per 64-row tile */
#define MLSTM_PROF_BWD_STATE 3      /* chunk end adjoints, last chunk to first */
#define MLSTM_PROF_BWD_DKV 4        /* dk, dv, di~ per 64-key tile */
#define MLSTM_PROF_BWD_GATE 5       /* forget-gate suffix sums */

/*
 * mlstm_bwd_chunkwise (same arguments, same result) that records
 * events[2 g] before and events[2 g + 1] after kernel group g, g = 0..5 as
 * above: twelve caller-created hipEvent_t handles, NULL entries skipped.
 */
int mlstm_prof_bwd_chunkwise(const mlstm_bwd_args* args, int chunk, void* workspace,
                             size_t workspace_bytes, void* stream, void* const* events);

/*
 * mlstm_step (same arguments, same result) that records the hipEvent_t
 * `before` and `after` on `stream` around the step kernel (NULL: skipped).
 */
int mlstm_prof_step(const mlstm_step_args* args, void* stream, void* before, void* after);

/*
 * The shader clock while other work runs. Launches one wave that sleeps
 * `iters` times s_sleep 127 (about 8k shader cycles each; iters in
 * [1, 2^24]) and writes the shader-clock counter (s_memtime) at its start and
 * end to ticks[0], ticks[1], and the constant-rate counter (s_memrealtime) to
 * ticks[2], ticks[3]: four uint64 in caller-owned, 8-byte-aligned device
 * memory. Launched on a second stream just before a workload, the ratio of
 * the two differences times the constant counter's rate is the clock under
 * that workload. Asynchronous on `stream`; returns MLSTM_ERR_NULLPTR,
 * MLSTM_ERR_BAD_SHAPE or MLSTM_ERR_MISALIGNED on bad arguments before
 * anything is enqueued.
 */
int mlstm_clock_probe(unsigned long long* ticks, int iters, void* stream);

/*
 * A copy of `bytes` (a positive multiple of 16384) from device memory src to
 * device memory dst through LDS with direct-to-LDS loads (global_load_lds,
 * 16 bytes per lane, the instruction the fused kernels stage their tiles
 * with) and 16-byte vector stores: a kernel of known traffic for calibrating
 * the HBM byte counters (FETCH_SIZE, WRITE_SIZE) on that load path.
 * Asynchronous on `stream`; MLSTM_ERR_NULLPTR, MLSTM_ERR_BAD_SHAPE,
 * MLSTM_ERR_MISALIGNED (16 bytes) or MLSTM_ERR_ALIAS (overlap) before
 * anything is enqueued.
 */
int mlstm_prof_copy_lds(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLSTM_PROF_H_ */
