/*
 * mlstm.h -- C ABI of the MI355X (gfx950) mLSTM matrix-memory cell forward.
 *
 * The cell (xLSTM guide, aifetchly blog, "mLSTM: Matrix Key-Value Memory and
 * Covariance Updates", recurrent formulation; stabiliser from "The Stabilizer
 * State" of the same guide), per batch entry b and head h:
 *
 *   log f_t = logsigmoid(f~_t)         forget gate, carried in log space
 *   i_t     = exp(i~_t)                exponential input gate
 *   m_t     = max(log f_t + m_{t-1}, i~_t)
 *   C~_t    = exp(log f_t + m_{t-1} - m_t) C~_{t-1} + exp(i~_t - m_t) v_t k_t^T
 *   n~_t    = exp(log f_t + m_{t-1} - m_t) n~_{t-1} + exp(i~_t - m_t) k_t
 *   h_t     = sigmoid(o~_t) * (C~_t q_t) / max(|n~_t . q_t|, exp(-m_t))
 *
 * which equals h_t = o_t * C_t q_t / max(|n_t . q_t|, 1) in true units
 * (C = exp(m) C~, n = exp(m) n~). Keys are used as given: any 1/sqrt(d_qk)
 * scaling belongs to the caller's key projection.
 *
 * Conventions for every entry point:
 *  - All pointers are DEVICE pointers (hipMalloc / torch CUDA tensors) unless
 *    said otherwise; all arrays are contiguous, row-major, 16-byte aligned.
 *  - q, k: [B, H, T, d_qk]; v, o_pre, h: [B, H, T, d_v], all of `dtype`.
 *    i_pre, f_pre: [B, H, T] float32 (gate PREactivations).
 *  - State: C [B, H, d_v, d_qk] float32 (the pages' orientation C = v k^T,
 *    row index = value dimension), n [B, H, d_qk] float32, m [B, H] float32,
 *    all in stabilised units (C~, n~, m).
 *  - The caller owns every buffer and the stream. The library never
 *    allocates or frees memory and never synchronises; work is enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream) and errors of the
 *    asynchronous execution surface at the caller's next synchronisation.
 *  - Return value: MLSTM_OK (0) or a negative mlstm_status. Argument checks
 *    run on the host before anything is enqueued; on an error nothing is
 *    enqueued. mlstm_last_error() describes the most recent error of the
 *    calling thread.
 */
#ifndef MLSTM_H_
#define MLSTM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLSTM_ABI_VERSION 4

typedef enum mlstm_status {
  MLSTM_OK = 0,
  MLSTM_ERR_NULLPTR = -1,      /* a required pointer is NULL */
  MLSTM_ERR_BAD_SHAPE = -2,    /* a size is negative/zero where it must not be, or not a supported multiple */
  MLSTM_ERR_BAD_DTYPE = -3,    /* dtype is neither MLSTM_FP32 nor MLSTM_BF16 */
  MLSTM_ERR_MISALIGNED = -4,   /* a pointer is not 16-byte aligned */
  MLSTM_ERR_ALIAS = -5,        /* an output overlaps an input or another output */
  MLSTM_ERR_WORKSPACE = -6,    /* workspace NULL or smaller than the size query returns */
  MLSTM_ERR_UNSUPPORTED = -7,  /* valid but outside what this build implements (e.g. d_qk) */
  MLSTM_ERR_HIP = -8           /* the HIP runtime reported an error at launch */
} mlstm_status;

typedef enum mlstm_dtype {
  MLSTM_FP32 = 0,  /* float32 inputs/outputs, float32 MFMA (16x16x4) arithmetic */
  MLSTM_BF16 = 1   /* bfloat16 inputs/outputs, bf16 MFMA (16x16x32) with float32 accumulation */
} mlstm_dtype;

/* Arguments of a full-sequence forward (chunkwise or parallel form). */
typedef struct mlstm_fwd_args {
  int64_t B, H, T;        /* batch, heads, tokens; B, H >= 1, T >= 0 */
  int64_t d_qk, d_v;      /* head dims: d_qk in {64, 128, 256} (fp32: {64, 128}); d_v a multiple of 64 */
  int32_t dtype;          /* mlstm_dtype of q, k, v, o_pre, h */
  const void* q;          /* [B,H,T,d_qk] */
  const void* k;          /* [B,H,T,d_qk] */
  const void* v;          /* [B,H,T,d_v]  */
  const void* o_pre;      /* [B,H,T,d_v]  output-gate preactivation; in mlstm_fwd_chunkwise with
                             MLSTM_BF16 and d_v a multiple of 128 it may be NULL: no output gate,
                             h = C q / max(|n^T q|, 1) (the block of mlstm_block.h applies its gate
                             outside the cell) */
  const float* i_pre;     /* [B,H,T]      input-gate preactivation */
  const float* f_pre;     /* [B,H,T]      forget-gate preactivation */
  void* h;                /* [B,H,T,d_v]  output (written) */
  const float* C0;        /* optional initial state [B,H,d_v,d_qk]; NULL = zero state */
  const float* n0;        /* [B,H,d_qk]; required iff C0 != NULL */
  const float* m0;        /* [B,H];      required iff C0 != NULL */
  float* C_out;           /* optional final state [B,H,d_v,d_qk]; NULL = not written */
  float* n_out;           /* [B,H,d_qk]; required iff C_out != NULL */
  float* m_out;           /* [B,H];      required iff C_out != NULL */
} mlstm_fwd_args;

/*
 * Chunkwise-parallel forward for full sequences (xLSTM guide, "Exploit
 * Chunkwise Hardware Kernels for Production Training": sequences split into
 * chunks; dense matrix products inside a chunk, the state passed between
 * chunks). `chunk` is the number of tokens between stored states: a multiple
 * of 64 in [64, 8192]; T need not be a multiple of it (the last chunk is
 * ragged). Kernels: gate prefix sums over 64-token tiles; the inter-chunk
 * state (each chunk's local end state, then their in-order fold into every
 * chunk's start state, all float32); and the output kernel, which walks each
 * chunk's tiles from its start state with decay-masked Q K^T, P V, the
 * carried-state term (the float32 state as two bf16 terms for MLSTM_BF16)
 * and the state update on MFMA. (bfloat16 with d_v a multiple of 128; other
 * shapes run a two-pass variant that stores every chunk's start state in
 * float32.) The
 * workspace holds those states and the per-token gate prefix sums; its size
 * comes from mlstm_fwd_chunkwise_workspace_size(). Outputs must not overlap
 * inputs, each other or the workspace.
 */
size_t mlstm_fwd_chunkwise_workspace_size(const mlstm_fwd_args* args, int chunk);
int mlstm_fwd_chunkwise(const mlstm_fwd_args* args, int chunk, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Parallel (dual, quadratic) form for short sequences (xLSTM guide, "The
 * Dual Formulation": decay matrix log D_tj = sum_{l=j+1..t} log f_l + i~_j
 * for j <= t; H~ = (D o Q K^T) V divided row-wise by the same sum with V
 * replaced by ones, floored at 1). Tiled over 64x64 key blocks with the exact
 * row stabiliser computed from prefix maxima, so no T x T matrix is stored.
 * 1 <= T <= 8192 (T = 0 is accepted and only copies/zeroes the state). The
 * final state, if requested, comes from the state pass run as one chunk.
 */
size_t mlstm_fwd_parallel_workspace_size(const mlstm_fwd_args* args);
int mlstm_fwd_parallel(const mlstm_fwd_args* args, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Arguments of one recurrent decode step. */
typedef struct mlstm_step_args {
  int64_t B, H;           /* B, H >= 1 */
  int64_t d_qk, d_v;      /* d_qk a multiple of 64 in [64, 512]; d_v a multiple of 32 */
  int32_t dtype;          /* mlstm_dtype of q, k, v, o_pre, h (state is always float32) */
  const void* q;          /* [B,H,d_qk] */
  const void* k;          /* [B,H,d_qk] */
  const void* v;          /* [B,H,d_v]  */
  const void* o_pre;      /* [B,H,d_v]  */
  const float* i_pre;     /* [B,H] */
  const float* f_pre;     /* [B,H] */
  float* C;               /* [B,H,d_v,d_qk] state, updated IN PLACE */
  const float* n_in;      /* [B,H,d_qk] state before the step */
  const float* m_in;      /* [B,H]      state before the step */
  float* n_out;           /* [B,H,d_qk] state after the step; must not overlap n_in (ping-pong) */
  float* m_out;           /* [B,H]      state after the step; must not overlap m_in */
  void* h;                /* [B,H,d_v]  output */
} mlstm_step_args;

/*
 * One token of recurrent inference (xLSTM guide, recurrent formulation
 * "Inference Mode"; constant memory per step). Reads and rewrites C once
 * (bandwidth-bound); n and m are ping-ponged because every workgroup of a
 * head reads the old n, m while one of them writes the new ones.
 */
int mlstm_step(const mlstm_step_args* args, void* stream);

/*
 * mlstm_fwd_chunkwise without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments (minus the workspace),
 * same result, same kernels. The scratch comes from a fixed device array of
 * mlstm_fwd_chunkwise_noalloc_limit() bytes (64 MiB) that each GPU the
 * library runs on holds until the process ends; the call allocates nothing.
 * A call whose workspace would exceed it (mlstm_fwd_chunkwise_workspace_size
 * above the limit, e.g. very long sequences with short chunks) returns
 * MLSTM_ERR_UNSUPPORTED before anything is enqueued. All calls on one GPU
 * share its array: calls that may overlap in time on one GPU (different
 * streams, or different threads) race and must be serialised by the caller.
 * The first call on a device looks up the array's address there
 * (hipGetSymbolAddress) and may return MLSTM_ERR_HIP if that fails.
 */
size_t mlstm_fwd_chunkwise_noalloc_limit(void);
int mlstm_fwd_chunkwise_noalloc(const mlstm_fwd_args* args, int chunk, void* stream);

/* Arguments of a chunkwise backward pass (gradient of a loss through h). */
typedef struct mlstm_bwd_args {
  int64_t B, H, T;        /* as for the forward */
  int64_t d_qk, d_v;      /* bf16: d_qk in {64, 128, 256}, d_v in {64, 128, 256, 512};
                             fp32: d_qk in {64, 128}, d_v in {64, 128, 256} */
  int32_t dtype;          /* mlstm_dtype of q, k, v, o_pre, h, dh and of dq, dk, dv, do_pre */
  const void* q;          /* [B,H,T,d_qk] the forward's inputs */
  const void* k;          /* [B,H,T,d_qk] */
  const void* v;          /* [B,H,T,d_v]  */
  const void* o_pre;      /* [B,H,T,d_v]  */
  const float* i_pre;     /* [B,H,T]      */
  const float* f_pre;     /* [B,H,T]      */
  const void* h;          /* [B,H,T,d_v]  the forward's output for these inputs */
  const void* dh;         /* [B,H,T,d_v]  dL/dh, the incoming gradient */
  const float* C0;        /* the forward's initial state [B,H,d_v,d_qk], or NULL (zero state) */
  const float* n0;        /* [B,H,d_qk]; required iff C0 != NULL */
  const float* m0;        /* [B,H];      required iff C0 != NULL */
  void* dq;               /* [B,H,T,d_qk] outputs (written) */
  void* dk;               /* [B,H,T,d_qk] */
  void* dv;               /* [B,H,T,d_v]  */
  void* do_pre;           /* [B,H,T,d_v]  dL/d o_pre */
  float* di_pre;          /* [B,H,T]      dL/d i_pre */
  float* df_pre;          /* [B,H,T]      dL/d f_pre */
  float* dC0;             /* optional [B,H,d_v,d_qk]: dL/d C0 (stabilised units), NULL = not wanted */
  float* dn0;             /* [B,H,d_qk]; required iff dC0 != NULL */
  float* dm0;             /* [B,H];      required iff dC0 != NULL */
} mlstm_bwd_args;

/*
 * Chunkwise backward pass: the gradient of a loss L through the outputs h
 * of mlstm_fwd_chunkwise with respect to q, k, v and the three gate
 * preactivations, and (when dC0 is given) the initial state, for training
 * (xLSTM guide, aifetchly blog: the dual and chunkwise forms are what make
 * the mLSTM trainable in parallel, "The Dual Formulation: How mLSTM Enables
 * Parallel GPU Training" and "Exploit Chunkwise Hardware Kernels for
 * Production Training"). L reaches the cell only through h: no gradient of
 * the final state is taken in. `h` must be the forward's output for the same
 * inputs and initial state (it supplies num/den for the normaliser and
 * output-gate terms). The chunk states are recomputed (gate prefix sums and
 * the inter-chunk state pass, as in the forward); then per 64-row tile dq,
 * dL/d o_pre and g = dh o / den; the chunks' end adjoints from the last
 * chunk to the first; per 64-key tile dk, dv, dL/d i_pre; and the forget
 * gate's gradient as suffix sums of q.dq - k.dk that stop at a zero forget
 * gate. dC0 is the gradient with respect to the stabilised C~0 as passed
 * (without C0: at the zero state, m0 = 0); dm0 = <dC0, C~0> + dn0 . n~0.
 * `chunk`: multiple of 64 in [64, 8192]. Outputs must not overlap inputs,
 * each other or the workspace (size from mlstm_bwd_chunkwise_workspace_size).
 * Other shapes return MLSTM_ERR_UNSUPPORTED.
 */
size_t mlstm_bwd_chunkwise_workspace_size(const mlstm_bwd_args* args, int chunk);
int mlstm_bwd_chunkwise(const mlstm_bwd_args* args, int chunk, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static string). */
const char* mlstm_status_string(int status);
/* Message of the calling thread's most recent error ("" if none). */
const char* mlstm_last_error(void);
/* MLSTM_ABI_VERSION of the loaded library. */
int mlstm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLSTM_H_ */
