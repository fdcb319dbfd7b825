// Internal interface between the C ABI layer (host validation, workspace
// carving) and the HIP kernels. Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlstm_impl {

enum KernelId { K_GATE = 0, K_STATE = 1, K_OUT = 2, K_STEP = 3, K_COUNT = 4 };

// Per-token / per-chunk gate prefix data written by the gate kernel and read
// by the state pass and the output kernel. Token arrays are [BH][T], chunk
// arrays [BH][Nc].
// The prefix sums and everything derived from them are float64: a long
// chunk of strong forgetting makes b large while the differences b_t - b_j
// that matter stay small, and float32 would lose them to cancellation.
struct GateBuffers {
  double* u;    // i~_j - b_j, with b the in-chunk cumulative log forget gate
  double* b;    // in-chunk cumulative log forget gate (a zero forget gate counts as 0 here)
  double* mp;   // max of u over [reset(t), t] within the chunk
  int* rs;      // position (in chunk) of the last zero forget gate at or before t, -1 if none
  double* g;    // chunk total of b
  double* U;    // mp at the chunk's last token
  int* R;       // rs at the chunk's last token
  float* w0;    // exp(u_j - U) for keys at or after the chunk's last zero forget gate, else 0
  uint16_t* wb; // 64-token tiles only, [BH][Nt][3][64]: bfloat16 bits of a three-term split
                // w0 = hi + lo + lo2 (about 24 bits); null when not wanted
};

// Chunk-start states written by the state pass: Cs [BH][Nc][V][K] fp32 (or
// bf16 when cs_bf16: the backward pass, which multiplies them as bf16),
// ns [BH][Nc][K] fp32, ms [BH][Nc] fp64.
struct ChunkStates {
  void* Cs;
  float* ns;
  double* ms;
  int cs_bf16 = 0;
};

// Chunk states of the fused path (mlstm_fused.hip), S chunks of TPS 64-token
// tiles: C [BH][S-1][V][K] and n [BH][S-1][K] float32 hold each chunk's local
// end state and then, folded in order, the start states of chunks 1..S-1;
// mloc, mstart and G [BH][S-1] float64 are the local end stabiliser, the start
// stabiliser and the chunk's log-forget total.
struct SegStates {
  float* C;
  float* n;
  double* mloc;
  double* mstart;
  double* G;
  int S;
  int TPS;
};

struct FwdLaunch {
  int64_t BH, T, K, V;
  int L;           // chunk length (multiple of 64)
  int64_t Nc;      // number of chunks
  int bf16;        // 1: bf16 inputs/outputs, 0: fp32
  const void *q, *k, *v, *o;
  const float *i_pre, *f_pre;
  void* h;
  const float *C0, *n0, *m0;
  float *C_out, *n_out, *m_out;
  const hipEvent_t* marks;   // [K_COUNT][2] events around each kernel group, or null
};

struct StepLaunch {
  int64_t BH, K, V;
  int bf16;
  const void *q, *k, *v, *o;
  const float *i_pre, *f_pre;
  float* C;
  const float *n_in, *m_in;
  float *n_out, *m_out;
  void* h;
  const hipEvent_t* marks;   // [K_COUNT][2] events around the step kernel, or null
};

// Backward pass (mlstm_bwd.hip). The forward's gate kernel and state pass
// run first (chunk-start states in `cs`); then the four backward kernels.
enum BwdKernelId { B_FWD_GATE = 0, B_FWD_STATE = 1, B_DQ = 2, B_STATE = 3, B_DKV = 4, B_GATE = 5, B_COUNT = 6 };

struct BwdLaunch {
  int64_t BH, T, K, V;
  int L;           // chunk length (multiple of 64)
  int64_t Nc;      // number of chunks
  int bf16;
  const void *q, *k, *v, *o, *h, *dh;
  const float *i_pre, *f_pre;
  void *dq, *dk, *dv, *dout;
  float *di, *df;
  const float *C0, *n0, *m0;
  float *dC0, *dn0, *dm0;
  const hipEvent_t* marks;   // [B_COUNT][2] events around each kernel, or null
};

// Workspace of the backward kernels: g per token [BH][T][V] in the input
// dtype; the chunk end adjoints [BH][Nc][V][K] float32; dz, q . dq [BH][T],
// the end adjoints' normaliser part [BH][Nc][K] float32 and log scale
// [BH][Nc] float64.
struct BwdBuffers {
  void* G;
  float* dz;
  float* qdq;
  void* Es;
  float* es;
  double* Ms;
  float* L0;    // chunk 0's share of the adjoint [BH][V][K] (initial state's gradient)
  float* L0e;   // [BH][K]
};
bool bwd_supported(int bf16, int64_t K, int64_t V);
hipError_t launch_bwd(const BwdLaunch& b, const GateBuffers& gb, const ChunkStates& cs, const BwdBuffers& bb,
                      hipStream_t s);

// sLSTM forward (slstm.hip): pre [B,T,4,H,D], R [H,4,D,D], h [B,T,H,D];
// optional state [B,H,D] in (c0 == NULL: zero state) and out (c_out == NULL:
// not written), all float32
struct SlstmLaunch {
  int64_t B, H, T, D;
  const float *pre, *R;
  float* h;
  const float *c0, *n0, *m0, *h0;
  float *c_out, *n_out, *m_out, *h_out;
};
bool slstm_supported(int64_t D);
hipError_t launch_slstm(const SlstmLaunch& a, hipStream_t s);

hipError_t launch_gate(const FwdLaunch& a, const GateBuffers& gb, hipStream_t s);
// Inter-chunk state pass; `cs` may have null Cs/ns/ms when no chunk-start
// states are needed (only the final state).
hipError_t launch_state(const FwdLaunch& a, const GateBuffers& gb, const ChunkStates& cs,
                        hipStream_t s);
// Output kernel. `cs.Cs == nullptr` with a.C0 set: the initial state is read
// from C0/n0/m0 (float32) as the carried state of the single chunk.
hipError_t launch_out(const FwdLaunch& a, const GateBuffers& gb, const ChunkStates& cs,
                      hipStream_t s);
// T == 0: final state = initial state (or zero).
hipError_t launch_copy_state(const FwdLaunch& a, hipStream_t s);
hipError_t launch_step(const StepLaunch& a, hipStream_t s);
// one sleeping wave; ticks[0..1]: shader-clock counter, ticks[2..3]:
// constant-rate counter, at its start and end
hipError_t launch_clock_probe(unsigned long long* ticks, int iters, hipStream_t s);
// direct-to-LDS copy of `bytes` (a positive multiple of 16 KiB) for counter calibration
hipError_t launch_lds_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);

// bfloat16 kernels with transposed LDS operand loads (mlstm_bf16.hip). The
// state pass takes any d_v multiple of 64; the output kernel needs
// bf16_fast_path() (d_v a multiple of 128).
bool bf16_fast_path(const FwdLaunch& a);
hipError_t launch_state_bf16(const FwdLaunch& a, const GateBuffers& gb, const ChunkStates& cs,
                             hipStream_t s);
hipError_t launch_out_bf16(const FwdLaunch& a, const GateBuffers& gb, const ChunkStates& cs,
                           hipStream_t s);

// Fused path (mlstm_fused.hip): bf16 with d_v a multiple of 128. `a` counts
// 64-token tiles (a.L == 64, a.Nc tiles); the gate buffers are per tile.
bool fused_path(int bf16, int64_t K, int64_t V);
hipError_t launch_fused(const FwdLaunch& a, const GateBuffers& gb, const SegStates& ss, hipStream_t s);

// Segments of one sequence (mlstm_fused.hip, mlstm_segments.hip).
// A segment's summary: its end state from the empty state (m = -inf) and the
// sum G of its log forget gates, per head. C [BH][V][K], n [BH][K], m [BH]
// float32, G [BH] float64.
struct SummaryOut {
  float *C, *n, *m;
  double* G;
};
// The summary from the chunk-local states of all ss.S chunks (every chunk
// full: T == ss.S * chunk) folded from the empty state; the gate buffers as
// for launch_fused, ss holding ss.S (not ss.S - 1) chunk entries.
hipError_t launch_summary(const FwdLaunch& a, const GateBuffers& gb, const SegStates& ss, const SummaryOut& o,
                          hipStream_t s);
// The summary of an empty segment: C = n = 0, m = -inf, G = 0.
hipError_t launch_summary_empty(const SummaryOut& o, int64_t BH, int64_t K, int64_t V, hipStream_t s);
// The state after `count` segments with the stacked summaries (Cs, ns, ms, Gs:
// [count][BH][...]) folded in order into the start state (C0, n0, m0), or into
// the zero state with m0 = 0 when C0 is null. K % 4 == 0, 16-byte aligned
// state arrays.
struct CombineLaunch {
  int64_t BH, K, V, count;
  const float *C0, *n0, *m0;
  const float *Cs, *ns, *ms;
  const double* Gs;
  float *C, *n, *m;
};
hipError_t launch_state_combine(const CombineLaunch& c, hipStream_t s);

// mLSTM block around the cell (mlstm_block.hip).
//
// GEMM: C = alpha A B^T + bias (+ R) per batch entry (b1, b2), A [M][K] and
// B [N][K] bf16 (k contiguous, row pitches lda, ldb), float32 accumulation;
// C bf16 or float32, element (m, n) at C + m ldc + n (c_trans: C + n ldc + m);
// bias [N] float32 at bias + b2 sbias2 (or null); R bf16 at
// R + m ldr + n (or null; not with c_trans). Batch offsets in elements:
// X + b1 sX1 + b2 sX2. Needs K % 64 == 0, N % 4 == 0 (M % 4 == 0 with
// c_trans) and 16-byte aligned rows.
struct GemmLaunch {
  int64_t M, N, K, nb1, nb2;
  const void* A; int64_t lda, sA1, sA2;
  const void* B; int64_t ldb, sB1, sB2;
  void* C; int64_t ldc, sC1, sC2;
  int c_fp32, c_trans;
  float alpha;
  const float* bias; int64_t sbias2;
  const void* R; int64_t ldr, sR1, sR2;
};
hipError_t launch_gemm(const GemmLaunch& g, hipStream_t s);
int gemm_tile();   // output tile edge (rows and columns per workgroup)

// rows x D bf16 -> bf16, D % 8 == 0, D <= 8192
hipError_t launch_layernorm(const void* x, const float* w, const float* b, void* y, int64_t rows, int64_t D,
                            float eps, hipStream_t s);

// xc = swish(causal conv(xm)) and the gate preactivations from xc; E % 128 == 0,
// H <= 32, KC in 1..4
struct ConvLaunch {
  int64_t B, T, E, H, KC;
  const void* xm; int64_t ldx;
  const float *cw, *cb;
  void* xc;
  const void *wi, *wf;
  const float *bi, *bf;
  float *i_pre, *f_pre;
};
hipError_t launch_conv_gate(const ConvLaunch& c, hipStream_t s);

// y = (GroupNorm(h) + skip xc) sigmoid(z), one group per head over dv (dv % 8 == 0, dv <= 2048)
struct GnLaunch {
  int64_t B, T, H, dv;
  const void *h, *xc, *z; int64_t ldz;
  const float *gw, *gb, *skip;
  void* y;
  float eps;
};
hipError_t launch_groupnorm_gate(const GnLaunch& g, hipStream_t s);

}  // namespace mlstm_impl
