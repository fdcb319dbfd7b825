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
  uint16_t* wb; // 64-token tiles only, [BH][Nt][2][64]: bfloat16 bits of w0 (hi) and of
                // w0 - hi (lo), a two-term split of w0; null when not wanted
};

// Chunk-start states written by the state pass: Cs [BH][Nc][V][K] (bf16 or
// fp32), ns [BH][Nc][K] fp32, ms [BH][Nc] fp64.
struct ChunkStates {
  void* Cs;
  float* ns;
  double* ms;
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
};

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

void set_launch_events(int kernel, hipEvent_t before, hipEvent_t after);

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

}  // namespace mlstm_impl
