// Host-only stand-ins for the HIP launchers of libmlstm, for the sanitizer
// build of the C ABI layer (tests/native/abi_sanitized.cpp). They enqueue
// nothing and touch no memory: each records which launcher was called and
// checks the shapes the ABI layer hands it. The support predicates restate
// the library's rules (fused path: bf16 with d_v a multiple of 128 and d_qk
// in {64, 128, 256}; backward shapes; sLSTM D).
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <stdlib.h>

#include "../../linear_recurrent_sequence_fwd_amd/csrc/mlstm_launch.h"

namespace mlstm_impl {

int g_calls[20];

static hipError_t seen(int id, bool ok) {
  ++g_calls[id];
  if (!ok) {
    fprintf(stderr, "launcher %d called with inconsistent arguments\n", id);
    abort();
  }
  return hipSuccess;
}

static bool fwd_ok(const FwdLaunch& f) {
  return f.BH >= 1 && f.T >= 1 && f.K % 64 == 0 && f.V % 64 == 0 && f.L % 64 == 0 && f.Nc >= 1 &&
         (f.Nc - 1) * (int64_t)f.L < f.T;
}

bool fused_path(int bf16, int64_t K, int64_t V) { return bf16 && V % 128 == 0 && (K == 64 || K == 128 || K == 256); }
bool bf16_fast_path(const FwdLaunch& a) { return a.bf16 && a.V % 64 == 0; }
bool slstm_supported(int64_t D) { return D == 16 || D == 32 || D == 64 || D == 128; }
bool bwd_supported(int bf16, int64_t K, int64_t V) {
  if (bf16) return (K == 64 || K == 128 || K == 256) && (V == 64 || V == 128 || V == 256 || V == 512);
  return (K == 64 || K == 128) && (V == 64 || V == 128 || V == 256);
}

hipError_t launch_gate(const FwdLaunch& a, const GateBuffers& gb, hipStream_t) {
  return seen(0, fwd_ok(a) && gb.u && gb.b && gb.mp && gb.rs && gb.w0 && gb.g && gb.U && gb.R);
}
hipError_t launch_state(const FwdLaunch& a, const GateBuffers&, const ChunkStates&, hipStream_t) { return seen(1, fwd_ok(a)); }
hipError_t launch_out(const FwdLaunch& a, const GateBuffers&, const ChunkStates&, hipStream_t) { return seen(2, fwd_ok(a)); }
hipError_t launch_copy_state(const FwdLaunch& a, hipStream_t) { return seen(3, a.T == 0); }
hipError_t launch_step(const StepLaunch& a, hipStream_t) { return seen(4, a.BH >= 1 && a.K % 64 == 0); }
hipError_t launch_clock_probe(unsigned long long* t, int iters, hipStream_t) { return seen(5, t && iters >= 1); }
hipError_t launch_lds_copy(const void* s, void* d, int64_t bytes, hipStream_t) {
  return seen(6, s && d && bytes > 0 && bytes % 16384 == 0);
}
hipError_t launch_state_bf16(const FwdLaunch& a, const GateBuffers&, const ChunkStates&, hipStream_t) { return seen(7, fwd_ok(a)); }
hipError_t launch_out_bf16(const FwdLaunch& a, const GateBuffers&, const ChunkStates&, hipStream_t) { return seen(8, fwd_ok(a)); }
hipError_t launch_fused(const FwdLaunch& a, const GateBuffers& gb, const SegStates& ss, hipStream_t) {
  return seen(9, fwd_ok(a) && a.L == 64 && gb.wb && ss.S >= 1 && ss.TPS >= 1);
}
hipError_t launch_slstm(const SlstmLaunch& a, hipStream_t) { return seen(10, a.B >= 1 && a.H >= 1 && slstm_supported(a.D)); }
hipError_t launch_bwd(const BwdLaunch& b, const GateBuffers&, const ChunkStates&, const BwdBuffers& bb, hipStream_t) {
  return seen(11, b.T == 0 || (bb.G && bb.dz && bb.qdq && bb.Es && bb.es && bb.Ms && bb.L0 && bb.L0e));
}

hipError_t launch_gemm(const GemmLaunch& g, hipStream_t) {
  return seen(12, g.M >= 1 && g.N >= 1 && g.K % 64 == 0 && g.N % 4 == 0 && g.nb1 >= 1 && g.nb2 >= 1 && g.A &&
                      g.B && g.C && g.lda >= g.K && g.ldb >= g.K);
}
int gemm_tile() { return 256; }
hipError_t launch_layernorm(const void* x, const float* w, const float* b, void* y, int64_t rows, int64_t D, float,
                            hipStream_t) {
  return seen(13, x && w && b && y && rows >= 1 && D % 8 == 0);
}
hipError_t launch_conv_gate(const ConvLaunch& c, hipStream_t) {
  return seen(14, c.B >= 1 && c.T >= 1 && c.E % 128 == 0 && c.H >= 1 && c.H <= 32 && c.KC >= 1 && c.KC <= 4 &&
                      c.ldx == 2 * c.E && c.xm && c.xc && c.i_pre && c.f_pre);
}
hipError_t launch_summary(const FwdLaunch& a, const GateBuffers& gb, const SegStates& ss, const SummaryOut& o,
                          hipStream_t) {
  return seen(16, fwd_ok(a) && a.L == 64 && gb.wb && ss.S >= 1 && ss.TPS >= 1 &&
                      (int64_t)ss.S * ss.TPS == a.Nc && a.T == a.Nc * 64 && o.C && o.n && o.m && o.G);
}
hipError_t launch_summary_empty(const SummaryOut& o, int64_t BH, int64_t K, int64_t V, hipStream_t) {
  return seen(17, o.C && o.n && o.m && o.G && BH >= 1 && K >= 1 && V >= 1);
}
hipError_t launch_state_combine(const CombineLaunch& c, hipStream_t) {
  return seen(18, c.BH >= 1 && c.K >= 1 && c.K % 4 == 0 && c.V >= 1 && c.count >= 0 &&
                      (c.count == 0 || (c.Cs && c.ns && c.ms && c.Gs)) && c.C && c.n && c.m &&
                      (c.C0 ? c.n0 && c.m0 : !c.n0 && !c.m0));
}
hipError_t launch_groupnorm_gate(const GnLaunch& g, hipStream_t) {
  return seen(15, g.B >= 1 && g.T >= 1 && g.H * g.dv > 0 && g.dv % 8 == 0 && g.ldz == 2 * g.H * g.dv && g.h &&
                      g.xc && g.z && g.y);
}

}  // namespace mlstm_impl
