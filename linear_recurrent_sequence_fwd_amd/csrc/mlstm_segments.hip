// Segments of one sequence on gfx950: the fold of a state with a segment's
// summary, and the summary of an empty segment.
//
// The matrix memory after a stretch of tokens is the decayed start state plus
// the stretch's own sum of products (nareshka notes, "B. mLSTM", the
// parallelisation formula; the chunk-to-chunk state of the xLSTM guide's
// "Exploit Chunkwise Hardware Kernels for Production Training"). With the
// segment's summary (C~s, n~s, ms) and its log-forget total G, the state after
// it, started from (C~0, n~0, m0), is
//   m' = max(m0 + G, ms),  C~' = exp(m0 + G - m') C~0 + exp(ms - m') C~s
// and the same for n~. The summary itself comes from the chunk-state kernels
// (launch_summary in mlstm_fused.hip).
//
// Both kernels are elementwise and bandwidth-bound (a few MiB per summary):
// the per-head scalars in float64.

#include "mlstm_device.h"

namespace mlstm_impl {

namespace {

constexpr int kSegThreads = 256;

// Grid: (heads) x (blocks over (V K + K) / 4). Thread u of head bh owns four
// consecutive floats of C~ (u < V K / 4) or of n~ and folds the `count`
// stacked summaries into them in order, four summaries' loads in flight at a
// time.
__global__ __launch_bounds__(kSegThreads) void state_combine_kernel(CombineLaunch a) {
  const int64_t bh = blockIdx.x % a.BH;
  const int64_t u = (blockIdx.x / a.BH) * kSegThreads + threadIdx.x;
  const int64_t nc4 = a.V * a.K / 4, nn4 = a.K / 4;
  if (u >= nc4 + nn4) return;
  const bool is_n = u >= nc4;
  const int64_t per = is_n ? a.K : a.V * a.K;              // floats of one head's C~ or n~
  const int64_t head = bh * per + (is_n ? (u - nc4) * 4 : u * 4);
  const int64_t stack = a.BH * per;                         // floats of one summary's C~ or n~
  double m = a.C0 ? (double)a.m0[bh] : 0.0;                 // the zero state starts at m = 0
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
  if (a.C0) x = *reinterpret_cast<const f32x4*>((is_n ? a.n0 : a.C0) + head);
  const float* ys = (is_n ? a.ns : a.Cs) + head;
  constexpr int kB = 4;
  for (int64_t s0 = 0; s0 < a.count; s0 += kB) {
    f32x4 y[kB];
#pragma unroll
    for (int e = 0; e < kB; ++e) y[e] = *reinterpret_cast<const f32x4*>(ys + min(s0 + e, a.count - 1) * stack);
#pragma unroll
    for (int e = 0; e < kB; ++e) {
      const int64_t s = s0 + e;
      if (s < a.count) {
        const double G = a.Gs[s * a.BH + bh], ms = (double)a.ms[s * a.BH + bh];
        const double carried = m + G;                       // -inf after a zero forget gate
        double mn = fmax(carried, ms);
        if (mn == -INFINITY) mn = 0.0;                      // nothing at all: an all-zero state
        const float al = carried == -INFINITY ? 0.f : (float)exp(carried - mn);
        const float be = ms == -INFINITY ? 0.f : (float)exp(ms - mn);
        x = al * x + be * y[e];
        m = mn;
      }
    }
  }
  *reinterpret_cast<f32x4*>((is_n ? a.n : a.C) + head) = x;
  if (u == 0) a.m[bh] = (float)m;
}

__global__ __launch_bounds__(kSegThreads) void summary_empty_kernel(SummaryOut o, int64_t BH, int64_t K, int64_t V) {
  const int64_t u = (int64_t)blockIdx.x * kSegThreads + threadIdx.x;
  const int64_t nc = BH * V * K, nn = BH * K;
  if (u < nc) o.C[u] = 0.f;
  else if (u < nc + nn) o.n[u - nc] = 0.f;
  else if (u < nc + nn + BH) {
    o.m[u - nc - nn] = -INFINITY;
    o.G[u - nc - nn] = 0.0;
  }
}

}  // namespace

hipError_t launch_state_combine(const CombineLaunch& c, hipStream_t s) {
  const int64_t blocks = ((c.V * c.K + c.K) / 4 + kSegThreads - 1) / kSegThreads;
  hipLaunchKernelGGL(state_combine_kernel, dim3((unsigned)(c.BH * blocks)), dim3(kSegThreads), 0, s, c);
  return hipGetLastError();
}

hipError_t launch_summary_empty(const SummaryOut& o, int64_t BH, int64_t K, int64_t V, hipStream_t s) {
  const int64_t n = BH * V * K + BH * K + BH;
  hipLaunchKernelGGL(summary_empty_kernel, dim3((unsigned)((n + kSegThreads - 1) / kSegThreads)),
                     dim3(kSegThreads), 0, s, o, BH, K, V);
  return hipGetLastError();
}

}  // namespace mlstm_impl
