// sLSTM scalar-memory cell forward on gfx950 (xLSTM guide, aifetchly blog,
// "The Twin Cells: sLSTM and mLSTM Mathematical Formulations", sLSTM
// step-by-step recurrent equations).
//
// The recurrence is sequential in t: step t needs h_{t-1} of every cell of
// the head before any of its gates can be formed. One workgroup per (batch
// entry, head) therefore walks the whole sequence. Its 4 D threads hold the
// head's stacked recurrent matrix [4 D][D] (row g D + e: gate g of cell e) in
// registers, so the matrix is read from memory once: the quad of threads
// 4i..4i+3 holds rows 4i..4i+3, each thread one quarter of their columns.
// Per step:
//   1. each thread multiplies its 4 x D/4 block with its quarter of h_{t-1}
//      (D/16 16-byte LDS reads, a quarter of what a whole row would need);
//      two exchanges within the quad (DPP) leave row j's sum in thread j,
//      which adds the preactivation P_t[j] (loaded a block of 8 steps
//      earlier). The threads of gate z apply tanh and those of gate o the
//      sigmoid here, so that the four gates' waves share the transcendental
//      work;
//   2. barrier; threads d < D take the four gates of cell d, update m, c, n
//      in registers and write h_t[d] into a ring of the last 8 steps' h in
//      LDS (the next step reads it there);
//   3. barrier.
// Every 8 steps the ring goes to HBM and the next 8 steps' preactivations are
// loaded, in one batch per thread.
// Exponentials use the hardware base-2 exponential with the argument scaled
// by log2(e), tanh(x) = 1 - 2 / (exp(2x) + 1) and the divisions the hardware
// reciprocal: a few ulp each, far inside the float32 bar of 1e-4.
// The work per step is 4 D^2 fused multiply-adds spread over the workgroup
// plus two barriers, so a step is bound by issue latency, not by HBM or the
// ALUs; throughput comes from running the B * H sequences side by side.

#include <hip/hip_runtime.h>

#include <float.h>
#include <stdint.h>

#include "mlstm_launch.h"

namespace mlstm_impl {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
// 1 - 2 / (e^{2x} + 1): exact limits +-1 for large |x| (e^{2x} -> inf or 0)
__device__ __forceinline__ float tanh_fast(float x) {
  return fmaf(-2.f, __builtin_amdgcn_rcpf(exp_fast(2.f * x) + 1.f), 1.f);
}
__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.f + exp_fast(-x)); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]

template <int D>
__global__ __launch_bounds__(4 * D) void slstm_kernel(SlstmLaunch a) {
  constexpr int NT = 4 * D;
  constexpr int DS = D / 4;     // cells of h (columns of R) per thread
  constexpr int HS = DS + 4;    // LDS stride of one quarter of h (the pad spreads the quarters over banks)
  const int64_t H = a.H, T = a.T;
  const int64_t b = blockIdx.x / H, hh = blockIdx.x % H;
  const int j = threadIdx.x;
  const int g = j / D, e = j % D;
  const int qd = j & 3;
  // h of the last RB steps, each step's h as four padded quarters: the
  // matrix-vector product of step t reads h_{t-1} here, and the block's h go
  // to HBM together at the start of the next block (see below)
  constexpr int RB = 8;   // (the asm statement below names its 8 registers)
  __shared__ __attribute__((aligned(16))) float s_hr[RB][4 * HS];
  __shared__ float s_g[NT];
  auto hpos = [](int cell) { return (cell / DS) * HS + cell % DS; };

  // The quad of threads 4i..4i+3 holds rows 4i..4i+3 of the head's stacked
  // recurrent matrix [4 D][D] (row g D + e: gate g of cell e), thread 4i + q
  // the columns of quarter q. Slot s of a thread holds row 4i + sigma(s),
  // sigma = (0, 2, 1, 3), the order in which the two-step reduction below
  // leaves row 4i + q's sum in thread 4i + q.
  float r[4][DS];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    const int row = (j & ~3) + ((sl & 1) << 1) + (sl >> 1);
    const f32x4v* src = reinterpret_cast<const f32x4v*>(a.R + (hh * NT + row) * D + qd * DS);
#pragma unroll
    for (int k = 0; k < DS / 4; ++k) {
      const f32x4v x = src[k];
      r[sl][4 * k] = x[0];
      r[sl][4 * k + 1] = x[1];
      r[sl][4 * k + 2] = x[2];
      r[sl][4 * k + 3] = x[3];
    }
  }
  // cell state: thread d < D owns cell d. The zero state starts from
  // m_0 = -inf instead of 0: the same h and the same true-unit state in exact
  // arithmetic (a stabiliser shift of an all-zero state changes nothing), and
  // then n_t >= 1 at every step (m_t = i~_t gives exp(i~_t - m_t) = 1, else
  // the forget factor is 1 and n_t >= n_{t-1}), so c / n cannot underflow.
  const int64_t sidx = (b * H + hh) * D + j;
  float c = 0.f, n = 0.f, m = -INFINITY, hv = 0.f;
  if (j < D && a.c0) {
    c = a.c0[sidx];
    n = a.n0[sidx];
    m = a.m0[sidx];
    hv = a.h0[sidx];
  }
  if (j < D) s_hr[RB - 1][hpos(j)] = hv;
  // P_t[j] sits at pre[((b T + t) 4 + g) H + hh) D + e]
  const int64_t pstride = 4 * H * D;
  const float* pre = a.pre + (b * T * 4 + g) * H * D + hh * D + e;
  float* hout = a.h + (b * T * H + hh) * D + j;
  // The steps run in blocks of RB. At the start of a block the wave takes the
  // preactivations loaded one block earlier, stores the previous block's h
  // and loads the next block's preactivations. Loads and stores are then
  // issued together once per block, and the one wait for loaded data
  // (which, with stores in flight, waits for every memory operation of the
  // wave) falls on operations a whole block old.
  float pn[RB];
#pragma unroll
  for (int q = 0; q < RB; ++q) pn[q] = q < T ? pre[q * pstride] : 0.f;
  __syncthreads();
  for (int64_t t0 = 0; t0 < T; t0 += RB) {
    float pc[RB];
#pragma unroll
    for (int q = 0; q < RB; ++q) pc[q] = pn[q];
    // taken here, before this block's stores and loads are issued
    asm volatile("" ::"v"(pc[0]), "v"(pc[1]), "v"(pc[2]), "v"(pc[3]), "v"(pc[4]), "v"(pc[5]), "v"(pc[6]),
                 "v"(pc[7]));
    if (t0 > 0 && j < D) {
#pragma unroll
      for (int q = 0; q < RB; ++q) hout[(t0 - RB + q) * H * D] = s_hr[q][hpos(j)];
    }
#pragma unroll
    for (int q = 0; q < RB; ++q) pn[q] = t0 + RB + q < T ? pre[(t0 + RB + q) * pstride] : 0.f;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int64_t t = t0 + q;
      if (t >= T) break;   // uniform over the workgroup
      const float p = pc[q];
      const f32x4v* hp = reinterpret_cast<const f32x4v*>(&s_hr[(q + RB - 1) % RB][qd * HS]);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < DS / 4; ++k) {
        const f32x4v x = hp[k];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int sl = 0; sl < 4; ++sl) acc[sl] = fmaf(r[sl][4 * k + c], x[c], acc[sl]);
      }
      // sum over the quad: after the exchange with the neighbour (lane ^ 1)
      // a thread keeps two rows, after the one with lane ^ 2 a single row
      const bool o1 = j & 1, o2 = j & 2;
      float k0 = o1 ? acc[2] : acc[0], k1 = o1 ? acc[3] : acc[1];
      k0 += dpp_f<kQuadXor1>(o1 ? acc[0] : acc[2]);
      k1 += dpp_f<kQuadXor1>(o1 ? acc[1] : acc[3]);
      const float gp = p + (o2 ? k1 : k0) + dpp_f<kQuadXor2>(o2 ? k0 : k1);
      s_g[j] = g == 2 ? tanh_fast(gp) : (g == 3 ? sigmoid_fast(gp) : gp);
      __syncthreads();   // all gates of step t formed
      if (j < D) {
        const float it = s_g[j], ft = s_g[D + j], zt = s_g[2 * D + j], ot = s_g[3 * D + j];
        const float mn = fmaxf(m + ft, it);
        const float fa = exp_fast(ft + m - mn), ia = exp_fast(it - mn);
        c = fa * c + ia * zt;
        n = fa * n + ia;
        m = mn;
        hv = ot * c * __builtin_amdgcn_rcpf(fmaxf(n, FLT_MIN));   // sigmoid(o~) c / n
        s_hr[q][hpos(j)] = hv;
      }
      __syncthreads();   // h_t published; s_g free for step t + 1
    }
  }
  // the last block's h (each thread stores what it wrote itself)
  if (T > 0 && j < D) {
    const int64_t tl = ((T - 1) / RB) * RB;
#pragma unroll
    for (int q = 0; q < RB; ++q)
      if (tl + q < T) hout[(tl + q) * H * D] = s_hr[q][hpos(j)];
  }
  if (j < D && a.c_out) {
    a.c_out[sidx] = c;
    a.n_out[sidx] = n;
    a.m_out[sidx] = (T == 0 && !a.c0) ? 0.f : m;   // the zero state reports m = 0
    a.h_out[sidx] = hv;
  }
}

}  // namespace

bool slstm_supported(int64_t D) { return D == 16 || D == 32 || D == 64 || D == 128; }

hipError_t launch_slstm(const SlstmLaunch& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.H));
  switch (a.D) {
    case 16: hipLaunchKernelGGL(slstm_kernel<16>, grid, dim3(64), 0, s, a); break;
    case 32: hipLaunchKernelGGL(slstm_kernel<32>, grid, dim3(128), 0, s, a); break;
    case 64: hipLaunchKernelGGL(slstm_kernel<64>, grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(slstm_kernel<128>, grid, dim3(512), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mlstm_impl
