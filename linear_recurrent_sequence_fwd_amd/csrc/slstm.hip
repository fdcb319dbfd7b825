// sLSTM scalar-memory cell forward on gfx950 (xLSTM guide, aifetchly blog,
// "The Twin Cells: sLSTM and mLSTM Mathematical Formulations", sLSTM
// step-by-step recurrent equations).
//
// The recurrence is sequential in t: step t needs h_{t-1} of every cell of
// the head before any of its gates can be formed. One workgroup per (batch
// entry, head) therefore walks the whole sequence. Its 4 D threads hold the
// head's recurrent matrix [4 D][D] (row g D + e: gate g of cell e) in
// registers, so the matrix is read from memory once: the quad of threads
// 4i..4i+3 holds the four gate rows of cell i, each thread one quarter of
// their columns. Per step:
//   1. each thread multiplies its 4 x D/4 block with its quarter of h_{t-1}
//      (D/16 16-byte LDS reads, a quarter of what a whole row would need);
//      thread 4i + q adds the preactivation P_t of gate q of cell i (loaded
//      a block of 8 steps earlier);
//   2. two exchanges within the quad (DPP) give all four of its threads the
//      four gate preactivations of cell i; each updates the cell's m, c, n
//      (kept identically in the four threads) and the first writes h_t[i]
//      into a ring of the last 16 steps' h in LDS;
//   3. one barrier: the next step reads h_t there.
// The steps run in blocks of 8; during each block the previous block's h go
// from the ring to HBM and the next block's preactivations are loaded, in one
// batch per thread.
// The cell state c, n, m is carried in float64. With the exponential forget
// gate m grows by f~ every step (to hundreds over long sequences), and the
// exponent f~ + m_{t-1} - m_t, a small difference of large numbers, would
// lose an ulp of m (3e-5 at m = 430) per step in float32; c and n sum
// thousands of weighted terms of both signs, and rounding them to float32 at
// every step alone costs 1.1e-4 of max|h| over 2048 steps of the benchmark
// workload. The factor exp(f~ + m_{t-1} - m_t) or exp(i~ - m_t) is taken
// from its float64 exponent to about one float32 ulp. Exponentials use the hardware base-2 exponential
// with the argument scaled by log2(e), tanh(x) = 1 - 2 / (exp(2x) + 1) and
// the divisions the hardware reciprocal: a few ulp each, far inside the
// float32 bar of 1e-4.
// The work per step is 4 D^2 fused multiply-adds spread over the workgroup,
// five transcendentals per thread and one barrier: the step is bound by
// vector-instruction issue on its one CU, not by HBM. Throughput comes from
// running the B * H sequences side by side.

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

// exp(d) for a float64 argument d <= 0 (or -inf), to about one float32 ulp
// whatever its size: d log2(e) = n + f with an integer n and f in [0, 1),
// the hardware base-2 exponential of f, scaled by 2^n. (Rounding d log2(e)
// itself to float32 would cost |d| float32 ulps, which the forget and input
// factors would pass on to the state at every step.)
__device__ __forceinline__ float exp_f64arg(double d) {
  const double y = d * 1.4426950408889634;
  const double n = fmax(floor(y), -200.0);   // below 2^-200 the result is 0 anyway
  return ldexpf(__builtin_amdgcn_exp2f((float)(y - n)), (int)n);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]

template <int D>
__global__ __launch_bounds__(4 * D) void slstm_kernel(SlstmLaunch a) {
  constexpr int DS = D / 4;     // cells of h (columns of R) per thread
  constexpr int HS = DS + 4;    // LDS stride of one quarter of h (the pad spreads the quarters over banks)
  const int64_t H = a.H, T = a.T;
  const int64_t b = blockIdx.x / H, hh = blockIdx.x % H;
  const int j = threadIdx.x;
  const int cell = j >> 2, qd = j & 3;
  // h of the last 2 RB steps, each step's h as four padded quarters; step t
  // writes slot t mod 2 RB. The matrix-vector product of step t reads h_{t-1}
  // here, and each block of RB steps' h goes to HBM during the next block,
  // from the half of the ring that block does not write.
  constexpr int RB = 8;   // (the asm statement below names its 8 registers)
  __shared__ __attribute__((aligned(16))) float s_hr[2 * RB][4 * HS];
  auto hpos = [](int c) { return (c / DS) * HS + c % DS; };

  // The quad of threads 4i..4i+3 holds the four gate rows of cell i of the
  // head's recurrent matrix (slot g: gate g), thread 4i + q the columns of
  // quarter q.
  float r[4][DS];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const f32x4v* src = reinterpret_cast<const f32x4v*>(a.R + ((hh * 4 + g) * D + cell) * D + qd * DS);
#pragma unroll
    for (int k = 0; k < DS / 4; ++k) {
      const f32x4v x = src[k];
      r[g][4 * k] = x[0];
      r[g][4 * k + 1] = x[1];
      r[g][4 * k + 2] = x[2];
      r[g][4 * k + 3] = x[3];
    }
  }
  // State of cell i, kept (identically) by all four threads of its quad. An
  // empty state (no state given, or a given one with c = n = 0) starts from
  // m_0 = -inf instead of its m: the same h and the same true-unit state in
  // exact arithmetic (a stabiliser shift of an all-zero state changes
  // nothing), and then n_t >= 1 at every step (m_t = i~_t gives
  // exp(i~_t - m_t) = 1, else the forget factor is 1 and n_t >= n_{t-1}), so
  // c / n cannot underflow.
  const int64_t sidx = (b * H + hh) * D + cell;
  float hv = 0.f, m_given = 0.f;
  double c = 0.0, n = 0.0, m = -INFINITY;
  if (a.c0) {
    c = (double)a.c0[sidx];
    n = (double)a.n0[sidx];
    m_given = a.m0[sidx];
    hv = a.h0[sidx];
    if (c != 0.0 || n != 0.0) m = (double)m_given;
  }
  if (qd == 0) s_hr[2 * RB - 1][hpos(cell)] = hv;
  // thread 4i + q loads P_t of gate q of cell i, at
  // pre[((b T + t) 4 + q) H + hh) D + i]
  const int64_t pstride = 4 * H * D;
  const float* pre = a.pre + (b * T * 4 + qd) * H * D + hh * D + cell;
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
    const int half = (int)(t0 & RB);   // this block's half of the ring
    float pc[RB];
#pragma unroll
    for (int q = 0; q < RB; ++q) pc[q] = pn[q];
    // taken here, before this block's stores and loads are issued
    asm volatile("" ::"v"(pc[0]), "v"(pc[1]), "v"(pc[2]), "v"(pc[3]), "v"(pc[4]), "v"(pc[5]), "v"(pc[6]),
                 "v"(pc[7]));
    if (t0 > 0 && j < D) {
#pragma unroll
      for (int q = 0; q < RB; ++q) hout[(t0 - RB + q) * H * D] = s_hr[(half ^ RB) + q][hpos(j)];
    }
#pragma unroll
    for (int q = 0; q < RB; ++q) pn[q] = t0 + RB + q < T ? pre[(t0 + RB + q) * pstride] : 0.f;
#pragma unroll
    for (int q = 0; q < RB; ++q) {
      const int64_t t = t0 + q;
      if (t >= T) break;   // uniform over the workgroup
      const float p = pc[q];
      const f32x4v* hp = reinterpret_cast<const f32x4v*>(&s_hr[(half + q + 2 * RB - 1) % (2 * RB)][qd * HS]);
      // the partial sums start from zero and P enters after them, so that the
      // long chain of products is not rounded at the size of P (the forget
      // gate's rounding errors add up in the state's weights over the steps)
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < DS / 4; ++k) {
        const f32x4v x = hp[k];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int g = 0; g < 4; ++g) acc[g] = fmaf(r[g][4 * k + cc], x[cc], acc[g]);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g] += qd == g ? p : 0.f;
      // sum over the quad (lane ^ 1, then lane ^ 2): every thread of the quad
      // ends with the same four gate preactivations of its cell (each sum is
      // formed in the same order up to commuted operands, so bit for bit)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g] += dpp_f<kQuadXor1>(acc[g]);
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[g] += dpp_f<kQuadXor2>(acc[g]);
      const double it = (double)acc[0];
      const float zt = tanh_fast(acc[2]);
      const double mf = m + (double)acc[1];
      // of the factors exp(f~ + m_{t-1} - m_t) and exp(i~ - m_t) the one of
      // the term that sets the new maximum is exactly 1
      const bool fkeep = mf >= it;
      const float ex = exp_f64arg(fkeep ? it - mf : mf - it);
      const double fa = fkeep ? 1.0 : (double)ex, ia = fkeep ? (double)ex : 1.0;
      c = fma(fa, c, ia * (double)zt);
      n = fma(fa, n, ia);
      m = fmax(mf, it);
      // sigmoid(o~) c / n = c / (n (1 + exp(-o~))): one reciprocal
      hv = (float)c * __builtin_amdgcn_rcpf(fmaxf((float)n, FLT_MIN) * (1.f + exp_fast(-acc[3])));
      if (qd == 0) s_hr[half + q][hpos(cell)] = hv;
      __syncthreads();   // h_t published
    }
  }
  // the last block's h
  if (T > 0 && j < D) {
    const int64_t tl = ((T - 1) / RB) * RB;
    const int half = (int)(tl & RB);
#pragma unroll
    for (int q = 0; q < RB; ++q)
      if (tl + q < T) hout[(tl + q) * H * D] = s_hr[half + q][hpos(j)];
  }
  if (qd == 0 && a.c_out) {
    if (T == 0) {   // after no step the state is returned as given (the zero state with m = 0)
      a.c_out[sidx] = (float)c;
      a.n_out[sidx] = (float)n;
      a.m_out[sidx] = m_given;
    } else {
      // m leaves as float32; c and n take the factor exp(m - m32), so that
      // exp(m32) c and exp(m32) n are the carried true-unit state
      const float m32 = (float)m;
      const double sc = (double)exp_fast((float)(m - (double)m32));
      a.c_out[sidx] = (float)(c * sc);
      a.n_out[sidx] = (float)(n * sc);
      a.m_out[sidx] = m32;
    }
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
