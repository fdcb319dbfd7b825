// HIP kernels of the mLSTM matrix-memory cell forward for gfx950 (CDNA4).
//
// Method (xLSTM guide, aifetchly blog): the stabilised recurrence of
// "mLSTM: Matrix Key-Value Memory and Covariance Updates" with the running
// max of "The Stabilizer State", evaluated chunkwise as in "Exploit Chunkwise
// Hardware Kernels for Production Training" and, inside a chunk, through the
// decay matrix of "The Dual Formulation":
//
//   log D_tj = sum_{l=j+1..t} log f_l + i~_j            (j <= t, same chunk)
//
// Notation inside a chunk that starts at token t0 with carried state
// (C~, n~, m_prev): b_t = sum_{l=t0..t} log f_l, u_j = i~_j - b_j. Then
// log D_tj = u_j + b_t, the carried state enters row t with log weight
// b_t + m_prev, and the row stabiliser of the recurrence is
//   m_t = b_t + r_t,  r_t = max(m_prev, max_{j<=t} u_j),
// so every weight exp(u_j - r_t) and exp(m_prev - r_t) is at most 1 and the
// denominator floor of 1 (true units) is exp(-(b_t + r_t)). A zero forget
// gate (f~ = -inf) kills every earlier key and the carried state: the kernels
// carry the position of the last such gate instead of a -inf in b.
//
// Kernels:
//   gate_kernel   per (head, chunk): b, u, the masked prefix max of u, reset
//                 positions, chunk totals (gate64_kernel: one wave per
//                 64-token chunk).
//   state_kernel  per (head, 64x64 tile of C): walks the chunks in order,
//                 stores each chunk's start state and carries C~ (float32 in
//                 MFMA accumulators) with C~ <- a C~ + K_c^T diag(w) V_c.
//   out_kernel    per (head, 64-row query tile, block of v columns): the
//                 carried-state term Q C~^T, the decay-masked Q K^T on MFMA,
//                 P V on MFMA, normaliser and output gate.
//   step_kernel   one decode step per (head, block of C rows), bandwidth-bound
//                 on the float32 state.

#include "mlstm_device.h"

namespace mlstm_impl {

namespace {

// ------------------------------------------------------------------ gate kernel

struct GateArgs {
  const float* i_pre;
  const float* f_pre;
  int64_t T, Nc, BH;
  int L;
  GateBuffers gb;
};

// One workgroup per (head, chunk). Each thread takes a contiguous run of
// tokens; three passes: sums of log f, then b and u with the segmented max,
// then the masked prefix max and reset positions. log f itself is a float32
// evaluation; its sums and everything derived from them are float64.
__global__ __launch_bounds__(kThreads) void gate_kernel(GateArgs a) {
  __shared__ __attribute__((aligned(16))) double sd[8];
  __shared__ __attribute__((aligned(16))) int si[8];
  const int64_t c = blockIdx.x % a.Nc;
  const int64_t bh = blockIdx.x / a.Nc;
  const int64_t t0 = c * a.L;
  const int Lc = (int)min((int64_t)a.L, a.T - t0);
  const int64_t base = bh * a.T + t0;
  const float* fi = a.f_pre + base;
  const float* ii = a.i_pre + base;
  const int E = (Lc + kThreads - 1) / kThreads;
  const int j0 = min((int)threadIdx.x * E, Lc);
  const int j1 = min(j0 + E, Lc);

  double s = 0.0;
  for (int j = j0; j < j1; ++j) {
    const float lf = log_sigmoid(fi[j]);
    s += (lf == -INFINITY) ? 0.0 : (double)lf;
  }
  double run = block_excl_sum(s, sd);

  SegMax loc{0, -INFINITY};
  int rloc = -1;
  for (int j = j0; j < j1; ++j) {
    const float lf = log_sigmoid(fi[j]);
    const int reset = (lf == -INFINITY);
    run += reset ? 0.0 : (double)lf;
    const double u = (double)ii[j] - run;
    a.gb.b[base + j] = run;
    a.gb.u[base + j] = u;
    loc = seg_combine(loc, SegMax{reset, u});
    if (reset) rloc = j;
  }
  SegMax cur = block_excl_segmax(loc, si, sd);
  int rcur = block_excl_max_int(rloc, si + 4);

  for (int j = j0; j < j1; ++j) {
    const int reset = (fi[j] == -INFINITY);
    cur = seg_combine(cur, SegMax{reset, a.gb.u[base + j]});
    if (reset) rcur = j;
    a.gb.mp[base + j] = cur.v;
    a.gb.rs[base + j] = rcur;
  }
  __shared__ double sU;
  __shared__ int sR;
  if (j0 < j1 && j1 == Lc) {
    a.gb.g[bh * a.Nc + c] = run;
    a.gb.U[bh * a.Nc + c] = cur.v;
    a.gb.R[bh * a.Nc + c] = rcur;
    sU = cur.v;
    sR = rcur;
  }
  __syncthreads();
  // chunk-local weights of the state update: exp(u_j - U) <= 1, zero before a reset
  for (int j = j0; j < j1; ++j)
    a.gb.w0[base + j] = (j >= sR && sU != -INFINITY) ? expf((float)(a.gb.u[base + j] - sU)) : 0.f;
}

// One wave per 64-token chunk (four chunks per workgroup), one token per lane:
// the same quantities as gate_kernel with the scans done across the wave.
// The running max restarts at a zero forget gate: lane t takes lane t - d's
// partial max only when t - d is at or after its own last reset.
__global__ __launch_bounds__(kThreads) void gate64_kernel(GateArgs a) {
  const int64_t chunk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (chunk >= a.BH * a.Nc) return;   // whole waves only
  const int64_t c = chunk % a.Nc, bh = chunk / a.Nc;
  const int lane = threadIdx.x & 63;
  const int64_t t0 = c * kTile;
  const int Lc = (int)min((int64_t)kTile, a.T - t0);
  const bool valid = lane < Lc;
  const int64_t base = bh * a.T + t0;
  const float fi = valid ? a.f_pre[base + lane] : 0.f;
  const float ii = valid ? a.i_pre[base + lane] : 0.f;
  const float lf = log_sigmoid(fi);
  const bool reset = valid && lf == -INFINITY;
  double b = (valid && !reset) ? (double)lf : 0.0;
  int rs = reset ? lane : -1;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double yb = __shfl_up(b, d, 64);
    const int yr = __shfl_up(rs, d, 64);
    if (lane >= d) {
      b += yb;
      rs = max(rs, yr);
    }
  }
  const double u = valid ? (double)ii - b : -INFINITY;
  double mp = u;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(mp, d, 64);
    if (lane >= d && lane - d >= rs) mp = fmax(mp, y);
  }
  const int last = Lc - 1;
  const double gc = __shfl(b, last, 64);
  const double Uc = __shfl(mp, last, 64);
  const int Rc = __shfl(rs, last, 64);
  if (valid) {
    a.gb.b[base + lane] = b;
    a.gb.u[base + lane] = u;
    a.gb.mp[base + lane] = mp;
    a.gb.rs[base + lane] = rs;
    a.gb.w0[base + lane] = (lane >= Rc && Uc != -INFINITY) ? expf((float)(u - Uc)) : 0.f;
  }
  if (a.gb.wb) {   // w0 = hi + lo + lo2, three bfloat16 terms (about 24 bits)
    const float w0 = (valid && lane >= Rc && Uc != -INFINITY) ? expf((float)(u - Uc)) : 0.f;
    const __bf16 hi = (__bf16)w0;
    const float rest = w0 - (float)hi;
    const __bf16 lo = (__bf16)rest;
    const __bf16 lo2 = (__bf16)(rest - (float)lo);
    uint16_t* dst = a.gb.wb + (bh * a.Nc + c) * 3 * kTile;
    dst[lane] = __builtin_bit_cast(uint16_t, hi);
    dst[kTile + lane] = __builtin_bit_cast(uint16_t, lo);
    dst[2 * kTile + lane] = __builtin_bit_cast(uint16_t, lo2);
  }
  if (lane == 0) {
    a.gb.g[bh * a.Nc + c] = gc;
    a.gb.U[bh * a.Nc + c] = Uc;
    a.gb.R[bh * a.Nc + c] = Rc;
  }
}

// ------------------------------------------------------------------ state pass

template <typename TI, typename TS>
struct StateArgs {
  const TI* k;
  const TI* v;
  GateBuffers gb;
  const float *C0, *n0, *m0;
  TS* Cs;
  float* ns;
  double* ms;
  float *C_out, *n_out, *m_out;
  int64_t T, Nc, V;
  int L;
};

template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 x);
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 x) {
  *reinterpret_cast<f32x4*>(p) = x;
}

// One workgroup per (head, 64 k x 64 v tile of C). The tile lives in MFMA
// accumulators as C^T[k][v]: wave (wk, wv) holds 32 x 32 of it, lane l,
// register r of sub-tile (a, b) is k = 32 wk + 16 a + 4 (l/16) + r,
// v = 32 wv + 16 b + l%16, i.e. four consecutive k of one row of C.
template <typename TI, typename TS, int K>
__global__ __launch_bounds__(kThreads) void state_kernel(StateArgs<TI, TS> a) {
  constexpr int E = Frag<TI>::E;
  constexpr int KSTEP = 4 * E;
  constexpr int SP = kTile + Frag<TI>::PAD;
  constexpr int KT = K / 64;
  __shared__ __attribute__((aligned(16))) TI sKt[64 * SP];   // K_c^T tile: [k][j]
  __shared__ __attribute__((aligned(16))) TI sVt[64 * SP];   // (diag(w) V_c)^T tile: [v][j]
  __shared__ __attribute__((aligned(16))) float sw[kTile];

  const int64_t ntile = KT * (a.V / 64);
  const int64_t bh = blockIdx.x / ntile;
  const int tile = (int)(blockIdx.x % ntile);
  const int kt = tile % KT, vt = tile / KT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wk = w & 1, wv = w >> 1;
  const int64_t V = a.V;

  f32x4 acc[2][2];
  float n_reg = 0.f;
  double m_prev = 0.0;
  const bool own_n = (vt == 0) && (tid < 64);
  const int kcol = 64 * kt + tid;   // k handled by own_n threads
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (a.C0) {
    const float* C0 = a.C0 + bh * V * K;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const int kk = 64 * kt + 32 * wk + 16 * x + 4 * lg;
        const int vv = 64 * vt + 32 * wv + 16 * y + l16;
        acc[x][y] = *reinterpret_cast<const f32x4*>(C0 + (int64_t)vv * K + kk);
      }
    if (own_n) n_reg = a.n0[bh * K + kcol];
    m_prev = (double)a.m0[bh];
  }

  const TI* kbase = a.k + bh * a.T * K + 64 * kt;
  const TI* vbase = a.v + bh * a.T * V + 64 * vt;
  for (int64_t c = 0; c < a.Nc; ++c) {
    const int64_t t0 = c * a.L;
    const int Lc = (int)min((int64_t)a.L, a.T - t0);
    if (a.Cs) {
      TS* Cs = a.Cs + (bh * a.Nc + c) * V * K;
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          const int kk = 64 * kt + 32 * wk + 16 * x + 4 * lg;
          const int vv = 64 * vt + 32 * wv + 16 * y + l16;
          store4<TS>(Cs + (int64_t)vv * K + kk, acc[x][y]);
        }
      if (own_n) a.ns[(bh * a.Nc + c) * K + kcol] = n_reg;
      if (tile == 0 && tid == 0) a.ms[bh * a.Nc + c] = m_prev;
    }
    const double gc = a.gb.g[bh * a.Nc + c];
    const double Uc = a.gb.U[bh * a.Nc + c];
    const int Rc = a.gb.R[bh * a.Nc + c];
    double Rm = fmax(Rc >= 0 ? -INFINITY : m_prev, Uc);
    if (Rm == -INFINITY) Rm = 0.0;
    const float decay = Rc >= 0 ? 0.f : expf((float)(m_prev - Rm));
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] *= decay;
    n_reg *= decay;

    for (int j0 = 0; j0 < Lc; j0 += kTile) {
      const int nj = min(kTile, Lc - j0);
      __syncthreads();
      if (tid < kTile) {
        const int j = j0 + tid;
        sw[tid] = (tid < nj && j >= Rc) ? expf((float)(a.gb.u[bh * a.T + t0 + j] - Rm)) : 0.f;
      }
      __syncthreads();
      stage_transposed<64, SP>(sKt, kbase + (t0 + j0) * K, K, nj, nullptr);
      stage_transposed<64, SP>(sVt, vbase + (t0 + j0) * V, V, nj, sw);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kTile; kk += KSTEP) {
        typename Frag<TI>::type A[2], B[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) A[x] = ld_frag<TI>(sKt + (32 * wk + 16 * x + l16) * SP + kk + lg * E);
#pragma unroll
        for (int y = 0; y < 2; ++y) B[y] = ld_frag<TI>(sVt + (32 * wv + 16 * y + l16) * SP + kk + lg * E);
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
          for (int y = 0; y < 2; ++y) acc[x][y] = mma(A[x], B[y], acc[x][y]);
      }
      if (own_n) {
        float s = 0.f;
        for (int j = 0; j < nj; ++j) s += sw[j] * to_f32(sKt[tid * SP + j]);
        n_reg += s;
      }
    }
    m_prev = gc + Rm;
  }

  if (a.C_out) {
    float* Co = a.C_out + bh * V * K;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const int kk = 64 * kt + 32 * wk + 16 * x + 4 * lg;
        const int vv = 64 * vt + 32 * wv + 16 * y + l16;
        *reinterpret_cast<f32x4*>(Co + (int64_t)vv * K + kk) = acc[x][y];
      }
    if (own_n) a.n_out[bh * K + kcol] = n_reg;
    if (tile == 0 && tid == 0) a.m_out[bh] = (float)m_prev;
  }
}

// ------------------------------------------------------------------ output kernel

template <typename TI, typename TS>
struct OutArgs {
  const TI *q, *k, *v, *o;
  TI* h;
  GateBuffers gb;
  const TS* Cs;      // chunk-start states [BH][Nc][V][K], or the initial state [BH][V][K]
  const float* ns;   // [BH][Nc][K] or [BH][K]
  const double* ms;  // [BH][Nc] (chunk-start stabilisers), or null with ms_f set
  const float* ms_f; // [BH] (the caller's initial m) when ms is null
  int64_t cs_chunks; // Nc when Cs holds per-chunk states, 1 for an initial state
  int zero_first;    // per-chunk states only: chunk 0 starts from the zero state
  int64_t T, Nc, V;
  int L;
};

// One workgroup per (head, 64-row query tile, 64*NT value columns). Wave w
// owns all 64 rows of the columns [16 NT w, 16 NT (w+1)) of the block, and
// rows [16 w, 16 w + 16) of the score tile.
template <typename TI, typename TS, int K, int NT>
__global__ __launch_bounds__(kThreads) void out_kernel(OutArgs<TI, TS> a) {
  constexpr int E = Frag<TI>::E;
  constexpr int KSTEP = 4 * E;
  constexpr int QP = K + Frag<TI>::PAD;
  constexpr int TP = kTile + Frag<TI>::PAD;
  constexpr int VB = 64 * NT;
  __shared__ __attribute__((aligned(16))) TI sQ[kTile * QP];
  __shared__ __attribute__((aligned(16))) TI sK[kTile * QP];
  __shared__ __attribute__((aligned(16))) TI sVt[VB * TP];
  __shared__ __attribute__((aligned(16))) TI sP[kTile * TP];
  __shared__ __attribute__((aligned(16))) double s_r[kTile], s_u[kTile];
  __shared__ __attribute__((aligned(16))) float s_sc[kTile], s_fl[kTile], s_dn[kTile], s_di[kTile];
  __shared__ __attribute__((aligned(16))) int s_rs[kTile];

  const int64_t V = a.V, T = a.T;
  const int64_t nvb = V / VB;
  const int64_t nqt = (T + kTile - 1) / kTile;
  const int64_t vb = blockIdx.x % nvb;
  const int64_t qb = (blockIdx.x / nvb) % nqt;
  const int64_t bh = blockIdx.x / (nvb * nqt);
  const int64_t row0 = qb * kTile;
  const int64_t c = row0 / a.L;
  const int64_t t0 = c * a.L;
  const int st = (int)((row0 - t0) / kTile);
  const int nrows = (int)min((int64_t)kTile, T - row0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  const bool has_state = a.Cs != nullptr && (c > 0 || !a.zero_first);
  const int64_t sidx = bh * a.cs_chunks + (a.cs_chunks == 1 ? 0 : c);
  const double m_prev = !has_state ? 0.0 : (a.ms ? a.ms[sidx] : (double)a.ms_f[sidx]);

  if (tid < kTile) {
    double r = 0.0;
    float sc = 0.f, fl = 1.f;
    int rs = 0;
    if (tid < nrows) {
      const int64_t t = bh * T + row0 + tid;
      rs = a.gb.rs[t];
      const bool carry = has_state && rs < 0;
      r = fmax(carry ? m_prev : -INFINITY, a.gb.mp[t]);
      if (r == -INFINITY) r = 0.0;
      sc = carry ? expf((float)(m_prev - r)) : 0.f;
      fl = expf((float)(-(a.gb.b[t] + r)));
    }
    s_r[tid] = r;
    s_sc[tid] = sc;
    s_fl[tid] = fl;
    s_rs[tid] = rs;
  }
  stage_rows<TI, K, QP>(sQ, a.q + (bh * T + row0) * K, K, nrows);
  __syncthreads();

  f32x4 acc[4][NT];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < NT; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int vcol0 = (int)(vb * VB) + w * 16 * NT;

  if (has_state) {
    {  // normaliser term of the carried state: sc_t * (q_t . n~)
      const int row = tid >> 2, part = tid & 3;
      const float* nst = a.ns + sidx * K;
      float d = 0.f;
      for (int kk = part * (K / 4); kk < (part + 1) * (K / 4); ++kk)
        d += to_f32(sQ[row * QP + kk]) * nst[kk];
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      if (part == 0) s_dn[row] = d * s_sc[row];
    }
    const TS* Cst = a.Cs + sidx * V * K;
    for (int kk = 0; kk < K; kk += KSTEP) {
      typename Frag<TI>::type A[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) A[x] = ld_frag<TI>(sQ + (16 * x + l16) * QP + kk + lg * E);
#pragma unroll
      for (int y = 0; y < NT; ++y) {
        const auto B = StateFrag<TI, TS>::load(Cst + (int64_t)(vcol0 + 16 * y + l16) * K + kk + lg * E);
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[x][y] = mma(A[x], B, acc[x][y]);
      }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sc = s_sc[16 * x + 4 * lg + r];
#pragma unroll
        for (int y = 0; y < NT; ++y) acc[x][y][r] *= sc;
      }
  } else if (tid < kTile) {
    s_dn[tid] = 0.f;
  }

  float rsum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int jb = 0; jb <= st; ++jb) {
    const int64_t key0 = t0 + (int64_t)jb * kTile;
    const int nkeys = (int)min((int64_t)kTile, T - key0);
    __syncthreads();
    stage_rows<TI, K, QP>(sK, a.k + (bh * T + key0) * K, K, nkeys);
    stage_transposed<VB, TP>(sVt, a.v + (bh * T + key0) * V + vb * VB, V, nkeys, nullptr);
    if (tid < kTile) s_u[tid] = tid < nkeys ? a.gb.u[bh * T + key0 + tid] : -INFINITY;
    __syncthreads();

    f32x4 sacc[4];
#pragma unroll
    for (int y = 0; y < 4; ++y) sacc[y] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kk = 0; kk < K; kk += KSTEP) {
      const auto A = ld_frag<TI>(sQ + (16 * w + l16) * QP + kk + lg * E);
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const auto B = ld_frag<TI>(sK + (16 * y + l16) * QP + kk + lg * E);
        sacc[y] = mma(A, B, sacc[y]);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = 16 * w + 4 * lg + r;
      const int tq = st * kTile + tl;
      const double rr = s_r[tl];
      const int rs = s_rs[tl];
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int jl = 16 * y + l16;
        const int jk = jb * kTile + jl;
        const bool keep = (tl < nrows) && (jk <= tq) && (jk >= rs);
        const float p = keep ? sacc[y][r] * expf((float)(s_u[jl] - rr)) : 0.f;
        rsum[r] += p;
        sP[tl * TP + jl] = from_f32<TI>(p);
      }
    }
    __syncthreads();
    for (int jj = 0; jj < kTile; jj += KSTEP) {
      typename Frag<TI>::type A[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) A[x] = ld_frag<TI>(sP + (16 * x + l16) * TP + jj + lg * E);
#pragma unroll
      for (int y = 0; y < NT; ++y) {
        const auto B = ld_frag<TI>(sVt + (w * 16 * NT + 16 * y + l16) * TP + jj + lg * E);
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[x][y] = mma(A[x], B, acc[x][y]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float x = rsum[r];
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    if (l16 == 0) s_di[16 * w + 4 * lg + r] = x;
  }
  __syncthreads();

#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = 16 * x + 4 * lg + r;
      if (tl >= nrows) continue;
      const float den = s_di[tl] + s_dn[tl];
      const float inv = 1.f / fmaxf(fmaxf(fabsf(den), s_fl[tl]), FLT_MIN);
      const int64_t rowoff = (bh * T + row0 + tl) * V;
#pragma unroll
      for (int y = 0; y < NT; ++y) {
        const int64_t idx = rowoff + vcol0 + 16 * y + l16;
        const float og = sigmoid(to_f32(a.o[idx]));
        a.h[idx] = from_f32<TI>(og * acc[x][y][r] * inv);
      }
    }
}

// ------------------------------------------------------------------ T = 0 state copy

__global__ void copy_state_kernel(const float* C0, const float* n0, const float* m0, float* C, float* n,
                                  float* m, int64_t nC, int64_t nn, int64_t nm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nC) C[i] = C0 ? C0[i] : 0.f;
  if (i < nn) n[i] = n0 ? n0[i] : 0.f;
  if (i < nm) m[i] = m0 ? m0[i] : 0.f;
}

// ------------------------------------------------------------------ decode step

template <typename TI>
struct StepArgs {
  const TI *q, *k, *v, *o;
  const float *i_pre, *f_pre;
  float* C;
  const float *n_in, *m_in;
  float *n_out, *m_out;
  TI* h;
  int64_t V;
};

template <typename TI, int VEC>
__device__ __forceinline__ void load_vec(const TI* p, float* out) {
#pragma unroll
  for (int e = 0; e < VEC; ++e) out[e] = to_f32(p[e]);
}

// VEC consecutive floats with the widest aligned vector loads.
template <int VEC>
__device__ __forceinline__ void load_f32(const float* p, float* out) {
  if constexpr (VEC % 4 == 0) {
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(p + e);
      out[e] = x[0]; out[e + 1] = x[1]; out[e + 2] = x[2]; out[e + 3] = x[3];
    }
  } else if constexpr (VEC % 2 == 0) {
#pragma unroll
    for (int e = 0; e < VEC; e += 2) {
      const f32x2 x = *reinterpret_cast<const f32x2*>(p + e);
      out[e] = x[0]; out[e + 1] = x[1];
    }
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) out[e] = p[e];
  }
}
template <int VEC>
__device__ __forceinline__ void store_f32(float* p, const float* in) {
  if constexpr (VEC % 4 == 0) {
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      *reinterpret_cast<f32x4*>(p + e) = f32x4{in[e], in[e + 1], in[e + 2], in[e + 3]};
  } else if constexpr (VEC % 2 == 0) {
#pragma unroll
    for (int e = 0; e < VEC; e += 2) *reinterpret_cast<f32x2*>(p + e) = f32x2{in[e], in[e + 1]};
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) p[e] = in[e];
  }
}

// One workgroup per (head, 4*RPW rows of C). Lane l owns the d_qk columns
// [VEC l, VEC l + VEC) of every row; wave w owns RPW consecutive rows.
template <typename TI, int K, int RPW>
__global__ __launch_bounds__(kThreads) void step_kernel(StepArgs<TI> a) {
  constexpr int VEC = K / 64;
  const int64_t V = a.V;
  const int64_t nvb = (V + 4 * RPW - 1) / (4 * RPW);
  const int64_t vb = blockIdx.x % nvb;
  const int64_t bh = blockIdx.x / nvb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t row0 = vb * 4 * RPW + w * RPW;

  const float lf = log_sigmoid(a.f_pre[bh]);
  const float mi = a.m_in[bh];
  const float ig = a.i_pre[bh];
  const float m_new = fmaxf(lf + mi, ig);
  const float fa = expf(lf + mi - m_new);
  const float fb = expf(ig - m_new);

  float q[VEC], kv[VEC], nn[VEC];
  load_vec<TI, VEC>(a.q + bh * K + lane * VEC, q);
  load_vec<TI, VEC>(a.k + bh * K + lane * VEC, kv);
  load_f32<VEC>(a.n_in + bh * K + lane * VEC, nn);
#pragma unroll
  for (int e = 0; e < VEC; ++e) nn[e] = fa * nn[e] + fb * kv[e];
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) dot += nn[e] * q[e];
  dot = wave_sum(dot);
  const float inv = 1.f / fmaxf(fmaxf(fabsf(dot), expf(-m_new)), FLT_MIN);
  if (vb == 0 && w == 0) {
    store_f32<VEC>(a.n_out + bh * K + lane * VEC, nn);
    if (lane == 0) a.m_out[bh] = m_new;
  }

  float cr[RPW][VEC];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int64_t row = row0 + i;
    if (row < V) load_f32<VEC>(a.C + (bh * V + row) * K + lane * VEC, cr[i]);
  }
  float mine = 0.f;
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int64_t row = row0 + i;
    if (row >= V) break;
    const float vv = fb * to_f32(a.v[bh * V + row]);
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      cr[i][e] = fa * cr[i][e] + vv * kv[e];
      part += cr[i][e] * q[e];
    }
    store_f32<VEC>(a.C + (bh * V + row) * K + lane * VEC, cr[i]);
    part = wave_sum(part);
    if (lane == i) mine = part;
  }
  if (lane < RPW && row0 + lane < V) {
    const int64_t idx = bh * V + row0 + lane;
    a.h[idx] = from_f32<TI>(sigmoid(to_f32(a.o[idx])) * mine * inv);
  }
}

// ------------------------------------------------------------------ dispatch helpers

template <typename TI, typename TS, int K>
hipError_t run_state(const FwdLaunch& f, const GateBuffers& gb, const ChunkStates& cs, hipStream_t s) {
  StateArgs<TI, TS> a;
  a.k = static_cast<const TI*>(f.k);
  a.v = static_cast<const TI*>(f.v);
  a.gb = gb;
  a.C0 = f.C0; a.n0 = f.n0; a.m0 = f.m0;
  a.Cs = static_cast<TS*>(cs.Cs);
  a.ns = cs.ns; a.ms = cs.ms;
  a.C_out = f.C_out; a.n_out = f.n_out; a.m_out = f.m_out;
  a.T = f.T; a.Nc = f.Nc; a.V = f.V; a.L = f.L;
  const int64_t grid = f.BH * (K / 64) * (f.V / 64);
  mark_before(f.marks, K_STATE, s);
  hipLaunchKernelGGL((state_kernel<TI, TS, K>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  mark_after(f.marks, K_STATE, s);
  return hipGetLastError();
}

template <typename TI, typename TS, int K, int NT>
hipError_t run_out(const FwdLaunch& f, const GateBuffers& gb, const void* Cs, const float* ns,
                   const double* ms, const float* ms_f, int64_t cs_chunks, hipStream_t s) {
  OutArgs<TI, TS> a;
  a.q = static_cast<const TI*>(f.q);
  a.k = static_cast<const TI*>(f.k);
  a.v = static_cast<const TI*>(f.v);
  a.o = static_cast<const TI*>(f.o);
  a.h = static_cast<TI*>(f.h);
  a.gb = gb;
  a.Cs = static_cast<const TS*>(Cs);
  a.ns = ns; a.ms = ms; a.ms_f = ms_f; a.cs_chunks = cs_chunks;
  a.zero_first = (f.C0 == nullptr);
  a.T = f.T; a.Nc = f.Nc; a.V = f.V; a.L = f.L;
  const int64_t nqt = (f.T + kTile - 1) / kTile;
  const int64_t grid = f.BH * nqt * (f.V / (64 * NT));
  mark_before(f.marks, K_OUT, s);
  hipLaunchKernelGGL((out_kernel<TI, TS, K, NT>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  mark_after(f.marks, K_OUT, s);
  return hipGetLastError();
}

template <typename TI, typename TS, int K>
hipError_t run_out_nt(const FwdLaunch& f, const GateBuffers& gb, const void* Cs, const float* ns,
                      const double* ms, const float* ms_f, int64_t cs_chunks, hipStream_t s) {
  const int64_t nv = f.V / 64;
  if (nv % 4 == 0) return run_out<TI, TS, K, 4>(f, gb, Cs, ns, ms, ms_f, cs_chunks, s);
  if (nv % 2 == 0) return run_out<TI, TS, K, 2>(f, gb, Cs, ns, ms, ms_f, cs_chunks, s);
  return run_out<TI, TS, K, 1>(f, gb, Cs, ns, ms, ms_f, cs_chunks, s);
}

// fp32 at d_qk = 128 with four 64-column blocks is the largest tile that fits
// the 160 KiB of LDS; keep fp32 to two blocks for headroom.
template <typename TS, int K>
hipError_t run_out_fp32(const FwdLaunch& f, const GateBuffers& gb, const void* Cs, const float* ns,
                        const double* ms, const float* ms_f, int64_t cs_chunks, hipStream_t s) {
  const int64_t nv = f.V / 64;
  if (nv % 2 == 0) return run_out<float, TS, K, 2>(f, gb, Cs, ns, ms, ms_f, cs_chunks, s);
  return run_out<float, TS, K, 1>(f, gb, Cs, ns, ms, ms_f, cs_chunks, s);
}

template <typename TI, int K>
hipError_t run_step(const StepLaunch& st, hipStream_t s) {
  constexpr int RPW = 8;
  StepArgs<TI> a;
  a.q = static_cast<const TI*>(st.q);
  a.k = static_cast<const TI*>(st.k);
  a.v = static_cast<const TI*>(st.v);
  a.o = static_cast<const TI*>(st.o);
  a.i_pre = st.i_pre; a.f_pre = st.f_pre;
  a.C = st.C; a.n_in = st.n_in; a.m_in = st.m_in; a.n_out = st.n_out; a.m_out = st.m_out;
  a.h = static_cast<TI*>(st.h);
  a.V = st.V;
  const int64_t nvb = (st.V + 4 * RPW - 1) / (4 * RPW);
  const int64_t grid = st.BH * nvb;
  mark_before(st.marks, K_STEP, s);
  hipLaunchKernelGGL((step_kernel<TI, K, RPW>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  mark_after(st.marks, K_STEP, s);
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_gate(const FwdLaunch& f, const GateBuffers& gb, hipStream_t s) {
  GateArgs a;
  a.i_pre = f.i_pre;
  a.f_pre = f.f_pre;
  a.T = f.T; a.Nc = f.Nc; a.BH = f.BH; a.L = f.L;
  a.gb = gb;
  mark_before(f.marks, K_GATE, s);
  if (f.L == kTile)
    hipLaunchKernelGGL(gate64_kernel, dim3((unsigned)((f.BH * f.Nc + 3) / 4)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(gate_kernel, dim3((unsigned)(f.BH * f.Nc)), dim3(kThreads), 0, s, a);
  mark_after(f.marks, K_GATE, s);
  return hipGetLastError();
}

hipError_t launch_state(const FwdLaunch& f, const GateBuffers& gb, const ChunkStates& cs, hipStream_t s) {
  if (f.bf16) return launch_state_bf16(f, gb, cs, s);
  {
    switch (f.K) {
      case 64: return run_state<float, float, 64>(f, gb, cs, s);
      case 128: return run_state<float, float, 128>(f, gb, cs, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_out(const FwdLaunch& f, const GateBuffers& gb, const ChunkStates& cs, hipStream_t s) {
  if (bf16_fast_path(f)) return launch_out_bf16(f, gb, cs, s);
  if (cs.Cs) {   // per-chunk states from the state pass
    if (f.bf16) {
      switch (f.K) {
        case 64: return run_out_nt<__bf16, __bf16, 64>(f, gb, cs.Cs, cs.ns, cs.ms, nullptr, f.Nc, s);
        case 128: return run_out_nt<__bf16, __bf16, 128>(f, gb, cs.Cs, cs.ns, cs.ms, nullptr, f.Nc, s);
        case 256: return run_out_nt<__bf16, __bf16, 256>(f, gb, cs.Cs, cs.ns, cs.ms, nullptr, f.Nc, s);
      }
    } else {
      switch (f.K) {
        case 64: return run_out_fp32<float, 64>(f, gb, cs.Cs, cs.ns, cs.ms, nullptr, f.Nc, s);
        case 128: return run_out_fp32<float, 128>(f, gb, cs.Cs, cs.ns, cs.ms, nullptr, f.Nc, s);
      }
    }
  } else {       // one chunk; carried state = the caller's float32 initial state (or none)
    if (f.bf16) {
      switch (f.K) {
        case 64: return run_out_nt<__bf16, float, 64>(f, gb, f.C0, f.n0, nullptr, f.m0, 1, s);
        case 128: return run_out_nt<__bf16, float, 128>(f, gb, f.C0, f.n0, nullptr, f.m0, 1, s);
        case 256: return run_out_nt<__bf16, float, 256>(f, gb, f.C0, f.n0, nullptr, f.m0, 1, s);
      }
    } else {
      switch (f.K) {
        case 64: return run_out_fp32<float, 64>(f, gb, f.C0, f.n0, nullptr, f.m0, 1, s);
        case 128: return run_out_fp32<float, 128>(f, gb, f.C0, f.n0, nullptr, f.m0, 1, s);
      }
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_copy_state(const FwdLaunch& f, hipStream_t s) {
  if (!f.C_out) return hipSuccess;
  const int64_t nC = f.BH * f.V * f.K;
  const int64_t blocks = (nC + 255) / 256;
  hipLaunchKernelGGL(copy_state_kernel, dim3((unsigned)blocks), dim3(256), 0, s, f.C0, f.n0, f.m0,
                     f.C_out, f.n_out, f.m_out, nC, f.BH * f.K, f.BH);
  return hipGetLastError();
}

// Clock probe: one wave that sleeps `iters` times s_sleep 127 (about 8k
// shader cycles each) and records the shader-clock counter (s_memtime) and
// the constant-rate counter (s_memrealtime) before and after. Launched beside
// other work, the two differences give the shader clock under that work.
__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* ticks, int iters) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) __builtin_amdgcn_s_sleep(127);
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    ticks[0] = t0;
    ticks[1] = t1;
    ticks[2] = r0;
    ticks[3] = r1;
  }
}

// Direct-to-LDS copy (counter calibration): each workgroup of 256 threads
// moves 16 KiB per iteration; every lane issues four 16-byte global_load_lds
// (the same instruction the fused kernels stage their tiles with), then the
// tile is read back from LDS and stored with 16-byte vector stores.
typedef __attribute__((address_space(1))) void cal_global_void;
typedef __attribute__((address_space(3))) void cal_lds_void;
__global__ __launch_bounds__(256) void lds_copy_kernel(const char* src, char* dst, int64_t nblk) {
  __shared__ __attribute__((aligned(16))) char buf[16384];
  const int tid = threadIdx.x, w = tid >> 6;
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const char* s = src + blk * 16384;
    char* d = dst + blk * 16384;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      __builtin_amdgcn_global_load_lds((cal_global_void*)(s + k * 4096 + tid * 16),
                                       (cal_lds_void*)(buf + k * 4096 + w * 1024), 16, 0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<f32x4*>(d + k * 4096 + tid * 16) = *reinterpret_cast<const f32x4*>(buf + k * 4096 + tid * 16);
    __syncthreads();
  }
}

hipError_t launch_lds_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t nblk = bytes / 16384;
  const int64_t grid = nblk < 2048 ? nblk : 2048;
  hipLaunchKernelGGL(lds_copy_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const char*>(src),
                     static_cast<char*>(dst), nblk);
  return hipGetLastError();
}

hipError_t launch_clock_probe(unsigned long long* ticks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, s, ticks, iters);
  return hipGetLastError();
}

hipError_t launch_step(const StepLaunch& st, hipStream_t s) {
#define MLSTM_STEP_CASE(KK)                                        \
  case KK:                                                         \
    return st.bf16 ? run_step<__bf16, KK>(st, s) : run_step<float, KK>(st, s);
  switch (st.K) {
    MLSTM_STEP_CASE(64)
    MLSTM_STEP_CASE(128)
    MLSTM_STEP_CASE(192)
    MLSTM_STEP_CASE(256)
    MLSTM_STEP_CASE(320)
    MLSTM_STEP_CASE(384)
    MLSTM_STEP_CASE(448)
    MLSTM_STEP_CASE(512)
  }
#undef MLSTM_STEP_CASE
  return hipErrorInvalidValue;
}

}  // namespace mlstm_impl
