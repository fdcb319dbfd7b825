// Fused chunkwise forward of the mLSTM cell for bfloat16 inputs on gfx950.
//
// Same mathematics as the two-pass kernels (xLSTM guide, aifetchly blog:
// recurrence of "mLSTM: Matrix Key-Value Memory and Covariance Updates",
// running max of "The Stabilizer State", decay matrix of "The Dual
// Formulation", chunking of "Exploit Chunkwise Hardware Kernels for Production
// Training"), organised so that the d_v x d_qk state never leaves the chip
// inside a chunk:
//
//   seg_kernel<LOCAL>  one workgroup per (head, 128 value columns, chunk).
//                      Holds its 128 x d_qk slice of C~ (float32) in MFMA
//                      accumulators and walks the chunk in 64-token tiles.
//                      Per tile: Q K^T on MFMA, decay mask and stabiliser in
//                      registers, P V and Q C~^T on MFMA, normaliser and output
//                      gate, then C~ <- a C~ + K^T diag(w) V on MFMA and the
//                      same for n~ (a two-column MFMA tile carrying the weights
//                      as bf16 hi + lo). The LOCAL variant only accumulates the
//                      chunk's own end state from zero (no outputs).
//   seg_combine_kernel folds the chunks' local end states in order into the
//                      start state of every chunk (elementwise, float32).
//
// Chunks are independent given their start states, so the sequence dimension
// supplies the parallelism that the few heads of a large layer lack.

#include "mlstm_device.h"

namespace mlstm_impl {

namespace {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kVB = 128;                     // value columns per workgroup
constexpr double kMaxDefer = 50.0;           // largest pending log decay kept out of the accumulators
constexpr float kLog2eF = 1.4426950408889634f;

// Transposed operand fragment from a row-major LDS tile X (row pitch P):
// lane l (i = l%16, g = l/16) receives X[kin0 + 8g + e][n0 + i], e = 0..7.
// ds_read_b64_tr_b16 hands lane i of each 16-lane group element (i mod 4) of
// the 8-byte rows addressed by lanes 4e + i/4 of that group.
__device__ __forceinline__ bf16x8 frag_tr(const __bf16* X, int P, int kin0, int n0) {
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  const __bf16* p = X + (kin0 + 8 * g + (i >> 2)) * P + n0 + 4 * (i & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * P));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row-major operand fragment whose contraction index follows the accumulator
// layout of C^T: lane (g, i) receives X[row][k0 + 4g + e] for e = 0..3 and
// X[row][k0 + 16 + 4g + e - 4] for e = 4..7. A contraction is a sum, so any
// permutation of its index works as long as both operands use it.
__device__ __forceinline__ bf16x8 frag_split(const __bf16* X, int P, int row, int k0) {
  const int g = (threadIdx.x & 63) >> 4;
  const __bf16* p = X + row * P + k0 + 4 * g;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 pack_bf16(f32x4 a, f32x4 b) {
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
  r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
  return r;
}

template <typename F, int... S>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl(f, std::make_integer_sequence<int, N>{});
}

struct SegArgs {
  const __bf16 *q, *k, *v, *o;
  __bf16* h;
  GateBuffers gb;            // per 64-token tile
  const float *C0, *n0, *m0;
  float* Cseg;               // [BH][S-1][V][K]: chunk-local end states, then start states of chunks 1..S-1
  float* nseg;               // [BH][S-1][K]
  double* mloc;              // [BH][S-1] local end stabiliser
  double* mstart;            // [BH][S-1] stabiliser at the start of chunks 1..S-1
  double* Gseg;              // [BH][S-1] sum of log f over the chunk, -inf when it holds a zero forget gate
  float *C_out, *n_out, *m_out;
  int64_t T, Nt, V, BH;      // Nt = number of 64-token tiles
  int TPS;                   // tiles per chunk
  int S;                     // chunks
};

template <int K, bool LOCAL>
struct SegLds {
  static constexpr int QP = K + 16;       // sQ/sK row pitch: 8 dwords mod 32 banks
  static constexpr int VP = kVB + 16;     // sV row pitch
  static constexpr int OP = kVB + 8;      // sO row pitch
  static constexpr int PP = kTile + 8;    // sP row pitch
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + (LOCAL ? 0 : kTile * QP * 2);
  static constexpr int oV = oK + kTile * QP * 2;
  static constexpr int oO = oV + kTile * VP * 2;
  static constexpr int oP = oO + (LOCAL ? 0 : kTile * OP * 2);
  static constexpr int oN = oP + (LOCAL ? 0 : kTile * PP * 2);
  static constexpr int oW = oN + (LOCAL ? 0 : K * 4);
  static constexpr int oRow = oW + kTile * 4;
  static constexpr int oDen = oRow + (LOCAL ? 0 : 5 * kTile * 4);
  static constexpr int bytes = oDen + (LOCAL ? 0 : 8 * kTile * 4);
};

// Wave w owns value columns [32 w, 32 w + 32) of the workgroup's 128 and
// keeps C~^T[k][v] for all k of them: register r of Ct[kx][y] in lane (g, i)
// is k = 16 kx + 4 g + r, v = 32 w + 16 y + i. The normaliser is carried in
// Nacc: for k = 16 kx + 4 g + r with kx in this wave's quarter, lane i = 0
// holds the part weighted by the bf16 high halves of the weights and lane
// i = 1 the part weighted by the low halves; n~ is their sum.
template <int K, bool LOCAL>
__global__ __launch_bounds__(kThreads, 1) void seg_kernel(SegArgs a) {
  using L = SegLds<K, LOCAL>;
  constexpr int QP = L::QP, VP = L::VP, OP = L::OP, PP = L::PP;
  constexpr int KS = K / 32;     // 32-deep steps over d_qk
  constexpr int KX = K / 16;     // 16-row tiles of C^T along d_qk
  constexpr int KXW = KX / 4;    // normaliser tiles per wave
  constexpr int QV = K / 32;     // 16-byte vectors per thread of a 64 x K tile
  constexpr int VV = 4;          // 16-byte vectors per thread of a 64 x 128 tile
  __shared__ __attribute__((aligned(16))) char smem[L::bytes];
  __bf16* sQ = reinterpret_cast<__bf16*>(smem + L::oQ);
  __bf16* sK = reinterpret_cast<__bf16*>(smem + L::oK);
  __bf16* sV = reinterpret_cast<__bf16*>(smem + L::oV);
  __bf16* sO = reinterpret_cast<__bf16*>(smem + L::oO);
  __bf16* sP = reinterpret_cast<__bf16*>(smem + L::oP);
  float* sn = reinterpret_cast<float*>(smem + L::oN);
  float* s_w = reinterpret_cast<float*>(smem + L::oW);
  float* s_r2 = reinterpret_cast<float*>(smem + L::oRow);
  float* s_sc = s_r2 + kTile;
  float* s_fl = s_sc + kTile;
  float* s_u2 = s_fl + kTile;
  int* s_rs = reinterpret_cast<int*>(s_u2 + kTile);
  float* s_den = reinterpret_cast<float*>(smem + L::oDen);   // [4][64] row sums of P per wave
  float* s_dn = s_den + 4 * kTile;                           // [4][64] q . n~ partials per wave

  const int64_t BH = a.BH, T = a.T, V = a.V, Nt = a.Nt;
  const int nvb = (int)(V / kVB);
  const int64_t bh = blockIdx.x % BH;
  const int64_t rest = blockIdx.x / BH;
  const int vb = (int)(rest % nvb);
  const int seg = (int)(rest / nvb);
  const int64_t tile0 = (int64_t)seg * a.TPS;
  const int64_t tile1 = min(tile0 + a.TPS, Nt);
  // The wave index is made a scalar so that branches on it are scalar
  // branches: an MFMA is not masked by EXEC, so an MFMA that only some waves
  // may run must sit behind a real branch.
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int64_t vcol0 = (int64_t)vb * kVB;
  const int64_t nseg1 = a.S - 1;

  // ---------------- carried state
  f32x4 Ct[KX][2];
  f32x4 Nacc[KXW];
  double m_prev;
  bool has_state;
  const float* Cinit = nullptr;
  const float* ninit = nullptr;
  if constexpr (LOCAL) {
    m_prev = -INFINITY;   // empty: the local state starts from nothing
    has_state = false;
  } else if (seg == 0) {
    Cinit = a.C0 ? a.C0 + bh * V * K : nullptr;
    ninit = a.C0 ? a.n0 + bh * K : nullptr;
    m_prev = a.C0 ? (double)a.m0[bh] : 0.0;
    has_state = a.C0 != nullptr;
  } else {
    const int64_t sidx = bh * nseg1 + seg - 1;
    Cinit = a.Cseg + sidx * V * K;
    ninit = a.nseg + sidx * K;
    m_prev = a.mstart[sidx];
    has_state = true;
  }
#pragma unroll
  for (int kx = 0; kx < KX; ++kx)
#pragma unroll
    for (int y = 0; y < 2; ++y)
      Ct[kx][y] = Cinit ? *reinterpret_cast<const f32x4*>(Cinit + (vcol0 + 32 * w + 16 * y + i) * K + 16 * kx + 4 * g)
                        : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < KXW; ++x) {
    const int kx = w * KXW + x;
    Nacc[x] = (ninit && i == 0) ? *reinterpret_cast<const f32x4*>(ninit + 16 * kx + 4 * g)
                                : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // The tiles' decays are not applied to the accumulators one by one (a VALU
  // pass over 128 accumulator registers per tile): the registers hold X with
  // C~ = exp(logD) X, n~ = exp(logD) Xn, new keys enter with weight
  // exp(u_j - Rm - logD), and X is rescaled only when logD would fall below
  // -kMaxDefer (or on a zero decay).
  double logD = 0.0;
  double Gsum = 0.0;
  bool reset_seen = false;

  // ---------------- next-tile registers; loads are unconditional (rows clamped
  // into the tile) so that no branch forces the load counter to drain
  bf16x8 pq[QV], pk[QV], pv[VV], po[VV];
  double r_u = 0.0, r_mp = 0.0, r_b = 0.0, r_mp0 = 0.0;
  int r_rs = -1, r_rs0 = -1;
  double t_g = 0.0, t_U = 0.0;
  int t_R = -1;
  auto issue = [&](int64_t tau) {
    const int64_t t0 = tau * kTile;
    const int last = (int)min((int64_t)kTile, T - t0) - 1;
    const int64_t tok0 = bh * T + t0;
#pragma unroll
    for (int e = 0; e < QV; ++e) {
      const int it = tid + kThreads * e;
      const int row = min(it / (K / 8), last), cv = it % (K / 8);
      if constexpr (!LOCAL) pq[e] = *reinterpret_cast<const bf16x8*>(a.q + (tok0 + row) * K + 8 * cv);
      pk[e] = *reinterpret_cast<const bf16x8*>(a.k + (tok0 + row) * K + 8 * cv);
    }
#pragma unroll
    for (int e = 0; e < VV; ++e) {
      const int it = tid + kThreads * e;
      const int row = min(it / (kVB / 8), last), cv = it % (kVB / 8);
      pv[e] = *reinterpret_cast<const bf16x8*>(a.v + (tok0 + row) * V + vcol0 + 8 * cv);
      if constexpr (!LOCAL) po[e] = *reinterpret_cast<const bf16x8*>(a.o + (tok0 + row) * V + vcol0 + 8 * cv);
    }
    const int j = min(lane, last);
    r_u = a.gb.u[tok0 + j];
    if constexpr (!LOCAL) {
      r_mp = a.gb.mp[tok0 + j];
      r_b = a.gb.b[tok0 + j];
      r_rs = a.gb.rs[tok0 + j];
      r_mp0 = a.gb.mp[tok0];
      r_rs0 = a.gb.rs[tok0];
    }
    t_g = a.gb.g[bh * Nt + tau];
    t_U = a.gb.U[bh * Nt + tau];
    t_R = a.gb.R[bh * Nt + tau];
  };

  issue(tile0);
  for (int64_t tau = tile0; tau < tile1; ++tau) {
    const int64_t t0 = tau * kTile;
    const int Lc = (int)min((int64_t)kTile, T - t0);
    const int64_t tok0 = bh * T + t0;

    __syncthreads();   // the previous tile's LDS reads are done
    // ---------------- stage tile tau
#pragma unroll
    for (int e = 0; e < QV; ++e) {
      const int it = tid + kThreads * e;
      const int row = it / (K / 8), cv = it % (K / 8);
      if constexpr (!LOCAL) *reinterpret_cast<bf16x8*>(&sQ[row * QP + 8 * cv]) = pq[e];
      *reinterpret_cast<bf16x8*>(&sK[row * QP + 8 * cv]) = pk[e];
    }
#pragma unroll
    for (int e = 0; e < VV; ++e) {
      const int it = tid + kThreads * e;
      const int row = it / (kVB / 8), cv = it % (kVB / 8);
      *reinterpret_cast<bf16x8*>(&sV[row * VP + 8 * cv]) = pv[e];
      if constexpr (!LOCAL) *reinterpret_cast<bf16x8*>(&sO[row * OP + 8 * cv]) = po[e];
    }
    // tile scalars of the state update: Rm = max(m_prev, U) (U alone after a
    // zero forget gate), decay exp(m_prev - Rm), key weights exp(u_j - Rm)
    double Rm = fmax(t_R >= 0 ? -INFINITY : m_prev, t_U);
    if constexpr (!LOCAL) {
      if (Rm == -INFINITY) Rm = 0.0;
    }
    const bool live = Rm != -INFINITY;
    const double ld = (t_R >= 0 || m_prev == -INFINITY || !live) ? -INFINITY : m_prev - Rm;
    const double m_next = live ? t_g + Rm : -INFINITY;
    // deferred decay after this tile: keep logD + ld, or rescale X by it
    const bool rescale = logD + ld < -kMaxDefer;
    const double logD_next = rescale ? 0.0 : logD + ld;
    if (tid < kTile) {
      const int j = tid;
      s_w[j] = (j >= t_R && j < Lc && t_U != -INFINITY && live) ? expf((float)(r_u - Rm - logD_next)) : 0.f;
      if constexpr (!LOCAL) {
        // row stabiliser r_t = max(m_prev if no zero gate at or before t, prefix max of u)
        const bool carry0 = has_state && r_rs0 < 0;
        double ref = fmax(carry0 ? m_prev : -INFINITY, r_mp0);
        if (ref == -INFINITY) ref = 0.0;
        const bool valid = j < Lc;
        const bool carry = has_state && r_rs < 0;
        double r = fmax(carry ? m_prev : -INFINITY, r_mp);
        if (r == -INFINITY) r = 0.0;
        s_r2[j] = valid ? (float)((r - ref) * (double)kLog2eF) : 0.f;
        s_sc[j] = (valid && carry) ? expf((float)(m_prev - r + logD)) : 0.f;
        s_fl[j] = valid ? expf((float)(-(r_b + r))) : 1.f;
        s_rs[j] = r_rs;
        s_u2[j] = valid ? (float)((r_u - ref) * (double)kLog2eF) : -INFINITY;
      }
    }
    if constexpr (!LOCAL) {
      // n~ for the q . n~ term of this tile
#pragma unroll
      for (int x = 0; x < KXW; ++x) {
        f32x4 nv;
#pragma unroll
        for (int r = 0; r < 4; ++r) nv[r] = Nacc[x][r] + __shfl_xor(Nacc[x][r], 1, 64);
        if (i == 0) *reinterpret_cast<f32x4*>(&sn[16 * (w * KXW + x) + 4 * g]) = nv;
      }
    }
    if constexpr (LOCAL) {
      Gsum += t_g;
      reset_seen = reset_seen || t_R >= 0;
    }
    __syncthreads();   // tile tau staged
    if (tau + 1 < tile1) issue(tau + 1);

    if constexpr (!LOCAL) {
      // ---------------- Q K^T (this wave's 16 keys x 64 rows), Q C~^T, q . n~
      f32x4 sacc[4], acc[4][2], dacc[4];
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        sacc[z] = dacc[z] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc[z][0] = acc[z][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      unroll<KS>([&](auto s_c) {
        constexpr int s = decltype(s_c)::value;
        bf16x8 A[4];
#pragma unroll
        for (int z = 0; z < 4; ++z) A[z] = frag_split(sQ, QP, 16 * z + i, 32 * s);
        const bf16x8 Kf = frag_split(sK, QP, 16 * w + i, 32 * s);
#pragma unroll
        for (int z = 0; z < 4; ++z) sacc[z] = mma(Kf, A[z], sacc[z]);
        bf16x8 Bc[2];
#pragma unroll
        for (int y = 0; y < 2; ++y) Bc[y] = pack_bf16(Ct[2 * s][y], Ct[2 * s + 1][y]);
#pragma unroll
        for (int z = 0; z < 4; ++z)
#pragma unroll
          for (int y = 0; y < 2; ++y) acc[z][y] = mma(A[z], Bc[y], acc[z][y]);
        if (w == (s & 3)) {
          const f32x4 n0v = *reinterpret_cast<const f32x4*>(&sn[32 * s + 4 * g]);
          const f32x4 n1v = *reinterpret_cast<const f32x4*>(&sn[32 * s + 16 + 4 * g]);
          bf16x8 Bn;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float nval = e < 4 ? n0v[e] : n1v[e - 4];
            const __bf16 hi = (__bf16)nval;
            const __bf16 lo = (__bf16)(nval - (float)hi);
            Bn[e] = i == 0 ? hi : (i == 1 ? lo : (__bf16)0.f);
          }
#pragma unroll
          for (int z = 0; z < 4; ++z) dacc[z] = mma(A[z], Bn, dacc[z]);
        }
      });
      // q . n~ partial of this wave (normaliser columns hi + lo)
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        f32x4 d;
#pragma unroll
        for (int r = 0; r < 4; ++r) d[r] = dacc[z][r] + __shfl_xor(dacc[z][r], 1, 64);
        if (i == 0) *reinterpret_cast<f32x4*>(&s_dn[w * kTile + 16 * z + 4 * g]) = d;
      }
      // the carried-state term enters row t with weight exp(m_prev - r_t)
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const f32x4 sc = *reinterpret_cast<const f32x4*>(&s_sc[16 * z + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[z][0][r] *= sc[r];
          acc[z][1][r] *= sc[r];
        }
      }
      // ---------------- P = S o D: lane holds S^T[j = 16 w + 4 g + r][t = 16 z + i]
      const f32x4 u2 = *reinterpret_cast<const f32x4*>(&s_u2[16 * w + 4 * g]);
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const int tl = 16 * z + i;
        const float r2 = s_r2[tl];
        const int rs = s_rs[tl];
        bf16x4 pk4;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jk = 16 * w + 4 * g + r;
          const bool keep = (tl < Lc) && (jk <= tl) && (jk >= rs);
          const float p = keep ? sacc[z][r] * __builtin_amdgcn_exp2f(u2[r] - r2) : 0.f;
          psum += p;
          pk4[r] = (__bf16)p;
        }
        *reinterpret_cast<bf16x4*>(&sP[tl * PP + 16 * w + 4 * g]) = pk4;
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        if (g == 0) s_den[w * kTile + tl] = psum;
      }
      __syncthreads();   // sP, s_den, s_dn complete
      // ---------------- P V
#pragma unroll
      for (int jj = 0; jj < kTile; jj += 32) {
        bf16x8 A[4], B[2];
#pragma unroll
        for (int z = 0; z < 4; ++z) A[z] = *reinterpret_cast<const bf16x8*>(&sP[(16 * z + i) * PP + jj + 8 * g]);
#pragma unroll
        for (int y = 0; y < 2; ++y) B[y] = frag_tr(sV, VP, jj, 32 * w + 16 * y);
#pragma unroll
        for (int z = 0; z < 4; ++z)
#pragma unroll
          for (int y = 0; y < 2; ++y) acc[z][y] = mma(A[z], B[y], acc[z][y]);
      }
      // ---------------- normaliser, output gate; h staged in place of O
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const int t4 = 16 * z + 4 * g;
        f32x4 den = *reinterpret_cast<const f32x4*>(&s_den[t4]);
        f32x4 dn = *reinterpret_cast<const f32x4*>(&s_dn[t4]);
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
          den += *reinterpret_cast<const f32x4*>(&s_den[ww * kTile + t4]);
          dn += *reinterpret_cast<const f32x4*>(&s_dn[ww * kTile + t4]);
        }
        const f32x4 sc = *reinterpret_cast<const f32x4*>(&s_sc[t4]);
        const f32x4 fl = *reinterpret_cast<const f32x4*>(&s_fl[t4]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float d = den[r] + sc[r] * dn[r];
          const float inv = __builtin_amdgcn_rcpf(fmaxf(fmaxf(fabsf(d), fl[r]), FLT_MIN));
#pragma unroll
          for (int y = 0; y < 2; ++y) {
            __bf16* p = &sO[(t4 + r) * OP + 32 * w + 16 * y + i];
            const float og = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2eF * (float)*p));
            *p = (__bf16)(og * acc[z][y][r] * inv);
          }
        }
      }
      __syncthreads();   // h tile complete
#pragma unroll
      for (int e = 0; e < VV; ++e) {
        const int it = tid + kThreads * e;
        const int row = it / (kVB / 8), cv = it % (kVB / 8);
        if (row < Lc)
          *reinterpret_cast<bf16x8*>(a.h + (tok0 + row) * V + vcol0 + 8 * cv) =
              *reinterpret_cast<const bf16x8*>(&sO[row * OP + 8 * cv]);
      }
    }

    // ---------------- state update: C~ <- decay C~ + K^T diag(w) V, n~ likewise
    if (rescale) {   // uniform over the workgroup
      const float f = (float)exp(logD + ld);
#pragma unroll
      for (int kx = 0; kx < KX; ++kx) {
        Ct[kx][0] *= f;
        Ct[kx][1] *= f;
      }
#pragma unroll
      for (int x = 0; x < KXW; ++x) Nacc[x] *= f;
    }
#pragma unroll
    for (int ts = 0; ts < kTile; ts += 32) {
      const f32x4 wa = *reinterpret_cast<const f32x4*>(&s_w[ts + 8 * g]);
      const f32x4 wb = *reinterpret_cast<const f32x4*>(&s_w[ts + 8 * g + 4]);
      bf16x8 Bv[2], Bw;
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const bf16x8 raw = frag_tr(sV, VP, ts, 32 * w + 16 * y);
#pragma unroll
        for (int e = 0; e < 8; ++e) Bv[y][e] = (__bf16)((float)raw[e] * (e < 4 ? wa[e] : wb[e - 4]));
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float wt = e < 4 ? wa[e] : wb[e - 4];
        const __bf16 hi = (__bf16)wt;
        const __bf16 lo = (__bf16)(wt - (float)hi);
        Bw[e] = i == 0 ? hi : (i == 1 ? lo : (__bf16)0.f);
      }
#pragma unroll
      for (int kx = 0; kx < KX; ++kx) {
        const bf16x8 Ak = frag_tr(sK, QP, ts, 16 * kx);
        Ct[kx][0] = mma(Ak, Bv[0], Ct[kx][0]);
        Ct[kx][1] = mma(Ak, Bv[1], Ct[kx][1]);
        if (kx / KXW == w) Nacc[kx % KXW] = mma(Ak, Bw, Nacc[kx % KXW]);
      }
    }
    m_prev = m_next;
    logD = logD_next;
    has_state = true;
  }
  const float fD = (float)exp(logD);

  // ---------------- end state of the chunk
  float* Cdst = nullptr;
  float* ndst = nullptr;
  if constexpr (LOCAL) {
    const int64_t sidx = bh * nseg1 + seg;
    Cdst = a.Cseg + sidx * V * K;
    ndst = vb == 0 ? a.nseg + sidx * K : nullptr;
    if (vb == 0 && tid == 0) {
      a.mloc[sidx] = m_prev;
      a.Gseg[sidx] = reset_seen ? -INFINITY : Gsum;
    }
  } else if (seg == a.S - 1 && a.C_out) {
    Cdst = a.C_out + bh * V * K;
    ndst = vb == 0 ? a.n_out + bh * K : nullptr;
    if (vb == 0 && tid == 0) a.m_out[bh] = (float)m_prev;
  }
  if (Cdst) {
#pragma unroll
    for (int kx = 0; kx < KX; ++kx)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        *reinterpret_cast<f32x4*>(Cdst + (vcol0 + 32 * w + 16 * y + i) * K + 16 * kx + 4 * g) = fD * Ct[kx][y];
  }
  if (ndst) {
#pragma unroll
    for (int x = 0; x < KXW; ++x) {
      f32x4 nv;
#pragma unroll
      for (int r = 0; r < 4; ++r) nv[r] = fD * (Nacc[x][r] + __shfl_xor(Nacc[x][r], 1, 64));
      if (i == 0) *reinterpret_cast<f32x4*>(ndst + 16 * (w * KXW + x) + 4 * g) = nv;
    }
  }
}

// ------------------------------------------------------------------ chunk combine

struct CombineArgs {
  const float *C0, *n0, *m0;
  float* Cseg;
  float* nseg;
  const double* mloc;
  double* mstart;
  const double* Gseg;
  int64_t V, K, BH;
  int S;
};

// Folds the local end states of chunks 0..S-2 in order: with the start state
// (C~, m) of chunk s and its local end state (C~loc, mloc) and log-forget total
// G, the start of chunk s+1 is m' = max(m + G, mloc),
// C~' = exp(m + G - m') C~ + exp(mloc - m') C~loc (the same for n~). Each
// thread owns four consecutive floats of one head's C~ or n~; the result
// overwrites the local state in place.
__global__ __launch_bounds__(kThreads) void seg_combine_kernel(CombineArgs a) {
  const int64_t BH = a.BH;
  const int64_t bh = blockIdx.x % BH;
  const int64_t u = (blockIdx.x / BH) * kThreads + threadIdx.x;
  const int64_t nc4 = a.V * a.K / 4, nn4 = a.K / 4;
  if (u >= nc4 + nn4) return;
  const bool is_n = u >= nc4;
  const int64_t off = is_n ? (u - nc4) * 4 : u * 4;
  const int64_t stride = is_n ? a.K : a.V * a.K;
  float* base = (is_n ? a.nseg : a.Cseg) + off;
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
  double m = 0.0;
  if (a.C0) {
    x = *reinterpret_cast<const f32x4*>((is_n ? a.n0 + bh * a.K : a.C0 + bh * a.V * a.K) + off);
    m = (double)a.m0[bh];
  }
  const int64_t ns = a.S - 1;
  constexpr int B = 8;
  for (int64_t s0 = 0; s0 < ns; s0 += B) {
    f32x4 y[B];
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const int64_t s = min(s0 + e, ns - 1);
      y[e] = *reinterpret_cast<const f32x4*>(base + (bh * ns + s) * stride);
    }
#pragma unroll
    for (int e = 0; e < B; ++e) {
      const int64_t s = s0 + e;
      if (s < ns) {
        const int64_t sidx = bh * ns + s;
        const double G = a.Gseg[sidx], ml = a.mloc[sidx];
        const double mc = G == -INFINITY ? -INFINITY : m + G;
        double mn = fmax(mc, ml);
        if (mn == -INFINITY) mn = 0.0;
        const float al = mc == -INFINITY ? 0.f : expf((float)(mc - mn));
        const float be = ml == -INFINITY ? 0.f : expf((float)(ml - mn));
        x = al * x + be * y[e];
        *reinterpret_cast<f32x4*>(base + sidx * stride) = x;
        if (u == 0) a.mstart[sidx] = mn;
        m = mn;
      }
    }
  }
}

template <int K>
hipError_t run_seg(const FwdLaunch& f, const GateBuffers& gb, const SegStates& ss, hipStream_t s) {
  SegArgs a;
  a.q = static_cast<const __bf16*>(f.q);
  a.k = static_cast<const __bf16*>(f.k);
  a.v = static_cast<const __bf16*>(f.v);
  a.o = static_cast<const __bf16*>(f.o);
  a.h = static_cast<__bf16*>(f.h);
  a.gb = gb;
  a.C0 = f.C0; a.n0 = f.n0; a.m0 = f.m0;
  a.Cseg = ss.C; a.nseg = ss.n; a.mloc = ss.mloc; a.mstart = ss.mstart; a.Gseg = ss.G;
  a.C_out = f.C_out; a.n_out = f.n_out; a.m_out = f.m_out;
  a.T = f.T; a.Nt = f.Nc; a.V = f.V; a.BH = f.BH;
  a.TPS = ss.TPS; a.S = ss.S;
  const int64_t nvb = f.V / kVB;
  if (ss.S > 1) {
    mark_before(K_STATE, s);
    hipLaunchKernelGGL((seg_kernel<K, true>), dim3((unsigned)(f.BH * nvb * (ss.S - 1))), dim3(kThreads), 0, s, a);
    CombineArgs c;
    c.C0 = f.C0; c.n0 = f.n0; c.m0 = f.m0;
    c.Cseg = ss.C; c.nseg = ss.n; c.mloc = ss.mloc; c.mstart = ss.mstart; c.Gseg = ss.G;
    c.V = f.V; c.K = K; c.BH = f.BH; c.S = ss.S;
    const int64_t units = f.V * K / 4 + K / 4;
    const int64_t blocks = (units + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(f.BH * blocks)), dim3(kThreads), 0, s, c);
    mark_after(K_STATE, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  mark_before(K_OUT, s);
  hipLaunchKernelGGL((seg_kernel<K, false>), dim3((unsigned)(f.BH * nvb * ss.S)), dim3(kThreads), 0, s, a);
  mark_after(K_OUT, s);
  return hipGetLastError();
}

}  // namespace

bool fused_path(int bf16, int64_t K, int64_t V) {
  return bf16 && V % kVB == 0 && (K == 64 || K == 128 || K == 256);
}

hipError_t launch_fused(const FwdLaunch& f, const GateBuffers& gb, const SegStates& ss, hipStream_t s) {
  switch (f.K) {
    case 64: return run_seg<64>(f, gb, ss, s);
    case 128: return run_seg<128>(f, gb, ss, s);
    case 256: return run_seg<256>(f, gb, ss, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mlstm_impl
