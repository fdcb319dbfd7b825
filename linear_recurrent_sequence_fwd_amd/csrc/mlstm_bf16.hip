// bfloat16 kernels of the chunkwise mLSTM forward for gfx950: the
// inter-chunk state pass and the intra-chunk output kernel, tuned for the
// shapes where d_v is a multiple of 128. Same mathematics as the generic
// kernels in mlstm_kernels.hip (xLSTM guide, aifetchly blog: recurrence of
// "mLSTM: Matrix Key-Value Memory and Covariance Updates", stabiliser of "The
// Stabilizer State", decay matrix of "The Dual Formulation", chunking of
// "Exploit Chunkwise Hardware Kernels for Production Training").
//
// What differs from the generic kernels:
//  * operands whose contraction runs over tokens (K^T and V in the state
//    update, V in P V) are staged row-major with coalesced 16-byte loads and
//    read transposed by ds_read_b64_tr_b16: within each 16-lane group, lane i
//    receives element (i mod 4) of the 8-byte rows addressed by lanes
//    4e + i/4, e = 0..3, so lane j addressing row kin0 + j/4, column
//    n0 + 4 (j mod 4) hands lane i the column n0 + i of rows kin0..kin0+3;
//  * workgroups are numbered head-fastest, so with 8 heads (or a multiple)
//    all tiles of one head run on one XCD and share its L2;
//  * global loads of the next token blocks are issued before the current
//    block's MFMAs (register prefetch), LDS is double-buffered in the state
//    pass, and the output kernel stages O and h through LDS for 16-byte
//    global accesses.

#include "mlstm_device.h"

namespace mlstm_impl {

namespace {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposed operand fragment from a row-major LDS tile X (row pitch P):
// lane l (i = l%16, g = l/16) receives X[kin0 + 8g + e][n0 + i], e = 0..7.
__device__ __forceinline__ bf16x8 ld_frag_tr(const __bf16* X, int P, int kin0, int n0) {
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  const __bf16* p = X + (kin0 + 8 * g + (i >> 2)) * P + n0 + 4 * (i & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * P));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Calls f(std::integral_constant<int, s>) for s = 0..N-1, unrolled.
template <typename F, int... S>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kStatePrefetch = 4;   // token blocks in flight per state-pass workgroup

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
  return z;
}

__device__ __forceinline__ bf16x8 scale8(bf16x8 x, float s) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)((float)x[e] * s);
  return r;
}

// ------------------------------------------------------------------ state pass

struct StateArgsB {
  const __bf16* k;
  const __bf16* v;
  GateBuffers gb;
  const float *C0, *n0, *m0;
  float* Cs;
  float* ns;
  double* ms;
  float *C_out, *n_out, *m_out;
  int64_t T, Nc, V, BH;
  int L;
  int cs_bf16;   // store the chunk-start states as bf16 (Cs then points to bf16)
};

// One workgroup per (head, 64 k x 64 v tile of C^T), four waves of 32 x 32.
// Walks the sequence in 64-token blocks. Block b's K and V rows and weights
// are loaded NPF blocks ahead into registers (issued in the order they are
// consumed, so the in-order vmcnt waits never drain the ring), written to LDS
// buffer b%2 with V scaled by the chunk-local weights w0_j = exp(u_j - U_c),
// and contracted over tokens on MFMA into a per-chunk accumulator. At the
// chunk's end the carried tile becomes decay*C + alpha*acc_chunk with
// Rm = max(m_prev, U_c), decay = exp(m_prev - Rm), alpha = exp(U_c - Rm), and
// m advances to g_c + Rm; at the next chunk's start it is stored (float32). The
// chunk scalars (g, U, R) are loaded one chunk ahead. The normaliser n is the
// same contraction with V replaced by ones: the waves with wv = 0 of the
// v-tile-0 workgroups compute it as one more 16-column MFMA tile, with each
// weight split into three bf16 terms (w = hi + lo + lo2) so that n keeps about 24
// bits, because rows where n^T q nearly cancels would magnify a rounded n.
template <int K, int NPF>
__global__ __launch_bounds__(kThreads) void state_kernel_bf16(StateArgsB a) {
  constexpr int KT = K / 64;
  constexpr int P = kTile + 16;     // LDS row pitch (elements)
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][kTile * P];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][kTile * P];
  __shared__ __attribute__((aligned(16))) __bf16 sw[2][3][kTile];   // [buffer][hi, lo, lo2][token]

  const int64_t BH = a.BH, V = a.V, T = a.T;
  const int64_t bh = blockIdx.x % BH;
  const int tile = (int)(blockIdx.x / BH);
  const int kt = tile % KT, vt = tile / KT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int wk = w & 1, wv = w >> 1;
  const bool n_tile = (vt == 0) && (wv == 0);

  f32x4 acc[2][2], tacc[2][2], nacc[2], tn[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    nacc[x] = tn[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = tacc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  double m_prev = 0.0;
  if (a.C0) {
    const float* C0 = a.C0 + bh * V * K;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int kk = 64 * kt + 32 * wk + 16 * x + 4 * g;
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const int64_t vv = 64 * vt + 32 * wv + 16 * y + i;
        acc[x][y] = *reinterpret_cast<const f32x4*>(C0 + vv * K + kk);
      }
      if (n_tile) nacc[x] = *reinterpret_cast<const f32x4*>(a.n0 + bh * K + kk);
    }
    m_prev = (double)a.m0[bh];
  }

  // this thread stages rows r0 and r0 + 32 of each block, columns 8 cg .. 8 cg + 7
  const int r0 = tid >> 3, cg = tid & 7;
  const __bf16* kp = a.k + (bh * T + r0) * K + 64 * kt + 8 * cg;
  const __bf16* vp = a.v + (bh * T + r0) * V + 64 * vt + 8 * cg;
  const float* wp = a.gb.w0 + bh * T + r0;
  const int nsb = (int)((T + kTile - 1) / kTile);

  bf16x8 pk[NPF][2], pv[NPF][2];
  float pw[NPF][2];
#pragma unroll
  for (int s = 0; s < NPF; ++s)
#pragma unroll
    for (int e = 0; e < 2; ++e) { pk[s][e] = zero8(); pv[s][e] = zero8(); pw[s][e] = 0.f; }
  // rows beyond T keep finite stale values in pk/pv and weight 0
  auto issue = [&](int sb, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int64_t t = (int64_t)sb * kTile + r0 + 32 * e;
      const int64_t off = (int64_t)sb * kTile + 32 * e;
      if (t < T) {
        pk[SLOT][e] = *reinterpret_cast<const bf16x8*>(kp + off * K);
        pv[SLOT][e] = *reinterpret_cast<const bf16x8*>(vp + off * V);
        pw[SLOT][e] = wp[off];
      } else {
        pw[SLOT][e] = 0.f;
      }
    }
  };

  // chunk scalars: current (cg_, cU, cR) and the next chunk's, loaded a chunk ahead
  double cgv = a.gb.g[bh * a.Nc], cUv = a.gb.U[bh * a.Nc];
  int cRv = a.gb.R[bh * a.Nc];
  double ngv = 0.0, nUv = 0.0;
  int nRv = -1;
  int64_t c = 0;
  int jc = 0;
  int Lc = (int)min((int64_t)a.L, T);
  float decay = 1.f, alpha = 1.f;
  double m_next = 0.0;

  auto body = [&](int sb, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    if (sb >= nsb) return;
    if (jc == 0) {   // chunk start: store the carried state, derive this chunk's scalars
      if (a.Cs) {
        float* Cs = a.Cs + (bh * a.Nc + c) * V * K;
        __bf16* Cb = reinterpret_cast<__bf16*>(a.Cs) + (bh * a.Nc + c) * V * K;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int kk = 64 * kt + 32 * wk + 16 * x + 4 * g;
#pragma unroll
          for (int y = 0; y < 2; ++y) {
            const int64_t vv = 64 * vt + 32 * wv + 16 * y + i;
            if (a.cs_bf16) {
              bf16x4 o;
#pragma unroll
              for (int r = 0; r < 4; ++r) o[r] = (__bf16)acc[x][y][r];
              *reinterpret_cast<bf16x4*>(Cb + vv * K + kk) = o;
            } else {
              *reinterpret_cast<f32x4*>(Cs + vv * K + kk) = acc[x][y];
            }
          }
          if (n_tile && i == 0) *reinterpret_cast<f32x4*>(a.ns + (bh * a.Nc + c) * K + kk) = nacc[x];
        }
        if (tile == 0 && tid == 0) a.ms[bh * a.Nc + c] = m_prev;
      }
      double Rm = fmax(cRv >= 0 ? -INFINITY : m_prev, cUv);
      if (Rm == -INFINITY) Rm = 0.0;
      decay = cRv >= 0 ? 0.f : expf((float)(m_prev - Rm));
      alpha = cUv == -INFINITY ? 0.f : expf((float)(cUv - Rm));
      m_next = cgv + Rm;
      if (c + 1 < a.Nc) {
        ngv = a.gb.g[bh * a.Nc + c + 1];
        nUv = a.gb.U[bh * a.Nc + c + 1];
        nRv = a.gb.R[bh * a.Nc + c + 1];
      }
    }
    const int buf = sb & 1;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = r0 + 32 * e;
      const float wf = pw[SLOT][e];
      *reinterpret_cast<bf16x8*>(&sK[buf][row * P + 8 * cg]) = pk[SLOT][e];
      *reinterpret_cast<bf16x8*>(&sV[buf][row * P + 8 * cg]) = scale8(pv[SLOT][e], wf);
      if (cg == 0) {
        const __bf16 hi = (__bf16)wf;
        const float rest = wf - (float)hi;
        const __bf16 lo = (__bf16)rest;
        sw[buf][0][row] = hi;
        sw[buf][1][row] = lo;
        sw[buf][2][row] = (__bf16)(rest - (float)lo);
      }
    }
    if (sb + NPF < nsb) issue(sb + NPF, slot_c);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTile; kk += 32) {
      bf16x8 A[2], B[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) A[x] = ld_frag_tr(sK[buf], P, kk, 32 * wk + 16 * x);
#pragma unroll
      for (int y = 0; y < 2; ++y) B[y] = ld_frag_tr(sV[buf], P, kk, 32 * wv + 16 * y);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) tacc[x][y] = mma(A[x], B[y], tacc[x][y]);
      if (n_tile) {
        const bf16x8 Bh = *reinterpret_cast<const bf16x8*>(&sw[buf][0][kk + 8 * g]);
        const bf16x8 Bl = *reinterpret_cast<const bf16x8*>(&sw[buf][1][kk + 8 * g]);
        const bf16x8 Bl2 = *reinterpret_cast<const bf16x8*>(&sw[buf][2][kk + 8 * g]);
#pragma unroll
        for (int x = 0; x < 2; ++x) tn[x] = mma(A[x], Bl2, mma(A[x], Bl, mma(A[x], Bh, tn[x])));
      }
    }
    jc += kTile;
    if (jc >= Lc) {   // chunk end: fold the chunk's contribution into the carried state
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        nacc[x] = decay * nacc[x] + alpha * tn[x];
        tn[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          acc[x][y] = decay * acc[x][y] + alpha * tacc[x][y];
          tacc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      m_prev = m_next;
      ++c;
      jc = 0;
      Lc = (int)min((int64_t)a.L, T - c * a.L);
      cgv = ngv; cUv = nUv; cRv = nRv;
    }
  };

  static_for<NPF>([&](auto s) {
    if (decltype(s)::value < nsb) issue(decltype(s)::value, s);
  });
  for (int sb = 0; sb < nsb; sb += NPF)
    static_for<NPF>([&](auto s) { body(sb + decltype(s)::value, s); });

  if (a.C_out) {
    float* Co = a.C_out + bh * V * K;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int kk = 64 * kt + 32 * wk + 16 * x + 4 * g;
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const int64_t vv = 64 * vt + 32 * wv + 16 * y + i;
        *reinterpret_cast<f32x4*>(Co + vv * K + kk) = acc[x][y];
      }
      if (n_tile && i == 0) *reinterpret_cast<f32x4*>(a.n_out + bh * K + kk) = nacc[x];
    }
    if (tile == 0 && tid == 0) a.m_out[bh] = (float)m_prev;
  }
}

// ------------------------------------------------------------------ output kernel

struct OutArgsB {
  const __bf16 *q, *k, *v, *o;
  __bf16* h;
  GateBuffers gb;
  const float* Cs;   // chunk-start states [BH][Nc][V][K] (float32), or null
  const float* ns;   // [BH][Nc][K]
  const double* ms;  // [BH][Nc]
  const float* C0f;  // initial state [BH][V][K] (float32) for the one-chunk form, or null
  const float* n0;
  const float* m0;
  int zero_first;    // chunk 0 starts from the zero state
  int64_t T, Nc, V, BH;
  int L;
};

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// One workgroup per (head, 64-row query tile, 64*NT value columns), four
// waves; wave w owns all 64 rows of the block's columns [16 NT w, 16 NT (w+1))
// and the 16 keys [16 w, 16 w + 16) of each score tile. LDS stays under 80 KiB
// so that two workgroups share a CU. Global loads are issued in the order they
// are consumed (Q, n, state fragments a few k-steps ahead, then per key block
// K fragments and the V tile one block ahead, the O tile during the last
// block). Decay weights use float32 exponents relative to the first row's
// stabiliser, exp2(log2e (u_j - ref) - log2e (r_t - ref)).
template <int K, int NT>
__global__ __launch_bounds__(kThreads, 2) void out_kernel_bf16(OutArgsB a) {
  constexpr int VB = 64 * NT;
  constexpr int QP = K + 8;
  constexpr int VP = VB + 8;
  constexpr int PP = kTile + 8;
  constexpr int VVEC = kTile * VB / 8 / kThreads;   // 16-byte V/O vectors per thread
  constexpr int QVEC = kTile * K / 8 / kThreads;    // 16-byte Q vectors per thread
  constexpr int KS = K / 32;                         // k-steps of the contractions over d_qk
  constexpr int D = 2;                               // state k-steps in flight
  __shared__ __attribute__((aligned(16))) __bf16 sQ[kTile * QP];
  __shared__ __attribute__((aligned(16))) __bf16 sV[kTile * VP];
  __shared__ __attribute__((aligned(16))) __bf16 sP[kTile * PP];
  __shared__ __attribute__((aligned(16))) float sn[K];
  __shared__ __attribute__((aligned(16))) float s_u2[2][kTile];
  __shared__ __attribute__((aligned(16))) float s_r2[kTile], s_sc[kTile], s_fl[kTile], s_dn[kTile];
  __shared__ __attribute__((aligned(16))) float s_den[4][kTile];
  __shared__ __attribute__((aligned(16))) int s_rs[kTile];

  const int64_t V = a.V, T = a.T, BH = a.BH;
  const int64_t nvb = V / VB;
  const int64_t bh = blockIdx.x % BH;
  const int64_t rest = blockIdx.x / BH;
  const int64_t vb = rest % nvb;
  const int64_t qb = rest / nvb;
  const int64_t row0 = qb * kTile;
  const int64_t c = row0 / a.L;
  const int64_t t0 = c * a.L;
  const int st = (int)((row0 - t0) / kTile);
  const int nrows = (int)min((int64_t)kTile, T - row0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int col0 = w * 16 * NT;

  const bool chunk_states = a.Cs != nullptr;
  const bool has_state = chunk_states ? (c > 0 || !a.zero_first) : (a.C0f != nullptr);
  const double m_prev = !has_state ? 0.0
                        : (chunk_states ? a.ms[bh * a.Nc + c] : (double)a.m0[bh]);
  const int64_t vrow0 = vb * VB + col0;

  // ---------------- prologue: loads in consumption order
  bf16x8 pq[QVEC];
  {
    const __bf16* qg = a.q + (bh * T + row0) * K;
#pragma unroll
    for (int e = 0; e < QVEC; ++e) {
      const int it = tid + kThreads * e;
      const int row = it / (K / 8), cv = it % (K / 8);
      pq[e] = row < nrows ? *reinterpret_cast<const bf16x8*>(qg + (int64_t)row * K + 8 * cv) : zero8();
    }
  }
  float nval = 0.f;
  const float* nsrc = !has_state ? nullptr : (chunk_states ? a.ns + (bh * a.Nc + c) * K : a.n0 + bh * K);
  if (has_state && tid < K) nval = nsrc[tid];
  // row data (threads 0..63): stabiliser inputs of row tid and of row 0 (the reference)
  double mp_t = 0.0, b_t = 0.0, mp_0 = 0.0, u_k = -INFINITY;
  int rs_t = 0, rs_0 = 0;
  if (tid < kTile) {
    const int64_t tb = bh * T + row0;
    mp_0 = a.gb.mp[tb];
    rs_0 = a.gb.rs[tb];
    if (tid < nrows) {
      mp_t = a.gb.mp[tb + tid];
      b_t = a.gb.b[tb + tid];
      rs_t = a.gb.rs[tb + tid];
    }
    if (t0 + tid < T) u_k = a.gb.u[bh * T + t0 + tid];
  }
  // float32 state fragments, split into bf16 hi + lo at their MFMAs: rows
  // whose q is nearly orthogonal to a dominant key make C~ q a strongly
  // cancelling sum, which one bf16 rounding of C~ would swamp
  f32x4 Bst[D][NT][2];
  const float* Cst = chunk_states ? a.Cs + (bh * a.Nc + c) * V * K : (a.C0f ? a.C0f + bh * V * K : nullptr);
  auto load_state = [&](int s, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
#pragma unroll
    for (int y = 0; y < NT; ++y) {
      const int64_t off = (vrow0 + 16 * y + i) * K + 32 * s + 8 * g;
      Bst[SL][y][0] = *reinterpret_cast<const f32x4*>(Cst + off);
      Bst[SL][y][1] = *reinterpret_cast<const f32x4*>(Cst + off + 4);
    }
  };
  if (has_state) {
    static_for<D>([&](auto s) {
      if (decltype(s)::value < KS) load_state(decltype(s)::value, s);
    });
  }
  bf16x8 Kf[KS];
  auto load_k = [&](int jb) {
    const int64_t key = t0 + (int64_t)jb * kTile + 16 * w + i;
    const __bf16* kg = a.k + (bh * T + key) * K + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) Kf[s] = key < T ? *reinterpret_cast<const bf16x8*>(kg + 32 * s) : zero8();
  };
  load_k(0);
  bf16x8 pv[VVEC];
  auto load_tile = [&](const __bf16* src, int64_t rows_valid) {   // 64 rows x VB columns, row pitch V
#pragma unroll
    for (int e = 0; e < VVEC; ++e) {
      const int it = tid + kThreads * e;
      const int row = it / (VB / 8), cv = it % (VB / 8);
      pv[e] = row < rows_valid ? *reinterpret_cast<const bf16x8*>(src + (int64_t)row * V + 8 * cv) : zero8();
    }
  };
  load_tile(a.v + (bh * T + t0) * V + vb * VB, min((int64_t)kTile, T - t0));

  // ---------------- prologue: LDS fills
#pragma unroll
  for (int e = 0; e < QVEC; ++e) {
    const int it = tid + kThreads * e;
    const int row = it / (K / 8), cv = it % (K / 8);
    *reinterpret_cast<bf16x8*>(&sQ[row * QP + 8 * cv]) = pq[e];
  }
  if (tid < K) sn[tid] = nval;
  double ref = 0.0;
  if (tid < kTile) {
    const bool carry0 = has_state && rs_0 < 0;
    ref = fmax(carry0 ? m_prev : -INFINITY, mp_0);
    if (ref == -INFINITY) ref = 0.0;
    float r2 = 0.f, sc = 0.f, fl = 1.f;
    if (tid < nrows) {
      const bool carry = has_state && rs_t < 0;
      double r = fmax(carry ? m_prev : -INFINITY, mp_t);
      if (r == -INFINITY) r = 0.0;
      r2 = (float)((r - ref) * (double)kLog2e);
      sc = carry ? expf((float)(m_prev - r)) : 0.f;
      fl = expf((float)(-(b_t + r)));
    }
    s_r2[tid] = r2;
    s_sc[tid] = sc;
    s_fl[tid] = fl;
    s_rs[tid] = rs_t;
    s_u2[0][tid] = (float)((u_k - ref) * (double)kLog2e);
  }
  __syncthreads();

  f32x4 acc[4][NT];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < NT; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---------------- carried-state term: (Q C~^T) scaled per row, and sc_t (q_t . n~)
  if (has_state) {
    {
      const int row = tid >> 2, part = tid & 3;
      float d = 0.f;
#pragma unroll 8
      for (int kk = part * (K / 4); kk < (part + 1) * (K / 4); ++kk) d += (float)sQ[row * QP + kk] * sn[kk];
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      if (part == 0) s_dn[row] = d * s_sc[row];
    }
    static_for<KS>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      bf16x8 A[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) A[x] = *reinterpret_cast<const bf16x8*>(&sQ[(16 * x + i) * QP + 32 * s + 8 * g]);
#pragma unroll
      for (int y = 0; y < NT; ++y) {
        const f32x4 x0 = Bst[s % D][y][0], x1 = Bst[s % D][y][1];
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = (__bf16)x0[e];
          hi[4 + e] = (__bf16)x1[e];
          lo[e] = (__bf16)(x0[e] - (float)hi[e]);
          lo[4 + e] = (__bf16)(x1[e] - (float)hi[4 + e]);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[x][y] = mma(A[x], lo, mma(A[x], hi, acc[x][y]));
      }
      if constexpr (s + D < KS) load_state(s + D, std::integral_constant<int, s % D>{});
    });
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sc = s_sc[16 * x + 4 * g + r];
#pragma unroll
        for (int y = 0; y < NT; ++y) acc[x][y][r] *= sc;
      }
  } else if (tid < kTile) {
    s_dn[tid] = 0.f;
  }

  // ---------------- intra-chunk key blocks jb = 0..st
  float rsum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int jb = 0; jb <= st; ++jb) {
    const int64_t key0 = t0 + (int64_t)jb * kTile;
    __syncthreads();   // previous block's P V done: sV, sP free
#pragma unroll
    for (int e = 0; e < VVEC; ++e) {
      const int it = tid + kThreads * e;
      const int row = it / (VB / 8), cv = it % (VB / 8);
      *reinterpret_cast<bf16x8*>(&sV[row * VP + 8 * cv]) = pv[e];
    }
    double u_next = -INFINITY;
    if (jb < st) {
      load_tile(a.v + (bh * T + key0 + kTile) * V + vb * VB, min((int64_t)kTile, T - key0 - kTile));
      if (tid < kTile && key0 + kTile + tid < T) u_next = a.gb.u[bh * T + key0 + kTile + tid];
    } else {
      load_tile(a.o + (bh * T + row0) * V + vb * VB, nrows);   // O tile for the epilogue
    }
    // S^T: this wave's 16 keys x 64 rows
    f32x4 sacc[4];
#pragma unroll
    for (int z = 0; z < 4; ++z) sacc[z] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(&sQ[(16 * z + i) * QP + 32 * s + 8 * g]);
        sacc[z] = mma(Kf[s], B, sacc[z]);
      }
    }
    if (jb < st) load_k(jb + 1);
    // P = S o D: lane holds S^T[j = 16 w + 4 g + r][t = 16 z + i]
    float u2[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) u2[r] = s_u2[jb & 1][16 * w + 4 * g + r];
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      const int tl = 16 * z + i;
      const int tq = st * kTile + tl;
      const float r2 = s_r2[tl];
      const int rs = s_rs[tl];
      bf16x4 pk4;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jk = jb * kTile + 16 * w + 4 * g + r;
        const bool keep = (tl < nrows) && (jk <= tq) && (jk >= rs);
        const float p = keep ? sacc[z][r] * fast_exp2(u2[r] - r2) : 0.f;
        psum += p;
        pk4[r] = (__bf16)p;
      }
      *reinterpret_cast<bf16x4*>(&sP[tl * PP + 16 * w + 4 * g]) = pk4;
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      rsum[z] += psum;
    }
    if (jb < st && tid < kTile) s_u2[(jb + 1) & 1][tid] = (float)((u_next - ref) * (double)kLog2e);
    __syncthreads();   // sP and sV complete
#pragma unroll
    for (int jj = 0; jj < kTile; jj += 32) {
      bf16x8 A[4], B[NT];
#pragma unroll
      for (int x = 0; x < 4; ++x) A[x] = *reinterpret_cast<const bf16x8*>(&sP[(16 * x + i) * PP + jj + 8 * g]);
#pragma unroll
      for (int y = 0; y < NT; ++y) B[y] = ld_frag_tr(sV, VP, jj, col0 + 16 * y);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < NT; ++y) acc[x][y] = mma(A[x], B[y], acc[x][y]);
    }
  }
  if (g == 0) {
#pragma unroll
    for (int z = 0; z < 4; ++z) s_den[w][16 * z + i] = rsum[z];
  }
  __syncthreads();   // all P V done; s_den complete; sV free

  // ---------------- output gate and normalisation, staged through LDS
#pragma unroll
  for (int e = 0; e < VVEC; ++e) {
    const int it = tid + kThreads * e;
    const int row = it / (VB / 8), cv = it % (VB / 8);
    *reinterpret_cast<bf16x8*>(&sV[row * VP + 8 * cv]) = pv[e];
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = 16 * x + 4 * g + r;
      const float den = s_den[0][tl] + s_den[1][tl] + s_den[2][tl] + s_den[3][tl] + s_dn[tl];
      const float inv = fast_rcp(fmaxf(fmaxf(fabsf(den), s_fl[tl]), FLT_MIN));
#pragma unroll
      for (int y = 0; y < NT; ++y) {
        __bf16* p = &sV[tl * VP + col0 + 16 * y + i];
        const float og = fast_rcp(1.f + fast_exp2(-kLog2e * (float)*p));
        *p = (__bf16)(og * acc[x][y][r] * inv);
      }
    }
  __syncthreads();
  const int64_t obase = (bh * T + row0) * V + vb * VB;
#pragma unroll
  for (int e = 0; e < VVEC; ++e) {
    const int it = tid + kThreads * e;
    const int row = it / (VB / 8), cv = it % (VB / 8);
    if (row < nrows)
      *reinterpret_cast<bf16x8*>(a.h + obase + (int64_t)row * V + 8 * cv) =
          *reinterpret_cast<const bf16x8*>(&sV[row * VP + 8 * cv]);
  }
}

template <int K>
hipError_t run_state_b(const FwdLaunch& f, const GateBuffers& gb, const ChunkStates& cs, hipStream_t s) {
  StateArgsB a;
  a.k = static_cast<const __bf16*>(f.k);
  a.v = static_cast<const __bf16*>(f.v);
  a.gb = gb;
  a.C0 = f.C0; a.n0 = f.n0; a.m0 = f.m0;
  a.Cs = static_cast<float*>(cs.Cs);
  a.ns = cs.ns; a.ms = cs.ms;
  a.cs_bf16 = cs.cs_bf16;
  a.C_out = f.C_out; a.n_out = f.n_out; a.m_out = f.m_out;
  a.T = f.T; a.Nc = f.Nc; a.V = f.V; a.BH = f.BH; a.L = f.L;
  const int64_t grid = f.BH * (K / 64) * (f.V / 64);
  mark_before(f.marks, K_STATE, s);
  hipLaunchKernelGGL((state_kernel_bf16<K, kStatePrefetch>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  mark_after(f.marks, K_STATE, s);
  return hipGetLastError();
}

template <int K, int NT>
hipError_t run_out_b(const FwdLaunch& f, const GateBuffers& gb, const ChunkStates& cs, hipStream_t s) {
  OutArgsB a;
  a.q = static_cast<const __bf16*>(f.q);
  a.k = static_cast<const __bf16*>(f.k);
  a.v = static_cast<const __bf16*>(f.v);
  a.o = static_cast<const __bf16*>(f.o);
  a.h = static_cast<__bf16*>(f.h);
  a.gb = gb;
  a.Cs = static_cast<const float*>(cs.Cs);
  a.ns = cs.ns; a.ms = cs.ms;
  a.C0f = cs.Cs ? nullptr : f.C0;
  a.n0 = f.n0; a.m0 = f.m0;
  a.zero_first = f.C0 == nullptr;
  a.T = f.T; a.Nc = f.Nc; a.V = f.V; a.BH = f.BH; a.L = f.L;
  const int64_t nqt = (f.T + kTile - 1) / kTile;
  const int64_t grid = f.BH * nqt * (f.V / (64 * NT));
  mark_before(f.marks, K_OUT, s);
  hipLaunchKernelGGL((out_kernel_bf16<K, NT>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  mark_after(f.marks, K_OUT, s);
  return hipGetLastError();
}

template <int K>
hipError_t run_out_b_nt(const FwdLaunch& f, const GateBuffers& gb, const ChunkStates& cs, hipStream_t s) {
  const int64_t nv = f.V / 64;
  if (nv % 4 == 0) return run_out_b<K, 4>(f, gb, cs, s);
  if (nv % 2 == 0) return run_out_b<K, 2>(f, gb, cs, s);
  return run_out_b<K, 1>(f, gb, cs, s);
}

}  // namespace

bool bf16_fast_path(const FwdLaunch& f) { return f.bf16 && f.V % 64 == 0; }

hipError_t launch_state_bf16(const FwdLaunch& f, const GateBuffers& gb, const ChunkStates& cs, hipStream_t s) {
  switch (f.K) {
    case 64: return run_state_b<64>(f, gb, cs, s);
    case 128: return run_state_b<128>(f, gb, cs, s);
    case 256: return run_state_b<256>(f, gb, cs, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_out_bf16(const FwdLaunch& f, const GateBuffers& gb, const ChunkStates& cs, hipStream_t s) {
  switch (f.K) {
    case 64: return run_out_b_nt<64>(f, gb, cs, s);
    case 128: return run_out_b_nt<128>(f, gb, cs, s);
    case 256: return run_out_b_nt<256>(f, gb, cs, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mlstm_impl
