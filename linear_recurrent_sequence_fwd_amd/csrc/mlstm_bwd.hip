// HIP kernels of the chunkwise mLSTM backward pass for gfx950: the gradients
// of a loss through the cell's outputs h with respect to q, k, v, the three
// gate preactivations and the initial state.
//
// The pages present the dual and chunkwise forms as what makes the mLSTM
// trainable (xLSTM guide, aifetchly blog, "The Dual Formulation: How mLSTM
// Enables Parallel GPU Training"; "Exploit Chunkwise Hardware Kernels for
// Production Training"). This is the reverse mode of the same chunkwise
// evaluation, in the notation of the forward kernels (mlstm_kernels.hip): a
// chunk starting at t0 with carried stabiliser m_prev, b_t the in-chunk
// cumulative log forget gate, u_j = i~_j - b_j, r_t the row stabiliser
// (m_t = b_t + r_t), P_tj = exp(u_j - r_t) the decay weight of key j in row t
// and sc_t = exp(m_prev - r_t) the weight of the carried state.
//
// With the stabilised denominator den_t = max(|z_t|, exp(-m_t)) (z_t the
// stabilised n_t . q_t) the per-row quantities are
//   g_t  = dh_t sigmoid(o~_t) / den_t
//   dz_t = -sign(z_t) [|z_t| > exp(-m_t)] (dh_t . h_t) / den_t
//   do~_t = dh_t h_t (1 - sigmoid(o~_t))
// and, inside a chunk (intra) plus through the carried state (inter),
//   dq_t = sum_j P_tj (g_t . v_j + dz_t) k_j + sc_t (C~^T g_t + dz_t n~)
//   dk_j = sum_t P_tj (g_t . v_j + dz_t) q_t + w_j (A^T v_j + a)
//   dv_j = sum_t P_tj (q_t . k_j) g_t + w_j A k_j
//   di~_j = k_j . dk_j,   dlog f_l = sum_{t >= l} (q_t . dq_t - k_t . dk_t)
// where (A, a) is the adjoint of the state at the chunk's end: every later
// row s contributes g_s q_s^T (dz_s q_s) with true weight
// exp(sum of log f from the chunk end to s) exp(-m_s), and w_j is key j's
// weight to the chunk end. The forget-gate sum stops at a zero forget gate
// (no weight crosses it), whose own gradient is 0.
//
// Kernels (after the forward's gate kernel and state pass, which give the
// gate prefix data and every chunk's start state):
//   bwd_dq_kernel     per (head, 64-row tile): the row denominators from
//                     Q K^T over the chunk's key tiles, then g, dz, do~, dq
//                     (G V^T and (P o (G V^T + dz)) K on MFMA, plus the
//                     carried-state term G C~); writes g for the next two
//   bwd_local_kernel  per (head, 64 x 64 tile of A, chunk): the chunk's own
//                     share of the adjoint at its start, G^T diag(w) Q on MFMA
//   bwd_fold_kernel   per head and element group: chains the shares from
//                     the last chunk to the first into every chunk's end
//                     adjoint (float32), and the initial state's gradient
//   bwd_dkv_kernel    per (head, 64-key tile): the end adjoint's term, then
//                     the chunk's later query tiles: S = Q K^T, G V^T, and
//                     dk += (P o (G V^T + dz))^T Q, dv += (P o S)^T G
//   bwd_gate_map_kernel, bwd_gate_kernel
//                     per (head, chunk): the forget-gate suffix sums as a
//                     reverse scan of affine maps (each chunk's map, then
//                     the later chunks' maps composed into the run entering
//                     the chunk), and the initial-state stabiliser gradient
//
// Operand fragments: every product is a sequence of 16x16x32 steps in which
// lane (i, g) of the wave supplies A[i][8g .. 8g+7] and B[i][8g .. 8g+7]
// (D = A B^T, D[4g + r][i] in register r). For bfloat16 that is one
// v_mfma_f32_16x16x32_bf16; for float32 it is eight v_mfma_f32_16x16x4_f32,
// the s-th taking element 8g + s of each lane, which covers the same 32
// contraction indices in another order.

#include "mlstm_device.h"

namespace mlstm_impl {

namespace {

constexpr int kBT = 512;   // threads of the dq and dk/dv kernels: eight waves
constexpr float kL2e = 1.4426950408889634f;

typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((address_space(3))) bf16x4 lds_b4;

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> { using type = bf16x8; };
template <> struct Vec8<float> { using type = f32x8; };
template <typename T> using vec8 = typename Vec8<T>::type;

template <typename T> constexpr int lds_pad() { return sizeof(T) == 2 ? 8 : 4; }

__device__ __forceinline__ bf16x8 load8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ f32x8 load8(const float* p) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p);
  const f32x4 y = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}
__device__ __forceinline__ void store8(__bf16* p, bf16x8 x) { *reinterpret_cast<bf16x8*>(p) = x; }
__device__ __forceinline__ void store8(float* p, f32x8 x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void store4(__bf16* p, f32x4 x) {
  bf16x4 o;
  o[0] = (__bf16)x[0]; o[1] = (__bf16)x[1]; o[2] = (__bf16)x[2]; o[3] = (__bf16)x[3];
  *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ __forceinline__ void store4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }

template <typename T> __device__ __forceinline__ vec8<T> zero_v8() {
  vec8<T> z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (T)0.f;
  return z;
}

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) { return mma(a, b, c); }
__device__ __forceinline__ f32x4 mma32(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = mma(a[s], b[s], c);
  return c;
}

// lane (i, g): row r0 + i, elements k0 + 8g .. k0 + 8g + 7 of a row-major
// array (LDS or global) with row pitch P
template <typename T>
__device__ __forceinline__ vec8<T> frag_rows(const T* X, int64_t P, int r0, int k0) {
  const int lane = threadIdx.x & 63;
  return load8(X + (int64_t)(r0 + (lane & 15)) * P + k0 + 8 * (lane >> 4));
}
// the same from global memory, zero for rows at or beyond `nrows`
template <typename T>
__device__ __forceinline__ vec8<T> frag_rows_lim(const T* X, int64_t P, int r0, int k0, int nrows) {
  const int lane = threadIdx.x & 63;
  const int r = r0 + (lane & 15);
  return r < nrows ? load8(X + (int64_t)r * P + k0 + 8 * (lane >> 4)) : zero_v8<T>();
}

// lane (i, g): column n0 + i of rows k0 + 8g .. k0 + 8g + 7 of a row-major
// LDS tile with row pitch P. bfloat16: two ds_read_b64_tr_b16, which hand
// lane i of each 16-lane group element (i mod 4) of the 8-byte rows that
// lanes 4e + i/4 address: lane l addressing row k0 + 8g + l/4, column
// n0 + 4 (l mod 4) (and 4 rows further for the second) gives lane i column
// n0 + i of the group's rows.
__device__ __forceinline__ bf16x8 frag_cols(const __bf16* X, int P, int k0, int n0) {
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  const __bf16* p = X + (k0 + 8 * g + (i >> 2)) * P + n0 + 4 * (i & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(p + 4 * P));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x8 frag_cols(const float* X, int P, int k0, int n0) {
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = X[(k0 + 8 * g + e) * P + n0 + i];
  return r;
}

// Copy rows [0, 64) x columns [0, NC) of a row-major global array (row pitch
// gp) into LDS (row pitch SP); rows at or beyond `nrows` become zero. Each
// thread issues all its loads before the first store, so the tile costs one
// memory latency rather than one per 16-byte piece.
template <int NT, typename T, int NC, int SP>
__device__ __forceinline__ void stage(T* __restrict__ s, const T* __restrict__ g, int64_t gp, int nrows) {
  constexpr int EV = 16 / sizeof(T);
  constexpr int VPR = NC / EV;
  constexpr int N = (kTile * VPR + NT - 1) / NT;
  f32x4 x[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int it = (int)threadIdx.x + n * NT;
    const int row = it / VPR, cv = it % VPR;
    x[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (it < kTile * VPR && row < nrows) x[n] = *reinterpret_cast<const f32x4*>(g + (int64_t)row * gp + cv * EV);
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const int it = (int)threadIdx.x + n * NT;
    const int row = it / VPR, cv = it % VPR;
    if (it < kTile * VPR) *reinterpret_cast<f32x4*>(s + row * SP + cv * EV) = x[n];
  }
}
// The same copy as direct-to-LDS buffer loads: no registers, every load of
// the tile in flight at once. Rows [0, nrows) of NC elements lie contiguous
// in global memory; the LDS image (row pitch SP, a whole number of 16-byte
// pieces) is filled 1 KiB per wave-wide load, a row's padding pieces
// repeating its last data piece. Loads past the buffer's nrows * NC elements
// return zero, so the rows beyond `nrows` come out zero. The caller's next
// __syncthreads waits for the loads (a workgroup fence waits for direct-to-LDS
// loads as for LDS stores).
typedef __attribute__((address_space(3))) void lds_void_t;
template <int NT, typename T, int NC, int SP, int ROWS = kTile>
__device__ __forceinline__ void stage_dma(T* __restrict__ s, const T* __restrict__ g, int nrows) {
  constexpr int CPR = SP * (int)sizeof(T) / 16;   // 16-byte pieces per LDS row
  constexpr int DPR = NC * (int)sizeof(T) / 16;   // data pieces per row
  static_assert(SP * sizeof(T) % 16 == 0 && NC * sizeof(T) % 16 == 0, "whole 16-byte pieces");
  constexpr int NP = ROWS * CPR;   // pieces of the LDS image; a partial last load runs on fewer lanes
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T*>(g), (short)0, nrows * NC * (int)sizeof(T), 0x00020000);
  for (int n = w; n < (NP + 63) / 64; n += NT / 64) {
    const int c = 64 * n + lane, row = c / CPR, ch = min(c % CPR, DPR - 1);
    if (NP % 64 == 0 || c < NP)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t*)(reinterpret_cast<char*>(s) + 1024 * n), 16,
                                               row * NC * (int)sizeof(T) + 16 * ch, 0, 0, 0);
  }
}
// The same copy one 16-byte piece at a time (few registers: for loops that
// already hold many accumulators).
template <int NT, typename T, int NC, int SP>
__device__ __forceinline__ void stage_lean(T* __restrict__ s, const T* __restrict__ g, int64_t gp, int nrows) {
  constexpr int EV = 16 / sizeof(T);
  constexpr int VPR = NC / EV;
  for (int it = threadIdx.x; it < kTile * VPR; it += NT) {
    const int row = it / VPR, cv = it % VPR;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (row < nrows) x = *reinterpret_cast<const f32x4*>(g + (int64_t)row * gp + cv * EV);
    *reinterpret_cast<f32x4*>(s + row * SP + cv * EV) = x;
  }
}
// Two such copies with all loads of both issued before any store.
template <int NT, typename T, int NC1, int SP1, int NC2, int SP2>
__device__ __forceinline__ void stage2(T* __restrict__ s1, const T* __restrict__ g1, int64_t gp1,
                                       T* __restrict__ s2, const T* __restrict__ g2, int64_t gp2, int nrows) {
  constexpr int EV = 16 / sizeof(T);
  constexpr int VPR1 = NC1 / EV, VPR2 = NC2 / EV;
  constexpr int N1 = (kTile * VPR1 + NT - 1) / NT, N2 = (kTile * VPR2 + NT - 1) / NT;
  f32x4 x1[N1], x2[N2];
#pragma unroll
  for (int n = 0; n < N1; ++n) {
    const int it = (int)threadIdx.x + n * NT, row = it / VPR1, cv = it % VPR1;
    x1[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (it < kTile * VPR1 && row < nrows) x1[n] = *reinterpret_cast<const f32x4*>(g1 + (int64_t)row * gp1 + cv * EV);
  }
#pragma unroll
  for (int n = 0; n < N2; ++n) {
    const int it = (int)threadIdx.x + n * NT, row = it / VPR2, cv = it % VPR2;
    x2[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (it < kTile * VPR2 && row < nrows) x2[n] = *reinterpret_cast<const f32x4*>(g2 + (int64_t)row * gp2 + cv * EV);
  }
#pragma unroll
  for (int n = 0; n < N1; ++n) {
    const int it = (int)threadIdx.x + n * NT, row = it / VPR1, cv = it % VPR1;
    if (it < kTile * VPR1) *reinterpret_cast<f32x4*>(s1 + row * SP1 + cv * EV) = x1[n];
  }
#pragma unroll
  for (int n = 0; n < N2; ++n) {
    const int it = (int)threadIdx.x + n * NT, row = it / VPR2, cv = it % VPR2;
    if (it < kTile * VPR2) *reinterpret_cast<f32x4*>(s2 + row * SP2 + cv * EV) = x2[n];
  }
}
// Copy an LDS tile (row pitch SP) to rows [0, nrows) of a global array.
template <int NT, typename T, int NC, int SP>
__device__ __forceinline__ void unstage(T* __restrict__ g, int64_t gp, const T* __restrict__ s, int nrows) {
  constexpr int EV = 16 / sizeof(T);
  constexpr int VPR = NC / EV;
  for (int it = threadIdx.x; it < kTile * VPR; it += NT) {
    const int row = it / VPR, cv = it % VPR;
    if (row < nrows)
      *reinterpret_cast<f32x4*>(g + (int64_t)row * gp + cv * EV) =
          *reinterpret_cast<const f32x4*>(s + row * SP + cv * EV);
  }
}

struct BwdArgs {
  const void *q, *k, *v, *o, *h, *dh;    // [BH][T][d] of the input dtype
  const float *f_pre;
  void *dq, *dk, *dv, *dout;             // [BH][T][d]
  float *di, *df;                        // [BH][T]
  GateBuffers gb;
  const void* Cs;                        // forward chunk-start states [BH][Nc][V][K], input dtype
  const float* ns;                       // [BH][Nc][K]
  const double* ms;                      // [BH][Nc]
  void* G;                               // g per token [BH][T][V]
  float* dz;                             // dz per token [BH][T]
  float* qdq;                            // q . dq per token [BH][T]
  float* Es;                             // end adjoint of every chunk [BH][Nc][V][K]: float32, or its bf16 hi/lo terms
  float* es;                             // [BH][Nc][K]
  double* Ms;                            // its log scale [BH][Nc] (-inf: zero)
  float* L0;                             // chunk 0's share [BH][V][K] (initial state's gradient)
  float* L0e;                            // [BH][K]
  const float *C0, *n0, *m0;             // initial state, or null
  float *dC0, *dn0, *dm0;                // its gradient, or null
  int zero_first;                        // no initial state: chunk 0 starts from zero
  int es_split;                          // bfloat16: Es holds hi, lo bf16 terms interleaved by 4 (see bwd_fold_kernel)
  int64_t T, Nc, V, K, BH;
  int L;
};

// Row stabiliser r_t of the forward (see the file comment) for token t of
// chunk c; `carry` tells whether the carried state reaches row t.
__device__ __forceinline__ double row_stab(const BwdArgs& a, int64_t bh, int64_t t, bool has_state,
                                           double m_prev, bool* carry) {
  const int rs = a.gb.rs[bh * a.T + t];
  const bool cr = has_state && rs < 0;
  double r = fmax(cr ? m_prev : -INFINITY, a.gb.mp[bh * a.T + t]);
  if (r == -INFINITY) r = 0.0;
  if (carry) *carry = cr;
  return r;
}

// ------------------------------------------------------------------ dq kernel

template <typename TI, int K, int V>
struct DqLds {
  static constexpr int PAD = lds_pad<TI>();
  static constexpr int QP = K + PAD, GP = V + PAD, AP = kTile + PAD;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + kTile * QP * (int)sizeof(TI);
  static constexpr int oG = oK + kTile * QP * (int)sizeof(TI);
  static constexpr int oA = oG + kTile * GP * (int)sizeof(TI);
  static constexpr int oF = oA + kTile * AP * (int)sizeof(TI);
  // float arrays: u2, r2, sc, den, sg, dz [64] each; zp, qd [4][64]; n [K]; then int rs [64]
  static constexpr int nF = 6 * kTile + 8 * kTile + K;
  static constexpr int oI = oF + nF * 4;
  static constexpr int bytes = oI + kTile * 4;
  static_assert(bytes <= 160 * 1024, "fits the LDS of a CU");
};

template <typename TI, int K, int V>
__global__ __launch_bounds__(kBT) void bwd_dq_kernel(BwdArgs a) {
  using L = DqLds<TI, K, V>;
  constexpr int QP = L::QP, GP = L::GP, AP = L::AP;
  constexpr int CT = K / 64;   // 16-column output tiles per wave
  __shared__ __attribute__((aligned(16))) char smem[L::bytes];
  TI* sQ = reinterpret_cast<TI*>(smem + L::oQ);
  TI* sK = reinterpret_cast<TI*>(smem + L::oK);
  TI* sG = reinterpret_cast<TI*>(smem + L::oG);
  TI* sA = reinterpret_cast<TI*>(smem + L::oA);
  float* f = reinterpret_cast<float*>(smem + L::oF);
  float *s_u2 = f, *s_r2 = f + 64, *s_sc = f + 128, *s_den = f + 192, *s_sg = f + 256, *s_dz = f + 320;
  float *s_zp = f + 384, *s_qd = f + 640, *s_n = f + 896;
  int* s_rs = reinterpret_cast<int*>(smem + L::oI);

  const int64_t T = a.T, BH = a.BH;
  const int64_t bh = blockIdx.x % BH;
  const int64_t row0 = (int64_t)(blockIdx.x / BH) * kTile;
  const int64_t c = row0 / a.L;
  const int64_t t0 = c * a.L;
  const int st = (int)((row0 - t0) / kTile);
  const int nrows = (int)min((int64_t)kTile, T - row0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int jw = w & 3, zs = 2 * (w >> 2);   // score tiles: keys 16 jw.., query groups zs, zs + 1
  const int rh = w >> 2, cw = w & 3;         // output: rows 32 rh.., columns (K / 4) cw..

  const bool has_state = c > 0 || !a.zero_first;
  const double m_prev = has_state ? a.ms[bh * a.Nc + c] : 0.0;
  const double ref = row_stab(a, bh, row0, has_state, m_prev, nullptr);

  const TI* qg = static_cast<const TI*>(a.q) + bh * T * K;
  const TI* kg = static_cast<const TI*>(a.k) + bh * T * K;
  const TI* vg = static_cast<const TI*>(a.v) + bh * T * V;

  // ---------------- row data, Q tile, carried normaliser
  if (tid < kTile) {
    float r2 = 0.f, sc = 0.f, fl = 1.f;
    int rs = 0;
    if (tid < nrows) {
      const int64_t t = row0 + tid;
      bool carry;
      const double r = row_stab(a, bh, t, has_state, m_prev, &carry);
      r2 = (float)((r - ref) * (double)kL2e);
      sc = carry ? expf((float)(m_prev - r)) : 0.f;
      fl = expf((float)(-(a.gb.b[bh * T + t] + r)));
      rs = a.gb.rs[bh * T + t];
    }
    s_r2[tid] = r2;
    s_sc[tid] = sc;
    s_den[tid] = fl;   // the floor for now
    s_rs[tid] = rs;
  }
  for (int d = tid; d < K; d += kBT) s_n[d] = has_state ? a.ns[(bh * a.Nc + c) * K + d] : 0.f;
  stage_dma<kBT, TI, K, QP>(sQ, qg + row0 * K, nrows);

  // ---------------- z_t = sum_j P_tj (q_t . k_j) + sc_t (q_t . n~)
  float zrow[2] = {0.f, 0.f};
  for (int jb = 0; jb <= st; ++jb) {
    const int64_t key0 = t0 + (int64_t)jb * kTile;
    const int kvalid = (int)min((int64_t)kTile, T - key0);
    // this wave's 16 keys, all loads issued together
    vec8<TI> Kf[K / 32];
#pragma unroll
    for (int ks = 0; ks < K / 32; ++ks) Kf[ks] = frag_rows_lim(kg + key0 * K, K, 16 * jw, 32 * ks, kvalid);
    __syncthreads();   // s_u2 free; sQ, row data published
    if (tid < kTile)
      s_u2[tid] = key0 + tid < T ? (float)((a.gb.u[bh * T + key0 + tid] - ref) * (double)kL2e) : -INFINITY;
    f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < K / 32; ++ks) {
#pragma unroll
      for (int zz = 0; zz < 2; ++zz) sacc[zz] = mma32(Kf[ks], frag_rows(sQ, QP, 16 * (zs + zz), 32 * ks), sacc[zz]);
    }
    __syncthreads();   // s_u2 written
    // lane holds S^T[j = 16 jw + 4 g + r][t = 16 (zs + zz) + i]
#pragma unroll
    for (int zz = 0; zz < 2; ++zz) {
      const int tl = 16 * (zs + zz) + i;
      const int tq = st * kTile + tl;
      const float r2 = s_r2[tl];
      const int rs = s_rs[tl];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jw + 4 * g + r;
        const int jk = jb * kTile + j;
        const bool keep = tl < nrows && jk <= tq && jk >= rs;
        zrow[zz] += keep ? sacc[zz][r] * exp2f(s_u2[j] - r2) : 0.f;
      }
    }
  }
#pragma unroll
  for (int zz = 0; zz < 2; ++zz) {
    zrow[zz] += __shfl_xor(zrow[zz], 16, 64);
    zrow[zz] += __shfl_xor(zrow[zz], 32, 64);
    if (g == 0) s_zp[jw * 64 + 16 * (zs + zz) + i] = zrow[zz];
  }
  {   // q_t . n~, eight threads per row
    const int row = tid >> 3, part = tid & 7;
    float d = 0.f;
    for (int kk = part * (K / 8); kk < (part + 1) * (K / 8); ++kk) d += to_f32(sQ[row * QP + kk]) * s_n[kk];
    d += __shfl_xor(d, 1, 64);
    d += __shfl_xor(d, 2, 64);
    d += __shfl_xor(d, 4, 64);
    if (part == 0) s_qd[row] = d;
  }
  __syncthreads();
  if (tid < kTile) {
    const float z = s_zp[tid] + s_zp[64 + tid] + s_zp[128 + tid] + s_zp[192 + tid] + s_sc[tid] * s_qd[tid];
    const float fl = s_den[tid];
    s_den[tid] = fmaxf(fmaxf(fabsf(z), fl), FLT_MIN);
    s_sg[tid] = fabsf(z) > fl ? (z > 0.f ? 1.f : -1.f) : 0.f;
  }
  __syncthreads();

  // ---------------- g = dh sigmoid(o~) / den, do~ = dh h (1 - sigmoid(o~)), dz; eight rows per wave
  {
    const TI* dhg = static_cast<const TI*>(a.dh) + (bh * T + row0) * V;
    const TI* hg = static_cast<const TI*>(a.h) + (bh * T + row0) * V;
    const TI* og = static_cast<const TI*>(a.o) + (bh * T + row0) * V;
    TI* Gg = static_cast<TI*>(a.G) + (bh * T + row0) * V;
    TI* dog = static_cast<TI*>(a.dout) + (bh * T + row0) * V;
    // the rows' dh, h and o~ pieces for RB rows at a time are loaded before
    // any is used (one memory latency per group of rows)
    constexpr int RB = 4, CPL = (V / 8 + 63) / 64;   // rows per group; 8-element pieces per lane and row
    for (int r0 = 0; r0 < 8; r0 += RB) {
      vec8<TI> dh8[RB][CPL], h8[RB][CPL], o8[RB][CPL];
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const int row = 8 * w + r0 + q;
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
          const int cv = lane + 64 * u;
          dh8[q][u] = h8[q][u] = o8[q][u] = zero_v8<TI>();
          if (row < nrows && cv < V / 8) {
            const int64_t off = (int64_t)row * V + 8 * cv;
            dh8[q][u] = load8(dhg + off);
            h8[q][u] = load8(hg + off);
            o8[q][u] = load8(og + off);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const int row = 8 * w + r0 + q;
        const bool valid = row < nrows;
        const float inv = 1.f / s_den[row];
        float dot = 0.f;
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
          const int cv = lane + 64 * u;
          if (cv >= V / 8) continue;
          vec8<TI> gv = zero_v8<TI>();
          if (valid) {
            const int64_t off = (int64_t)row * V + 8 * cv;
            vec8<TI> dov;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float dh = to_f32(dh8[q][u][e]), hv = to_f32(h8[q][u][e]);
              const float sg = sigmoid(to_f32(o8[q][u][e]));
              dot += dh * hv;
              gv[e] = from_f32<TI>(dh * sg * inv);
              dov[e] = from_f32<TI>(dh * hv * (1.f - sg));
            }
            store8(Gg + off, gv);
            store8(dog + off, dov);
          }
          store8(sG + row * GP + 8 * cv, gv);
        }
        dot = wave_sum(dot);
        if (lane == 0) s_dz[row] = valid ? -s_sg[row] * dot * inv : 0.f;
      }
    }
  }
  __syncthreads();

  // ---------------- carried-state term: sc_t (G C~ + dz_t n~)
  f32x4 acc[2][CT];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < CT; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (has_state) {
    // the chunk's start state, stored by the state pass in the operand type
    // (rounded once: the carried term of dq does not cancel the way the
    // state's products with single keys can), 32 rows (values) at a time
    // through the two halves of the K region, the next block's
    // direct-to-LDS loads in flight while this one's products run
    const TI* Cst = static_cast<const TI*>(a.Cs) + (bh * a.Nc + c) * V * K;
    TI* const Cb[2] = {sK, sK + 32 * QP};
    stage_dma<kBT, TI, K, QP, 32>(Cb[0], Cst, 32);
#pragma unroll
    for (int vb = 0; vb < V / 32; ++vb) {
      __syncthreads();   // block vb landed; the other half's readers are done
      if (vb + 1 < V / 32) stage_dma<kBT, TI, K, QP, 32>(Cb[(vb + 1) & 1], Cst + (int64_t)32 * (vb + 1) * K, 32);
      vec8<TI> A[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) A[x] = frag_rows(sG, GP, 32 * rh + 16 * x, 32 * vb);
#pragma unroll
      for (int y = 0; y < CT; ++y) {
        const vec8<TI> B = frag_cols(Cb[vb & 1], QP, 0, (K / 4) * cw + 16 * y);
#pragma unroll
        for (int x = 0; x < 2; ++x) acc[x][y] = mma32(A[x], B, acc[x][y]);
      }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tl = 32 * rh + 16 * x + 4 * g + r;
        const float sc = s_sc[tl], dzt = s_dz[tl];
#pragma unroll
        for (int y = 0; y < CT; ++y) acc[x][y][r] = sc * (acc[x][y][r] + dzt * s_n[(K / 4) * cw + 16 * y + i]);
      }
  }

  // ---------------- intra-chunk key tiles: dq += (P o (G V^T + dz)) K
  constexpr int VGM = sizeof(TI) == 2 ? 8 : 4;       // V fragments loaded as one group
  constexpr int VG = (V / 32) < VGM ? (V / 32) : VGM;
  for (int jb = 0; jb <= st; ++jb) {
    const int64_t key0 = t0 + (int64_t)jb * kTile;
    const int kvalid = (int)min((int64_t)kTile, T - key0);
    vec8<TI> Vf[VG];
#pragma unroll
    for (int q = 0; q < VG; ++q) Vf[q] = frag_rows_lim(vg + key0 * V, V, 16 * jw, 32 * q, kvalid);
    __syncthreads();   // sK, sA, s_u2 free
    stage_dma<kBT, TI, K, QP>(sK, kg + key0 * K, kvalid);
    if (tid < kTile)
      s_u2[tid] = tid < kvalid ? (float)((a.gb.u[bh * T + key0 + tid] - ref) * (double)kL2e) : -INFINITY;
    f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < V / 32; kb += VG) {
      if (kb > 0) {
#pragma unroll
        for (int q = 0; q < VG; ++q) Vf[q] = frag_rows_lim(vg + key0 * V, V, 16 * jw, 32 * (kb + q), kvalid);
      }
#pragma unroll
      for (int q = 0; q < VG; ++q)
#pragma unroll
        for (int zz = 0; zz < 2; ++zz) sacc[zz] = mma32(Vf[q], frag_rows(sG, GP, 16 * (zs + zz), 32 * (kb + q)), sacc[zz]);
    }
    __syncthreads();   // s_u2, sK written
#pragma unroll
    for (int zz = 0; zz < 2; ++zz) {
      const int tl = 16 * (zs + zz) + i;
      const int tq = st * kTile + tl;
      const float r2 = s_r2[tl], dzt = s_dz[tl];
      const int rs = s_rs[tl];
      f32x4 pa;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jw + 4 * g + r;
        const int jk = jb * kTile + j;
        const bool keep = tl < nrows && jk <= tq && jk >= rs;
        pa[r] = keep ? exp2f(s_u2[j] - r2) * (sacc[zz][r] + dzt) : 0.f;
      }
      store4(sA + tl * AP + 16 * jw + 4 * g, pa);
    }
    __syncthreads();   // sA complete
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      vec8<TI> A[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) A[x] = frag_rows(sA, AP, 32 * rh + 16 * x, 32 * ks);
#pragma unroll
      for (int y = 0; y < CT; ++y) {
        const vec8<TI> B = frag_cols(sK, QP, 32 * ks, (K / 4) * cw + 16 * y);
#pragma unroll
        for (int x = 0; x < 2; ++x) acc[x][y] = mma32(A[x], B, acc[x][y]);
      }
    }
  }

  // ---------------- epilogue: q . dq per row, dq through LDS, dz and q . dq out
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = 32 * rh + 16 * x + 4 * g + r;
      float p = 0.f;
#pragma unroll
      for (int y = 0; y < CT; ++y) p += acc[x][y][r] * to_f32(sQ[tl * QP + (K / 4) * cw + 16 * y + i]);
      p += __shfl_xor(p, 1, 64);
      p += __shfl_xor(p, 2, 64);
      p += __shfl_xor(p, 4, 64);
      p += __shfl_xor(p, 8, 64);
      if (i == 0) s_qd[64 * cw + tl] = p;
    }
  __syncthreads();   // all MFMA reads of sK done
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < CT; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sK[(32 * rh + 16 * x + 4 * g + r) * QP + (K / 4) * cw + 16 * y + i] = from_f32<TI>(acc[x][y][r]);
  __syncthreads();
  unstage<kBT, TI, K, QP>(static_cast<TI*>(a.dq) + (bh * T + row0) * K, K, sK, nrows);
  if (tid < nrows) {
    a.qdq[bh * T + row0 + tid] = s_qd[tid] + s_qd[64 + tid] + s_qd[128 + tid] + s_qd[192 + tid];
    a.dz[bh * T + row0 + tid] = s_dz[tid];
  }
}

// ------------------------------------------------------------------ reverse state pass

template <typename TI, int K>
struct RsLds {
  static constexpr int PAD = lds_pad<TI>();
  static constexpr int P = kTile + PAD;
  static constexpr int oG = 0;                                   // g tile [64 tokens][64 v]
  static constexpr int oQ = oG + kTile * P * (int)sizeof(TI);    // w q tile [64 tokens][64 d]
  static constexpr int oF = oQ + kTile * P * (int)sizeof(TI);    // float: w [256], wdz [256], ep [4][64]
  static constexpr int bytes = oF + (2 * kThreads + 4 * kTile) * 4;
};

// One workgroup per (head, 64 v x 64 d tile, chunk c), four waves of 32 x 32:
// chunk c's own share of the adjoint at its start, the sum over its tokens s
// before its first zero forget gate of w_s g_s q_s^T with
// w_s = exp(r_first - r_s) <= 1 (its log scale is -r_first), float32, into
// the slot of chunk c - 1 (chunk 0's, wanted for the initial state's
// gradient only, into L0). The normaliser part (v-tile-0 workgroups) is the
// same sum with g_s replaced by dz_s, on the vector ALU from the staged q.
// Chunks are independent here; bwd_fold_kernel chains them. The weights of
// 256 tokens are formed in one pass, and each 64-token block's g and q are
// loaded into registers while the previous block's products run, so a block
// costs no memory latency of its own.
template <typename TI, int K>
__global__ __launch_bounds__(kThreads) void bwd_local_kernel(BwdArgs a) {
  using L = RsLds<TI, K>;
  constexpr int P = L::P;
  constexpr int KT = K / 64;
  __shared__ __attribute__((aligned(16))) char smem[L::bytes];
  TI* sG = reinterpret_cast<TI*>(smem + L::oG);
  TI* sQ = reinterpret_cast<TI*>(smem + L::oQ);
  float* s_w = reinterpret_cast<float*>(smem + L::oF);
  float* s_wdz = s_w + kThreads;
  float* s_ep = s_wdz + kThreads;

  const int64_t T = a.T, BH = a.BH, V = a.V;
  const int ntile = KT * (int)(V / 64);
  const int64_t bh = blockIdx.x % BH;
  const int64_t rest = blockIdx.x / BH;
  const int tile = (int)(rest % ntile);
  const int64_t c = rest / ntile + (a.dC0 ? 0 : 1);
  const int kt = tile % KT, vt = tile / KT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int wk = w & 1, wv = w >> 1;
  const bool e_tile = vt == 0;

  const TI* qg = static_cast<const TI*>(a.q) + bh * T * K + 64 * kt;
  const TI* Gg = static_cast<const TI*>(a.G) + bh * T * V + 64 * vt;
  const int64_t t0 = c * a.L;
  const int Lc = (int)min((int64_t)a.L, T - t0);
  const bool has_state = c > 0 || !a.zero_first;
  const double m_prev = has_state ? a.ms[bh * a.Nc + c] : 0.0;
  const double r_first = row_stab(a, bh, t0, has_state, m_prev, nullptr);

  f32x4 lacc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) lacc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
  float le = 0.f;
  // this thread's staging items: item it = tid + kThreads u is row it / 8,
  // 16-byte piece it % 8 of the block's g and q tiles (rows past the chunk: zero)
  constexpr int kItems = kTile * 8 / kThreads;
  vec8<TI> gr[kItems], qr[kItems];
  auto load_block = [&](int jb) {
    const int64_t tb = t0 + jb;
    const int nv = min(kTile, Lc - jb);
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
      const int it = tid + kThreads * u, row = it >> 3, cv = it & 7;
      gr[u] = qr[u] = zero_v8<TI>();
      if (row < nv) {
        gr[u] = load8(Gg + (tb + row) * V + 8 * cv);
        qr[u] = load8(qg + (tb + row) * K + 8 * cv);
      }
    }
  };
  load_block(0);
  for (int jb = 0; jb < Lc; jb += kTile) {
    const int nv = min(kTile, Lc - jb);
    const int sb = jb % kThreads;   // the block's first token within its weight pass
    if (jb > 0) {
      __syncthreads();   // the previous block's reads of the tiles and weights are done
      if (e_tile && tid < kTile) le += s_ep[tid] + s_ep[64 + tid] + s_ep[128 + tid] + s_ep[192 + tid];
    }
    if (sb == 0) {   // the weights of the next kThreads tokens, one per thread
      const int64_t tt = t0 + jb + tid;
      float wt = 0.f, wdz = 0.f;
      if (jb + tid < Lc && a.gb.rs[bh * T + tt] < 0) {
        const double r = row_stab(a, bh, tt, has_state, m_prev, nullptr);
        wt = expf((float)(r_first - r));
        wdz = wt * a.dz[bh * T + tt];
      }
      s_w[tid] = wt;
      s_wdz[tid] = wdz;
      __syncthreads();
    }
    // stage w g[tokens][64 v] and q[tokens][64 d]. The weight goes on g: a
    // rounding of w_s g_s perturbs each term in proportion to itself, so the
    // adjoint's products with later keys (which can cancel strongly) keep
    // their accuracy; q stays exact.
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
      const int it = tid + kThreads * u, row = it >> 3, cv = it & 7;
      const float wt = s_w[sb + row];
      vec8<TI> gv;
#pragma unroll
      for (int e = 0; e < 8; ++e) gv[e] = from_f32<TI>(to_f32(gr[u][e]) * wt);
      store8(sG + row * P + 8 * cv, gv);
      store8(sQ + row * P + 8 * cv, qr[u]);
    }
    if (jb + kTile < Lc) load_block(jb + kTile);   // in flight during this block's products
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kTile; kk += 32) {
      vec8<TI> A[2], B[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) A[x] = frag_cols(sG, P, kk, 32 * wv + 16 * x);
#pragma unroll
      for (int y = 0; y < 2; ++y) B[y] = frag_cols(sQ, P, kk, 32 * wk + 16 * y);
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) lacc[x][y] = mma32(A[x], B[y], lacc[x][y]);
    }
    if (e_tile) {   // normaliser part from the staged q: four threads per d, 16 tokens each
      const int d = tid & 63, part = tid >> 6;
      float sum = 0.f;
      for (int row = 16 * part; row < 16 * part + 16; ++row)
        if (row < nv) sum += s_wdz[sb + row] * to_f32(sQ[row * P + d]);
      s_ep[part * 64 + d] = sum;
    }
  }
  if (e_tile) {
    __syncthreads();
    if (tid < kTile) le += s_ep[tid] + s_ep[64 + tid] + s_ep[128 + tid] + s_ep[192 + tid];
  }
  float* dst = c > 0 ? a.Es + (bh * a.Nc + c - 1) * V * K : a.L0 + bh * V * K;
  float* edst = c > 0 ? a.es + (bh * a.Nc + c - 1) * K : a.L0e + bh * K;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int64_t vv = 64 * vt + 32 * wv + 16 * x + 4 * g;
      const int dd = 64 * kt + 32 * wk + 16 * y + i;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(vv + r) * K + dd] = lacc[x][y][r];
    }
  if (e_tile && tid < kTile) edst[64 * kt + tid] = le;
}

// The chunks' end adjoints from their local shares, last chunk to first:
// one thread per four consecutive elements of a head's d_v x d_qk adjoint
// (and d_qk / 4 threads for its normaliser part). With A = 0, M = -inf after
// the last chunk, for c = Nc-1 .. 1: the slot of chunk c receives A (the
// adjoint at its end), and with chunk c's local share Lc (in slot c - 1)
//   M' = max(-r_first(c), g_c + M if chunk c has no zero forget gate),
//   A' = exp(-r_first(c) - M') Lc + exp(g_c + M - M') A;
// slot 0 receives the last A. With the initial state's gradient wanted, one
// more step with chunk 0's share gives dC~0 = exp(m0 + M) A (and dn~0).
__global__ __launch_bounds__(kThreads) void bwd_fold_kernel(BwdArgs a) {
  const int64_t K = a.K, V = a.V, Nc = a.Nc;
  const int64_t vk4 = V * K / 4, k4 = K / 4, per_head = vk4 + k4;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= a.BH * per_head) return;
  const int64_t bh = gid / per_head, x = gid % per_head;
  const bool is_e = x >= vk4;
  float* base = is_e ? a.es + bh * Nc * K + 4 * (x - vk4) : a.Es + bh * Nc * V * K + 4 * x;
  const int64_t stride = is_e ? K : V * K;
  f32x4 A = {0.f, 0.f, 0.f, 0.f};
  double M = -INFINITY;
  auto fold = [&](int64_t c, const f32x4& Lc) {
    const bool has_state = c > 0 || !a.zero_first;
    const double m_prev = has_state ? a.ms[bh * Nc + c] : 0.0;
    const double Mloc = -row_stab(a, bh, c * a.L, has_state, m_prev, nullptr);
    const bool open = a.gb.R[bh * Nc + c] < 0;
    const double Mc = (open && M != -INFINITY) ? a.gb.g[bh * Nc + c] + M : -INFINITY;
    const double Mn = fmax(Mloc, Mc);
    const float al = expf((float)(Mloc - Mn));
    const float be = Mc == -INFINITY ? 0.f : expf((float)(Mc - Mn));
    A = al * Lc + be * A;
    M = Mn;
  };
  // The end adjoints of the value-key matrix: for bfloat16 inputs each group
  // of four as its bf16 terms hi (4) then lo (4), in the same 16 bytes, the
  // operand form the dk/dv kernel multiplies with. Slot c's local share has
  // been read before slot c is written, so the slots can be rewritten in place.
  const bool split = a.es_split && !is_e;
  auto put = [&](float* p, const f32x4& v) {
    if (split) {
      bf16x4 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hi[r] = (__bf16)v[r];
        lo[r] = (__bf16)(v[r] - (float)hi[r]);
      }
      *reinterpret_cast<bf16x4*>(p) = hi;
      *reinterpret_cast<bf16x4*>(p + 2) = lo;
    } else {
      *reinterpret_cast<f32x4*>(p) = v;
    }
  };
  for (int64_t c = Nc - 1; c >= 1; --c) {
    put(base + c * stride, A);
    if (x == 0) a.Ms[bh * Nc + c] = M;
    fold(c, *reinterpret_cast<const f32x4*>(base + (c - 1) * stride));
  }
  put(base, A);
  if (x == 0) a.Ms[bh * Nc] = M;
  if (a.dC0) {
    const float* l0 = is_e ? a.L0e + bh * K + 4 * (x - vk4) : a.L0 + bh * V * K + 4 * x;
    fold(0, *reinterpret_cast<const f32x4*>(l0));
    const double m0 = a.C0 ? (double)a.m0[bh] : 0.0;
    const float sc = M == -INFINITY ? 0.f : expf((float)(m0 + M));
    float* d0 = is_e ? a.dn0 + bh * K + 4 * (x - vk4) : a.dC0 + bh * V * K + 4 * x;
    *reinterpret_cast<f32x4*>(d0) = sc * A;
  }
}

// ------------------------------------------------------------------ dk / dv kernel

template <typename TI, int K, int V>
struct DkvLds {
  static constexpr int PAD = lds_pad<TI>();
  static constexpr int QP = K + PAD, GP = V + PAD, AP = kTile + PAD;
  static constexpr int oQ = 0;                                    // Q tile / K_j / end-adjoint block
  static constexpr int oG = oQ + kTile * QP * (int)sizeof(TI);    // G tile / V_j
  static constexpr int oA = oG + kTile * GP * (int)sizeof(TI);    // (P o (G V^T + dz))^T
  static constexpr int oB = oA + kTile * AP * (int)sizeof(TI);    // (P o S)^T
  static constexpr int oF = oB + kTile * AP * (int)sizeof(TI);
  // float: u2, r2, dz, wj [64]; di [4][64]; e [K]; then int rs [64]
  static constexpr int nF = 4 * kTile + 4 * kTile + K;
  static constexpr int oI = oF + nF * 4;
  // blocks of 32 end-adjoint rows: bfloat16, each row as 4-element groups of
  // hi then lo (pitch EP elements); float32, rows of K (pitch QP). The first
  // buffer is the Q region, the second follows.
  static constexpr int EP = sizeof(TI) == 2 ? 2 * K + 16 : QP;
  static constexpr int oE2 = (oI + kTile * 4 + 15) / 16 * 16;
  static constexpr int bytes = oE2 + 32 * EP * (int)sizeof(TI);
  static_assert(32 * EP * sizeof(TI) <= kTile * QP * sizeof(TI), "an adjoint block fits the Q region");
  static_assert(bytes <= 160 * 1024, "fits the LDS of a CU");
};

// Transposed operand fragment of an interleaved adjoint block (row pitch P):
// lane (i, g) receives the hi (part 0) or lo (part 1) terms of column n0 + i
// of rows k0 + 8 g .. + 7, where column d's terms sit at 2 d - d % 4 (hi)
// and 4 further (lo) of its row, as the fold kernel stores them.
__device__ __forceinline__ bf16x8 frag_cols_il(const __bf16* X, int P, int k0, int n0, int part) {
  const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
  const __bf16* p = X + (k0 + 8 * g + (i >> 2)) * P + 2 * n0 + 8 * (i & 3) + 4 * part;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_b4*)(p + 4 * P));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Row operand fragment of an interleaved adjoint block: lane (i, g) receives
// the hi and lo terms of row r0 + i, columns k0 + 8 g .. + 7.
__device__ __forceinline__ void frag_rows_il(const __bf16* X, int P, int r0, int k0, bf16x8& hi, bf16x8& lo) {
  const int lane = threadIdx.x & 63;
  const __bf16* p = X + (r0 + (lane & 15)) * P + 2 * (k0 + 8 * (lane >> 4));
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
  const bf16x8 b = *reinterpret_cast<const bf16x8*>(p + 8);
  hi = __builtin_shufflevector(a, b, 0, 1, 2, 3, 8, 9, 10, 11);
  lo = __builtin_shufflevector(a, b, 4, 5, 6, 7, 12, 13, 14, 15);
}

template <typename TI, int K, int V>
__global__ __launch_bounds__(kBT) void bwd_dkv_kernel(BwdArgs a) {
  using L = DkvLds<TI, K, V>;
  constexpr int QP = L::QP, GP = L::GP, AP = L::AP;
  constexpr int CK = K / 64;   // 16-column output tiles per wave
  __shared__ __attribute__((aligned(16))) char smem[L::bytes];
  TI* sQ = reinterpret_cast<TI*>(smem + L::oQ);
  TI* sG = reinterpret_cast<TI*>(smem + L::oG);
  TI* sA = reinterpret_cast<TI*>(smem + L::oA);
  TI* sB = reinterpret_cast<TI*>(smem + L::oB);
  float* f = reinterpret_cast<float*>(smem + L::oF);
  float *s_u2 = f, *s_r2 = f + 64, *s_dz = f + 128, *s_wj = f + 192, *s_di = f + 256, *s_e = f + 512;
  int* s_rs = reinterpret_cast<int*>(smem + L::oI);

  const int64_t T = a.T, BH = a.BH;
  const int64_t bh = blockIdx.x % BH;
  const int64_t key0 = (int64_t)(blockIdx.x / BH) * kTile;
  const int64_t c = key0 / a.L;
  const int64_t t0 = c * a.L;
  const int jt = (int)((key0 - t0) / kTile);
  const int nkeys = (int)min((int64_t)kTile, T - key0);
  const int ntiles = (int)((min(T, t0 + a.L) - t0 + kTile - 1) / kTile);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int jw = w & 3, zs = 2 * (w >> 2);   // score tiles: keys 16 jw.., query groups zs, zs + 1
  const int rh = w >> 2, cw = w & 3;         // outputs: key rows 32 rh.., columns (d / 4) cw..

  const bool has_state = c > 0 || !a.zero_first;
  const double m_prev = has_state ? a.ms[bh * a.Nc + c] : 0.0;
  const double ref = row_stab(a, bh, key0, has_state, m_prev, nullptr);

  const TI* qg = static_cast<const TI*>(a.q) + bh * T * K;
  const TI* kg = static_cast<const TI*>(a.k) + bh * T * K;
  const TI* vg = static_cast<const TI*>(a.v) + bh * T * V;
  const TI* Gg = static_cast<const TI*>(a.G) + bh * T * V;

  // dk: wave (rh, cw) owns key rows 32 rh .. + 31, columns (K / 4) cw .. ;
  // dv: wave w owns key rows 16 jw .. + 15 and the value tiles 2 vb + rh
  // (16 columns each, vb = 0 .. V / 32 - 1), so that every 32-row block of
  // the end adjoint below gives each wave the same share of the work
  constexpr int NVT = V / 32;
  f32x4 ak[2][CK], av[NVT];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < CK; ++y) ak[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int y = 0; y < NVT; ++y) av[y] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's 16 keys: the A operand of dv's end-adjoint term and the B
  // operand of S = Q K^T
  vec8<TI> Kf[K / 32];
#pragma unroll
  for (int ks = 0; ks < K / 32; ++ks) Kf[ks] = frag_rows_lim(kg + key0 * K, K, 16 * jw, 32 * ks, nkeys);

  // ---------------- key data; the end adjoint's term w_j (A^T v_j + a), w_j A k_j
  const double Mc = a.Ms[bh * a.Nc + c];
  const bool later = Mc != -INFINITY;
  if (tid < kTile) {
    float u2 = -INFINITY, wj = 0.f;
    if (tid < nkeys) {
      const double u = a.gb.u[bh * T + key0 + tid];
      u2 = (float)((u - ref) * (double)kL2e);
      const int Rc = a.gb.R[bh * a.Nc + c];
      if (later && (int)(key0 - t0) + tid >= Rc) wj = expf((float)(u + a.gb.g[bh * a.Nc + c] + Mc));
    }
    s_u2[tid] = u2;
    s_wj[tid] = wj;
  }
  if (later) {
    // The end adjoint A is float32. Its products with a key (k_j . A) can
    // cancel strongly (rows whose g is large because their q . k is small),
    // so for bfloat16 it enters the MFMAs as two terms, hi + lo, which the
    // fold kernel stores interleaved in place of the float32 values. It is
    // streamed once, 32 rows (values) at a time, through two LDS buffers,
    // the next block's direct-to-LDS loads in flight while this one's
    // products run; each block serves both
    //   dk[j][d] += sum_v V_j[j][v] A[v][d]   (every wave: its dk tile)
    //   dv[j][v] += sum_d K_j[j][d] A[v][d]   (every wave: value tile 2 vb + rh)
    constexpr int EP = L::EP;
    TI* Ebuf[2] = {sQ, reinterpret_cast<TI*>(smem + L::oE2)};
    for (int d = tid; d < K; d += kBT) s_e[d] = a.es[(bh * a.Nc + c) * K + d];
    stage_dma<kBT, TI, V, GP>(sG, vg + key0 * V, nkeys);
    const float* Es = a.Es + (bh * a.Nc + c) * V * K;
    auto load_block = [&](int vb, TI* dst) {
      if constexpr (sizeof(TI) == 2) {
        stage_dma<kBT, __bf16, 2 * K, EP, 32>(reinterpret_cast<__bf16*>(dst),
                                              reinterpret_cast<const __bf16*>(Es) + (int64_t)32 * vb * 2 * K, 32);
      } else {
        stage_dma<kBT, float, K, EP, 32>(reinterpret_cast<float*>(dst), Es + (int64_t)32 * vb * K, 32);
      }
    };
    load_block(0, Ebuf[0]);
#pragma unroll
    for (int vb = 0; vb < V / 32; ++vb) {
      __syncthreads();   // block vb (and V_j) landed; the other buffer's last readers are done
      if (vb + 1 < V / 32) load_block(vb + 1, Ebuf[(vb + 1) & 1]);
      const TI* Eb = Ebuf[vb & 1];
      vec8<TI> A[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) A[x] = frag_rows(sG, GP, 32 * rh + 16 * x, 32 * vb);
#pragma unroll
      for (int y = 0; y < CK; ++y) {
        if constexpr (sizeof(TI) == 2) {
          const bf16x8 Bh = frag_cols_il(Eb, EP, 0, (K / 4) * cw + 16 * y, 0);
          const bf16x8 Bl = frag_cols_il(Eb, EP, 0, (K / 4) * cw + 16 * y, 1);
#pragma unroll
          for (int x = 0; x < 2; ++x) ak[x][y] = mma32(A[x], Bl, mma32(A[x], Bh, ak[x][y]));
        } else {
          const vec8<TI> B = frag_cols(Eb, EP, 0, (K / 4) * cw + 16 * y);
#pragma unroll
          for (int x = 0; x < 2; ++x) ak[x][y] = mma32(A[x], B, ak[x][y]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < K / 32; ++ks) {
        if constexpr (sizeof(TI) == 2) {
          bf16x8 Bh, Bl;
          frag_rows_il(Eb, EP, 16 * rh, 32 * ks, Bh, Bl);
          av[vb] = mma32(Kf[ks], Bl, mma32(Kf[ks], Bh, av[vb]));
        } else {
          av[vb] = mma32(Kf[ks], frag_rows(Eb, EP, 16 * rh, 32 * ks), av[vb]);
        }
      }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jl = 32 * rh + 16 * x + 4 * g + r;
        const float wj = s_wj[jl];
#pragma unroll
        for (int y = 0; y < CK; ++y) ak[x][y][r] = wj * (ak[x][y][r] + s_e[(K / 4) * cw + 16 * y + i]);
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float wj = s_wj[16 * jw + 4 * g + r];
#pragma unroll
      for (int y = 0; y < NVT; ++y) av[y][r] *= wj;
    }
  }

  // ---------------- the chunk's query tiles at or after this key tile
  constexpr int VGM = 4;   // V_j fragments loaded as one group
  constexpr int VG = (V / 32) < VGM ? (V / 32) : VGM;
  for (int sb = jt; sb < ntiles; ++sb) {
    const int64_t qrow0 = t0 + (int64_t)sb * kTile;
    const int nq = (int)min((int64_t)kTile, T - qrow0);
    __syncthreads();   // sQ, sG, sA, sB and the row data free
    stage_dma<kBT, TI, K, QP>(sQ, qg + qrow0 * K, nq);
    stage_dma<kBT, TI, V, GP>(sG, Gg + qrow0 * V, nq);
    if (tid < kTile) {
      float r2 = 0.f, dzt = 0.f;
      int rs = kTile * 1024;   // no key passes jk >= rs for rows beyond T
      if (tid < nq) {
        const int64_t t = qrow0 + tid;
        const double r = row_stab(a, bh, t, has_state, m_prev, nullptr);
        r2 = (float)((r - ref) * (double)kL2e);
        dzt = a.dz[bh * T + t];
        rs = a.gb.rs[bh * T + t];
      }
      s_r2[tid] = r2;
      s_dz[tid] = dzt;
      s_rs[tid] = rs;
    }
    __syncthreads();
    // S[t][j] and (G V^T)[t][j] for this wave's keys and query groups
    f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    f32x4 gacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < K / 32; ++ks)
#pragma unroll
      for (int zz = 0; zz < 2; ++zz) sacc[zz] = mma32(frag_rows(sQ, QP, 16 * (zs + zz), 32 * ks), Kf[ks], sacc[zz]);
#pragma unroll
    for (int kb = 0; kb < V / 32; kb += VG) {
      vec8<TI> Vf[VG];
#pragma unroll
      for (int q = 0; q < VG; ++q) Vf[q] = frag_rows_lim(vg + key0 * V, V, 16 * jw, 32 * (kb + q), nkeys);
#pragma unroll
      for (int q = 0; q < VG; ++q)
#pragma unroll
        for (int zz = 0; zz < 2; ++zz)
          gacc[zz] = mma32(frag_rows(sG, GP, 16 * (zs + zz), 32 * (kb + q)), Vf[q], gacc[zz]);
    }
    // lane holds [t = 16 (zs + zz) + 4 g + r][j = 16 jw + i]
    {
      const int j = 16 * jw + i;
      const int jk = jt * kTile + j;
      const float u2 = s_u2[j];
#pragma unroll
      for (int zz = 0; zz < 2; ++zz) {
        f32x4 pa, pb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tl = 16 * (zs + zz) + 4 * g + r;
          const int tq = sb * kTile + tl;
          const bool keep = tl < nq && j < nkeys && jk <= tq && jk >= s_rs[tl];
          const float p = keep ? exp2f(u2 - s_r2[tl]) : 0.f;
          pa[r] = p * (gacc[zz][r] + s_dz[tl]);
          pb[r] = p * sacc[zz][r];
        }
        store4(sA + j * AP + 16 * (zs + zz) + 4 * g, pa);
        store4(sB + j * AP + 16 * (zs + zz) + 4 * g, pb);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      vec8<TI> A[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) A[x] = frag_rows(sA, AP, 32 * rh + 16 * x, 32 * ks);
#pragma unroll
      for (int y = 0; y < CK; ++y) {
        const vec8<TI> B = frag_cols(sQ, QP, 32 * ks, (K / 4) * cw + 16 * y);
#pragma unroll
        for (int x = 0; x < 2; ++x) ak[x][y] = mma32(A[x], B, ak[x][y]);
      }
      const vec8<TI> B2 = frag_rows(sB, AP, 16 * jw, 32 * ks);
#pragma unroll
      for (int y = 0; y < NVT; ++y) av[y] = mma32(B2, frag_cols(sG, GP, 32 * ks, 16 * (2 * y + rh)), av[y]);
    }
  }

  // ---------------- epilogue: di = k . dk, dk and dv through LDS
  __syncthreads();   // all MFMA reads of sQ, sG done
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jl = 32 * rh + 16 * x + 4 * g + r;
      float p = 0.f;
#pragma unroll
      for (int y = 0; y < CK; ++y) {
        const int d = (K / 4) * cw + 16 * y + i;
        const float kv = jl < nkeys ? to_f32(kg[(key0 + jl) * K + d]) : 0.f;
        p += ak[x][y][r] * kv;
        sQ[jl * QP + d] = from_f32<TI>(ak[x][y][r]);
      }

      p += __shfl_xor(p, 1, 64);
      p += __shfl_xor(p, 2, 64);
      p += __shfl_xor(p, 4, 64);
      p += __shfl_xor(p, 8, 64);
      if (i == 0) s_di[64 * cw + jl] = p;
    }
#pragma unroll
  for (int y = 0; y < NVT; ++y)
#pragma unroll
    for (int r = 0; r < 4; ++r) sG[(16 * jw + 4 * g + r) * GP + 16 * (2 * y + rh) + i] = from_f32<TI>(av[y][r]);
  __syncthreads();
  unstage<kBT, TI, K, QP>(static_cast<TI*>(a.dk) + (bh * T + key0) * K, K, sQ, nkeys);
  unstage<kBT, TI, V, GP>(static_cast<TI*>(a.dv) + (bh * T + key0) * V, V, sG, nkeys);
  if (tid < nkeys) a.di[bh * T + key0 + tid] = s_di[tid] + s_di[64 + tid] + s_di[128 + tid] + s_di[192 + tid];
}

// ------------------------------------------------------------------ forget-gate gradient

// One workgroup per head. dF_t = q_t . dq_t - k_t . dk_t; the gradient of
// log f_l is the sum of dF_t from l up to the next zero forget gate
// (exclusive), and 0 at a zero forget gate itself and, without an initial
// state, at the first token; df~ = dlog f sigmoid(-f~). Each thread takes a
// contiguous run of tokens, thread p the p-th run from the end. A run maps
// the sum flowing into it from the right to the sum flowing out of its left
// end by an affine map c -> alpha c + beta (alpha = 0 where a zero forget
// gate blocks the flow); a scan of the composed maps over the threads gives
// every run its inflow. Float64 sums. Also dm0 = <dC~0, C~0> + dn~0 . n~0.
// The forget-gate gradient needs, per token, run_l = 0 at a blocked token (a
// zero forget gate, or the first token without an initial state) and
// q.dq_l - di_l + run_{l+1} otherwise: a reverse scan over the sequence. A
// stretch of tokens acts on the run entering at its end as x -> A x + B
// (A = 0 once a token in it is blocked), and stretches compose. Both kernels
// below take one workgroup per (head, chunk): the first stores each chunk's
// map, the second composes the maps of the later chunks into the run
// entering its chunk and writes df. The maps live in the end-adjoint
// normaliser buffer, which the dk/dv kernel has finished with.
struct RevMap {
  double A, B;
};

__device__ __forceinline__ double* gate_maps(const BwdArgs& a) { return reinterpret_cast<double*>(a.es); }

// The map of tokens [lo, hi) of one head (the entering run applied at hi - 1).
__device__ __forceinline__ RevMap token_run_map(const BwdArgs& a, int64_t bh, int64_t lo, int64_t hi) {
  const float* fp = a.f_pre + bh * a.T;
  const float* qd = a.qdq + bh * a.T;
  const float* di = a.di + bh * a.T;
  RevMap m{1.0, 0.0};
  for (int64_t l = hi - 1; l >= lo; --l) {
    if (fp[l] == -INFINITY || (l == 0 && a.zero_first)) {
      m = RevMap{0.0, 0.0};
    } else {
      m.B += (double)qd[l] - (double)di[l];
    }
  }
  return m;
}

// Scan of the threads' maps within the workgroup, thread 0 holding the
// latest stretch: returns the composition of the threads before this one
// (the later stretches) and, in *total, the whole workgroup's map.
__device__ __forceinline__ RevMap rev_scan(RevMap m, RevMap* total, double* s_a, double* s_b) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  double A_ = m.A, B_ = m.B;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double ao = __shfl_up(A_, d, 64), bo = __shfl_up(B_, d, 64);
    if (lane >= d) {
      B_ = A_ * bo + B_;
      A_ = A_ * ao;
    }
  }
  if (lane == 63) { s_a[w] = A_; s_b[w] = B_; }
  __syncthreads();
  double Aw = 1.0, Bw = 0.0;   // the waves before this one (later stretches), composed
  for (int q = 0; q < w; ++q) {
    Bw = s_a[q] * Bw + s_b[q];
    Aw = s_a[q] * Aw;
  }
  double Ae = __shfl_up(A_, 1, 64), Bx = __shfl_up(B_, 1, 64);
  if (lane == 0) { Ae = 1.0; Bx = 0.0; }
  double At = 1.0, Bt = 0.0;
  for (int q = 0; q < kThreads / 64; ++q) {
    Bt = s_a[q] * Bt + s_b[q];
    At = s_a[q] * At;
  }
  *total = RevMap{At, Bt};
  return RevMap{Ae * Aw, Ae * Bw + Bx};
}

// This thread's tokens of chunk c: contiguous runs, thread 0 the last.
__device__ __forceinline__ void chunk_run(const BwdArgs& a, int64_t c, int64_t* lo, int64_t* hi) {
  const int64_t p0 = c * a.L, p1 = min(p0 + a.L, a.T);
  const int64_t E = (p1 - p0 + kThreads - 1) / kThreads;
  const int64_t run_idx = kThreads - 1 - threadIdx.x;
  *lo = min(p0 + run_idx * E, p1);
  *hi = min(*lo + E, p1);
}

__device__ __forceinline__ double block_sum(double s, double* s_red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  __syncthreads();   // s_red free (earlier readers done)
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = s;
  __syncthreads();
  return s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

__global__ __launch_bounds__(kThreads) void bwd_gate_map_kernel(BwdArgs a) {
  __shared__ double s_a[kThreads / 64], s_b[kThreads / 64], s_red[kThreads / 64];
  const int64_t bh = blockIdx.x / a.Nc, c = blockIdx.x % a.Nc;
  int64_t lo, hi;
  chunk_run(a, c, &lo, &hi);
  RevMap tot;
  rev_scan(token_run_map(a, bh, lo, hi), &tot, s_a, s_b);
  // this chunk's share of sum(dC0 o C0) + sum(dn0 o n0), the initial
  // stabiliser's gradient (0 without an initial state)
  double s = 0.0;
  if (a.dm0 && a.C0) {
    const int64_t VK = a.V * a.K, N = VK + a.K, per = (N + a.Nc - 1) / a.Nc;
    const int64_t x1 = min((c + 1) * per, N);
    for (int64_t x = c * per + threadIdx.x; x < x1; x += kThreads)
      s += x < VK ? (double)a.dC0[bh * VK + x] * (double)a.C0[bh * VK + x]
                  : (double)a.dn0[bh * a.K + x - VK] * (double)a.n0[bh * a.K + x - VK];
  }
  s = block_sum(s, s_red);
  if (threadIdx.x == 0) {
    double* gm = gate_maps(a) + (bh * a.Nc + c) * 4;
    gm[0] = tot.A;
    gm[1] = tot.B;
    gm[2] = s;
  }
}

__global__ __launch_bounds__(kThreads) void bwd_gate_kernel(BwdArgs a) {
  __shared__ double s_a[kThreads / 64], s_b[kThreads / 64], s_red[kThreads / 64];
  const int64_t bh = blockIdx.x / a.Nc, c = blockIdx.x % a.Nc;
  const double* gm = gate_maps(a) + bh * a.Nc * 4;
  // the run entering the chunk: chunks c+1 .. Nc-1, in contiguous groups per
  // thread (thread 0 the last), composed and applied to 0
  RevMap carry_tot;
  {
    const int64_t nq = a.Nc - 1 - c, E = (nq + kThreads - 1) / kThreads;
    const int64_t run_idx = kThreads - 1 - threadIdx.x;
    const int64_t q0 = c + 1 + min(run_idx * E, nq), q1 = c + 1 + min((run_idx + 1) * E, nq);
    RevMap m{1.0, 0.0};
    for (int64_t q = q1 - 1; q >= q0; --q) {
      const double Aq = gm[q * 4], Bq = gm[q * 4 + 1];
      m = RevMap{Aq * m.A, Aq * m.B + Bq};
    }
    rev_scan(m, &carry_tot, s_a, s_b);
  }
  const double carry_in = carry_tot.B;
  __syncthreads();   // s_a, s_b reused
  int64_t lo, hi;
  chunk_run(a, c, &lo, &hi);
  RevMap tot;
  const RevMap ex = rev_scan(token_run_map(a, bh, lo, hi), &tot, s_a, s_b);
  const float* fp = a.f_pre + bh * a.T;
  const float* qd = a.qdq + bh * a.T;
  const float* di = a.di + bh * a.T;
  double run = ex.A * carry_in + ex.B;
  for (int64_t l = hi - 1; l >= lo; --l) {
    const double val = (double)qd[l] - (double)di[l] + run;
    if (fp[l] == -INFINITY || (l == 0 && a.zero_first)) {
      a.df[bh * a.T + l] = 0.f;
      run = 0.0;
    } else {
      a.df[bh * a.T + l] = (float)(val * (double)sigmoid(-fp[l]));
      run = val;
    }
  }
  if (a.dm0 && c == 0) {
    double s = 0.0;
    for (int64_t q = threadIdx.x; q < a.Nc; q += kThreads) s += gm[q * 4 + 2];
    s = block_sum(s, s_red);
    if (threadIdx.x == 0) a.dm0[bh] = (float)s;
  }
}

// T = 0: the loss does not depend on the initial state.
__global__ void bwd_zero_init_kernel(float* dC0, float* dn0, float* dm0, int64_t nC, int64_t nn, int64_t nm) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x < nC) dC0[x] = 0.f;
  if (x < nn) dn0[x] = 0.f;
  if (x < nm) dm0[x] = 0.f;
}

template <typename TI, int K, int V>
hipError_t run_bwd(const BwdLaunch& b, const BwdArgs& a, hipStream_t s) {
  const int64_t nqt = (b.T + kTile - 1) / kTile;
  mark_before(b.marks, B_DQ, s);
  hipLaunchKernelGGL((bwd_dq_kernel<TI, K, V>), dim3((unsigned)(b.BH * nqt)), dim3(kBT), 0, s, a);
  mark_after(b.marks, B_DQ, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  mark_before(b.marks, B_STATE, s);
  const int64_t nloc = b.Nc - (b.dC0 ? 0 : 1);   // chunks whose share is needed
  if (nloc > 0) {
    hipLaunchKernelGGL((bwd_local_kernel<TI, K>), dim3((unsigned)(b.BH * (K / 64) * (V / 64) * nloc)),
                       dim3(kThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t nfold = b.BH * (V * K / 4 + K / 4);
  hipLaunchKernelGGL(bwd_fold_kernel, dim3((unsigned)((nfold + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
  mark_after(b.marks, B_STATE, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mark_before(b.marks, B_DKV, s);
  hipLaunchKernelGGL((bwd_dkv_kernel<TI, K, V>), dim3((unsigned)(b.BH * nqt)), dim3(kBT), 0, s, a);
  mark_after(b.marks, B_DKV, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  mark_before(b.marks, B_GATE, s);
  hipLaunchKernelGGL(bwd_gate_map_kernel, dim3((unsigned)(b.BH * b.Nc)), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(bwd_gate_kernel, dim3((unsigned)(b.BH * b.Nc)), dim3(kThreads), 0, s, a);
  mark_after(b.marks, B_GATE, s);
  return hipGetLastError();
}

template <typename TI, int K>
hipError_t run_bwd_v(const BwdLaunch& b, const BwdArgs& a, hipStream_t s) {
  switch (b.V) {
    case 64: return run_bwd<TI, K, 64>(b, a, s);
    case 128: return run_bwd<TI, K, 128>(b, a, s);
    case 256: return run_bwd<TI, K, 256>(b, a, s);
  }
  if constexpr (sizeof(TI) == 2) {
    if (b.V == 512) return run_bwd<TI, K, 512>(b, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool bwd_supported(int bf16, int64_t K, int64_t V) {
  if (bf16) return (K == 64 || K == 128 || K == 256) && (V == 64 || V == 128 || V == 256 || V == 512);
  return (K == 64 || K == 128) && (V == 64 || V == 128 || V == 256);
}

hipError_t launch_bwd(const BwdLaunch& b, const GateBuffers& gb, const ChunkStates& cs, const BwdBuffers& bb,
                      hipStream_t s) {
  if (b.T == 0) {
    if (!b.dC0) return hipSuccess;
    const int64_t nC = b.BH * b.V * b.K;
    hipLaunchKernelGGL(bwd_zero_init_kernel, dim3((unsigned)((nC + 255) / 256)), dim3(256), 0, s, b.dC0, b.dn0,
                       b.dm0, nC, b.BH * b.K, b.BH);
    return hipGetLastError();
  }
  BwdArgs a;
  a.q = b.q; a.k = b.k; a.v = b.v; a.o = b.o; a.h = b.h; a.dh = b.dh;
  a.f_pre = b.f_pre;
  a.dq = b.dq; a.dk = b.dk; a.dv = b.dv; a.dout = b.dout;
  a.di = b.di; a.df = b.df;
  a.gb = gb;
  a.Cs = cs.Cs; a.ns = cs.ns; a.ms = cs.ms;
  a.G = bb.G; a.dz = bb.dz; a.qdq = bb.qdq;
  a.Es = static_cast<float*>(bb.Es); a.es = bb.es; a.Ms = bb.Ms;
  a.L0 = bb.L0; a.L0e = bb.L0e;
  a.C0 = b.C0; a.n0 = b.n0; a.m0 = b.m0;
  a.dC0 = b.dC0; a.dn0 = b.dn0; a.dm0 = b.dm0;
  a.zero_first = b.C0 == nullptr;
  a.es_split = b.bf16 ? 1 : 0;
  a.T = b.T; a.Nc = b.Nc; a.V = b.V; a.K = b.K; a.BH = b.BH; a.L = b.L;
  if (b.bf16) {
    switch (b.K) {
      case 64: return run_bwd_v<__bf16, 64>(b, a, s);
      case 128: return run_bwd_v<__bf16, 128>(b, a, s);
      case 256: return run_bwd_v<__bf16, 256>(b, a, s);
    }
  } else {
    switch (b.K) {
      case 64: return run_bwd_v<float, 64>(b, a, s);
      case 128: return run_bwd_v<float, 128>(b, a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace mlstm_impl
