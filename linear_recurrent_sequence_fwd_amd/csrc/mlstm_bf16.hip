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
  __bf16* Cs;
  float* ns;
  double* ms;
  float *C_out, *n_out, *m_out;
  int64_t T, Nc, V, BH;
  int L;
};

// One workgroup per (head, 64 k x 64 v tile of C^T), four waves of 32 x 32.
// Walks the sequence in 64-token blocks: block b's K and V rows are loaded two
// blocks ahead into registers, written to LDS buffer b%2 (V scaled by the
// block's weights w_j), then contracted over tokens on MFMA. At each chunk
// start the carried tile is stored (bf16) and rescaled. The normaliser n is
// the same contraction with V replaced by ones; the waves with wv = 0 of the
// v-tile-0 workgroups compute it as one more 16-column MFMA tile, with each
// weight split into two bf16 terms (w = hi + lo) so that n keeps about 17
// bits: rows where n^T q nearly cancels would magnify a bf16-rounded n.
template <int K>
__global__ __launch_bounds__(kThreads) void state_kernel_bf16(StateArgsB a) {
  constexpr int KT = K / 64;
  constexpr int P = kTile + 16;     // LDS row pitch (elements)
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][kTile * P];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][kTile * P];
  __shared__ __attribute__((aligned(16))) __bf16 sw[2][2][kTile];   // [buffer][hi, lo][token]

  const int64_t BH = a.BH, V = a.V, T = a.T;
  const int64_t bh = blockIdx.x % BH;
  const int tile = (int)(blockIdx.x / BH);
  const int kt = tile % KT, vt = tile / KT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int wk = w & 1, wv = w >> 1;
  const bool n_tile = (vt == 0) && (wv == 0);

  f32x4 acc[2][2], nacc[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    nacc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
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

  const __bf16* kb = a.k + bh * T * K + 64 * kt;
  const __bf16* vbp = a.v + bh * T * V + 64 * vt;
  const double* ub = a.gb.u + bh * T;
  const int nsb = (int)((T + kTile - 1) / kTile);

  // prefetch ring: two blocks in flight, two 16-byte vectors of K and V per thread
  bf16x8 pk[2][2], pv[2][2];
  double pu[2][2];
  auto issue = [&](int sb, int slot) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int it = tid + kThreads * e;
      const int row = it >> 3, cg = it & 7;
      const int64_t t = (int64_t)sb * kTile + row;
      if (sb < nsb && t < T) {
        pk[slot][e] = *reinterpret_cast<const bf16x8*>(kb + t * K + 8 * cg);
        pv[slot][e] = *reinterpret_cast<const bf16x8*>(vbp + t * V + 8 * cg);
        pu[slot][e] = ub[t];
      } else {
        pk[slot][e] = zero8();
        pv[slot][e] = zero8();
        pu[slot][e] = -INFINITY;
      }
    }
  };

  double Rm = 0.0, m_next = 0.0;
  int Rc = -1;
  auto body = [&](int sb, auto slot_c) {
    constexpr int SLOT = decltype(slot_c)::value;
    const int64_t tb = (int64_t)sb * kTile;
    const int64_t c = tb / a.L;
    const int64_t t0 = c * a.L;
    const int jc = (int)(tb - t0);
    const int Lc = (int)min((int64_t)a.L, T - t0);
    if (jc == 0) {
      if (a.Cs) {
        __bf16* Cs = a.Cs + (bh * a.Nc + c) * V * K;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int kk = 64 * kt + 32 * wk + 16 * x + 4 * g;
#pragma unroll
          for (int y = 0; y < 2; ++y) {
            const int64_t vv = 64 * vt + 32 * wv + 16 * y + i;
            bf16x4 o;
            o[0] = (__bf16)acc[x][y][0]; o[1] = (__bf16)acc[x][y][1];
            o[2] = (__bf16)acc[x][y][2]; o[3] = (__bf16)acc[x][y][3];
            *reinterpret_cast<bf16x4*>(Cs + vv * K + kk) = o;
          }
          if (n_tile && i == 0) *reinterpret_cast<f32x4*>(a.ns + (bh * a.Nc + c) * K + kk) = nacc[x];
        }
        if (tile == 0 && tid == 0) a.ms[bh * a.Nc + c] = m_prev;
      }
      const double gc = a.gb.g[bh * a.Nc + c];
      const double Uc = a.gb.U[bh * a.Nc + c];
      Rc = a.gb.R[bh * a.Nc + c];
      Rm = fmax(Rc >= 0 ? -INFINITY : m_prev, Uc);
      if (Rm == -INFINITY) Rm = 0.0;
      const float decay = Rc >= 0 ? 0.f : expf((float)(m_prev - Rm));
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        nacc[x] *= decay;
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] *= decay;
      }
      m_next = gc + Rm;
    }
    const int buf = sb & 1;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int it = tid + kThreads * e;
      const int row = it >> 3, cg = it & 7;
      const float wf = (jc + row < Lc && jc + row >= Rc) ? expf((float)(pu[SLOT][e] - Rm)) : 0.f;
      *reinterpret_cast<bf16x8*>(&sK[buf][row * P + 8 * cg]) = pk[SLOT][e];
      *reinterpret_cast<bf16x8*>(&sV[buf][row * P + 8 * cg]) = scale8(pv[SLOT][e], wf);
      if (cg == 0) {
        const __bf16 hi = (__bf16)wf;
        sw[buf][0][row] = hi;
        sw[buf][1][row] = (__bf16)(wf - (float)hi);
      }
    }
    issue(sb + 2, SLOT);
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
        for (int y = 0; y < 2; ++y) acc[x][y] = mma(A[x], B[y], acc[x][y]);
      if (n_tile) {
        const bf16x8 Bh = *reinterpret_cast<const bf16x8*>(&sw[buf][0][kk + 8 * g]);
        const bf16x8 Bl = *reinterpret_cast<const bf16x8*>(&sw[buf][1][kk + 8 * g]);
#pragma unroll
        for (int x = 0; x < 2; ++x) nacc[x] = mma(A[x], Bl, mma(A[x], Bh, nacc[x]));
      }
    }
    if (jc + kTile >= Lc) m_prev = m_next;
  };

  issue(0, 0);
  issue(1, 1);
  for (int sb = 0; sb < nsb; sb += 2) {
    body(sb, std::integral_constant<int, 0>{});
    if (sb + 1 < nsb) body(sb + 1, std::integral_constant<int, 1>{});
  }

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
  const __bf16* Cs;  // chunk-start states [BH][Nc][V][K] (bf16), or null
  const float* ns;   // [BH][Nc][K]
  const double* ms;  // [BH][Nc]
  const float* C0f;  // initial state [BH][V][K] (float32) for the one-chunk form, or null
  const float* n0;
  const float* m0;
  int zero_first;    // chunk 0 starts from the zero state
  int64_t T, Nc, V, BH;
  int L;
};

constexpr int kOutThreads = 512;   // eight wave64

// One workgroup per (head, 64-row query tile, 128*NT value columns). Wave w
// owns all 64 rows of the columns [16 NT w, 16 NT (w+1)) of the block. The
// score tile S^T (keys x rows) is split as (w mod 4) -> 16 keys,
// (w / 4) -> 32 rows, with the keys' rows of K read straight from global
// memory; P goes through LDS, V is staged row-major and read transposed.
template <int K, int NT>
__global__ __launch_bounds__(kOutThreads) void out_kernel_bf16(OutArgsB a) {
  constexpr int VB = 128 * NT;
  constexpr int QP = K + 16;
  constexpr int VP = VB + 16;
  constexpr int PP = kTile + 16;
  constexpr int VVEC = kTile * VB / 8 / kOutThreads;   // 16-byte V vectors per thread
  __shared__ __attribute__((aligned(16))) __bf16 sQ[kTile * QP];
  __shared__ __attribute__((aligned(16))) __bf16 sV[kTile * VP];
  __shared__ __attribute__((aligned(16))) __bf16 sP[kTile * PP];
  __shared__ __attribute__((aligned(16))) double s_r[kTile], s_u[2][kTile];
  __shared__ __attribute__((aligned(16))) float s_sc[kTile], s_fl[kTile], s_dn[kTile], s_den[4][kTile];
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
  const int col0 = w * 16 * NT;                 // wave's first column within the block

  // carried state of this chunk: per-chunk states, or the caller's initial state
  const bool chunk_states = a.Cs != nullptr;
  const bool has_state = chunk_states ? (c > 0 || !a.zero_first) : (a.C0f != nullptr);
  const double m_prev = !has_state ? 0.0
                        : (chunk_states ? a.ms[bh * a.Nc + c] : (double)a.m0[bh]);

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
    s_u[0][tid] = tid < (int)min((int64_t)kTile, T - t0) ? a.gb.u[bh * T + t0 + tid] : -INFINITY;
  }
  {  // Q tile, row-major
    constexpr int QV = K / 8;
    const __bf16* qg = a.q + (bh * T + row0) * K;
    for (int it = tid; it < kTile * QV; it += kOutThreads) {
      const int row = it / QV, cv = it % QV;
      const bf16x8 x = row < nrows ? *reinterpret_cast<const bf16x8*>(qg + (int64_t)row * K + 8 * cv) : zero8();
      *reinterpret_cast<bf16x8*>(&sQ[row * QP + 8 * cv]) = x;
    }
  }
  // V tile of key block 0 in flight while the carried-state term runs
  bf16x8 pv[VVEC];
  auto issue_v = [&](int jb) {
    const int64_t key0 = t0 + (int64_t)jb * kTile;
    const int nkeys = (int)min((int64_t)kTile, T - key0);
    const __bf16* vg = a.v + (bh * T + key0) * V + vb * VB;
#pragma unroll
    for (int e = 0; e < VVEC; ++e) {
      const int it = tid + kOutThreads * e;
      const int row = it / (VB / 8), cv = it % (VB / 8);
      pv[e] = row < nkeys ? *reinterpret_cast<const bf16x8*>(vg + (int64_t)row * V + 8 * cv) : zero8();
    }
  };
  issue_v(0);
  __syncthreads();

  f32x4 acc[4][NT];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < NT; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (has_state) {
    {  // normaliser of the carried state: sc_t (q_t . n~)
      const int row = tid >> 3, part = tid & 7;
      const float* nst = chunk_states ? a.ns + (bh * a.Nc + c) * K : a.n0 + bh * K;
      float d = 0.f;
#pragma unroll
      for (int kk = part * (K / 8); kk < (part + 1) * (K / 8); ++kk) d += (float)sQ[row * QP + kk] * nst[kk];
      d += __shfl_xor(d, 1, 64);
      d += __shfl_xor(d, 2, 64);
      d += __shfl_xor(d, 4, 64);
      if (part == 0) s_dn[row] = d * s_sc[row];
    }
    const int64_t vrow0 = vb * VB + col0;
    if (chunk_states) {
      const __bf16* Cst = a.Cs + (bh * a.Nc + c) * V * K;
#pragma unroll 2
      for (int kk = 0; kk < K; kk += 32) {
        bf16x8 A[4], B[NT];
#pragma unroll
        for (int y = 0; y < NT; ++y)
          B[y] = *reinterpret_cast<const bf16x8*>(Cst + (vrow0 + 16 * y + i) * K + kk + 8 * g);
#pragma unroll
        for (int x = 0; x < 4; ++x) A[x] = *reinterpret_cast<const bf16x8*>(&sQ[(16 * x + i) * QP + kk + 8 * g]);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < NT; ++y) acc[x][y] = mma(A[x], B[y], acc[x][y]);
      }
    } else {
      const float* Cst = a.C0f + bh * V * K;
      for (int kk = 0; kk < K; kk += 32) {
        bf16x8 A[4], B[NT];
#pragma unroll
        for (int y = 0; y < NT; ++y) {
          const float* p = Cst + (vrow0 + 16 * y + i) * K + kk + 8 * g;
#pragma unroll
          for (int e = 0; e < 8; ++e) B[y][e] = (__bf16)p[e];
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) A[x] = *reinterpret_cast<const bf16x8*>(&sQ[(16 * x + i) * QP + kk + 8 * g]);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < NT; ++y) acc[x][y] = mma(A[x], B[y], acc[x][y]);
      }
    }
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

  // intra-chunk blocks: keys of block jb <= st
  const int jt = w & 3;            // this wave's 16 keys of the score tile
  const int tp = w >> 2;           // this wave's 32 rows (two 16-row tiles)
  float rsum[2] = {0.f, 0.f};
  for (int jb = 0; jb <= st; ++jb) {
    const int64_t key0 = t0 + (int64_t)jb * kTile;
    __syncthreads();   // previous block's P V done: sV, sP free
#pragma unroll
    for (int e = 0; e < VVEC; ++e) {
      const int it = tid + kOutThreads * e;
      const int row = it / (VB / 8), cv = it % (VB / 8);
      *reinterpret_cast<bf16x8*>(&sV[row * VP + 8 * cv]) = pv[e];
    }
    if (jb < st) {
      issue_v(jb + 1);
      if (tid < kTile) {
        const int64_t key1 = key0 + kTile;
        s_u[(jb + 1) & 1][tid] = key1 + tid < T ? a.gb.u[bh * T + key1 + tid] : -INFINITY;
      }
    }
    // S^T tile: 16 keys x 32 rows for this wave
    bf16x8 Kf[K / 32];
    {
      const int64_t key = key0 + 16 * jt + i;
      const __bf16* kg = a.k + (bh * T + key) * K + 8 * g;
#pragma unroll
      for (int s = 0; s < K / 32; ++s)
        Kf[s] = key < T ? *reinterpret_cast<const bf16x8*>(kg + 32 * s) : zero8();
    }
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < K / 32; ++s) {
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const bf16x8 B = *reinterpret_cast<const bf16x8*>(&sQ[(32 * tp + 16 * z + i) * QP + 32 * s + 8 * g]);
        sacc[z] = mma(Kf[s], B, sacc[z]);
      }
    }
#pragma unroll
    for (int z = 0; z < 2; ++z) {
      const int tl = 32 * tp + 16 * z + i;        // row of this lane
      const int tq = st * kTile + tl;             // its position in the chunk
      const double rr = s_r[tl];
      const int rs = s_rs[tl];
      bf16x4 pk;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jl = 16 * jt + 4 * g + r;
        const int jk = jb * kTile + jl;
        const bool keep = (tl < nrows) && (jk <= tq) && (jk >= rs);
        const float p = keep ? sacc[z][r] * expf((float)(s_u[jb & 1][jl] - rr)) : 0.f;
        psum += p;
        pk[r] = (__bf16)p;
      }
      *reinterpret_cast<bf16x4*>(&sP[tl * PP + 16 * jt + 4 * g]) = pk;
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      rsum[z] += psum;
    }
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
    for (int z = 0; z < 2; ++z) s_den[jt][32 * tp + 16 * z + i] = rsum[z];
  }
  __syncthreads();   // all P V done; s_den complete; sV free for the output tile

  // output gate: stage O through LDS, combine in registers, write h back through LDS
  const int64_t obase = (bh * T + row0) * V + vb * VB;
  for (int it = tid; it < kTile * VB / 8; it += kOutThreads) {
    const int row = it / (VB / 8), cv = it % (VB / 8);
    const bf16x8 x = row < nrows ? *reinterpret_cast<const bf16x8*>(a.o + obase + (int64_t)row * V + 8 * cv)
                                 : zero8();
    *reinterpret_cast<bf16x8*>(&sV[row * VP + 8 * cv]) = x;
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tl = 16 * x + 4 * g + r;
      const float den = s_den[0][tl] + s_den[1][tl] + s_den[2][tl] + s_den[3][tl] + s_dn[tl];
      const float inv = 1.f / fmaxf(fmaxf(fabsf(den), s_fl[tl]), FLT_MIN);
#pragma unroll
      for (int y = 0; y < NT; ++y) {
        __bf16* p = &sV[tl * VP + col0 + 16 * y + i];
        *p = (__bf16)(sigmoid((float)*p) * acc[x][y][r] * inv);
      }
    }
  __syncthreads();
  for (int it = tid; it < kTile * VB / 8; it += kOutThreads) {
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
  a.Cs = static_cast<__bf16*>(cs.Cs);
  a.ns = cs.ns; a.ms = cs.ms;
  a.C_out = f.C_out; a.n_out = f.n_out; a.m_out = f.m_out;
  a.T = f.T; a.Nc = f.Nc; a.V = f.V; a.BH = f.BH; a.L = f.L;
  const int64_t grid = f.BH * (K / 64) * (f.V / 64);
  mark_before(K_STATE, s);
  hipLaunchKernelGGL((state_kernel_bf16<K>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  mark_after(K_STATE, s);
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
  a.Cs = static_cast<const __bf16*>(cs.Cs);
  a.ns = cs.ns; a.ms = cs.ms;
  a.C0f = cs.Cs ? nullptr : f.C0;
  a.n0 = f.n0; a.m0 = f.m0;
  a.zero_first = f.C0 == nullptr;
  a.T = f.T; a.Nc = f.Nc; a.V = f.V; a.BH = f.BH; a.L = f.L;
  const int64_t nqt = (f.T + kTile - 1) / kTile;
  const int64_t grid = f.BH * nqt * (f.V / (128 * NT));
  mark_before(K_OUT, s);
  hipLaunchKernelGGL((out_kernel_bf16<K, NT>), dim3((unsigned)grid), dim3(kOutThreads), 0, s, a);
  mark_after(K_OUT, s);
  return hipGetLastError();
}

template <int K>
hipError_t run_out_b_nt(const FwdLaunch& f, const GateBuffers& gb, const ChunkStates& cs, hipStream_t s) {
  const int64_t nv = f.V / 128;
  if (nv % 4 == 0) return run_out_b<K, 4>(f, gb, cs, s);
  if (nv % 2 == 0) return run_out_b<K, 2>(f, gb, cs, s);
  return run_out_b<K, 1>(f, gb, cs, s);
}

}  // namespace

bool bf16_fast_path(const FwdLaunch& f) { return f.bf16 && f.V % 128 == 0; }

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
