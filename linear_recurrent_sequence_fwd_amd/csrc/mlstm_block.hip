// HIP kernels of the mLSTM block around the cell for gfx950: the residual
// block with pre-up-projection of the hu-po page "Introduction to xLSTM
// architecture" (section "Residual Block with Pre-Up Projection"), with the
// cell's projections and gates of the xLSTM guide (aifetchly), "mLSTM: Matrix
// Key-Value Memory and Covariance Updates", recurrent formulation.
//
// Per batch entry, x [T, D] and inner width E = 2 D = H d_v:
//   xn = LayerNorm(x)                          layernorm_kernel
//   [xm | z] = xn W_up^T + b_up                gemm_kernel ([T, 2E], bf16)
//   xc = swish(causal conv(xm)),               conv_gate_kernel (xc bf16; the
//   i~, f~ = xc w_{i,f}^T + b_{i,f}              gate projections on MFMA from
//                                                the rounded xc, float32)
//   q, k, v = per-head projections             gemm_kernel, batched over
//                                                (batch entry, head), written
//                                                straight into the cell's
//                                                [B, H, T, d] layout
//   h~ = ungated cell                          the fused chunkwise kernels
//   y = (GroupNorm(h~) + skip xc) sigmoid(z)   groupnorm_gate_kernel
//   out = x + y W_down^T + b_down              gemm_kernel with the residual
//                                                in its epilogue
//
// The projections are dense contractions and run on bf16 MFMA with float32
// accumulation; the rest reads and writes each activation once.

#include "mlstm_device.h"
#include "mlstm_launch.h"

namespace mlstm_impl {

namespace {

typedef __attribute__((address_space(3))) void lds_void_b_t;
constexpr unsigned kRsrcFlags = 0x00020000;

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void st8(__bf16* p, bf16x8 x) { *reinterpret_cast<bf16x8*>(p) = x; }

// ------------------------------------------------------------------ GEMM
//
// C = alpha A B^T + bias (+ R), A [M, K] and B [N, K] bf16 with k contiguous,
// float32 accumulation. One workgroup of eight waves per 256 x 256 output
// tile: wave (wm, wn) = (w & 3, w >> 2) owns rows 64 wm .. + 63 and columns
// 128 wn .. + 127, 4 x 8 accumulator tiles of 16 x 16. The contraction runs
// in stages of 64: both operand tiles of the next stage are copied into LDS
// with direct-to-LDS buffer loads while the current stage's 64 MFMAs per
// wave run. Loads past the last valid row return zero. An LDS row is the
// stage's 64 elements (eight 16-byte chunks) with chunk c of row r stored at
// position c ^ (r mod 8), so the rows of a fragment read fall on different
// banks (a padded pitch measured half of the LDS cycles in bank conflicts).
//
// Tiles are numbered XCD by XCD (workgroup b runs on XCD b mod 8), and
// within an XCD in groups of four tile rows with the row fastest, so the
// workgroups an XCD runs at one time share A row blocks and B column blocks
// in its L2.
constexpr int kGT = 512;
constexpr int kGB = 256;                     // tile rows and columns
constexpr int kGK = 64;                      // contraction depth per stage
constexpr int kGP = kGK;                     // LDS row pitch (elements): eight swizzled chunks
constexpr int kGLoads = kGB * kGK * 2 / 1024; // wave-wide loads per operand tile
constexpr int kGTileB = kGB * kGP * 2;       // bytes of one operand tile in LDS
static_assert(kGK == 64, "eight 16-byte chunks per row, swizzled by row mod 8");
// The output tile leaves through LDS in two halves of 128 rows, float32,
// row pitch 264 (66 16-byte chunks: the 16-byte writes of 16 rows fall on
// different banks), so that every store covers whole rows.
constexpr int kGCP = kGB + 8;
constexpr int kGSmem = 4 * kGTileB > (kGB / 2) * kGCP * 4 ? 4 * kGTileB : (kGB / 2) * kGCP * 4;

struct GemmDev {
  const __bf16 *A, *B;
  void* C;
  const float* bias;
  const __bf16* R;
  int64_t lda, ldb, ldc, ldr;
  int64_t sA1, sA2, sB1, sB2, sC1, sC2, sR1, sR2, sbias2;
  int M, N, K, nb2;
  int tiles_m, tiles_n, total;
  float alpha;
};

template <typename TO> __device__ __forceinline__ void store4v(TO* p, f32x4 v);
template <> __device__ __forceinline__ void store4v<__bf16>(__bf16* p, f32x4 v) {
  bf16x4 o;
  o[0] = (__bf16)v[0]; o[1] = (__bf16)v[1]; o[2] = (__bf16)v[2]; o[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = o;
}
template <> __device__ __forceinline__ void store4v<float>(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// TRANS: C is written transposed, element (m, n) at C + n ldc + m (no R).
template <typename TO, bool TRANS>
__global__ __launch_bounds__(kGT) void gemm_kernel(GemmDev a) {
  __shared__ __attribute__((aligned(16))) char smem[kGSmem];   // [stage buffer][A, B]; then the output halves
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = lane & 15, g = lane >> 4;
  const int wm = w & 3, wn = w >> 2;

  int pid = blockIdx.x;
  if (a.total % 8 == 0) pid = (int)(blockIdx.x % 8) * (a.total / 8) + (int)(blockIdx.x / 8);
  const int per = a.tiles_m * a.tiles_n;
  const int bat = pid / per;
  pid -= bat * per;
  constexpr int GM = 4;
  const int first_m = (pid / (GM * a.tiles_n)) * GM;
  const int gsize = min(a.tiles_m - first_m, GM);
  const int in_group = pid % (GM * a.tiles_n);
  const int tm = first_m + in_group % gsize, tn = in_group / gsize;
  const int b1 = bat / a.nb2, b2 = bat - b1 * a.nb2;
  const int m0 = tm * kGB, n0 = tn * kGB;
  const int rowsA = min(kGB, a.M - m0), rowsB = min(kGB, a.N - n0);

  const __bf16* Ab = a.A + b1 * a.sA1 + b2 * a.sA2 + (int64_t)m0 * a.lda;
  const __bf16* Bb = a.B + b1 * a.sB1 + b2 * a.sB2 + (int64_t)n0 * a.ldb;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(Ab), (short)0, (int)(rowsA * a.lda * 2), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(Bb), (short)0, (int)(rowsB * a.ldb * 2), kRsrcFlags);
  const int lda2 = (int)(a.lda * 2), ldb2 = (int)(a.ldb * 2);

  // wave-wide load n fills LDS bytes 1024 n .. + 1023 of a tile image: the
  // lane's position c = 64 n + lane is chunk c mod 8 of row c / 8 and takes
  // the row's chunk (c mod 8) ^ (row mod 8)
  auto load_stage = [&](int kt, int buf) {
    char* la = smem + buf * 2 * kGTileB;
    char* lb = la + kGTileB;
    const int kb = kt * kGK * 2;
    for (int n = w; n < kGLoads; n += kGT / 64) {
      const int c = 64 * n + lane, row = c >> 3, lc = (c & 7) ^ (row & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_b_t*)(la + 1024 * n), 16, row * lda2 + kb + 16 * lc, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_b_t*)(lb + 1024 * n), 16, row * ldb2 + kb + 16 * lc, 0, 0, 0);
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 8; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / kGK;
  load_stage(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();   // stage kt landed (every wave waited for its loads); the other buffer's readers are done
    if (kt + 1 < nk) load_stage(kt + 1, (kt + 1) & 1);
    const __bf16* sA = reinterpret_cast<const __bf16*>(smem + (kt & 1) * 2 * kGTileB);
    const __bf16* sB = reinterpret_cast<const __bf16*>(smem + (kt & 1) * 2 * kGTileB + kGTileB);
#pragma unroll
    for (int ks = 0; ks < kGK / 32; ++ks) {
      bf16x8 fa[4], fb[8];
#pragma unroll
      for (int x = 0; x < 4; ++x) fa[x] = ld8(sA + (64 * wm + 16 * x + i) * kGP + 8 * ((4 * ks + g) ^ (i & 7)));
#pragma unroll
      for (int y = 0; y < 8; ++y) fb[y] = ld8(sB + (128 * wn + 16 * y + i) * kGP + 8 * ((4 * ks + g) ^ (i & 7)));
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 8; ++y)
          acc[x][y] = TRANS ? mma(fa[x], fb[y], acc[x][y]) : mma(fb[y], fa[x], acc[x][y]);
    }
  }

  TO* C = static_cast<TO*>(a.C) + b1 * a.sC1 + b2 * a.sC2;
  const float* bias = a.bias ? a.bias + b2 * a.sbias2 : nullptr;
  if constexpr (!TRANS) {
    // register r of lane (i, g): row m0 + 64 wm + 16 x + i, column n0 + 128 wn + 16 y + 4 g + r.
    // alpha acc + bias goes to LDS (float32) by the waves holding the half's
    // rows; then wave w stores rows w, w + 8, ... of the half, each one
    // contiguous run of the row, adding the residual before the one rounding.
    const __bf16* R = a.R ? a.R + b1 * a.sR1 + b2 * a.sR2 : nullptr;
    float* sc = reinterpret_cast<float*>(smem);
    __syncthreads();   // every wave's last reads of the operand tiles are done
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if ((wm >> 1) == half) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int row = 64 * (wm & 1) + 16 * x + i;
#pragma unroll
          for (int y = 0; y < 8; ++y) {
            const int col = 128 * wn + 16 * y + 4 * g;
            f32x4 v = acc[x][y] * a.alpha;
            if (bias && n0 + col < a.N) v += *reinterpret_cast<const f32x4*>(bias + n0 + col);
            *reinterpret_cast<f32x4*>(sc + row * kGCP + col) = v;
          }
        }
      }
      __syncthreads();
      const int n = n0 + 4 * lane;
#pragma unroll 4
      for (int r = w; r < kGB / 2; r += kGT / 64) {
        const int m = m0 + (kGB / 2) * half + r;
        if (m < a.M && n < a.N) {
          f32x4 v = *reinterpret_cast<const f32x4*>(sc + r * kGCP + 4 * lane);
          if (R) {
            const bf16x4 rr = *reinterpret_cast<const bf16x4*>(R + (int64_t)m * a.ldr + n);
            v += f32x4{(float)rr[0], (float)rr[1], (float)rr[2], (float)rr[3]};
          }
          store4v<TO>(C + (int64_t)m * a.ldc + n, v);
        }
      }
      if (half == 0) __syncthreads();   // the second half overwrites the staging area
    }
  } else {
    // register r of lane (i, g): row m0 + 64 wm + 16 x + 4 g + r, column n0 + 128 wn + 16 y + i
#pragma unroll
    for (int y = 0; y < 8; ++y) {
      const int n = n0 + 128 * wn + 16 * y + i;
      if (n >= a.N) continue;
      const float bn = bias ? bias[n] : 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int m = m0 + 64 * wm + 16 * x + 4 * g;
        if (m >= a.M) continue;
        store4v<TO>(C + (int64_t)n * a.ldc + m, acc[x][y] * a.alpha + bn);
      }
    }
  }
}

// ------------------------------------------------------------------ layer norm

// One wave per row of D elements (D a multiple of 8, at most 512 CH): lane
// takes pieces lane, lane + 64, ... of eight; mean, then the mean squared
// deviation from registers; (x - mean) / sqrt(var + eps) w + b in bf16.
template <int CH>
__global__ __launch_bounds__(256) void layernorm_kernel(const __bf16* __restrict__ x, const float* __restrict__ w,
                                                        const float* __restrict__ b, __bf16* __restrict__ y,
                                                        int64_t rows, int D, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const __bf16* xr = x + row * D;
  float v[CH][8];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = 8 * (lane + 64 * c);
    bf16x8 p = {};
    if (col < D) p = ld8(xr + col);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[c][e] = (float)p[e];
      s += v[c][e];
    }
  }
  const float mean = wave_sum(s) / (float)D;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = 8 * (lane + 64 * c);
    if (col < D) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[c][e] - mean;
        q += d * d;
      }
    }
  }
  const float rstd = 1.f / sqrtf(wave_sum(q) / (float)D + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = 8 * (lane + 64 * c);
    if (col < D) {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + col), w1 = *reinterpret_cast<const f32x4*>(w + col + 4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(b + col), b1 = *reinterpret_cast<const f32x4*>(b + col + 4);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float we = e < 4 ? w0[e] : w1[e - 4], be = e < 4 ? b0[e] : b1[e - 4];
        o[e] = (__bf16)((v[c][e] - mean) * rstd * we + be);
      }
      st8(y + row * D + col, o);
    }
  }
}

// ------------------------------------------------------------------ conv + Swish + gates

struct ConvDev {
  const __bf16* xm;      // [B T] rows of pitch ldx (the first E columns of the up-projection)
  int64_t ldx;
  const float *cw, *cb;  // [E][KC] taps oldest first, [E]
  __bf16* xc;            // [B T][E]
  const __bf16 *wi, *wf; // [H][E] each
  const float *bi, *bf;  // [H]
  float *i_pre, *f_pre;  // [B H][T]
  int64_t T;
  int E, H, KC, ntb;     // ntb: 16-token blocks per batch entry
};

__device__ __forceinline__ float swish_f(float y) { return y * __builtin_amdgcn_rcpf(1.f + __expf(-y)); }

// One workgroup of eight waves per (batch entry, 16 tokens). Wave w takes
// the 512-channel blocks w, w + 8, ... of the inner width; lane l of a block
// owns channels 8 l .. 8 l + 7 and loads, once, its taps, its bias and rows
// t0 - KC + 1 .. t0 + 15 of those channels (each row load is 1 KiB contiguous
// over the wave), forms the 16 tokens' outputs (Swish, bf16), stores them and
// writes them into the wave's LDS tile [16 tokens][512] (16-byte chunk c of
// row r at position c ^ r, so neither the row writes nor the fragment reads
// below share banks). Read back as the A operand of the gate MFMAs (lane
// (i, g): token i, channels 8 g .. of a 32-deep step; B: the gate weights,
// rows 16 nb + i of [w_i; w_f]) they give the block's share of the gate
// preactivations; the waves' shares meet in LDS (each in its own wave's
// tile, which only that wave uses) and are added in a fixed order.
constexpr int kConvWaves = 8;
constexpr int kConvTok = 16;
constexpr int kConvCh = 512;      // channels per wave and block

template <int KC, int NB>
__global__ __launch_bounds__(64 * kConvWaves) void conv_gate_kernel(ConvDev a) {
  __shared__ __attribute__((aligned(16))) __bf16 s_tile[kConvWaves][kConvTok * kConvCh];
  static_assert(NB * 64 * 16 <= kConvTok * kConvCh * 2, "the gate shares fit in a wave's tile");
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.x / a.ntb;
  const int64_t t0 = (int64_t)(blockIdx.x % a.ntb) * kConvTok;
  const int nblk = (a.E + kConvCh - 1) / kConvCh;
  __bf16* tile = s_tile[w];
  f32x4 gacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) gacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int blk = w; blk < nblk; blk += kConvWaves) {
    const int c0 = blk * kConvCh;
    const int cc = c0 + 8 * lane;
    const bool cv = cc < a.E;
    // rows t0 - KC + 1 .. t0 + 15, all loads issued before any use
    constexpr int NR = kConvTok + KC - 1;
    bf16x8 xr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int64_t tt = t0 - (KC - 1) + r;
      xr[r] = bf16x8{};
      if (cv && tt >= 0 && tt < a.T) xr[r] = ld8(a.xm + (b * a.T + tt) * a.ldx + cc);
    }
    f32x4 cwv[2 * KC], cb[2];
#pragma unroll
    for (int q = 0; q < 2 * KC; ++q)
      cwv[q] = cv ? *reinterpret_cast<const f32x4*>(a.cw + (int64_t)cc * KC + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 2; ++q) cb[q] = cv ? *reinterpret_cast<const f32x4*>(a.cb + cc + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tk = 0; tk < kConvTok; ++tk) {
      const int64_t t = t0 + tk;
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float y = cb[e / 4][e % 4];
#pragma unroll
        for (int j = 0; j < KC; ++j) y = fmaf(cwv[(e * KC + j) / 4][(e * KC + j) % 4], (float)xr[tk + j][e], y);
        o[e] = t < a.T && cv ? (__bf16)swish_f(y) : (__bf16)0.f;
      }
      if (cv && t < a.T) st8(a.xc + (b * a.T + t) * a.E + cc, o);
      *reinterpret_cast<bf16x8*>(tile + tk * kConvCh + 8 * (lane ^ tk)) = o;
    }
    // the block's gate shares: 16 steps of 32 channels (the wave's own LDS
    // tile: its stores above are seen by its reads below)
#pragma unroll 4
    for (int ks = 0; ks < kConvCh / 32; ++ks) {
      const int kc = c0 + 32 * ks + 8 * g;
      const bf16x8 xa = *reinterpret_cast<const bf16x8*>(tile + i * kConvCh + 8 * ((4 * ks + g) ^ i));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int n = 16 * nb + i;
        bf16x8 wv = {};
        if (kc < a.E) {
          if (n < a.H) wv = ld8(a.wi + (int64_t)n * a.E + kc);
          else if (n < 2 * a.H) wv = ld8(a.wf + (int64_t)(n - a.H) * a.E + kc);
        }
        gacc[nb] = mma(xa, wv, gacc[nb]);   // D[token 4 g + r][gate 16 nb + i]
      }
    }
  }
  // the wave's gate shares, [gate block][lane], at the start of its tile
  auto part = [&](int v, int nb) { return reinterpret_cast<f32x4*>(s_tile[v]) + nb * 64 + lane; };
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) *part(w, nb) = gacc[nb];
  __syncthreads();
  // wave w finishes gate block w
  if (w < NB) {
    f32x4 sum = *part(0, w);
#pragma unroll
    for (int v = 1; v < kConvWaves; ++v) sum += *part(v, w);
    const int n = 16 * w + i;
    if (n < 2 * a.H) {
      const bool isf = n >= a.H;
      const int hh = isf ? n - a.H : n;
      const float bias = isf ? a.bf[hh] : a.bi[hh];
      float* dst = (isf ? a.f_pre : a.i_pre) + (b * a.H + hh) * a.T;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t tt = t0 + 4 * g + r;
        if (tt < a.T) dst[tt] = sum[r] + bias;
      }
    }
  }
}

// ------------------------------------------------------------------ group norm + skip + output gate

struct GnDev {
  const __bf16* h;        // cell output [B H][T][dv]
  const __bf16* xc;       // [B T][E]
  const __bf16* z;        // [B T] rows of pitch ldz (the second half of the up-projection)
  int64_t ldz;
  const float *gw, *gb, *skip;   // [E]
  __bf16* y;              // [B T][E]
  int64_t T, rows;        // rows = B T H
  int H, dv;
  float inv_dv;           // 1 / dv (exact for a power of two)
  float eps;
};

// One wave per (batch entry, token, head): the head's d_v outputs normalised
// over d_v, then (. w + b + skip xc) sigmoid(z). Grid (token, group of four
// heads, batch entry), a wave per head of the group, so that every index is
// a block or wave number (no division). A lane takes pieces of eight
// channels; every load of the wave (h, xc, z and the three parameter
// vectors) is issued before the first reduction.
template <int CH>
__global__ __launch_bounds__(256) void groupnorm_gate_kernel(GnDev a) {
  const int hh = (int)blockIdx.y * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (hh >= a.H) return;
  const int lane = threadIdx.x & 63;
  const int64_t b = blockIdx.z, t = blockIdx.x;
  const int64_t bt = b * a.T + t;
  const __bf16* hr = a.h + ((b * a.H + hh) * a.T + t) * a.dv;
  const int64_t E = (int64_t)a.H * a.dv;
  const int64_t col0 = (int64_t)hh * a.dv;
  bf16x8 hv[CH], xv[CH], zv[CH];
  f32x4 pw[CH][2], pb[CH][2], ps[CH][2];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = 8 * (lane + 64 * c);
    hv[c] = xv[c] = zv[c] = bf16x8{};
    if (col < a.dv) {
      const int64_t ec = col0 + col;
      hv[c] = ld8(hr + col);
      xv[c] = ld8(a.xc + bt * E + ec);
      zv[c] = ld8(a.z + bt * a.ldz + ec);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pw[c][u] = *reinterpret_cast<const f32x4*>(a.gw + ec + 4 * u);
        pb[c][u] = *reinterpret_cast<const f32x4*>(a.gb + ec + 4 * u);
        ps[c][u] = *reinterpret_cast<const f32x4*>(a.skip + ec + 4 * u);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)hv[c][e];
  const float mean = wave_sum(s) * a.inv_dv;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = 8 * (lane + 64 * c);
    if (col < a.dv) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = (float)hv[c][e] - mean;
        q += d * d;
      }
    }
  }
  const float rstd = 1.f / sqrtf(wave_sum(q) * a.inv_dv + a.eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int col = 8 * (lane + 64 * c);
    if (col < a.dv) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gw = pw[c][e / 4][e % 4], gb = pb[c][e / 4][e % 4], sk = ps[c][e / 4][e % 4];
        const float gn = ((float)hv[c][e] - mean) * rstd * gw + gb;
        const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-(float)zv[c][e]));
        o[e] = (__bf16)((gn + sk * (float)xv[c][e]) * sg);
      }
      st8(a.y + bt * E + col0 + col, o);
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_gemm(const GemmLaunch& g, hipStream_t s) {
  GemmDev a;
  a.A = static_cast<const __bf16*>(g.A);
  a.B = static_cast<const __bf16*>(g.B);
  a.C = g.C;
  a.bias = g.bias;
  a.R = static_cast<const __bf16*>(g.R);
  a.lda = g.lda; a.ldb = g.ldb; a.ldc = g.ldc; a.ldr = g.ldr;
  a.sA1 = g.sA1; a.sA2 = g.sA2; a.sB1 = g.sB1; a.sB2 = g.sB2;
  a.sC1 = g.sC1; a.sC2 = g.sC2; a.sR1 = g.sR1; a.sR2 = g.sR2; a.sbias2 = g.sbias2;
  a.M = (int)g.M; a.N = (int)g.N; a.K = (int)g.K; a.nb2 = (int)g.nb2;
  a.tiles_m = (int)((g.M + kGB - 1) / kGB);
  a.tiles_n = (int)((g.N + kGB - 1) / kGB);
  a.total = (int)(g.nb1 * g.nb2 * a.tiles_m * a.tiles_n);
  a.alpha = g.alpha;
  const dim3 grid((unsigned)a.total), block(kGT);
  if (g.c_fp32) {
    if (g.c_trans) hipLaunchKernelGGL((gemm_kernel<float, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<float, false>), grid, block, 0, s, a);
  } else {
    if (g.c_trans) hipLaunchKernelGGL((gemm_kernel<__bf16, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<__bf16, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

int gemm_tile() { return kGB; }

hipError_t launch_layernorm(const void* x, const float* w, const float* b, void* y, int64_t rows, int64_t D,
                            float eps, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const __bf16* xi = static_cast<const __bf16*>(x);
  __bf16* yo = static_cast<__bf16*>(y);
  const int d = (int)D;
  if (D <= 512) hipLaunchKernelGGL(layernorm_kernel<1>, grid, block, 0, s, xi, w, b, yo, rows, d, eps);
  else if (D <= 1024) hipLaunchKernelGGL(layernorm_kernel<2>, grid, block, 0, s, xi, w, b, yo, rows, d, eps);
  else if (D <= 2048) hipLaunchKernelGGL(layernorm_kernel<4>, grid, block, 0, s, xi, w, b, yo, rows, d, eps);
  else if (D <= 4096) hipLaunchKernelGGL(layernorm_kernel<8>, grid, block, 0, s, xi, w, b, yo, rows, d, eps);
  else hipLaunchKernelGGL(layernorm_kernel<16>, grid, block, 0, s, xi, w, b, yo, rows, d, eps);
  return hipGetLastError();
}

template <int KC>
hipError_t launch_conv_kc(const ConvDev& a, int nb, dim3 grid, dim3 block, hipStream_t s) {
  if (nb == 1) hipLaunchKernelGGL((conv_gate_kernel<KC, 1>), grid, block, 0, s, a);
  else if (nb == 2) hipLaunchKernelGGL((conv_gate_kernel<KC, 2>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((conv_gate_kernel<KC, 4>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_conv_gate(const ConvLaunch& c, hipStream_t s) {
  ConvDev a;
  a.xm = static_cast<const __bf16*>(c.xm);
  a.ldx = c.ldx;
  a.cw = c.cw; a.cb = c.cb;
  a.xc = static_cast<__bf16*>(c.xc);
  a.wi = static_cast<const __bf16*>(c.wi);
  a.wf = static_cast<const __bf16*>(c.wf);
  a.bi = c.bi; a.bf = c.bf;
  a.i_pre = c.i_pre; a.f_pre = c.f_pre;
  a.T = c.T; a.E = (int)c.E; a.H = (int)c.H; a.KC = (int)c.KC;
  a.ntb = (int)((c.T + kConvTok - 1) / kConvTok);
  const int nb = (int)((2 * c.H + 15) / 16);   // 16-gate blocks: 1, 2, or up to 4
  const dim3 grid((unsigned)(c.B * a.ntb)), block(64 * kConvWaves);
  switch (c.KC) {
    case 1: return launch_conv_kc<1>(a, nb, grid, block, s);
    case 2: return launch_conv_kc<2>(a, nb, grid, block, s);
    case 3: return launch_conv_kc<3>(a, nb, grid, block, s);
    case 4: return launch_conv_kc<4>(a, nb, grid, block, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_groupnorm_gate(const GnLaunch& g, hipStream_t s) {
  GnDev a;
  a.h = static_cast<const __bf16*>(g.h);
  a.xc = static_cast<const __bf16*>(g.xc);
  a.z = static_cast<const __bf16*>(g.z);
  a.ldz = g.ldz;
  a.gw = g.gw; a.gb = g.gb; a.skip = g.skip;
  a.y = static_cast<__bf16*>(g.y);
  a.T = g.T; a.rows = g.B * g.T * g.H;
  a.H = (int)g.H; a.dv = (int)g.dv;
  a.inv_dv = 1.f / (float)g.dv;
  a.eps = g.eps;
  const dim3 grid((unsigned)g.T, (unsigned)((g.H + 3) / 4), (unsigned)g.B), block(256);
  if (g.dv <= 512) hipLaunchKernelGGL(groupnorm_gate_kernel<1>, grid, block, 0, s, a);
  else if (g.dv <= 1024) hipLaunchKernelGGL(groupnorm_gate_kernel<2>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(groupnorm_gate_kernel<4>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace mlstm_impl
