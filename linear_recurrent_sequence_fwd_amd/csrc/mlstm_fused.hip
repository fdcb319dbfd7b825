// Fused chunkwise forward of the mLSTM cell for bfloat16 inputs on gfx950.
//
// Same mathematics as the two-pass kernels (xLSTM guide, aifetchly blog:
// recurrence of "mLSTM: Matrix Key-Value Memory and Covariance Updates",
// running max of "The Stabilizer State", decay matrix of "The Dual
// Formulation", chunking of "Exploit Chunkwise Hardware Kernels for Production
// Training"), organised so that the d_v x d_qk state never leaves the chip
// inside a chunk:
//
//   local_kernel       one workgroup per (head, 128 value columns, chunk but
//                      the last): the chunk's own end state from an empty
//                      state, C~loc = sum of decayed K^T diag(w) V over its
//                      tiles on MFMA; a loader wave streams the tiles into
//                      triple-buffered LDS with direct-to-LDS loads.
//   seg_combine_kernel folds the chunks' local end states in order into the
//                      start state of every chunk (elementwise, float32).
//                      With every chunk's local state and the fold started
//                      from the empty state, the two kernels also give a
//                      segment's summary (launch_summary). With at most
//                      seven local states of at least eight tiles each, the
//                      output kernel folds instead (below) and this kernel
//                      is not launched.
//   out_kernel_fused   one workgroup per (head, 128 value columns, chunk).
//                      Starts from its chunk's start state (read, or folded
//                      from the earlier chunks' local states in its prologue).
//                      Holds its 128 x d_qk slice of C~ (float32) in MFMA
//                      accumulators, split over its waves by halves of d_qk
//                      and 32-column groups, and walks the chunk in 64-token
//                      tiles. Per tile: Q K^T and Q C~^T on MFMA (C~ as bf16
//                      hi + lo; partial sums over each half of d_qk,
//                      exchanged through LDS), q . n~ on MFMA (n~ as three
//                      bf16 terms), the state update C~ <- a C~ + K^T diag(w) V
//                      on MFMA and the same for n~ (three MFMA columns
//                      carrying the weights as three bf16 terms), decay mask
//                      and stabiliser in registers, P V on MFMA, normaliser
//                      and output gate.
//                      q, k and v reach LDS by direct-to-LDS copies issued one
//                      tile ahead.
//
// Chunks are independent given their start states, so the sequence dimension
// supplies the parallelism that the few heads of a large layer lack.

#include "mlstm_device.h"

namespace mlstm_impl {

namespace {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

constexpr int kVB = 128;                     // value columns per workgroup
constexpr double kMaxDefer = 70.0;           // largest pending log decay kept out of the accumulators
constexpr float kLog2eF = 1.4426950408889634f;
constexpr int kWaitLgkm0 = 0xC07F;           // s_waitcnt lgkmcnt(0), other counters untouched
constexpr int kBufferDword3 = 0x00020000;    // buffer resource word 3 for raw (unformatted) access on gfx9
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// Transposed operand fragment from a row-major LDS tile X (row pitch P):
// lane l (i = l%16, g = l/16) receives X[kin0 + 8g + e][n0 + i], e = 0..7.
// ds_read_b64_tr_b16 hands lane i of each 16-lane group element (i mod 4) of
// the 8-byte rows addressed by lanes 4e + i/4 of that group.
__device__ __forceinline__ bf16x8 frag_tr(const __bf16* X, int P, int kin0, int n0, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const __bf16* p = X + (kin0 + 8 * g + (i >> 2)) * P + n0 + 4 * (i & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * P));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Transposed K fragment for 16-row tile kx = 2 s + h of the state C~^T, in
// the register layout where row 4 c + r of the tile holds k = 32 s + 8 c + 4 h
// + r: lane (g, i) receives X[kin0 + 8 g + e][32 s + 4 h + 8 (i / 4) + i % 4].
// With this layout the tiles 2 s and 2 s + 1 of a lane hold the eight
// consecutive k = 32 s + 8 g .. + 7, the order of a plain 16-byte row read of
// Q or K, so the state packs directly into operand fragments.
//
// The address is formed in two parts: lane_off_trk is the lane's element
// offset for tile kx0 (even) at kin0 = 0, passed through an empty asm
// statement so that the compiler keeps it whole; frag_trk_at adds the
// constant part of tile kx0 + x at kin0. Each read address is then one step
// from the array X, which lets the compiler tell which LDS array a read
// touches (and not wait for copies in flight into other arrays).
__device__ __forceinline__ int lane_off_trk(int P, int kx0, int lane) {
  const int i = lane & 15, g = lane >> 4;
  int off = (8 * g + (i >> 2)) * P + 16 * kx0 + 8 * (i & 3);
  asm("" : "+v"(off));
  return off;
}
__device__ __forceinline__ bf16x8 frag_trk_at(const __bf16* X, int off, int P, int kin0, int x) {
  const __bf16* p = X + off + (kin0 * P + 32 * (x >> 1) + 4 * (x & 1));
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * P));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Offset along d_qk of the four consecutive k that lane group g holds in
// register tile kx of the state (see frag_trk).
__device__ __forceinline__ int state_k0(int kx, int g) { return 32 * (kx >> 1) + 8 * g + 4 * (kx & 1); }

// threadIdx.x through an opaque register move. Lane-dependent LDS and global
// addresses derived from it are recomputed in the phase that uses them
// instead of being hoisted out of the tile loop, where the compiler keeps
// dozens of them live across the whole tile (and spills them: a spill reload
// waits for every load in flight, including the next tile's prefetch).
// The move waits four cycles first. An MFMA reads its accumulator input over
// its first cycles after issue; the compiler spaces its own writes into such a
// register from the MFMA, but not an inline-asm write, and the register
// allocator may give the move a register that an MFMA just issued reads as
// that input (its last use).
__device__ __forceinline__ int fresh_tid() {
  int t;
  asm volatile("s_nop 3\n\tv_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

// Cross-lane sums without the LDS permute path: x + x of lane l ^ 1 (DPP
// quad permutation), and the sum over the four 16-lane rows of lanes with
// the same l % 16 (row swaps by 16 and 32 lanes). Every lane of a pair adds
// the two values in the same order, so the results agree bit for bit.
__device__ __forceinline__ float sum_xor1(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}
// x summed over the four lanes of its quad (lanes l ^ 1, l ^ 2, l ^ 3), in
// the same order on every lane of the quad
__device__ __forceinline__ float sum_quad(float x) {
  const float y = sum_xor1(x);
  return y + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, y), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum_rows(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = __builtin_bit_cast(float, (unsigned)a[0]) + __builtin_bit_cast(float, (unsigned)a[1]);
  const unsigned v = __builtin_bit_cast(unsigned, y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __builtin_bit_cast(float, (unsigned)b[0]) + __builtin_bit_cast(float, (unsigned)b[1]);
}

// exp of a float64 argument in float32, accurate to a few ulp whatever the
// argument's size: the argument is scaled by log2(e) in float64 and split
// into an integer n and a fraction f in [0, 1); the hardware base-2
// exponential takes f and the result is scaled by 2^n. (Rounding the whole
// argument to float32 would lose about 6e-8 of its size, which at the
// deferred decays' arguments of up to about 100 is several ulp of the result
// and, in the rows whose denominators cancel strongly, far more of h.)
// Results below about 2^-200 are 0.
__device__ __forceinline__ float exp_f64arg(double x) {
  const double y = x * 1.4426950408889634;
  const double n = fmin(fmax(floor(y), -200.0), 200.0);
  return ldexpf(__builtin_amdgcn_exp2f((float)(y - n)), (int)n);
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
  const unsigned lo = __builtin_amdgcn_readlane((unsigned)u, lane);
  const unsigned hi = __builtin_amdgcn_readlane((unsigned)(u >> 32), lane);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

// Workgroup barrier for LDS traffic only: waits for the wave's own LDS
// operations but, unlike __syncthreads, not for its global memory
// operations or direct-to-LDS loads in flight (their consumers wait for
// them explicitly). The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Raw buffer resource over `bytes` bytes from p: stores beyond the range are
// dropped and loads beyond it return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kBufferDword3);
}

struct Lanes {
  int tid, lane, i, g;   // thread, lane, lane % 16, lane / 16
};
__device__ __forceinline__ Lanes fresh_lanes() {
  const int t = fresh_tid();
  return Lanes{t, t & 63, t & 15, (t & 63) >> 4};
}

__device__ __forceinline__ bf16x8 pack_bf16(const f32x4& a, const f32x4& b) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)a[e];
    r[4 + e] = (__bf16)b[e];
  }
  return r;
}

// The bfloat16 rounding of what pack_bf16(a, b) leaves out: pack_bf16(a, b)
// + pack_bf16_rest(a, b, pack_bf16(a, b)) carries about 16 bits of a and b.
// x - float(h) is exact in float32 (h is x rounded to 8 significant bits), so
// it is formed in one bf16 dot product: (h0, h1) . (-1, 0) + x0 and
// (h0, h1) . (0, -1) + x1 take the pair of rounded values as they lie in one
// register, without widening them first.
// The multipliers are bit patterns in registers (element 0 = the low 16
// bits; bf16 -1 is 0xBF80), not inline constants, whose placement in a packed
// bf16 operand the encoding leaves open.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
// (x0 - float(h0), x1 - float(h1)) for the pair h = (h0, h1) of bf16 roundings
// of (x0, x1), both exact, in two bf16 dot products
__device__ __forceinline__ void minus_rounded(const bf16x2v& h, float& x0, float& x1) {
  unsigned u0 = 0x0000BF80u, u1 = 0xBF800000u;
  asm("" : "+v"(u0), "+v"(u1));
  x0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2v, u0), x0, false);
  x1 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2v, u1), x1, false);
}
__device__ __forceinline__ bf16x8 pack_bf16_rest(const f32x4& a, const f32x4& b, const bf16x8& hi) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; e += 2) {
    float a0 = a[e], a1 = a[e + 1], b0 = b[e], b1 = b[e + 1];
    minus_rounded(bf16x2v{hi[e], hi[e + 1]}, a0, a1);
    minus_rounded(bf16x2v{hi[4 + e], hi[5 + e]}, b0, b1);
    r[e] = (__bf16)a0;
    r[e + 1] = (__bf16)a1;
    r[4 + e] = (__bf16)b0;
    r[5 + e] = (__bf16)b1;
  }
  return r;
}
// x0, x1 as three bfloat16 terms each, hi + lo + lo2 (about 24 bits), as pairs
__device__ __forceinline__ void split3(float x0, float x1, bf16x2v& hi, bf16x2v& lo, bf16x2v& lo2) {
  hi = bf16x2v{(__bf16)x0, (__bf16)x1};
  minus_rounded(hi, x0, x1);
  lo = bf16x2v{(__bf16)x0, (__bf16)x1};
  minus_rounded(lo, x0, x1);
  lo2 = bf16x2v{(__bf16)x0, (__bf16)x1};
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
  int fold_here;             // 1: the output kernel folds the chunk start states itself (no fold kernel)
  float o_bias;              // 0, or -inf with o null: no output gate (sigmoid(o~) = 1)
};

constexpr int kOutWaves = 8;   // output kernel: two halves of d_qk x four 32-column groups, two waves per SIMD
constexpr int kFoldHere = 7;   // most local states an output workgroup folds itself
constexpr int kFoldMinTiles = 8;   // fewest 64-token tiles per chunk for that fold

// A 64-row bf16 tile (rows of E elements at a stride of RS elements in global
// memory; rows past `last` repeat row `last`) is copied into LDS rows of pitch
// P elements with direct-to-LDS buffer loads. Load n fills the 64 consecutive
// 16-byte chunks 64 n .. 64 n + 63 of the padded LDS image (chunk c lies in
// row c / (P / 8); padding chunks repeat the row's last data chunk), so the
// image takes P / 8 loads, issued in rounds: in round r wave w issues load
// min(NW r + w, P / 8 - 1) (a wave past the last load repeats it, the same
// bytes to the same place, so that every wave issues one load per round).
// The data are in LDS once the issuing wave's load counter has drained.
template <int P, int NW>
struct DmaTile {
  static constexpr int kLoads = P / 8;
  static constexpr int kRounds = (kLoads + NW - 1) / NW;
  static __device__ __forceinline__ int load(int w, int r) { return min(NW * r + w, kLoads - 1); }
};
// Byte offset in the tile of the chunk that lane `lane` of load n copies.
template <int E, int P>
__device__ __forceinline__ unsigned dma_src_off(int n, unsigned lane, unsigned rs, unsigned last) {
  constexpr unsigned CPR = P / 8;
  const unsigned c = 64u * (unsigned)n + lane;
  const unsigned row = min(c / CPR, last), ch = min(c % CPR, (unsigned)(E / 8 - 1));
  return 2u * (row * rs + 8u * ch);
}

// Two 8-byte values per lane exchanged between the lanes l and l ^ 16 of a
// pair of 16-lane rows: afterwards a lane in an even row holds (its own x1,
// its partner's x1) and a lane in an odd row (its partner's x0, its own x0).
// Applied again it undoes itself on the same layout, so it serves both to
// form 16-byte row pieces for stores and to split 16-byte loads.
__device__ __forceinline__ void swap_rows16(bf16x4& x1, bf16x4& x0) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  u32x2 a = __builtin_bit_cast(u32x2, x1), b = __builtin_bit_cast(u32x2, x0);
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const auto r = __builtin_amdgcn_permlane16_swap(a[d], b[d], false, false);
    a[d] = r[0];
    b[d] = r[1];
  }
  x1 = __builtin_bit_cast(bf16x4, a);
  x0 = __builtin_bit_cast(bf16x4, b);
}

// LDS of the output kernel. Q, K and V arrive by direct-to-LDS copies that
// the compute waves issue in the second half of the previous tile, each once
// the tile's reads of its single buffer are over (Q and V after the exchange
// barrier, K after the one that ends the state update); O is read into
// registers and H written from registers. Q, K and V are arrays of their own
// so that reads of one need not wait for copies in flight into another. The tile's per-key and per-row data and the
// normaliser operand are double-buffered: waves 0-3 prepare tile tau + 1's
// copy at the end of tile tau. The exchange area carries the partial sums that
// the two waves of a value-column group (one per half of d_qk) hand each other.
template <int K>
struct OutLds {
  static constexpr int QP = K + 16;       // sQ row pitch: 8 dwords mod 64 banks, conflict-free 16-byte row reads
  static constexpr int KP = K + 32;       // sK row pitch: 16 dwords mod 64 banks, conflict-free for frag_trk
  static constexpr int VP = kVB + 8;      // sV row pitch (transposed reads)
  static constexpr int PP = kTile + 8;    // sP row pitch
  // row pitch of the n~ terms: four rows read at once by 16-byte reads, which
  // at a pitch of 512 bytes all fall on the same banks (measured 4x the
  // cycles of 544 bytes)
  static constexpr int NTP = K + 16;
  // row pitch of the weight terms (the same four-row read; a 160-byte pitch
  // measured the whole kernel 14% slower, so it stays unpadded)
  static constexpr int WBP = kTile;
  static constexpr int qBytes = kTile * QP * 2;
  static constexpr int kBytes = kTile * KP * 2;
  static constexpr int vBytes = kTile * VP * 2;
  static constexpr int kXchg = 6;                    // f32x4 registers a wave hands its partner
  // sQ, sK and sV are arrays of their own; the rest shares one array at these offsets
  static constexpr int oP = 0;
  // double-buffered tile data, [2] of:
  static constexpr int nbBytes = 4 * NTP * 2;        // bf16 [4][NTP]: n~ at the tile's start as hi, lo, lo2, zero
  static constexpr int wBytes = kTile * 4;           // float [64] key weights
  static constexpr int wbBytes = 4 * WBP * 2;        // bf16 [4][WBP]: weights hi, lo, lo2, zero
  static constexpr int rowBytes = 5 * kTile * 4;     // r2, sc, fl, u2 (float), rs (int), [64] each
  static constexpr int infoBytes = 16;               // tile info: rescale flag (int), factor (float)
  static constexpr int bufBytes = nbBytes + wBytes + wbBytes + rowBytes + infoBytes;
  static constexpr int oBuf = oP + kTile * PP * 2;
  static constexpr int oDnm = oBuf + 2 * bufBytes;   // float [64] denominator max(|n~^T q|, floor) of each row
  static constexpr int oDen = oDnm + kTile * 4;      // float [4][64] row sums of P per key group
  static constexpr int oDn = oDen + 4 * kTile * 4;   // float [2][64] q . n~ of each row over each half of d_qk
  static constexpr int oX = oDn + 2 * kTile * 4;             // f32x4 [8 waves][kXchg][64 lanes]
  static constexpr int oFin = oX + kOutWaves * kXchg * 64 * 16;   // double [2]: final m, logD
  static constexpr int restBytes = oFin + 16;
  static_assert(qBytes + kBytes + vBytes + restBytes <= 160 * 1024, "fits the LDS of a CU");
};

// Wave w = 4 kh + cg owns value columns [32 cg, 32 cg + 32) of the
// workgroup's 128 and keeps C~^T[k][v] for the half kh of d_qk, k in
// [K/2 kh, K/2 kh + K/2), in registers: register r of Ct[x][cv] in lane
// (g, i) is k = K/2 kh + state_k0(x, g) + r, v = 32 cg + 16 cv + i. Waves w
// and w + 4 (same columns, the two halves of d_qk) form a pair.
//
// Q C~^T and Q K^T are contractions over d_qk: each wave forms them over its
// half for all 64 rows (value columns and keys as MFMA rows, H and S
// transposed), hands the partial sums of the partner's rows (rows 32 (1 - kh)
// .. + 31) to the partner through LDS and adds the partner's for its own rows
// 32 kh .. + 31. Afterwards wave (kh, cg) holds H^T for its 32 columns and its
// 32 rows, and S^T for keys [16 cg, +16) and its rows (register group z is
// rows 16 zg(z) .. + 15, zg(z) = (z + 2 kh) & 3: groups 0 and 1 are the
// wave's own rows). The normaliser n~ is carried as three MFMA columns in
// Nacc, for KXN 16-row tiles of the wave's half of d_qk (lane i = 0: the sum
// weighted by the bf16 high parts of the key weights, i = 1 and 2: by the two
// further bf16 terms of the weights, i = 3: zero; summed over the quad). Rows
// whose denominators cancel strongly need n~ to float32 accuracy, which two
// bf16 terms of the weights do not give.
//
// The tiles' decays are not applied to the accumulators one by one: the
// registers hold X with C~ = exp(logD) X, n~ = exp(logD) Xn, new keys enter
// with weight exp(u_j - Rm - logD_next), and X is rescaled only when logD
// would fall below -kMaxDefer (or on a zero decay); the tile data carry a
// flag for that, one scalar branch per tile.
template <int K>
__device__ __forceinline__ void out_body(const SegArgs& a, char* lq, char* lk, char* lv, char* smem) {
  using L = OutLds<K>;
  constexpr int QP = L::QP, KP = L::KP, VP = L::VP, PP = L::PP, NTP = L::NTP, WBP = L::WBP;
  constexpr int KH = K / 2;                                    // d_qk rows per half
  constexpr int KSH = KH / 32;                                 // 32-deep steps per half
  constexpr int KXH = KH / 16;                                 // 16-row state tiles per half
  constexpr int NW = kOutWaves;
  constexpr int KXN = KXH >= 4 ? KXH / 4 : 1;                  // normaliser tiles per wave
  static_assert(KSH >= 1 && KXH % 2 == 0, "d_qk halves of whole 32-deep steps");
  __bf16* sQ = reinterpret_cast<__bf16*>(lq);
  const __bf16* sK = reinterpret_cast<const __bf16*>(lk);
  __bf16* sV = reinterpret_cast<__bf16*>(lv);
  __bf16* sP = reinterpret_cast<__bf16*>(smem + L::oP);
  float* s_dnm = reinterpret_cast<float*>(smem + L::oDnm);
  float* s_den = reinterpret_cast<float*>(smem + L::oDen);
  float* s_dn = reinterpret_cast<float*>(smem + L::oDn);
  f32x4* s_x = reinterpret_cast<f32x4*>(smem + L::oX);
  double* s_fin = reinterpret_cast<double*>(smem + L::oFin);
  // views of one half of the double-buffered tile data
  struct TileBuf {
    __bf16* nt;
    float* w;
    __bf16* wb;
    float *r2, *sc, *fl, *u2;
    int* rs;
    int* info;
  };
  auto tile_buf = [&](int b) {
    char* base = smem + L::oBuf + b * L::bufBytes;
    TileBuf t;
    t.nt = reinterpret_cast<__bf16*>(base);
    t.w = reinterpret_cast<float*>(base + L::nbBytes);
    t.wb = reinterpret_cast<__bf16*>(base + L::nbBytes + L::wBytes);
    float* row = reinterpret_cast<float*>(base + L::nbBytes + L::wBytes + L::wbBytes);
    t.r2 = row;
    t.sc = row + kTile;
    t.fl = row + 2 * kTile;
    t.u2 = row + 3 * kTile;
    t.rs = reinterpret_cast<int*>(row + 4 * kTile);
    t.info = reinterpret_cast<int*>(row + 5 * kTile);
    return t;
  };

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
  const int cg = w & 3, kh = w >> 2;
  const int kg = cg;                                           // key block of the wave's S^T
  const int64_t vcol0 = (int64_t)vb * kVB;
  const int64_t nseg1 = a.S - 1;
  auto zg = [&](int z) { return (z + 2 * kh) & 3; };
  // global 16-row tile of d_qk of the wave's local tile x
  auto kxg = [&](int x) { return KXH * kh + x; };

  // ---------------- carried state
  f32x4 Ct[KXH][2];
  f32x4 Nacc[KXN];
  double m_start;
  bool has_state;
  const float* ninit = nullptr;
  const float* Cinit = nullptr;
  if (seg == 0) {
    Cinit = a.C0 ? a.C0 + bh * V * K : nullptr;
    ninit = a.C0 ? a.n0 + bh * K : nullptr;
    m_start = a.C0 ? (double)a.m0[bh] : 0.0;
    has_state = a.C0 != nullptr;
  } else if (!a.fold_here) {
    const int64_t sidx = bh * nseg1 + seg - 1;
    Cinit = a.Cseg + sidx * V * K;
    ninit = a.nseg + sidx * K;
    m_start = a.mstart[sidx];
    has_state = true;
  } else {
    has_state = true;
  }
  // the wave's share of a [V][K] state and of its n~ [K]
  auto state_at = [&](const float* C, int x, int cv) {
    return *reinterpret_cast<const f32x4*>(C + (vcol0 + 32 * cg + 16 * cv + i) * K + state_k0(kxg(x), g));
  };
#pragma unroll
  for (int x = 0; x < KXH; ++x)
#pragma unroll
    for (int cv = 0; cv < 2; ++cv) Ct[x][cv] = Cinit ? state_at(Cinit, x, cv) : f32x4{0.f, 0.f, 0.f, 0.f};
  // normaliser tiles of the wave: local tiles KXN cg .. + KXN - 1 of its half
  auto nx = [&](int x) { return KXN * cg + x; };
  auto n_live = [&](int x) { return nx(x) < KXH; };
#pragma unroll
  for (int x = 0; x < KXN; ++x)
    Nacc[x] = (ninit && i == 0 && n_live(x)) ? *reinterpret_cast<const f32x4*>(ninit + state_k0(kxg(nx(x)), g))
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
  if (seg > 0 && a.fold_here) {
    // The start state of chunk seg folded here from the local end states of
    // chunks 0..seg-1 (and the initial state), instead of by the fold
    // kernel. The stabiliser takes the fold's own float64 chain, m' =
    // max(m + G_s, mloc_s) (0 for an all-zero state); unrolled, local state s
    // enters with exp(mloc_s + G_{s+1} + ... + G_{seg-1} - m) and the initial
    // state with exp(m0 + G_0 + ... + G_{seg-1} - m), factors of at most 1.
    const int64_t sbase = bh * nseg1;
    double m = a.C0 ? (double)a.m0[bh] : 0.0;
    for (int s = 0; s < seg; ++s) {
      const double G = a.Gseg[sbase + s];
      const double mn = fmax(G == -INFINITY ? -INFINITY : m + G, a.mloc[sbase + s]);
      m = mn == -INFINITY ? 0.0 : mn;
    }
    m_start = m;
    double tail = 0.0;   // sum of G over the chunks after s
    for (int s = seg - 1; s >= 0; --s) {
      const double ml = a.mloc[sbase + s];
      const float c = (ml == -INFINITY || tail == -INFINITY) ? 0.f : exp_f64arg(ml + tail - m);
      if (c != 0.f) {
        const float* Cl = a.Cseg + (sbase + s) * V * K;
        f32x4 y[KXH][2];
#pragma unroll
        for (int x = 0; x < KXH; ++x)
#pragma unroll
          for (int cv = 0; cv < 2; ++cv) y[x][cv] = state_at(Cl, x, cv);
#pragma unroll
        for (int x = 0; x < KXH; ++x)
#pragma unroll
          for (int cv = 0; cv < 2; ++cv) Ct[x][cv] += c * y[x][cv];
        const float* nl = a.nseg + (sbase + s) * K;
#pragma unroll
        for (int x = 0; x < KXN; ++x)
          if (i == 0 && n_live(x)) Nacc[x] += c * *reinterpret_cast<const f32x4*>(nl + state_k0(kxg(nx(x)), g));
      }
      tail += a.Gseg[sbase + s];
    }
    if (a.C0 && tail != -INFINITY && a.m0[bh] != -INFINITY) {
      const float c = exp_f64arg((double)a.m0[bh] + tail - m);
      const float* C0 = a.C0 + bh * V * K;
#pragma unroll
      for (int x = 0; x < KXH; ++x)
#pragma unroll
        for (int cv = 0; cv < 2; ++cv) Ct[x][cv] += c * state_at(C0, x, cv);
      const float* n0 = a.n0 + bh * K;
#pragma unroll
      for (int x = 0; x < KXN; ++x)
        if (i == 0 && n_live(x)) Nacc[x] += c * *reinterpret_cast<const f32x4*>(n0 + state_k0(kxg(nx(x)), g));
    }
  }
  // zero rows of the weight and normaliser operands, both halves
  for (int b = 0; b < 2; ++b) {
    const TileBuf tb = tile_buf(b);
    if (tid < kTile) tb.wb[3 * WBP + tid] = (__bf16)0.f;
    for (int k = tid; k < K; k += 64 * kOutWaves) tb.nt[3 * NTP + k] = (__bf16)0.f;
  }

  // ---------------- copies of the next tile. Rows past the sequence end are
  // clamped into the tile (their results are masked), so no load depends on
  // a per-lane branch.
  auto last_row = [&](int64_t tau) { return (unsigned)(min((int64_t)kTile, T - tau * kTile) - 1); };
  using DQ = DmaTile<QP, NW>;
  using DK = DmaTile<KP, NW>;
  using DV = DmaTile<VP, NW>;
  constexpr int RQ = DQ::kRounds, RK = DK::kRounds, RV = DV::kRounds;
  // five issue slots each: Q and V after the barrier that ends their reads, K after the one that ends its reads
  static_assert(RK <= 5 && RQ <= 5 && RV <= 5, "copy rounds fit their slots");
  // Per-lane source offsets of this wave's copy rounds for a full tile,
  // computed once; a ragged last tile recomputes them with its rows clamped.
  unsigned offQ[RQ], offK[RK], offV[RV];
#pragma unroll
  for (int r = 0; r < RQ; ++r) offQ[r] = dma_src_off<K, QP>(DQ::load(w, r), (unsigned)lane, (unsigned)K, kTile - 1);
#pragma unroll
  for (int r = 0; r < RK; ++r) offK[r] = dma_src_off<K, KP>(DK::load(w, r), (unsigned)lane, (unsigned)K, kTile - 1);
#pragma unroll
  for (int r = 0; r < RV; ++r) offV[r] = dma_src_off<kVB, VP>(DV::load(w, r), (unsigned)lane, (unsigned)V, kTile - 1);
  auto dma_issue = [&](const __amdgpu_buffer_rsrc_t& src, unsigned off, char* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)dst, 16, (int)off, 0, 0, 0);
  };
  auto dma_q = [&](int64_t tau, int r) {
    const unsigned last = last_row(tau);
    const auto src = buffer_rsrc(a.q + (bh * T + tau * kTile) * K, (last + 1) * (unsigned)K * 2u);
    const int n = DQ::load(w, r);
    char* dst = lq + 1024 * n;
    if (last == kTile - 1) dma_issue(src, offQ[r], dst);
    else dma_issue(src, dma_src_off<K, QP>(n, (unsigned)fresh_lanes().lane, (unsigned)K, last), dst);
  };
  auto dma_k = [&](int64_t tau, int r) {
    const unsigned last = last_row(tau);
    const auto src = buffer_rsrc(a.k + (bh * T + tau * kTile) * K, (last + 1) * (unsigned)K * 2u);
    const int n = DK::load(w, r);
    char* dst = lk + 1024 * n;
    if (last == kTile - 1) dma_issue(src, offK[r], dst);
    else dma_issue(src, dma_src_off<K, KP>(n, (unsigned)fresh_lanes().lane, (unsigned)K, last), dst);
  };
  auto dma_v = [&](int64_t tau, int r) {
    const unsigned last = last_row(tau);
    const auto src = buffer_rsrc(a.v + (bh * T + tau * kTile) * V + vcol0, (last * (unsigned)V + kVB) * 2u);
    const int n = DV::load(w, r);
    char* dst = lv + 1024 * n;
    if (last == kTile - 1) dma_issue(src, offV[r], dst);
    else dma_issue(src, dma_src_off<kVB, VP>(n, (unsigned)fresh_lanes().lane, (unsigned)V, last), dst);
  };
  // O straight into the registers of the epilogue. For column half cv the
  // pair po[cv][1], po[cv][0] holds, once split by swap_rows16, columns
  // 32 cg + 16 cv + 4 g .. + 3 of rows 16 zg(1) + i and 16 zg(0) + i; it is
  // loaded as one 16-byte row piece per lane: a lane in an even 16-lane row
  // takes row zg(1), one in an odd row takes row zg(0), columns
  // 32 cg + 16 cv + 4 (g & 2) .. + 7. The same per-lane offsets address the
  // H stores. Both go through a buffer resource over the tile's valid rows:
  // loads past it return zero (their rows' results are never stored) and
  // stores past it are dropped.
  bf16x4 po[2][2];
  unsigned offO[2];
  // The epilogue of tile tau (normaliser, output gate, H stores) runs in tile
  // tau + 1: its arithmetic beside the first matrix phase, its two stores
  // once that tile's loaded registers are taken. It needs the tile's H^T
  // accumulators of the wave's own rows (eacc), its O (epo) and the row
  // denominators s_dnm, which are rewritten only after the exchange barrier.
  f32x4 eacc[2][2];
  bf16x4 epo[2][2];
  bf16x8 hv[2];
#pragma unroll
  for (int cv = 0; cv < 2; ++cv) {
    const unsigned t = 16 * zg((g & 1) ? 0 : 1) + i;
    offO[cv] = 2u * (t * (unsigned)V + 32 * cg + 16 * cv + 4 * (g & 2));
  }
  auto tile_rsrc_vo = [&](const __bf16* base, int64_t tau) {
    return buffer_rsrc(base + (bh * T + tau * kTile) * V + vcol0, (last_row(tau) * (unsigned)V + kVB) * 2u);
  };
  // Without an output gate (o null) the resource covers no bytes: the loads
  // return zero and touch no memory, and the exponent bias of -inf makes the
  // gate exactly one.
  auto load_o = [&](int64_t tau, int cv) {
    const __amdgpu_buffer_rsrc_t orsrc = a.o ? tile_rsrc_vo(a.o, tau) : buffer_rsrc(a.h, 0u);
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(orsrc, (int)offO[cv], 0, 0);
    const bf16x8 y = __builtin_bit_cast(bf16x8, x);
    po[cv][1] = __builtin_shufflevector(y, y, 0, 1, 2, 3);
    po[cv][0] = __builtin_shufflevector(y, y, 4, 5, 6, 7);
  };
  // gate data of the next tile, for the tile preparation of waves 0-3
  double r_u = 0.0, r_mp = 0.0, r_b = 0.0;
  int r_rs = -1;
  double t_g = 0.0, t_U = 0.0;
  int t_R = -1;
  auto load_gate = [&](int64_t tau) {
    const unsigned j = min((unsigned)fresh_lanes().lane, last_row(tau));
    const int64_t tok0 = bh * T + tau * kTile;
    r_u = (a.gb.u + tok0)[j];
    r_mp = (a.gb.mp + tok0)[j];
    r_b = (a.gb.b + tok0)[j];
    r_rs = (a.gb.rs + tok0)[j];
    t_g = a.gb.g[bh * Nt + tau];
    t_U = a.gb.U[bh * Nt + tau];
    t_R = a.gb.R[bh * Nt + tau];
  };

  // n~ of the next tile (every wave its own tiles) into half b of the tile
  // data, as three bfloat16 terms hi + lo + lo2 (about 24 bits: the rows
  // whose denominators cancel strongly need n~ to float32 accuracy), the
  // operand of q . n~ on MFMA. The byte offsets are kept whole (empty asm
  // statement), so that each store is one step from the array and the
  // compiler can tell it from the copies in flight.
  auto put_n = [&](int b) {
    const Lanes ln = fresh_lanes();
#pragma unroll
    for (int x = 0; x < KXN; ++x) {
      if (n_live(x)) {
        float n[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) n[r] = sum_quad(Nacc[x][r]);
        bf16x2v h01, l01, e01, h23, l23, e23;
        split3(n[0], n[1], h01, l01, e01);
        split3(n[2], n[3], h23, l23, e23);
        const bf16x4 t0 = __builtin_shufflevector(h01, h23, 0, 1, 2, 3);
        const bf16x4 t1 = __builtin_shufflevector(l01, l23, 0, 1, 2, 3);
        const bf16x4 t2 = __builtin_shufflevector(e01, e23, 0, 1, 2, 3);
        int off = L::oBuf + b * L::bufBytes + 2 * state_k0(kxg(nx(x)), ln.g);
        asm("" : "+v"(off));
        if (ln.i == 0) {
          *reinterpret_cast<bf16x4*>(smem + off) = t0;
          *reinterpret_cast<bf16x4*>(smem + off + 2 * NTP) = t1;
          *reinterpret_cast<bf16x4*>(smem + off + 4 * NTP) = t2;
        }
      }
    }
  };

  // Tile scalars and the per-key / per-row data of tile tau (waves 0-3, from
  // the gate registers of tau and the stabiliser chain m, logD at its start):
  // Rm = max(m if no zero forget gate in the tile, U), the decay exp(m - Rm),
  // key weights exp(u_j - Rm - logD_next), and the row stabiliser r_t =
  // max(m if no zero gate at or before t, prefix max of u).
  auto prep = [&](int64_t tau, const TileBuf& tb, double m, double logD, bool state) -> void {
    const int Lc = (int)min((int64_t)kTile, T - tau * kTile);
    double Rm = fmax(t_R >= 0 ? -INFINITY : m, t_U);
    if (Rm == -INFINITY) Rm = 0.0;
    const double ld = (t_R >= 0 || m == -INFINITY) ? -INFINITY : m - Rm;
    const bool rescale = logD + ld < -kMaxDefer;
    const double logD_next = rescale ? 0.0 : logD + ld;
    const int j = fresh_lanes().lane;
    if (w == 0) {
      const float wj = (j >= t_R && j < Lc && t_U != -INFINITY) ? exp_f64arg(r_u - Rm - logD_next) : 0.f;
      tb.w[j] = wj;
      // the weights of the normaliser's MFMA columns: wj = hi + lo + lo2 to
      // about 24 bits (rows whose denominators cancel strongly need n~ to
      // float32 accuracy)
      const __bf16 whi = (__bf16)wj;
      const float wr = wj - (float)whi;
      const __bf16 wlo = (__bf16)wr;
      tb.wb[j] = whi;
      int jl = WBP + j;   // kept whole: one step from the array (see put_n)
      asm("" : "+v"(jl));
      tb.wb[jl] = wlo;
      int jl2 = 2 * WBP + j;
      asm("" : "+v"(jl2));
      tb.wb[jl2] = (__bf16)(wr - (float)wlo);
      if (j == 0) {
        tb.info[0] = rescale ? 1 : 0;
        tb.info[1] = __builtin_bit_cast(int, rescale ? exp_f64arg(logD + ld) : 1.f);   // below e^-70
      }
    } else {
      const bool carry0 = state && __builtin_amdgcn_readlane(r_rs, 0) < 0;   // lane 0 holds the first token
      double ref = fmax(carry0 ? m : -INFINITY, readlane_f64(r_mp, 0));
      if (ref == -INFINITY) ref = 0.0;
      const bool valid = j < Lc;
      const bool carry = state && r_rs < 0;
      double r = fmax(carry ? m : -INFINITY, r_mp);
      if (r == -INFINITY) r = 0.0;
      if (w == 1) {
        tb.r2[j] = valid ? (float)((r - ref) * (double)kLog2eF) : 0.f;
        tb.u2[j] = valid ? (float)((r_u - ref) * (double)kLog2eF) : -INFINITY;
        tb.rs[j] = r_rs;
      } else if (w == 2) {
        tb.sc[j] = (valid && carry) ? exp_f64arg(m - r + logD) : 0.f;
      } else {
        tb.fl[j] = valid ? exp_f64arg(-(r_b + r)) : 1.f;
      }
    }
  };
  // the chain of the stabiliser over the tiles, carried by waves 0-3
  double m_chain = m_start, logD_chain = 0.0;
  auto advance = [&](double& m, double& logD) {
    double Rm = fmax(t_R >= 0 ? -INFINITY : m, t_U);
    if (Rm == -INFINITY) Rm = 0.0;
    const double ld = (t_R >= 0 || m == -INFINITY) ? -INFINITY : m - Rm;
    logD = logD + ld < -kMaxDefer ? 0.0 : logD + ld;
    m = t_g + Rm;
  };

  // ---------------- epilogue: per column half a lane forms four consecutive
  // columns of each of its two rows and stores them, paired with its partner
  // lane's, as 16-byte row pieces straight to H (the layout of load_o); rows
  // past the sequence end fall outside the buffer range and are dropped
  auto epi_math = [&]() {
    const Lanes le = fresh_lanes();
    float dnm[2];
#pragma unroll
    for (int z = 0; z < 2; ++z) dnm[z] = s_dnm[16 * zg(z) + le.i];
#pragma unroll
    for (int cv = 0; cv < 2; ++cv) {
      bf16x4 h4[2];
#pragma unroll
      for (int z = 0; z < 2; ++z) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // sigmoid(o) / D = 1 / ((1 + e^-o) D); e = 0 without an output gate
          const float e = __builtin_amdgcn_exp2f(fmaf(-kLog2eF, (float)epo[cv][z][r], a.o_bias));
          h4[z][r] = (__bf16)(eacc[z][cv][r] * __builtin_amdgcn_rcpf(fmaf(e, dnm[z], dnm[z])));
        }
      }
      swap_rows16(h4[1], h4[0]);
      hv[cv] = __builtin_shufflevector(h4[1], h4[0], 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  auto epi_store = [&](int64_t te) {
    const __amdgpu_buffer_rsrc_t hr = tile_rsrc_vo(a.h, te);
#pragma unroll
    for (int cv = 0; cv < 2; ++cv) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, hv[cv]), hr, (int)offO[cv], 0, 0);
  };
#pragma unroll
  for (int cv = 0; cv < 2; ++cv) {
    epo[cv][0] = epo[cv][1] = bf16x4{};
    eacc[0][cv] = eacc[1][cv] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (tid < kTile) s_dnm[tid] = 1.f;   // read (unused) by the first tile's epilogue pass

  for (int r = 0; r < RK; ++r) dma_k(tile0, r);
  for (int r = 0; r < RQ; ++r) dma_q(tile0, r);
  for (int r = 0; r < RV; ++r) dma_v(tile0, r);
  if (w < 4) {
    load_gate(tile0);
    prep(tile0, tile_buf(0), m_chain, logD_chain, has_state);
    advance(m_chain, logD_chain);
  }
  put_n(0);
  __builtin_amdgcn_s_waitcnt(0);
  for (int64_t tau = tile0; tau < tile1; ++tau) {
    const int64_t t0 = tau * kTile;
    const int Lc = (int)min((int64_t)kTile, T - t0);
    const int buf = (int)((tau - tile0) & 1);
    const TileBuf tb = tile_buf(buf);

    // this wave's copies of tile tau have landed (and its H stores of tile
    // tau - 1, which were issued last, have completed)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // tile tau in LDS, its tile data prepared; tile tau - 1's reads done
    const bool more = tau + 1 < tile1;
    // The copies of the next tile and the register loads go out
    // unconditionally (on the last tile they repeat it into buffers nobody
    // reads any more), so that every wave issues the same memory operations on
    // every tile and the compiler's waits for loaded registers are exact.
    const int64_t tn = more ? tau + 1 : tau;
    if (w < 4) load_gate(tn);   // consumed by the preparation of tile tau + 1 at the end of this one
    load_o(tau, 0);
    load_o(tau, 1);
    epi_math();   // the previous tile's (on the first tile a pass whose result is dropped)

    // ---------------- partial Q K^T (16 keys x 64 rows) and (Q C~^T)^T (32
    // columns x 64 rows) over this wave's half of d_qk
    f32x4 sacc[4], acc[4][2];
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      sacc[z] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[z][0] = acc[z][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // q . n~ over this wave's half of d_qk for rows 16 cg .. + 15: the three
    // terms of n~ as rows 0-2 of the A operand (row 3 onwards zero), summed
    // below from registers 0-2 of lanes g = 0
    f32x4 nqacc = f32x4{0.f, 0.f, 0.f, 0.f};
    const Lanes l1 = fresh_lanes();
    unroll<KSH>([&](auto s_c) {
      constexpr int s = decltype(s_c)::value;
      const int col = KH * kh + 32 * s + 8 * l1.g;
      bf16x8 fa[4];
#pragma unroll
      for (int z = 0; z < 4; ++z) fa[z] = *reinterpret_cast<const bf16x8*>(&sQ[(16 * zg(z) + l1.i) * QP + col]);
      const bf16x8 fk = *reinterpret_cast<const bf16x8*>(&sK[(16 * kg + l1.i) * KP + col]);
#pragma unroll
      for (int z = 0; z < 4; ++z) sacc[z] = mma(fk, fa[z], sacc[z]);
      const bf16x8 fq = *reinterpret_cast<const bf16x8*>(&sQ[(16 * cg + l1.i) * QP + col]);
      const bf16x8 fn = *reinterpret_cast<const bf16x8*>(&tb.nt[min(l1.i, 3) * NTP + col]);
      nqacc = mma(fn, fq, nqacc);
      // the carried state as two bf16 terms: rows whose q is nearly
      // orthogonal to a dominant key make C~ q a strongly cancelling sum
#pragma unroll
      for (int cv = 0; cv < 2; ++cv) {
        const bf16x8 Bc = pack_bf16(Ct[2 * s][cv], Ct[2 * s + 1][cv]);
        const bf16x8 Bl = pack_bf16_rest(Ct[2 * s][cv], Ct[2 * s + 1][cv], Bc);
#pragma unroll
        for (int z = 0; z < 4; ++z) acc[z][cv] = mma(Bl, fa[z], mma(Bc, fa[z], acc[z][cv]));
      }
    });
    // the partner's rows (groups 2 and 3) to the exchange area
    {
      const Lanes lx = fresh_lanes();
      f32x4* xo = s_x + w * L::kXchg * 64 + lx.lane;
      xo[0] = acc[2][0];
      xo[64] = acc[2][1];
      xo[128] = acc[3][0];
      xo[192] = acc[3][1];
      xo[256] = sacc[2];
      xo[320] = sacc[3];
    }
    // V^T fragments of P V and of the state update (columns 32 cg + 16 cv),
    // read before the copies into sV are issued
    bf16x8 Av[kTile / 32][2];
    {
      const Lanes lv = fresh_lanes();
#pragma unroll
      for (int jb = 0; jb < kTile / 32; ++jb)
#pragma unroll
        for (int cv = 0; cv < 2; ++cv) Av[jb][cv] = frag_tr(sV, VP, 32 * jb, 32 * cg + 16 * cv, lv.lane);
    }
    // ---------------- this half's q . n~ of rows 16 cg .. + 15 (the three
    // terms' partial sums added in float32). Register 3 (the zero row) is
    // added too: a result register left unread may be handed to the next
    // value at once, and an inline-asm write there (fresh_tid) is not held
    // back until the MFMA has written it.
    {
      const float nq = (nqacc[0] + nqacc[1]) + (nqacc[2] + nqacc[3]);
      const Lanes ln = fresh_lanes();
      if (ln.g == 0) s_dn[kh * kTile + 16 * cg + ln.i] = nq;
    }

    // The registers loaded at the top of the tile are taken here, before any
    // copy is issued: with copies or stores in flight the compiler can only
    // wait for all of the wave's memory operations. O is split into its
    // epilogue layout; the gate registers are marked as needed.
    swap_rows16(po[0][1], po[0][0]);
    swap_rows16(po[1][1], po[1][0]);
    if (w < 4) asm volatile("" ::"v"(r_u), "v"(r_mp), "v"(r_b), "v"(r_rs));
    if (tau > tile0) epi_store(tau - 1);
    lds_barrier();   // the exchange area is complete; Q and V of tile tau no longer read from LDS
    // ---------------- copies of the next tile's Q and V, in five slots from here on
    auto copy_qv = [&](int q) {
      if (q < RQ) dma_q(tn, q);
      if (q < RV) dma_v(tn, q);
    };
    copy_qv(0);
    // ---------------- the partner's partial sums for this wave's rows
    {
      const Lanes lx = fresh_lanes();
      const f32x4* xi = s_x + (w ^ 4) * L::kXchg * 64 + lx.lane;
      acc[0][0] += xi[0];
      acc[0][1] += xi[64];
      acc[1][0] += xi[128];
      acc[1][1] += xi[192];
      sacc[0] += xi[256];
      sacc[1] += xi[320];
    }
    // the carried-state term enters row t with weight exp(m_prev - r_t + logD);
    // acc[z][cv] register r in lane (g, i) is H^T[v = 32 cg + 16 cv + 4 g + r][t = 16 zg(z) + i]
    {
      const Lanes lp = fresh_lanes();
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const float sc = tb.sc[16 * zg(z) + lp.i];
        acc[z][0] *= sc;
        acc[z][1] *= sc;
      }
    }
    // ---------------- P = S o D: lane holds S^T[j = 16 kg + 4 g + r][t = 16 zg(zz) + i]
    auto phase_p = [&]() {
      const Lanes lp = fresh_lanes();
      const f32x4 u2 = *reinterpret_cast<const f32x4*>(&tb.u2[16 * kg + 4 * lp.g]);
#pragma unroll
      for (int zz = 0; zz < 2; ++zz) {
        const int tl = 16 * (2 * kh + zz) + lp.i;
        const float r2 = tb.r2[tl];
        const int rs = tb.rs[tl];
        bf16x4 pk4;
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jk = 16 * kg + 4 * lp.g + r;
          const bool keep = (tl < Lc) && (jk <= tl) && (jk >= rs);
          const float p = keep ? sacc[zz][r] * __builtin_amdgcn_exp2f(u2[r] - r2) : 0.f;
          psum += p;
          pk4[r] = (__bf16)p;
        }
        *reinterpret_cast<bf16x4*>(&sP[tl * PP + 16 * kg + 4 * lp.g]) = pk4;
        psum = sum_rows(psum);
        if (lp.g == 0) s_den[kg * kTile + tl] = psum;
        copy_qv(1 + zz);
      }
    };
    // ---------------- state update: C~ <- decay C~ + K^T diag(w) V, n~ likewise
    // (Q C~^T above used the state at the start of the tile)
    auto phase_u = [&]() {
      if (__builtin_amdgcn_readfirstlane(tb.info[0])) {   // uniform over the workgroup
        const float f = __builtin_bit_cast(float, tb.info[1]);
#pragma unroll
        for (int x = 0; x < KXH; ++x) {
          Ct[x][0] *= f;
          Ct[x][1] *= f;
        }
#pragma unroll
        for (int x = 0; x < KXN; ++x) Nacc[x] *= f;
      }
#pragma unroll
      for (int jb = 0; jb < kTile / 32; ++jb) {
        const int ts = 32 * jb;
        const Lanes lu = fresh_lanes();
        const f32x4 wa = *reinterpret_cast<const f32x4*>(&tb.w[ts + 8 * lu.g]);
        const f32x4 wb = *reinterpret_cast<const f32x4*>(&tb.w[ts + 8 * lu.g + 4]);
        bf16x8 Bv[2];
#pragma unroll
        for (int cv = 0; cv < 2; ++cv)
#pragma unroll
          for (int e = 0; e < 8; ++e) Bv[cv][e] = (__bf16)((float)Av[jb][cv][e] * (e < 4 ? wa[e] : wb[e - 4]));
        const bf16x8 Bw = *reinterpret_cast<const bf16x8*>(&tb.wb[min(lu.i, 3) * WBP + ts + 8 * lu.g]);
        // transposed K fragments through a ring of kRing registers: the read of
        // tile x + kRing - 1 is issued before the MFMAs of tile x
        constexpr int kRing = 4;
        bf16x8 Ak[kRing];
        const int koff = lane_off_trk(KP, kh * KXH, lu.lane);
        unroll<kRing - 1>([&](auto p_c) {
          constexpr int p = decltype(p_c)::value;
          if constexpr (p < KXH) Ak[p] = frag_trk_at(sK, koff, KP, ts, p);
        });
        unroll<KXH>([&](auto x_c) {
          constexpr int x = decltype(x_c)::value;
          if constexpr (x + kRing - 1 < KXH) Ak[(x + kRing - 1) % kRing] = frag_trk_at(sK, koff, KP, ts, x + kRing - 1);
          Ct[x][0] = mma(Ak[x % kRing], Bv[0], Ct[x][0]);
          Ct[x][1] = mma(Ak[x % kRing], Bv[1], Ct[x][1]);
          // the wave's n~ tiles take the same K fragments (scalar branch)
#pragma unroll
          for (int xn = 0; xn < KXN; ++xn)
            if (nx(xn) == x) Nacc[xn] = mma(Ak[x % kRing], Bw, Nacc[xn]);
          __builtin_amdgcn_sched_barrier(0);
        });
        copy_qv(3 + jb);
      }
    };
    // The two phases are independent: P is exponentials (VALU), the update
    // matrix products. (Taking them in opposite orders in the two waves of a
    // SIMD, or the update first, measured slower.)
    phase_p();
    phase_u();
    // the next tile's K: after the barrier no wave reads K of tile tau
    auto copy_k = [&](int r) {
      if (r < RK) dma_k(tn, r);
    };
    lds_barrier();   // sP, s_den, s_dn complete; K of tile tau no longer read from LDS
    copy_k(0);
    copy_k(1);
    if (w == 0) {   // max(|n~^T q|, floor) of row t = lane
      const int t = fresh_lanes().lane;
      const float den = s_den[t] + s_den[kTile + t] + s_den[2 * kTile + t] + s_den[3 * kTile + t];
      const float d = den + tb.sc[t] * (s_dn[t] + s_dn[kTile + t]);
      s_dnm[t] = fmaxf(fmaxf(fabsf(d), tb.fl[t]), FLT_MIN);
    }
    // ---------------- (P V)^T for the wave's rows; rows 0-31 have no keys
    // 32-63 (causal), so the half kh = 0 takes only the first 32 keys
    {
      const Lanes lv = fresh_lanes();
#pragma unroll
      for (int jb = 0; jb < kTile / 32; ++jb) {
        if (jb == 0 || kh == 1) {
          bf16x8 B[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) B[z] = *reinterpret_cast<const bf16x8*>(&sP[(16 * zg(z) + lv.i) * PP + 32 * jb + 8 * lv.g]);
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            acc[z][0] = mma(Av[jb][0], B[z], acc[z][0]);
            acc[z][1] = mma(Av[jb][1], B[z], acc[z][1]);
          }
        }
        copy_k(2 + jb);
      }
    }
    copy_k(4);
    // this tile's epilogue operands, for the next tile
#pragma unroll
    for (int cv = 0; cv < 2; ++cv) {
      epo[cv][0] = po[cv][0];
      epo[cv][1] = po[cv][1];
#pragma unroll
      for (int z = 0; z < 2; ++z) eacc[z][cv] = acc[z][cv];
    }
    // ---------------- the next tile's data into the other half (its readers
    // start after the next top barrier; this half's last readers were in tile
    // tau - 1)
    if (more) {
      const TileBuf nb = tile_buf(buf ^ 1);
      put_n(buf ^ 1);
      if (w < 4) {
        prep(tau + 1, nb, m_chain, logD_chain, true);
        advance(m_chain, logD_chain);
      }
    }
  }
  // the last tile's copies (repeats into unread buffers) land before the
  // workgroup can end and give up its LDS
  __builtin_amdgcn_s_waitcnt(0);
  if (w == 0 && lane == 0) {
    s_fin[0] = m_chain;
    s_fin[1] = logD_chain;
  }
  __syncthreads();   // final stabiliser chain and the last tile's row denominators published
  if (tile1 > tile0) {
    epi_math();
    epi_store(tile1 - 1);
  }
  const double m_fin = s_fin[0], logD_fin = s_fin[1];
  const float fD = (float)exp(logD_fin);

  // ---------------- final state of the sequence
  if (seg == a.S - 1 && a.C_out) {
    float* Cdst = a.C_out + bh * V * K;
#pragma unroll
    for (int x = 0; x < KXH; ++x)
#pragma unroll
      for (int cv = 0; cv < 2; ++cv)
        *reinterpret_cast<f32x4*>(Cdst + (vcol0 + 32 * cg + 16 * cv + i) * K + state_k0(kxg(x), g)) = fD * Ct[x][cv];
    if (vb == 0) {
      float* ndst = a.n_out + bh * K;
#pragma unroll
      for (int x = 0; x < KXN; ++x) {
        f32x4 nv;
#pragma unroll
        for (int r = 0; r < 4; ++r) nv[r] = fD * sum_quad(Nacc[x][r]);
        if (i == 0 && n_live(x)) *reinterpret_cast<f32x4*>(ndst + state_k0(kxg(nx(x)), g)) = nv;
      }
      if (tid == 0) a.m_out[bh] = (float)m_fin;
    }
  }
}

template <int K>
__global__ __launch_bounds__(64 * kOutWaves, 1) void out_kernel_fused(SegArgs a) {
  // The copy targets are separate objects: the compiler then knows that a
  // direct-to-LDS copy in flight into one of them does not touch the others,
  // and reads those without waiting for it.
  __shared__ __attribute__((aligned(16))) char lq[OutLds<K>::qBytes];
  __shared__ __attribute__((aligned(16))) char lk[OutLds<K>::kBytes];
  __shared__ __attribute__((aligned(16))) char lv[OutLds<K>::vBytes];
  __shared__ __attribute__((aligned(16))) char smem[OutLds<K>::restBytes];
  out_body<K>(a, lq, lk, lv, smem);
}

// ------------------------------------------------------------------ chunk-local end states

// The chunks' local end states (every chunk but the last, all of whose
// tiles are full): C~loc = sum over the chunk's tiles of the decayed K^T
// diag(w) V, computed by the same stabilised tile recurrence as the output
// kernel, starting from nothing. The compute waves (LocWaves) each own an
// equal share of the d_qk rows of C~^T for all 128 value columns (state in
// VGPRs), so every K^T
// fragment is read from LDS by one wave only and scaled there by the key
// weights; the V fragments are shared. A fifth wave only moves data: it copies tile tau + 1
// (K, the workgroup's 128 columns of V, the keys' in-tile weights w0 and the
// tile's gate scalars) straight into the other half of a double-buffered LDS
// area with direct-to-LDS loads while the compute waves work on tile tau.
// One barrier per tile; the compute waves issue no global loads in the loop.
constexpr int kMaxTiles = 8192 / kTile;   // tiles per chunk at the largest chunk

// Scalars of a chunk's local end state, scanned once from the tile gate
// scalars with the same float64 steps as the output kernel's tile loop, from
// an empty state: per tile the factor exp(U - Rm - logD_next) that turns the
// in-tile weights w0 into the key weights, and the factor that rescales the
// accumulators before the tile (1 when the decay is kept pending); at the end
// the chunk's m, logD, log-forget total G and whether it holds a zero gate.
struct LocScan {
  double m = -INFINITY, logD = 0.0, G = 0.0;
  bool reset = false, zero = true, any_rescale = false;
  // one tile with gate scalars gj, Uj, Rj; lane 0 writes its factors
  __device__ void step(double gj, double Uj, int Rj, float* cw, float* rf) {
    const double Rm = fmax(Rj >= 0 ? -INFINITY : m, Uj);
    const bool live = Rm != -INFINITY;
    const double ld = (Rj >= 0 || m == -INFINITY || !live) ? -INFINITY : m - Rm;
    const bool rescale = logD + ld < -kMaxDefer;
    const double logD_next = rescale ? 0.0 : logD + ld;
    const bool scale = rescale && !zero;   // rescaling a zero state is a no-op
    if ((threadIdx.x & 63) == 0) {
      *cw = (live && Uj != -INFINITY) ? exp_f64arg(Uj - Rm - logD_next) : 0.f;
      // the factor is below e^-70 (or zero): a float exp of the rounded
      // argument is as good as a float64 one and far cheaper
      *rf = scale ? exp_f64arg(logD + ld) : 1.f;
    }
    any_rescale = any_rescale || scale;
    m = live ? gj + Rm : -INFINITY;
    logD = logD_next;
    G += gj;
    reset = reset || Rj >= 0;
    if (live && Uj != -INFINITY) zero = false;
  }
};

// The same scan for up to 64 tiles at once, lane j taking tile j of the batch
// (gate scalars g, U, R of its tile; n tiles, carry-in state c). The chain
// m' = g + max(m, or -inf after a zero gate, U) is the max-plus map
// x -> max(x + a, b) with a = g (-inf on a zero gate) and b = g + U; these
// maps compose associatively, (a1, b1) then (a2, b2) giving (a1 + a2,
// max(b1 + a2, b2)), so an inclusive lane scan gives m after every tile. The
// pending decay logD is a prefix sum of ld that restarts at the tiles whose
// ld is -inf. The one case that does not fit, logD + ld falling below
// -kMaxDefer on a finite ld, returns false with c unchanged (the caller then
// takes the batch step by step).
__device__ bool local_scan_batch(double g, double U, int R, int n, LocScan& c, float* cw, float* rf) {
  const int lane = threadIdx.x & 63;
  const bool act = lane < n;
  double a = act ? (R >= 0 ? -INFINITY : g) : 0.0;
  double b = act ? g + U : -INFINITY;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double ap = __shfl_up(a, d), bp = __shfl_up(b, d);
    if (lane >= d) {
      b = fmax(bp + a, b);
      a = ap + a;
    }
  }
  const double m_after = fmax(c.m + a, b);
  double m_before = __shfl_up(m_after, 1);
  if (lane == 0) m_before = c.m;
  const double Rm = fmax(R >= 0 ? -INFINITY : m_before, U);
  const bool live = Rm != -INFINITY;
  const double ld = (R >= 0 || m_before == -INFINITY || !live) ? -INFINITY : m_before - Rm;
  // segmented prefix sum of ld, segments starting after the -inf tiles
  const bool flag = act && ld == -INFINITY;
  bool f = flag;
  double sm = (act && !flag) ? ld : 0.0;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double sp = __shfl_up(sm, d);
    const bool fp = __shfl_up((int)f, d) != 0;
    if (lane >= d) {
      sm = f ? sm : sp + sm;
      f = f || fp;
    }
  }
  const double logD_next = f ? sm : c.logD + sm;
  double logD_before = __shfl_up(logD_next, 1);
  if (lane == 0) logD_before = c.logD;
  if (__any(act && !flag && logD_before + ld < -kMaxDefer)) return false;
  const bool nonzero = act && live && U != -INFINITY;
  const unsigned long long nzmask = __ballot(nonzero);
  const bool zero_before = c.zero && (nzmask & ((1ull << lane) - 1ull)) == 0ull;
  const bool scale = flag && !zero_before;   // rescaling a zero state is a no-op
  if (act) {
    cw[lane] = nonzero ? exp_f64arg(U - Rm - logD_next) : 0.f;
    rf[lane] = scale ? exp_f64arg(logD_before + ld) : 1.f;   // zero: ld is -inf here
  }
  double gs = act ? g : 0.0;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) gs += __shfl_xor(gs, d);
  c.m = __shfl(m_after, n - 1);
  c.logD = __shfl(logD_next, n - 1);
  c.G += gs;
  c.reset = c.reset || __any(act && R >= 0);
  c.zero = c.zero && nzmask == 0ull;
  c.any_rescale = c.any_rescale || __any(scale);
  return true;
}

__device__ LocScan local_scan(const SegArgs& a, int64_t bh, int64_t tile0, int ntiles, float* s_cw, float* s_rf) {
  const int lane = threadIdx.x & 63;
  LocScan r;
  for (int base = 0; base < ntiles; base += 64) {
    const int n = min(64, ntiles - base);
    const int64_t t = bh * a.Nt + tile0 + base + min(lane, n - 1);
    const double gv = a.gb.g[t], Uv = a.gb.U[t];
    const int Rv = a.gb.R[t];
    if (!local_scan_batch(gv, Uv, Rv, n, r, s_cw + base, s_rf + base)) {
      for (int j = 0; j < n; ++j)
        r.step(readlane_f64(gv, j), readlane_f64(Uv, j), __builtin_amdgcn_readlane(Rv, j), s_cw + base + j, s_rf + base + j);
    }
  }
  return r;
}

template <int K>
struct LocLds {
  static constexpr int KP = K + 16;                 // 8 dwords mod 64 banks: conflict-free for frag_tr
  static constexpr int VP = kVB + 8;
  static constexpr int CPRK = KP / 8;               // 16-byte chunks per LDS row of K
  static constexpr int CPRV = VP / 8;
  static constexpr int kBytes = kTile * KP * 2;     // = 1024 * CPRK: CPRK direct loads
  static constexpr int vBytes = kTile * VP * 2;     // = 1024 * CPRV
  static constexpr int kBufs = 3;                   // tiles in LDS: the one in use and two ahead
  static constexpr int oK = 0;                      // [3] K tiles
  static constexpr int oV = oK + kBufs * kBytes;    // [3] V tiles
  static constexpr int oW = oV + kBufs * vBytes;    // [3][64] float w0
  static constexpr int oWb = oW + kBufs * kTile * 4;       // [3][4][64] bf16: w0 hi, lo, lo2, zero
  static constexpr int oCw = oWb + kBufs * 4 * kTile * 2;   // [kMaxTiles] float: tile weight factor
  static constexpr int oRf = oCw + kMaxTiles * 4;          // [kMaxTiles] float: accumulator rescale (1 = none)
  static constexpr int bytes = oRf + kMaxTiles * 4;
  // direct loads one tile's copy issues (a wave-wide load per 1 KiB of K and
  // V, one for w0, one for its split): the loader waits for a tile by
  // counting them
  static constexpr int kLoadsPerTile = CPRK + CPRV + 2;
  static_assert(kLoadsPerTile <= 63, "fits the vector-memory wait counter");
  static_assert(bytes <= 160 * 1024, "fits the LDS of a CU");
};
// Compute waves of local_kernel: eight (two per SIMD, 32 d_qk rows each) when
// d_qk allows, else four.
template <int K> struct LocWaves { static constexpr int value = K >= 128 ? 8 : 4; };

// s_waitcnt that waits until at most N vector-memory operations of the wave
// are outstanding (N <= 63; the LDS and export counters are left alone).
template <int N>
__device__ __forceinline__ void wait_vm_at_most() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The loader wave of local_kernel: tiles tau + 1 and tau + 2 on their way
// into the two free buffers of three while the compute waves work on tile
// tau. It waits only for the tile the compute waves need next (by the count
// of its direct loads still in flight) and meets them at barriers that wait
// for LDS traffic alone, so the copy of the tile after next stays in flight
// across the barrier.
template <int K>
__device__ __forceinline__ void local_loader(const SegArgs& a, char* smem) {
  using L = LocLds<K>;
  const int64_t BH = a.BH, T = a.T, V = a.V, Nt = a.Nt;
  const int nvb = (int)(V / kVB);
  const int64_t bh = blockIdx.x % BH;
  const int64_t rest = blockIdx.x / BH;
  const int vb = (int)(rest % nvb);
  const int seg = (int)(rest / nvb);
  const int64_t tile0 = (int64_t)seg * a.TPS;
  const int64_t tile1 = tile0 + a.TPS;
  const int64_t vcol0 = (int64_t)vb * kVB;
  // ---------------- loader wave: per-lane source offsets of the direct
  // loads (chunk c = 64 n + lane of a tile's padded LDS image lies in row
  // c / CPR; padding chunks repeat the row's last data chunk)
  const int lane = threadIdx.x & 63;
  unsigned offk[L::CPRK], offv[L::CPRV];
#pragma unroll
  for (int n = 0; n < L::CPRK; ++n) {
    const int c = 64 * n + lane, row = c / L::CPRK, ch = min(c % L::CPRK, K / 8 - 1);
    offk[n] = (unsigned)(row * K + 8 * ch);
  }
#pragma unroll
  for (int n = 0; n < L::CPRV; ++n) {
    const int c = 64 * n + lane, row = c / L::CPRV, ch = min(c % L::CPRV, kVB / 8 - 1);
    offv[n] = (unsigned)(row * V + 8 * ch);
  }
  auto dma = [&](int64_t tau, int buf) {
    const __bf16* kt = a.k + (bh * T + tau * kTile) * K;
    const __bf16* vt = a.v + (bh * T + tau * kTile) * V + vcol0;
    char* kd = smem + L::oK + buf * L::kBytes;
    char* vd = smem + L::oV + buf * L::vBytes;
#pragma unroll
    for (int n = 0; n < L::CPRK; ++n)
      __builtin_amdgcn_global_load_lds((global_void*)(kt + offk[n]), (lds_void*)(kd + 1024 * n), 16, 0, 0);
#pragma unroll
    for (int n = 0; n < L::CPRV; ++n)
      __builtin_amdgcn_global_load_lds((global_void*)(vt + offv[n]), (lds_void*)(vd + 1024 * n), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_void*)(a.gb.w0 + bh * T + tau * kTile + lane),
                                     (lds_void*)(smem + L::oW + buf * kTile * 4), 4, 0, 0);
    if (lane < 24)   // hi, lo and lo2 rows of the split weights, 384 bytes
      __builtin_amdgcn_global_load_lds((global_void*)(a.gb.wb + (bh * Nt + tau) * 3 * kTile + 8 * lane),
                                       (lds_void*)(smem + L::oWb + buf * 4 * kTile * 2), 16, 0, 0);
  };
  dma(tile0, 0);
  if (tile0 + 1 < tile1) {
    dma(tile0 + 1, 1);
    wait_vm_at_most<L::kLoadsPerTile>();   // tile tile0 has landed
  } else {
    wait_vm_at_most<0>();
  }
  int nbuf = 2;   // buffer of tile tau + 2
  for (int64_t tau = tile0; tau < tile1; ++tau) {
    lds_barrier();   // tile tau published; the buffer tile tau - 1 used is free
    if (tau + 2 < tile1) {
      dma(tau + 2, nbuf);
      nbuf = nbuf == L::kBufs - 1 ? 0 : nbuf + 1;
      wait_vm_at_most<L::kLoadsPerTile>();   // tile tau + 1 has landed, tau + 2 may be in flight
    } else {
      wait_vm_at_most<0>();
    }
  }
}

template <int K, bool RESCALE>
__device__ __forceinline__ void local_body(const SegArgs& a, char* smem, const LocScan& sc) {
  using L = LocLds<K>;
  constexpr int KP = L::KP, VP = L::VP;
  constexpr int KX = K / 16, NW = LocWaves<K>::value, KXW = KX / NW, VY = kVB / 16;
  static_assert(KX % NW == 0, "KX / NW row tiles per compute wave");
  const int64_t BH = a.BH, V = a.V;
  const int nvb = (int)(V / kVB);
  const int64_t bh = blockIdx.x % BH;
  const int64_t rest = blockIdx.x / BH;
  const int vb = (int)(rest % nvb);
  const int seg = (int)(rest / nvb);
  const int64_t tile0 = (int64_t)seg * a.TPS;
  const int64_t tile1 = tile0 + a.TPS;
  const int64_t vcol0 = (int64_t)vb * kVB;
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);

  // ---------------- compute waves: register r of Ct[x][y] in lane (g, i) is
  // C~^T[k = 16 (KXW w + x) + 4 g + r][v = 16 y + i]
  f32x4 Ct[KXW][VY];
  f32x4 Nacc[KXW];
#pragma unroll
  for (int x = 0; x < KXW; ++x) {
#pragma unroll
    for (int y = 0; y < VY; ++y) Ct[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
    Nacc[x] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float* s_cw = reinterpret_cast<const float*>(smem + L::oCw);
  const float* s_rf = reinterpret_cast<const float*>(smem + L::oRf);
  int buf = 0;   // buffer of tile tau
  for (int64_t tau = tile0; tau < tile1; ++tau, buf = buf == L::kBufs - 1 ? 0 : buf + 1) {
    lds_barrier();   // tile tau in buffer buf
    const int j = (int)(tau - tile0);
    const __bf16* sK = reinterpret_cast<const __bf16*>(smem + L::oK + buf * L::kBytes);
    const __bf16* sV = reinterpret_cast<const __bf16*>(smem + L::oV + buf * L::vBytes);
    const float* s_w0 = reinterpret_cast<const float*>(smem + L::oW + buf * kTile * 4);
    const __bf16* swb = reinterpret_cast<const __bf16*>(smem + L::oWb + buf * 4 * kTile * 2);
    // keys enter with weight exp(u_j - Rm - logD_next) = w0_j cw
    const float cw = s_cw[j];
    if constexpr (RESCALE) {
      const float f = s_rf[j];
      if (__builtin_amdgcn_readfirstlane(f != 1.f ? 1 : 0)) {
#pragma unroll
        for (int x = 0; x < KXW; ++x) {
#pragma unroll
          for (int y = 0; y < VY; ++y) Ct[x][y] *= f;
          Nacc[x] *= f;
        }
      }
    }
#pragma unroll
    for (int ts = 0; ts < kTile; ts += 32) {
      const Lanes lu = fresh_lanes();
      f32x4 wa = *reinterpret_cast<const f32x4*>(&s_w0[ts + 8 * lu.g]);
      f32x4 wb = *reinterpret_cast<const f32x4*>(&s_w0[ts + 8 * lu.g + 4]);
      wa *= cw;
      wb *= cw;
      // n~ operand: columns 0, 1, 2 the three bf16 terms of w0, the rest
      // zero; the product is scaled by cw in float32
      const bf16x8 Bw = *reinterpret_cast<const bf16x8*>(&swb[min(lu.i, 3) * kTile + ts + 8 * lu.g]);
      // this wave's K^T fragments: raw for n~, scaled by the key weights for C~
      bf16x8 As[KXW], Kr[KXW], Bv[4];
#pragma unroll
      for (int x = 0; x < KXW; ++x) Kr[x] = frag_tr(sK, KP, ts, 16 * (KXW * w + x), lu.lane);
      unroll<3>([&](auto y_c) {
        constexpr int y = decltype(y_c)::value;
        if constexpr (y < VY) Bv[y] = frag_tr(sV, VP, ts, 16 * y, lu.lane);
      });
#pragma unroll
      for (int x = 0; x < KXW; ++x) {
        const bf16x8 raw = Kr[x];
        Nacc[x] += cw * mma(raw, Bw, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 8; ++e) As[x][e] = (__bf16)((float)raw[e] * (e < 4 ? wa[e] : wb[e - 4]));
      }
      // V fragments through a ring of kRing: the read of column tile
      // y + kRing - 1 is issued before the MFMAs of tile y
      constexpr int kRing = 4;
      unroll<VY>([&](auto y_c) {
        constexpr int y = decltype(y_c)::value;
        if constexpr (y + kRing - 1 < VY) Bv[(y + kRing - 1) % kRing] = frag_tr(sV, VP, ts, 16 * (y + kRing - 1), lu.lane);
#pragma unroll
        for (int x = 0; x < KXW; ++x) Ct[x][y] = mma(As[x], Bv[y % kRing], Ct[x][y]);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  }
  const float fD = (float)exp(sc.logD);
  const Lanes le = fresh_lanes();
  const int64_t sidx = bh * (a.S - 1) + seg;
  float* Cdst = a.Cseg + sidx * V * K;
#pragma unroll
  for (int x = 0; x < KXW; ++x)
#pragma unroll
    for (int y = 0; y < VY; ++y)
      *reinterpret_cast<f32x4*>(Cdst + (vcol0 + 16 * y + le.i) * K + 16 * (KXW * w + x) + 4 * le.g) = fD * Ct[x][y];
  if (vb == 0) {
    float* ndst = a.nseg + sidx * K;
#pragma unroll
    for (int x = 0; x < KXW; ++x) {
      f32x4 nv;
#pragma unroll
      for (int r = 0; r < 4; ++r) nv[r] = fD * sum_quad(Nacc[x][r]);
      if (le.i == 0) *reinterpret_cast<f32x4*>(ndst + 16 * (KXW * w + x) + 4 * le.g) = nv;
    }
    if (w == 0 && le.lane == 0) {
      a.mloc[sidx] = sc.m;
      a.Gseg[sidx] = sc.reset ? -INFINITY : sc.G;
    }
  }
}

template <int K>
__global__ __launch_bounds__(64 * (LocWaves<K>::value + 1)) void local_kernel(SegArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[LocLds<K>::bytes];
  if (__builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) == LocWaves<K>::value) {
    local_loader<K>(a, smem);   // starts the first tile's copy at once
    return;
  }
  const int64_t bh = blockIdx.x % a.BH;
  const int seg = (int)(blockIdx.x / a.BH / (a.V / kVB));
  const int64_t tile0 = (int64_t)seg * a.TPS;
  using L = LocLds<K>;
  // zero rows of the split-weight operands (published by the first barrier);
  // every compute wave writes the same tile table and reads only its own writes
  if (threadIdx.x < kTile) {
#pragma unroll
    for (int b = 0; b < L::kBufs; ++b)
      reinterpret_cast<__bf16*>(smem + L::oWb + b * 4 * kTile * 2)[3 * kTile + threadIdx.x] = (__bf16)0.f;
  }
  const LocScan sc = local_scan(a, bh, tile0, a.TPS, reinterpret_cast<float*>(smem + L::oCw),
                                reinterpret_cast<float*>(smem + L::oRf));
  if (sc.any_rescale)
    local_body<K, true>(a, smem, sc);
  else
    local_body<K, false>(a, smem, sc);
}

// ------------------------------------------------------------------ chunk combine

struct CombineArgs {
  const float *C0 = nullptr, *n0 = nullptr, *m0 = nullptr;
  float* Cseg = nullptr;
  float* nseg = nullptr;
  const double* mloc = nullptr;
  double* mstart = nullptr;
  const double* Gseg = nullptr;
  // A segment summary instead: the fold starts from the empty state
  // (m = -inf), its end goes to these, and the folded states are not stored.
  SummaryOut out = {nullptr, nullptr, nullptr, nullptr};
  int64_t V = 0, K = 0, BH = 0;
  int S = 0;
};

// Folds the local end states of chunks 0..S-2 in order: with the start state
// (C~, m) of chunk s and its local end state (C~loc, mloc) and log-forget total
// G, the start of chunk s+1 is m' = max(m + G, mloc),
// C~' = exp(m + G - m') C~ + exp(mloc - m') C~loc (the same for n~). Each
// thread owns four consecutive floats of one head's C~ or n~; the result
// overwrites the local state in place. For a segment summary (a.out.C set)
// the fold starts from the empty state and only its end is written, with
// the sum of the chunks' log-forget totals.
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
  const bool summary = a.out.C != nullptr;
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
  double m = summary ? -INFINITY : 0.0, gsum = 0.0;
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
        // an all-zero state: m = 0 in a start state, kept at -inf in a summary
        if (mn == -INFINITY && !summary) mn = 0.0;
        const float al = mc == -INFINITY ? 0.f : exp_f64arg(mc - mn);
        const float be = ml == -INFINITY ? 0.f : exp_f64arg(ml - mn);
        x = al * x + be * y[e];
        gsum += G;
        if (!summary) {
          *reinterpret_cast<f32x4*>(base + sidx * stride) = x;
          if (u == 0) a.mstart[sidx] = mn;
        }
        m = mn;
      }
    }
  }
  if (summary) {
    *reinterpret_cast<f32x4*>((is_n ? a.out.n + bh * a.K : a.out.C + bh * a.V * a.K) + off) = x;
    if (u == 0) {
      a.out.m[bh] = (float)m;
      a.out.G[bh] = gsum;
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
  a.o_bias = f.o ? 0.f : -INFINITY;
  a.h = static_cast<__bf16*>(f.h);
  a.gb = gb;
  a.C0 = f.C0; a.n0 = f.n0; a.m0 = f.m0;
  a.Cseg = ss.C; a.nseg = ss.n; a.mloc = ss.mloc; a.mstart = ss.mstart; a.Gseg = ss.G;
  a.C_out = f.C_out; a.n_out = f.n_out; a.m_out = f.m_out;
  a.T = f.T; a.Nt = f.Nc; a.V = f.V; a.BH = f.BH;
  a.TPS = ss.TPS; a.S = ss.S;
  a.fold_here = 0;
  const int64_t nvb = f.V / kVB;
  if (ss.S > 1) {
    mark_before(f.marks, K_STATE, s);
    hipLaunchKernelGGL((local_kernel<K>), dim3((unsigned)(f.BH * nvb * (ss.S - 1))), dim3(64 * (LocWaves<K>::value + 1)), 0, s, a);
    // With few, long chunks each output workgroup folds its own start state
    // (its slice of at most kFoldHere local states, read from the cache);
    // otherwise the fold kernel writes the start states once. Each local
    // state costs the prologue about one memory latency, which a chunk walk
    // of fewer than kFoldMinTiles tiles does not win back (measured at
    // d_qk = d_v = 128, four tiles and seven states: 1.7 us slower than the
    // fold kernel; at d_qk = 256, d_v = 512, sixteen tiles: 4.5 us faster).
    a.fold_here = (ss.S - 1 <= kFoldHere && ss.TPS >= kFoldMinTiles) ? 1 : 0;
    if (!a.fold_here) {
      CombineArgs c;
      c.C0 = f.C0; c.n0 = f.n0; c.m0 = f.m0;
      c.Cseg = ss.C; c.nseg = ss.n; c.mloc = ss.mloc; c.mstart = ss.mstart; c.Gseg = ss.G;
      c.V = f.V; c.K = K; c.BH = f.BH; c.S = ss.S;
      const int64_t units = f.V * K / 4 + K / 4;
      const int64_t blocks = (units + kThreads - 1) / kThreads;
      hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(f.BH * blocks)), dim3(kThreads), 0, s, c);
    }
    mark_after(f.marks, K_STATE, s);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  mark_before(f.marks, K_OUT, s);
  hipLaunchKernelGGL((out_kernel_fused<K>), dim3((unsigned)(f.BH * nvb * ss.S)), dim3(64 * kOutWaves), 0, s, a);
  mark_after(f.marks, K_OUT, s);
  return hipGetLastError();
}

template <int K>
hipError_t run_summary(const FwdLaunch& f, const GateBuffers& gb, const SegStates& ss, const SummaryOut& o,
                       hipStream_t s) {
  SegArgs a{};
  a.k = static_cast<const __bf16*>(f.k);
  a.v = static_cast<const __bf16*>(f.v);
  a.gb = gb;
  a.Cseg = ss.C; a.nseg = ss.n; a.mloc = ss.mloc; a.mstart = ss.mstart; a.Gseg = ss.G;
  a.T = f.T; a.Nt = f.Nc; a.V = f.V; a.BH = f.BH;
  // every chunk takes a local state: the states are indexed by chunk as those
  // of chunks 0..S-2 of a sequence one chunk longer
  a.TPS = ss.TPS; a.S = ss.S + 1;
  const int64_t nvb = f.V / kVB;
  hipLaunchKernelGGL((local_kernel<K>), dim3((unsigned)(f.BH * nvb * ss.S)), dim3(64 * (LocWaves<K>::value + 1)), 0, s, a);
  CombineArgs c;
  c.Cseg = ss.C; c.nseg = ss.n; c.mloc = ss.mloc; c.mstart = ss.mstart; c.Gseg = ss.G;
  c.out = o;
  c.V = f.V; c.K = K; c.BH = f.BH; c.S = ss.S + 1;
  const int64_t units = f.V * K / 4 + K / 4;
  const int64_t blocks = (units + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(f.BH * blocks)), dim3(kThreads), 0, s, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_summary(const FwdLaunch& f, const GateBuffers& gb, const SegStates& ss, const SummaryOut& o,
                          hipStream_t s) {
  switch (f.K) {
    case 64: return run_summary<64>(f, gb, ss, o, s);
    case 128: return run_summary<128>(f, gb, ss, o, s);
    case 256: return run_summary<256>(f, gb, ss, o, s);
  }
  return hipErrorInvalidValue;
}

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
