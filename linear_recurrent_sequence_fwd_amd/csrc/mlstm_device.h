// Device-side helpers shared by the HIP translation units of the mLSTM
// library: vector types, activations, MFMA wrappers and operand loads,
// wave/workgroup scans, LDS staging. Internal; not part of the public ABI.
//
// MFMA layouts used (16x16 output tiles, one wave64):
//   A operand  lane l holds A[l%16][kin = (l/16)*E .. +E-1]
//   B operand  lane l holds B[l%16][kin = (l/16)*E .. +E-1]   (D = A . B^T)
//   D result   lane l, register r holds D[4*(l/16) + r][l%16]
// with E = 8 for v_mfma_f32_16x16x32_bf16 and E = 1 for v_mfma_f32_16x16x4_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "mlstm_launch.h"

namespace mlstm_impl {

// Events of the profiling entry points, recorded on the launch stream around
// a kernel group when the call carries them (marks[2 k], marks[2 k + 1]).
inline void mark_before(const hipEvent_t* marks, int k, hipStream_t s) {
  if (marks && marks[2 * k]) (void)hipEventRecord(marks[2 * k], s);
}
inline void mark_after(const hipEvent_t* marks, int k, hipStream_t s) {
  if (marks && marks[2 * k + 1]) (void)hipEventRecord(marks[2 * k + 1], s);
}

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int kThreads = 256;   // four wave64 per workgroup
constexpr int kTile = 64;       // tokens per tile


// ------------------------------------------------------------------ scalar helpers

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// log(sigmoid(x)) = min(x, 0) - log1p(exp(-|x|)); exact 0 at +inf and -inf at -inf.
__device__ __forceinline__ float log_sigmoid(float x) {
  return fminf(x, 0.f) - log1pf(expf(-fabsf(x)));
}
__device__ __forceinline__ float sigmoid(float x) {
  const float e = expf(-fabsf(x));
  const float r = 1.f / (1.f + e);
  return x >= 0.f ? r : e * r;
}

// ------------------------------------------------------------------ MFMA traits

template <typename T> struct Frag;
template <> struct Frag<__bf16> {
  using type = bf16x8;
  static constexpr int E = 8;     // elements per lane along the contraction
  static constexpr int PAD = 8;   // LDS row padding (elements)
};
template <> struct Frag<float> {
  using type = float;
  static constexpr int E = 1;
  static constexpr int PAD = 4;
};

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ typename Frag<T>::type ld_frag(const T* p);
template <> __device__ __forceinline__ bf16x8 ld_frag<__bf16>(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ __forceinline__ float ld_frag<float>(const float* p) { return *p; }

// Operand fragment of type TI read from a state stored as TS.
template <typename TI, typename TS> struct StateFrag;
template <> struct StateFrag<__bf16, __bf16> {
  static __device__ __forceinline__ bf16x8 load(const __bf16* p) { return ld_frag<__bf16>(p); }
};
template <> struct StateFrag<__bf16, float> {
  static __device__ __forceinline__ bf16x8 load(const float* p) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
    bf16x8 r;
    r[0] = (__bf16)x0[0]; r[1] = (__bf16)x0[1]; r[2] = (__bf16)x0[2]; r[3] = (__bf16)x0[3];
    r[4] = (__bf16)x1[0]; r[5] = (__bf16)x1[1]; r[6] = (__bf16)x1[2]; r[7] = (__bf16)x1[3];
    return r;
  }
};
template <> struct StateFrag<float, float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
};

// ------------------------------------------------------------------ wave / block scans

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

// Exclusive prefix over the 256 threads of a workgroup, one value per thread.
// `sbuf` holds at least 4 elements of LDS. Contains barriers: call uniformly.
__device__ inline double block_excl_sum(double x, double* sbuf) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  double excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.0;
  if (lane == 63) sbuf[w] = incl;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < w; ++i) off += sbuf[i];
  __syncthreads();
  return off + excl;
}

__device__ inline int block_excl_max_int(int x, int* sbuf) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl = max(incl, y);
  }
  int excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = -1;
  if (lane == 63) sbuf[w] = incl;
  __syncthreads();
  int off = -1;
  for (int i = 0; i < w; ++i) off = max(off, sbuf[i]);
  __syncthreads();
  return max(off, excl);
}

// Segmented running max: a set flag restarts the max at that element.
struct SegMax {
  int f;
  double v;
};
__device__ __forceinline__ SegMax seg_combine(SegMax l, SegMax r) {
  return SegMax{l.f | r.f, r.f ? r.v : fmax(l.v, r.v)};
}

__device__ inline SegMax block_excl_segmax(SegMax x, int* sflag, double* sval) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  SegMax incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    SegMax y;
    y.f = __shfl_up(incl.f, d, 64);
    y.v = __shfl_up(incl.v, d, 64);
    if (lane >= d) incl = seg_combine(y, incl);
  }
  SegMax excl;
  excl.f = __shfl_up(incl.f, 1, 64);
  excl.v = __shfl_up(incl.v, 1, 64);
  if (lane == 0) excl = SegMax{0, -INFINITY};
  if (lane == 63) { sflag[w] = incl.f; sval[w] = incl.v; }
  __syncthreads();
  SegMax off{0, -INFINITY};
  for (int i = 0; i < w; ++i) off = seg_combine(off, SegMax{sflag[i], sval[i]});
  __syncthreads();
  return seg_combine(off, excl);
}

// ------------------------------------------------------------------ LDS staging

// Copy a [64 rows][NC cols] tile (global row pitch gp elements) into LDS
// row-major with row pitch SP; rows >= nrows become zero.
template <typename T, int NC, int SP>
__device__ __forceinline__ void stage_rows(T* __restrict__ s, const T* __restrict__ g, int64_t gp,
                                           int nrows) {
  constexpr int EV = 16 / sizeof(T);        // elements per 16-byte vector
  constexpr int VPR = NC / EV;              // vectors per row
  constexpr int ITEMS = kTile * VPR;
  for (int it = threadIdx.x; it < ITEMS; it += kThreads) {
    const int row = it / VPR, cv = it % VPR;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (row < nrows) x = *reinterpret_cast<const f32x4*>(g + (int64_t)row * gp + cv * EV);
    *reinterpret_cast<f32x4*>(s + row * SP + cv * EV) = x;
  }
}

// Copy a [64 rows][NC cols] tile into LDS transposed, s[col][row] with row
// pitch SP, multiplying row j by scale[j] when scale is given; rows >= nrows
// become zero. Each work item takes two consecutive rows of one 16-byte
// column group and writes them as element pairs.
template <int NC, int SP>
__device__ __forceinline__ void stage_transposed(__bf16* __restrict__ s, const __bf16* __restrict__ g,
                                                 int64_t gp, int nrows, const float* scale) {
  constexpr int CG = NC / 8;
  constexpr int ITEMS = (kTile / 2) * CG;
  for (int it = threadIdx.x; it < ITEMS; it += kThreads) {
    const int rp = it % (kTile / 2), cg = it / (kTile / 2);
    const int r0 = 2 * rp, r1 = r0 + 1;
    bf16x8 x0, x1;
    for (int i = 0; i < 8; ++i) { x0[i] = (__bf16)0.f; x1[i] = (__bf16)0.f; }
    if (r0 < nrows) x0 = *reinterpret_cast<const bf16x8*>(g + (int64_t)r0 * gp + cg * 8);
    if (r1 < nrows) x1 = *reinterpret_cast<const bf16x8*>(g + (int64_t)r1 * gp + cg * 8);
    if (scale) {
      const float s0 = scale[r0], s1 = scale[r1];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x0[i] = (__bf16)((float)x0[i] * s0);
        x1[i] = (__bf16)((float)x1[i] * s1);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bf16x2 pr;
      pr[0] = x0[i];
      pr[1] = x1[i];
      *reinterpret_cast<bf16x2*>(s + (cg * 8 + i) * SP + r0) = pr;
    }
  }
}

template <int NC, int SP>
__device__ __forceinline__ void stage_transposed(float* __restrict__ s, const float* __restrict__ g,
                                                 int64_t gp, int nrows, const float* scale) {
  constexpr int CG = NC / 4;
  constexpr int ITEMS = (kTile / 2) * CG;
  for (int it = threadIdx.x; it < ITEMS; it += kThreads) {
    const int rp = it % (kTile / 2), cg = it / (kTile / 2);
    const int r0 = 2 * rp, r1 = r0 + 1;
    f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
    if (r0 < nrows) x0 = *reinterpret_cast<const f32x4*>(g + (int64_t)r0 * gp + cg * 4);
    if (r1 < nrows) x1 = *reinterpret_cast<const f32x4*>(g + (int64_t)r1 * gp + cg * 4);
    if (scale) {
      x0 *= scale[r0];
      x1 *= scale[r1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x2 pr;
      pr[0] = x0[i];
      pr[1] = x1[i];
      *reinterpret_cast<f32x2*>(s + (cg * 4 + i) * SP + r0) = pr;
    }
  }
}

}  // namespace

}  // namespace mlstm_impl
