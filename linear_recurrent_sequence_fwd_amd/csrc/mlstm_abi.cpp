// C ABI of the mLSTM cell forward: argument validation, workspace layout and
// dispatch to the HIP launchers. Every check runs on the host before any HIP
// call, so invalid arguments are rejected without touching a device.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mlstm.h"
#include "../../include/mlstm_block.h"
#include "../../include/mlstm_prof.h"
#include "../../include/mlstm_segments.h"
#include "../../include/slstm.h"
#include "mlstm_launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

constexpr int64_t kMaxChunk = 8192;
constexpr int64_t kMaxParallelT = 8192;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  const char* name;
  uintptr_t lo, hi;   // [lo, hi)
};

Range make_range(const char* name, const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool overlap(const Range& a, const Range& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// Outputs must not overlap inputs or each other.
int check_alias(const std::vector<Range>& in, const std::vector<Range>& out) {
  for (size_t i = 0; i < out.size(); ++i) {
    for (const Range& r : in)
      if (overlap(out[i], r))
        return fail(MLSTM_ERR_ALIAS, std::string(out[i].name) + " overlaps input " + r.name);
    for (size_t j = i + 1; j < out.size(); ++j)
      if (overlap(out[i], out[j]))
        return fail(MLSTM_ERR_ALIAS, std::string(out[i].name) + " overlaps output " + out[j].name);
  }
  return MLSTM_OK;
}

bool fwd_dqk_supported(int64_t d_qk, int32_t dtype) {
  if (dtype == MLSTM_BF16) return d_qk == 64 || d_qk == 128 || d_qk == 256;
  return d_qk == 64 || d_qk == 128;
}

// Shape/dtype/pointer checks shared by both forward forms (not the workspace).
// `gate_optional`: o_pre may be NULL (no output gate) where the fused
// chunkwise kernels run.
int validate_fwd(const mlstm_fwd_args* a, bool gate_optional = false) {
  if (!a) return fail(MLSTM_ERR_NULLPTR, "args is NULL");
  if (a->dtype != MLSTM_FP32 && a->dtype != MLSTM_BF16)
    return fail(MLSTM_ERR_BAD_DTYPE, "dtype must be MLSTM_FP32 or MLSTM_BF16");
  if (a->B < 1 || a->H < 1 || a->T < 0 || a->d_qk < 1 || a->d_v < 1)
    return fail(MLSTM_ERR_BAD_SHAPE, "need B >= 1, H >= 1, T >= 0, d_qk >= 1, d_v >= 1");
  if (a->d_v % 64 != 0) return fail(MLSTM_ERR_BAD_SHAPE, "d_v must be a multiple of 64");
  if (a->d_qk % 64 != 0) return fail(MLSTM_ERR_BAD_SHAPE, "d_qk must be a multiple of 64");
  if (!fwd_dqk_supported(a->d_qk, a->dtype))
    return fail(MLSTM_ERR_UNSUPPORTED, "d_qk must be 64, 128 or 256 (float32: 64 or 128)");
  if (a->d_v > 16384) return fail(MLSTM_ERR_UNSUPPORTED, "d_v above 16384");
  const bool any0 = a->C0 || a->n0 || a->m0, all0 = a->C0 && a->n0 && a->m0;
  if (any0 && !all0) return fail(MLSTM_ERR_NULLPTR, "C0, n0, m0 must be given together");
  const bool anyo = a->C_out || a->n_out || a->m_out, allo = a->C_out && a->n_out && a->m_out;
  if (anyo && !allo) return fail(MLSTM_ERR_NULLPTR, "C_out, n_out, m_out must be given together");
  if (a->T > 0 && (!a->q || !a->k || !a->v || !a->i_pre || !a->f_pre || !a->h))
    return fail(MLSTM_ERR_NULLPTR, "q, k, v, i_pre, f_pre and h are required when T > 0");
  if (a->T > 0 && !a->o_pre &&
      !(gate_optional && mlstm_impl::fused_path(a->dtype == MLSTM_BF16, a->d_qk, a->d_v)))
    return fail(MLSTM_ERR_NULLPTR, "o_pre is required (it may be NULL only for the chunkwise form with "
                                   "MLSTM_BF16 and d_v a multiple of 128)");
  const void* v16[] = {a->q, a->k, a->v, a->o_pre, a->h, a->C0, a->n0, a->C_out, a->n_out};
  for (const void* p : v16)
    if (p && !aligned(p, 16)) return fail(MLSTM_ERR_MISALIGNED, "array pointers must be 16-byte aligned");
  const void* v4[] = {a->i_pre, a->f_pre, a->m0, a->m_out};
  for (const void* p : v4)
    if (p && !aligned(p, 4)) return fail(MLSTM_ERR_MISALIGNED, "gate and m pointers must be 4-byte aligned");
  const int64_t es = a->dtype == MLSTM_BF16 ? 2 : 4;
  const int64_t BH = a->B * a->H;
  const int64_t nqk = BH * a->T * a->d_qk * es, nv = BH * a->T * a->d_v * es, ng = BH * a->T * 4;
  const int64_t nC = BH * a->d_v * a->d_qk * 4, nn = BH * a->d_qk * 4, nm = BH * 4;
  std::vector<Range> in = {make_range("q", a->q, nqk), make_range("k", a->k, nqk),
                           make_range("v", a->v, nv), make_range("o_pre", a->o_pre, nv),
                           make_range("i_pre", a->i_pre, ng), make_range("f_pre", a->f_pre, ng),
                           make_range("C0", a->C0, nC), make_range("n0", a->n0, nn),
                           make_range("m0", a->m0, nm)};
  std::vector<Range> out = {make_range("h", a->h, nv), make_range("C_out", a->C_out, nC),
                            make_range("n_out", a->n_out, nn), make_range("m_out", a->m_out, nm)};
  return check_alias(in, out);
}

struct WsLayout {
  size_t u, b, mp, rs, w0, g, U, R, Cs, ns, ms, total;
  size_t Cseg, nseg, mloc, mstart, Gseg, wb;
};

WsLayout layout(int64_t BH, int64_t T, int64_t Nc, int64_t K, int64_t V, int64_t cs_elem, bool states) {
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  w.u = take(BH * T * 8);
  w.b = take(BH * T * 8);
  w.mp = take(BH * T * 8);
  w.rs = take(BH * T * 4);
  w.w0 = take(BH * T * 4);
  w.g = take(BH * Nc * 8);
  w.U = take(BH * Nc * 8);
  w.R = take(BH * Nc * 4);
  if (states) {
    w.Cs = take(BH * Nc * V * K * cs_elem);
    w.ns = take(BH * Nc * K * 4);
    w.ms = take(BH * Nc * 8);
  }
  w.total = off;
  return w;
}

// bf16 with d_v a multiple of 128 runs the fused kernels: per-64-token gate
// data, and per chunk its local end state (later its start state).
bool use_fused(const mlstm_fwd_args* a) {
  return mlstm_impl::fused_path(a->dtype == MLSTM_BF16, a->d_qk, a->d_v);
}

struct FusedShape {
  int64_t Nt, TPS, S;
};

FusedShape fused_shape(int64_t T, int chunk) {
  FusedShape f;
  f.Nt = (T + 63) / 64;
  f.TPS = chunk / 64;
  f.S = (f.Nt + f.TPS - 1) / f.TPS;
  return f;
}

// `all_chunks`: a local state for every chunk (a segment summary), not only
// for chunks 0..S-2 (the forward, whose last chunk's state the output pass
// carries itself).
WsLayout layout_fused(int64_t BH, int64_t T, int chunk, int64_t K, int64_t V, bool all_chunks = false) {
  const FusedShape fs = fused_shape(T, chunk);
  WsLayout w = layout(BH, T, fs.Nt, K, V, 4, false);
  size_t off = w.total;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  const int64_t ns = all_chunks ? fs.S : fs.S - 1;
  w.Cseg = take(BH * ns * V * K * 4);
  w.nseg = take(BH * ns * K * 4);
  w.mloc = take(BH * ns * 8);
  w.mstart = take(BH * ns * 8);
  w.Gseg = take(BH * ns * 8);
  w.wb = take(BH * fs.Nt * 3 * 64 * 2);
  w.total = off;
  return w;
}

mlstm_impl::GateBuffers gate_buffers(char* ws, const WsLayout& w) {
  mlstm_impl::GateBuffers gb;
  gb.u = reinterpret_cast<double*>(ws + w.u);
  gb.b = reinterpret_cast<double*>(ws + w.b);
  gb.mp = reinterpret_cast<double*>(ws + w.mp);
  gb.rs = reinterpret_cast<int*>(ws + w.rs);
  gb.w0 = reinterpret_cast<float*>(ws + w.w0);
  gb.wb = nullptr;
  gb.g = reinterpret_cast<double*>(ws + w.g);
  gb.U = reinterpret_cast<double*>(ws + w.U);
  gb.R = reinterpret_cast<int*>(ws + w.R);
  return gb;
}

mlstm_impl::FwdLaunch fwd_launch(const mlstm_fwd_args* a, int L, int64_t Nc,
                                 const hipEvent_t* marks = nullptr) {
  mlstm_impl::FwdLaunch f;
  f.marks = marks;
  f.BH = a->B * a->H; f.T = a->T; f.K = a->d_qk; f.V = a->d_v;
  f.L = L; f.Nc = Nc; f.bf16 = a->dtype == MLSTM_BF16;
  f.q = a->q; f.k = a->k; f.v = a->v; f.o = a->o_pre;
  f.i_pre = a->i_pre; f.f_pre = a->f_pre; f.h = a->h;
  f.C0 = a->C0; f.n0 = a->n0; f.m0 = a->m0;
  f.C_out = a->C_out; f.n_out = a->n_out; f.m_out = a->m_out;
  return f;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLSTM_OK;
  return fail(MLSTM_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int check_grid(const mlstm_fwd_args* a) {
  const int64_t BH = a->B * a->H;
  const int64_t nqt = (a->T + 63) / 64;
  if (BH * nqt * (a->d_v / 64) > INT32_MAX)
    return fail(MLSTM_ERR_UNSUPPORTED, "problem too large for one launch grid");
  return MLSTM_OK;
}

int check_workspace(const mlstm_fwd_args* a, void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MLSTM_OK;
  if (!ws) return fail(MLSTM_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, kAlign)) return fail(MLSTM_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(MLSTM_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  const int64_t es = a->dtype == MLSTM_BF16 ? 2 : 4;
  const int64_t BH = a->B * a->H;
  const int64_t nqk = BH * a->T * a->d_qk * es, nv = BH * a->T * a->d_v * es, ng = BH * a->T * 4;
  const int64_t nC = BH * a->d_v * a->d_qk * 4, nn = BH * a->d_qk * 4, nm = BH * 4;
  std::vector<Range> other = {make_range("q", a->q, nqk), make_range("k", a->k, nqk),
                              make_range("v", a->v, nv), make_range("o_pre", a->o_pre, nv),
                              make_range("i_pre", a->i_pre, ng), make_range("f_pre", a->f_pre, ng),
                              make_range("C0", a->C0, nC), make_range("n0", a->n0, nn),
                              make_range("m0", a->m0, nm), make_range("h", a->h, nv),
                              make_range("C_out", a->C_out, nC), make_range("n_out", a->n_out, nn),
                              make_range("m_out", a->m_out, nm)};
  const Range wr = make_range("workspace", ws, (int64_t)need);
  for (const Range& r : other)
    if (overlap(wr, r)) return fail(MLSTM_ERR_ALIAS, std::string("workspace overlaps ") + r.name);
  return MLSTM_OK;
}

}  // namespace

extern "C" {

size_t mlstm_fwd_chunkwise_workspace_size(const mlstm_fwd_args* a, int chunk) {
  if (!a || a->T <= 0 || chunk < 64 || chunk % 64 != 0 || chunk > kMaxChunk) return 0;
  if (a->B < 1 || a->H < 1 || a->d_qk < 1 || a->d_v < 1) return 0;
  if (use_fused(a)) return layout_fused(a->B * a->H, a->T, chunk, a->d_qk, a->d_v).total;
  const int64_t Nc = (a->T + chunk - 1) / chunk;
  return layout(a->B * a->H, a->T, Nc, a->d_qk, a->d_v, 4, true).total;
}

}  // extern "C"

namespace {

int fwd_chunkwise(const mlstm_fwd_args* a, int chunk, void* workspace, size_t workspace_bytes,
                  void* stream, const hipEvent_t* marks) {
  g_last_error.clear();
  int st = validate_fwd(a, true);
  if (st) return st;
  if (chunk < 64 || chunk % 64 != 0 || chunk > kMaxChunk)
    return fail(MLSTM_ERR_BAD_SHAPE, "chunk must be a multiple of 64 in [64, 8192]");
  if ((st = check_grid(a))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t Nc = a->T > 0 ? (a->T + chunk - 1) / chunk : 0;
  mlstm_impl::FwdLaunch f = fwd_launch(a, chunk, Nc, marks);
  if (a->T == 0) return hip_status(mlstm_impl::launch_copy_state(f, s), "state copy");
  const size_t need = mlstm_fwd_chunkwise_workspace_size(a, chunk);
  if ((st = check_workspace(a, workspace, workspace_bytes, need))) return st;
  char* ws = static_cast<char*>(workspace);
  if (use_fused(a)) {
    const FusedShape fs = fused_shape(a->T, chunk);
    const mlstm_impl::FwdLaunch ft = fwd_launch(a, 64, fs.Nt, marks);
    const WsLayout w = layout_fused(ft.BH, ft.T, chunk, ft.K, ft.V);
    mlstm_impl::GateBuffers gb = gate_buffers(ws, w);
    gb.wb = reinterpret_cast<uint16_t*>(ws + w.wb);
    mlstm_impl::SegStates ss;
    ss.C = reinterpret_cast<float*>(ws + w.Cseg);
    ss.n = reinterpret_cast<float*>(ws + w.nseg);
    ss.mloc = reinterpret_cast<double*>(ws + w.mloc);
    ss.mstart = reinterpret_cast<double*>(ws + w.mstart);
    ss.G = reinterpret_cast<double*>(ws + w.Gseg);
    ss.S = (int)fs.S;
    ss.TPS = (int)fs.TPS;
    if ((st = hip_status(mlstm_impl::launch_gate(ft, gb, s), "gate kernel"))) return st;
    return hip_status(mlstm_impl::launch_fused(ft, gb, ss, s), "fused kernels");
  }
  const WsLayout w = layout(f.BH, f.T, Nc, f.K, f.V, 4, true);
  const mlstm_impl::GateBuffers gb = gate_buffers(ws, w);
  mlstm_impl::ChunkStates cs;
  cs.Cs = ws + w.Cs;
  cs.ns = reinterpret_cast<float*>(ws + w.ns);
  cs.ms = reinterpret_cast<double*>(ws + w.ms);
  if ((st = hip_status(mlstm_impl::launch_gate(f, gb, s), "gate kernel"))) return st;
  if ((st = hip_status(mlstm_impl::launch_state(f, gb, cs, s), "state kernel"))) return st;
  return hip_status(mlstm_impl::launch_out(f, gb, cs, s), "output kernel");
}

}  // namespace

extern "C" {

int mlstm_fwd_chunkwise(const mlstm_fwd_args* a, int chunk, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return fwd_chunkwise(a, chunk, workspace, workspace_bytes, stream, nullptr);
}

size_t mlstm_fwd_parallel_workspace_size(const mlstm_fwd_args* a) {
  if (!a || a->T <= 0 || a->B < 1 || a->H < 1) return 0;
  return layout(a->B * a->H, a->T, 1, a->d_qk, a->d_v, 4, false).total;
}

int mlstm_fwd_parallel(const mlstm_fwd_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = validate_fwd(a);
  if (st) return st;
  if (a->T > kMaxParallelT) return fail(MLSTM_ERR_UNSUPPORTED, "parallel form needs T <= 8192");
  if ((st = check_grid(a))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int L = (int)((a->T + 63) / 64 * 64);
  mlstm_impl::FwdLaunch f = fwd_launch(a, L > 0 ? L : 64, a->T > 0 ? 1 : 0);
  if (a->T == 0) return hip_status(mlstm_impl::launch_copy_state(f, s), "state copy");
  const size_t need = mlstm_fwd_parallel_workspace_size(a);
  if ((st = check_workspace(a, workspace, workspace_bytes, need))) return st;
  char* ws = static_cast<char*>(workspace);
  const WsLayout w = layout(f.BH, f.T, 1, f.K, f.V, 4, false);
  const mlstm_impl::GateBuffers gb = gate_buffers(ws, w);
  mlstm_impl::ChunkStates none{nullptr, nullptr, nullptr};
  if ((st = hip_status(mlstm_impl::launch_gate(f, gb, s), "gate kernel"))) return st;
  if ((st = hip_status(mlstm_impl::launch_out(f, gb, none, s), "output kernel"))) return st;
  if (a->C_out) return hip_status(mlstm_impl::launch_state(f, gb, none, s), "state kernel");
  return MLSTM_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ backward pass

namespace {

struct BwdLayout {
  WsLayout fw;   // gate prefix data and the forward's chunk-start states
  size_t G, dz, qdq, Es, es, Ms, L0, L0e, total;
};

BwdLayout layout_bwd(int64_t BH, int64_t T, int64_t Nc, int64_t K, int64_t V, int64_t elem) {
  BwdLayout b;
  b.fw = layout(BH, T, Nc, K, V, elem, true);   // chunk-start states in the input dtype
  size_t off = b.fw.total;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  b.G = take(BH * T * V * elem);
  b.dz = take(BH * T * 4);
  b.qdq = take(BH * T * 4);
  b.Es = take(BH * Nc * V * K * 4);
  b.es = take(BH * Nc * K * 4);
  b.Ms = take(BH * Nc * 8);
  b.L0 = take(BH * V * K * 4);
  b.L0e = take(BH * K * 4);
  b.total = off;
  return b;
}

int validate_bwd(const mlstm_bwd_args* a, int chunk) {
  if (!a) return fail(MLSTM_ERR_NULLPTR, "args is NULL");
  if (a->dtype != MLSTM_FP32 && a->dtype != MLSTM_BF16)
    return fail(MLSTM_ERR_BAD_DTYPE, "dtype must be MLSTM_FP32 or MLSTM_BF16");
  if (a->B < 1 || a->H < 1 || a->T < 0 || a->d_qk < 1 || a->d_v < 1)
    return fail(MLSTM_ERR_BAD_SHAPE, "need B >= 1, H >= 1, T >= 0, d_qk >= 1, d_v >= 1");
  if (chunk < 64 || chunk % 64 != 0 || chunk > kMaxChunk)
    return fail(MLSTM_ERR_BAD_SHAPE, "chunk must be a multiple of 64 in [64, 8192]");
  if (a->d_qk % 64 != 0 || a->d_v % 64 != 0)
    return fail(MLSTM_ERR_BAD_SHAPE, "d_qk and d_v must be multiples of 64");
  if (!mlstm_impl::bwd_supported(a->dtype == MLSTM_BF16, a->d_qk, a->d_v))
    return fail(MLSTM_ERR_UNSUPPORTED,
                "backward shapes: bf16 d_qk in {64,128,256}, d_v in {64,128,256,512}; "
                "fp32 d_qk in {64,128}, d_v in {64,128,256}");
  const bool any0 = a->C0 || a->n0 || a->m0, all0 = a->C0 && a->n0 && a->m0;
  if (any0 && !all0) return fail(MLSTM_ERR_NULLPTR, "C0, n0, m0 must be given together");
  const bool anyd = a->dC0 || a->dn0 || a->dm0, alld = a->dC0 && a->dn0 && a->dm0;
  if (anyd && !alld) return fail(MLSTM_ERR_NULLPTR, "dC0, dn0, dm0 must be given together");
  if (a->T > 0 && (!a->q || !a->k || !a->v || !a->o_pre || !a->i_pre || !a->f_pre || !a->h || !a->dh ||
                   !a->dq || !a->dk || !a->dv || !a->do_pre || !a->di_pre || !a->df_pre))
    return fail(MLSTM_ERR_NULLPTR, "inputs, h, dh and the six gradient outputs are required when T > 0");
  const void* v16[] = {a->q, a->k, a->v, a->o_pre, a->h, a->dh, a->dq, a->dk, a->dv, a->do_pre,
                       a->C0, a->n0, a->dC0, a->dn0};
  for (const void* p : v16)
    if (p && !aligned(p, 16)) return fail(MLSTM_ERR_MISALIGNED, "array pointers must be 16-byte aligned");
  const void* v4[] = {a->i_pre, a->f_pre, a->m0, a->di_pre, a->df_pre, a->dm0};
  for (const void* p : v4)
    if (p && !aligned(p, 4)) return fail(MLSTM_ERR_MISALIGNED, "gate and m pointers must be 4-byte aligned");
  const int64_t BH = a->B * a->H;
  if (BH * ((a->T + 63) / 64) > INT32_MAX || BH * (a->d_qk / 64) * (a->d_v / 64) > INT32_MAX)
    return fail(MLSTM_ERR_UNSUPPORTED, "problem too large for one launch grid");
  const int64_t es = a->dtype == MLSTM_BF16 ? 2 : 4;
  const int64_t nqk = BH * a->T * a->d_qk * es, nv = BH * a->T * a->d_v * es, ng = BH * a->T * 4;
  const int64_t nC = BH * a->d_v * a->d_qk * 4, nn = BH * a->d_qk * 4, nm = BH * 4;
  std::vector<Range> in = {make_range("q", a->q, nqk), make_range("k", a->k, nqk),
                           make_range("v", a->v, nv), make_range("o_pre", a->o_pre, nv),
                           make_range("i_pre", a->i_pre, ng), make_range("f_pre", a->f_pre, ng),
                           make_range("h", a->h, nv), make_range("dh", a->dh, nv),
                           make_range("C0", a->C0, nC), make_range("n0", a->n0, nn),
                           make_range("m0", a->m0, nm)};
  std::vector<Range> out = {make_range("dq", a->dq, nqk), make_range("dk", a->dk, nqk),
                            make_range("dv", a->dv, nv), make_range("do_pre", a->do_pre, nv),
                            make_range("di_pre", a->di_pre, ng), make_range("df_pre", a->df_pre, ng),
                            make_range("dC0", a->dC0, nC), make_range("dn0", a->dn0, nn),
                            make_range("dm0", a->dm0, nm)};
  int st = check_alias(in, out);
  if (st) return st;
  return MLSTM_OK;
}

size_t bwd_workspace_size(const mlstm_bwd_args* a, int chunk) {
  if (!a || a->T <= 0 || chunk < 64 || chunk % 64 != 0 || chunk > kMaxChunk) return 0;
  if (a->B < 1 || a->H < 1 || a->d_qk < 1 || a->d_v < 1) return 0;
  const int64_t Nc = (a->T + chunk - 1) / chunk;
  return layout_bwd(a->B * a->H, a->T, Nc, a->d_qk, a->d_v, a->dtype == MLSTM_BF16 ? 2 : 4).total;
}

int bwd_chunkwise(const mlstm_bwd_args* a, int chunk, void* workspace, size_t workspace_bytes, void* stream,
                  const hipEvent_t* marks) {
  g_last_error.clear();
  int st = validate_bwd(a, chunk);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t BH = a->B * a->H;
  const int64_t Nc = a->T > 0 ? (a->T + chunk - 1) / chunk : 0;
  mlstm_impl::BwdLaunch b;
  b.BH = BH; b.T = a->T; b.K = a->d_qk; b.V = a->d_v; b.L = chunk; b.Nc = Nc;
  b.bf16 = a->dtype == MLSTM_BF16;
  b.q = a->q; b.k = a->k; b.v = a->v; b.o = a->o_pre; b.h = a->h; b.dh = a->dh;
  b.i_pre = a->i_pre; b.f_pre = a->f_pre;
  b.dq = a->dq; b.dk = a->dk; b.dv = a->dv; b.dout = a->do_pre; b.di = a->di_pre; b.df = a->df_pre;
  b.C0 = a->C0; b.n0 = a->n0; b.m0 = a->m0;
  b.dC0 = a->dC0; b.dn0 = a->dn0; b.dm0 = a->dm0;
  b.marks = marks;
  const mlstm_impl::GateBuffers none_gb{};
  const mlstm_impl::ChunkStates none_cs{nullptr, nullptr, nullptr};
  const mlstm_impl::BwdBuffers none_bb{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (a->T == 0) return hip_status(mlstm_impl::launch_bwd(b, none_gb, none_cs, none_bb, s), "backward");
  const size_t need = bwd_workspace_size(a, chunk);
  if (!workspace) return fail(MLSTM_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, kAlign)) return fail(MLSTM_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(MLSTM_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  {
    const int64_t es = b.bf16 ? 2 : 4;
    const int64_t nqk = BH * a->T * a->d_qk * es, nv = BH * a->T * a->d_v * es, ng = BH * a->T * 4;
    const int64_t nC = BH * a->d_v * a->d_qk * 4, nn = BH * a->d_qk * 4, nm = BH * 4;
    const Range wr = make_range("workspace", workspace, (int64_t)need);
    const Range other[] = {make_range("q", a->q, nqk), make_range("k", a->k, nqk), make_range("v", a->v, nv),
                           make_range("o_pre", a->o_pre, nv), make_range("i_pre", a->i_pre, ng),
                           make_range("f_pre", a->f_pre, ng), make_range("h", a->h, nv),
                           make_range("dh", a->dh, nv), make_range("C0", a->C0, nC),
                           make_range("n0", a->n0, nn), make_range("m0", a->m0, nm),
                           make_range("dq", a->dq, nqk), make_range("dk", a->dk, nqk),
                           make_range("dv", a->dv, nv), make_range("do_pre", a->do_pre, nv),
                           make_range("di_pre", a->di_pre, ng), make_range("df_pre", a->df_pre, ng),
                           make_range("dC0", a->dC0, nC), make_range("dn0", a->dn0, nn),
                           make_range("dm0", a->dm0, nm)};
    for (const Range& r : other)
      if (overlap(wr, r)) return fail(MLSTM_ERR_ALIAS, std::string("workspace overlaps ") + r.name);
  }
  char* ws = static_cast<char*>(workspace);
  const BwdLayout w = layout_bwd(BH, a->T, Nc, a->d_qk, a->d_v, b.bf16 ? 2 : 4);
  const mlstm_impl::GateBuffers gb = gate_buffers(ws, w.fw);
  mlstm_impl::ChunkStates cs;
  cs.Cs = ws + w.fw.Cs;
  cs.ns = reinterpret_cast<float*>(ws + w.fw.ns);
  cs.ms = reinterpret_cast<double*>(ws + w.fw.ms);
  cs.cs_bf16 = b.bf16;
  mlstm_impl::BwdBuffers bb;
  bb.G = ws + w.G;
  bb.dz = reinterpret_cast<float*>(ws + w.dz);
  bb.qdq = reinterpret_cast<float*>(ws + w.qdq);
  bb.Es = ws + w.Es;
  bb.es = reinterpret_cast<float*>(ws + w.es);
  bb.Ms = reinterpret_cast<double*>(ws + w.Ms);
  bb.L0 = reinterpret_cast<float*>(ws + w.L0);
  bb.L0e = reinterpret_cast<float*>(ws + w.L0e);
  // the forward's gate prefix sums and chunk-start states (the K_GATE and
  // K_STATE event slots coincide with the backward's first two groups)
  mlstm_impl::FwdLaunch f{};
  f.BH = BH; f.T = a->T; f.K = a->d_qk; f.V = a->d_v; f.L = chunk; f.Nc = Nc; f.bf16 = b.bf16;
  f.q = a->q; f.k = a->k; f.v = a->v; f.o = a->o_pre;
  f.i_pre = a->i_pre; f.f_pre = a->f_pre; f.h = nullptr;
  f.C0 = a->C0; f.n0 = a->n0; f.m0 = a->m0;
  f.C_out = nullptr; f.n_out = nullptr; f.m_out = nullptr;
  f.marks = marks;
  if ((st = hip_status(mlstm_impl::launch_gate(f, gb, s), "gate kernel"))) return st;
  if ((st = hip_status(mlstm_impl::launch_state(f, gb, cs, s), "state kernel"))) return st;
  return hip_status(mlstm_impl::launch_bwd(b, gb, cs, bb, s), "backward kernels");
}

}  // namespace

extern "C" {

size_t mlstm_bwd_chunkwise_workspace_size(const mlstm_bwd_args* a, int chunk) {
  return bwd_workspace_size(a, chunk);
}

int mlstm_bwd_chunkwise(const mlstm_bwd_args* a, int chunk, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return bwd_chunkwise(a, chunk, workspace, workspace_bytes, stream, nullptr);
}

int mlstm_prof_bwd_chunkwise(const mlstm_bwd_args* a, int chunk, void* workspace, size_t workspace_bytes,
                             void* stream, void* const* events) {
  if (!events) return fail(MLSTM_ERR_NULLPTR, "events is NULL");
  hipEvent_t marks[2 * mlstm_impl::B_COUNT] = {};
  for (int x = 0; x < 2 * mlstm_impl::B_COUNT; ++x) marks[x] = static_cast<hipEvent_t>(events[x]);
  return bwd_chunkwise(a, chunk, workspace, workspace_bytes, stream, marks);
}

}  // extern "C"

namespace {

int step(const mlstm_step_args* a, void* stream, const hipEvent_t* marks) {
  g_last_error.clear();
  if (!a) return fail(MLSTM_ERR_NULLPTR, "args is NULL");
  if (a->dtype != MLSTM_FP32 && a->dtype != MLSTM_BF16)
    return fail(MLSTM_ERR_BAD_DTYPE, "dtype must be MLSTM_FP32 or MLSTM_BF16");
  if (a->B < 1 || a->H < 1 || a->d_qk < 1 || a->d_v < 1)
    return fail(MLSTM_ERR_BAD_SHAPE, "need B, H, d_qk, d_v >= 1");
  if (a->d_qk % 64 != 0) return fail(MLSTM_ERR_BAD_SHAPE, "d_qk must be a multiple of 64");
  if (a->d_qk > 512) return fail(MLSTM_ERR_UNSUPPORTED, "d_qk above 512");
  if (!a->q || !a->k || !a->v || !a->o_pre || !a->i_pre || !a->f_pre || !a->C || !a->n_in ||
      !a->m_in || !a->n_out || !a->m_out || !a->h)
    return fail(MLSTM_ERR_NULLPTR, "every pointer of a step is required");
  const void* v16[] = {a->C, a->n_in, a->n_out};
  for (const void* p : v16)
    if (!aligned(p, 16)) return fail(MLSTM_ERR_MISALIGNED, "C, n_in, n_out must be 16-byte aligned");
  const int64_t es = a->dtype == MLSTM_BF16 ? 2 : 4;
  const void* ve[] = {a->q, a->k, a->v, a->o_pre, a->h};
  for (const void* p : ve)
    if (!aligned(p, es)) return fail(MLSTM_ERR_MISALIGNED, "q, k, v, o_pre, h must be element-aligned");
  const void* v4[] = {a->i_pre, a->f_pre, a->m_in, a->m_out};
  for (const void* p : v4)
    if (!aligned(p, 4)) return fail(MLSTM_ERR_MISALIGNED, "gate and m pointers must be 4-byte aligned");
  const int64_t BH = a->B * a->H;
  if (BH * ((a->d_v + 31) / 32) > INT32_MAX) return fail(MLSTM_ERR_UNSUPPORTED, "too many heads");
  const int64_t nqk = BH * a->d_qk * es, nv = BH * a->d_v * es, ng = BH * 4;
  const int64_t nC = BH * a->d_v * a->d_qk * 4, nn = BH * a->d_qk * 4;
  std::vector<Range> in = {make_range("q", a->q, nqk), make_range("k", a->k, nqk),
                           make_range("v", a->v, nv), make_range("o_pre", a->o_pre, nv),
                           make_range("i_pre", a->i_pre, ng), make_range("f_pre", a->f_pre, ng),
                           make_range("n_in", a->n_in, nn), make_range("m_in", a->m_in, ng)};
  std::vector<Range> out = {make_range("h", a->h, nv), make_range("C", a->C, nC),
                            make_range("n_out", a->n_out, nn), make_range("m_out", a->m_out, ng)};
  int st = check_alias(in, out);
  if (st) return st;
  mlstm_impl::StepLaunch sl;
  sl.BH = BH; sl.K = a->d_qk; sl.V = a->d_v; sl.bf16 = a->dtype == MLSTM_BF16;
  sl.q = a->q; sl.k = a->k; sl.v = a->v; sl.o = a->o_pre;
  sl.i_pre = a->i_pre; sl.f_pre = a->f_pre;
  sl.C = a->C; sl.n_in = a->n_in; sl.m_in = a->m_in; sl.n_out = a->n_out; sl.m_out = a->m_out;
  sl.h = a->h;
  sl.marks = marks;
  return hip_status(mlstm_impl::launch_step(sl, static_cast<hipStream_t>(stream)), "step kernel");
}

}  // namespace

extern "C" {

int mlstm_step(const mlstm_step_args* a, void* stream) { return step(a, stream, nullptr); }

int slstm_fwd(const slstm_fwd_args* a, void* stream) {
  g_last_error.clear();
  if (!a) return fail(MLSTM_ERR_NULLPTR, "args is NULL");
  if (a->B < 1 || a->H < 1 || a->T < 0 || a->D < 1)
    return fail(MLSTM_ERR_BAD_SHAPE, "need B >= 1, H >= 1, T >= 0, D >= 1");
  if (!mlstm_impl::slstm_supported(a->D)) return fail(MLSTM_ERR_UNSUPPORTED, "D must be 16, 32, 64 or 128");
  if (a->B * a->H > INT32_MAX) return fail(MLSTM_ERR_UNSUPPORTED, "B * H above 2^31 - 1");
  const bool any0 = a->c0 || a->n0 || a->m0 || a->h0, all0 = a->c0 && a->n0 && a->m0 && a->h0;
  if (any0 && !all0) return fail(MLSTM_ERR_NULLPTR, "c0, n0, m0, h0 must be given together");
  const bool anyo = a->c_out || a->n_out || a->m_out || a->h_out;
  const bool allo = a->c_out && a->n_out && a->m_out && a->h_out;
  if (anyo && !allo) return fail(MLSTM_ERR_NULLPTR, "c_out, n_out, m_out, h_out must be given together");
  if (!a->R) return fail(MLSTM_ERR_NULLPTR, "R is required");
  if (a->T > 0 && (!a->pre || !a->h)) return fail(MLSTM_ERR_NULLPTR, "pre and h are required when T > 0");
  const void* v16[] = {a->pre, a->R, a->h, a->c0, a->n0, a->m0, a->h0, a->c_out, a->n_out, a->m_out, a->h_out};
  for (const void* p : v16)
    if (p && !aligned(p, 16)) return fail(MLSTM_ERR_MISALIGNED, "array pointers must be 16-byte aligned");
  const int64_t BH = a->B * a->H, D = a->D;
  const int64_t npre = BH * a->T * 4 * D * 4, nR = a->H * 4 * D * D * 4, nh = BH * a->T * D * 4, ns = BH * D * 4;
  std::vector<Range> in = {make_range("pre", a->pre, npre), make_range("R", a->R, nR),
                           make_range("c0", a->c0, ns), make_range("n0", a->n0, ns),
                           make_range("m0", a->m0, ns), make_range("h0", a->h0, ns)};
  std::vector<Range> out = {make_range("h", a->h, nh), make_range("c_out", a->c_out, ns),
                            make_range("n_out", a->n_out, ns), make_range("m_out", a->m_out, ns),
                            make_range("h_out", a->h_out, ns)};
  int st = check_alias(in, out);
  if (st) return st;
  if (a->T == 0 && !a->c_out) return MLSTM_OK;
  mlstm_impl::SlstmLaunch sl;
  sl.B = a->B; sl.H = a->H; sl.T = a->T; sl.D = D;
  sl.pre = a->pre; sl.R = a->R; sl.h = a->h;
  sl.c0 = a->c0; sl.n0 = a->n0; sl.m0 = a->m0; sl.h0 = a->h0;
  sl.c_out = a->c_out; sl.n_out = a->n_out; sl.m_out = a->m_out; sl.h_out = a->h_out;
  return hip_status(mlstm_impl::launch_slstm(sl, static_cast<hipStream_t>(stream)), "sLSTM kernel");
}

const char* mlstm_status_string(int status) {
  switch (status) {
    case MLSTM_OK: return "MLSTM_OK";
    case MLSTM_ERR_NULLPTR: return "MLSTM_ERR_NULLPTR";
    case MLSTM_ERR_BAD_SHAPE: return "MLSTM_ERR_BAD_SHAPE";
    case MLSTM_ERR_BAD_DTYPE: return "MLSTM_ERR_BAD_DTYPE";
    case MLSTM_ERR_MISALIGNED: return "MLSTM_ERR_MISALIGNED";
    case MLSTM_ERR_ALIAS: return "MLSTM_ERR_ALIAS";
    case MLSTM_ERR_WORKSPACE: return "MLSTM_ERR_WORKSPACE";
    case MLSTM_ERR_UNSUPPORTED: return "MLSTM_ERR_UNSUPPORTED";
    case MLSTM_ERR_HIP: return "MLSTM_ERR_HIP";
  }
  return "MLSTM_ERR_UNKNOWN";
}

const char* mlstm_last_error(void) { return g_last_error.c_str(); }

int mlstm_abi_version(void) { return MLSTM_ABI_VERSION; }

int mlstm_clock_probe(unsigned long long* ticks, int iters, void* stream) {
  if (!ticks) return fail(MLSTM_ERR_NULLPTR, "ticks is required");
  if (iters < 1 || iters > (1 << 24)) return fail(MLSTM_ERR_BAD_SHAPE, "iters must be in [1, 2^24]");
  if (reinterpret_cast<uintptr_t>(ticks) % 8) return fail(MLSTM_ERR_MISALIGNED, "ticks must be 8-byte aligned");
  return hip_status(mlstm_impl::launch_clock_probe(ticks, iters, static_cast<hipStream_t>(stream)), "clock probe");
}

int mlstm_prof_copy_lds(const void* src, void* dst, size_t bytes, void* stream) {
  g_last_error.clear();
  if (!src || !dst) return fail(MLSTM_ERR_NULLPTR, "src and dst are required");
  if (bytes == 0 || bytes % 16384 != 0) return fail(MLSTM_ERR_BAD_SHAPE, "bytes must be a positive multiple of 16384");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(MLSTM_ERR_MISALIGNED, "src and dst must be 16-byte aligned");
  if (overlap(make_range("src", src, (int64_t)bytes), make_range("dst", dst, (int64_t)bytes)))
    return fail(MLSTM_ERR_ALIAS, "dst overlaps src");
  return hip_status(mlstm_impl::launch_lds_copy(src, dst, (int64_t)bytes, static_cast<hipStream_t>(stream)),
                    "direct-to-LDS copy");
}

int mlstm_prof_fwd_chunkwise(const mlstm_fwd_args* a, int chunk, void* workspace, size_t workspace_bytes,
                             void* stream, void* const* events) {
  if (!events) return fail(MLSTM_ERR_NULLPTR, "events is NULL");
  hipEvent_t marks[2 * mlstm_impl::K_COUNT] = {};
  for (int g = 0; g < 3; ++g) {
    marks[2 * g] = static_cast<hipEvent_t>(events[2 * g]);
    marks[2 * g + 1] = static_cast<hipEvent_t>(events[2 * g + 1]);
  }
  return fwd_chunkwise(a, chunk, workspace, workspace_bytes, stream, marks);
}

int mlstm_prof_step(const mlstm_step_args* a, void* stream, void* before, void* after) {
  hipEvent_t marks[2 * mlstm_impl::K_COUNT] = {};
  marks[2 * mlstm_impl::K_STEP] = static_cast<hipEvent_t>(before);
  marks[2 * mlstm_impl::K_STEP + 1] = static_cast<hipEvent_t>(after);
  return step(a, stream, marks);
}

}  // extern "C"

// ------------------------------------------------------------------ no-allocation entry point
//
// Scratch of mlstm_fwd_chunkwise_noalloc: a file-scope device array that
// every GPU the library runs on holds, at its own address, until the process
// ends. Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept
// in a per-device table. Every call on a GPU shares that GPU's array.

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device of `stream` (the current
// device for the null stream), looked up on the first call for that device.
int scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLSTM_ERR_HIP, std::string("device of the stream: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLSTM_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess)
      return fail(MLSTM_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(MLSTM_ERR_HIP, std::string("hipSetDevice: ") + hipGetErrorString(e));
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr)
      return fail(MLSTM_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MLSTM_OK;
}

}  // namespace

extern "C" {

size_t mlstm_fwd_chunkwise_noalloc_limit(void) { return kScratchBytes; }

int mlstm_fwd_chunkwise_noalloc(const mlstm_fwd_args* a, int chunk, void* stream) {
  g_last_error.clear();
  int st = validate_fwd(a, true);
  if (st) return st;
  if (chunk < 64 || chunk % 64 != 0 || chunk > kMaxChunk)
    return fail(MLSTM_ERR_BAD_SHAPE, "chunk must be a multiple of 64 in [64, 8192]");
  const size_t need = mlstm_fwd_chunkwise_workspace_size(a, chunk);
  if (need > kScratchBytes)
    return fail(MLSTM_ERR_UNSUPPORTED, "this call needs " + std::to_string(need) +
                                           " bytes of scratch, above the 64 MiB of the no-allocation entry "
                                           "point (use mlstm_fwd_chunkwise with a workspace, or a longer chunk)");
  void* ws = nullptr;
  if (need > 0 && (st = scratch_for_stream(static_cast<hipStream_t>(stream), &ws))) return st;
  return fwd_chunkwise(a, chunk, ws, kScratchBytes, stream, nullptr);
}

}  // extern "C"

// ------------------------------------------------------------------ mLSTM block around the cell

namespace {

bool a16(const void* p) { return p && aligned(p, 16); }

// Bytes an operand of a strided batch can reach, from its base pointer.
Range batch_span(const char* name, const void* p, int64_t es, int64_t nb1, int64_t s1, int64_t nb2, int64_t s2,
                 int64_t rows, int64_t ld, int64_t cols) {
  if (!p || rows <= 0 || cols <= 0) return make_range(name, p, 0);
  const int64_t last = (nb1 - 1) * s1 + (nb2 - 1) * s2 + (rows - 1) * ld + cols;
  return make_range(name, p, last * es);
}

int validate_gemm(const mlstm_gemm_args* g) {
  if (!g) return fail(MLSTM_ERR_NULLPTR, "args is NULL");
  if (g->M < 1 || g->N < 1 || g->K < 1 || g->batch1 < 1 || g->batch2 < 1)
    return fail(MLSTM_ERR_BAD_SHAPE, "need M, N, K, batch1, batch2 >= 1");
  if (g->c_dtype != MLSTM_BF16 && g->c_dtype != MLSTM_FP32)
    return fail(MLSTM_ERR_BAD_DTYPE, "c_dtype must be MLSTM_BF16 or MLSTM_FP32");
  if (g->K % 64) return fail(MLSTM_ERR_BAD_SHAPE, "K must be a multiple of 64");
  if (g->N % 4) return fail(MLSTM_ERR_BAD_SHAPE, "N must be a multiple of 4");
  if (g->c_trans && g->M % 4) return fail(MLSTM_ERR_BAD_SHAPE, "M must be a multiple of 4 with c_trans");
  if (g->c_trans && g->R) return fail(MLSTM_ERR_UNSUPPORTED, "R is not supported with c_trans");
  if (!g->A || !g->B || !g->C) return fail(MLSTM_ERR_NULLPTR, "A, B and C are required");
  if (g->lda < g->K || g->ldb < g->K || g->ldc < (g->c_trans ? g->M : g->N) || (g->R && g->ldr < g->N))
    return fail(MLSTM_ERR_BAD_SHAPE, "row pitches must cover the rows (lda, ldb >= K; ldc >= N, or M with "
                                     "c_trans; ldr >= N)");
  // every row starts 16-byte aligned: bf16 pitches are multiples of 8 elements, float32 ones of 4
  const int64_t pitches[] = {g->lda, g->ldb, g->R ? g->ldr : 0, g->strideA1, g->strideA2,
                             g->strideB1, g->strideB2, g->R ? g->strideR1 : 0, g->R ? g->strideR2 : 0};
  for (int64_t v : pitches)
    if (v < 0 || v % 8) return fail(MLSTM_ERR_MISALIGNED, "pitches and batch strides of A, B and R must be "
                                                          "non-negative multiples of 8 elements");
  const int64_t cmul = g->c_dtype == MLSTM_BF16 ? 8 : 4;
  for (int64_t v : {g->ldc, g->strideC1, g->strideC2})
    if (v < 0 || v % cmul) return fail(MLSTM_ERR_MISALIGNED, "pitch and batch strides of C must be non-negative "
                                                             "multiples of 16 bytes");
  if (g->bias && (g->stride_bias2 < 0 || g->stride_bias2 % 4))
    return fail(MLSTM_ERR_MISALIGNED, "stride_bias2 must be a non-negative multiple of 4");
  const void* ptrs[] = {g->A, g->B, g->C, g->bias, g->R};
  for (const void* p : ptrs)
    if (p && !aligned(p, 16)) return fail(MLSTM_ERR_MISALIGNED, "arrays must be 16-byte aligned");
  const int64_t tile = mlstm_impl::gemm_tile();
  // the kernel forms a tile's byte range (256 rows of lda or ldb elements) and
  // its load offsets in 32 bits: row pitches up to 2^21 elements keep them below 2^31
  if (g->M > INT32_MAX / 2 || g->N > INT32_MAX / 2 || g->K > INT32_MAX / 2 ||
      g->lda > (int64_t)1 << 21 || g->ldb > (int64_t)1 << 21)
    return fail(MLSTM_ERR_UNSUPPORTED, "sizes or row pitches beyond the kernel's 32-bit offsets");
  const int64_t tiles = g->batch1 * g->batch2 * ((g->M + tile - 1) / tile) * ((g->N + tile - 1) / tile);
  if (tiles > INT32_MAX) return fail(MLSTM_ERR_UNSUPPORTED, "problem too large for one launch grid");
  const int64_t ces = g->c_dtype == MLSTM_BF16 ? 2 : 4;
  std::vector<Range> in = {
      batch_span("A", g->A, 2, g->batch1, g->strideA1, g->batch2, g->strideA2, g->M, g->lda, g->K),
      batch_span("B", g->B, 2, g->batch1, g->strideB1, g->batch2, g->strideB2, g->N, g->ldb, g->K),
      batch_span("bias", g->bias, 4, 1, 0, g->batch2, g->stride_bias2, 1, 0, g->N),
      batch_span("R", g->R, 2, g->batch1, g->strideR1, g->batch2, g->strideR2, g->M, g->ldr, g->N)};
  std::vector<Range> out = {g->c_trans
      ? batch_span("C", g->C, ces, g->batch1, g->strideC1, g->batch2, g->strideC2, g->N, g->ldc, g->M)
      : batch_span("C", g->C, ces, g->batch1, g->strideC1, g->batch2, g->strideC2, g->M, g->ldc, g->N)};
  return check_alias(in, out);
}

mlstm_impl::GemmLaunch gemm_launch(const mlstm_gemm_args* g) {
  mlstm_impl::GemmLaunch l;
  l.M = g->M; l.N = g->N; l.K = g->K; l.nb1 = g->batch1; l.nb2 = g->batch2;
  l.A = g->A; l.lda = g->lda; l.sA1 = g->strideA1; l.sA2 = g->strideA2;
  l.B = g->B; l.ldb = g->ldb; l.sB1 = g->strideB1; l.sB2 = g->strideB2;
  l.C = g->C; l.ldc = g->ldc; l.sC1 = g->strideC1; l.sC2 = g->strideC2;
  l.c_fp32 = g->c_dtype == MLSTM_FP32; l.c_trans = g->c_trans;
  l.alpha = g->alpha;
  l.bias = g->bias; l.sbias2 = g->stride_bias2;
  l.R = g->R; l.ldr = g->ldr; l.sR1 = g->strideR1; l.sR2 = g->strideR2;
  return l;
}

int validate_block(const mlstm_block_params* p, int64_t B, int64_t T) {
  if (!p) return fail(MLSTM_ERR_NULLPTR, "params is NULL");
  if (B < 1 || T < 0) return fail(MLSTM_ERR_BAD_SHAPE, "need B >= 1 and T >= 0");
  if (B > 65535) return fail(MLSTM_ERR_UNSUPPORTED, "B above 65535");
  const int64_t D = p->D, E = 2 * p->D;
  if (D < 64 || D % 64) return fail(MLSTM_ERR_BAD_SHAPE, "D must be a positive multiple of 64");
  if (D > 8192) return fail(MLSTM_ERR_UNSUPPORTED, "D above 8192");
  if (p->H < 1 || p->d_qk < 1 || p->d_v < 1 || p->H * p->d_v != E)
    return fail(MLSTM_ERR_BAD_SHAPE, "need H, d_qk, d_v >= 1 and H d_v == 2 D");
  if ((E / p->H) % 64) return fail(MLSTM_ERR_BAD_SHAPE, "the per-head input width 2 D / H must be a multiple of 64");
  if (p->H > 32) return fail(MLSTM_ERR_UNSUPPORTED, "more than 32 heads");
  if (!(p->d_qk == 64 || p->d_qk == 128 || p->d_qk == 256))
    return fail(MLSTM_ERR_UNSUPPORTED, "d_qk must be 64, 128 or 256");
  if (p->d_v % 128 || p->d_v > 2048) return fail(MLSTM_ERR_UNSUPPORTED, "d_v must be a multiple of 128 up to 2048");
  if (p->KC < 1 || p->KC > 4) return fail(MLSTM_ERR_UNSUPPORTED, "KC must be in 1..4");
  if (!(p->eps_ln >= 0.f) || !(p->eps_gn >= 0.f)) return fail(MLSTM_ERR_BAD_SHAPE, "epsilons must be >= 0");
  const void* ptrs[] = {p->ln_w, p->ln_b, p->W_up, p->b_up, p->conv_w, p->conv_b, p->W_q, p->W_k, p->b_q,
                        p->b_k, p->W_v, p->b_v, p->w_i, p->w_f, p->b_i, p->b_f, p->gn_w, p->gn_b, p->skip,
                        p->W_down, p->b_down};
  for (const void* q : ptrs) {
    if (!q) return fail(MLSTM_ERR_NULLPTR, "every parameter array is required");
    if (!aligned(q, 16)) return fail(MLSTM_ERR_MISALIGNED, "parameter arrays must be 16-byte aligned");
  }
  if (B * T > INT32_MAX / 2 || B * T * p->H / 4 > INT32_MAX)
    return fail(MLSTM_ERR_UNSUPPORTED, "problem too large for one launch grid");
  return MLSTM_OK;
}

// Ranges of the parameter arrays, for alias checks against outputs.
std::vector<Range> param_ranges(const mlstm_block_params* p) {
  const int64_t D = p->D, E = 2 * D, H = p->H, n_in = E / H;
  return {make_range("ln_w", p->ln_w, D * 4), make_range("ln_b", p->ln_b, D * 4),
          make_range("W_up", p->W_up, 2 * E * D * 2), make_range("b_up", p->b_up, 2 * E * 4),
          make_range("conv_w", p->conv_w, E * p->KC * 4), make_range("conv_b", p->conv_b, E * 4),
          make_range("W_q", p->W_q, H * p->d_qk * n_in * 2), make_range("W_k", p->W_k, H * p->d_qk * n_in * 2),
          make_range("b_q", p->b_q, H * p->d_qk * 4), make_range("b_k", p->b_k, H * p->d_qk * 4),
          make_range("W_v", p->W_v, H * p->d_v * n_in * 2), make_range("b_v", p->b_v, E * 4),
          make_range("w_i", p->w_i, H * E * 2), make_range("w_f", p->w_f, H * E * 2),
          make_range("b_i", p->b_i, H * 4), make_range("b_f", p->b_f, H * 4),
          make_range("gn_w", p->gn_w, E * 4), make_range("gn_b", p->gn_b, E * 4),
          make_range("skip", p->skip, E * 4), make_range("W_down", p->W_down, D * E * 2),
          make_range("b_down", p->b_down, D * 4)};
}

mlstm_fwd_args cell_args(const mlstm_block_params* p, int64_t B, int64_t T) {
  mlstm_fwd_args c;
  memset(&c, 0, sizeof(c));
  c.B = B; c.H = p->H; c.T = T; c.d_qk = p->d_qk; c.d_v = p->d_v; c.dtype = MLSTM_BF16;
  return c;
}

struct BlockWs {
  size_t off[10];   // xn, xup, xc, q, k, v, i_pre, f_pre, h, y
  size_t cell, cell_bytes, total;
};

BlockWs block_layout(const mlstm_block_params* p, int64_t B, int64_t T, int chunk) {
  BlockWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  const int64_t D = p->D, E = 2 * D, BT = B * T, BHT = B * p->H * T;
  w.off[0] = take(BT * D * 2);
  w.off[1] = take(BT * 2 * E * 2);
  w.off[2] = take(BT * E * 2);
  w.off[3] = take(BHT * p->d_qk * 2);
  w.off[4] = take(BHT * p->d_qk * 2);
  w.off[5] = take(BHT * p->d_v * 2);
  w.off[6] = take(BHT * 4);
  w.off[7] = take(BHT * 4);
  w.off[8] = take(BHT * p->d_v * 2);
  w.off[9] = take(BT * E * 2);
  const mlstm_fwd_args c = cell_args(p, B, T);
  w.cell_bytes = mlstm_fwd_chunkwise_workspace_size(&c, chunk);
  w.cell = take(w.cell_bytes);
  w.total = off;
  return w;
}

mlstm_impl::ConvLaunch conv_launch(const mlstm_block_params* p, int64_t B, int64_t T, const void* xup, void* xc,
                                   float* i_pre, float* f_pre) {
  mlstm_impl::ConvLaunch c;
  c.B = B; c.T = T; c.E = 2 * p->D; c.H = p->H; c.KC = p->KC;
  c.xm = xup; c.ldx = 4 * p->D;
  c.cw = p->conv_w; c.cb = p->conv_b;
  c.xc = xc;
  c.wi = p->w_i; c.wf = p->w_f; c.bi = p->b_i; c.bf = p->b_f;
  c.i_pre = i_pre; c.f_pre = f_pre;
  return c;
}

mlstm_impl::GnLaunch gn_launch(const mlstm_block_params* p, int64_t B, int64_t T, const void* h, const void* xc,
                               const void* xup, void* y) {
  const int64_t E = 2 * p->D;
  mlstm_impl::GnLaunch g;
  g.B = B; g.T = T; g.H = p->H; g.dv = p->d_v;
  g.h = h; g.xc = xc;
  g.z = static_cast<const char*>(xup) + E * 2;
  g.ldz = 2 * E;
  g.gw = p->gn_w; g.gb = p->gn_b; g.skip = p->skip;
  g.y = y;
  g.eps = p->eps_gn;
  return g;
}

}  // namespace

extern "C" {

int mlstm_gemm_bf16(const mlstm_gemm_args* g, void* stream) {
  g_last_error.clear();
  int st = validate_gemm(g);
  if (st) return st;
  return hip_status(mlstm_impl::launch_gemm(gemm_launch(g), static_cast<hipStream_t>(stream)), "GEMM kernel");
}

int mlstm_layernorm_bf16(const void* x, const float* w, const float* b, void* y, int64_t rows, int64_t D,
                         float eps, void* stream) {
  g_last_error.clear();
  if (rows < 0 || D < 8 || D % 8) return fail(MLSTM_ERR_BAD_SHAPE, "need rows >= 0 and D a positive multiple of 8");
  if (D > 8192) return fail(MLSTM_ERR_UNSUPPORTED, "D above 8192");
  if (!(eps >= 0.f)) return fail(MLSTM_ERR_BAD_SHAPE, "eps must be >= 0");
  if (rows == 0) return MLSTM_OK;
  if (!x || !w || !b || !y) return fail(MLSTM_ERR_NULLPTR, "x, w, b and y are required");
  if (!a16(x) || !a16(w) || !a16(b) || !a16(y)) return fail(MLSTM_ERR_MISALIGNED, "arrays must be 16-byte aligned");
  if (rows > (int64_t)INT32_MAX * 4) return fail(MLSTM_ERR_UNSUPPORTED, "too many rows for one launch grid");
  {
    std::vector<Range> in = {make_range("x", x, rows * D * 2), make_range("w", w, D * 4), make_range("b", b, D * 4)};
    std::vector<Range> out = {make_range("y", y, rows * D * 2)};
    const int st = check_alias(in, out);
    if (st) return st;
  }
  return hip_status(mlstm_impl::launch_layernorm(x, w, b, y, rows, D, eps, static_cast<hipStream_t>(stream)),
                    "layer norm kernel");
}

int mlstm_block_conv_gates(const mlstm_block_params* p, int64_t B, int64_t T, const void* xup, void* xc,
                           float* i_pre, float* f_pre, void* stream) {
  g_last_error.clear();
  int st = validate_block(p, B, T);
  if (st) return st;
  if (T == 0) return MLSTM_OK;
  if (!xup || !xc || !i_pre || !f_pre) return fail(MLSTM_ERR_NULLPTR, "xup, xc, i_pre and f_pre are required");
  if (!a16(xup) || !a16(xc) || !a16(i_pre) || !a16(f_pre))
    return fail(MLSTM_ERR_MISALIGNED, "arrays must be 16-byte aligned");
  const int64_t E = 2 * p->D, BT = B * T;
  std::vector<Range> in = param_ranges(p);
  in.push_back(make_range("xup", xup, BT * 2 * E * 2));
  std::vector<Range> out = {make_range("xc", xc, BT * E * 2), make_range("i_pre", i_pre, BT * p->H * 4),
                            make_range("f_pre", f_pre, BT * p->H * 4)};
  if ((st = check_alias(in, out))) return st;
  return hip_status(mlstm_impl::launch_conv_gate(conv_launch(p, B, T, xup, xc, i_pre, f_pre),
                                                 static_cast<hipStream_t>(stream)), "conv kernel");
}

int mlstm_block_groupnorm_gate(const mlstm_block_params* p, int64_t B, int64_t T, const void* h, const void* xc,
                               const void* xup, void* y, void* stream) {
  g_last_error.clear();
  int st = validate_block(p, B, T);
  if (st) return st;
  if (T == 0) return MLSTM_OK;
  if (!h || !xc || !xup || !y) return fail(MLSTM_ERR_NULLPTR, "h, xc, xup and y are required");
  if (!a16(h) || !a16(xc) || !a16(xup) || !a16(y)) return fail(MLSTM_ERR_MISALIGNED, "arrays must be 16-byte aligned");
  const int64_t E = 2 * p->D, BT = B * T;
  std::vector<Range> in = param_ranges(p);
  in.push_back(make_range("h", h, BT * E * 2));
  in.push_back(make_range("xc", xc, BT * E * 2));
  in.push_back(make_range("xup", xup, BT * 2 * E * 2));
  std::vector<Range> out = {make_range("y", y, BT * E * 2)};
  if ((st = check_alias(in, out))) return st;
  return hip_status(mlstm_impl::launch_groupnorm_gate(gn_launch(p, B, T, h, xc, xup, y),
                                                      static_cast<hipStream_t>(stream)), "group norm kernel");
}

size_t mlstm_block_fwd_workspace_size(const mlstm_block_params* p, int64_t B, int64_t T, int chunk) {
  if (!p || B < 1 || T <= 0 || chunk < 64 || chunk % 64 || chunk > kMaxChunk) return 0;
  if (p->D < 64 || p->H < 1 || p->d_qk < 1 || p->d_v < 1) return 0;
  return block_layout(p, B, T, chunk).total;
}

int mlstm_block_workspace_offsets(const mlstm_block_params* p, int64_t B, int64_t T, int chunk, size_t offsets[10]) {
  g_last_error.clear();
  if (!offsets) return fail(MLSTM_ERR_NULLPTR, "offsets is NULL");
  if (!p || B < 1 || T <= 0 || chunk < 64 || chunk % 64 || chunk > kMaxChunk || p->D < 64 || p->H < 1 ||
      p->d_qk < 1 || p->d_v < 1)
    return fail(MLSTM_ERR_BAD_SHAPE, "invalid sizes");
  const BlockWs w = block_layout(p, B, T, chunk);
  for (int j = 0; j < 10; ++j) offsets[j] = w.off[j];
  return MLSTM_OK;
}

int mlstm_block_fwd(const mlstm_block_params* p, int64_t B, int64_t T, const void* x, void* out, int chunk,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int st = validate_block(p, B, T);
  if (st) return st;
  if (chunk < 64 || chunk % 64 != 0 || chunk > kMaxChunk)
    return fail(MLSTM_ERR_BAD_SHAPE, "chunk must be a multiple of 64 in [64, 8192]");
  if (T == 0) return MLSTM_OK;
  if (!x || !out) return fail(MLSTM_ERR_NULLPTR, "x and out are required");
  if (!a16(x) || !a16(out)) return fail(MLSTM_ERR_MISALIGNED, "x and out must be 16-byte aligned");
  const BlockWs w = block_layout(p, B, T, chunk);
  if (!workspace) return fail(MLSTM_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, kAlign)) return fail(MLSTM_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (workspace_bytes < w.total)
    return fail(MLSTM_ERR_WORKSPACE, "workspace too small: need " + std::to_string(w.total) + " bytes");
  const int64_t D = p->D, E = 2 * D, H = p->H, BT = B * T, n_in = E / H;
  {
    std::vector<Range> in = param_ranges(p);
    in.push_back(make_range("x", x, BT * D * 2));
    std::vector<Range> outs = {make_range("out", out, BT * D * 2),
                               make_range("workspace", workspace, (int64_t)w.total)};
    if ((st = check_alias(in, outs))) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* xn = ws + w.off[0];
  void* xup = ws + w.off[1];
  void* xc = ws + w.off[2];
  void* q = ws + w.off[3];
  void* k = ws + w.off[4];
  void* v = ws + w.off[5];
  float* ip = reinterpret_cast<float*>(ws + w.off[6]);
  float* fp = reinterpret_cast<float*>(ws + w.off[7]);
  void* hc = ws + w.off[8];
  void* y = ws + w.off[9];

  if ((st = hip_status(mlstm_impl::launch_layernorm(x, p->ln_w, p->ln_b, xn, BT, D, p->eps_ln, s), "layer norm")))
    return st;
  mlstm_impl::GemmLaunch g{};
  g.nb1 = g.nb2 = 1;
  g.alpha = 1.f;
  // up-projection [BT][2E]
  g.M = BT; g.N = 2 * E; g.K = D;
  g.A = xn; g.lda = D; g.B = p->W_up; g.ldb = D; g.C = xup; g.ldc = 2 * E; g.bias = p->b_up;
  if ((st = hip_status(mlstm_impl::launch_gemm(g, s), "up-projection"))) return st;
  if ((st = hip_status(mlstm_impl::launch_conv_gate(conv_launch(p, B, T, xup, xc, ip, fp), s), "conv kernel")))
    return st;
  // per-head projections, batched over (batch entry, head), into [B][H][T][d]
  auto head_proj = [&](const void* A, int64_t lda, const void* W, int64_t n_out, const float* bias, void* C,
                       float alpha, const char* what) {
    mlstm_impl::GemmLaunch h{};
    h.M = T; h.N = n_out; h.K = n_in; h.nb1 = B; h.nb2 = H;
    h.A = A; h.lda = lda; h.sA1 = T * lda; h.sA2 = n_in;
    h.B = W; h.ldb = n_in; h.sB1 = 0; h.sB2 = n_out * n_in;
    h.C = C; h.ldc = n_out; h.sC1 = H * T * n_out; h.sC2 = T * n_out;
    h.alpha = alpha; h.bias = bias; h.sbias2 = n_out;
    return hip_status(mlstm_impl::launch_gemm(h, s), what);
  };
  if ((st = head_proj(xc, E, p->W_q, p->d_qk, p->b_q, q, 1.f, "q projection"))) return st;
  if ((st = head_proj(xc, E, p->W_k, p->d_qk, p->b_k, k, (float)(1.0 / std::sqrt((double)p->d_qk)),
                      "k projection")))
    return st;
  if ((st = head_proj(xup, 2 * E, p->W_v, p->d_v, p->b_v, v, 1.f, "v projection"))) return st;
  // the cell, ungated
  mlstm_fwd_args c = cell_args(p, B, T);
  c.q = q; c.k = k; c.v = v; c.o_pre = nullptr; c.i_pre = ip; c.f_pre = fp; c.h = hc;
  if ((st = fwd_chunkwise(&c, chunk, ws + w.cell, w.cell_bytes, stream, nullptr))) return st;
  if ((st = hip_status(mlstm_impl::launch_groupnorm_gate(gn_launch(p, B, T, hc, xc, xup, y), s), "group norm")))
    return st;
  // down-projection with the residual
  g = mlstm_impl::GemmLaunch{};
  g.nb1 = g.nb2 = 1;
  g.alpha = 1.f;
  g.M = BT; g.N = D; g.K = E;
  g.A = y; g.lda = E; g.B = p->W_down; g.ldb = E; g.C = out; g.ldc = D; g.bias = p->b_down;
  g.R = x; g.ldr = D;
  return hip_status(mlstm_impl::launch_gemm(g, s), "down-projection");
}

}  // extern "C"

// ------------------------------------------------------------------ segments

namespace {

int validate_summary(const mlstm_summary_args* a, int chunk) {
  if (!a) return fail(MLSTM_ERR_NULLPTR, "args is NULL");
  if (a->dtype != MLSTM_FP32 && a->dtype != MLSTM_BF16)
    return fail(MLSTM_ERR_BAD_DTYPE, "dtype must be MLSTM_FP32 or MLSTM_BF16");
  if (a->B < 1 || a->H < 1 || a->T < 0 || a->d_qk < 1 || a->d_v < 1)
    return fail(MLSTM_ERR_BAD_SHAPE, "need B >= 1, H >= 1, T >= 0, d_qk >= 1, d_v >= 1");
  if (chunk < 64 || chunk % 64 != 0 || chunk > kMaxChunk)
    return fail(MLSTM_ERR_BAD_SHAPE, "chunk must be a multiple of 64 in [64, 8192]");
  if (a->T % chunk != 0) return fail(MLSTM_ERR_BAD_SHAPE, "T must be a multiple of chunk (every chunk full)");
  if (!mlstm_impl::fused_path(a->dtype == MLSTM_BF16, a->d_qk, a->d_v) || a->d_v > 16384)
    return fail(MLSTM_ERR_UNSUPPORTED, "segment summaries need MLSTM_BF16, d_qk 64, 128 or 256 and d_v a "
                                       "multiple of 128 (at most 16384)");
  if (!a->C_out || !a->n_out || !a->m_out || !a->G_out)
    return fail(MLSTM_ERR_NULLPTR, "C_out, n_out, m_out and G_out are required");
  if (a->T > 0 && (!a->k || !a->v || !a->i_pre || !a->f_pre))
    return fail(MLSTM_ERR_NULLPTR, "k, v, i_pre and f_pre are required when T > 0");
  const void* v16[] = {a->k, a->v, a->C_out, a->n_out};
  for (const void* p : v16)
    if (p && !aligned(p, 16)) return fail(MLSTM_ERR_MISALIGNED, "array pointers must be 16-byte aligned");
  const void* v4[] = {a->i_pre, a->f_pre, a->m_out};
  for (const void* p : v4)
    if (p && !aligned(p, 4)) return fail(MLSTM_ERR_MISALIGNED, "gate and m pointers must be 4-byte aligned");
  if (!aligned(a->G_out, 8)) return fail(MLSTM_ERR_MISALIGNED, "G_out must be 8-byte aligned");
  const int64_t BH = a->B * a->H;
  if (BH * (a->d_v / 128) * (a->T / chunk) > INT32_MAX || BH * ((a->d_v * a->d_qk + a->d_qk) / 4 / 256 + 1) > INT32_MAX)
    return fail(MLSTM_ERR_UNSUPPORTED, "problem too large for one launch grid");
  const int64_t nqk = BH * a->T * a->d_qk * 2, nv = BH * a->T * a->d_v * 2, ng = BH * a->T * 4;
  const int64_t nC = BH * a->d_v * a->d_qk * 4, nn = BH * a->d_qk * 4, nm = BH * 4;
  std::vector<Range> in = {make_range("k", a->k, nqk), make_range("v", a->v, nv),
                           make_range("i_pre", a->i_pre, ng), make_range("f_pre", a->f_pre, ng)};
  std::vector<Range> out = {make_range("C_out", a->C_out, nC), make_range("n_out", a->n_out, nn),
                            make_range("m_out", a->m_out, nm), make_range("G_out", a->G_out, BH * 8)};
  return check_alias(in, out);
}

int validate_combine(const mlstm_combine_args* a) {
  if (!a) return fail(MLSTM_ERR_NULLPTR, "args is NULL");
  if (a->B < 1 || a->H < 1 || a->d_qk < 1 || a->d_v < 1 || a->count < 0)
    return fail(MLSTM_ERR_BAD_SHAPE, "need B >= 1, H >= 1, d_qk >= 1, d_v >= 1, count >= 0");
  if (a->d_qk % 4 != 0) return fail(MLSTM_ERR_BAD_SHAPE, "d_qk must be a multiple of 4");
  const bool any0 = a->C0 || a->n0 || a->m0, all0 = a->C0 && a->n0 && a->m0;
  if (any0 && !all0) return fail(MLSTM_ERR_NULLPTR, "C0, n0, m0 must be given together");
  if (!a->C_out || !a->n_out || !a->m_out) return fail(MLSTM_ERR_NULLPTR, "C_out, n_out and m_out are required");
  if (a->count > 0 && (!a->Cs || !a->ns || !a->ms || !a->Gs))
    return fail(MLSTM_ERR_NULLPTR, "Cs, ns, ms and Gs are required when count > 0");
  const void* v16[] = {a->C0, a->n0, a->Cs, a->ns, a->C_out, a->n_out};
  for (const void* p : v16)
    if (p && !aligned(p, 16)) return fail(MLSTM_ERR_MISALIGNED, "state arrays must be 16-byte aligned");
  const void* v4[] = {a->m0, a->ms, a->m_out};
  for (const void* p : v4)
    if (p && !aligned(p, 4)) return fail(MLSTM_ERR_MISALIGNED, "m arrays must be 4-byte aligned");
  if (a->Gs && !aligned(a->Gs, 8)) return fail(MLSTM_ERR_MISALIGNED, "Gs must be 8-byte aligned");
  const int64_t BH = a->B * a->H;
  if (a->d_v > (int64_t)1 << 20 || a->d_qk > (int64_t)1 << 20 || a->count > (int64_t)1 << 20 ||
      BH * ((a->d_v * a->d_qk + a->d_qk) / 4 / 256 + 1) > INT32_MAX)
    return fail(MLSTM_ERR_UNSUPPORTED, "problem too large for one launch grid");
  const int64_t nC = BH * a->d_v * a->d_qk * 4, nn = BH * a->d_qk * 4, nm = BH * 4, c = a->count;
  std::vector<Range> in = {make_range("C0", a->C0, nC), make_range("n0", a->n0, nn),
                           make_range("m0", a->m0, nm), make_range("Cs", a->Cs, c * nC),
                           make_range("ns", a->ns, c * nn), make_range("ms", a->ms, c * nm),
                           make_range("Gs", a->Gs, c * BH * 8)};
  std::vector<Range> out = {make_range("C_out", a->C_out, nC), make_range("n_out", a->n_out, nn),
                            make_range("m_out", a->m_out, nm)};
  return check_alias(in, out);
}

}  // namespace

extern "C" {

size_t mlstm_segment_summary_workspace_size(const mlstm_summary_args* a, int chunk) {
  if (!a || a->T <= 0 || a->B < 1 || a->H < 1 || chunk < 64 || chunk % 64 != 0 || chunk > kMaxChunk ||
      a->T % chunk != 0 || !mlstm_impl::fused_path(a->dtype == MLSTM_BF16, a->d_qk, a->d_v))
    return 0;
  return layout_fused(a->B * a->H, a->T, chunk, a->d_qk, a->d_v, true).total;
}

int mlstm_segment_summary(const mlstm_summary_args* a, int chunk, void* workspace, size_t workspace_bytes,
                          void* stream) {
  g_last_error.clear();
  int st = validate_summary(a, chunk);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t BH = a->B * a->H;
  const mlstm_impl::SummaryOut o{a->C_out, a->n_out, a->m_out, a->G_out};
  if (a->T == 0) return hip_status(mlstm_impl::launch_summary_empty(o, BH, a->d_qk, a->d_v, s), "summary fill");
  const size_t need = mlstm_segment_summary_workspace_size(a, chunk);
  if (!workspace) return fail(MLSTM_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, kAlign)) return fail(MLSTM_ERR_MISALIGNED, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(MLSTM_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
  {
    const int64_t nqk = BH * a->T * a->d_qk * 2, nv = BH * a->T * a->d_v * 2, ng = BH * a->T * 4;
    const int64_t nC = BH * a->d_v * a->d_qk * 4, nn = BH * a->d_qk * 4, nm = BH * 4;
    const Range wr = make_range("workspace", workspace, (int64_t)need);
    const Range other[] = {make_range("k", a->k, nqk), make_range("v", a->v, nv),
                           make_range("i_pre", a->i_pre, ng), make_range("f_pre", a->f_pre, ng),
                           make_range("C_out", a->C_out, nC), make_range("n_out", a->n_out, nn),
                           make_range("m_out", a->m_out, nm), make_range("G_out", a->G_out, BH * 8)};
    for (const Range& r : other)
      if (overlap(wr, r)) return fail(MLSTM_ERR_ALIAS, std::string("workspace overlaps ") + r.name);
  }
  const FusedShape fs = fused_shape(a->T, chunk);
  mlstm_impl::FwdLaunch f{};
  f.BH = BH; f.T = a->T; f.K = a->d_qk; f.V = a->d_v;
  f.L = 64; f.Nc = fs.Nt; f.bf16 = 1;
  f.k = a->k; f.v = a->v; f.i_pre = a->i_pre; f.f_pre = a->f_pre;
  const WsLayout w = layout_fused(BH, a->T, chunk, a->d_qk, a->d_v, true);
  char* ws = static_cast<char*>(workspace);
  mlstm_impl::GateBuffers gb = gate_buffers(ws, w);
  gb.wb = reinterpret_cast<uint16_t*>(ws + w.wb);
  mlstm_impl::SegStates ss;
  ss.C = reinterpret_cast<float*>(ws + w.Cseg);
  ss.n = reinterpret_cast<float*>(ws + w.nseg);
  ss.mloc = reinterpret_cast<double*>(ws + w.mloc);
  ss.mstart = reinterpret_cast<double*>(ws + w.mstart);
  ss.G = reinterpret_cast<double*>(ws + w.Gseg);
  ss.S = (int)fs.S;
  ss.TPS = (int)fs.TPS;
  if ((st = hip_status(mlstm_impl::launch_gate(f, gb, s), "gate kernel"))) return st;
  return hip_status(mlstm_impl::launch_summary(f, gb, ss, o, s), "summary kernels");
}

int mlstm_state_combine(const mlstm_combine_args* a, void* stream) {
  g_last_error.clear();
  const int st = validate_combine(a);
  if (st) return st;
  mlstm_impl::CombineLaunch c;
  c.BH = a->B * a->H; c.K = a->d_qk; c.V = a->d_v; c.count = a->count;
  c.C0 = a->C0; c.n0 = a->n0; c.m0 = a->m0;
  c.Cs = a->Cs; c.ns = a->ns; c.ms = a->ms; c.Gs = a->Gs;
  c.C = a->C_out; c.n = a->n_out; c.m = a->m_out;
  return hip_status(mlstm_impl::launch_state_combine(c, static_cast<hipStream_t>(stream)), "combine kernel");
}

}  // extern "C"
