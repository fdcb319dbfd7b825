// C ABI of the mLSTM cell forward: argument validation, workspace layout and
// dispatch to the HIP launchers. Every check runs on the host before any HIP
// call, so invalid arguments are rejected without touching a device.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/mlstm.h"
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
int validate_fwd(const mlstm_fwd_args* a) {
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
  if (a->T > 0 && (!a->q || !a->k || !a->v || !a->o_pre || !a->i_pre || !a->f_pre || !a->h))
    return fail(MLSTM_ERR_NULLPTR, "q, k, v, o_pre, i_pre, f_pre and h are required when T > 0");
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

WsLayout layout_fused(int64_t BH, int64_t T, int chunk, int64_t K, int64_t V) {
  const FusedShape fs = fused_shape(T, chunk);
  WsLayout w = layout(BH, T, fs.Nt, K, V, 4, false);
  size_t off = w.total;
  auto take = [&](size_t bytes) { const size_t o = off; off = align_up(off + bytes); return o; };
  const int64_t ns = fs.S - 1;
  w.Cseg = take(BH * ns * V * K * 4);
  w.nseg = take(BH * ns * K * 4);
  w.mloc = take(BH * ns * 8);
  w.mstart = take(BH * ns * 8);
  w.Gseg = take(BH * ns * 8);
  w.wb = take(BH * fs.Nt * 2 * 64 * 2);
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

mlstm_impl::FwdLaunch fwd_launch(const mlstm_fwd_args* a, int L, int64_t Nc) {
  mlstm_impl::FwdLaunch f;
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
  return layout(a->B * a->H, a->T, Nc, a->d_qk, a->d_v, a->dtype == MLSTM_BF16 ? 2 : 4, true).total;
}

int mlstm_fwd_chunkwise(const mlstm_fwd_args* a, int chunk, void* workspace, size_t workspace_bytes,
                        void* stream) {
  g_last_error.clear();
  int st = validate_fwd(a);
  if (st) return st;
  if (chunk < 64 || chunk % 64 != 0 || chunk > kMaxChunk)
    return fail(MLSTM_ERR_BAD_SHAPE, "chunk must be a multiple of 64 in [64, 8192]");
  if ((st = check_grid(a))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t Nc = a->T > 0 ? (a->T + chunk - 1) / chunk : 0;
  mlstm_impl::FwdLaunch f = fwd_launch(a, chunk, Nc);
  if (a->T == 0) return hip_status(mlstm_impl::launch_copy_state(f, s), "state copy");
  const size_t need = mlstm_fwd_chunkwise_workspace_size(a, chunk);
  if ((st = check_workspace(a, workspace, workspace_bytes, need))) return st;
  char* ws = static_cast<char*>(workspace);
  if (use_fused(a)) {
    const FusedShape fs = fused_shape(a->T, chunk);
    const mlstm_impl::FwdLaunch ft = fwd_launch(a, 64, fs.Nt);
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
  const WsLayout w = layout(f.BH, f.T, Nc, f.K, f.V, f.bf16 ? 2 : 4, true);
  const mlstm_impl::GateBuffers gb = gate_buffers(ws, w);
  mlstm_impl::ChunkStates cs;
  cs.Cs = ws + w.Cs;
  cs.ns = reinterpret_cast<float*>(ws + w.ns);
  cs.ms = reinterpret_cast<double*>(ws + w.ms);
  if ((st = hip_status(mlstm_impl::launch_gate(f, gb, s), "gate kernel"))) return st;
  if ((st = hip_status(mlstm_impl::launch_state(f, gb, cs, s), "state kernel"))) return st;
  return hip_status(mlstm_impl::launch_out(f, gb, cs, s), "output kernel");
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

int mlstm_step(const mlstm_step_args* a, void* stream) {
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
  return hip_status(mlstm_impl::launch_step(sl, static_cast<hipStream_t>(stream)), "step kernel");
}

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

int mlstm_set_launch_events(int kernel_id, void* before, void* after) {
  if (kernel_id < 0 || kernel_id >= mlstm_impl::K_COUNT)
    return fail(MLSTM_ERR_BAD_SHAPE, "kernel_id must be 0..3");
  mlstm_impl::set_launch_events(kernel_id, static_cast<hipEvent_t>(before), static_cast<hipEvent_t>(after));
  return MLSTM_OK;
}

}  // extern "C"
