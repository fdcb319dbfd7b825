// Drives every entry point of the mLSTM C ABI (include/mlstm.h,
// mlstm_block.h, mlstm_segments.h, slstm.h, mlstm_prof.h) through its argument checks and, with host-only stand-in
// launchers (abi_stub_launchers.cpp), through its workspace carving and
// dispatch, in a build with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code. Pointers are fabricated addresses that nothing
// dereferences. Exit status 0 when every expectation holds; the sanitizers
// abort on their own findings.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/mlstm.h"
#include "../../include/mlstm_block.h"
#include "../../include/mlstm_prof.h"
#include "../../include/mlstm_segments.h"
#include "../../include/slstm.h"

namespace mlstm_impl { extern int g_calls[20]; }

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static uintptr_t next_addr = 0x7C0000000000ull;
static void* take(size_t bytes) {
  const uintptr_t p = next_addr;
  next_addr += (bytes + 4095) / 4096 * 4096 + 4096;
  return reinterpret_cast<void*>(p);
}

static mlstm_fwd_args fwd(int64_t B, int64_t H, int64_t T, int64_t K, int64_t V, int dtype, bool state_in,
                          bool state_out) {
  mlstm_fwd_args a;
  memset(&a, 0, sizeof(a));
  const int64_t es = dtype == MLSTM_BF16 ? 2 : 4, BH = B * H;
  a.B = B; a.H = H; a.T = T; a.d_qk = K; a.d_v = V; a.dtype = dtype;
  a.q = take(BH * T * K * es); a.k = take(BH * T * K * es); a.v = take(BH * T * V * es);
  a.o_pre = take(BH * T * V * es); a.i_pre = (const float*)take(BH * T * 4); a.f_pre = (const float*)take(BH * T * 4);
  a.h = take(BH * T * V * es);
  if (state_in) { a.C0 = (const float*)take(BH * V * K * 4); a.n0 = (const float*)take(BH * K * 4); a.m0 = (const float*)take(BH * 4); }
  if (state_out) { a.C_out = (float*)take(BH * V * K * 4); a.n_out = (float*)take(BH * K * 4); a.m_out = (float*)take(BH * 4); }
  return a;
}

static mlstm_bwd_args bwd(int64_t B, int64_t H, int64_t T, int64_t K, int64_t V, int dtype, bool init) {
  mlstm_bwd_args a;
  memset(&a, 0, sizeof(a));
  const int64_t es = dtype == MLSTM_BF16 ? 2 : 4, BH = B * H;
  a.B = B; a.H = H; a.T = T; a.d_qk = K; a.d_v = V; a.dtype = dtype;
  a.q = take(BH * T * K * es); a.k = take(BH * T * K * es); a.v = take(BH * T * V * es);
  a.o_pre = take(BH * T * V * es); a.i_pre = (const float*)take(BH * T * 4); a.f_pre = (const float*)take(BH * T * 4);
  a.h = take(BH * T * V * es); a.dh = take(BH * T * V * es);
  a.dq = take(BH * T * K * es); a.dk = take(BH * T * K * es); a.dv = take(BH * T * V * es);
  a.do_pre = take(BH * T * V * es); a.di_pre = (float*)take(BH * T * 4); a.df_pre = (float*)take(BH * T * 4);
  if (init) { a.dC0 = (float*)take(BH * V * K * 4); a.dn0 = (float*)take(BH * K * 4); a.dm0 = (float*)take(BH * 4); }
  return a;
}

int main() {
  using mlstm_impl::g_calls;
  EXPECT(mlstm_abi_version() == MLSTM_ABI_VERSION);
  for (int s = 1; s >= -9; --s) EXPECT(mlstm_status_string(s) != nullptr);

  // ---- forward, chunkwise: every dtype / shape family reaches its launchers
  const int dts[2] = {MLSTM_FP32, MLSTM_BF16};
  for (int di = 0; di < 2; ++di) {
    for (int64_t V : {64, 128, 192, 512}) {
      for (int64_t T : {1, 63, 64, 65, 1000}) {
        for (int chunk : {64, 128, 1024}) {
          const int64_t K = dts[di] == MLSTM_BF16 ? 256 : 128;
          mlstm_fwd_args a = fwd(2, 3, T, K, V, dts[di], T % 2 == 0, T % 3 == 0);
          const size_t need = mlstm_fwd_chunkwise_workspace_size(&a, chunk);
          EXPECT(need > 0);
          void* ws = take(need);
          const int before = g_calls[0];
          EXPECT(mlstm_fwd_chunkwise(&a, chunk, ws, need, nullptr) == MLSTM_OK);
          EXPECT(g_calls[0] == before + 1);
          EXPECT(mlstm_fwd_chunkwise(&a, chunk, ws, need - 1, nullptr) == MLSTM_ERR_WORKSPACE);
          EXPECT(mlstm_fwd_chunkwise(&a, chunk, a.h, need, nullptr) == MLSTM_ERR_ALIAS);
          const size_t pneed = mlstm_fwd_parallel_workspace_size(&a);
          EXPECT(mlstm_fwd_parallel(&a, take(pneed), pneed, nullptr) == MLSTM_OK);
          void* ev[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
          EXPECT(mlstm_prof_fwd_chunkwise(&a, chunk, ws, need, nullptr, ev) == MLSTM_OK);
        }
      }
    }
  }
  {
    mlstm_fwd_args a = fwd(1, 1, 0, 64, 64, MLSTM_FP32, true, true);
    EXPECT(mlstm_fwd_chunkwise(&a, 64, nullptr, 0, nullptr) == MLSTM_OK);   // T = 0: state copy
    a = fwd(1, 1, 10, 64, 64, MLSTM_FP32, false, false);
    EXPECT(mlstm_fwd_chunkwise(nullptr, 64, nullptr, 0, nullptr) == MLSTM_ERR_NULLPTR);
    a.dtype = 9;
    EXPECT(mlstm_fwd_chunkwise(&a, 64, take(1 << 20), 1 << 20, nullptr) == MLSTM_ERR_BAD_DTYPE);
    a.dtype = MLSTM_FP32; a.d_qk = 96;
    EXPECT(mlstm_fwd_chunkwise(&a, 64, take(1 << 20), 1 << 20, nullptr) == MLSTM_ERR_BAD_SHAPE);
    a.d_qk = 256;
    EXPECT(mlstm_fwd_chunkwise(&a, 64, take(1 << 20), 1 << 20, nullptr) == MLSTM_ERR_UNSUPPORTED);
    a.d_qk = 64;
    EXPECT(mlstm_fwd_chunkwise(&a, 100, take(1 << 20), 1 << 20, nullptr) == MLSTM_ERR_BAD_SHAPE);
    a.q = (const char*)a.q + 2;
    EXPECT(mlstm_fwd_chunkwise(&a, 64, take(1 << 20), 1 << 20, nullptr) == MLSTM_ERR_MISALIGNED);
    EXPECT(strlen(mlstm_last_error()) > 0);
    mlstm_fwd_args p = fwd(1, 1, 9000, 64, 64, MLSTM_FP32, false, false);
    EXPECT(mlstm_fwd_parallel(&p, take(1 << 20), 1 << 20, nullptr) == MLSTM_ERR_UNSUPPORTED);
  }
  // no-allocation entry point: either it finds no device (error) or runs
  {
    mlstm_fwd_args a = fwd(1, 2, 500, 128, 256, MLSTM_BF16, false, false);
    const int st = mlstm_fwd_chunkwise_noalloc(&a, 128, nullptr);
    EXPECT(st == MLSTM_OK || st == MLSTM_ERR_HIP);
    mlstm_fwd_args big = fwd(1, 8, 131072, 256, 512, MLSTM_BF16, false, false);
    EXPECT(mlstm_fwd_chunkwise_noalloc(&big, 64, nullptr) == MLSTM_ERR_UNSUPPORTED);
    EXPECT(mlstm_fwd_chunkwise_noalloc_limit() == (size_t(64) << 20));
  }

  // ---- decode step
  {
    mlstm_step_args s;
    memset(&s, 0, sizeof(s));
    s.B = 4; s.H = 2; s.d_qk = 128; s.d_v = 96; s.dtype = MLSTM_BF16;
    const int64_t BH = 8;
    s.q = take(BH * 128 * 2); s.k = take(BH * 128 * 2); s.v = take(BH * 96 * 2); s.o_pre = take(BH * 96 * 2);
    s.i_pre = (const float*)take(BH * 4); s.f_pre = (const float*)take(BH * 4);
    s.C = (float*)take(BH * 96 * 128 * 4); s.n_in = (const float*)take(BH * 128 * 4); s.m_in = (const float*)take(BH * 4);
    s.n_out = (float*)take(BH * 128 * 4); s.m_out = (float*)take(BH * 4); s.h = take(BH * 96 * 2);
    EXPECT(mlstm_step(&s, nullptr) == MLSTM_OK);
    EXPECT(mlstm_prof_step(&s, nullptr, nullptr, nullptr) == MLSTM_OK);
    s.n_out = (float*)s.n_in;
    EXPECT(mlstm_step(&s, nullptr) == MLSTM_ERR_ALIAS);
  }

  // ---- backward
  for (int di = 0; di < 2; ++di) {
    for (int64_t V : {64, 256}) {
      for (int64_t T : {1, 77, 300}) {
        for (int chunk : {64, 192}) {
          mlstm_bwd_args b = bwd(2, 2, T, 64, V, dts[di], T > 1);
          const size_t need = mlstm_bwd_chunkwise_workspace_size(&b, chunk);
          EXPECT(need > 0);
          void* ws = take(need);
          const int before = g_calls[11];
          EXPECT(mlstm_bwd_chunkwise(&b, chunk, ws, need, nullptr) == MLSTM_OK);
          EXPECT(g_calls[11] == before + 1);
          EXPECT(mlstm_bwd_chunkwise(&b, chunk, ws, need - 1, nullptr) == MLSTM_ERR_WORKSPACE);
          void* ev[12] = {};
          EXPECT(mlstm_prof_bwd_chunkwise(&b, chunk, ws, need, nullptr, ev) == MLSTM_OK);
          b.dq = const_cast<void*>(b.q);
          EXPECT(mlstm_bwd_chunkwise(&b, chunk, ws, need, nullptr) == MLSTM_ERR_ALIAS);
        }
      }
    }
  }
  {
    mlstm_bwd_args b = bwd(1, 1, 10, 256, 1024, MLSTM_BF16, false);
    EXPECT(mlstm_bwd_chunkwise(&b, 64, take(1 << 20), 1 << 20, nullptr) == MLSTM_ERR_UNSUPPORTED);
    b = bwd(1, 1, 0, 64, 64, MLSTM_FP32, true);
    EXPECT(mlstm_bwd_chunkwise(&b, 64, nullptr, 0, nullptr) == MLSTM_OK);   // zero the state gradient
  }

  // ---- sLSTM
  {
    slstm_fwd_args s;
    memset(&s, 0, sizeof(s));
    s.B = 2; s.H = 3; s.T = 50; s.D = 64;
    s.pre = (const float*)take(6 * 50 * 4 * 64 * 4); s.R = (const float*)take(3 * 4 * 64 * 64 * 4);
    s.h = (float*)take(6 * 50 * 64 * 4);
    EXPECT(slstm_fwd(&s, nullptr) == MLSTM_OK);
    s.D = 48;
    EXPECT(slstm_fwd(&s, nullptr) == MLSTM_ERR_UNSUPPORTED);
  }

  // ---- measurement helpers
  {
    unsigned long long* ticks = (unsigned long long*)take(32);
    EXPECT(mlstm_clock_probe(ticks, 10, nullptr) == MLSTM_OK);
    EXPECT(mlstm_clock_probe(ticks, 0, nullptr) == MLSTM_ERR_BAD_SHAPE);
    void* src = take(1 << 20);
    void* dst = take(1 << 20);
    EXPECT(mlstm_prof_copy_lds(src, dst, 1 << 20, nullptr) == MLSTM_OK);
    EXPECT(mlstm_prof_copy_lds(src, (char*)src + 16384, 32768, nullptr) == MLSTM_ERR_ALIAS);
  }

  // ---- mLSTM block: the whole block through its nine launches, and each step
  {
    const int64_t D = 256, E = 512, H = 4, dqk = 64, dv = 128, KC = 4, B = 2, T = 100;
    mlstm_block_params p;
    memset(&p, 0, sizeof(p));
    p.D = D; p.H = H; p.d_qk = dqk; p.d_v = dv; p.KC = KC; p.eps_ln = 1e-5f; p.eps_gn = 1e-5f;
    p.ln_w = (const float*)take(D * 4); p.ln_b = (const float*)take(D * 4);
    p.W_up = take(2 * E * D * 2); p.b_up = (const float*)take(2 * E * 4);
    p.conv_w = (const float*)take(E * KC * 4); p.conv_b = (const float*)take(E * 4);
    p.W_q = take(H * dqk * (E / H) * 2); p.W_k = take(H * dqk * (E / H) * 2);
    p.b_q = (const float*)take(H * dqk * 4); p.b_k = (const float*)take(H * dqk * 4);
    p.W_v = take(H * dv * (E / H) * 2); p.b_v = (const float*)take(E * 4);
    p.w_i = take(H * E * 2); p.w_f = take(H * E * 2);
    p.b_i = (const float*)take(H * 4); p.b_f = (const float*)take(H * 4);
    p.gn_w = (const float*)take(E * 4); p.gn_b = (const float*)take(E * 4); p.skip = (const float*)take(E * 4);
    p.W_down = take(D * E * 2); p.b_down = (const float*)take(D * 4);
    void* x = take(B * T * D * 2);
    void* out = take(B * T * D * 2);
    const size_t need = mlstm_block_fwd_workspace_size(&p, B, T, 64);
    EXPECT(need > 0);
    void* ws = take(need);
    int before[20];
    for (int j = 0; j < 20; ++j) before[j] = g_calls[j];
    EXPECT(mlstm_block_fwd(&p, B, T, x, out, 64, ws, need, nullptr) == MLSTM_OK);
    EXPECT(g_calls[12] == before[12] + 5);   // up, q, k, v, down
    EXPECT(g_calls[13] == before[13] + 1 && g_calls[14] == before[14] + 1 && g_calls[15] == before[15] + 1);
    EXPECT(g_calls[9] == before[9] + 1);     // the cell's fused kernels, ungated
    size_t offs[10];
    EXPECT(mlstm_block_workspace_offsets(&p, B, T, 64, offs) == MLSTM_OK);
    for (int j = 1; j < 10; ++j) EXPECT(offs[j] > offs[j - 1]);
    EXPECT(offs[9] + (size_t)(B * T * E * 2) <= need);
    EXPECT(mlstm_block_fwd(&p, B, T, x, out, 64, ws, need - 1, nullptr) == MLSTM_ERR_WORKSPACE);
    EXPECT(mlstm_block_fwd(&p, B, T, x, out, 64, nullptr, need, nullptr) == MLSTM_ERR_WORKSPACE);
    EXPECT(mlstm_block_fwd(&p, B, T, x, x, 64, ws, need, nullptr) == MLSTM_ERR_ALIAS);
    EXPECT(mlstm_block_fwd(&p, B, T, x, (void*)p.W_up, 64, ws, need, nullptr) == MLSTM_ERR_ALIAS);
    EXPECT(mlstm_block_fwd(&p, B, T, x, out, 100, ws, need, nullptr) == MLSTM_ERR_BAD_SHAPE);
    EXPECT(mlstm_block_fwd(&p, B, 0, x, out, 64, nullptr, 0, nullptr) == MLSTM_OK);
    EXPECT(mlstm_block_fwd(nullptr, B, T, x, out, 64, ws, need, nullptr) == MLSTM_ERR_NULLPTR);
    mlstm_block_params bad = p;
    bad.d_v = 64;
    EXPECT(mlstm_block_fwd(&bad, B, T, x, out, 64, ws, need, nullptr) == MLSTM_ERR_BAD_SHAPE);
    bad = p; bad.d_qk = 32;
    EXPECT(mlstm_block_fwd(&bad, B, T, x, out, 64, ws, need, nullptr) == MLSTM_ERR_UNSUPPORTED);
    bad = p; bad.KC = 5;
    EXPECT(mlstm_block_fwd(&bad, B, T, x, out, 64, ws, need, nullptr) == MLSTM_ERR_UNSUPPORTED);
    bad = p; bad.skip = nullptr;
    EXPECT(mlstm_block_fwd(&bad, B, T, x, out, 64, ws, need, nullptr) == MLSTM_ERR_NULLPTR);
    bad = p; bad.b_up = (const float*)((const char*)p.b_up + 4);
    EXPECT(mlstm_block_fwd(&bad, B, T, x, out, 64, ws, need, nullptr) == MLSTM_ERR_MISALIGNED);

    void* xup = take(B * T * 2 * E * 2);
    void* xc = take(B * T * E * 2);
    float* ip = (float*)take(B * H * T * 4);
    float* fp = (float*)take(B * H * T * 4);
    EXPECT(mlstm_block_conv_gates(&p, B, T, xup, xc, ip, fp, nullptr) == MLSTM_OK);
    EXPECT(mlstm_block_conv_gates(&p, B, T, xup, xup, ip, fp, nullptr) == MLSTM_ERR_ALIAS);
    EXPECT(mlstm_block_conv_gates(&p, B, T, xup, xc, ip, nullptr, nullptr) == MLSTM_ERR_NULLPTR);
    void* hc = take(B * H * T * dv * 2);
    void* y = take(B * T * E * 2);
    EXPECT(mlstm_block_groupnorm_gate(&p, B, T, hc, xc, xup, y, nullptr) == MLSTM_OK);
    EXPECT(mlstm_block_groupnorm_gate(&p, B, T, hc, xc, xup, xc, nullptr) == MLSTM_ERR_ALIAS);
    EXPECT(mlstm_layernorm_bf16(x, p.ln_w, p.ln_b, out, B * T, D, 1e-5f, nullptr) == MLSTM_OK);
    EXPECT(mlstm_layernorm_bf16(x, p.ln_w, p.ln_b, out, B * T, 12, 1e-5f, nullptr) == MLSTM_ERR_BAD_SHAPE);
    EXPECT(mlstm_layernorm_bf16(x, p.ln_w, p.ln_b, x, B * T, D, 1e-5f, nullptr) == MLSTM_ERR_ALIAS);

    mlstm_gemm_args g;
    memset(&g, 0, sizeof(g));
    g.M = 200; g.N = 96; g.K = 128; g.batch1 = 2; g.batch2 = 3;
    g.A = take(6 * 200 * 128 * 2); g.lda = 128; g.strideA1 = 3 * 200 * 128; g.strideA2 = 200 * 128;
    g.B = take(3 * 96 * 128 * 2); g.ldb = 128; g.strideB1 = 0; g.strideB2 = 96 * 128;
    g.C = take(6 * 200 * 96 * 4); g.ldc = 96; g.strideC1 = 3 * 200 * 96; g.strideC2 = 200 * 96;
    g.c_dtype = MLSTM_FP32; g.alpha = 1.f;
    g.bias = (const float*)take(3 * 96 * 4); g.stride_bias2 = 96;
    EXPECT(mlstm_gemm_bf16(&g, nullptr) == MLSTM_OK);
    mlstm_gemm_args gb = g;
    gb.K = 100;
    EXPECT(mlstm_gemm_bf16(&gb, nullptr) == MLSTM_ERR_BAD_SHAPE);
    gb = g; gb.c_dtype = 5;
    EXPECT(mlstm_gemm_bf16(&gb, nullptr) == MLSTM_ERR_BAD_DTYPE);
    gb = g; gb.C = (char*)g.A + 64;
    EXPECT(mlstm_gemm_bf16(&gb, nullptr) == MLSTM_ERR_ALIAS);
    gb = g; gb.lda = 132;
    EXPECT(mlstm_gemm_bf16(&gb, nullptr) == MLSTM_ERR_MISALIGNED);
    gb = g; gb.c_trans = 1; gb.R = take(200 * 96 * 2); gb.ldr = 96;
    EXPECT(mlstm_gemm_bf16(&gb, nullptr) == MLSTM_ERR_UNSUPPORTED);
    EXPECT(mlstm_gemm_bf16(nullptr, nullptr) == MLSTM_ERR_NULLPTR);
  }

  {   // segments: summary and fold
    const int64_t B = 1, H = 2, T = 512, K = 128, V = 256, BH = B * H;
    mlstm_summary_args a;
    memset(&a, 0, sizeof(a));
    a.B = B; a.H = H; a.T = T; a.d_qk = K; a.d_v = V; a.dtype = MLSTM_BF16;
    a.k = take(BH * T * K * 2); a.v = take(BH * T * V * 2);
    a.i_pre = (const float*)take(BH * T * 4); a.f_pre = (const float*)take(BH * T * 4);
    a.C_out = (float*)take(BH * V * K * 4); a.n_out = (float*)take(BH * K * 4);
    a.m_out = (float*)take(BH * 4); a.G_out = (double*)take(BH * 8);
    const size_t need = mlstm_segment_summary_workspace_size(&a, 128);
    EXPECT(need > 0);
    void* ws = take(need);
    int before[20];
    for (int j = 0; j < 20; ++j) before[j] = g_calls[j];
    EXPECT(mlstm_segment_summary(&a, 128, ws, need, nullptr) == MLSTM_OK);
    EXPECT(g_calls[0] == before[0] + 1 && g_calls[16] == before[16] + 1);
    EXPECT(mlstm_segment_summary(&a, 128, ws, need - 1, nullptr) == MLSTM_ERR_WORKSPACE);
    EXPECT(mlstm_segment_summary(&a, 192, ws, need, nullptr) == MLSTM_ERR_BAD_SHAPE);   // 512 % 192
    EXPECT(mlstm_segment_summary(&a, 100, ws, need, nullptr) == MLSTM_ERR_BAD_SHAPE);
    mlstm_summary_args b = a;
    b.dtype = MLSTM_FP32;
    EXPECT(mlstm_segment_summary(&b, 128, ws, need, nullptr) == MLSTM_ERR_UNSUPPORTED);
    b = a; b.d_v = 192;
    EXPECT(mlstm_segment_summary(&b, 128, ws, need, nullptr) == MLSTM_ERR_UNSUPPORTED);
    b = a; b.G_out = nullptr;
    EXPECT(mlstm_segment_summary(&b, 128, ws, need, nullptr) == MLSTM_ERR_NULLPTR);
    b = a; b.G_out = (double*)((char*)a.G_out + 4);
    EXPECT(mlstm_segment_summary(&b, 128, ws, need, nullptr) == MLSTM_ERR_MISALIGNED);
    b = a; b.n_out = (float*)a.C_out;
    EXPECT(mlstm_segment_summary(&b, 128, ws, need, nullptr) == MLSTM_ERR_ALIAS);
    EXPECT(mlstm_segment_summary(&a, 128, (void*)a.k, need, nullptr) == MLSTM_ERR_ALIAS);
    b = a; b.T = 0;
    EXPECT(mlstm_segment_summary_workspace_size(&b, 128) == 0);
    EXPECT(mlstm_segment_summary(&b, 128, nullptr, 0, nullptr) == MLSTM_OK);
    EXPECT(g_calls[17] == before[17] + 1);
    EXPECT(mlstm_segment_summary(nullptr, 128, ws, need, nullptr) == MLSTM_ERR_NULLPTR);

    mlstm_combine_args c;
    memset(&c, 0, sizeof(c));
    c.B = B; c.H = H; c.d_qk = K; c.d_v = V; c.count = 1;
    c.Cs = a.C_out; c.ns = a.n_out; c.ms = a.m_out; c.Gs = a.G_out;
    c.C_out = (float*)take(BH * V * K * 4); c.n_out = (float*)take(BH * K * 4); c.m_out = (float*)take(BH * 4);
    EXPECT(mlstm_state_combine(&c, nullptr) == MLSTM_OK);   // from the zero state
    c.C0 = (const float*)take(BH * V * K * 4); c.n0 = (const float*)take(BH * K * 4); c.m0 = (const float*)take(BH * 4);
    EXPECT(mlstm_state_combine(&c, nullptr) == MLSTM_OK);
    EXPECT(g_calls[18] == before[18] + 2);
    mlstm_combine_args d = c;
    d.m0 = nullptr;
    EXPECT(mlstm_state_combine(&d, nullptr) == MLSTM_ERR_NULLPTR);
    d = c; d.C_out = (float*)c.C0;
    EXPECT(mlstm_state_combine(&d, nullptr) == MLSTM_ERR_ALIAS);
    d = c; d.m_out = c.n_out;
    EXPECT(mlstm_state_combine(&d, nullptr) == MLSTM_ERR_ALIAS);
    d = c; d.Gs = (const double*)((const char*)c.Gs + 4);
    EXPECT(mlstm_state_combine(&d, nullptr) == MLSTM_ERR_MISALIGNED);
    d = c; d.d_v = 0;
    EXPECT(mlstm_state_combine(&d, nullptr) == MLSTM_ERR_BAD_SHAPE);
    d = c; d.count = -1;
    EXPECT(mlstm_state_combine(&d, nullptr) == MLSTM_ERR_BAD_SHAPE);
    d = c; d.count = 0; d.Cs = nullptr; d.ns = nullptr; d.ms = nullptr; d.Gs = nullptr;
    EXPECT(mlstm_state_combine(&d, nullptr) == MLSTM_OK);   // the start state itself
    d = c; d.C_out = (float*)((char*)c.C_out + 4);
    EXPECT(mlstm_state_combine(&d, nullptr) == MLSTM_ERR_MISALIGNED);
    EXPECT(mlstm_state_combine(nullptr, nullptr) == MLSTM_ERR_NULLPTR);
  }

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi_sanitized: all expectations held\n");
  return 0;
}
