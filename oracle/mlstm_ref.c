/*
 * mlstm_ref.c -- plain float64 CPU oracle of the mLSTM cell recurrence, in C.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, the smoke check and the bench's CPU
 * baseline load it (through oracle/mlstm_ref.py). It shares no code, header,
 * table or helper with the HIP library. It exists because the NumPy oracle
 * (mlstm_oracle.py) is memory-bound at the full workload sizes; this is the
 * same step recurrence, one (batch, head) sequence per thread, so that every
 * output of the 7B-layer, long-context and decode workloads can be compared.
 *
 * What it computes (xLSTM guide, aifetchly blog: "mLSTM: Matrix Key-Value
 * Memory and Covariance Updates", recurrent formulation; "The Stabilizer
 * State"; exponential input gate of "The Innovation: Exponential Gating and
 * Dynamic Normalization"), per sequence, for t = 1..T:
 *
 *   log f = logsigmoid(f~) = min(f~, 0) - log1p(exp(-|f~|))
 *   m'    = max(log f + m, i~)
 *   C~   <- exp(log f + m - m') C~ + exp(i~ - m') v k^T      (d_v x d_qk)
 *   n~   <- exp(log f + m - m') n~ + exp(i~ - m') k
 *   h     = sigmoid(o~) * (C~ q) / max(|n~ . q|, exp(-m'))
 *
 * with the readings of the NumPy oracle: logsigmoid forget gate, exp input
 * gate, the floor of 1 on the true (unstabilised) normaliser, C oriented
 * d_v x d_qk with h = C q, no 1/sqrt(d) scaling and no epsilon.
 *
 * Pinned in tests/test_oracle_ref.py against the pinned NumPy oracle and
 * directly against the brute-force product form of the pages' closed form.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

static double logsigmoid(double x) { return fmin(x, 0.0) - log1p(exp(-fabs(x))); }

static double sigmoid(double x) {
  const double e = exp(-fabs(x));
  return x >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

typedef struct {
  int64_t BH, T, K, V;
  const float *q, *k, *v, *i_pre, *f_pre, *o_pre;
  double *C, *n, *m, *h;
  int64_t first, stride;   /* this worker takes sequences first, first + stride, ... */
  double* num;             /* d_v scratch of this worker */
} Job;

/* The recurrence over T steps for one sequence s, state updated in place. */
static void run_sequence(const Job* J, int64_t s) {
  const int64_t T = J->T, K = J->K, V = J->V;
  double* C = J->C + s * V * K;
  double* n = J->n + s * K;
  double m = J->m[s];
  double* num = J->num;
  for (int64_t t = 0; t < T; ++t) {
    const int64_t tok = s * T + t;
    const float* q = J->q + tok * K;
    const float* k = J->k + tok * K;
    const float* v = J->v + tok * V;
    const float* o = J->o_pre + tok * V;
    const double ip = (double)J->i_pre[tok];
    const double lf = logsigmoid((double)J->f_pre[tok]);
    const double m_new = fmax(lf + m, ip);
    const double fs = exp(lf + m - m_new);   /* stabilised forget factor */
    const double is = exp(ip - m_new);       /* stabilised input factor */
    double nq = 0.0;
    for (int64_t c = 0; c < K; ++c) {
      n[c] = fs * n[c] + is * (double)k[c];
      nq += n[c] * (double)q[c];
    }
    for (int64_t r = 0; r < V; ++r) {
      double* row = C + r * K;
      const double iv = is * (double)v[r];
      double acc = 0.0;
      for (int64_t c = 0; c < K; ++c) {
        row[c] = fs * row[c] + iv * (double)k[c];
        acc += row[c] * (double)q[c];
      }
      num[r] = acc;
    }
    const double den = fmax(fabs(nq), exp(-m_new));
    double* h = J->h + tok * V;
    for (int64_t r = 0; r < V; ++r) h[r] = sigmoid((double)o[r]) * num[r] / den;
    m = m_new;
  }
  J->m[s] = m;
}

static void* worker(void* p) {
  const Job* J = (const Job*)p;
  for (int64_t s = J->first; s < J->BH; s += J->stride) run_sequence(J, s);
  return NULL;
}

/*
 * BH independent sequences of T tokens. Inputs are float32 arrays (exactly
 * the values given to the GPU, bf16 ones already widened):
 *   q, k [BH, T, K]; v, o_pre [BH, T, V]; i_pre, f_pre [BH, T].
 * State, float64, stabilised units, updated in place (the caller sets the
 * initial state; zeros with m = 0 for the zero state):
 *   C [BH, V, K], n [BH, K], m [BH].
 * Output h [BH, T, V] float64. Returns 0, or -1 when threads cannot start.
 */
int mlstm_ref_run(int64_t BH, int64_t T, int64_t K, int64_t V, const float* q, const float* k,
                  const float* v, const float* i_pre, const float* f_pre, const float* o_pre,
                  double* C, double* n, double* m, double* h, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > BH) nthreads = (int)BH;
  if (nthreads < 1) return 0;
  Job* jobs = (Job*)calloc((size_t)nthreads, sizeof(Job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  double* scratch = (double*)calloc((size_t)nthreads * (size_t)V, sizeof(double));
  if (!jobs || !th || !scratch) {
    free(jobs); free(th); free(scratch);
    return -1;
  }
  int started = 0, rc = 0;
  for (int w = 0; w < nthreads; ++w) {
    Job* J = &jobs[w];
    J->BH = BH; J->T = T; J->K = K; J->V = V;
    J->q = q; J->k = k; J->v = v; J->i_pre = i_pre; J->f_pre = f_pre; J->o_pre = o_pre;
    J->C = C; J->n = n; J->m = m; J->h = h;
    J->first = w; J->stride = nthreads;
    J->num = scratch + (size_t)w * (size_t)V;
  }
  for (int w = 0; w < nthreads; ++w) {
    if (pthread_create(&th[w], NULL, worker, &jobs[w]) != 0) { rc = -1; break; }
    ++started;
  }
  for (int w = 0; w < started; ++w) pthread_join(th[w], NULL);
  free(jobs); free(th); free(scratch);
  return rc;
}

/* ------------------------------------------------------------------ gradients
 *
 * Reverse mode of the same recurrence (the chain rule step by step), for a
 * loss whose gradient dh = dL/dh is given. With the stabilised factors
 * f'_t = exp(log f_t + m_{t-1} - m_t) and i'_t = exp(i~_t - m_t) of the
 * forward, den~_t = max(|z~_t|, exp(-m_t)), z~_t = n~_t . q_t and
 * num~_t = C~_t q_t:
 *
 *   g_t   = dh_t sigmoid(o~_t) / den~_t
 *   dz_t  = -sign(z~_t) [|z~_t| > exp(-m_t)] (g_t . num~_t) / den~_t
 *   dq_t  = C~_t^T g_t + dz_t n~_t
 *   do~_t = dh_t (num~_t / den~_t) sigmoid(o~_t) (1 - sigmoid(o~_t))
 *   E_t   = g_t q_t^T + f'_{t+1} E_{t+1},  e_t = dz_t q_t + f'_{t+1} e_{t+1}
 *   dv_t  = i'_t E_t k_t,  dk_t = i'_t (E_t^T v_t + e_t),  di~_t = k_t . dk_t
 *   df~_t = f'_t (<E_t, C~_{t-1}> + e_t . n~_{t-1}) sigmoid(-f~_t)
 *   dC~_0 = f'_1 E_1,  dn~_0 = f'_1 e_1,  dm_0 = <dC~_0, C~_0> + dn~_0 . n~_0
 *
 * (E, e are the adjoints of the true state scaled by exp(m_t).) The forward
 * sweep computes g, dz, dq and do~ and keeps the state every S steps; the
 * reverse sweep recomputes each S-step segment's states from its checkpoint
 * and walks it backwards. Pinned in tests against the NumPy gradient oracle.
 */
typedef struct {
  int64_t BH, T, K, V, S;
  const float *q, *k, *v, *i_pre, *f_pre, *o_pre, *dh;
  const double *C0, *n0, *m0;
  double *dq, *dk, *dv, *di, *df, *dout, *dC0, *dn0, *dm0;
  int64_t first, stride;
  int failed;
} BwdJob;

static int bwd_sequence(const BwdJob* J, int64_t s) {
  const int64_t T = J->T, K = J->K, V = J->V, S = J->S;
  const int64_t VK = V * K;
  const int64_t nseg = (T + S - 1) / S;
  double* C = (double*)calloc((size_t)VK, sizeof(double));
  double* n = (double*)calloc((size_t)K, sizeof(double));
  double* E = (double*)calloc((size_t)VK, sizeof(double));
  double* e = (double*)calloc((size_t)K, sizeof(double));
  double* num = (double*)calloc((size_t)V, sizeof(double));
  double* ckC = (double*)calloc((size_t)(nseg > 0 ? nseg : 1) * (size_t)VK, sizeof(double));
  double* ckn = (double*)calloc((size_t)(nseg > 0 ? nseg : 1) * (size_t)K, sizeof(double));
  double* segC = (double*)calloc((size_t)S * (size_t)VK, sizeof(double));
  double* segn = (double*)calloc((size_t)S * (size_t)K, sizeof(double));
  double* fp = (double*)calloc((size_t)(T > 0 ? T : 1), sizeof(double));
  double* ip = (double*)calloc((size_t)(T > 0 ? T : 1), sizeof(double));
  double* dz = (double*)calloc((size_t)(T > 0 ? T : 1), sizeof(double));
  double* g = (double*)calloc((size_t)(T > 0 ? T : 1) * (size_t)V, sizeof(double));
  int ok = C && n && E && e && num && ckC && ckn && segC && segn && fp && ip && dz && g;
  if (ok) {
    if (J->C0) {
      for (int64_t x = 0; x < VK; ++x) C[x] = J->C0[s * VK + x];
      for (int64_t c = 0; c < K; ++c) n[c] = J->n0[s * K + c];
    }
    double m = J->m0 ? J->m0[s] : 0.0;
    /* forward sweep */
    for (int64_t t = 0; t < T; ++t) {
      if (t % S == 0) {
        for (int64_t x = 0; x < VK; ++x) ckC[(t / S) * VK + x] = C[x];
        for (int64_t c = 0; c < K; ++c) ckn[(t / S) * K + c] = n[c];
      }
      const int64_t tok = s * T + t;
      const float* q = J->q + tok * K;
      const float* k = J->k + tok * K;
      const float* v = J->v + tok * V;
      const float* o = J->o_pre + tok * V;
      const float* dh = J->dh + tok * V;
      const double ipre = (double)J->i_pre[tok];
      const double lf = logsigmoid((double)J->f_pre[tok]);
      const double m_new = fmax(lf + m, ipre);
      fp[t] = exp(lf + m - m_new);
      ip[t] = exp(ipre - m_new);
      double z = 0.0;
      for (int64_t c = 0; c < K; ++c) {
        n[c] = fp[t] * n[c] + ip[t] * (double)k[c];
        z += n[c] * (double)q[c];
      }
      for (int64_t r = 0; r < V; ++r) {
        double* row = C + r * K;
        const double iv = ip[t] * (double)v[r];
        double acc = 0.0;
        for (int64_t c = 0; c < K; ++c) {
          row[c] = fp[t] * row[c] + iv * (double)k[c];
          acc += row[c] * (double)q[c];
        }
        num[r] = acc;
      }
      const double floor_ = exp(-m_new);
      const double den = fmax(fabs(z), floor_);
      double gnum = 0.0;
      double* gt = g + t * V;
      double* dout = J->dout + tok * V;
      for (int64_t r = 0; r < V; ++r) {
        const double og = sigmoid((double)o[r]);
        gt[r] = (double)dh[r] * og / den;
        gnum += gt[r] * num[r];
        dout[r] = (double)dh[r] * (num[r] / den) * og * (1.0 - og);
      }
      dz[t] = fabs(z) > floor_ ? -(z > 0.0 ? 1.0 : -1.0) * gnum / den : 0.0;
      double* dq = J->dq + tok * K;
      for (int64_t c = 0; c < K; ++c) dq[c] = dz[t] * n[c];
      for (int64_t r = 0; r < V; ++r) {
        const double* row = C + r * K;
        for (int64_t c = 0; c < K; ++c) dq[c] += row[c] * gt[r];
      }
      m = m_new;
    }
    /* reverse sweep, one segment at a time */
    double f_next = 0.0;
    for (int64_t sg = nseg - 1; sg >= 0; --sg) {
      const int64_t t0 = sg * S;
      const int64_t t1 = t0 + S < T ? t0 + S : T;
      /* segC[i], segn[i]: state before step t0 + i */
      for (int64_t x = 0; x < VK; ++x) segC[x] = ckC[sg * VK + x];
      for (int64_t c = 0; c < K; ++c) segn[c] = ckn[sg * K + c];
      for (int64_t t = t0; t + 1 < t1; ++t) {
        const int64_t i = t - t0, tok = s * T + t;
        const float* k = J->k + tok * K;
        const float* v = J->v + tok * V;
        for (int64_t r = 0; r < V; ++r) {
          const double iv = ip[t] * (double)v[r];
          for (int64_t c = 0; c < K; ++c)
            segC[(i + 1) * VK + r * K + c] = fp[t] * segC[i * VK + r * K + c] + iv * (double)k[c];
        }
        for (int64_t c = 0; c < K; ++c) segn[(i + 1) * K + c] = fp[t] * segn[i * K + c] + ip[t] * (double)k[c];
      }
      for (int64_t t = t1 - 1; t >= t0; --t) {
        const int64_t i = t - t0, tok = s * T + t;
        const float* q = J->q + tok * K;
        const float* k = J->k + tok * K;
        const float* v = J->v + tok * V;
        const double* gt = g + t * V;
        for (int64_t c = 0; c < K; ++c) e[c] = dz[t] * (double)q[c] + f_next * e[c];
        for (int64_t r = 0; r < V; ++r)
          for (int64_t c = 0; c < K; ++c) E[r * K + c] = gt[r] * (double)q[c] + f_next * E[r * K + c];
        double* dk = J->dk + tok * K;
        double* dv = J->dv + tok * V;
        for (int64_t c = 0; c < K; ++c) dk[c] = e[c];
        double ec = 0.0;
        for (int64_t r = 0; r < V; ++r) {
          const double* row = E + r * K;
          const double* prev = segC + i * VK + r * K;
          double ek = 0.0;
          for (int64_t c = 0; c < K; ++c) {
            ek += row[c] * (double)k[c];
            dk[c] += row[c] * (double)v[r];
            ec += row[c] * prev[c];
          }
          dv[r] = ip[t] * ek;
        }
        double kd = 0.0;
        for (int64_t c = 0; c < K; ++c) {
          dk[c] *= ip[t];
          kd += (double)k[c] * dk[c];
          ec += e[c] * segn[i * K + c];
        }
        J->di[tok] = kd;
        J->df[tok] = fp[t] * ec * sigmoid(-(double)J->f_pre[tok]);
        f_next = fp[t];
      }
    }
    double dm = 0.0;
    for (int64_t x = 0; x < VK; ++x) {
      J->dC0[s * VK + x] = f_next * E[x];
      if (J->C0) dm += J->dC0[s * VK + x] * J->C0[s * VK + x];
    }
    for (int64_t c = 0; c < K; ++c) {
      J->dn0[s * K + c] = f_next * e[c];
      if (J->C0) dm += J->dn0[s * K + c] * J->n0[s * K + c];
    }
    J->dm0[s] = dm;
  }
  free(C); free(n); free(E); free(e); free(num); free(ckC); free(ckn);
  free(segC); free(segn); free(fp); free(ip); free(dz); free(g);
  return ok ? 0 : -1;
}

static void* bwd_worker(void* p) {
  BwdJob* J = (BwdJob*)p;
  for (int64_t s = J->first; s < J->BH; s += J->stride)
    if (bwd_sequence(J, s) != 0) J->failed = 1;
  return NULL;
}

/*
 * Gradients of sum(dh * h) for BH independent sequences. Inputs as for
 * mlstm_ref_run plus dh [BH, T, V] (float32); optional initial state
 * C0 [BH, V, K], n0 [BH, K], m0 [BH] (float64, stabilised units; NULL = zero
 * state with m = 0). Outputs, float64: dq, dk [BH, T, K]; dv, dout (of the
 * output-gate preactivation) [BH, T, V]; di, df [BH, T]; dC0 [BH, V, K],
 * dn0 [BH, K], dm0 [BH]. seg = checkpoint interval (<= 0: about sqrt(T)).
 * Returns 0, or -1 when memory or threads are not available.
 */
int mlstm_ref_bwd(int64_t BH, int64_t T, int64_t K, int64_t V, const float* q, const float* k,
                  const float* v, const float* i_pre, const float* f_pre, const float* o_pre,
                  const float* dh, const double* C0, const double* n0, const double* m0,
                  double* dq, double* dk, double* dv, double* di, double* df, double* dout,
                  double* dC0, double* dn0, double* dm0, int64_t seg, int nthreads) {
  if (seg <= 0) {
    seg = 1;
    while (seg * seg < T) ++seg;
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > BH) nthreads = (int)BH;
  if (nthreads < 1) return 0;
  BwdJob* jobs = (BwdJob*)calloc((size_t)nthreads, sizeof(BwdJob));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs); free(th);
    return -1;
  }
  for (int w = 0; w < nthreads; ++w) {
    BwdJob* J = &jobs[w];
    J->BH = BH; J->T = T; J->K = K; J->V = V; J->S = seg;
    J->q = q; J->k = k; J->v = v; J->i_pre = i_pre; J->f_pre = f_pre; J->o_pre = o_pre; J->dh = dh;
    J->C0 = C0; J->n0 = n0; J->m0 = m0;
    J->dq = dq; J->dk = dk; J->dv = dv; J->di = di; J->df = df; J->dout = dout;
    J->dC0 = dC0; J->dn0 = dn0; J->dm0 = dm0;
    J->first = w; J->stride = nthreads;
  }
  int started = 0, rc = 0;
  for (int w = 0; w < nthreads; ++w) {
    if (pthread_create(&th[w], NULL, bwd_worker, &jobs[w]) != 0) { rc = -1; break; }
    ++started;
  }
  for (int w = 0; w < started; ++w) pthread_join(th[w], NULL);
  for (int w = 0; w < started; ++w)
    if (jobs[w].failed) rc = -1;
  free(jobs); free(th);
  return rc;
}
