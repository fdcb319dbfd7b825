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
