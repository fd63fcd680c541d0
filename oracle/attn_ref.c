/*
 * ORACLE -- test infrastructure only.  Nothing on the product path may link,
 * load or call this file; only the tests, the smoke check and the bench's CPU
 * baseline leg do.
 *
 * What it computes: plain softmax attention over every key of every KV block,
 * non-causal, grouped-query (query head h reads KV head h / (Hq/Hkv)), in
 * fp64, by the direct two-pass form:
 *     s_j = scale * <Q[q,h,:], K[j,g,:]>              for all keys j
 *     m   = max_j s_j,   l = sum_j exp(s_j - m)
 *     O[q,h,:] = sum_j exp(s_j - m) V[j,g,:] / l,     LSE[h,q] = m + ln l
 * The Syncopate summary page ("Experiments", paper sec. 6.1 and Fig. 9)
 * evaluates ring attention, where each rank's queries meet the KV blocks that
 * travel around the ring; the blocks together are the whole key sequence, so
 * the ring result must equal attention over all keys at once.  The per-block
 * online merge the ring kernel performs is a re-association of this sum; the
 * merge itself is written out in attention.py only to check that identity.
 *
 * Layouts: Q [Sq][Hq][d], K and V [Skv][Hkv][d] (row-major, bf16 bits);
 * O [Sq][Hq][d] fp64; LSE [Hq][Sq] fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

typedef struct {
  const uint16_t *Q, *K, *V;
  int64_t Sq, Skv;
  int Hq, Hkv, d;
  double scale;
  const int64_t* qidx; /* sampled mode: query row per sample (NULL = all) */
  const int32_t* hidx; /* sampled mode: query head per sample */
  int64_t count;       /* number of (q,h) pairs */
  double *O, *LSE;
  int nthreads, tid;
} job_t;

/* One (q, h) pair; writes d outputs to o and the log-sum-exp to *lse. */
static void one_row(const job_t* j, int64_t q, int h, double* s, double* o, double* lse) {
  const int g = h / (j->Hq / j->Hkv);
  const uint16_t* qv = j->Q + ((q * j->Hq) + h) * j->d;
  double m = -INFINITY;
  for (int64_t k = 0; k < j->Skv; ++k) {
    const uint16_t* kv = j->K + ((k * j->Hkv) + g) * j->d;
    double dot = 0.0;
    for (int e = 0; e < j->d; ++e) dot += bf16_to_f64(qv[e]) * bf16_to_f64(kv[e]);
    s[k] = dot * j->scale;
    if (s[k] > m) m = s[k];
  }
  double l = 0.0;
  for (int e = 0; e < j->d; ++e) o[e] = 0.0;
  for (int64_t k = 0; k < j->Skv; ++k) {
    const double p = exp(s[k] - m);
    l += p;
    const uint16_t* vv = j->V + ((k * j->Hkv) + g) * j->d;
    for (int e = 0; e < j->d; ++e) o[e] += p * bf16_to_f64(vv[e]);
  }
  for (int e = 0; e < j->d; ++e) o[e] /= l;
  *lse = m + log(l);
}

static void* worker(void* p) {
  job_t* j = (job_t*)p;
  double* s = (double*)malloc(sizeof(double) * (size_t)(j->Skv > 0 ? j->Skv : 1));
  for (int64_t t = j->tid; t < j->count; t += j->nthreads) {
    int64_t q;
    int h;
    if (j->qidx) {
      q = j->qidx[t];
      h = j->hidx[t];
      one_row(j, q, h, s, j->O + t * j->d, j->LSE + t);
    } else {
      q = t / j->Hq;
      h = (int)(t % j->Hq);
      one_row(j, q, h, s, j->O + ((q * j->Hq) + h) * j->d, j->LSE + (int64_t)h * j->Sq + q);
    }
  }
  free(s);
  return NULL;
}

static int run(job_t* base) {
  int nt = base->nthreads < 1 ? 1 : base->nthreads;
  pthread_t* th = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
  job_t* jobs = (job_t*)calloc((size_t)nt, sizeof(job_t));
  if (!th || !jobs) { free(th); free(jobs); return -1; }
  for (int t = 0; t < nt; ++t) {
    jobs[t] = *base;
    jobs[t].nthreads = nt;
    jobs[t].tid = t;
    pthread_create(&th[t], NULL, worker, &jobs[t]);
  }
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
  return 0;
}

static int valid(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t Sq, int64_t Skv,
                 int Hq, int Hkv, int d) {
  return Q && K && V && Sq >= 0 && Skv > 0 && Hq > 0 && Hkv > 0 && d > 0 && Hq % Hkv == 0;
}

/* Every (q, h): O [Sq][Hq][d], LSE [Hq][Sq]. */
int oracle_attention_f64(const uint16_t* Q, const uint16_t* K, const uint16_t* V, int64_t Sq,
                         int64_t Skv, int Hq, int Hkv, int d, double scale, double* O, double* LSE,
                         int nthreads) {
  if (!valid(Q, K, V, Sq, Skv, Hq, Hkv, d) || !O || !LSE) return -1;
  job_t j = {Q, K, V, Sq, Skv, Hq, Hkv, d, scale, NULL, NULL, Sq * Hq, O, LSE, nthreads, 0};
  return run(&j);
}

/* Sampled pairs (qidx[t], hidx[t]): O [count][d], LSE [count]. */
int oracle_attention_f64_sampled(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                 int64_t Sq, int64_t Skv, int Hq, int Hkv, int d, double scale,
                                 const int64_t* qidx, const int32_t* hidx, int64_t count, double* O,
                                 double* LSE, int nthreads) {
  if (!valid(Q, K, V, Sq, Skv, Hq, Hkv, d) || !O || !LSE || !qidx || !hidx) return -1;
  for (int64_t t = 0; t < count; ++t)
    if (qidx[t] < 0 || qidx[t] >= Sq || hidx[t] < 0 || hidx[t] >= Hq) return -1;
  job_t j = {Q, K, V, Sq, Skv, Hq, Hkv, d, scale, qidx, hidx, count, O, LSE, nthreads, 0};
  return run(&j);
}
