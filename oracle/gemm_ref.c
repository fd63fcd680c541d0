/*
 * ORACLE -- test infrastructure only.  Nothing on the product path may link,
 * load or call this file; only the tests, the smoke check and the bench's CPU
 * baseline leg do.
 *
 * What it computes: the plain product R = A . B in fp64, with A the gathered
 * M x K activation (every shard at its natural rows) and B the K x N weight.
 * The chunk-overlapped kernel must reach exactly this result: the Syncopate
 * review page (pith.science, "Core claim" and "What would settle it") states
 * that the transformed fused kernel keeps the local kernel's semantics and
 * that its outputs should match the unfused kernel's; the Syncopate summary
 * page ("Core method", paper sec. 5) describes the local kernel as an ordinary
 * tiled GEMM.  So the oracle is the definition of a matrix product, written
 * out: one fp64 accumulator per output element, k ascending.
 *
 * Inputs are bfloat16 bit patterns; each is widened exactly to fp64.  A
 * bf16 x bf16 product is exact in fp64, so the only rounding is in the fp64
 * running sum (error <= K * 2^-53 * sum|a*b|).
 *
 * B layouts: 0 = row-major [K][N]; 1 = row-major [N][K] (a Linear layer's
 * weight stored output-major).
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

/* B element (k, j) for either layout. */
static double b_at(const uint16_t* B, int b_layout, int64_t N, int64_t K, int64_t k, int64_t j) {
  return b_layout == 0 ? bf16_to_f64(B[k * N + j]) : bf16_to_f64(B[j * K + k]);
}

typedef struct {
  const uint16_t* A;
  const uint16_t* B;
  int b_layout;
  int64_t M, N, K;
  const int64_t* rows; /* NULL: every row; else a list of output rows */
  const int64_t* cols; /* sampled mode: column per sample */
  int64_t count;       /* sampled mode: number of samples */
  double* R;
  int nthreads, tid;
  double* bcol; /* scratch: one widened column of B, K entries */
} job_t;

/* Full product: thread tid owns rows tid, tid+nthreads, ... */
static void* full_worker(void* p) {
  job_t* j = (job_t*)p;
  double* arow = (double*)malloc(sizeof(double) * (size_t)j->K);
  for (int64_t i = j->tid; i < j->M; i += j->nthreads) {
    for (int64_t k = 0; k < j->K; ++k) arow[k] = bf16_to_f64(j->A[i * j->K + k]);
    for (int64_t c = 0; c < j->N; ++c) {
      double acc = 0.0;
      for (int64_t k = 0; k < j->K; ++k) acc += arow[k] * b_at(j->B, j->b_layout, j->N, j->K, k, c);
      j->R[i * j->N + c] = acc;
    }
  }
  free(arow);
  return NULL;
}

/* Sampled elements: R[s] = sum_k A[rows[s]][k] * B[k][cols[s]]. */
static void* sampled_worker(void* p) {
  job_t* j = (job_t*)p;
  for (int64_t s = j->tid; s < j->count; s += j->nthreads) {
    int64_t i = j->rows[s], c = j->cols[s];
    double acc = 0.0;
    for (int64_t k = 0; k < j->K; ++k)
      acc += bf16_to_f64(j->A[i * j->K + k]) * b_at(j->B, j->b_layout, j->N, j->K, k, c);
    j->R[s] = acc;
  }
  return NULL;
}

static int run(job_t* base, void* (*fn)(void*)) {
  int nt = base->nthreads < 1 ? 1 : base->nthreads;
  pthread_t* th = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
  job_t* jobs = (job_t*)calloc((size_t)nt, sizeof(job_t));
  if (!th || !jobs) { free(th); free(jobs); return -1; }
  for (int t = 0; t < nt; ++t) {
    jobs[t] = *base;
    jobs[t].nthreads = nt;
    jobs[t].tid = t;
    pthread_create(&th[t], NULL, fn, &jobs[t]);
  }
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  free(th);
  free(jobs);
  return 0;
}

/* R[M][N] = A[M][K] . B  (fp64).  Returns 0 on success. */
int oracle_gemm_f64(const uint16_t* A, const uint16_t* B, int b_layout, int64_t M, int64_t N,
                    int64_t K, double* R, int nthreads) {
  if (!A || !B || !R || M < 0 || N < 0 || K < 0 || (b_layout != 0 && b_layout != 1)) return -1;
  job_t j = {A, B, b_layout, M, N, K, NULL, NULL, 0, R, nthreads, 0, NULL};
  return run(&j, full_worker);
}

/* out[s] = (A . B)[rows[s]][cols[s]] for s < count (fp64). */
int oracle_gemm_f64_sampled(const uint16_t* A, const uint16_t* B, int b_layout, int64_t M,
                            int64_t N, int64_t K, const int64_t* rows, const int64_t* cols,
                            int64_t count, double* out, int nthreads) {
  if (!A || !B || !out || !rows || !cols || (b_layout != 0 && b_layout != 1)) return -1;
  for (int64_t s = 0; s < count; ++s)
    if (rows[s] < 0 || rows[s] >= M || cols[s] < 0 || cols[s] >= N) return -1;
  job_t j = {A, B, b_layout, M, N, K, rows, cols, count, out, nthreads, 0, NULL};
  return run(&j, sampled_worker);
}
