/*
 * mgattn oracle: plain, slow, f64 CPU reference for segmented softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or constant with the HIP library.
 *
 * What it computes (the plain definition, no blocking, no online softmax):
 *
 *   for every segment g = [a, b) of cu_seqlens, every head h, every query i in [a, b):
 *     keys J = [a, b)                 (causal flag set: J = [a, i])
 *     s_j  = scale * sum_c Q[i,h,c] * K[j,h,c]          for j in J
 *     m    = max_j s_j,   w_j = exp(s_j - m),   Z = sum_j w_j
 *     O[i,h,:] = sum_j (w_j / Z) * V[j,h,:]
 *
 * Sources on the pages:
 *  - vllm.cpp issue #1545 ("Muse Glimmer's vision tower runs 50 layers on the naive
 *    attention kernel"), section "Why this one is bad": the tower's attention is
 *    non-causal, H=16, head_dim=96.
 *  - same issue, section "The fix": the block-diagonal window mask is a set of
 *    per-segment row slices, each attended on its own, and the flash rung also
 *    honours a causal flag.
 *  - same issue, second comment, "Two of the three labelled uncertainties are now
 *    resolved": windows are 32x32 = 1024 patches.
 *  - vllm.cpp PR #1579 ("route the perception encoder off the correctness-grade
 *    attention kernel"), paragraph "Numerics, both halves": naive and flash kernels
 *    compute the same function and differ only in f32 summation grouping.
 *
 * Precision: every stored input element (bf16 bits or f32) is widened exactly to
 * f64; the scale is the caller's f32 value widened to f64; exp is libm's f64 exp;
 * all sums run sequentially in ascending key / channel order.  Reading taken where
 * the pages are silent: the scale is whatever the caller passes (the vision pages
 * print none; the text tower uses head_dim^-1/2); the max is subtracted before exp,
 * which changes nothing mathematically.
 *
 * Inputs are [T, H, d] row-major (element (t,h,c) at (t*H + h)*d + c).  dtype 0 = f32,
 * 1 = bf16 (raw uint16 bits), 2 = f64 (test convenience, not an ABI dtype).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2

/* Exact widening of one stored element to f64. */
static double elem(const void* base, int dtype, int64_t idx) {
  if (dtype == ORACLE_F32) {
    return (double)((const float*)base)[idx];
  } else if (dtype == ORACLE_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return ((const double*)base)[idx];
}

typedef struct {
  const void *q, *k, *v;
  int H, d, causal, dtype;
  double scale;
} problem;

/* One query row: softmax weights over its keys (w must hold b-a doubles) and the
 * weighted sum of V into o[0..d).  key_lo/key_hi are the segment bounds [a, b). */
static void attend_row(const problem* p, int64_t key_lo, int64_t key_hi, int64_t i,
                       int h, double* w, double* o) {
  const int H = p->H, d = p->d;
  int64_t last = p->causal ? i + 1 : key_hi; /* exclusive end of the keys seen */
  int64_t nk = last - key_lo;
  double m = -INFINITY;
  for (int64_t j = 0; j < nk; ++j) {
    double dot = 0.0;
    int64_t qi = (i * H + h) * (int64_t)d;
    int64_t kj = ((key_lo + j) * H + h) * (int64_t)d;
    for (int c = 0; c < d; ++c) dot += elem(p->q, p->dtype, qi + c) * elem(p->k, p->dtype, kj + c);
    w[j] = p->scale * dot;
    if (w[j] > m) m = w[j];
  }
  double z = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    w[j] = exp(w[j] - m);
    z += w[j];
  }
  for (int64_t j = 0; j < nk; ++j) w[j] /= z;
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  for (int64_t j = 0; j < nk; ++j) {
    int64_t vj = ((key_lo + j) * H + h) * (int64_t)d;
    for (int c = 0; c < d; ++c) o[c] += w[j] * elem(p->v, p->dtype, vj + c);
  }
}

/* Which segment holds token t (cu_seqlens is non-decreasing). */
static int segment_of(const int32_t* cu, int n_seg, int64_t t) {
  for (int g = 0; g < n_seg; ++g)
    if (t >= cu[g] && t < cu[g + 1]) return g;
  return -1;
}

/* ---- work split over (segment, head) pairs, one pthread per worker ---- */

typedef struct {
  const problem* p;
  const int32_t* cu;
  int n_seg;
  double* out;
  int64_t next;       /* next (segment, head) item, shared */
  pthread_mutex_t mu;
} full_job;

static void* full_worker(void* arg) {
  full_job* job = (full_job*)arg;
  const problem* p = job->p;
  int64_t max_len = 0;
  for (int g = 0; g < job->n_seg; ++g)
    if (job->cu[g + 1] - job->cu[g] > max_len) max_len = job->cu[g + 1] - job->cu[g];
  double* w = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
  int64_t n_items = (int64_t)job->n_seg * p->H;
  for (;;) {
    pthread_mutex_lock(&job->mu);
    int64_t item = job->next++;
    pthread_mutex_unlock(&job->mu);
    if (item >= n_items) break;
    int g = (int)(item / p->H), h = (int)(item % p->H);
    int64_t a = job->cu[g], b = job->cu[g + 1];
    for (int64_t i = a; i < b; ++i)
      attend_row(p, a, b, i, h, w, job->out + (i * p->H + h) * (int64_t)p->d);
  }
  free(w);
  return NULL;
}

static int check_args(const int32_t* cu, int n_seg, int H, int d, int dtype) {
  if (!cu || n_seg < 1 || H < 1 || d < 1) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16 && dtype != ORACLE_F64) return -1;
  if (cu[0] != 0) return -1;
  for (int g = 0; g < n_seg; ++g)
    if (cu[g + 1] < cu[g]) return -1;
  return 0;
}

/* Whole output [T, H, d] in f64.  Returns 0, or -1 on malformed arguments. */
int mgattn_oracle_f64(const void* q, const void* k, const void* v, double* out,
                      const int32_t* cu_seqlens, int n_seg, int H, int d, float scale,
                      int causal, int dtype, int n_threads) {
  if (check_args(cu_seqlens, n_seg, H, d, dtype) != 0 || !q || !k || !v || !out) return -1;
  problem p = {q, k, v, H, d, causal != 0, dtype, (double)scale};
  full_job job;
  job.p = &p;
  job.cu = cu_seqlens;
  job.n_seg = n_seg;
  job.out = out;
  job.next = 0;
  pthread_mutex_init(&job.mu, NULL);
  if (n_threads < 1) n_threads = 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n_threads);
  int started = 0;
  for (int t = 0; t < n_threads; ++t)
    if (pthread_create(&th[t], NULL, full_worker, &job) == 0) ++started;
  if (started == 0) full_worker(&job);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&job.mu);
  return 0;
}

/* ---- selected (token, head) rows only, for full-size checks ---- */

typedef struct {
  const problem* p;
  const int32_t* cu;
  int n_seg;
  int64_t n_rows;
  const int64_t* tok;
  const int32_t* head;
  double* out; /* [n_rows, d] */
  int64_t next;
  int bad;
  pthread_mutex_t mu;
} rows_job;

static void* rows_worker(void* arg) {
  rows_job* job = (rows_job*)arg;
  const problem* p = job->p;
  double* w = NULL;
  int64_t w_cap = 0;
  for (;;) {
    pthread_mutex_lock(&job->mu);
    int64_t r = job->next++;
    pthread_mutex_unlock(&job->mu);
    if (r >= job->n_rows) break;
    int64_t t = job->tok[r];
    int h = job->head[r];
    int g = segment_of(job->cu, job->n_seg, t);
    if (g < 0 || h < 0 || h >= p->H) {
      pthread_mutex_lock(&job->mu);
      job->bad = 1;
      pthread_mutex_unlock(&job->mu);
      continue;
    }
    int64_t a = job->cu[g], b = job->cu[g + 1];
    if (b - a > w_cap) {
      free(w);
      w_cap = b - a;
      w = (double*)malloc(sizeof(double) * (size_t)w_cap);
    }
    attend_row(p, a, b, t, h, w, job->out + r * (int64_t)p->d);
  }
  free(w);
  return NULL;
}

/* Rows O[tok[r], head[r], :] for r < n_rows into out[r*d .. r*d+d).  Returns 0, or -1
 * on malformed arguments or a token outside every segment. */
int mgattn_oracle_rows_f64(const void* q, const void* k, const void* v, double* out,
                           const int32_t* cu_seqlens, int n_seg, int H, int d, float scale,
                           int causal, int dtype, int64_t n_rows, const int64_t* tok,
                           const int32_t* head, int n_threads) {
  if (check_args(cu_seqlens, n_seg, H, d, dtype) != 0 || !q || !k || !v || !out) return -1;
  if (n_rows < 0 || (n_rows > 0 && (!tok || !head))) return -1;
  problem p = {q, k, v, H, d, causal != 0, dtype, (double)scale};
  rows_job job;
  job.p = &p;
  job.cu = cu_seqlens;
  job.n_seg = n_seg;
  job.n_rows = n_rows;
  job.tok = tok;
  job.head = head;
  job.out = out;
  job.next = 0;
  job.bad = 0;
  pthread_mutex_init(&job.mu, NULL);
  if (n_threads < 1) n_threads = 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n_threads);
  int started = 0;
  for (int t = 0; t < n_threads; ++t)
    if (pthread_create(&th[t], NULL, rows_worker, &job) == 0) ++started;
  if (started == 0) rows_worker(&job);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th);
  pthread_mutex_destroy(&job.mu);
  return job.bad ? -1 : 0;
}

/* Softmax weights of one query row (token t, head h) over the keys it sees, in key
 * order from the segment start; w must hold the segment length.  Returns the number
 * of weights written, or -1. */
int64_t mgattn_oracle_weights_f64(const void* q, const void* k, const void* v,
                                  const int32_t* cu_seqlens, int n_seg, int H, int d,
                                  float scale, int causal, int dtype, int64_t t, int h,
                                  double* w, double* o) {
  if (check_args(cu_seqlens, n_seg, H, d, dtype) != 0 || !q || !k || !v || !w || !o) return -1;
  int g = segment_of(cu_seqlens, n_seg, t);
  if (g < 0 || h < 0 || h >= H) return -1;
  problem p = {q, k, v, H, d, causal != 0, dtype, (double)scale};
  int64_t a = cu_seqlens[g], b = cu_seqlens[g + 1];
  attend_row(&p, a, b, t, h, w, o);
  return causal ? t + 1 - a : b - a;
}
