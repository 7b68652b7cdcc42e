/*
 * attn_oracle.c -- fp64 CPU oracle for grouped-query softmax attention (forward).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite (tests/),
 * __graft_entry__.smoke() and the cpu_baseline leg of bench.py may load or
 * call this library.  The GPU path never links, imports or calls it, and it
 * shares no code, header, table or helper with the GPU path.
 *
 * What it computes.  The workload of the PipeThreader evaluation is the
 * FlashAttention forward pass at LLaMA3-8B/70B head shapes (page
 * "PipeThreader: Software-Defined Pipelining for Efficient DNN Execution
 * (OSDI 2025)" summary, section "实验与结果", citing the paper's section 6.2 /
 * Fig.12), decomposed there into load / mma / softmax sTasks (same page,
 * section "核心方法").  FlashAttention's online softmax is an exact algebraic
 * rearrangement of plain softmax attention, so this oracle evaluates the
 * plain definition directly, with no tiling, no running maximum and no
 * rescaling:
 *
 *   g = Hq / Hkv,  c = floor(h / g)        (query head h reads KV head c)
 *   A(i) = {0..i+Sk-Sq} if causal else {0..Sk-1}  (key j allowed for query i)
 *   s_j  = scale * sum_{d ascending} q[b,i,h,d] * k[b,j,c,d]      j in A(i)
 *   m    = max_j s_j
 *   w_j  = exp(s_j - m)
 *   l    = sum_{j ascending} w_j
 *   O[b,i,h,:] = (sum_{j ascending} w_j * v[b,j,c,:]) / l
 *   LSE[b,h,i] = m + log(l)                (natural log of the scaled scores)
 *
 * The readings it takes where the pages are silent (GQA head map; causal
 * alignment at the bottom right, so query i sits at key position i + Sk - Sq
 * and the square case Sq == Sk is the usual j <= i; natural-log LSE of the
 * scaled scores; the scale as the fp32 value the GPU receives) are stated in
 * the comments above.  Causal needs Sq <= Sk, so every row has a key.  All
 * arithmetic is IEEE binary64 from the exact fp16 input values; it is built
 * with -O2 -ffp-contract=off so every sum runs in the order written.
 *
 * Layouts (row-major, contiguous): one batch entry at a time,
 *   q [Sq][Hq][D], k [Sk][Hkv][D], v [Sk][Hkv][D] as raw fp16 bit patterns.
 * Output per requested (head, row) item n: o[n*D .. n*D+D-1], lse[n].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Exact IEEE-754 binary16 -> binary64: sign, 5-bit exponent (bias 15),
 * 10-bit fraction; subnormals are frac * 2^-24; exponent 31 is inf/NaN. */
double oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double mag;
  if (expo == 0) {
    mag = ldexp((double)frac, -24);
  } else if (expo == 31) {
    mag = frac ? NAN : INFINITY;
  } else {
    mag = ldexp((double)(frac | 0x400), expo - 25);
  }
  return sign ? -mag : mag;
}

typedef struct {
  const uint16_t* q;
  const double* kd; /* widened k, [Sk][Hkv][D] */
  const double* vd; /* widened v, [Sk][Hkv][D] */
  int Sq, Sk, Hq, Hkv, D, causal;
  double sigma;
  const int32_t* heads;
  const int32_t* rows;
  int64_t n;
  double* o;
  double* lse;
  int64_t next; /* shared work counter */
  int failed;
} job_t;

static void one_row(const job_t* J, int64_t item, double* scores, double* qrow, double* acc) {
  const int Sk = J->Sk, Hq = J->Hq, Hkv = J->Hkv, D = J->D;
  const int off = J->Sk - J->Sq; /* key position of query row 0, bottom-right alignment */
  const int h = J->heads[item];
  const int i = J->rows[item];
  const int g = Hq / Hkv;
  const int c = h / g;
  const int nkeys = J->causal ? i + 1 + off : Sk;

  for (int d = 0; d < D; ++d) qrow[d] = oracle_half_to_double(J->q[((int64_t)i * Hq + h) * D + d]);

  double m = -INFINITY;
  for (int j = 0; j < nkeys; ++j) {
    const double* kr = J->kd + ((int64_t)j * Hkv + c) * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qrow[d] * kr[d];
    scores[j] = J->sigma * dot;
    if (scores[j] > m) m = scores[j];
  }

  double l = 0.0;
  for (int d = 0; d < D; ++d) acc[d] = 0.0;
  for (int j = 0; j < nkeys; ++j) {
    double w = exp(scores[j] - m);
    l += w;
    const double* vr = J->vd + ((int64_t)j * Hkv + c) * D;
    for (int d = 0; d < D; ++d) acc[d] += w * vr[d];
  }

  double* out = J->o + item * D;
  for (int d = 0; d < D; ++d) out[d] = acc[d] / l;
  J->lse[item] = m + log(l);
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  double* scores = (double*)malloc(sizeof(double) * (size_t)J->Sk);
  double* qrow = (double*)malloc(sizeof(double) * (size_t)J->D);
  double* acc = (double*)malloc(sizeof(double) * (size_t)J->D);
  if (!scores || !qrow || !acc) {
    __atomic_store_n(&J->failed, 1, __ATOMIC_SEQ_CST);
  } else {
    for (;;) {
      int64_t item = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
      if (item >= J->n) break;
      one_row(J, item, scores, qrow, acc);
    }
  }
  free(scores);
  free(qrow);
  free(acc);
  return NULL;
}

/* Computes n output rows of one batch entry with Sq query rows and Sk keys.
 * Returns 0 on success, 1 on invalid arguments (including causal with
 * Sq > Sk), 2 on allocation/thread failure. */
int oracle_attn_rows_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v, int Sq, int Sk, int Hq, int Hkv,
                        int D, int causal, float scale, const int32_t* heads, const int32_t* rows, int64_t n,
                        double* o, double* lse, int nthreads) {
  if (!q || !k || !v || !heads || !rows || !o || !lse) return 1;
  if (Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv != 0 || n < 0) return 1;
  if (causal != 0 && causal != 1) return 1;
  if (causal && Sq > Sk) return 1;
  for (int64_t t = 0; t < n; ++t)
    if (heads[t] < 0 || heads[t] >= Hq || rows[t] < 0 || rows[t] >= Sq) return 1;
  if (n == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > n) nthreads = (int)n;

  const int64_t kv_elems = (int64_t)Sk * Hkv * D;
  double* kd = (double*)malloc(sizeof(double) * (size_t)kv_elems);
  double* vd = (double*)malloc(sizeof(double) * (size_t)kv_elems);
  if (!kd || !vd) {
    free(kd);
    free(vd);
    return 2;
  }
  for (int64_t x = 0; x < kv_elems; ++x) {
    kd[x] = oracle_half_to_double(k[x]);
    vd[x] = oracle_half_to_double(v[x]);
  }

  job_t J;
  memset(&J, 0, sizeof(J));
  J.q = q;
  J.kd = kd;
  J.vd = vd;
  J.Sq = Sq;
  J.Sk = Sk;
  J.Hq = Hq;
  J.Hkv = Hkv;
  J.D = D;
  J.causal = causal;
  J.sigma = (double)scale;
  J.heads = heads;
  J.rows = rows;
  J.n = n;
  J.o = o;
  J.lse = lse;

  int rc = 0;
  pthread_t* tids = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  if (!tids) {
    rc = 2;
  } else {
    for (int t = 0; t < nthreads; ++t) {
      if (pthread_create(&tids[t], NULL, worker, &J) != 0) break;
      ++started;
    }
    if (started == 0) worker(&J); /* no thread could start: run inline */
    for (int t = 0; t < started; ++t) pthread_join(tids[t], NULL);
    if (J.failed) rc = 2;
  }
  free(tids);
  free(kd);
  free(vd);
  return rc;
}

/* The square case Sq == Sk == S. */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int S, int Hq, int Hkv, int D,
                     int causal, float scale, const int32_t* heads, const int32_t* rows, int64_t n, double* o,
                     double* lse, int nthreads) {
  return oracle_attn_rows_ex(q, k, v, S, S, Hq, Hkv, D, causal, scale, heads, rows, n, o, lse, nthreads);
}
