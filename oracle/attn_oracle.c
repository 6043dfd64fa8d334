/*
 * Attention-forward oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code, header or constant with the HIP library.
 *
 * What it computes (PipeThreader, OSDI'25 summary page, "FlashAttention-3"
 * paragraph): FlashAttention is an efficient implementation of ordinary full
 * attention -- acc_s = Q K^T, a softmax over each row of acc_s gives P, and
 * O = P V. The blockwise online-softmax method (load, the two matrix products,
 * online softmax, output rescale and accumulate -- same page, Fig 7; the
 * "PipeThreader and TileLang" page, section 4.1) reaches that same result in
 * exact arithmetic, so the oracle is the plain definition written out, with
 * the whole softmax row materialised, not the online recurrence.
 *
 * The pages do not define the scale, the causal mask or the log-sum-exp; the
 * readings taken here are:
 *   s_ij  = sigma * sum_k q_ik k_jk        sigma = the float32 scale, widened
 *   J_i   = {0..N-1} (full)  or  {0..i} (causal: key j visible iff j <= i)
 *   m_i   = max_{j in J_i} s_ij
 *   w_ij  = exp(s_ij - m_i) on J_i, 0 elsewhere;  l_i = sum_j w_ij
 *   P_ij  = w_ij / l_i;   O_i = sum_j P_ij v_j
 *   LSE_i = m_i + ln(l_i)   (natural log of sum_{j in J_i} exp(s_ij))
 * Inputs are bf16 bit patterns, widened exactly to double; every step is fp64
 * with sums in index order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* One output row. Returns 0, or 1 if the materialised softmax row does not sum
 * to 1 within 1e-12 (a self-check of the definition above). */
static int one_row(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t N, int64_t d,
                   int causal, double sigma, int64_t i, double* w, double* out_row,
                   double* lse_out) {
  int64_t nvis = causal ? i + 1 : N;
  const uint16_t* qi = q + i * d;
  /* logits s_ij over the visible keys */
  double m = -INFINITY;
  for (int64_t j = 0; j < nvis; ++j) {
    const uint16_t* kj = k + j * d;
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += widen_bf16(qi[c]) * widen_bf16(kj[c]);
    double s = sigma * dot;
    w[j] = s;
    if (s > m) m = s;
  }
  /* exponentiate relative to the row max, sum, normalise */
  double l = 0.0;
  for (int64_t j = 0; j < nvis; ++j) {
    w[j] = exp(w[j] - m);
    l += w[j];
  }
  double psum = 0.0;
  for (int64_t j = 0; j < nvis; ++j) {
    w[j] = w[j] / l;
    psum += w[j];
  }
  /* O_i = sum_j P_ij v_j */
  for (int64_t c = 0; c < d; ++c) out_row[c] = 0.0;
  for (int64_t j = 0; j < nvis; ++j) {
    const uint16_t* vj = v + j * d;
    for (int64_t c = 0; c < d; ++c) out_row[c] += w[j] * widen_bf16(vj[c]);
  }
  *lse_out = m + log(l);
  return fabs(psum - 1.0) <= 1e-12 ? 0 : 1;
}

/*
 * Attention forward for a chosen set of output rows.
 *   q, k, v : bf16 bits, [B][H][N][d] contiguous
 *   rows    : flat row ids r = (b*H + h)*N + i, each in [0, B*H*N); NULL = all
 *   out     : [n_rows][d] doubles;  lse : [n_rows] doubles
 *   threads : OpenMP threads (<= 0: runtime default)
 * Returns 0 on success, -1 on bad arguments, or the number of rows whose
 * softmax failed the sum-to-one self-check.
 */
int oracle_attn_fwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                         int64_t H, int64_t N, int64_t d, int causal, float scale,
                         const int64_t* rows, int64_t n_rows, double* out, double* lse,
                         int threads) {
  if (B < 0 || H < 0 || N < 0 || d < 1) return -1;
  int64_t total = B * H * N;
  if (rows == NULL) n_rows = total;
  if (n_rows == 0) return 0;
  if (!q || !k || !v || !out || !lse) return -1;
  for (int64_t t = 0; rows && t < n_rows; ++t)
    if (rows[t] < 0 || rows[t] >= total) return -1;
  double sigma = (double)scale;
  int bad = 0;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads) reduction(+ : bad)
#endif
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
    for (int64_t t = 0; t < n_rows; ++t) {
      int64_t r = rows ? rows[t] : t;
      int64_t bh = r / N, i = r % N;
      int64_t head = bh * N * d;
      bad += one_row(q + head, k + head, v + head, N, d, causal, sigma, i, w, out + t * d,
                     lse + t);
    }
    free(w);
  }
  (void)threads;
  return bad;
}

/*
 * Decoding: Nq query rows per (batch, head) against Nkv cached keys, every
 * query seeing every key (the same definition with a rectangular score
 * matrix, as in the split-KV decoding microbenchmark the pages list).
 *   q : [B][H][Nq][d];  k, v : [B][H][Nkv][d]  (bf16 bits, contiguous)
 *   rows : flat query-row ids (b*H + h)*Nq + i in [0, B*H*Nq); NULL = all
 * Same outputs and return codes as oracle_attn_fwd_rows.
 */
int oracle_attn_decode_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                            int64_t H, int64_t Nq, int64_t Nkv, int64_t d, float scale,
                            const int64_t* rows, int64_t n_rows, double* out, double* lse,
                            int threads) {
  if (B < 0 || H < 0 || Nq < 0 || Nkv < 1 || d < 1) return -1;
  int64_t total = B * H * Nq;
  if (rows == NULL) n_rows = total;
  if (n_rows == 0) return 0;
  if (!q || !k || !v || !out || !lse) return -1;
  for (int64_t t = 0; rows && t < n_rows; ++t)
    if (rows[t] < 0 || rows[t] >= total) return -1;
  const double sigma = scale;  /* the float32 scale, widened exactly */
  int bad = 0;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads) reduction(+ : bad)
#endif
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)Nkv);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
    for (int64_t t = 0; t < n_rows; ++t) {
      int64_t r = rows ? rows[t] : t;
      int64_t bh = r / Nq, i = r % Nq;
      bad += one_row(q + bh * Nq * d, k + bh * Nkv * d, v + bh * Nkv * d, Nkv, d, 0, sigma, i, w,
                     out + t * d, lse + t);
    }
    free(w);
  }
  (void)threads;
  return bad;
}

/* Number of threads an OpenMP region would use by default (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
