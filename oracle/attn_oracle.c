/*
 * Attention (forward, decoding, backward, MLA decoding) and Mamba2 ChunkScan
 * oracle: plain, slow, fp64 CPU reference.
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

/*
 * Backward: the gradient of the forward above. The pages name the attention
 * backward pass as a second schedule to pipeline (the Twill write-up,
 * section 3.2) without restating it; it is the derivative of the definition
 * above, so the oracle writes that derivative out. With dO the upstream
 * gradient of O (the LSE output is taken to carry none) and P, O the
 * forward's softmax and output, recomputed here in fp64:
 *   D_i   = sum_c dO_ic O_ic
 *   dP_ij = sum_c dO_ic v_jc                       (j in J_i)
 *   dS_ij = P_ij (dP_ij - D_i)                     (softmax Jacobian times dP)
 *   dQ_i  = sigma sum_{j in J_i} dS_ij k_j
 *   dK_j  = sigma sum_{i : j in J_i} dS_ij q_i
 *   dV_j  = sum_{i : j in J_i} P_ij dO_i
 * For a key row, P_ij = exp(s_ij - LSE_i) with LSE_i from the row's softmax.
 */

/* Softmax row i (P into w), its output row and LSE, and D_i. */
static int bwd_row_stats(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dout, int64_t N, int64_t d, int causal, double sigma,
                         int64_t i, double* w, double* o_row, double* lse, double* D) {
  int bad = one_row(q, k, v, N, d, causal, sigma, i, w, o_row, lse);
  double acc = 0.0;
  for (int64_t c = 0; c < d; ++c) acc += widen_bf16(dout[i * d + c]) * o_row[c];
  *D = acc;
  return bad;
}

/* dQ_i for query row i of one head. */
static int bwd_dq_row(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* dout, int64_t N, int64_t d, int causal, double sigma,
                      int64_t i, double* w, double* o_row, double* dq_row) {
  double lse, D;
  int bad = bwd_row_stats(q, k, v, dout, N, d, causal, sigma, i, w, o_row, &lse, &D);
  const int64_t last_key = causal ? i : N - 1;
  for (int64_t c = 0; c < d; ++c) dq_row[c] = 0.0;
  for (int64_t j = 0; j <= last_key; ++j) {
    double dp = 0.0;
    for (int64_t c = 0; c < d; ++c) dp += widen_bf16(dout[i * d + c]) * widen_bf16(v[j * d + c]);
    double ds = w[j] * (dp - D);
    for (int64_t c = 0; c < d; ++c) dq_row[c] += sigma * ds * widen_bf16(k[j * d + c]);
  }
  return bad;
}

/* dK_j and dV_j for key row j of one head, given every row's LSE and D. */
static void bwd_dkdv_row(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dout, int64_t N, int64_t d, int causal, double sigma,
                         const double* lse, const double* D, int64_t j, double* dk_row,
                         double* dv_row) {
  for (int64_t c = 0; c < d; ++c) dk_row[c] = dv_row[c] = 0.0;
  for (int64_t i = causal ? j : 0; i < N; ++i) {
    double dot = 0.0, dp = 0.0;
    for (int64_t c = 0; c < d; ++c) {
      dot += widen_bf16(q[i * d + c]) * widen_bf16(k[j * d + c]);
      dp += widen_bf16(dout[i * d + c]) * widen_bf16(v[j * d + c]);
    }
    double p = exp(sigma * dot - lse[i]);
    double ds = p * (dp - D[i]);
    for (int64_t c = 0; c < d; ++c) {
      dv_row[c] += p * widen_bf16(dout[i * d + c]);
      dk_row[c] += sigma * ds * widen_bf16(q[i * d + c]);
    }
  }
}

/*
 * Attention backward for chosen rows.
 *   q, k, v, dout : bf16 bits, [B][H][N][d] contiguous
 *   qrows : flat query-row ids (b*H + h)*N + i whose dQ is wanted (NULL = all)
 *   krows : flat key-row ids (b*H + h)*N + j whose dK, dV are wanted (NULL = all)
 *   dq : [n_qrows][d];  dk, dv : [n_krows][d]  (doubles)
 * Returns 0, -1 on bad arguments, or the number of softmax rows failing the
 * sum-to-one self-check.
 */
int oracle_attn_bwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dout, int64_t B, int64_t H, int64_t N, int64_t d,
                         int causal, float scale, const int64_t* qrows, int64_t n_qrows,
                         double* dq, const int64_t* krows, int64_t n_krows, double* dk,
                         double* dv, int threads) {
  if (B < 0 || H < 0 || N < 0 || d < 1) return -1;
  int64_t total = B * H * N;
  if (qrows == NULL) n_qrows = total;
  if (krows == NULL) n_krows = total;
  if (!q || !k || !v || !dout) return -1;
  if ((n_qrows > 0 && !dq) || (n_krows > 0 && (!dk || !dv))) return -1;
  for (int64_t t = 0; qrows && t < n_qrows; ++t)
    if (qrows[t] < 0 || qrows[t] >= total) return -1;
  for (int64_t t = 0; krows && t < n_krows; ++t)
    if (krows[t] < 0 || krows[t] >= total) return -1;
  const double sig = scale;  /* the float32 scale, widened exactly */
  int bad = 0;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#endif
  /* dQ rows */
#ifdef _OPENMP
#pragma omp parallel num_threads(threads) reduction(+ : bad)
#endif
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* o_row = (double*)malloc(sizeof(double) * (size_t)d);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
    for (int64_t t = 0; t < n_qrows; ++t) {
      int64_t r = qrows ? qrows[t] : t;
      int64_t head = (r / N) * N * d;
      bad += bwd_dq_row(q + head, k + head, v + head, dout + head, N, d, causal, sig, r % N, w,
                        o_row, dq + t * d);
    }
    free(o_row);
    free(w);
  }
  /* dK, dV rows, one head at a time: every row's LSE and D first */
  double* lse = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  double* D = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  for (int64_t bh = 0; bh < B * H && n_krows > 0; ++bh) {
    int64_t want = 0;
    for (int64_t t = 0; t < n_krows; ++t) want += ((krows ? krows[t] : t) / N) == bh;
    if (want == 0) continue;
    const int64_t head = bh * N * d;
#ifdef _OPENMP
#pragma omp parallel num_threads(threads) reduction(+ : bad)
#endif
    {
      double* w = (double*)malloc(sizeof(double) * (size_t)N);
      double* o_row = (double*)malloc(sizeof(double) * (size_t)d);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
      for (int64_t i = 0; i < N; ++i)
        bad += bwd_row_stats(q + head, k + head, v + head, dout + head, N, d, causal, sig, i, w,
                             o_row, lse + i, D + i);
      free(o_row);
      free(w);
    }
#ifdef _OPENMP
#pragma omp parallel for num_threads(threads) schedule(dynamic, 4)
#endif
    for (int64_t t = 0; t < n_krows; ++t) {
      int64_t r = krows ? krows[t] : t;
      if (r / N != bh) continue;
      bwd_dkdv_row(q + head, k + head, v + head, dout + head, N, d, causal, sig, lse, D, r % N,
                   dk + t * d, dv + t * d);
    }
  }
  free(D);
  free(lse);
  (void)threads;
  return bad;
}

/*
 * Mamba2 ChunkScan (PipeThreader summary page, "Running example: Mamba2" and
 * Fig 6(a)): the sequence is processed in chunks; inside a chunk the matrix
 * cb is scaled by the exponential decay built from dA and by dt, and its
 * product with x is accumulated into the output. Written out, for step s of
 * chunk c (c = s / L, m = s - cL) and head h:
 *   out[b][s][h][:] = sum_{k = 0..m} cb[b][c][m][k]
 *                         * exp(dA_cumsum[b][h][c][m] - dA_cumsum[b][h][c][k])
 *                         * dt[b][h][c][k] * x[b][cL + k][h][:]
 * Only steps k <= m of the same chunk contribute (the decay runs forward in
 * time; the term carried across chunks by the state is a separate operation
 * the pages do not include here).
 *   x  : bf16 bits [B][S][H][P];   cb : bf16 bits [B][nc][L][L]
 *   dt, dacs : float [B][H][nc][L]  (nc = ceil(S / L))
 *   rows : flat output-row ids (b*S + s)*H + h in [0, B*S*H); NULL = all
 *   out  : [n_rows][P] doubles
 */
int oracle_chunk_scan_rows(const uint16_t* x, const uint16_t* cb, const float* dt, const float* dacs,
                           int64_t B, int64_t S, int64_t H, int64_t P, int64_t L, const int64_t* rows,
                           int64_t n_rows, double* out, int threads) {
  if (B < 0 || S < 0 || H < 1 || P < 1 || L < 1) return -1;
  int64_t total = B * S * H;
  if (rows == NULL) n_rows = total;
  if (n_rows == 0) return 0;
  if (!x || !cb || !dt || !dacs || !out) return -1;
  for (int64_t t = 0; rows && t < n_rows; ++t)
    if (rows[t] < 0 || rows[t] >= total) return -1;
  const int64_t nc = (S + L - 1) / L;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for num_threads(threads) schedule(dynamic, 16)
#endif
  for (int64_t t = 0; t < n_rows; ++t) {
    int64_t r = rows ? rows[t] : t;
    int64_t h = r % H, s = (r / H) % S, b = r / (H * S);
    int64_t c = s / L, m = s % L;
    const uint16_t* cb_row = cb + ((b * nc + c) * L + m) * L;
    const float* dt_c = dt + ((b * H + h) * nc + c) * L;
    const float* da_c = dacs + ((b * H + h) * nc + c) * L;
    double* o = out + t * P;
    for (int64_t p = 0; p < P; ++p) o[p] = 0.0;
    for (int64_t k = 0; k <= m; ++k) {
      double w = widen_bf16(cb_row[k]) * exp((double)da_c[m] - (double)da_c[k]) * (double)dt_c[k];
      const uint16_t* xk = x + ((b * S + c * L + k) * H + h) * P;
      for (int64_t p = 0; p < P; ++p) o[p] += w * widen_bf16(xk[p]);
    }
  }
  (void)threads;
  return 0;
}

/*
 * MLA decoding (multi-head latent attention, the decoding operator the
 * PipeThreader summary page's "Discussion" paragraph cites as an 80-line
 * program against 500-plus lines by hand), in the absorbed form: every query head attends to one shared cache of latent
 * rows; a row's first Dv values are its value, all Dk values its key.
 *   q  : bf16 bits [B][H][Dk];   kv : bf16 bits [B][N][Dk]
 *   s_hj = sigma * q_h . kv_j;  P = softmax_j;  out_h = sum_j P_hj kv_j[0:Dv]
 *   lse_h = ln sum_j exp(s_hj)
 *   rows : flat (b*H + h) ids, NULL = all;  out [n_rows][Dv], lse [n_rows]
 */
int oracle_mla_decode_rows(const uint16_t* q, const uint16_t* kv, int64_t B, int64_t H, int64_t N, int64_t Dk,
                           int64_t Dv, float scale, const int64_t* rows, int64_t n_rows, double* out,
                           double* lse, int threads) {
  if (B < 0 || H < 0 || N < 1 || Dk < 1 || Dv < 1 || Dv > Dk) return -1;
  int64_t total = B * H;
  if (rows == NULL) n_rows = total;
  if (n_rows == 0) return 0;
  if (!q || !kv || !out || !lse) return -1;
  for (int64_t t = 0; rows && t < n_rows; ++t)
    if (rows[t] < 0 || rows[t] >= total) return -1;
  const double sg = scale;  /* the float32 scale, widened exactly */
  int bad = 0;
#ifdef _OPENMP
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads) reduction(+ : bad)
#endif
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)N);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 4)
#endif
    for (int64_t t = 0; t < n_rows; ++t) {
      int64_t r = rows ? rows[t] : t;
      const uint16_t* qh = q + r * Dk;
      const uint16_t* kvb = kv + (r / H) * N * Dk;
      double m = -INFINITY;
      for (int64_t j = 0; j < N; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < Dk; ++c) dot += widen_bf16(qh[c]) * widen_bf16(kvb[j * Dk + c]);
        w[j] = sg * dot;
        if (w[j] > m) m = w[j];
      }
      double l = 0.0;
      for (int64_t j = 0; j < N; ++j) {
        const double e = exp(w[j] - m);
        w[j] = e;
        l += e;
      }
      double* o = out + t * Dv;
      for (int64_t c = 0; c < Dv; ++c) o[c] = 0.0;
      double psum = 0.0;
      for (int64_t j = 0; j < N; ++j) {
        const double p = w[j] / l;
        psum += p;
        for (int64_t c = 0; c < Dv; ++c) o[c] += p * widen_bf16(kvb[j * Dk + c]);
      }
      lse[t] = m + log(l);
      bad += fabs(psum - 1.0) <= 1e-12 ? 0 : 1;
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
