/*
 * CPU oracle for HiLS (Hierarchical Landmark Sparse) attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it computes is the plain definition of the operator, written from:
 *   [HiLS-p5] "Hierarchical Sparse Attention Done Right" abstract (chatpaper
 *             page, English and German text): each query attends to every
 *             retrieved chunk on its own, and the per-chunk outputs are fused
 *             by the chunk retrieval scores.
 *   [HiLS-p1] ai-feeds summary of the same paper, section "Method" >
 *             "Input & chunking" (fixed-size chunks with landmark
 *             representatives) and "Key modules" items 1-2 (landmark scores,
 *             chunk-level softmax, top-k chunks, per-chunk attention, fusion).
 *   [HiLS-p2] paper.oopus.info review, section 2 "Core method" (landmark per
 *             chunk, score, in-chunk attention, weighted fusion) and section 3
 *             (head dim 64, chunk size 64).
 *   [HiLS-p1] "Method" > "Input & chunking" also names a low-rank query
 *             calibration: a learned affine map of Q that serves retrieval.
 *             Read as an optional retrieval query Qr (same layout as Q, made
 *             outside the operator) that replaces Q in the landmark scores,
 *             and so in the selection and the fusion weights, while the
 *             per-chunk attention keeps Q.  Without Qr the scores use Q.
 *   [HiLS-p1] "Method" > "Input & chunking" further mentions a landmark-free
 *             alternative.  Read as: the landmark of a chunk is the mean of
 *             its keys (rounded to fp32, then to the element type); for the
 *             query's own chunk only the keys up to the query are averaged,
 *             so nothing after the query enters its scores and a decode step
 *             equals the prefill row at the same position.
 *   [HiLS-p1] "Method" > "Input & chunking" speaks of a few landmarks per
 *             chunk (usually its first and last token) and "Key modules"
 *             item 1 of a softmax over a chunk's landmark scores before the
 *             chunk-level one.  Read, for m landmarks per chunk, as: the
 *             chunk score is the log-sum-exp of its m landmark scores (the
 *             normaliser of that inner softmax), rounded to fp32 once; with
 *             m = 1 it is the plain score.
 * Points the pages leave open are fixed as follows (one landmark key per
 * chunk; scale 1/sqrt(d) on both softmax levels; top-k ties go to the lower
 * chunk index; the query's own chunk is always in the set, is not counted in
 * k, is scored by its own landmark and is attended causally; when fewer than
 * k past chunks exist all of them are taken; the fusion softmax runs over the
 * selected set only; the selection is a hard constant in the backward pass).
 *
 * Arithmetic: every input element (bf16 bit pattern or fp32) is widened to
 * double; all sums, exponentials and logarithms are in double.  Chunk scores
 * are rounded to fp32 once, so that selection decisions are taken on fp32
 * scores exactly as the GPU path takes them; everything downstream of the
 * selection stays in double.  Outputs are double.
 *
 * Layouts (row-major, head dim innermost):
 *   Q,K,V,dO [B,H,L,d]   Klm [B,H,N,d] with N = ceil(L/C)
 *   idx [B,H,L,k+1] int32: slots 0..m-1 = selected past chunks in order
 *       (score desc, index asc); slots m..k-1 = -1; slot k = own chunk.
 *   sel, w, lse [B,H,L,k+1] double (sel = the fp32 score, -inf when unused;
 *       w = 0 and lse = -inf when unused).
 *   O [B,H,L,d] double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define DT_BF16 0
#define DT_F32 1

/* bf16 is the upper half of an IEEE binary32; widening appends 16 zero bits. */
static double elem(const void* p, int64_t i, int dt) {
  if (dt == DT_F32) return (double)((const float*)p)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double dot_row(const void* A, int64_t ra, const void* Bm, int64_t rb, int64_t d, int dt) {
  double s = 0.0;
  for (int64_t e = 0; e < d; ++e) s += elem(A, ra * d + e, dt) * elem(Bm, rb * d + e, dt);
  return s;
}

typedef struct {
  const void *Q, *K, *V, *Klm;
  const void* Qr;  /* retrieval queries for the landmark scores (NULL: the attention queries) */
  int64_t B, H, L, d, C, k, N;
  int64_t Lkv;  /* rows per (b,h) in K/V (L for prefill, Lmax for a decode cache) */
  int64_t Nlm;  /* rows per (b,h) in Klm */
  double scale;
  int dt;
  int lf;  /* landmark-free: the own chunk's landmark is the mean of its keys up to the query */
  int64_t m;  /* landmarks per chunk (0 or 1: one); Klm is then [B,H,N,m,d] */
} prob_t;

#define MAX_D 256

/* double -> fp32 (round to nearest even) -> element type (bf16: round to nearest even on the bits) */
static double round_dt(double x, int dt) {
  float f = (float)x;
  if (dt == DT_F32) return (double)f;
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  b = (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
  memcpy(&f, &b, sizeof f);
  return (double)f;
}

static void store_dt(void* p, int64_t i, double x, int dt) {
  float f = (float)x;
  if (dt == DT_F32) { ((float*)p)[i] = f; return; }
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  ((uint16_t*)p)[i] = (uint16_t)(b >> 16);
}

/* mean of key rows row0 .. row0+n-1, each element rounded as a landmark element */
static void key_mean(const void* K, int64_t row0, int64_t n, int64_t d, int dt, double* out) {
  for (int64_t e = 0; e < d; ++e) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += elem(K, (row0 + i) * d + e, dt);
    out[e] = round_dt(s / (double)n, dt);
  }
}

typedef struct { float s; int32_t j; } cand_t;

/* total order of the selection: higher fp32 score first, lower index on ties */
static int cand_cmp(const void* a, const void* b) {
  const cand_t* x = (const cand_t*)a;
  const cand_t* y = (const cand_t*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}

/* chunk score of query row t against landmark j (HiLS-p2 section 2, step 1):
 * scale * <q_t, Klm_j>, computed in double and rounded to fp32.  Landmark-free
 * chunks: the own chunk's landmark is the mean of its keys jC..t. */
static float chunk_score(const prob_t* P, const void* q, int64_t qrow, int64_t bh, int64_t t, int64_t j) {
  const void* qs = P->Qr ? P->Qr : q;
  if (P->lf && j == t / P->C) {
    double m[MAX_D];
    key_mean(P->K, bh * P->Lkv + j * P->C, t - j * P->C + 1, P->d, P->dt, m);
    double s = 0.0;
    for (int64_t e = 0; e < P->d; ++e) s += elem(qs, qrow * P->d + e, P->dt) * m[e];
    return (float)(P->scale * s);
  }
  if (P->m > 1) {
    /* several landmarks: log-sum-exp of their scores */
    double a[64], amax = -INFINITY, z = 0.0;
    for (int64_t r = 0; r < P->m; ++r) {
      a[r] = P->scale * dot_row(qs, qrow, P->Klm, (bh * P->Nlm + j) * P->m + r, P->d, P->dt);
      if (a[r] > amax) amax = a[r];
    }
    for (int64_t r = 0; r < P->m; ++r) z += exp(a[r] - amax);
    return (float)(amax + log(z));
  }
  return (float)(P->scale * dot_row(qs, qrow, P->Klm, bh * P->Nlm + j, P->d, P->dt));
}

/*
 * Selection (HiLS-p1 "Key modules" item 2, top-k chunks): the m = min(k, c)
 * past chunks with the largest scores under (score desc, index asc).
 * Writes idx[0..k] and the fp32 score of each slot into sel[0..k].
 */
static void select_chunks(const prob_t* P, const void* q, int64_t qrow, int64_t bh, int64_t t,
                          const double* override_s, int32_t* idx, double* sel) {
  int64_t c = t / P->C;
  int64_t m = c < P->k ? c : P->k;
  cand_t* cs = (cand_t*)malloc(sizeof(cand_t) * (size_t)(c > 0 ? c : 1));
  for (int64_t j = 0; j < c; ++j) {
    cs[j].s = override_s ? (float)override_s[j] : chunk_score(P, q, qrow, bh, t, j);
    cs[j].j = (int32_t)j;
  }
  qsort(cs, (size_t)c, sizeof(cand_t), cand_cmp);
  for (int64_t r = 0; r < P->k; ++r) {
    idx[r] = r < m ? cs[r].j : -1;
    sel[r] = r < m ? (double)cs[r].s : -INFINITY;
  }
  idx[P->k] = (int32_t)c;
  sel[P->k] = override_s ? (double)(float)override_s[c] : (double)chunk_score(P, q, qrow, bh, t, c);
  free(cs);
}

/*
 * Attention of query row t inside one chunk j (HiLS-p1 "Key modules" item 2,
 * HiLS-p5: each query attends to each retrieved chunk independently).
 * Keys are the whole chunk for a past chunk and jC..t for the own chunk.
 * Returns lse_j and writes o_j[0..d-1] = sum_i softmax_i(a) v_i.
 */
static double chunk_attention(const prob_t* P, const void* q, int64_t qrow, int64_t bh, int64_t t,
                              int64_t j, double* o_j, double* a_buf) {
  int64_t lo = j * P->C;
  int64_t hi = (j == t / P->C) ? t : lo + P->C - 1;
  int64_t n = hi - lo + 1;
  double amax = -INFINITY;
  for (int64_t i = 0; i < n; ++i) {
    a_buf[i] = P->scale * dot_row(q, qrow, P->K, bh * P->Lkv + lo + i, P->d, P->dt);
    if (a_buf[i] > amax) amax = a_buf[i];
  }
  double z = 0.0;
  for (int64_t i = 0; i < n; ++i) z += exp(a_buf[i] - amax);
  double lse = amax + log(z);
  for (int64_t e = 0; e < P->d; ++e) o_j[e] = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double p = exp(a_buf[i] - lse);
    for (int64_t e = 0; e < P->d; ++e) o_j[e] += p * elem(P->V, (bh * P->Lkv + lo + i) * P->d + e, P->dt);
  }
  return lse;
}

/*
 * One query row: selection (or the given idx), fusion weights, per-chunk
 * attention, fused output.  Fusion weights are the softmax of the chunk
 * scores over the selected set (HiLS-p1 "Key modules" item 1, chunk-level
 * softmax; item 2 and HiLS-p5, score-weighted fusion).
 */
static void row_forward(const prob_t* P, const void* q, int64_t qrow, int64_t bh, int64_t t,
                        int use_idx, const double* override_s, int32_t* idx, double* sel,
                        double* w, double* lse, double* o) {
  int64_t k1 = P->k + 1;
  int64_t c = t / P->C;
  if (use_idx) {
    for (int64_t r = 0; r < k1; ++r) {
      if (idx[r] < 0) { sel[r] = -INFINITY; continue; }
      sel[r] = override_s ? (double)(float)override_s[idx[r]]
                          : (double)chunk_score(P, q, qrow, bh, t, idx[r]);
    }
  } else {
    select_chunks(P, q, qrow, bh, t, override_s, idx, sel);
  }
  /* chunk-level softmax over the selected set */
  double smax = -INFINITY;
  for (int64_t r = 0; r < k1; ++r) if (idx[r] >= 0 && sel[r] > smax) smax = sel[r];
  double zs = 0.0;
  for (int64_t r = 0; r < k1; ++r) if (idx[r] >= 0) zs += exp(sel[r] - smax);
  double* oj = (double*)malloc(sizeof(double) * (size_t)P->d);
  double* abuf = (double*)malloc(sizeof(double) * (size_t)P->C);
  for (int64_t e = 0; e < P->d; ++e) o[e] = 0.0;
  for (int64_t r = 0; r < k1; ++r) {
    if (idx[r] < 0) { w[r] = 0.0; lse[r] = -INFINITY; continue; }
    w[r] = exp(sel[r] - smax) / zs;
    lse[r] = chunk_attention(P, q, qrow, bh, t, idx[r], oj, abuf);
    for (int64_t e = 0; e < P->d; ++e) o[e] += w[r] * oj[e];
  }
  (void)c;
  free(oj);
  free(abuf);
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

/* Landmark scores S[b,h,t,j] = fp32(scale <q_t, Klm_j>) for j <= t/C, -inf otherwise. */
void oracle_landmark_scores(const void* Q, const void* Klm, double* S, int64_t B, int64_t H,
                            int64_t L, int64_t d, int64_t C, double scale, int dt, int nthreads) {
  prob_t P = {Q, NULL, NULL, Klm, NULL, B, H, L, d, C, 0, (L + C - 1) / C, L, (L + C - 1) / C, scale, dt};
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t row = 0; row < B * H * L; ++row) {
    int64_t bh = row / L, t = row % L;
    for (int64_t j = 0; j < P.N; ++j)
      S[row * P.N + j] = (j <= t / C) ? (double)chunk_score(&P, Q, row, bh, t, j) : -INFINITY;
  }
}

/* Scores of the listed rows only (flattened (b*H+h)*L+t); S is [nrows][N]. */
void oracle_landmark_scores_rows(const void* Q, const void* Klm, double* S, int64_t B, int64_t H, int64_t L,
                                 int64_t d, int64_t C, double scale, int dt, const int64_t* rows, int64_t nrows,
                                 int nthreads) {
  prob_t P = {Q, NULL, NULL, Klm, NULL, B, H, L, d, C, 0, (L + C - 1) / C, L, (L + C - 1) / C, scale, dt};
  set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t row = rows[r], bh = row / L, t = row % L;
    for (int64_t j = 0; j < P.N; ++j)
      S[r * P.N + j] = (j <= t / C) ? (double)chunk_score(&P, Q, row, bh, t, j) : -INFINITY;
  }
}

/*
 * Forward over all rows, or over a list of rows (rows != NULL: flattened
 * (b*H+h)*L+t indices; outputs are then packed per listed row).
 * use_idx: take the selection from idx instead of computing it.
 * override_s: optional [B,H,L,N] double chunk scores used instead of the
 * landmark scores for both selection and fusion (a test hook).
 * Returns the number of threads used.
 */
static void fwd_rows(const prob_t* P, const int64_t* rows, int64_t nrows, int use_idx, const double* override_s,
                     int32_t* idx, double* sel, double* w, double* lse, double* O) {
  int64_t total = rows ? nrows : P->B * P->H * P->L;
  int64_t k1 = P->k + 1, L = P->L, N = P->N, d = P->d;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < total; ++r) {
    int64_t row = rows ? rows[r] : r;
    int64_t bh = row / L, t = row % L;
    row_forward(P, P->Q, row, bh, t, use_idx, override_s ? override_s + row * N : NULL,
                idx + r * k1, sel + r * k1, w + r * k1, lse + r * k1, O + r * d);
  }
}

int oracle_fwd(const void* Q, const void* Qr, const void* K, const void* V, const void* Klm,
               int64_t B, int64_t H, int64_t L, int64_t d, int64_t C, int64_t k, double scale,
               int dt, const int64_t* rows, int64_t nrows, int use_idx, const double* override_s,
               int32_t* idx, double* sel, double* w, double* lse, double* O, int nthreads) {
  int64_t N = (L + C - 1) / C;
  prob_t P = {Q, K, V, Klm, Qr, B, H, L, d, C, k, N, L, N, scale, dt, 0};
  int used = set_threads(nthreads);
  fwd_rows(&P, rows, nrows, use_idx, override_s, idx, sel, w, lse, O);
  return used;
}

/*
 * Landmark-free chunk keys: Klm row j of every (b,h) = the mean of key rows
 * jC .. jC+C-1, rounded to fp32 and then to the element type, for the nchunks
 * complete chunks.  K has Lk rows per (b,h), Klm has Nlm rows per (b,h).
 */
void oracle_chunk_means(const void* K, int64_t Lk, void* Klm, int64_t Nlm, int64_t B, int64_t H,
                        int64_t nchunks, int64_t d, int64_t C, int dt, int nthreads) {
  set_threads(nthreads);
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    double m[MAX_D];
    for (int64_t j = 0; j < nchunks; ++j) {
      key_mean(K, bh * Lk + j * C, C, d, dt, m);
      for (int64_t e = 0; e < d; ++e) store_dt(Klm, (bh * Nlm + j) * d + e, m[e], dt);
    }
  }
}

/*
 * Forward with landmark-free chunks: the past chunks' landmarks are their key
 * means (written to Klm_out, [B,H,N,d] in the element type), the own chunk's
 * is the mean of its keys up to the query.  L must be a multiple of C.
 */
int oracle_fwd_lf(const void* Q, const void* Qr, const void* K, const void* V, void* Klm_out,
                  int64_t B, int64_t H, int64_t L, int64_t d, int64_t C, int64_t k, double scale,
                  int dt, const int64_t* rows, int64_t nrows, int use_idx,
                  int32_t* idx, double* sel, double* w, double* lse, double* O, int nthreads) {
  if (L % C || d > MAX_D) return -1;
  int64_t N = L / C;
  oracle_chunk_means(K, L, Klm_out, N, B, H, N, d, C, dt, nthreads);
  prob_t P = {Q, K, V, Klm_out, Qr, B, H, L, d, C, k, N, L, N, scale, dt, 1};
  int used = set_threads(nthreads);
  fwd_rows(&P, rows, nrows, use_idx, NULL, idx, sel, w, lse, O);
  return used;
}

/*
 * One decode step for every (b,h): write k_new, v_new into row n of the
 * caches (this oracle's own host copies), then run the forward of query row
 * t = n over keys 0..n and landmark rows 0..n/C.  The landmark row of the
 * open chunk n/C is read as the caller supplied it.
 * Caches are [B,H,Lmax,d]; Klm is [B,H,Nmax,d].
 * use_idx: idx holds a given selection on entry (as in oracle_fwd); the step
 * then scores and attends to those chunks instead of selecting its own.
 */
static int decode_common(const void* q, const void* qr, const void* k_new, const void* v_new, void* Kc, void* Vc,
                         void* Klm, int lf, int64_t mlm, int64_t n, int64_t Lmax, int64_t Nmax, int64_t B, int64_t H,
                         int64_t d, int64_t C, int64_t k, double scale, int dt, int32_t* idx,
                         double* sel, double* w, double* lse, double* o, int nthreads, int use_idx) {
  int64_t esz = dt == DT_F32 ? 4 : 2;
  for (int64_t bh = 0; bh < B * H; ++bh) {
    memcpy((char*)Kc + ((bh * Lmax + n) * d) * esz, (const char*)k_new + bh * d * esz, (size_t)(d * esz));
    memcpy((char*)Vc + ((bh * Lmax + n) * d) * esz, (const char*)v_new + bh * d * esz, (size_t)(d * esz));
  }
  if (lf) {
    /* landmark-free: the open chunk's landmark row becomes the mean of its keys so far */
    int64_t c = n / C;
    double m[MAX_D];
    for (int64_t bh = 0; bh < B * H; ++bh) {
      key_mean(Kc, bh * Lmax + c * C, n - c * C + 1, d, dt, m);
      for (int64_t e = 0; e < d; ++e) store_dt(Klm, (bh * Nmax + c) * d + e, m[e], dt);
    }
  }
  prob_t P = {q, Kc, Vc, Klm, qr, B, H, n + 1, d, C, k, Nmax, Lmax, Nmax, scale, dt, lf, mlm};
  int used = set_threads(nthreads);
  int64_t k1 = k + 1;
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < B * H; ++bh)
    row_forward(&P, q, bh, bh, n, use_idx, NULL, idx + bh * k1, sel + bh * k1, w + bh * k1,
                lse + bh * k1, o + bh * d);
  return used;
}

int oracle_decode(const void* q, const void* qr, const void* k_new, const void* v_new, void* Kc, void* Vc,
                  const void* Klm, int64_t n, int64_t Lmax, int64_t Nmax, int64_t B, int64_t H,
                  int64_t d, int64_t C, int64_t k, double scale, int dt, int32_t* idx,
                  double* sel, double* w, double* lse, double* o, int nthreads, int use_idx) {
  return decode_common(q, qr, k_new, v_new, Kc, Vc, (void*)Klm, 0, 1, n, Lmax, Nmax, B, H, d, C, k, scale, dt, idx,
                       sel, w, lse, o, nthreads, use_idx);
}

/*
 * Decode step with landmark-free chunks: after the append, landmark row n/C
 * of Klm (the caller's host array, updated in place) becomes the mean of the
 * open chunk's keys so far; rows of earlier chunks are read as given (their
 * key means).
 */
int oracle_decode_lf(const void* q, const void* qr, const void* k_new, const void* v_new, void* Kc, void* Vc,
                     void* Klm, int64_t n, int64_t Lmax, int64_t Nmax, int64_t B, int64_t H,
                     int64_t d, int64_t C, int64_t k, double scale, int dt, int32_t* idx,
                     double* sel, double* w, double* lse, double* o, int nthreads, int use_idx) {
  if (d > MAX_D) return -1;
  return decode_common(q, qr, k_new, v_new, Kc, Vc, Klm, 1, 1, n, Lmax, Nmax, B, H, d, C, k, scale, dt, idx, sel, w,
                       lse, o, nthreads, use_idx);
}

/*
 * Backward with the selection held fixed (idx given), gradients in double.
 * For row t with g = dO_t, selected set S, weights w_j, per-chunk outputs o_j,
 * per-chunk probabilities p_i (softmax inside chunk j):
 *   D_j = g.o_j,  D = sum_j w_j D_j,  ds_j = w_j (D_j - D)
 *   da_i = w_j p_i (g.v_i - D_j)           for key i of chunk j
 *   dV_i += w_j p_i g,  dK_i += scale da_i q_t,  dQ_t += scale da_i k_i
 *   dQ_t += scale ds_j Klm_j,  dKlm_j += scale ds_j q_t
 * (the chain rule through the fused output, the chunk-level softmax, the
 * in-chunk softmax and both dot-product scores; the hard selection carries no
 * gradient).  dQ, dK, dV are [B,H,L,d]; dKlm is [B,H,N,d].  Work is split
 * across (b,h) only, so every accumulation is sequential in row order.
 * With retrieval queries Qr the scores are scale <qr_t, Klm_j>: the ds terms
 * then give dQr_t = scale sum_j ds_j Klm_j (written to dQr, [B,H,L,d]) and
 * dKlm_j += scale ds_j qr_t, and dQ keeps the in-chunk terms only.
 */
static int bwd_common(const void* Q, const void* Qr, const void* K, const void* V, const void* Klm, int lf,
                      int64_t m, const void* dO, const int32_t* idx_in, int64_t B, int64_t H, int64_t L, int64_t d,
                      int64_t C, int64_t k, double scale, int dt, double* dQ, double* dQr, double* dK, double* dV,
                      double* dKlm, int nthreads) {
  int64_t N = (L + C - 1) / C;
  prob_t P = {Q, K, V, Klm, Qr, B, H, L, d, C, k, N, L, N, scale, dt, lf, m};
  int used = set_threads(nthreads);
  int64_t k1 = k + 1;
  memset(dQ, 0, sizeof(double) * (size_t)(B * H * L * d));
  memset(dK, 0, sizeof(double) * (size_t)(B * H * L * d));
  memset(dV, 0, sizeof(double) * (size_t)(B * H * L * d));
  memset(dKlm, 0, sizeof(double) * (size_t)(B * H * N * (m > 1 ? m : 1) * d));
  if (dQr) memset(dQr, 0, sizeof(double) * (size_t)(B * H * L * d));
  double* dS = dQr ? dQr : dQ;  /* where the score gradients go */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)k1);
    double* sel = (double*)malloc(sizeof(double) * (size_t)k1);
    double* w = (double*)malloc(sizeof(double) * (size_t)k1);
    double* lse = (double*)malloc(sizeof(double) * (size_t)k1);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    double* oj = (double*)malloc(sizeof(double) * (size_t)(k1 * d));
    double* Dj = (double*)malloc(sizeof(double) * (size_t)k1);
    double* abuf = (double*)malloc(sizeof(double) * (size_t)C);
    double* g = (double*)malloc(sizeof(double) * (size_t)d);
    double* qv = (double*)malloc(sizeof(double) * (size_t)d);
    double* qrv = (double*)malloc(sizeof(double) * (size_t)d);
    for (int64_t t = 0; t < L; ++t) {
      int64_t row = bh * L + t;
      memcpy(idx, idx_in + row * k1, sizeof(int32_t) * (size_t)k1);
      row_forward(&P, Q, row, bh, t, 1, NULL, idx, sel, w, lse, o);
      for (int64_t e = 0; e < d; ++e) {
        g[e] = elem(dO, row * d + e, dt);
        qv[e] = elem(Q, row * d + e, dt);
        qrv[e] = elem(Qr ? Qr : Q, row * d + e, dt);
      }
      /* per-chunk outputs o_j and D_j = g.o_j */
      double D = 0.0;
      for (int64_t r = 0; r < k1; ++r) {
        Dj[r] = 0.0;
        if (idx[r] < 0) continue;
        chunk_attention(&P, Q, row, bh, t, idx[r], oj + r * d, abuf);
        for (int64_t e = 0; e < d; ++e) Dj[r] += g[e] * oj[r * d + e];
        D += w[r] * Dj[r];
      }
      for (int64_t r = 0; r < k1; ++r) {
        if (idx[r] < 0) continue;
        int64_t j = idx[r];
        double ds = w[r] * (Dj[r] - D);
        if (lf && r == k) {
          /* landmark-free own chunk: the landmark is the mean m of keys jC..t (its rounding
           * passed straight through), so dS_t += scale ds m and every averaged key gets
           * scale ds qr_t / count */
          double m[MAX_D];
          int64_t cnt = t - j * C + 1;
          key_mean(K, bh * L + j * C, cnt, d, dt, m);
          for (int64_t e = 0; e < d; ++e) dS[row * d + e] += scale * ds * m[e];
          for (int64_t i = j * C; i <= t; ++i)
            for (int64_t e = 0; e < d; ++e) dK[(bh * L + i) * d + e] += scale * ds * qrv[e] / (double)cnt;
        } else if (P.m > 1) {
          /* chunk score = log-sum-exp of its landmark scores: landmark r takes the share p_r */
          double a[64], amax = -INFINITY, z = 0.0;
          for (int64_t u = 0; u < P.m; ++u) {
            a[u] = scale * dot_row(Qr ? Qr : Q, row, Klm, (bh * N + j) * P.m + u, d, dt);
            if (a[u] > amax) amax = a[u];
          }
          for (int64_t u = 0; u < P.m; ++u) z += exp(a[u] - amax);
          for (int64_t u = 0; u < P.m; ++u) {
            double pu = exp(a[u] - amax) / z;
            int64_t lr = (bh * N + j) * P.m + u;
            for (int64_t e = 0; e < d; ++e) {
              dS[row * d + e] += scale * ds * pu * elem(Klm, lr * d + e, dt);
              dKlm[lr * d + e] += scale * ds * pu * qrv[e];
            }
          }
        } else {
          for (int64_t e = 0; e < d; ++e) {
            dS[row * d + e] += scale * ds * elem(Klm, (bh * N + j) * d + e, dt);
            dKlm[(bh * N + j) * d + e] += scale * ds * qrv[e];
          }
        }
        int64_t lo = j * C;
        int64_t hi = (j == t / C) ? t : lo + C - 1;
        for (int64_t i = lo; i <= hi; ++i) {
          double a = scale * dot_row(Q, row, K, bh * L + i, d, dt);
          double p = exp(a - lse[r]);
          double gv = 0.0;
          for (int64_t e = 0; e < d; ++e) gv += g[e] * elem(V, (bh * L + i) * d + e, dt);
          double da = w[r] * p * (gv - Dj[r]);
          for (int64_t e = 0; e < d; ++e) {
            dV[(bh * L + i) * d + e] += w[r] * p * g[e];
            dK[(bh * L + i) * d + e] += scale * da * qv[e];
            dQ[row * d + e] += scale * da * elem(K, (bh * L + i) * d + e, dt);
          }
        }
      }
    }
    if (lf) {
      /* a past chunk's landmark is the mean of its C keys: each key gets dKlm_j / C */
      for (int64_t j = 0; j < N; ++j)
        for (int64_t i = j * C; i < (j + 1) * C && i < L; ++i)
          for (int64_t e = 0; e < d; ++e) dK[(bh * L + i) * d + e] += dKlm[(bh * N + j) * d + e] / (double)C;
    }
    free(idx); free(sel); free(w); free(lse); free(o); free(oj); free(Dj); free(abuf); free(g); free(qv); free(qrv);
  }
  return used;
}

int oracle_bwd(const void* Q, const void* Qr, const void* K, const void* V, const void* Klm, const void* dO,
               const int32_t* idx_in, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
               int64_t k, double scale, int dt, double* dQ, double* dQr, double* dK, double* dV, double* dKlm,
               int nthreads) {
  return bwd_common(Q, Qr, K, V, Klm, 0, 1, dO, idx_in, B, H, L, d, C, k, scale, dt, dQ, dQr, dK, dV, dKlm,
                    nthreads);
}

/*
 * Backward of the landmark-free forward (selection fixed by idx): the landmarks are the key
 * means (formed here, as the forward forms them), so the score gradients reach the keys.
 * dKlm receives the gradient with respect to the past chunks' means (already folded into dK).
 */
int oracle_bwd_lf(const void* Q, const void* Qr, const void* K, const void* V, const void* dO,
                  const int32_t* idx_in, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
                  int64_t k, double scale, int dt, double* dQ, double* dQr, double* dK, double* dV, double* dKlm,
                  int nthreads) {
  if (L % C || d > MAX_D) return -1;
  int64_t N = L / C;
  void* Klm = malloc((size_t)(B * H * N * d) * (dt == DT_F32 ? 4 : 2));
  oracle_chunk_means(K, L, Klm, N, B, H, N, d, C, dt, nthreads);
  int used = bwd_common(Q, Qr, K, V, Klm, 1, 1, dO, idx_in, B, H, L, d, C, k, scale, dt, dQ, dQr, dK, dV, dKlm,
                        nthreads);
  free(Klm);
  return used;
}

/*
 * Forward and backward with m landmarks per chunk (Klm [B,H,N,m,d], 1 <= m <= 64): the chunk score
 * is the log-sum-exp of the chunk's landmark scores; dKlm is [B,H,N,m,d].
 */
int oracle_fwd_ml(const void* Q, const void* Qr, const void* K, const void* V, const void* Klm, int64_t m,
                  int64_t B, int64_t H, int64_t L, int64_t d, int64_t C, int64_t k, double scale,
                  int dt, const int64_t* rows, int64_t nrows, int use_idx,
                  int32_t* idx, double* sel, double* w, double* lse, double* O, int nthreads) {
  if (m < 1 || m > 64) return -1;
  int64_t N = (L + C - 1) / C;
  prob_t P = {Q, K, V, Klm, Qr, B, H, L, d, C, k, N, L, N, scale, dt, 0, m};
  int used = set_threads(nthreads);
  fwd_rows(&P, rows, nrows, use_idx, NULL, idx, sel, w, lse, O);
  return used;
}

int oracle_bwd_ml(const void* Q, const void* Qr, const void* K, const void* V, const void* Klm, int64_t m,
                  const void* dO, const int32_t* idx_in, int64_t B, int64_t H, int64_t L, int64_t d, int64_t C,
                  int64_t k, double scale, int dt, double* dQ, double* dQr, double* dK, double* dV, double* dKlm,
                  int nthreads) {
  if (m < 1 || m > 64) return -1;
  return bwd_common(Q, Qr, K, V, Klm, 0, m, dO, idx_in, B, H, L, d, C, k, scale, dt, dQ, dQr, dK, dV, dKlm,
                    nthreads);
}

/* Decode step with m landmarks per chunk (Klm [B,H,Nmax,m,d]): scores as in oracle_fwd_ml. */
int oracle_decode_ml(const void* q, const void* qr, const void* k_new, const void* v_new, void* Kc, void* Vc,
                     const void* Klm, int64_t m, int64_t n, int64_t Lmax, int64_t Nmax, int64_t B, int64_t H,
                     int64_t d, int64_t C, int64_t k, double scale, int dt, int32_t* idx,
                     double* sel, double* w, double* lse, double* o, int nthreads, int use_idx) {
  if (m < 1 || m > 64) return -1;
  return decode_common(q, qr, k_new, v_new, Kc, Vc, (void*)Klm, 0, m, n, Lmax, Nmax, B, H, d, C, k, scale, dt, idx,
                       sel, w, lse, o, nthreads, use_idx);
}
