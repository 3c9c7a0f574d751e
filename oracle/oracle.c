/*
 * CPU oracle for the W4A16 skinny matmul -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow and obviously correct: the definition written out in double
 * precision.  Only the test suite, the smoke check and the bench's CPU
 * baseline leg load it.  It shares no code, header, table or constant with
 * the GPU library, and neither side includes or links the other.
 *
 * What it computes (every passage cited is from the pages this project
 * follows; the weight format is the one the qwen-warp/llamAmpere article
 * describes in section "qwen-warp: keep the activations in bf16"):
 *
 *   code     q(n,k) in 0..15 : 4-bit nibbles, two per byte.  Weights are
 *            "words of eight nibbles" read little-endian, so byte j of row n
 *            holds k = 2j in its low nibble and k = 2j+1 in its high nibble.
 *   level    q - 8 : the article subtracts 136 from 128+q, "nibble minus 8",
 *            and reports that all sixteen nibbles land on -8..7 exactly.
 *   scale    s(n,g) : one bf16 scale per 128 columns of a row, g = k/128
 *            (same section; the byte table's 0.656 GB int4 lm_head of
 *            248,320 x 5,120 confirms one bf16 per 128 weights).
 *   weight   w(n,k) = (q(n,k) - 8) * s(n, k/128)
 *   output   y(t,n) = sum_k w(n,k) * x(t,k),  x bf16, y accumulated in double.
 *   tolerance scale  A(t,n) = sum_k |w(n,k) * x(t,k)|.
 *
 * Every product w*x is exact in double (4 + 8 + 8 significant bits), so the
 * only rounding is the summation, about K * 2^-53 relative.
 *
 * The gathered head (swift-qwen3.8 project page, "Body, heads and drafter":
 * the drafter's head keeps only those lm_head rows that belong to the draft
 * vocabulary) scores output row i with weight row row_ids[i].  Greedy
 * verification keeps a draft that equals the argmax of its verify row
 * (article section "What each one calls the same answer"); the argmax here
 * returns, per
 * activation row t, the maximum and the lowest vocabulary id attaining it,
 * never a NaN.  Ids outside [0, n_rows) give a NaN output row.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GROUP 128

/* bf16 bit pattern -> double.  A bf16 is the top half of an IEEE float. */
double oracle_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* 4-bit code of column k in a packed row: even k low nibble, odd k high. */
int oracle_code(const uint8_t* packed_row, int64_t k) {
  uint8_t byte = packed_row[k / 2];
  return (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* Dequantised weight w(n,k) = (q - 8) * s(n, k/128), exact in double. */
double oracle_weight(const uint8_t* packed, const uint16_t* scales, int64_t K, int64_t n, int64_t k) {
  const uint8_t* row = packed + n * (K / 2);
  int level = oracle_code(row, k) - 8;
  double s = oracle_bf16(scales[n * (K / ORACLE_GROUP) + k / ORACLE_GROUP]);
  return (double)level * s;
}

/* One output row r of the weight against all T activation rows (the
 * definition, summed over k in order). */
static void row_dot(const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int64_t K, int T, int64_t r,
                    double* y_col, double* a_col, int64_t stride) {
  for (int t = 0; t < T; ++t) {
    double sum = 0.0, asum = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double p = oracle_weight(packed, scales, K, r, k) * oracle_bf16(x[(int64_t)t * K + k]);
      sum += p;
      asum += fabs(p);
    }
    y_col[(int64_t)t * stride] = sum;
    if (a_col) a_col[(int64_t)t * stride] = asum;
  }
}

typedef struct {
  const int32_t* row_ids; /* NULL: identity */
  int64_t n_out, n_rows, K;
  int T;
  const uint8_t* packed;
  const uint16_t* scales;
  const uint16_t* x;
  double *y, *a;
  int64_t begin, end;
} work_t;

static void* run_rows(void* p) {
  work_t* w = (work_t*)p;
  for (int64_t i = w->begin; i < w->end; ++i) {
    int64_t r = w->row_ids ? (int64_t)w->row_ids[i] : i;
    if (r < 0 || r >= w->n_rows) {
      for (int t = 0; t < w->T; ++t) {
        w->y[(int64_t)t * w->n_out + i] = NAN;
        if (w->a) w->a[(int64_t)t * w->n_out + i] = NAN;
      }
      continue;
    }
    row_dot(w->packed, w->scales, w->x, w->K, w->T, r, w->y + i, w->a ? w->a + i : NULL, w->n_out);
  }
  return NULL;
}

static void run_threaded(work_t base, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (base.n_out < nthreads) nthreads = base.n_out > 0 ? (int)base.n_out : 1;
  work_t jobs[256];
  pthread_t th[256];
  int started[256] = {0};
  int64_t per = (base.n_out + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = base;
    jobs[t].begin = per * t < base.n_out ? per * t : base.n_out;
    jobs[t].end = per * (t + 1) < base.n_out ? per * (t + 1) : base.n_out;
    if (t > 0 && pthread_create(&th[t], NULL, run_rows, &jobs[t]) == 0) started[t] = 1;
  }
  run_rows(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) {
    if (started[t])
      pthread_join(th[t], NULL);
    else
      run_rows(&jobs[t]);
  }
}

/* y[t][n] and A[t][n] (a may be NULL) for the full matrix, N x K, T rows. */
void oracle_matmul(const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int64_t N, int64_t K, int T,
                   double* y, double* a, int nthreads) {
  work_t w = {NULL, N, N, K, T, packed, scales, x, y, a, 0, 0};
  run_threaded(w, nthreads);
}

/* Gathered rows: y[t][i] uses weight row row_ids[i]; NaN for ids outside
 * [0, n_rows).  Also serves to evaluate any sample of rows of a matrix. */
void oracle_gather(const int32_t* row_ids, int64_t n_ids, const uint8_t* packed, const uint16_t* scales,
                   int64_t n_rows, const uint16_t* x, int64_t K, int T, double* y, double* a, int nthreads) {
  work_t w = {row_ids, n_ids, n_rows, K, T, packed, scales, x, y, a, 0, 0};
  run_threaded(w, nthreads);
}

/* Second, separately written form of the same definition: dequantise a whole
 * row first (walking the bytes, two levels per byte), then take T dot
 * products.  The tests require it to agree with oracle_matmul. */
void oracle_matmul_dequant_first(const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int64_t N,
                                 int64_t K, int T, double* y) {
  double* wrow = (double*)malloc(sizeof(double) * (size_t)K);
  if (!wrow) return;
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* bytes = packed + n * (K / 2);
    for (int64_t j = 0; j < K / 2; ++j) {
      double s = oracle_bf16(scales[n * (K / ORACLE_GROUP) + (2 * j) / ORACLE_GROUP]);
      wrow[2 * j] = (double)((int)(bytes[j] & 0x0F) - 8) * s;
      wrow[2 * j + 1] = (double)((int)(bytes[j] >> 4) - 8) * s;
    }
    for (int t = 0; t < T; ++t) {
      double sum = 0.0;
      for (int64_t k = 0; k < K; ++k) sum += wrow[k] * oracle_bf16(x[(int64_t)t * K + k]);
      y[(int64_t)t * N + n] = sum;
    }
  }
  free(wrow);
}

/* Per activation row t of y[T][n]: the largest non-NaN value and the lowest
 * vocabulary id attaining it (ids[i], or i when ids is NULL).  gap_out[t] is
 * that maximum minus the largest value carried by any other id (+inf if none).
 * No non-NaN entry: id -1, value NaN, gap NaN. */
void oracle_argmax(const double* y, const int32_t* ids, int64_t n, int T, int32_t* id_out, double* val_out,
                   double* gap_out) {
  for (int t = 0; t < T; ++t) {
    const double* row = y + (int64_t)t * n;
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i) {
      if (isnan(row[i])) continue;
      int64_t id = ids ? ids[i] : i;
      if (best < 0 || row[i] > row[best] || (row[i] == row[best] && id < (ids ? ids[best] : best))) best = i;
    }
    if (best < 0) {
      id_out[t] = -1;
      val_out[t] = NAN;
      if (gap_out) gap_out[t] = NAN;
      continue;
    }
    int64_t best_id = ids ? ids[best] : best;
    double second = -INFINITY;
    int have_second = 0;
    for (int64_t i = 0; i < n; ++i) {
      int64_t id = ids ? ids[i] : i;
      if (isnan(row[i]) || id == best_id) continue;
      if (!have_second || row[i] > second) second = row[i];
      have_second = 1;
    }
    id_out[t] = (int32_t)best_id;
    val_out[t] = row[best];
    if (gap_out) gap_out[t] = have_second ? row[best] - second : INFINITY;
  }
}

/* ------------------------------------------------------ verify epilogue ----
 *
 * Per-row top-k.  The OpenJet engine page ("How it gets its speed") hands
 * its sampler the highest 32 scores of every verified row, and the
 * qwen-warp article ("What each one calls the same answer") rescores the 16
 * highest candidates of the quantized head.  Definition used here: for each
 * activation row t of y[T][n], the k largest non-NaN scores with their
 * vocabulary ids (ids[i], or i when ids is NULL), in descending order of
 * score, equal scores in ascending order of id -- so entry 0 is the argmax
 * defined above.  -0 and +0 are equal scores.  With fewer than k non-NaN
 * scores the rest of the row is id -1, value NaN.  The implementation is
 * the definition: collect, sort everything, take the first k.
 */
typedef struct {
  double v;
  int64_t id;
} cand_t;

static int cand_before(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;
}

void oracle_topk(const double* y, const int32_t* ids, int64_t n, int T, int k, int32_t* id_out, double* val_out) {
  cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
  if (!c) return;
  for (int t = 0; t < T; ++t) {
    const double* row = y + (int64_t)t * n;
    int64_t m = 0;
    for (int64_t i = 0; i < n; ++i) {
      if (isnan(row[i])) continue;
      c[m].v = row[i];
      c[m].id = ids ? (int64_t)ids[i] : i;
      ++m;
    }
    qsort(c, (size_t)m, sizeof(cand_t), cand_before);
    for (int j = 0; j < k; ++j) {
      id_out[(int64_t)t * k + j] = j < m ? (int32_t)c[j].id : -1;
      val_out[(int64_t)t * k + j] = j < m ? c[j].v : NAN;
    }
  }
  free(c);
}

/* Greedy verification.  qwen-warp article, "What each one calls the same
 * answer": under greedy decoding a draft is kept when it equals the target's
 * argmax on its verify row; OpenJet engine page, "How it works": the check
 * runs on the GPU, and only the tokens it accepts are copied to the host.
 *
 * n_seq sequences of `rows` verify rows each.  Row r of sequence s carries
 * the target model's greedy choice target[s*rows + r] for the token after
 * position r; draft[s*(rows-1) + j] is the drafted token fed as the input of
 * row j+1.  Draft j is accepted when drafts 0..j-1 were and
 * target[s*rows + j] equals it (a negative target, i.e. no valid row, never
 * matches).  With a accepted drafts the cycle emits the target choices of
 * rows 0..a: the accepted drafts themselves followed by one more token of
 * the target model.  accepted[s] = a; tokens[s*rows + r] = target[s*rows + r]
 * for r <= a and -1 after.
 */
void oracle_greedy_accept(const int32_t* target, const int32_t* draft, int n_seq, int rows, int32_t* accepted,
                          int32_t* tokens) {
  for (int s = 0; s < n_seq; ++s) {
    int a = 0;
    while (a < rows - 1 && target[s * rows + a] >= 0 && target[s * rows + a] == draft[s * (rows - 1) + a]) ++a;
    accepted[s] = a;
    for (int r = 0; r < rows; ++r) tokens[s * rows + r] = r <= a ? target[s * rows + r] : -1;
  }
}

/* Draft-head id list with the sequence's tokens.  OpenJet engine page ("How
 * it gets its speed"): the drafter's head scores a fixed list of 32,768
 * common tokens, extended at run time by whichever ids of the current
 * sequence the list lacks; verification scores every vocabulary id.
 * Definition used here: the base list as given, then every id of seq in
 * order of first appearance that lies in [0, n_rows) and is neither in the
 * base list nor already added.  out has n_base + n_seq slots; the slots
 * after the union are -1.  Returns the length of the union. */
int64_t oracle_draft_union(const int32_t* base, int64_t n_base, const int32_t* seq, int64_t n_seq, int64_t n_rows,
                           int32_t* out) {
  unsigned char* seen = (unsigned char*)calloc((size_t)(n_rows > 0 ? n_rows : 1), 1);
  if (!seen) return -1;
  int64_t m = 0;
  for (int64_t i = 0; i < n_base; ++i) {
    out[m++] = base[i];
    if (base[i] >= 0 && base[i] < n_rows) seen[base[i]] = 1;
  }
  for (int64_t i = 0; i < n_seq; ++i) {
    int32_t id = seq[i];
    if (id < 0 || id >= n_rows || seen[id]) continue;
    seen[id] = 1;
    out[m++] = id;
  }
  for (int64_t i = m; i < n_base + n_seq; ++i) out[i] = -1;
  free(seen);
  return m;
}
