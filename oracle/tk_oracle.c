/*
 * CPU oracle for the exact row-wise bf16 top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or constant with the HIP library it checks.
 *
 * What is computed (TensorFold PR #713 "the drafter's attention and top-k use
 * more of the GPU", change 3 and the Exactness table):
 *   - each row's top-k entries ordered by score, highest first, with ties
 *     between equal scores going to the lower column (token) index;
 *   - per row an entry count and a non-finite mask;
 *   - the cases that must be exact: ties, both zeros, NaN and infinities, and
 *     padded row strides.
 * Readings taken where that page is silent (each is a plain reading):
 *   - NaN of any sign or payload is never an entry; it sets mask bit 1;
 *   - +inf and -inf are ranked by value and set mask bits 2 and 4;
 *   - +0 and -0 compare equal (ties go to the lower column); an entry's value
 *     is the input's own bit pattern, so a -0 entry stays 0x8000;
 *   - count = min(k, number of non-NaN columns); entry slots at and past
 *     count hold index -1 and value 0x7FC0;
 *   - row_stride is in elements; columns [cols, row_stride) are never read.
 *
 * The same for IEEE binary32 (fp32) rows, tko_topk_f32, with 32-bit inputs,
 * 32-bit entry values (the input's own bits) and the fill value 0x7FC00000
 * (a quiet fp32 NaN).
 *
 * The same for IEEE binary16 (fp16) rows, tko_topk_f16: the definition is
 * the same, only the widening of a 16-bit pattern to its value differs (the
 * pages' rows are bf16; fp16 logits are this library's extension, and take
 * the same readings: NaN excluded and flagged, infinities ranked, zeros
 * equal, padding never read).
 *
 * Method: every value is widened exactly to double, non-NaN values are
 * collected with their column, and the list is sorted with qsort under the
 * comparison "larger value first, then smaller column first".  Because no two
 * entries share a column, that comparison is a strict total order and the
 * sorted list is unique.  The first min(k, n) entries are the answer.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  double value;
  int32_t col;
} tko_entry;

/* Exact widening of a bf16 bit pattern: bf16 is the top half of a binary32. */
static double bf16_value(uint32_t bits) {
  uint32_t u = (bits & 0xFFFFu) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Exact widening of an IEEE binary16 pattern: sign, 5-bit exponent (bias
 * 15), 10-bit fraction; exponent 0 holds zeros and subnormals (fraction *
 * 2^-24), exponent 31 infinities (fraction 0) and NaN. */
static double f16_value(uint32_t bits) {
  const int sign = (bits >> 15) & 1, e = (bits >> 10) & 31, f = bits & 1023;
  double v;
  if (e == 31) v = f ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)f, -24);
  else v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* Exact widening of an IEEE binary32 pattern. */
static double f32_value(uint32_t bits) {
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* qsort comparator: negative when a comes first in (score desc, column asc). */
static int score_then_lower_column(const void *pa, const void *pb) {
  const tko_entry *a = (const tko_entry *)pa;
  const tko_entry *b = (const tko_entry *)pb;
  if (a->value > b->value) return -1;
  if (a->value < b->value) return 1;
  if (a->col < b->col) return -1;
  if (a->col > b->col) return 1;
  return 0;
}

typedef struct {
  double (*widen)(uint32_t);  /* exact value of one input word */
  int word;                   /* bytes per input and entry value: 2 or 4 */
  uint32_t fill;              /* entry value of empty slots */
  int64_t row_begin, row_end, cols, row_stride;
  int32_t k;
  const void *in;
  int32_t *out_idx;
  void *out_val;
  int32_t *out_count;
  uint32_t *out_nonfinite;
  int status;
} tko_job;

static uint32_t word_at(const void *base, int64_t i, int word) {
  return word == 2 ? ((const uint16_t *)base)[i] : ((const uint32_t *)base)[i];
}

static void put_word(void *base, int64_t i, uint32_t v, int word) {
  if (word == 2) ((uint16_t *)base)[i] = (uint16_t)v;
  else ((uint32_t *)base)[i] = v;
}

static void *run_rows(void *arg) {
  tko_job *job = (tko_job *)arg;
  tko_entry *list = (tko_entry *)malloc((size_t)(job->cols > 0 ? job->cols : 1) * sizeof(tko_entry));
  if (!list) {
    job->status = -1;
    return NULL;
  }
  for (int64_t r = job->row_begin; r < job->row_end; ++r) {
    const int64_t row = r * job->row_stride;
    uint32_t mask = 0;
    int64_t n = 0;
    for (int64_t c = 0; c < job->cols; ++c) {
      double v = job->widen(word_at(job->in, row + c, job->word));
      if (isnan(v)) {
        mask |= 1u;
        continue;
      }
      if (isinf(v)) mask |= (v > 0) ? 2u : 4u;
      list[n].value = v;
      list[n].col = (int32_t)c;
      ++n;
    }
    qsort(list, (size_t)n, sizeof(tko_entry), score_then_lower_column);
    int64_t count = n < job->k ? n : job->k;
    for (int64_t j = 0; j < job->k; ++j) {
      int64_t o = r * job->k + j;
      if (j < count) {
        job->out_idx[o] = list[j].col;
        put_word(job->out_val, o, word_at(job->in, row + list[j].col, job->word), job->word);
      } else {
        job->out_idx[o] = -1;
        put_word(job->out_val, o, job->fill, job->word);
      }
    }
    job->out_count[r] = (int32_t)count;
    job->out_nonfinite[r] = mask;
  }
  free(list);
  job->status = 0;
  return NULL;
}

static int topk_rows(double (*widen)(uint32_t), int word, uint32_t fill, int64_t rows, int64_t cols,
                     int64_t row_stride, int32_t k, const void *in, int32_t *out_idx, void *out_val,
                     int32_t *out_count, uint32_t *out_nonfinite, int32_t threads) {
  if (rows < 0 || cols < 0 || cols > INT32_MAX || row_stride < cols || k < 1) return -1;
  if (rows == 0) return 0;
  if ((cols > 0 && !in) || !out_idx || !out_val || !out_count || !out_nonfinite) return -1;
  if (threads < 1) threads = 1;
  if (threads > rows) threads = (int32_t)rows;

  tko_job *jobs = (tko_job *)calloc((size_t)threads, sizeof(tko_job));
  pthread_t *tids = (pthread_t *)calloc((size_t)threads, sizeof(pthread_t));
  if (!jobs || !tids) {
    free(jobs);
    free(tids);
    return -1;
  }
  for (int32_t t = 0; t < threads; ++t) {
    tko_job *j = &jobs[t];
    j->widen = widen;
    j->word = word;
    j->fill = fill;
    j->row_begin = rows * t / threads;
    j->row_end = rows * (t + 1) / threads;
    j->cols = cols;
    j->row_stride = row_stride;
    j->k = k;
    j->in = in;
    j->out_idx = out_idx;
    j->out_val = out_val;
    j->out_count = out_count;
    j->out_nonfinite = out_nonfinite;
    j->status = -1;
  }
  int started = 0;
  for (int32_t t = 1; t < threads; ++t) {
    if (pthread_create(&tids[t], NULL, run_rows, &jobs[t]) != 0) break;
    started = t;
  }
  run_rows(&jobs[0]);
  /* rows of threads that could not start run here, in order */
  for (int32_t t = started + 1; t < threads; ++t) run_rows(&jobs[t]);
  for (int32_t t = 1; t <= started; ++t) pthread_join(tids[t], NULL);
  int status = 0;
  for (int32_t t = 0; t < threads; ++t)
    if (jobs[t].status != 0) status = -1;
  free(jobs);
  free(tids);
  return status;
}

/*
 * Row-wise top-k of a rows x cols bf16 matrix stored with row_stride elements
 * between row starts.  Outputs are dense: out_idx/out_val [rows][k],
 * out_count/out_nonfinite [rows].  Rows are split into contiguous blocks over
 * `threads` POSIX threads (threads <= 1 runs on the caller's thread).
 * Returns 0, or -1 for invalid arguments or an allocation failure.
 */
int tko_topk_bf16(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                  int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                  int32_t threads) {
  return topk_rows(bf16_value, 2, 0x7FC0u, rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite,
                   threads);
}

/* The same for fp16 bit patterns. */
int tko_topk_f16(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint16_t *in,
                 int32_t *out_idx, uint16_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                 int32_t threads) {
  return topk_rows(f16_value, 2, 0x7FC0u, rows, cols, row_stride, k, in, out_idx, out_val, out_count, out_nonfinite,
                   threads);
}

/* The same for fp32 bit patterns: 32-bit entry values, fill 0x7FC00000. */
int tko_topk_f32(int64_t rows, int64_t cols, int64_t row_stride, int32_t k, const uint32_t *in,
                 int32_t *out_idx, uint32_t *out_val, int32_t *out_count, uint32_t *out_nonfinite,
                 int32_t threads) {
  return topk_rows(f32_value, 4, 0x7FC00000u, rows, cols, row_stride, k, in, out_idx, out_val, out_count,
                   out_nonfinite, threads);
}

/* Exact widenings, exposed for the pins. */
double tko_bf16_value(uint16_t bits) { return bf16_value(bits); }
double tko_f16_value(uint16_t bits) { return f16_value(bits); }

