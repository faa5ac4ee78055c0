/*
 * oracle_driver.c -- runs every entry point of oracle/oracle.c over a sweep of
 * shapes, built with AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure: tests/test_sanitize.py builds and runs it on the CPU).
 *
 * Every buffer is allocated at its exact size, so a read or write past an end
 * stops the run.  Beside memory safety it checks properties that hold for any
 * correct implementation of the definition the oracle computes:
 *   - a row with no visible key has lse = -inf and out = 0; any other row is
 *     a convex combination of value rows (finite, within [min v, max v]);
 *   - attention over a key set equals the log-sum-exp merge of attention over
 *     its two halves;
 *   - explicit row lists give the rows of the full (rows = NULL) call;
 *   - sum_j dV_j = sum_i dO_i over the rows that see a key (the probabilities
 *     of a row sum to 1), per key/value head;
 *   - invalid arguments return -1.
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_attention_rows(const void *q, const void *k, const void *v, int dtype, int B, int Hq,
                          int Hkv, int64_t Nq, int64_t Nk, int d, const int64_t *q_pos,
                          const int64_t *k_pos, int causal, double scale, int64_t n_rows,
                          const int64_t *rows, double *out, double *lse, int n_threads);
int oracle_merge_rows(const double *o_a, const double *l_a, const double *o_b,
                      const double *l_b, int64_t n_rows, int d, double *o_out, double *l_out);
int oracle_bwd_stats(const void *q, const void *k, const void *v, const void *dout, int dtype,
                     int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int d,
                     const int64_t *q_pos, const int64_t *k_pos, int causal, double scale,
                     int64_t n_rows, const int64_t *rows, double *lse, double *delta,
                     int n_threads);
int oracle_bwd_dq(const void *q, const void *k, const void *v, const void *dout, int dtype,
                  int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int d,
                  const int64_t *q_pos, const int64_t *k_pos, int causal, double scale,
                  const double *lse_all, const double *delta_all, int64_t n_rows,
                  const int64_t *rows, double *dq, int n_threads);
int oracle_bwd_dkv(const void *q, const void *k, const void *v, const void *dout, int dtype,
                   int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int d,
                   const int64_t *q_pos, const int64_t *k_pos, int causal, double scale,
                   const double *lse_all, const double *delta_all, int64_t n_rows,
                   const int64_t *rows, double *dk, double *dv, int n_threads);
double oracle_f16_to_double(uint16_t h);
double oracle_bf16_to_double(uint16_t b);

static int failures = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      ++failures;                                         \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                       \
      fputc('\n', stderr);                                \
    }                                                     \
  } while (0)

/* xorshift64*: deterministic test data */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}
static double unif(void) { return (double)(rnd() >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0; }

static size_t elem_size(int dtype) { return dtype == 0 ? 4 : 2; }

/* A finite value of the storage type near x (f32; bf16 by truncation; f16 by
 * building the bit pattern of a value in [-2, 2]). */
static void store(void *base, int64_t i, int dtype, double x) {
  if (dtype == 0) {
    ((float *)base)[i] = (float)x;
  } else if (dtype == 2) {
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    ((uint16_t *)base)[i] = (uint16_t)(u >> 16);
  } else {
    /* f16: sign, exponent 10..15 (values 2^-5 .. 2^0 scale), random fraction */
    uint16_t s = x < 0 ? 0x8000u : 0u;
    uint16_t e = (uint16_t)(10 + (rnd() % 6));
    uint16_t f = (uint16_t)(rnd() & 0x3FFu);
    ((uint16_t *)base)[i] = (uint16_t)(s | (e << 10) | f);
  }
}
static double decode(const void *base, int64_t i, int dtype) {
  if (dtype == 0) return ((const float *)base)[i];
  if (dtype == 1) return oracle_f16_to_double(((const uint16_t *)base)[i]);
  return oracle_bf16_to_double(((const uint16_t *)base)[i]);
}

static void *tensor(int64_t n, int dtype) {
  void *p = malloc((size_t)(n > 0 ? n : 1) * elem_size(dtype));
  for (int64_t i = 0; i < n; ++i) store(p, i, dtype, unif());
  return p;
}

static void run_case(int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int d, int dtype,
                     int causal, int64_t q_shift) {
  const int group = Hq / Hkv;
  void *q = tensor((int64_t)B * Nq * Hq * d, dtype);
  void *k = tensor((int64_t)B * Nk * Hkv * d, dtype);
  void *v = tensor((int64_t)B * Nk * Hkv * d, dtype);
  void *dout = tensor((int64_t)B * Nq * Hq * d, dtype);
  int64_t *q_pos = malloc(sizeof(int64_t) * (size_t)(Nq > 0 ? Nq : 1));
  int64_t *k_pos = malloc(sizeof(int64_t) * (size_t)(Nk > 0 ? Nk : 1));
  /* queries aligned with the last keys, shifted by q_shift (negative: some
   * rows see no key under the causal rule) */
  for (int64_t i = 0; i < Nq; ++i) q_pos[i] = Nk - Nq + i + q_shift;
  for (int64_t j = 0; j < Nk; ++j) k_pos[j] = j;
  const double scale = 1.0 / sqrt((double)d);
  const int64_t nr = (int64_t)B * Nq * Hq;
  double *out = malloc(sizeof(double) * (size_t)(nr * d > 0 ? nr * d : 1));
  double *lse = malloc(sizeof(double) * (size_t)(nr > 0 ? nr : 1));

  int rc = oracle_attention_rows(q, k, v, dtype, B, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal,
                                 scale, nr, NULL, out, lse, 2);
  CHECK(rc == 0, "attention rc %d", rc);

  /* empty rows and convex combinations */
  for (int64_t r = 0; r < nr; ++r) {
    const int64_t hq = r % Hq, i = (r / Hq) % Nq, b = r / ((int64_t)Hq * Nq);
    const int64_t g = hq / group;
    int64_t nvis = 0;
    for (int64_t j = 0; j < Nk; ++j) nvis += (!causal || k_pos[j] <= q_pos[i]);
    if (nvis == 0) {
      CHECK(isinf(lse[r]) && lse[r] < 0, "row %lld: no key but lse %g", (long long)r, lse[r]);
      for (int t = 0; t < d; ++t) CHECK(out[r * d + t] == 0.0, "row %lld: no key, out != 0", (long long)r);
      continue;
    }
    CHECK(isfinite(lse[r]), "row %lld: lse %g", (long long)r, lse[r]);
    for (int t = 0; t < d; ++t) {
      double lo = INFINITY, hi = -INFINITY;
      for (int64_t j = 0; j < Nk; ++j) {
        if (causal && k_pos[j] > q_pos[i]) continue;
        const double x = decode(v, ((b * Nk + j) * Hkv + g) * d + t, dtype);
        lo = x < lo ? x : lo;
        hi = x > hi ? x : hi;
      }
      const double o = out[r * d + t], tol = 1e-12 * (fabs(lo) + fabs(hi) + 1.0);
      CHECK(o >= lo - tol && o <= hi + tol, "row %lld col %d: %g outside [%g, %g]",
            (long long)r, t, o, lo, hi);
    }
  }

  /* explicit row list (every third row, reversed) matches the full call */
  {
    int64_t n = 0;
    int64_t *rows = malloc(sizeof(int64_t) * 3 * (size_t)(nr > 0 ? nr : 1));
    for (int64_t r = nr - 1; r >= 0; r -= 3) {
      rows[3 * n] = r / ((int64_t)Hq * Nq);
      rows[3 * n + 1] = (r / Hq) % Nq;
      rows[3 * n + 2] = r % Hq;
      ++n;
    }
    double *o2 = malloc(sizeof(double) * (size_t)(n * d > 0 ? n * d : 1));
    double *l2 = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    rc = oracle_attention_rows(q, k, v, dtype, B, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal,
                               scale, n, rows, o2, l2, 1);
    CHECK(rc == 0, "row-list attention rc %d", rc);
    for (int64_t m = 0; m < n; ++m) {
      const int64_t r = (rows[3 * m] * Nq + rows[3 * m + 1]) * Hq + rows[3 * m + 2];
      CHECK(l2[m] == lse[r] || (isinf(l2[m]) && isinf(lse[r])), "row list lse differs");
      for (int t = 0; t < d; ++t) CHECK(o2[m * d + t] == out[r * d + t], "row list out differs");
    }
    free(rows);
    free(o2);
    free(l2);
  }

  /* merge of the two key halves == all keys (B = 1 views: split k/v rows) */
  if (B == 1 && Nk >= 2) {
    const int64_t h = Nk / 2;
    const size_t kv_half = (size_t)(h * Hkv * d) * elem_size(dtype);
    double *oa = malloc(sizeof(double) * (size_t)(nr * d > 0 ? nr * d : 1));
    double *la = malloc(sizeof(double) * (size_t)(nr > 0 ? nr : 1));
    double *ob = malloc(sizeof(double) * (size_t)(nr * d > 0 ? nr * d : 1));
    double *lb = malloc(sizeof(double) * (size_t)(nr > 0 ? nr : 1));
    rc = oracle_attention_rows(q, k, v, dtype, 1, Hq, Hkv, Nq, h, d, q_pos, k_pos, causal,
                               scale, nr, NULL, oa, la, 2);
    CHECK(rc == 0, "first half rc %d", rc);
    rc = oracle_attention_rows(q, (const char *)k + kv_half, (const char *)v + kv_half, dtype, 1,
                               Hq, Hkv, Nq, Nk - h, d, q_pos, k_pos + h, causal, scale, nr, NULL,
                               ob, lb, 2);
    CHECK(rc == 0, "second half rc %d", rc);
    rc = oracle_merge_rows(oa, la, ob, lb, nr, d, oa, la);  /* in place, as documented */
    CHECK(rc == 0, "merge rc %d", rc);
    for (int64_t r = 0; r < nr; ++r) {
      if (isinf(lse[r])) {
        CHECK(isinf(la[r]) && la[r] < 0, "merged empty row");
        continue;
      }
      CHECK(fabs(la[r] - lse[r]) <= 1e-12 * (1.0 + fabs(lse[r])), "merged lse %g vs %g", la[r],
            lse[r]);
      for (int t = 0; t < d; ++t)
        CHECK(fabs(oa[r * d + t] - out[r * d + t]) <= 1e-12, "merged out differs");
    }
    free(oa);
    free(la);
    free(ob);
    free(lb);
  }

  /* backward: stats, dq, dkv; sum_j dV_j = sum_i dO_i over rows with a key */
  {
    double *l3 = malloc(sizeof(double) * (size_t)(nr > 0 ? nr : 1));
    double *delta = malloc(sizeof(double) * (size_t)(nr > 0 ? nr : 1));
    double *dq = malloc(sizeof(double) * (size_t)(nr * d > 0 ? nr * d : 1));
    const int64_t nk_rows = (int64_t)B * Nk * Hkv;
    double *dk = malloc(sizeof(double) * (size_t)(nk_rows * d > 0 ? nk_rows * d : 1));
    double *dv = malloc(sizeof(double) * (size_t)(nk_rows * d > 0 ? nk_rows * d : 1));
    rc = oracle_bwd_stats(q, k, v, dout, dtype, B, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal, scale,
                          nr, NULL, l3, delta, 2);
    CHECK(rc == 0, "bwd_stats rc %d", rc);
    rc = oracle_bwd_dq(q, k, v, dout, dtype, B, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal, scale,
                       l3, delta, nr, NULL, dq, 2);
    CHECK(rc == 0, "bwd_dq rc %d", rc);
    rc = oracle_bwd_dkv(q, k, v, dout, dtype, B, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal, scale,
                        l3, delta, nk_rows, NULL, dk, dv, 2);
    CHECK(rc == 0, "bwd_dkv rc %d", rc);
    for (int64_t r = 0; r < nr * d; ++r) CHECK(isfinite(dq[r]), "dq not finite");
    for (int b = 0; b < B; ++b)
      for (int g = 0; g < Hkv; ++g)
        for (int t = 0; t < d; ++t) {
          double sv = 0.0, so = 0.0, mag = 0.0;
          for (int64_t j = 0; j < Nk; ++j) sv += dv[(((int64_t)b * Nk + j) * Hkv + g) * d + t];
          for (int hq = g * group; hq < (g + 1) * group; ++hq)
            for (int64_t i = 0; i < Nq; ++i) {
              const int64_t r = ((int64_t)b * Nq + i) * Hq + hq;
              if (isinf(l3[r])) continue;
              const double x = decode(dout, r * d + t, dtype);
              so += x;
              mag += fabs(x);
            }
          CHECK(fabs(sv - so) <= 1e-11 * (1.0 + mag), "sum dV %g vs sum dO %g", sv, so);
        }
    free(l3);
    free(delta);
    free(dq);
    free(dk);
    free(dv);
  }

  free(q);
  free(k);
  free(v);
  free(dout);
  free(q_pos);
  free(k_pos);
  free(out);
  free(lse);
}

static void invalid_arguments(void) {
  float x[64] = {0};
  int64_t pos[4] = {0, 1, 2, 3};
  double o[64], l[4];
  /* null pointers, Hq not a multiple of Hkv, bad dtype, missing positions, row
   * count that does not match rows = NULL, a row triple out of range */
  CHECK(oracle_attention_rows(NULL, x, x, 0, 1, 1, 1, 4, 4, 4, pos, pos, 1, 1.0, 4, NULL, o, l, 1) == -1, "null q");
  CHECK(oracle_attention_rows(x, x, x, 0, 1, 3, 2, 1, 4, 4, pos, pos, 0, 1.0, 3, NULL, o, l, 1) == -1, "Hq not a multiple of Hkv");
  CHECK(oracle_attention_rows(x, x, x, 7, 1, 1, 1, 4, 4, 4, pos, pos, 0, 1.0, 4, NULL, o, l, 1) == -1, "dtype");
  CHECK(oracle_attention_rows(x, x, x, 0, 1, 1, 1, 4, 4, 4, NULL, pos, 1, 1.0, 4, NULL, o, l, 1) == -1, "q_pos");
  CHECK(oracle_attention_rows(x, x, x, 0, 1, 1, 1, 4, 4, 4, pos, pos, 1, 1.0, 3, NULL, o, l, 1) == -1, "n_rows");
  int64_t bad_row[3] = {0, 9, 0};
  CHECK(oracle_attention_rows(x, x, x, 0, 1, 1, 1, 4, 4, 4, pos, pos, 1, 1.0, 1, bad_row, o, l, 1) == -1, "row range");
  CHECK(oracle_merge_rows(o, l, NULL, l, 1, 4, o, l) == -1, "merge null");
  CHECK(oracle_merge_rows(o, l, o, l, -1, 4, o, l) == -1, "merge n_rows");
  CHECK(oracle_bwd_stats(x, x, x, NULL, 0, 1, 1, 1, 4, 4, 4, pos, pos, 1, 1.0, 4, NULL, l, l, 1) == -1, "bwd null dout");
  CHECK(oracle_bwd_dq(x, x, x, x, 0, 1, 1, 1, 4, 4, 4, pos, pos, 1, 1.0, NULL, l, 4, NULL, o, 1) == -1, "dq null lse");
  CHECK(oracle_bwd_dkv(x, x, x, x, 0, 1, 1, 1, 4, 4, 4, pos, pos, 1, 1.0, l, l, 3, NULL, o, o, 1) == -1, "dkv n_rows");
}

int main(void) {
  static const int ds[] = {1, 16, 64, 128};
  static const int heads[][2] = {{1, 1}, {4, 2}, {4, 1}};
  static const int64_t lens[][2] = {{1, 1}, {5, 3}, {3, 5}, {17, 33}, {40, 40}};
  int cases = 0;
  for (int dt = 0; dt < 3; ++dt)
    for (size_t di = 0; di < sizeof ds / sizeof ds[0]; ++di)
      for (size_t hi = 0; hi < sizeof heads / sizeof heads[0]; ++hi)
        for (size_t li = 0; li < sizeof lens / sizeof lens[0]; ++li)
          for (int causal = 0; causal < 2; ++causal)
            for (int B = 1; B <= 2; ++B) {
              const int64_t shift = causal ? -(int64_t)(li % 3) * 2 : 0;
              run_case(B, heads[hi][0], heads[hi][1], lens[li][0], lens[li][1], ds[di], dt, causal,
                       shift);
              ++cases;
            }
  /* no keys at all, and no queries */
  run_case(1, 2, 1, 4, 0, 16, 2, 1, 0);
  run_case(1, 2, 1, 0, 4, 16, 1, 0, 0);
  cases += 2;
  invalid_arguments();
  printf("oracle_driver: %d cases, %d failures\n", cases, failures);
  return failures ? 1 : 0;
}
