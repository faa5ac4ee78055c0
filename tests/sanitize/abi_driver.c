/*
 * abi_driver.c -- the host side of the C ABI (include/rattn.h) under
 * AddressSanitizer and UndefinedBehaviorSanitizer, without a GPU (test
 * infrastructure: tests/test_sanitize.py links it against a copy of the
 * library whose host code is built with both sanitizers, and runs it on the
 * CPU).
 *
 * Every call here is refused by the host-side checks, or has no work, before
 * anything is enqueued, so no kernel is launched and the fake device pointers
 * (aligned integers) are never dereferenced.  The calls cover each entry
 * point's checks of pointers, sizes, offsets, segment arrays, dtype, head
 * dimension and ring arguments, the overflow guards of the size arithmetic,
 * the split heuristic over a grid of shapes (a pure host function), and every
 * status string.  Exit status 0 when every call returns what the header
 * promises.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rattn.h"

static int failures = 0, calls = 0;
#define EXPECT(call, want)                                                        \
  do {                                                                            \
    const int got_ = (call);                                                      \
    ++calls;                                                                      \
    if (got_ != (want)) {                                                         \
      ++failures;                                                                 \
      fprintf(stderr, "FAIL line %d: %s returned %d, expected %d\n", __LINE__, #call, \
              got_, (int)(want));                                                 \
    }                                                                             \
  } while (0)

/* fake DEVICE pointers: 16-byte aligned, never dereferenced */
#define DP(i) ((void *)(uintptr_t)(0x10000u * ((i) + 1)))
#define FP(i) ((float *)DP(i))
#define IP(i) ((const int32_t *)DP(i))

static int fwd(const void *q, const void *k, int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d,
               int dtype, int causal, int W, int zigzag, int rank) {
  return rattn_fwd(q, k, DP(2), DP(3), FP(4), B, Hq, Hkv, Nq, N, d, dtype, 0.f, causal, W, zigzag,
                   rank, NULL);
}

static void check_fwd(void) {
  EXPECT(fwd(NULL, DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 1, 0, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 0, 2, 2, 64, 64, 64, RATTN_BF16, 1, 1, 0, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 3, 2, 64, 64, 64, RATTN_BF16, 1, 1, 0, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 0, 64, 64, 64, RATTN_BF16, 1, 1, 0, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 48, RATTN_BF16, 1, 1, 0, -1), RATTN_EUNSUPPORTED);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 256, RATTN_BF16, 1, 1, 0, -1), RATTN_EUNSUPPORTED);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 64, 3, 1, 1, 0, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 2, 1, 0, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 1, 2, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 0, 0, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 33, 0, -1), RATTN_EUNSUPPORTED);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 3, 0, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 68, 68, 64, RATTN_BF16, 1, 4, 1, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 4, 0, 4), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 4, 0, -2), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 16, 64, 64, RATTN_BF16, 1, 4, 0, -1), RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 4, 0, 1), RATTN_EINVAL);
  EXPECT(fwd((const char *)DP(0) + 2, DP(1), 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 1, 0, -1),
         RATTN_EINVAL);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, -4, -4, 64, RATTN_BF16, 1, 1, 0, -1), RATTN_EINVAL);
  /* element counts that overflow 64-bit offsets, and 2^31-row sequences */
  EXPECT(fwd(DP(0), DP(1), 1 << 30, 1 << 30, 1 << 30, 1 << 20, 1 << 20, 128, RATTN_BF16, 1, 1, 0,
             -1),
         RATTN_EUNSUPPORTED);
  EXPECT(fwd(DP(0), DP(1), 1, 1, 1, (int64_t)1 << 31, (int64_t)1 << 31, 64, RATTN_BF16, 1, 1, 0,
             -1),
         RATTN_EUNSUPPORTED);
  EXPECT(fwd(DP(0), DP(1), 1, 1, 1, INT64_MAX, INT64_MAX, 64, RATTN_BF16, 1, 1, 0, -1),
         RATTN_EUNSUPPORTED);
  /* no work: OK without a launch, null pointers allowed for empty tensors */
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 0, 0, 64, RATTN_BF16, 1, 1, 0, -1), RATTN_OK);
  EXPECT(fwd(DP(0), DP(1), 1, 2, 2, 0, 0, 64, RATTN_BF16, 1, 4, 1, -1), RATTN_OK);
  EXPECT(rattn_fwd(NULL, NULL, NULL, NULL, NULL, 1, 2, 2, 0, 0, 64, RATTN_F16, 0.f, 1, 1, 0, -1,
                   NULL),
         RATTN_OK);
  EXPECT(fwd(DP(0), NULL, 1, 2, 2, 64, 64, 64, RATTN_BF16, 1, 1, 0, -1), RATTN_EINVAL);
}

static void check_split(void) {
  const int64_t need = 4LL * 1 * 64 * 2 * 65;
  EXPECT(rattn_fwd_split(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 2, 2, 64, 64, 64, RATTN_BF16, 0.f,
                         1, 1, 0, -1, 0, FP(5), need, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_split(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 2, 2, 64, 64, 64, RATTN_BF16, 0.f,
                         1, 1, 0, -1, 65, FP(5), need, NULL),
         RATTN_EUNSUPPORTED);
  EXPECT(rattn_fwd_split(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 2, 2, 64, 64, 64, RATTN_BF16, 0.f,
                         1, 1, 0, -1, 4, NULL, need, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_split(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 2, 2, 64, 64, 64, RATTN_BF16, 0.f,
                         1, 1, 0, -1, 4, FP(5), 100, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_split(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 2, 2, 64, 64, 64, RATTN_BF16, 0.f,
                         1, 1, 0, -1, 4, (float *)((char *)DP(5) + 4), need, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_split(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 2, 2, 0, 0, 64, RATTN_BF16, 0.f, 1,
                         1, 0, -1, 4, NULL, 0, NULL),
         RATTN_OK);
  /* the fixed-scratch variant refuses what does not fit before any device call */
  EXPECT(rattn_fwd_split_noalloc(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 2, 2, 65536, 65536, 64,
                                 RATTN_BF16, 0.f, 1, 1, 0, -1, 64, NULL),
         RATTN_ESCRATCH);
  EXPECT(rattn_fwd_split_noalloc(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 32, 8, 1024, 1024, 128,
                                 RATTN_BF16, 0.f, 1, 1, 0, -1, 2, NULL),
         RATTN_ESCRATCH);
  EXPECT(rattn_fwd_split_noalloc(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 3, 2, 64, 64, 64,
                                 RATTN_BF16, 0.f, 1, 1, 0, -1, 4, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_split_noalloc(DP(0), DP(1), DP(2), DP(3), FP(4), 1, 2, 2, 0, 0, 64, RATTN_BF16,
                                 0.f, 1, 1, 0, -1, 4, NULL),
         RATTN_OK);
  /* split heuristic: always in [1, 64], 1 for what rattn_fwd rejects */
  static const int64_t lens[] = {0, 1, 64, 255, 256, 1000, 4096, 131072, (int64_t)1 << 40};
  static const int ds[] = {16, 32, 48, 64, 128};
  for (size_t a = 0; a < sizeof lens / sizeof lens[0]; ++a)
    for (size_t b = 0; b < sizeof lens / sizeof lens[0]; ++b)
      for (size_t c = 0; c < sizeof ds / sizeof ds[0]; ++c)
        for (int W = 1; W <= 8; W *= 2)
          for (int hq = 1; hq <= 64; hq *= 8) {
            const int h = rattn_split_hint(2, hq, lens[a], lens[b], ds[c], RATTN_BF16, W, W > 1,
                                           W > 1 ? 0 : -1, 256);
            ++calls;
            if (h < 1 || h > 64) {
              ++failures;
              fprintf(stderr, "FAIL split hint %d\n", h);
            }
          }
  EXPECT(rattn_split_hint(1, 1, 4096, 4096, 128, RATTN_BF16, 1, 0, -1, 256), 8);
  EXPECT(rattn_split_hint(0, 1, 4096, 4096, 128, RATTN_BF16, 1, 0, -1, 256), 1);
  EXPECT(rattn_split_hint(1, 1, 4096, 4096, 128, RATTN_BF16, 1, 0, -1, 0), 1);
}

static void check_steps(void) {
  int64_t qs[2] = {0, 0}, ql[2] = {32, 0}, ks[2] = {0, 0}, kl[2] = {32, 0};
  int64_t bad_len[2] = {30, 0}, neg[2] = {40, -8};
#define STEP(q_, qlen, klen, q_rows, q_off, k_rows, k_off, d, dtype, causal)                     \
  rattn_fwd_step(q_, DP(1), DP(2), FP(3), FP(4), 1, 4, 2, q_rows, q_off, 32, k_rows, k_off, 32, d, \
                 dtype, 0.f, causal, qs, qlen, ks, klen, NULL)
  /* no query rows: OK without a launch (null q and out allowed) */
  int64_t zero[2] = {0, 0};
  EXPECT(rattn_fwd_step(DP(0), DP(1), DP(2), FP(3), FP(4), 1, 4, 2, 32, 0, 0, 32, 0, 32, 128,
                        RATTN_F16, 0.f, 1, qs, zero, ks, kl, NULL),
         RATTN_OK);
  EXPECT(rattn_fwd_step(NULL, DP(1), DP(2), NULL, FP(4), 1, 4, 2, 32, 0, 0, 32, 0, 32, 128,
                        RATTN_F16, 0.f, 1, qs, zero, ks, kl, NULL),
         RATTN_OK);
  EXPECT(STEP(NULL, ql, kl, 32, 0, 32, 0, 128, RATTN_F16, 1), RATTN_EINVAL);
  EXPECT(STEP(DP(0), bad_len, kl, 32, 0, 32, 0, 128, RATTN_F16, 1), RATTN_EINVAL);
  EXPECT(STEP(DP(0), neg, kl, 32, 0, 32, 0, 128, RATTN_F16, 1), RATTN_EINVAL);
  EXPECT(STEP(DP(0), ql, kl, 32, 0, 32, 0, 12, RATTN_F16, 1), RATTN_EUNSUPPORTED);
  EXPECT(STEP(DP(0), ql, kl, 32, 0, 32, 0, 128, -1, 1), RATTN_EINVAL);
  EXPECT(STEP(DP(0), ql, kl, 32, 0, 32, 0, 128, RATTN_F16, -1), RATTN_EINVAL);
  EXPECT(STEP(DP(0), ql, kl, 32, 1, 32, 0, 128, RATTN_F16, 1), RATTN_EINVAL);   /* q_off + Nq > q_rows */
  EXPECT(STEP(DP(0), ql, kl, 64, -1, 32, 0, 128, RATTN_F16, 1), RATTN_EINVAL);  /* q_off < 0 */
  EXPECT(STEP(DP(0), ql, kl, 31, 0, 32, 0, 128, RATTN_F16, 1), RATTN_EINVAL);
  EXPECT(STEP(DP(0), ql, kl, 32, 0, 64, 40, 128, RATTN_F16, 1), RATTN_EINVAL);
  EXPECT(STEP(DP(0), ql, kl, 32, 0, 64, -1, 128, RATTN_F16, 1), RATTN_EINVAL);
  EXPECT(rattn_fwd_step(DP(0), DP(1), DP(2), FP(3), FP(4), 1, 4, 2, 32, 0, 32, 32, 0, 32, 128,
                        RATTN_F16, 0.f, 1, NULL, NULL, NULL, NULL, NULL),
         RATTN_EINVAL);
  /* merged step: the output row range must fit */
  EXPECT(rattn_fwd_step_merge(DP(0), DP(1), DP(2), FP(3), FP(4), 1, 4, 2, 32, 0, 32, 32, 0, 32,
                              128, RATTN_F16, 0.f, 1, qs, ql, ks, kl, 64, 40, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_step_merge(DP(0), DP(1), DP(2), FP(3), FP(4), 1, 4, 2, 32, 0, 32, 32, 0, 32,
                              128, RATTN_F16, 0.f, 1, qs, ql, ks, kl, 16, 0, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_step_merge(DP(0), DP(1), DP(2), FP(3), FP(4), 1, 4, 2, 32, 0, 32, 32, 0, 32,
                              128, RATTN_F16, 0.f, 1, qs, ql, ks, kl, 64, -1, NULL),
         RATTN_EINVAL);
  /* backward step: same checks of rows and segments */
  EXPECT(rattn_bwd_step(DP(0), DP(1), DP(2), DP(3), FP(4), FP(5), FP(6), FP(7), FP(8), 1, 4, 2,
                        32, 0, 32, 32, 0, 32, 128, RATTN_F16, 0.f, 1, qs, bad_len, ks, kl, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_bwd_step(DP(0), DP(1), DP(2), DP(3), FP(4), FP(5), FP(6), FP(7), FP(8), 1, 4, 2,
                        32, 8, 32, 32, 0, 32, 128, RATTN_F16, 0.f, 1, qs, ql, ks, kl, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_bwd_step(NULL, DP(1), DP(2), DP(3), FP(4), FP(5), FP(6), FP(7), FP(8), 1, 4, 2,
                        32, 0, 32, 32, 0, 32, 128, RATTN_F16, 0.f, 1, qs, ql, ks, kl, NULL),
         RATTN_EINVAL);
#undef STEP
}

static void check_merge_varlen_bwd(void) {
  EXPECT(rattn_merge(NULL, FP(1), FP(2), FP(3), 1, 2, 16, 8, 0, 64, NULL), RATTN_EINVAL);
  EXPECT(rattn_merge(FP(0), NULL, FP(2), FP(3), 1, 2, 16, 8, 0, 64, NULL), RATTN_EINVAL);
  EXPECT(rattn_merge(FP(0), FP(1), FP(2), FP(3), 0, 2, 16, 8, 0, 64, NULL), RATTN_EINVAL);
  EXPECT(rattn_merge(FP(0), FP(1), FP(2), FP(3), 1, 2, 16, -1, 0, 64, NULL), RATTN_EINVAL);
  EXPECT(rattn_merge(FP(0), FP(1), FP(2), FP(3), 1, 2, 16, 8, 9, 64, NULL), RATTN_EINVAL);
  EXPECT(rattn_merge(FP(0), FP(1), FP(2), FP(3), 1, 2, 16, 8, -1, 64, NULL), RATTN_EINVAL);
  EXPECT(rattn_merge(FP(0), FP(1), FP(2), FP(3), 1, 2, 16, 8, 0, 8, NULL), RATTN_EUNSUPPORTED);
  EXPECT(rattn_merge(FP(0), FP(1), FP(2), FP(3), 1, 2, 16, 0, 0, 64, NULL), RATTN_OK);

  EXPECT(rattn_fwd_varlen(DP(0), DP(1), DP(2), DP(3), FP(4), NULL, NULL, NULL, NULL, 2, 64, 128,
                          128, 4, 2, 64, RATTN_BF16, 0.f, 1, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_varlen(DP(0), DP(1), DP(2), DP(3), FP(4), IP(5), IP(6), IP(7), IP(8), -1, 64,
                          128, 128, 4, 2, 64, RATTN_BF16, 0.f, 1, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_varlen(DP(0), DP(1), DP(2), DP(3), FP(4), IP(5), IP(6), IP(7), IP(8), 2, 64,
                          128, 128, 4, 3, 64, RATTN_BF16, 0.f, 1, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_fwd_varlen(DP(0), DP(1), DP(2), DP(3), FP(4), IP(5), IP(6), IP(7), IP(8), 2, 64,
                          128, 128, 4, 2, 40, RATTN_BF16, 0.f, 1, NULL),
         RATTN_EUNSUPPORTED);
  EXPECT(rattn_fwd_varlen(DP(0), DP(1), DP(2), DP(3), FP(4), IP(5), IP(6), IP(7), IP(8), 0, 64,
                          128, 128, 4, 2, 64, RATTN_BF16, 0.f, 1, NULL),
         RATTN_OK);

  EXPECT(rattn_bwd_delta(NULL, DP(1), FP(2), 64, 64, RATTN_BF16, NULL), RATTN_EINVAL);
  EXPECT(rattn_bwd_delta(DP(0), DP(1), FP(2), -1, 64, RATTN_BF16, NULL), RATTN_EINVAL);
  EXPECT(rattn_bwd_delta(DP(0), DP(1), FP(2), 64, 8, RATTN_BF16, NULL), RATTN_EUNSUPPORTED);
  EXPECT(rattn_bwd_delta(DP(0), DP(1), FP(2), 0, 64, RATTN_BF16, NULL), RATTN_OK);

  EXPECT(rattn_bwd(NULL, DP(1), DP(2), DP(3), FP(4), DP(5), DP(6), DP(7), DP(8), FP(9), 1, 2, 2,
                   64, 64, 64, RATTN_BF16, 0.f, 1, 1, 0, -1, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_bwd(DP(0), DP(1), DP(2), DP(3), FP(4), DP(5), DP(6), DP(7), DP(8), NULL, 1, 2, 2,
                   64, 64, 64, RATTN_BF16, 0.f, 1, 1, 0, -1, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_bwd(DP(0), DP(1), DP(2), DP(3), FP(4), DP(5), DP(6), DP(7), DP(8), FP(9), 1, 3, 2,
                   64, 64, 64, RATTN_BF16, 0.f, 1, 1, 0, -1, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_bwd(DP(0), DP(1), DP(2), DP(3), FP(4), DP(5), DP(6), DP(7), DP(8), FP(9), 1, 2, 2,
                   64, 64, 48, RATTN_BF16, 0.f, 1, 1, 0, -1, NULL),
         RATTN_EUNSUPPORTED);
  EXPECT(rattn_bwd(DP(0), DP(1), DP(2), DP(3), FP(4), DP(5), DP(6), DP(7), DP(8), FP(9), 1, 2, 2,
                   64, 64, 64, RATTN_BF16, 0.f, 1, 3, 0, -1, NULL),
         RATTN_EINVAL);
  EXPECT(rattn_bwd_varlen(DP(0), DP(1), DP(2), DP(3), FP(4), DP(5), DP(6), DP(7), DP(8), FP(9),
                          NULL, IP(11), IP(12), IP(13), 2, 64, 64, 128, 128, 4, 2, 64, RATTN_BF16,
                          0.f, 1, NULL),
         RATTN_EINVAL);
}

static void check_status_strings(void) {
  for (int s = -8; s <= 2; ++s) {
    const char *t = rattn_status_string(s);
    ++calls;
    if (!t || !t[0]) {
      ++failures;
      fprintf(stderr, "FAIL status string %d\n", s);
    }
  }
  ++calls;
  if (strcmp(rattn_status_string(12345), "unknown status") != 0) {
    ++failures;
    fprintf(stderr, "FAIL unknown status string\n");
  }
}

int main(void) {
  check_fwd();
  check_split();
  check_steps();
  check_merge_varlen_bwd();
  check_status_strings();
  printf("abi_driver: %d calls, %d failures\n", calls, failures);
  return failures ? 1 : 0;
}
