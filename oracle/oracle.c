/*
 * oracle.c -- fp64 CPU reference for exact attention.  TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load
 * this library.  It shares no code, header or constant with the HIP path
 * (ring_attention_amd/), and the HIP path never loads it.
 *
 * What it computes is the plain definition of attention, not any blockwise
 * algorithm:
 *
 *   Attn(Q,K,V) = softmax(scale * Q K^T) V
 *
 * as stated at the top of the guijiagi.com page "ring-attention-explained"
 * (section on the memory wall of naive attention, first formula), with
 * scale = 1/sqrt(d) by default (same formula; also the default softmax_scale
 * of the flash-attn usage example on the yz520gzy FlashAttention chapter).
 * The blockwise pages (youngju.dev "Ring Attention" analysis, blockwise and
 * ring functions; guijiagi.com "key insight" and "mathematical proof"
 * sections) state that the blockwise / ring computation reaches exactly this
 * result, so the definition is the oracle.
 *
 * Per query row (b, i, hq), with global position pq(i):
 *   g     = hq / (Hq / Hkv)                 contiguous GQA groups (a reading:
 *                                           the pages name GQA but no mapping)
 *   A     = { j : !causal or pk(j) <= pq(i) }   (causal: a key is visible iff it
 *                                           is not later than the query; the
 *                                           youngju.dev causal step masks the
 *                                           strict upper triangle)
 *   s_j   = scale * sum_t q[b,i,hq,t] * k[b,j,g,t]
 *   M     = max_{j in A} s_j
 *   Z     = sum_{j in A} exp(s_j - M)
 *   O     = sum_{j in A} exp(s_j - M) v[b,j,g,:] / Z
 *   LSE   = M + ln Z                        (natural log; the youngju.dev
 *                                           backward uses P = exp(S - lse))
 *   A empty:  O = 0, LSE = -inf.
 *
 * Two passes per row (max, then the weighted sums), everything in double,
 * no blocking.  The second half of this file holds the gradients of the same
 * definition (dQ, dK, dV of a loss with upstream gradient dO).  Inputs are read in their storage type (fp32, fp16 or bf16 bit
 * patterns) and converted exactly to double by the decoders below.
 *
 * Layout: q [B, Nq, Hq, d], k and v [B, Nk, Hkv, d], contiguous, row-major
 * (batch, sequence, heads, head_dim) as in the flash-attn usage example.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 * (no -ffast-math: every operation is IEEE double in program order).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2 };

/* IEEE binary16 -> double, exact.  sign(1) exponent(5, bias 15) fraction(10). */
double oracle_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);               /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(f | 0x400), e - 25);  /* (1024 + f) * 2^(e-15-10) */
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32: widen, then convert. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float x;
    memcpy(&x, &u, sizeof x);
    return (double)x;
}

/* Tables of the two decoders above, one entry per 16-bit pattern, so that the
 * inner loops read a table instead of calling the decoder. */
static double lut_f16[65536], lut_bf16[65536];
static int lut_ready;

static void build_luts(void)
{
    if (lut_ready) return;
    for (uint32_t b = 0; b < 65536; ++b) {
        lut_f16[b] = oracle_f16_to_double((uint16_t)b);
        lut_bf16[b] = oracle_bf16_to_double((uint16_t)b);
    }
    lut_ready = 1;
}

static double load(const void *base, int64_t idx, int dtype)
{
    switch (dtype) {
    case ORACLE_F32: return (double)((const float *)base)[idx];
    case ORACLE_F16: return lut_f16[((const uint16_t *)base)[idx]];
    default:         return lut_bf16[((const uint16_t *)base)[idx]];
    }
}

/*
 * One query row (b, i, hq): the definition above, two passes.  `dtype` is a
 * compile-time constant at each call site below, so the decoder switch in
 * load() folds away; the arithmetic is the same for every dtype.
 */
static inline __attribute__((always_inline)) void
attend_row(const void *q, const void *k, const void *v, const int dtype, int Hq, int Hkv,
           int64_t Nq, int64_t Nk, int d, const int64_t *q_pos, const int64_t *k_pos,
           int causal, double scale, int group, int64_t b, int64_t i, int64_t hq,
           double *s, double *qrow, double *acc, double *o, double *lse_r)
{
    const int64_t g = hq / group;
    for (int t = 0; t < d; ++t)
        qrow[t] = load(q, ((b * Nq + i) * Hq + hq) * d + t, dtype);

    /* pass 1: scores of the visible keys and their maximum */
    double M = -INFINITY;
    int64_t n_visible = 0;
    for (int64_t j = 0; j < Nk; ++j) {
        if (causal && k_pos[j] > q_pos[i]) {
            s[j] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        const int64_t kbase = ((b * Nk + j) * Hkv + g) * d;
        for (int t = 0; t < d; ++t)
            dot += qrow[t] * load(k, kbase + t, dtype);
        s[j] = scale * dot;
        if (s[j] > M) M = s[j];
        ++n_visible;
    }
    if (n_visible == 0) {
        for (int t = 0; t < d; ++t) o[t] = 0.0;
        *lse_r = -INFINITY;
        return;
    }
    /* pass 2: normaliser and weighted sum of values */
    double Z = 0.0;
    for (int t = 0; t < d; ++t) acc[t] = 0.0;
    for (int64_t j = 0; j < Nk; ++j) {
        if (causal && k_pos[j] > q_pos[i]) continue;
        const double w = exp(s[j] - M);
        Z += w;
        const int64_t vbase = ((b * Nk + j) * Hkv + g) * d;
        for (int t = 0; t < d; ++t)
            acc[t] += w * load(v, vbase + t, dtype);
    }
    for (int t = 0; t < d; ++t) o[t] = acc[t] / Z;
    *lse_r = M + log(Z);
}

/*
 * Attention for a list of query rows.
 *   rows     : n_rows triples (b, i, hq), or NULL for every row in (b, i, hq)
 *              row-major order (n_rows must then equal B*Nq*Hq)
 *   q_pos    : [Nq] global position of each query row (used when causal)
 *   k_pos    : [Nk] global position of each key row   (used when causal)
 *   out      : [n_rows, d] double
 *   lse      : [n_rows] double
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_attention_rows(const void *q, const void *k, const void *v, int dtype,
                          int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int d,
                          const int64_t *q_pos, const int64_t *k_pos, int causal,
                          double scale, int64_t n_rows, const int64_t *rows,
                          double *out, double *lse, int n_threads)
{
    if (!q || !k || !v || !out || !lse || B < 1 || Hq < 1 || Hkv < 1 || d < 1 ||
        Nq < 0 || Nk < 0 || Hq % Hkv != 0 || (causal && (!q_pos || !k_pos)) ||
        dtype < ORACLE_F32 || dtype > ORACLE_BF16)
        return -1;
    if (!rows && n_rows != (int64_t)B * Nq * Hq)
        return -1;
    const int group = Hq / Hkv;
    int bad = 0;
    build_luts();  /* before the parallel region: no concurrent writers */
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif

#pragma omp parallel reduction(| : bad)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qrow || !acc) {
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t b, i, hq;
                if (rows) {
                    b = rows[3 * r]; i = rows[3 * r + 1]; hq = rows[3 * r + 2];
                } else {
                    hq = r % Hq; i = (r / Hq) % Nq; b = r / ((int64_t)Hq * Nq);
                }
                if (b < 0 || b >= B || i < 0 || i >= Nq || hq < 0 || hq >= Hq) {
                    bad = 1;
                    continue;
                }
                double *o = out + r * d;
                switch (dtype) {
                case ORACLE_F32:
                    attend_row(q, k, v, ORACLE_F32, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal,
                               scale, group, b, i, hq, s, qrow, acc, o, lse + r);
                    break;
                case ORACLE_F16:
                    attend_row(q, k, v, ORACLE_F16, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal,
                               scale, group, b, i, hq, s, qrow, acc, o, lse + r);
                    break;
                default:
                    attend_row(q, k, v, ORACLE_BF16, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal,
                               scale, group, b, i, hq, s, qrow, acc, o, lse + r);
                    break;
                }
            }
        }
        free(s);
        free(qrow);
        free(acc);
    }
    return bad ? -1 : 0;
}

/*
 * Merge of two partial attention results over disjoint key sets, row by row:
 * the definition of softmax over a union.  If (o_a, l_a) is attention over key
 * set A and (o_b, l_b) over B, then over A u B
 *   lse = log(exp(l_a) + exp(l_b))
 *   o   = exp(l_a - lse) o_a + exp(l_b - lse) o_b
 * (the log-sum-exp correction the Twinkle page uses to accumulate ring steps;
 * written here from the definition, not from that page's sigmoid form).
 * An empty set has lse = -inf and contributes nothing; both empty -> o = 0,
 * lse = -inf.  Arrays are [n_rows, d] and [n_rows]; result written to o_out,
 * l_out (may alias o_a, l_a).
 */
int oracle_merge_rows(const double *o_a, const double *l_a, const double *o_b,
                      const double *l_b, int64_t n_rows, int d, double *o_out,
                      double *l_out)
{
    if (!o_a || !l_a || !o_b || !l_b || !o_out || !l_out || d < 1 || n_rows < 0)
        return -1;
    for (int64_t r = 0; r < n_rows; ++r) {
        const double a = l_a[r], b = l_b[r];
        if (a == -INFINITY && b == -INFINITY) {
            for (int t = 0; t < d; ++t) o_out[r * d + t] = 0.0;
            l_out[r] = -INFINITY;
            continue;
        }
        const double m = a > b ? a : b;
        const double ea = exp(a - m), eb = exp(b - m);  /* exp(-inf) = 0 */
        const double z = ea + eb;
        for (int t = 0; t < d; ++t)
            o_out[r * d + t] = (ea * o_a[r * d + t] + eb * o_b[r * d + t]) / z;
        l_out[r] = m + log(z);
    }
    return 0;
}

/*
 * ---------------------------------------------------------------------------
 * Gradients of the definition above (backward pass).
 *
 * For a loss with upstream gradient dO = dL/dO, differentiating
 *   O_i = sum_j P_ij v_j,  P_ij = exp(s_ij - LSE_i),  s_ij = scale q_i . k_j
 * gives (chain rule through the softmax, whose Jacobian row is
 * P_ij (delta_jl - P_il)):
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   D_i   = dO_i . O_i              (= sum_j P_ij dP_ij)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale sum_j dS_ij k_j
 *   dK_j  = scale sum_i dS_ij q_i
 * with sums over visible pairs only (a masked pair has P = 0).  This is the
 * recomputation backward of the youngju.dev "Ring Attention" analysis
 * (ring_attention_backward: P recomputed from the saved LSE, D as the row sum
 * of dO * O, scale applied to dS) written from the derivative of the plain
 * definition.  With GQA a key/value head is shared by the query heads of its
 * group, so dK and dV sum over those heads (a reading: the pages show no GQA
 * backward).  A query row with no visible key has O = 0 and contributes
 * nothing.  Everything in double, per row, no blocking.
 *
 * dout has the storage dtype of q, k and v.
 * ---------------------------------------------------------------------------
 */

/* LSE_i and D_i = dO_i . O_i of one query row, O and LSE from attend_row. */
static inline __attribute__((always_inline)) void
bwd_stats_row(const void *q, const void *k, const void *v, const void *dout, const int dtype,
              int Hq, int Hkv, int64_t Nq, int64_t Nk, int d, const int64_t *q_pos,
              const int64_t *k_pos, int causal, double scale, int group, int64_t b, int64_t i,
              int64_t hq, double *s, double *qrow, double *acc, double *o, double *lse_r,
              double *delta_r)
{
    attend_row(q, k, v, dtype, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal, scale, group, b, i,
               hq, s, qrow, acc, o, lse_r);
    double dsum = 0.0;
    for (int t = 0; t < d; ++t)
        dsum += load(dout, ((b * Nq + i) * Hq + hq) * d + t, dtype) * o[t];
    *delta_r = dsum;
}

static int bwd_check(const void *q, const void *k, const void *v, const void *dout, int dtype,
                     int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int d,
                     const int64_t *q_pos, const int64_t *k_pos, int causal)
{
    return !q || !k || !v || !dout || B < 1 || Hq < 1 || Hkv < 1 || d < 1 || Nq < 0 ||
           Nk < 0 || Hq % Hkv != 0 || (causal && (!q_pos || !k_pos)) || dtype < ORACLE_F32 ||
           dtype > ORACLE_BF16;
}

/*
 * Per query row (b, i, hq): lse = LSE_i and delta = D_i.
 *   rows : n_rows triples (b, i, hq), or NULL for every row in (b, i, hq)
 *          row-major order (n_rows must then equal B*Nq*Hq)
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_bwd_stats(const void *q, const void *k, const void *v, const void *dout, int dtype,
                     int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int d,
                     const int64_t *q_pos, const int64_t *k_pos, int causal, double scale,
                     int64_t n_rows, const int64_t *rows, double *lse, double *delta,
                     int n_threads)
{
    if (bwd_check(q, k, v, dout, dtype, B, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal) ||
        !lse || !delta || (!rows && n_rows != (int64_t)B * Nq * Hq))
        return -1;
    const int group = Hq / Hkv;
    int bad = 0;
    build_luts();
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        if (!s || !qrow || !acc || !o) {
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t b, i, hq;
                if (rows) {
                    b = rows[3 * r]; i = rows[3 * r + 1]; hq = rows[3 * r + 2];
                } else {
                    hq = r % Hq; i = (r / Hq) % Nq; b = r / ((int64_t)Hq * Nq);
                }
                if (b < 0 || b >= B || i < 0 || i >= Nq || hq < 0 || hq >= Hq) {
                    bad = 1;
                    continue;
                }
                switch (dtype) {
                case ORACLE_F32:
                    bwd_stats_row(q, k, v, dout, ORACLE_F32, Hq, Hkv, Nq, Nk, d, q_pos, k_pos,
                                  causal, scale, group, b, i, hq, s, qrow, acc, o, lse + r,
                                  delta + r);
                    break;
                case ORACLE_F16:
                    bwd_stats_row(q, k, v, dout, ORACLE_F16, Hq, Hkv, Nq, Nk, d, q_pos, k_pos,
                                  causal, scale, group, b, i, hq, s, qrow, acc, o, lse + r,
                                  delta + r);
                    break;
                default:
                    bwd_stats_row(q, k, v, dout, ORACLE_BF16, Hq, Hkv, Nq, Nk, d, q_pos, k_pos,
                                  causal, scale, group, b, i, hq, s, qrow, acc, o, lse + r,
                                  delta + r);
                    break;
                }
            }
        }
        free(s);
        free(qrow);
        free(acc);
        free(o);
    }
    return bad ? -1 : 0;
}

/*
 * dQ rows.  lse_all, delta_all: [B, Nq, Hq] from oracle_bwd_stats (only the
 * entries of the requested rows are read).  rows as in oracle_bwd_stats;
 * dq: [n_rows, d].
 */
int oracle_bwd_dq(const void *q, const void *k, const void *v, const void *dout, int dtype,
                  int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int d,
                  const int64_t *q_pos, const int64_t *k_pos, int causal, double scale,
                  const double *lse_all, const double *delta_all, int64_t n_rows,
                  const int64_t *rows, double *dq, int n_threads)
{
    if (bwd_check(q, k, v, dout, dtype, B, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal) ||
        !lse_all || !delta_all || !dq || (!rows && n_rows != (int64_t)B * Nq * Hq))
        return -1;
    const int group = Hq / Hkv;
    int bad = 0;
    build_luts();
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *dorow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!qrow || !dorow) {
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t b, i, hq;
                if (rows) {
                    b = rows[3 * r]; i = rows[3 * r + 1]; hq = rows[3 * r + 2];
                } else {
                    hq = r % Hq; i = (r / Hq) % Nq; b = r / ((int64_t)Hq * Nq);
                }
                double *g_out = dq + r * d;
                for (int t = 0; t < d; ++t) g_out[t] = 0.0;
                if (b < 0 || b >= B || i < 0 || i >= Nq || hq < 0 || hq >= Hq) {
                    bad = 1;
                    continue;
                }
                const int64_t row = (b * Nq + i) * Hq + hq;
                const double L = lse_all[row], Dl = delta_all[row];
                if (L == -INFINITY) continue;   /* nothing visible: O = 0 */
                const int64_t g = hq / group;
                for (int t = 0; t < d; ++t) {
                    qrow[t] = load(q, row * d + t, dtype);
                    dorow[t] = load(dout, row * d + t, dtype);
                }
                for (int64_t j = 0; j < Nk; ++j) {
                    if (causal && k_pos[j] > q_pos[i]) continue;
                    const int64_t kb = ((b * Nk + j) * Hkv + g) * d;
                    double dot = 0.0, dp = 0.0;
                    for (int t = 0; t < d; ++t) {
                        dot += qrow[t] * load(k, kb + t, dtype);
                        dp += dorow[t] * load(v, kb + t, dtype);
                    }
                    const double P = exp(scale * dot - L);
                    const double dS = P * (dp - Dl);
                    for (int t = 0; t < d; ++t) g_out[t] += dS * load(k, kb + t, dtype);
                }
                for (int t = 0; t < d; ++t) g_out[t] *= scale;
            }
        }
        free(qrow);
        free(dorow);
    }
    return bad ? -1 : 0;
}

/*
 * dK and dV rows of key/value head rows (b, j, g): sums over the query heads
 * g*group .. g*group+group-1 and every query row that sees key j.
 *   rows : n_rows triples (b, j, g), or NULL for every row in (b, j, g)
 *          row-major order (n_rows must then equal B*Nk*Hkv)
 *   lse_all, delta_all: [B, Nq, Hq] (the rows of the group's heads are read)
 *   dk, dv: [n_rows, d]
 */
int oracle_bwd_dkv(const void *q, const void *k, const void *v, const void *dout, int dtype,
                   int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, int d,
                   const int64_t *q_pos, const int64_t *k_pos, int causal, double scale,
                   const double *lse_all, const double *delta_all, int64_t n_rows,
                   const int64_t *rows, double *dk, double *dv, int n_threads)
{
    if (bwd_check(q, k, v, dout, dtype, B, Hq, Hkv, Nq, Nk, d, q_pos, k_pos, causal) ||
        !lse_all || !delta_all || !dk || !dv || (!rows && n_rows != (int64_t)B * Nk * Hkv))
        return -1;
    const int group = Hq / Hkv;
    int bad = 0;
    build_luts();
#ifdef _OPENMP
    if (n_threads > 0)
        omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
#pragma omp parallel reduction(| : bad)
    {
        double *krow = (double *)malloc(sizeof(double) * (size_t)d);
        double *vrow = (double *)malloc(sizeof(double) * (size_t)d);
        if (!krow || !vrow) {
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t b, j, g;
                if (rows) {
                    b = rows[3 * r]; j = rows[3 * r + 1]; g = rows[3 * r + 2];
                } else {
                    g = r % Hkv; j = (r / Hkv) % Nk; b = r / ((int64_t)Hkv * Nk);
                }
                double *gk = dk + r * d, *gv = dv + r * d;
                for (int t = 0; t < d; ++t) gk[t] = gv[t] = 0.0;
                if (b < 0 || b >= B || j < 0 || j >= Nk || g < 0 || g >= Hkv) {
                    bad = 1;
                    continue;
                }
                const int64_t kb = ((b * Nk + j) * Hkv + g) * d;
                for (int t = 0; t < d; ++t) {
                    krow[t] = load(k, kb + t, dtype);
                    vrow[t] = load(v, kb + t, dtype);
                }
                for (int64_t hq = g * group; hq < (g + 1) * group; ++hq) {
                    for (int64_t i = 0; i < Nq; ++i) {
                        if (causal && k_pos[j] > q_pos[i]) continue;
                        const int64_t row = (b * Nq + i) * Hq + hq;
                        const double L = lse_all[row], Dl = delta_all[row];
                        if (L == -INFINITY) continue;
                        double dot = 0.0, dp = 0.0;
                        for (int t = 0; t < d; ++t) {
                            dot += load(q, row * d + t, dtype) * krow[t];
                            dp += load(dout, row * d + t, dtype) * vrow[t];
                        }
                        const double P = exp(scale * dot - L);
                        const double dS = P * (dp - Dl);
                        for (int t = 0; t < d; ++t) {
                            gk[t] += dS * load(q, row * d + t, dtype);
                            gv[t] += P * load(dout, row * d + t, dtype);
                        }
                    }
                }
                for (int t = 0; t < d; ++t) gk[t] *= scale;
            }
        }
        free(krow);
        free(vrow);
    }
    return bad ? -1 : 0;
}
