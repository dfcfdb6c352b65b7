/*
 * kda_oracle.c -- fp64 CPU oracle for the chunked forward of Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  The GPU library never includes, links or
 * calls anything from this directory, and this file shares no code with it.
 *
 * What it computes (the plain token recurrence the chunked method reaches exactly):
 *   For every sequence b and value head h, with query/key head hq = h / (n_v / n_qk):
 *     S  = initial_state[b, h]            (a d_v x d_k matrix; rows are value channels)
 *     for each token t of the sequence:
 *       S[:, j] *= exp(g[t, j])           per-channel decay of the key columns
 *       r  = v_t - S k_t                  delta-rule residual
 *       S += beta_t * r k_t^T             rank-1 write
 *       o_t = scale * S q_t               read after the write
 *     final_state[b, h] = S
 *   Optionally q and k rows are L2-normalised first (x / sqrt(sum x^2 + 1e-6)) and beta is
 *   the logistic sigmoid of the stored value.
 *   With ORACLE_SCALAR_GATE, g holds one value per (token, value head), laid out like beta,
 *   and exp(g_t) decays every key column alike: the scalar-gate (GDN) form of the same rule.
 *   oracle_kda_fwd_raw_gate takes the raw bf16 gate instead and activates it per (token, key
 *   channel j) of value head h as
 *       g = lower_bound * sigmoid(exp(A_log[h]) * (g_raw + dt_bias[h, j]))
 *   (a reading, see below), then runs the same recurrence.
 *
 * Sources (the pages this follows):
 *   - vLLM PR #43195 summary "KDA chunk prefill decay uses exp2", section 功能与动机: the
 *     recurrence decays the state with a natural-base exp(g) (state *= exp(g)).
 *   - FlashKDA README (CANNBot-DSL sample, Ascend 950), section 功能说明: gamma_t is the exp of
 *     the running sum of g, the chunk matrices use gamma*K for the written key and gamma^-1*K for
 *     the read key, which fixes decay-then-write and read-after-write; q/k row L2 normalise and
 *     beta sigmoid are fused options; section 参数说明: the state's last two axes are (Dv, Dk);
 *     the three layouts BNSD / BSND / TND and the cu_seqlens prefix sum (sections 参数说明 and
 *     约束说明).
 *   - vLLM PR #42076 summary (GDN KKT kernel precision on Hopper), sections 实现拆解 and 关键源码片段,
 *     and vLLM PR #45000 summary (GDN KKT compile time on RDNA), 关键源码片段: the GDN kernel
 *     forms the product of beta-scaled keys with the raw keys and applies the gate g only
 *     afterwards, which a gate shared by all key channels of a token allows.
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *   - L2-norm epsilon 1e-6 inside the square root.
 *   - GQA: value head h reads query/key head h / (n_v / n_qk) (contiguous groups).
 *   - BNSD/BSND with cu_seqlens: batch row b holds cu[b+1]-cu[b] valid tokens at its start;
 *     out rows past that length are left untouched by this oracle.
 *   - initial_state == NULL means a zero state; final_state == NULL means it is not returned.
 *   - Scalar gate: one fp32 value per (token, value head), the natural-log decay of every key
 *     channel of that token (the GDN pages show the gate applied after the key product, which
 *     only a channel-independent gate permits).
 *   - Raw-gate activation.  The FlashKDA README (sections 参数说明, 快速开始, 约束说明) takes
 *     a raw bf16 gate shaped like v, A_log [Nv] (a per-value-head log time scale), dt_bias
 *     [Nv, D] (a gate bias) and lower_bound in [-5, 0] (the gate's lower bound), and prints no
 *     formula.  Read here as: bias the raw gate, scale it by the head's time scale
 *     exp(A_log), squash it with the logistic sigmoid and scale by lower_bound, so every
 *     activated gate lies in [lower_bound, 0] -- the form of the 8K-prefill workload's own
 *     gate, -5 * sigmoid(N(0,1)).  The pins check this function's arithmetic (sigmoid(0) = 1/2,
 *     saturation at lower_bound, the exp(A_log) scale per value head, the dt_bias index, the
 *     range); whether it is FlashKDA's own formula cannot be checked from the pages.
 *
 * Parity pins for this function live in the CPU test suite: a hand-worked two-token example,
 * an independent brute-force evaluation of the chunk equations, and closed-form invariants.
 * Compile-time planted mistakes (KDA_ORACLE_MUTANT) let the tests show that every pin set
 * catches a wrong oracle; the default build defines none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef KDA_ORACLE_MUTANT
#define KDA_ORACLE_MUTANT 0
#endif

enum { ORACLE_BNSD = 0, ORACLE_BSND = 1, ORACLE_TND = 2 };
enum { ORACLE_QK_L2NORM = 1u, ORACLE_BETA_SIGMOID = 2u, ORACLE_SCALAR_GATE = 4u };

static double bf16_bits_to_double(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Element offset of (sequence b, token t, head h, channel 0) for a [.., D] tensor. */
static size_t row_offset(int layout, int b, int t, int h, int n_heads, int seq_len,
                         const int32_t *cu, int d) {
    switch (layout) {
    case ORACLE_BNSD: return (((size_t)b * n_heads + h) * seq_len + t) * (size_t)d;
    case ORACLE_BSND: return (((size_t)b * seq_len + t) * n_heads + h) * (size_t)d;
    default:          return (((size_t)cu[b] + t) * n_heads + h) * (size_t)d;
    }
}

/* Offset of beta(sequence b, token t, head h) for a [..] tensor with no channel axis. */
static size_t beta_offset(int layout, int b, int t, int h, int n_heads, int seq_len,
                          const int32_t *cu) {
    switch (layout) {
    case ORACLE_BNSD: return ((size_t)b * n_heads + h) * seq_len + t;
    case ORACLE_BSND: return ((size_t)b * seq_len + t) * n_heads + h;
    default:          return ((size_t)cu[b] + t) * n_heads + h;
    }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int oracle_mutant_id(void) { return KDA_ORACLE_MUTANT; }

/*
 * Returns 0 on success, a negative number on invalid arguments.
 * out:          doubles in v's shape and layout; only value channels dv in [dv_lo, dv_hi) of
 *               valid rows are written.
 * final_state:  doubles [batch, n_v, d_v, d_k] (NULL: not written); only rows [dv_lo, dv_hi).
 * initial_state: fp32 [batch, n_v, d_v, d_k] or NULL.
 * cu_seqlens:   int32 [batch + 1]; required for TND, optional (valid lengths) otherwise.
 * Work is split over (sequence, value head, block of 16 state rows), the independent chains
 * of the recurrence: every state row evolves on its own given q, k, g and beta.
 */
/* The raw gate and its activation parameters (oracle_kda_fwd_raw_gate). */
typedef struct {
    const uint16_t *raw;      /* bf16 bits, v's shape and layout */
    const float *a_log;       /* [n_v] */
    const float *dt_bias;     /* [n_v, d_k] */
    double lower_bound;
} raw_gate;

/* Activated gate of key channel j of value head h: lower_bound * sigmoid(exp(A_log[h]) *
 * (g_raw + dt_bias[h, j])), in fp64. */
static double activate_gate(const raw_gate *rg, size_t og, int h, int j, int d_k) {
    const double x0 = bf16_bits_to_double(rg->raw[og + (size_t)j]) +
                      (double)rg->dt_bias[(size_t)h * d_k + j];
#if KDA_ORACLE_MUTANT == 14
    const double x = (double)rg->a_log[h] * x0;        /* planted: time scale not exponentiated */
#else
    const double x = exp((double)rg->a_log[h]) * x0;
#endif
#if KDA_ORACLE_MUTANT == 15
    return rg->lower_bound / (1.0 + exp(x));           /* planted: sigmoid of -x */
#else
    return rg->lower_bound / (1.0 + exp(-x));
#endif
}

static int kda_fwd_core(int layout, int batch, int seq_len, int n_qk, int n_v, int d_k, int d_v,
                        double scale, unsigned flags,
                        const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                        const raw_gate *rg,
                        const uint16_t *beta, const float *initial_state, const int32_t *cu_seqlens,
                        int dv_lo, int dv_hi, double *out, double *final_state) {
    if (layout < ORACLE_BNSD || layout > ORACLE_TND) return -1;
    if (batch < 1 || n_qk < 1 || n_v < n_qk || n_v % n_qk != 0 || d_k < 1 || d_v < 1) return -2;
    if (layout == ORACLE_TND && cu_seqlens == NULL) return -3;
    if (layout != ORACLE_TND && seq_len < 1) return -4;
    if (dv_lo < 0 || dv_hi > d_v || dv_lo >= dv_hi) return -5;
    if (!q || !k || !v || (!g && !rg) || !beta || !out) return -6;
    if (rg && (!rg->raw || !rg->a_log || !rg->dt_bias || (flags & ORACLE_SCALAR_GATE))) return -7;

    const int group = n_v / n_qk;
    const int scalar_gate = (flags & ORACLE_SCALAR_GATE) != 0;
    (void)group;
    (void)scale;
    const int rows_per_chain = 16;
    const int n_blocks = (dv_hi - dv_lo + rows_per_chain - 1) / rows_per_chain;
    const long n_chains = (long)batch * n_v * n_blocks;

    #pragma omp parallel
    {
        double *S  = (double *)malloc(sizeof(double) * (size_t)rows_per_chain * d_k);
        double *qh = (double *)malloc(sizeof(double) * (size_t)d_k);
        double *kh = (double *)malloc(sizeof(double) * (size_t)d_k);
        double *dec = (double *)malloc(sizeof(double) * (size_t)d_k);

        #pragma omp for schedule(dynamic, 1)
        for (long chain = 0; chain < n_chains; ++chain) {
            const int blk = (int)(chain % n_blocks);
            const int h = (int)((chain / n_blocks) % n_v);
            const int b = (int)(chain / ((long)n_blocks * n_v));
#if KDA_ORACLE_MUTANT == 5
            const int hq = h % n_qk;                    /* planted: wrong GQA head map */
#else
            const int hq = h / group;
#endif
            const int r0 = dv_lo + blk * rows_per_chain;
            const int r1 = (r0 + rows_per_chain < dv_hi) ? r0 + rows_per_chain : dv_hi;
            const int nr = r1 - r0;
            int len;
            if (layout == ORACLE_TND || cu_seqlens) len = cu_seqlens[b + 1] - cu_seqlens[b];
            else len = seq_len;

            /* S rows r0..r1-1 of the [d_v, d_k] state */
            for (int i = 0; i < nr; ++i)
                for (int j = 0; j < d_k; ++j) {
                    double s0 = 0.0;
                    if (initial_state) {
                        const size_t base = ((size_t)b * n_v + h) * (size_t)d_v * d_k;
#if KDA_ORACLE_MUTANT == 9
                        /* planted: state read transposed, as [d_k, d_v] */
                        s0 = (j < d_v && (r0 + i) < d_k)
                                 ? initial_state[base + (size_t)j * d_v + (r0 + i)] : 0.0;
#else
                        s0 = initial_state[base + (size_t)(r0 + i) * d_k + j];
#endif
                    }
                    S[(size_t)i * d_k + j] = s0;
                }

            for (int t = 0; t < len; ++t) {
                const size_t oq = row_offset(layout, b, t, hq, n_qk, seq_len, cu_seqlens, d_k);
                const size_t ov = row_offset(layout, b, t, h, n_v, seq_len, cu_seqlens, d_v);
                const size_t og = row_offset(layout, b, t, h, n_v, seq_len, cu_seqlens, d_k);
                const size_t ob = beta_offset(layout, b, t, h, n_v, seq_len, cu_seqlens);

                for (int j = 0; j < d_k; ++j) {
                    qh[j] = bf16_bits_to_double(q[oq + j]);
                    kh[j] = bf16_bits_to_double(k[oq + j]);
                }
#if KDA_ORACLE_MUTANT != 8
                if (flags & ORACLE_QK_L2NORM) {
                    double sq = 0.0, sk = 0.0;
                    for (int j = 0; j < d_k; ++j) { sq += qh[j] * qh[j]; sk += kh[j] * kh[j]; }
                    const double iq = 1.0 / sqrt(sq + 1e-6), ik = 1.0 / sqrt(sk + 1e-6);
                    for (int j = 0; j < d_k; ++j) { qh[j] *= iq; kh[j] *= ik; }
                }
#endif
                double bt = bf16_bits_to_double(beta[ob]);
#if KDA_ORACLE_MUTANT != 7
                if (flags & ORACLE_BETA_SIGMOID) bt = 1.0 / (1.0 + exp(-bt));
#endif
                for (int j = 0; j < d_k; ++j) {
                    /* gate of channel j: its own value, or the token's one value (scalar gate) */
#if KDA_ORACLE_MUTANT == 13
                    /* planted: scalar gate of the query/key head instead of the value head */
                    const size_t gi = scalar_gate
                        ? beta_offset(layout, b, t, hq, n_v, seq_len, cu_seqlens) : og + (size_t)j;
#else
                    const size_t gi = scalar_gate ? ob : og + (size_t)j;
#endif
                    if (rg) {   /* raw gate: activated here */
                        dec[j] = exp(activate_gate(rg, og, h, j, d_k));
                        continue;
                    }
#if KDA_ORACLE_MUTANT == 11
                    /* planted: gate taken from the previous token */
                    size_t gip = gi;
                    if (t > 0)
                        gip = scalar_gate ? beta_offset(layout, b, t - 1, h, n_v, seq_len, cu_seqlens)
                                          : row_offset(layout, b, t - 1, h, n_v, seq_len,
                                                       cu_seqlens, d_k) + (size_t)j;
                    dec[j] = (t > 0) ? exp((double)g[gip]) : 1.0;
#elif KDA_ORACLE_MUTANT == 12
                    dec[j] = exp2((double)g[gi]);  /* planted: wrong base */
#else
                    dec[j] = exp((double)g[gi]);
#endif
                }

                for (int i = 0; i < nr; ++i) {
                    double *Si = S + (size_t)i * d_k;
                    const int dv = r0 + i;
#if KDA_ORACLE_MUTANT == 3
                    /* planted: decay the value rows instead of the key columns */
                    const double drow = (dv >= d_k) ? 1.0
                                        : rg ? exp(activate_gate(rg, og, h, dv, d_k))
                                             : exp((double)g[scalar_gate ? ob : og + dv]);
                    for (int j = 0; j < d_k; ++j) Si[j] *= drow;
#elif KDA_ORACLE_MUTANT == 1
                    /* planted: decay applied after the write (below) */
#else
                    for (int j = 0; j < d_k; ++j) Si[j] *= dec[j];
#endif
#if KDA_ORACLE_MUTANT == 2
                    double o_before = 0.0;      /* planted: read before the write */
                    for (int j = 0; j < d_k; ++j) o_before += Si[j] * qh[j];
#endif
                    double sk = 0.0;
                    for (int j = 0; j < d_k; ++j) sk += Si[j] * kh[j];
                    const double vi = bf16_bits_to_double(v[ov + dv]);
#if KDA_ORACLE_MUTANT == 4
                    const double coef = bt * (vi + sk);          /* planted: sign */
#elif KDA_ORACLE_MUTANT == 10
                    const double coef = bt * vi - sk;             /* planted: beta on v only */
#else
                    const double coef = bt * (vi - sk);
#endif
                    for (int j = 0; j < d_k; ++j) Si[j] += coef * kh[j];
#if KDA_ORACLE_MUTANT == 1
                    for (int j = 0; j < d_k; ++j) Si[j] *= dec[j];
#endif
                    double o = 0.0;
                    for (int j = 0; j < d_k; ++j) o += Si[j] * qh[j];
#if KDA_ORACLE_MUTANT == 2
                    o = o_before;
#endif
#if KDA_ORACLE_MUTANT == 6
                    out[ov + dv] = o;                             /* planted: no scale */
#else
                    out[ov + dv] = scale * o;
#endif
                }
            }

            if (final_state) {
                const size_t base = ((size_t)b * n_v + h) * (size_t)d_v * d_k;
                for (int i = 0; i < nr; ++i)
                    memcpy(final_state + base + (size_t)(r0 + i) * d_k, S + (size_t)i * d_k,
                           sizeof(double) * (size_t)d_k);
            }
        }
        free(S);
        free(qh);
        free(kh);
        free(dec);
    }
    return 0;
}

int oracle_kda_fwd(int layout, int batch, int seq_len, int n_qk, int n_v, int d_k, int d_v,
                   double scale, unsigned flags,
                   const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                   const uint16_t *beta, const float *initial_state, const int32_t *cu_seqlens,
                   int dv_lo, int dv_hi, double *out, double *final_state) {
    return kda_fwd_core(layout, batch, seq_len, n_qk, n_v, d_k, d_v, scale, flags, q, k, v, g,
                        NULL, beta, initial_state, cu_seqlens, dv_lo, dv_hi, out, final_state);
}

/* The same with the raw bf16 gate g_raw (v's shape) activated per token and key channel (see
 * the top of this file); scalar gate not allowed (returns -7). */
int oracle_kda_fwd_raw_gate(int layout, int batch, int seq_len, int n_qk, int n_v, int d_k,
                            int d_v, double scale, unsigned flags,
                            const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const uint16_t *g_raw, const float *a_log, const float *dt_bias,
                            double lower_bound, const uint16_t *beta, const float *initial_state,
                            const int32_t *cu_seqlens, int dv_lo, int dv_hi, double *out,
                            double *final_state) {
    const raw_gate rg = {g_raw, a_log, dt_bias, lower_bound};
    return kda_fwd_core(layout, batch, seq_len, n_qk, n_v, d_k, d_v, scale, flags, q, k, v, NULL,
                        &rg, beta, initial_state, cu_seqlens, dv_lo, dv_hi, out, final_state);
}
