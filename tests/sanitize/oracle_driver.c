/* The fp64 oracle driven over small inputs of every layout and option, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (every buffer is allocated at its exact size,
 * so a read or write past one is reported).  Exits non-zero on a wrong return code or a
 * non-finite result. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_kda_fwd(int layout, int batch, int seq_len, int n_qk, int n_v, int d_k, int d_v,
                   double scale, unsigned flags, const uint16_t *q, const uint16_t *k,
                   const uint16_t *v, const float *g, const uint16_t *beta,
                   const float *initial_state, const int32_t *cu_seqlens, int dv_lo, int dv_hi,
                   double *out, double *final_state);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng >> 8; }
static float unif(void) { return (float)(next() & 0xffff) / 65536.0f; }   /* [0, 1) */
static uint16_t bf16_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return (uint16_t)(u >> 16); }

static int fails = 0;

static void run(int layout, int batch, int seq_len, int n_qk, int n_v, int d, unsigned flags,
                int with_init, const int32_t *lengths, int dv_lo, int dv_hi) {
    int32_t *cu = NULL;
    long tokens = (long)batch * seq_len;
    if (lengths) {
        cu = malloc(sizeof(int32_t) * (size_t)(batch + 1));
        cu[0] = 0;
        for (int b = 0; b < batch; ++b) cu[b + 1] = cu[b] + lengths[b];
        if (layout == 2) { tokens = cu[batch]; seq_len = cu[batch]; }
    }
    const int sg = (flags & 4u) != 0;
    const size_t nq = (size_t)tokens * n_qk * d, nv = (size_t)tokens * n_v * d;
    const size_t nb = (size_t)tokens * n_v, ns = (size_t)batch * n_v * d * d;
    uint16_t *q = malloc(nq * 2), *k = malloc(nq * 2), *v = malloc(nv * 2), *be = malloc(nb * 2);
    float *g = malloc((sg ? nb : nv) * 4), *init = with_init ? malloc(ns * 4) : NULL;
    double *out = malloc(nv * 8), *fin = malloc(ns * 8);
    for (size_t i = 0; i < nq; ++i) { q[i] = bf16_bits(unif() - 0.5f); k[i] = bf16_bits(unif() - 0.5f); }
    for (size_t i = 0; i < nv; ++i) v[i] = bf16_bits(2.0f * unif() - 1.0f);
    for (size_t i = 0; i < (sg ? nb : nv); ++i) g[i] = -5.0f * unif();
    for (size_t i = 0; i < nb; ++i) be[i] = bf16_bits(unif());
    if (init) for (size_t i = 0; i < ns; ++i) init[i] = 0.1f * (unif() - 0.5f);
    for (size_t i = 0; i < nv; ++i) out[i] = 0.0;
    const int rc = oracle_kda_fwd(layout, batch, seq_len, n_qk, n_v, d, d, 0.125, flags, q, k, v,
                                  g, be, init, cu, dv_lo, dv_hi, out, fin);
    if (rc != 0) { printf("FAIL rc %d (layout %d)\n", rc, layout); ++fails; }
    for (size_t i = 0; i < nv; ++i)
        if (!isfinite(out[i])) { printf("FAIL non-finite out\n"); ++fails; break; }
    free(q); free(k); free(v); free(be); free(g); free(init); free(out); free(fin); free(cu);
}

int main(void) {
    const int32_t lens[3] = {5, 1, 70};
    for (unsigned flags = 0; flags < 8; ++flags) {
        run(0, 2, 37, 1, 2, 16, flags, 1, NULL, 0, 16);
        run(1, 2, 37, 2, 4, 16, flags, 0, NULL, 3, 11);
        run(2, 3, 0, 1, 3, 8, flags, 1, lens, 0, 8);
        run(0, 3, 70, 1, 1, 8, flags, 1, lens, 0, 8);   /* valid lengths with BNSD */
    }
    /* argument checks return errors without touching the buffers */
    uint16_t x = 0; float f = 0.f; double o = 0.0;
    if (oracle_kda_fwd(5, 1, 1, 1, 1, 4, 4, 1.0, 0u, &x, &x, &x, &f, &x, NULL, NULL, 0, 4, &o, NULL) >= 0) ++fails;
    if (oracle_kda_fwd(0, 1, 1, 2, 3, 4, 4, 1.0, 0u, &x, &x, &x, &f, &x, NULL, NULL, 0, 4, &o, NULL) >= 0) ++fails;
    if (oracle_kda_fwd(2, 1, 1, 1, 1, 4, 4, 1.0, 0u, &x, &x, &x, &f, &x, NULL, NULL, 0, 4, &o, NULL) >= 0) ++fails;
    if (oracle_kda_fwd(0, 1, 1, 1, 1, 4, 4, 1.0, 0u, &x, &x, &x, &f, &x, NULL, NULL, 2, 9, &o, NULL) >= 0) ++fails;
    printf("oracle sanitizer runs done, failures %d\n", fails);
    return fails == 0 ? 0 : 1;
}
