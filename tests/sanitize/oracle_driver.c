/*
 * oracle_driver.c -- runs the CPU oracle's entry points on small seeded
 * problems, for the AddressSanitizer / UndefinedBehaviorSanitizer build of
 * oracle/da2_oracle.c that tests/test_sanitizers.py makes and runs.  Any
 * sanitizer report ends the program with a nonzero status; a wrong return
 * code does too.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int or_regions(int F, int Hv, int Wv, int C);
int or_layout(int F, int Hv, int Wv, int C, int32_t *perm);
int or_partition_c(int Hv, int Wv, int C, int32_t *tok, int32_t *nvalid);
int or_plan(int B, int H, int F, int Hv, int Wv, int C, int d, const uint16_t *q, const uint16_t *k, int32_t full_bp,
            int32_t hi_bp, int32_t lo_bp, double lambda, int scope, int skip_means, uint32_t *keys, uint8_t *tier,
            double *qavg, double *kavg, float *qmx, float *kmx);
int or_attention(int B, int H, int F, int Hv, int Wv, int C, int d, const uint16_t *q, const uint16_t *k,
                 const uint16_t *v, const uint8_t *tier, int nqb, const int32_t *qblocks, double *out, double *amb);
int or_attention_pfx(int B, int H, int F, int Hv, int Wv, int C, int d, const uint16_t *q, const uint16_t *k,
                     const uint16_t *v, int Lp, const uint16_t *qp, const uint16_t *kp, const uint16_t *vp,
                     const int32_t *valid, int pt, const uint8_t *tier, int nqb, const int32_t *qblocks, int nprow,
                     const int32_t *prows, double *out, double *outp, double *amb);
int64_t or_attention_trace(int F, int Hv, int Wv, int C, int d, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           const uint8_t *tier, int u, int64_t cap, int32_t *key, int32_t *tr_tier, double *s,
                           double *w, double *wq, double *m, double *Z, double *out);
int or_dense(int B, int H, int N, int d, const uint16_t *q, const uint16_t *k, const uint16_t *v, int nrows,
             const int32_t *rows, double *out);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static double uniform(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) * 0x1p-53;
}

static uint16_t to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

static uint16_t *random_bf16(size_t n, float scale)
{
    uint16_t *p = malloc(sizeof(uint16_t) * (n ? n : 1));
    for (size_t i = 0; i < n; i++)
        p[i] = to_bf16((float)((uniform() * 2.0 - 1.0) * scale));
    return p;
}

#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            exit(2);                                                  \
        }                                                             \
    } while (0)

static void problem(int B, int H, int F, int Hv, int Wv, int C, int d)
{
    int N = F * Hv * Wv, R = or_regions(F, Hv, Wv, C), T = R * (C / 64);
    CHECK(R > 0);
    size_t n = (size_t)B * H * N * d, rr = (size_t)B * H * R * R;
    uint16_t *q = random_bf16(n, 2.0f), *k = random_bf16(n, 2.0f), *v = random_bf16(n, 1.0f);
    uint32_t *keys = malloc(sizeof(uint32_t) * rr);
    uint8_t *tier = malloc(rr);
    double *qa = malloc(sizeof(double) * B * H * R * d), *ka = malloc(sizeof(double) * B * H * R * d);
    float *qm = malloc(sizeof(float) * B * H * R * d), *km = malloc(sizeof(float) * B * H * R * d);
    const int means = C == 64;   /* block-mean tiles exist at C = 64 only */
    CHECK(or_plan(B, H, F, Hv, Wv, C, d, q, k, 1000, 2000, 3000, 0.2, 0, means, keys, tier, qa, ka, qm, km) == 0);
    /* every tier value, skips included */
    static const uint8_t tiers[6] = {0, 1, 4, 8, 16, 32};
    for (size_t i = 0; i < rr; i += 3) {
        tier[i] = tiers[(int)(uniform() * 6) % 6];
        if (!means && tier[i] == 1)
            tier[i] = 0;
    }
    double *out = malloc(sizeof(double) * (size_t)B * H * T * 64 * d);
    double *amb = malloc(sizeof(double) * (size_t)B * H * T * 64 * d);
    CHECK(or_attention(B, H, F, Hv, Wv, C, d, q, k, v, tier, T, NULL, out, amb) == 0);
    for (size_t i = 0; i < (size_t)B * H * T * 64 * d; i++)
        CHECK(isfinite(out[i]) && amb[i] >= 0.0);
    /* a text prefix, one batch element with fewer valid keys */
    int Lp = 70;
    size_t np = (size_t)B * H * Lp * d;
    uint16_t *qp = random_bf16(np, 2.0f), *kp = random_bf16(np, 2.0f), *vp = random_bf16(np, 1.0f);
    int32_t *valid = malloc(sizeof(int32_t) * B);
    for (int b = 0; b < B; b++)
        valid[b] = b ? 33 : Lp;
    int32_t prows[3] = {0, 32, Lp - 1}, qb[2] = {0, T - 1};
    double *outp = malloc(sizeof(double) * (size_t)B * H * 3 * d);
    double *out2 = malloc(sizeof(double) * (size_t)B * H * 2 * 64 * d);
    double *amb2 = malloc(sizeof(double) * (size_t)B * H * 2 * 64 * d);
    for (size_t i = 0; i < rr; i++)
        if (tier[i] == 32) tier[i] = 16;
    CHECK(or_attention_pfx(B, H, F, Hv, Wv, C, d, q, k, v, Lp, qp, kp, vp, valid, 16, tier, 2, qb, 3, prows, out2,
                           outp, amb2) == 0);
    /* one traced row, the dense reference */
    int64_t cap = (int64_t)T * 64;
    int32_t *key = malloc(sizeof(int32_t) * cap), *tt = malloc(sizeof(int32_t) * cap);
    double *s = malloc(sizeof(double) * cap), *w = malloc(sizeof(double) * cap);
    double *wq = malloc(sizeof(double) * cap), *m = malloc(sizeof(double) * cap);
    double Z, orow[128];
    CHECK(or_attention_trace(F, Hv, Wv, C, d, q, k, v, tier, 5, cap, key, tt, s, w, wq, m, &Z, orow) >= 0);
    int32_t rows[3] = {0, N / 2, N - 1};
    double *dn = malloc(sizeof(double) * (size_t)B * H * 3 * d);
    CHECK(or_dense(B, H, N, d, q, k, v, 3, rows, dn) == 0);
    free(q); free(k); free(v); free(keys); free(tier); free(qa); free(ka); free(qm); free(km);
    free(out); free(amb); free(qp); free(kp); free(vp); free(valid); free(outp); free(out2); free(amb2);
    free(key); free(tt); free(s); free(w); free(wq); free(m); free(dn);
}

int main(void)
{
    /* partitions of every frame up to 40 x 40 (those with one) */
    for (int Hv = 1; Hv <= 40; Hv++)
        for (int Wv = 1; Wv <= 40; Wv++) {
            int Rf = (Hv * Wv + 63) / 64;
            int32_t *tok = malloc(sizeof(int32_t) * Rf * 64), *nv = malloc(sizeof(int32_t) * Rf);
            int got = or_partition_c(Hv, Wv, 64, tok, nv);
            if (got >= 0) {
                CHECK(got == Rf);
                int32_t *perm = malloc(sizeof(int32_t) * 2 * Rf * 64);
                CHECK(or_layout(2, Hv, Wv, 64, perm) == 0);
                free(perm);
            }
            free(tok);
            free(nv);
        }
    problem(1, 2, 2, 16, 16, 64, 64);    /* the 8x8 grid */
    problem(2, 1, 2, 12, 20, 64, 64);    /* a ragged partition */
    problem(1, 1, 1, 17, 31, 64, 128);
    problem(1, 2, 2, 16, 24, 128, 64);   /* block capacity 128 */
    problem(1, 1, 1, 9, 10, 128, 128);   /* one region of 90 tokens: a part-empty second tile */
    printf("oracle driver ok\n");
    return 0;
}
