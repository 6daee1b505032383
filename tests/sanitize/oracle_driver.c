/*
 * Sanitizer driver for the fp64 oracle (test infrastructure): calls every
 * oracle function on small seeded inputs, well-formed and malformed, so an
 * AddressSanitizer / UndefinedBehaviorSanitizer build of spec_oracle.c can
 * report any out-of-bounds access, leak of undefined values into indexing,
 * or undefined arithmetic.  Exit status 0 when every call returned.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* splitmix64: a seeded stream of 64-bit words */
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double unif(void) { return (double)(next_u64() >> 11) * 0x1.0p-53; }

/* approximately normal: sum of 12 uniforms, centred */
static float gauss(void)
{
    double s = 0.0;
    for (int i = 0; i < 12; ++i)
        s += unif();
    return (float)(s - 6.0);
}

static uint16_t to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

/* logits [n] of either dtype, scale * N(0,1), some -inf */
static void *logits(int dt, size_t n, float scale, int with_minus_inf)
{
    void *p = malloc(n * (dt == ORACLE_BF16 ? 2 : 4));
    for (size_t i = 0; i < n; ++i) {
        float v = scale * gauss();
        if (with_minus_inf && (next_u64() % 7) == 0)
            v = -INFINITY;
        if (dt == ORACLE_BF16)
            ((uint16_t *)p)[i] = to_bf16(v);
        else
            ((float *)p)[i] = v;
    }
    return p;
}

static void run_chain(int dt, int B, int K, int V, int malformed)
{
    const int L = K + 1;
    void *T = logits(dt, (size_t)B * L * V, 3.0f, malformed);
    void *D = logits(dt, (size_t)B * K * V, 3.0f, 0);
    int32_t *x = malloc(sizeof(int32_t) * (size_t)B * K);
    float *u = malloc(sizeof(float) * (size_t)B * L);
    for (int i = 0; i < B * K; ++i)
        x[i] = (int32_t)(next_u64() % (uint64_t)V);
    for (int i = 0; i < B * L; ++i)
        u[i] = (float)unif();
    if (malformed) {
        x[0] = -1;
        if (B * K > 1)
            x[1] = V;
        if (B * K > 2)
            x[2] = INT32_MAX;
    }
    int32_t *tok = malloc(sizeof(int32_t) * (size_t)B * L), *len = malloc(sizeof(int32_t) * B);
    int32_t *st = malloc(sizeof(int32_t) * B), *fl = malloc(sizeof(int32_t) * B);
    int32_t *dec = malloc(sizeof(int32_t) * B);
    double *tlp = malloc(sizeof(double) * (size_t)B * L), *blp = malloc(sizeof(double) * (size_t)B * L);
    oracle_greedy(T, dt, x, B, K, V, tok, len, tlp, blp, st, dec);
    oracle_exact(T, D, dt, x, u, B, K, V, 1e-6, 1e-11, tok, len, tlp, blp, st, fl, dec);
    oracle_relaxed(T, dt, x, u, B, K, V, 0.1, 4, 1e-6, 1e-11, tok, len, tlp, blp, st, fl, dec);
    oracle_power(T, D, dt, x, u, B, K, V, 0.5, 1e-6, 1e-11, tok, len, tlp, blp, st, fl, dec);
    oracle_power(T, D, dt, x, u, B, K, V, 0.0, 1e-6, 1e-11, tok, len, tlp, blp, st, fl, dec);
    double *M = malloc(sizeof(double) * (size_t)B * L), *S = malloc(sizeof(double) * (size_t)B * L);
    int64_t *g = malloc(sizeof(int64_t) * (size_t)B * L);
    oracle_row_stats(T, dt, (long)B * L, V, M, g, S);
    int32_t *ys = malloc(sizeof(int32_t) * (size_t)B * K), *fs = malloc(sizeof(int32_t) * (size_t)B * K);
    double *lq = malloc(sizeof(double) * (size_t)B * K);
    oracle_sample(D, dt, u, (long)B * K, V, 1e-11, ys, lq, fs);
    int32_t *n = malloc(sizeof(int32_t) * B), *res = malloc(sizeof(int32_t) * B);
    double *w = malloc(sizeof(double) * (size_t)B * V), *Z = malloc(sizeof(double) * B);
    for (int b = 0; b < B; ++b)
        n[b] = (int32_t)(next_u64() % (uint64_t)L);
    oracle_terminal_weights(0, T, D, dt, n, B, K, V, w, Z, res);
    oracle_terminal_weights(1, T, NULL, dt, n, B, K, V, w, Z, res);
    oracle_terminal_weights(2, D, NULL, dt, n, B, K, V, w, Z, res);
    free(T); free(D); free(x); free(u); free(tok); free(len); free(st); free(fl); free(dec);
    free(tlp); free(blp); free(M); free(S); free(g); free(ys); free(fs); free(lq); free(n);
    free(res); free(w); free(Z);
}

static void run_tree(int dt, int B, int N, int V, int malformed)
{
    void *T = logits(dt, (size_t)B * N * V, 3.0f, 0);
    int32_t *tok = malloc(sizeof(int32_t) * (size_t)B * N), *par = malloc(sizeof(int32_t) * (size_t)B * N);
    int32_t *nn = malloc(sizeof(int32_t) * B);
    for (int b = 0; b < B; ++b) {
        par[(size_t)b * N] = -1;
        tok[(size_t)b * N] = 0;
        for (int i = 1; i < N; ++i) {
            par[(size_t)b * N + i] = (int32_t)(next_u64() % (uint64_t)i);
            tok[(size_t)b * N + i] = (int32_t)(next_u64() % (uint64_t)V);
        }
        nn[b] = 1 + (int32_t)(next_u64() % (uint64_t)N);
    }
    if (malformed) {
        nn[0] = 0;
        if (N > 2) {
            par[2] = 5;       /* not below its child */
            tok[N - 1] = -7;  /* outside the vocabulary */
        }
        if (B > 1)
            nn[1] = N + 9;
    }
    int32_t *path = malloc(sizeof(int32_t) * (size_t)B * N), *otok = malloc(sizeof(int32_t) * (size_t)B * N);
    int32_t *len = malloc(sizeof(int32_t) * B), *st = malloc(sizeof(int32_t) * B);
    double *tlp = malloc(sizeof(double) * (size_t)B * N), *blp = malloc(sizeof(double) * (size_t)B * N);
    oracle_tree(T, dt, tok, par, nn, B, N, V, path, otok, len, tlp, blp, st);
    oracle_tree(T, dt, tok, par, NULL, B, N, V, path, otok, len, tlp, blp, st);
    free(T); free(tok); free(par); free(nn); free(path); free(otok); free(len); free(st);
    free(tlp); free(blp);
}

int main(void)
{
    oracle_set_threads(2);
    for (int dt = 0; dt < 2; ++dt) {
        for (int m = 0; m < 2; ++m) {
            run_chain(dt, 3, 4, 32, m);
            run_chain(dt, 2, 1, 1, m);      /* V = 1 */
            run_chain(dt, 2, 3, 2, m);
            run_chain(dt, 4, 5, 4099, m);   /* past one 4096-token chunk */
            run_tree(dt, 3, 9, 17, m);
            run_tree(dt, 2, 1, 5, m);       /* root only */
            run_tree(dt, 2, 64, 40, m);
        }
    }
    printf("oracle sanitizer driver: all calls returned\n");
    return 0;
}
