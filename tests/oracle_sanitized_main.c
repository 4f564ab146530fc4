/*
 * Memory- and UB-checked run of every CPU oracle function (test
 * infrastructure): built together with oracle/oracle.c under
 * -fsanitize=address,undefined by tests/test_oracle_sanitized.py.
 *
 * Every buffer is malloc'ed at exactly the size the function's contract
 * states, so an out-of-bounds access in the oracle is reported by the
 * address sanitizer; undefined integer or shift behaviour by the
 * undefined-behaviour sanitizer (both abort: -fno-sanitize-recover).  Each
 * call is also checked against a closed form or a brute-force recomputation
 * written here, so a sanitizer-clean but wrong result fails too.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float or_half_to_float(uint16_t h);
float or_bf16_to_float(uint16_t b);
uint16_t or_float_to_bf16(float f);
int or_quantize_q8(const float *x, int64_t rows, int64_t cols, int8_t *q, float *d);
int64_t or_unpack_ternary(const uint8_t *qs, int64_t n, int64_t k, int8_t *w);
int or_unpack_grid1(const uint8_t *qs, const uint16_t *qh, const int8_t *grid, int64_t n, int64_t k,
                    int8_t *w);
int or_unpack_sign1(const uint8_t *signs, const uint8_t *sc, int64_t n, int64_t k, int8_t *w);
int or_matvec_q8(const int8_t *w, const uint16_t *d16, int64_t R, int64_t K, const int8_t *xq,
                 const float *xd, int32_t *isums, double *y, double *tsum);
int or_matvec_bf16(const int8_t *w, const uint16_t *d16, int64_t R, int64_t K, const uint16_t *x,
                   double *y, double *tsum);
int or_route_topk(const float *logits, int64_t T, int64_t E, int top_k, int32_t *ids, double *w);
int or_group(const int32_t *ids, int64_t A, int32_t E, int32_t *offsets, int32_t *sorted,
             int32_t *active, int32_t *n_active);
void or_swiglu(const float *g, const float *u, int64_t n, double *h);
void or_combine(const float *out, const float *w, int64_t T, int top_k, int64_t H, double *y,
                double *ty);

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { /* xorshift64*, test data only */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float rnd_f(void) { return ((float)(rnd() >> 8) / 16777216.0f) * 2.0f - 1.0f; }

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

static void scalars(void) {
    CHECK(or_half_to_float(0x3C00) == 1.0f);
    CHECK(or_half_to_float(0x0001) == ldexpf(1.0f, -24));
    CHECK(or_half_to_float(0x8400) == -ldexpf(1.0f, -14));
    CHECK(isinf(or_half_to_float(0x7C00)) && isnan(or_half_to_float(0x7E00)));
    for (uint32_t h = 0; h < 65536; ++h) (void)or_half_to_float((uint16_t)h);
    CHECK(or_bf16_to_float(0x3F80) == 1.0f);
    CHECK(or_float_to_bf16(1.00390625f) == 0x3F80); /* tie to even */
    CHECK(or_float_to_bf16(1.01171875f) == 0x3F82); /* tie, odd -> up */
    CHECK(or_float_to_bf16(INFINITY) == 0x7F80);
}

static void q8(void) {
    const int64_t rows = 3, cols = 96;
    float *x = xmalloc(sizeof(float) * rows * cols);
    int8_t *q = xmalloc(rows * cols);
    float *d = xmalloc(sizeof(float) * rows * (cols / 32));
    for (int64_t i = 0; i < rows * cols; ++i) x[i] = 3.0f * rnd_f();
    for (int j = 0; j < 32; ++j) x[32 + j] = 0.0f; /* an all-zero block */
    CHECK(or_quantize_q8(x, rows, cols, q, d) == 0);
    CHECK(d[1] == 0.0f);
    for (int64_t b = 0; b < rows * (cols / 32); ++b) {
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[32 * b + j]));
        CHECK(d[b] == amax / 127.0f);
        for (int j = 0; j < 32; ++j) {
            CHECK(q[32 * b + j] >= -127 && q[32 * b + j] <= 127);
            if (d[b] > 0.0f) CHECK(fabsf(x[32 * b + j] - q[32 * b + j] * d[b]) <= d[b] * 0.5001f);
        }
    }
    x[5] = NAN;
    CHECK(or_quantize_q8(x, rows, cols, q, d) != 0);
    CHECK(or_quantize_q8(x, rows, 33, q, d) != 0);
    free(x);
    free(q);
    free(d);
}

static void unpack(void) {
    /* ternary: all 256 bytes in one row of 1024 weights */
    const int64_t k = 1024;
    uint8_t *qs = xmalloc(k / 4);
    int8_t *w = xmalloc(k);
    int64_t want_bad = 0;
    for (int i = 0; i < 256; ++i) {
        qs[i] = (uint8_t)i;
        for (int f = 0; f < 4; ++f) want_bad += ((i >> (2 * f)) & 3) == 3;
    }
    CHECK(or_unpack_ternary(qs, 1, k, w) == want_bad);
    for (int i = 0; i < 256; ++i)
        for (int f = 0; f < 4; ++f) {
            const int c = (i >> (2 * f)) & 3;
            CHECK(w[4 * i + f] == (c == 1 ? 1 : c == 2 ? -1 : 0));
        }
    CHECK(or_unpack_ternary(qs, 1, 6, w) < 0);
    free(qs);
    free(w);

    /* grid1: two rows of 512 weights, random indices */
    const int64_t n = 2, kg = 512;
    uint8_t *gqs = xmalloc(n * kg / 8);
    uint16_t *gqh = xmalloc(sizeof(uint16_t) * n * kg / 32);
    int8_t *grid = xmalloc(2048 * 8);
    int8_t *wg = xmalloc(n * kg);
    for (int i = 0; i < 2048 * 8; ++i) grid[i] = (int8_t)((int)(rnd() % 3) - 1);
    for (int64_t i = 0; i < n * kg / 8; ++i) gqs[i] = (uint8_t)rnd();
    for (int64_t i = 0; i < n * kg / 32; ++i) gqh[i] = (uint16_t)(rnd() & 0x0FFF);
    CHECK(or_unpack_grid1(gqs, gqh, grid, n, kg, wg) == 0);
    for (int64_t r = 0; r < n; ++r)
        for (int64_t g = 0; g < kg / 8; ++g) { /* group g of the row: block g/32, group g%32 */
            const unsigned idx = gqs[r * (kg / 8) + g] |
                                 (((gqh[r * (kg / 32) + g / 4] >> (3 * (g % 4))) & 7u) << 8);
            for (int j = 0; j < 8; ++j) CHECK(wg[r * kg + 8 * g + j] == grid[idx * 8 + j]);
        }
    CHECK(or_unpack_grid1(gqs, gqh, grid, n, 100, wg) != 0);

    /* sub-scaled signs */
    uint8_t *sg = xmalloc(n * kg / 8);
    uint8_t *sc = xmalloc(n * kg / 32);
    for (int64_t i = 0; i < n * kg / 8; ++i) sg[i] = (uint8_t)rnd();
    for (int64_t i = 0; i < n * kg / 32; ++i) sc[i] = (uint8_t)rnd();
    CHECK(or_unpack_sign1(sg, sc, n, kg, wg) == 0);
    for (int64_t c = 0; c < n * kg; ++c) {
        const int s = (sg[c / 8] >> (c % 8)) & 1;
        const int m = (sc[c / 32] >> (4 * ((c / 16) % 2))) & 15;
        CHECK(wg[c] == (s ? -m : m));
    }
    free(gqs);
    free(gqh);
    free(grid);
    free(wg);
    free(sg);
    free(sc);
}

static void matvec(void) {
    const int64_t R = 5, K = 768;
    int8_t *w = xmalloc(R * K);
    uint16_t *d16 = xmalloc(sizeof(uint16_t) * R * (K / 256));
    int8_t *xq = xmalloc(K);
    float *xd = xmalloc(sizeof(float) * (K / 32));
    int32_t *is = xmalloc(sizeof(int32_t) * R * (K / 32));
    double *y = xmalloc(sizeof(double) * R), *t = xmalloc(sizeof(double) * R);
    uint16_t *xb = xmalloc(sizeof(uint16_t) * K);
    for (int64_t i = 0; i < R * K; ++i) w[i] = (int8_t)((int)(rnd() % 3) - 1);
    for (int64_t i = 0; i < R * (K / 256); ++i) d16[i] = 0x3C00; /* 1.0 */
    for (int64_t i = 0; i < K; ++i) xq[i] = (int8_t)((int)(rnd() % 255) - 127);
    for (int64_t i = 0; i < K / 32; ++i) xd[i] = 0.25f;
    CHECK(or_matvec_q8(w, d16, R, K, xq, xd, is, y, t) == 0);
    for (int64_t r = 0; r < R; ++r) {
        int64_t tot = 0, tabs = 0;
        for (int64_t s = 0; s < K / 32; ++s) {
            int64_t acc = 0;
            for (int j = 0; j < 32; ++j) acc += (int64_t)w[r * K + 32 * s + j] * xq[32 * s + j];
            CHECK(is[r * (K / 32) + s] == acc);
            tot += acc;
            tabs += acc < 0 ? -acc : acc;
        }
        CHECK(y[r] == 0.25 * (double)tot); /* unit scales: exact */
        CHECK(t[r] == 0.25 * (double)tabs);
    }
    CHECK(or_matvec_q8(w, d16, R, K, xq, xd, NULL, y, t) == 0);
    CHECK(or_matvec_q8(w, d16, R, 100, xq, xd, NULL, y, t) != 0);
    for (int64_t i = 0; i < K; ++i) xb[i] = 0x3F80; /* bf16 1.0 */
    CHECK(or_matvec_bf16(w, d16, R, K, xb, y, t) == 0);
    for (int64_t r = 0; r < R; ++r) {
        int64_t s = 0, a = 0;
        for (int64_t k = 0; k < K; ++k) {
            s += w[r * K + k];
            a += w[r * K + k] != 0;
        }
        CHECK(y[r] == (double)s && t[r] == (double)a);
    }
    free(w);
    free(d16);
    free(xq);
    free(xd);
    free(is);
    free(y);
    free(t);
    free(xb);
}

static void route_group(void) {
    const int64_t T = 7, E = 9;
    const int k = 9; /* top_k == E */
    float *l = xmalloc(sizeof(float) * T * E);
    int32_t *ids = xmalloc(sizeof(int32_t) * T * k);
    double *w = xmalloc(sizeof(double) * T * k);
    for (int64_t i = 0; i < T * E; ++i) l[i] = (float)(rnd() % 4); /* many ties */
    CHECK(or_route_topk(l, T, E, k, ids, w) == 0);
    for (int64_t t = 0; t < T; ++t) {
        double s = 0.0;
        for (int j = 0; j < k; ++j) {
            s += w[t * k + j];
            if (j) {
                const float a = l[t * E + ids[t * k + j - 1]], b = l[t * E + ids[t * k + j]];
                CHECK(a > b || (a == b && ids[t * k + j - 1] < ids[t * k + j]));
            }
        }
        CHECK(fabs(s - 1.0) < 1e-12);
    }
    CHECK(or_route_topk(l, T, E, (int)E + 1, ids, w) != 0);
    l[3] = INFINITY;
    CHECK(or_route_topk(l, T, E, 2, ids, w) != 0);

    /* grouping with empty experts, and with no assignments at all */
    const int64_t A = 11;
    const int32_t G = 6;
    int32_t *gid = xmalloc(sizeof(int32_t) * A), *off = xmalloc(sizeof(int32_t) * (G + 1));
    int32_t *srt = xmalloc(sizeof(int32_t) * A), *act = xmalloc(sizeof(int32_t) * G), na = -1;
    for (int64_t a = 0; a < A; ++a) gid[a] = (int32_t)((a * 5) % 4) * 2; /* experts 0,2,4,6 -> only <6 */
    for (int64_t a = 0; a < A; ++a) if (gid[a] >= G) gid[a] = 1;
    CHECK(or_group(gid, A, G, off, srt, act, &na) == 0);
    CHECK(off[0] == 0 && off[G] == A);
    for (int32_t e = 0; e < G; ++e)
        for (int32_t i = off[e]; i < off[e + 1]; ++i) {
            CHECK(gid[srt[i]] == e);
            if (i > off[e]) CHECK(srt[i] > srt[i - 1]);
        }
    for (int32_t i = 0; i < na; ++i) CHECK(off[act[i] + 1] > off[act[i]]);
    CHECK(or_group(gid, 0, G, off, srt, act, &na) == 0 && na == 0 && off[G] == 0);
    gid[0] = G;
    CHECK(or_group(gid, A, G, off, srt, act, &na) != 0);
    free(l);
    free(ids);
    free(w);
    free(gid);
    free(off);
    free(srt);
    free(act);
}

static void swiglu_combine(void) {
    const int64_t n = 5;
    float g[5] = {0.0f, 1.0f, -1.0f, 40.0f, -40.0f}, u[5] = {2.0f, 2.0f, 2.0f, 0.5f, 3.0f};
    double *h = xmalloc(sizeof(double) * n);
    or_swiglu(g, u, n, h);
    CHECK(h[0] == 0.0 && fabs(h[3] - 20.0) < 1e-12 && fabs(h[4]) < 1e-15);
    CHECK(fabs(h[1] - 2.0 / (1.0 + exp(-1.0))) < 1e-15);
    free(h);
    const int64_t T = 3, H = 4;
    const int k = 2;
    float *out = xmalloc(sizeof(float) * T * k * H), *w = xmalloc(sizeof(float) * T * k);
    double *y = xmalloc(sizeof(double) * T * H), *ty = xmalloc(sizeof(double) * T * H);
    for (int64_t i = 0; i < T * k * H; ++i) out[i] = (float)(i % 7) - 3.0f;
    for (int64_t i = 0; i < T * k; ++i) w[i] = 0.5f;
    or_combine(out, w, T, k, H, y, ty);
    for (int64_t t = 0; t < T; ++t)
        for (int64_t c = 0; c < H; ++c) {
            const double a = out[(t * k) * H + c], b = out[(t * k + 1) * H + c];
            CHECK(y[t * H + c] == 0.5 * a + 0.5 * b);
            CHECK(ty[t * H + c] == 0.5 * fabs(a) + 0.5 * fabs(b));
        }
    free(out);
    free(w);
    free(y);
    free(ty);
}

int main(void) {
    scalars();
    q8();
    unpack();
    matvec();
    route_group();
    swiglu_combine();
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle sanitized run: OK\n");
    return 0;
}
