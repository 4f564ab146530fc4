/*
 * CPU oracle for the packed 1-bit-class MoE expert path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code with the HIP library.
 *
 * Plain, slow and sequential per output: every output element is computed by
 * one loop in a fixed order (integers exact, floating point in fp64 unless a
 * step is defined in fp32), so results do not depend on the thread count.
 * OpenMP only spreads independent output rows over threads.
 *
 * What each function follows:
 *  - int8 activations with integer dot products against packed expert weights
 *    that are never expanded: Parakon Runtime README, "How it works".
 *  - the q8 activation rule (per 32 values: scale = max|x| / 127, round half
 *    away from zero) and the fp32 scale application y = sum_blocks d_w *
 *    sum_sub d_x * int32 dot: the workload definition of this library, after
 *    the q8_1 activation path of the pxq_llama README ("Updates - 2026-07-28").
 *  - routing to the top-k experts with no dropping: llama-modchip summary,
 *    "Key highlights".
 *  - stable grouping of tokens by expert (grouped-MoE GEMM, ragged tails):
 *    pxq_llama README, "What's PXQ?" and "Run".
 *  - fused gate/up with SiLU: pxq_llama README, "Updates - 2026-07-28".
 *  - dequant-per-tile prefill GEMM: Parakon Runtime README, "How it works".
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_ERR_SHAPE -1
#define OR_ERR_VALUE -2

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void or_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* IEEE binary16 bit pattern -> float, exactly (every half is a float). */
float or_half_to_float(uint16_t h) {
    uint32_t sign = (h >> 15) & 1u, ex = (h >> 10) & 0x1fu, man = h & 0x3ffu;
    float v;
    if (ex == 0)
        v = ldexpf((float)man, -24);                    /* subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexpf((float)(man | 0x400u), (int)ex - 25); /* (1024+man) * 2^(ex-25) */
    return sign ? -v : v;
}

/* bf16 bit pattern -> float (bf16 is the top half of a float). */
float or_bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* float -> bf16 bit pattern, round to nearest, ties to even (finite inputs). */
uint16_t or_float_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) /* inf / nan: keep, quiet nans */
        return (uint16_t)((u >> 16) | ((u & 0x007fffffu) ? 0x40u : 0u));
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/*
 * q8 activation quantization, per 32 consecutive values of a row, in fp32:
 *   amax = max |x|;  d = amax / 127;  q = clamp(round_half_away(x / d), -127, 127);
 *   amax == 0 gives d = 0 and q = 0.
 * Both divisions are single correctly rounded fp32 divisions.
 * Returns OR_ERR_VALUE on a non-finite input (inputs must be finite).
 */
int or_quantize_q8(const float *x, int64_t rows, int64_t cols, int8_t *q, float *d) {
    if (cols <= 0 || cols % 32 != 0 || rows < 0) return OR_ERR_SHAPE;
    for (int64_t i = 0; i < rows * cols; ++i)
        if (!isfinite(x[i])) return OR_ERR_VALUE;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < cols / 32; ++b) {
            const float *xb = x + r * cols + 32 * b;
            int8_t *qb = q + r * cols + 32 * b;
            float amax = 0.0f;
            for (int j = 0; j < 32; ++j) {
                float a = fabsf(xb[j]);
                if (a > amax) amax = a;
            }
            float db = amax / 127.0f;
            d[r * (cols / 32) + b] = db;
            for (int j = 0; j < 32; ++j) {
                if (db == 0.0f) {
                    qb[j] = 0;
                    continue;
                }
                float v = roundf(xb[j] / db); /* C roundf: halfway cases away from zero */
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                qb[j] = (int8_t)v;
            }
        }
    }
    return OR_OK;
}

/*
 * Ternary unpack: weight k of row n is field (k % 4) of byte k / 4, i.e.
 * bits 2*(k%4) .. 2*(k%4)+1; code 0 -> 0, 1 -> +1, 2 -> -1, 3 invalid.
 * Writes w int8 [n][k]; returns the number of code-3 fields (0 when valid).
 */
int64_t or_unpack_ternary(const uint8_t *qs, int64_t n, int64_t k, int8_t *w) {
    if (k % 4 != 0) return OR_ERR_SHAPE;
    int64_t bad = 0;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t c = 0; c < k; ++c) {
            unsigned code = (qs[r * (k / 4) + c / 4] >> (2 * (c % 4))) & 3u;
            int8_t v = 0;
            if (code == 1) v = 1;
            else if (code == 2) v = -1;
            else if (code == 3) ++bad;
            w[r * k + c] = v;
        }
    }
    return bad;
}

/*
 * Grid1 unpack: in 256-weight block b of a row, group g (0..31) covers weights
 * 256b + 8g .. 256b + 8g + 7.  Its 11-bit codebook index is
 *   qs[32b + g]  |  ((qh[8b + g/4] >> (3 * (g % 4))) & 7) << 8
 * and weight 256b + 8g + j equals grid[index][j].
 */
int or_unpack_grid1(const uint8_t *qs, const uint16_t *qh, const int8_t *grid,
                    int64_t n, int64_t k, int8_t *w) {
    if (k % 256 != 0) return OR_ERR_SHAPE;
    for (int64_t r = 0; r < n; ++r) {
        const uint8_t *qsr = qs + r * (k / 8);
        const uint16_t *qhr = qh + r * (k / 32);
        for (int64_t b = 0; b < k / 256; ++b) {
            for (int g = 0; g < 32; ++g) {
                unsigned lo = qsr[32 * b + g];
                unsigned hi = (qhr[8 * b + g / 4] >> (3 * (g % 4))) & 7u;
                unsigned idx = lo | (hi << 8);
                for (int j = 0; j < 8; ++j)
                    w[r * k + 256 * b + 8 * g + j] = grid[idx * 8 + j];
            }
        }
    }
    return OR_OK;
}

/*
 * Sub-scaled sign unpack (1-bit sign codes with one fp16 anchor per row and a
 * 4-bit sub-scale per 16 weights: pxq_llama README, "What's PXQ?", the PXQ1
 * tier).  Weight c of row r is the integer
 *   sc * (s ? -1 : +1),   s  = (signs[r][c / 8] >> (c % 8)) & 1,
 *                         sc = (sc_bytes[r][c / 32] >> (4 * ((c / 16) % 2))) & 15,
 * times the row's anchor, which the caller applies as the row's scale in
 * every 256-weight block of the mat-vec.  |w| <= 15.
 */
int or_unpack_sign1(const uint8_t *signs, const uint8_t *sc, int64_t n, int64_t k, int8_t *w) {
    if (k % 32 != 0) return OR_ERR_SHAPE;
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t c = 0; c < k; ++c) {
            const unsigned s = (signs[r * (k / 8) + c / 8] >> (c % 8)) & 1u;
            const unsigned m = (sc[r * (k / 32) + c / 32] >> (4 * ((c / 16) % 2))) & 15u;
            w[r * k + c] = (int8_t)(s ? -(int)m : (int)m);
        }
    }
    return OR_OK;
}

/*
 * Mat-vec of R unpacked weight rows w int8 [R][K] (scales d16 fp16 [R][K/256])
 * against one q8 activation row (xq int8 [K], xd float [K/32]):
 *   isum[r][s] = sum_{j<32} w[r][32s+j] * xq[32s+j]          (exact integer)
 *   y[r]       = sum_b d_w[r][b] * sum_{s in b} xd[s] * isum[r][s]   (fp64)
 *   tsum[r]    = sum_b sum_{s in b} |d_w[r][b] * xd[s] * isum[r][s]|
 * isums may be NULL.  Returns OR_ERR_VALUE if an isum leaves int32 range.
 */
int or_matvec_q8(const int8_t *w, const uint16_t *d16, int64_t R, int64_t K,
                 const int8_t *xq, const float *xd, int32_t *isums, double *y, double *tsum) {
    if (K % 256 != 0) return OR_ERR_SHAPE;
    int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int64_t r = 0; r < R; ++r) {
        double acc = 0.0, tabs = 0.0;
        for (int64_t b = 0; b < K / 256; ++b) {
            double dw = (double)or_half_to_float(d16[r * (K / 256) + b]);
            for (int64_t s = 8 * b; s < 8 * b + 8; ++s) {
                int64_t is = 0;
                for (int j = 0; j < 32; ++j)
                    is += (int64_t)w[r * K + 32 * s + j] * (int64_t)xq[32 * s + j];
                if (is > INT32_MAX || is < INT32_MIN) err = 1;
                if (isums) isums[r * (K / 32) + s] = (int32_t)is;
                double term = dw * (double)xd[s] * (double)is;
                acc += term;
                tabs += fabs(term);
            }
        }
        y[r] = acc;
        tsum[r] = tabs;
    }
    return err ? OR_ERR_VALUE : OR_OK;
}

/*
 * Same rows against one bf16 activation row x [K] (prefill):
 *   y[r]    = sum_b d_w[r][b] * sum_{k in b} x[k] * w[r][k]        (fp64)
 *   tsum[r] = sum_b |d_w[r][b]| * sum_{k in b} |x[k] * w[r][k]|
 */
int or_matvec_bf16(const int8_t *w, const uint16_t *d16, int64_t R, int64_t K,
                   const uint16_t *x, double *y, double *tsum) {
    if (K % 256 != 0) return OR_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        double acc = 0.0, tabs = 0.0;
        for (int64_t b = 0; b < K / 256; ++b) {
            double dw = (double)or_half_to_float(d16[r * (K / 256) + b]);
            double blk = 0.0, babs = 0.0;
            for (int64_t k = 256 * b; k < 256 * b + 256; ++k) {
                double p = (double)or_bf16_to_float(x[k]) * (double)w[r * K + k];
                blk += p;
                babs += fabs(p);
            }
            acc += dw * blk;
            tabs += fabs(dw) * babs;
        }
        y[r] = acc;
        tsum[r] = tabs;
    }
    return OR_OK;
}

/*
 * Router: per token, the top_k largest logits in descending order (equal
 * logits: lower expert index first), then softmax over the selected logits
 * only:  w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), in fp64.
 */
int or_route_topk(const float *logits, int64_t T, int64_t E, int top_k,
                  int32_t *ids, double *w) {
    if (top_k < 1 || top_k > E) return OR_ERR_SHAPE;
    for (int64_t i = 0; i < T * E; ++i)
        if (!isfinite(logits[i])) return OR_ERR_VALUE;
    int err = 0;
#pragma omp parallel for schedule(static) reduction(| : err)
    for (int64_t t = 0; t < T; ++t) {
        const float *l = logits + t * E;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        if (!taken) { err = 1; continue; }
        for (int j = 0; j < top_k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
            taken[best] = 1;
            ids[t * top_k + j] = (int32_t)best;
        }
        double l0 = (double)l[ids[t * top_k]], s = 0.0;
        for (int j = 0; j < top_k; ++j) {
            double ex = exp((double)l[ids[t * top_k + j]] - l0);
            w[t * top_k + j] = ex;
            s += ex;
        }
        for (int j = 0; j < top_k; ++j) w[t * top_k + j] /= s;
        free(taken);
    }
    return err ? OR_ERR_VALUE : OR_OK;
}

/*
 * Stable grouping of the A = T*top_k assignments (a = t*top_k + j) by expert:
 * offsets [E+1] = exclusive prefix sum of the per-expert counts; sorted holds
 * every a ordered by (ids[a], a); active lists the experts with at least one
 * assignment in increasing id order, and *n_active their number.
 */
int or_group(const int32_t *ids, int64_t A, int32_t E, int32_t *offsets, int32_t *sorted,
             int32_t *active, int32_t *n_active) {
    for (int64_t a = 0; a < A; ++a)
        if (ids[a] < 0 || ids[a] >= E) return OR_ERR_VALUE;
    int64_t *fill = (int64_t *)calloc((size_t)E + 1, sizeof(int64_t));
    if (!fill) return OR_ERR_VALUE;
    for (int32_t e = 0; e <= E; ++e) offsets[e] = 0;
    for (int64_t a = 0; a < A; ++a) offsets[ids[a] + 1] += 1;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (int32_t e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int64_t a = 0; a < A; ++a) sorted[fill[ids[a]]++] = (int32_t)a;
    int32_t na = 0;
    for (int32_t e = 0; e < E; ++e)
        if (offsets[e + 1] > offsets[e]) active[na++] = e;
    *n_active = na;
    free(fill);
    return OR_OK;
}

/* SwiGLU in fp64: h = silu(g) * u,  silu(z) = z / (1 + exp(-z)). */
void or_swiglu(const float *g, const float *u, int64_t n, double *h) {
    for (int64_t i = 0; i < n; ++i) {
        double z = (double)g[i];
        h[i] = z / (1.0 + exp(-z)) * (double)u[i];
    }
}

/*
 * Weighted combine: y[t][n] = sum_{j<top_k} w[t][j] * out[t*top_k + j][n] (fp64),
 * ty[t][n] = sum_j |w[t][j] * out[t*top_k + j][n]|.
 */
void or_combine(const float *out, const float *w, int64_t T, int top_k, int64_t H,
                double *y, double *ty) {
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < H; ++n) {
            double acc = 0.0, tabs = 0.0;
            for (int j = 0; j < top_k; ++j) {
                double p = (double)w[t * top_k + j] * (double)out[(t * top_k + j) * H + n];
                acc += p;
                tabs += fabs(p);
            }
            y[t * H + n] = acc;
            ty[t * H + n] = tabs;
        }
}
