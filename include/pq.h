/*
 * pq.h -- C ABI of libpq: packed 1-bit-class MoE expert kernels for AMD
 * Instinct MI355X (CDNA4, gfx950).
 *
 * The library runs the routed-expert FFN of a Mixture-of-Experts layer whose
 * expert weights stay in packed 1-bit-class block formats in device memory
 * and are read directly by the kernels; no dequantized copy of a weight
 * matrix is ever written (Parakon Runtime README, "How it works": fused
 * mat-vec kernels read the quantized blocks and accumulate against int8
 * activations; large prompt batches use a dequant-per-tile GEMM).
 *
 * Conventions for every entry point
 *  - Array arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains memory and keeps no state between
 *    calls other than a per-device cache of the compute-unit count.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  No call synchronizes the stream or the device.
 *  - All argument checks run on the host before the first HIP call; on a
 *    failed check nothing is enqueued.  On any status other than PQ_OK the
 *    contents of the output buffers are undefined.
 *  - No C++ exception crosses this interface.
 *  - Calls that share output buffers must be ordered by the caller; calls on
 *    different streams with disjoint outputs may run concurrently.
 *
 * Tokens, experts, assignments
 *  - T = n_tokens, E = n_experts, k = top_k; A = T*k assignments.  The
 *    assignment of token t to its j-th selected expert has id a = t*k + j.
 *  - Expert weight tensors are [E][rows][cols]; an expert computes
 *    out[n] = sum_c W[n][c] * act[c] for each of its rows n.
 *
 * Packed formats (structure of arrays; each plane contiguous, row-major)
 *  - ternary (2.0625 bits/weight): qs uint8 [E][rows][cols/4], four 2-bit
 *    codes per byte, weight 4i+j of a row in bits 2j..2j+1 of byte i; code 0
 *    -> 0, 1 -> +1, 2 -> -1 (code 3 is invalid; kernel output on code 3 is
 *    unspecified).  d: IEEE fp16 bits [E][rows][cols/256], one scale per
 *    256-weight row block.  Ternary routed experts: modelium.tech article on
 *    Parallax 8B kappa, "What exactly is available".
 *  - grid1 (1.5625 bits/weight): per 256-weight row block b, 32 groups of 8
 *    weights; group g has the 11-bit codebook index
 *    qs[32b+g] | ((qh[8b+g/4] >> 3*(g%4)) & 7) << 8, and weights
 *    256b+8g+j = grid[index][j].  qs uint8 [E][rows][cols/8], qh uint16
 *    [E][rows][cols/32] (bits 12..15 ignored), d fp16 bits [E][rows][cols/256],
 *    grid int8 [2048][8] with entries in {-1,0,+1}.  1-bit codebook formats
 *    after the dynamic 1-bit family: Parakon Runtime README, "How it works"
 *    and "Attribution"; IQ1_S-class routed experts: llama-modchip summary.
 *  - q8 activations: per 32 consecutive values of a row, d = max|x| / 127
 *    (fp32, correctly rounded), q = round_half_away_from_zero(x / d) clamped to
 *    [-127, 127] as int8; max|x| = 0 gives d = 0 and q = 0.  xq int8
 *    [rows][cols], xd float [rows][cols/32].
 *  - Mat-vec result per row n:  sum_b d_w[n][b] * sum_{s in b} xd[s] *
 *    isum[n][s], with isum[n][s] = sum_{j<32} w[n][32s+j] * xq[32s+j] an exact
 *    int32 block sum; fp32 output.
 */
#ifndef PQ_H
#define PQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PQ_ABI_VERSION 2

typedef enum pq_status {
    PQ_OK = 0,
    PQ_ERR_NULL = 1,        /* a required pointer is NULL */
    PQ_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    PQ_ERR_ALIGN = 3,       /* a pointer is not aligned as documented */
    PQ_ERR_UNSUPPORTED = 4, /* valid arguments this build has no kernel for */
    PQ_ERR_HIP = 5,         /* a HIP call or kernel launch failed */
    PQ_ERR_SELFTEST = 6     /* pq_selftest: a known answer did not come out */
} pq_status;

enum {
    PQ_EPI_F32 = 0,         /* out0 = float [A][rows] */
    PQ_EPI_SWIGLU_Q8 = 1,   /* out0 = int8 hq [A][rows], out1 = float hd [A][rows/32] */
    PQ_EPI_SWIGLU_BF16 = 2, /* out0 = bf16 bits h [A][rows] */
    PQ_EPI_F32_COMBINE = 3  /* out0 = float y [n_tokens][rows] (+=), out1 = float topk_w */
};

/* Weight formats (pq_plan). */
enum { PQ_FMT_TERNARY = 0, PQ_FMT_GRID1 = 1, PQ_FMT_SIGN1 = 2 };

/* Entry-point families (pq_plan). */
enum {
    PQ_CALL_MATVEC = 0,          /* pq_moe_matvec_{ternary,grid1,sign1} */
    PQ_CALL_TILE_Q8 = 1,         /* pq_moe_tile_q8_{ternary,grid1,sign1} */
    PQ_CALL_GEMM = 2,            /* pq_moe_gemm_dequant_tile{,_sign1} */
    PQ_CALL_DECODE1_GATE_UP = 3  /* pq_moe_decode1_gate_up_{ternary,grid1,sign1} */
};

/* Kernels a call launches (bit flags returned by pq_plan). */
enum {
    PQ_PLAN_MATVEC = 1,          /* grouped mat-vec, all of an expert's assignments per work item */
    PQ_PLAN_MATVEC_PAIRS = 2,    /* grouped mat-vec, pairs of an expert's assignments per work item */
    PQ_PLAN_MATVEC_TOK1 = 4,     /* one-token mat-vec (one workgroup per slot and 32-row tile) */
    PQ_PLAN_TILE_Q8 = 8,         /* int8-MFMA tile (every expert, or with MATVEC_PAIRS those of 8+ assignments) */
    PQ_PLAN_GEMM = 16,           /* bf16 dequant-per-tile MFMA GEMM */
    PQ_PLAN_DECODE1_ROUTED = 32, /* one-token gate/up that routes and quantizes itself */
    PQ_PLAN_DEBUG = 64,          /* the kernels' debug variants (dbg != NULL) */
    PQ_PLAN_MIXED = 128          /* with TILE_Q8 | MATVEC_PAIRS: both in one launch (ternary, rows of 768 or 2048) */
};

/* hipStream_t, passed as an opaque pointer; NULL = null stream. */
typedef void *pq_stream;

/* Ternary expert tensor [n_experts][rows][cols]. qs: 16-byte aligned; d: 2-byte aligned. */
typedef struct pq_ternary_w {
    const uint8_t *qs;
    const uint16_t *d;
    int32_t n_experts, rows, cols;
} pq_ternary_w;

/* Grid1 expert tensor [n_experts][rows][cols]. qs 16-byte, qh 8-byte, d 2-byte,
   grid 16-byte aligned. */
typedef struct pq_grid1_w {
    const uint8_t *qs;
    const uint16_t *qh;
    const uint16_t *d;
    const int8_t *grid;
    int32_t n_experts, rows, cols;
} pq_grid1_w;

/* Sub-scaled sign expert tensor [n_experts][rows][cols] (1-bit sign codes, a
   4-bit sub-scale per 16 weights, one fp16 anchor per row: pxq_llama README,
   "What's PXQ?", the PXQ1 tier).  signs uint8 [E][rows][cols/8]: bit j of
   byte i is the sign of weight 8i+j (1 = negative); sc uint8
   [E][rows][cols/32]: byte i holds the sub-scales (0..15) of weights 32i..
   32i+15 (low nibble) and 32i+16..32i+31 (high nibble); d fp16 bits
   [E][rows]: the row's anchor.  Weight = d * sc * (+-1).  signs 16-byte, sc
   4-byte, d 2-byte aligned. */
typedef struct pq_sign1_w {
    const uint8_t *signs;
    const uint8_t *sc;
    const uint16_t *d;
    int32_t n_experts, rows, cols;
} pq_sign1_w;

/* Output of pq_group_tokens_by_expert, consumed by the expert kernels. */
typedef struct pq_groups {
    const int32_t *expert_offsets; /* [n_experts+1] */
    const int32_t *sorted_assign;  /* [n_tokens*top_k] */
    const int32_t *active_experts; /* [n_experts]; first *n_active entries valid */
    const int32_t *n_active;       /* [1] */
    int32_t n_tokens, top_k, n_experts;
} pq_groups;

/* Optional debug outputs of the expert kernels (a separate kernel variant is
   used when dbg != NULL; the production variant writes none of these).  Each
   pointer may be NULL.  isums: int32 [A][rows][cols/32] block sums of `w`,
   isums_up: the same for `w_up`; g, u: fp32 [A][rows] outputs of `w` and
   `w_up` before the epilogue; h: fp32 [A][rows] silu(g)*u before rounding or
   quantization. */
typedef struct pq_debug {
    int32_t *isums;
    int32_t *isums_up;
    float *g;
    float *u;
    float *h;
} pq_debug;

/*
 * q8 activation quantization (Parakon Runtime README, "How it works": int8
 * activations for the dp4a-style decode path; rule as in the header above).
 *   x  float [n_rows][cols] -> xq int8 [n_rows][cols], xd float [n_rows][cols/32]
 * cols % 32 == 0; x and xq 16-byte aligned.  Inputs must be finite (output on
 * non-finite input is unspecified).  n_rows == 0 is a no-op.
 */
pq_status pq_quantize_act_q8(const float *x, int32_t n_rows, int32_t cols,
                             int8_t *xq, float *xd, pq_stream stream);

/*
 * Router: per token, the top_k largest of n_experts fp32 logits in descending
 * order (equal logits: lower expert index first), then softmax over those
 * top_k logits only: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0).  Every
 * selected expert is evaluated; nothing is dropped (llama-modchip summary,
 * "Key highlights").
 *   logits float [n_tokens][n_experts] -> topk_ids int32 [n_tokens][top_k],
 *   topk_w float [n_tokens][top_k].
 * 1 <= top_k <= min(16, n_experts); n_experts <= 1024.  Logits must be finite.
 */
pq_status pq_moe_route_topk(const float *logits, int32_t n_tokens, int32_t n_experts,
                            int32_t top_k, int32_t *topk_ids, float *topk_w,
                            pq_stream stream);

/*
 * Stable grouping of the A = n_tokens*top_k assignments by expert (the grouped
 * MoE path and ragged tails of the pxq_llama README, "What's PXQ?" and "Run").
 *   expert_offsets [n_experts+1]: exclusive prefix sum of per-expert counts;
 *   sorted_assign [A]: every assignment id, ordered by (expert, id);
 *   active_experts [n_experts]: the experts with at least one assignment, in
 *   increasing id order; *n_active: their number.
 * The expert kernels rely on these invariants (for a grouping made by hand
 * as well): an expert's assignments end where the next active expert's
 * begin.
 * topk_ids must hold values in [0, n_experts) (out-of-range ids give
 * unspecified output).  n_experts <= 1024; A <= 1<<20.
 */
pq_status pq_group_tokens_by_expert(const int32_t *topk_ids, int32_t n_tokens, int32_t top_k,
                                    int32_t n_experts, int32_t *expert_offsets,
                                    int32_t *sorted_assign, int32_t *active_experts,
                                    int32_t *n_active, pq_stream stream);

/*
 * Decode prep: pq_quantize_act_q8 of x [n_tokens][hidden], pq_moe_route_topk
 * of logits [n_tokens][n_experts] and pq_group_tokens_by_expert of the
 * result, with outputs identical to those three calls (same layouts as
 * there); if y_zero != NULL it is also set to zero, float [n_tokens][hidden]
 * (for PQ_EPI_F32_COMBINE).  One launch of one workgroup (one wave per token
 * for the selection) when 1 <= n_tokens <= 16, n_tokens*top_k <= 256 and
 * n_tokens*n_experts <= 1024; otherwise two launches: the q8 and the routing side by side in one, the
 * grouping in the other.  n_experts <= 1024, top_k <= 16 and <= n_experts,
 * n_tokens*top_k <= 1<<20, hidden % 32 == 0 (PQ_ERR_SHAPE otherwise).
 * n_tokens == 0 writes the empty grouping (offsets all 0, *n_active = 0);
 * then only expert_offsets, active_experts and n_active must be non-NULL.
 * (Parakon Runtime README, "How it works": int8 activations; llama-modchip
 * summary, "Key highlights": top-k with no dropping; pxq_llama README,
 * "What's PXQ?": grouped experts.)
 */
pq_status pq_moe_decode_prep(const float *x, const float *logits, int32_t n_tokens,
                             int32_t hidden, int32_t n_experts, int32_t top_k, int8_t *xq,
                             float *xd, int32_t *topk_ids, float *topk_w,
                             int32_t *expert_offsets, int32_t *sorted_assign,
                             int32_t *active_experts, int32_t *n_active, float *y_zero,
                             pq_stream stream);

/*
 * Grouped expert mat-vec over packed ternary weights against q8 activations
 * (Parakon Runtime README, "How it works": fused decode mat-vec reading the
 * packed blocks directly with int8 dot products; gate/up fusion with SiLU:
 * pxq_llama README, "Updates - 2026-07-28").
 *
 * For every assignment a (expert e = its group), with activation row
 * r = act_by_token ? a / top_k : a  (xq [n_rows][cols], xd [n_rows][cols/32]):
 *   PQ_EPI_F32:       out0 float [A][rows]: W_e . act_r
 *   PQ_EPI_SWIGLU_Q8: needs w_up (same shape); g = W_e . act_r, u = Wup_e . act_r,
 *                     h = silu(g) * u in fp32, then q8 of h per 32 rows:
 *                     out0 int8 [A][rows], out1 float [A][rows/32]; rows % 32 == 0.
 *   PQ_EPI_F32_COMBINE: the weighted combine fused into the mat-vec (for the
 *                     down projection, act_by_token == 0): out0 float y
 *                     [n_tokens][rows] receives y[a/top_k][n] += topk_w[a] *
 *                     (W_e . act_a) by fp32 atomic adds, so y must hold zeros
 *                     (pq_moe_decode_prep can clear it) and the order of the
 *                     top_k additions is unspecified (the result can differ in
 *                     the last bits between runs); out1 = topk_w float
 *                     [n_tokens][top_k] (read only).  Saves the separate
 *                     pq_moe_combine launch at a few tokens.
 * cols % 256 == 0 and cols/64 in {4,8,12,16,24,32,48,64} (cols 256..4096);
 * rows >= 1.  w->n_experts == g->n_experts.  dbg may be NULL.
 */
pq_status pq_moe_matvec_ternary(const pq_ternary_w *w, const pq_ternary_w *w_up,
                                const pq_groups *g, const int8_t *xq, const float *xd,
                                int32_t act_by_token, int32_t epilogue, void *out0,
                                void *out1, const pq_debug *dbg, pq_stream stream);

/*
 * The same over grid1 weights (1-bit codebook format).  The codebook is staged
 * in LDS once per workgroup.  cols % 256 == 0 and cols/128 in
 * {2,4,8,12,16,24,32,48,64} (cols 256..8192).
 */
pq_status pq_moe_matvec_grid1(const pq_grid1_w *w, const pq_grid1_w *w_up,
                              const pq_groups *g, const int8_t *xq, const float *xd,
                              int32_t act_by_token, int32_t epilogue, void *out0,
                              void *out1, const pq_debug *dbg, pq_stream stream);

/*
 * The same over sub-scaled sign weights (pq_sign1_w): the 16-weight +-1 sums
 * times their sub-scales give the exact int32 sum of each q8 block, and the
 * row's anchor is the scale of every block, so the outputs are those of the
 * other formats' definition with w = d * sc * (+-1).  cols % 256 == 0 and
 * cols/128 in {2,4,8,12,16,24,32,48,64} (cols 256..8192).  One token
 * (without dbg) runs the one-token kernel, other token counts the grouped
 * mat-vec, with the experts of 8+ assignments of a large batch on the
 * int8-MFMA tile (pq_moe_tile_q8_sign1) as for the other formats.
 */
pq_status pq_moe_matvec_sign1(const pq_sign1_w *w, const pq_sign1_w *w_up,
                              const pq_groups *g, const int8_t *xq, const float *xd,
                              int32_t act_by_token, int32_t epilogue, void *out0,
                              void *out1, const pq_debug *dbg, pq_stream stream);

/*
 * One mat-vec from fp32 activations in a single launch (the fused decode
 * mat-vec of the Parakon Runtime README, "How it works", reading the packed
 * blocks against int8 activations, with the q8 step inside the launch):
 *   y float [rows] = W[expert] . q8(x),  x float [cols],
 * x quantized per 32 by the rule of pq_quantize_act_q8 (the same codes and
 * scales, computed again by every workgroup into its LDS), then the one-token
 * arithmetic of pq_moe_matvec_* with PQ_EPI_F32, so y is bit-identical to
 * pq_quantize_act_q8 followed by that call for one token routed to `expert`.
 * 0 <= expert < w->n_experts (PQ_ERR_SHAPE otherwise); cols as for
 * pq_moe_matvec_* of the format (PQ_ERR_UNSUPPORTED otherwise); x 16-byte,
 * y 4-byte aligned; x finite.  Nothing but y is written; y may not overlap x.
 */
pq_status pq_matvec_x32_ternary(const pq_ternary_w *w, int32_t expert, const float *x, float *y,
                                pq_stream stream);
pq_status pq_matvec_x32_grid1(const pq_grid1_w *w, int32_t expert, const float *x, float *y,
                              pq_stream stream);
pq_status pq_matvec_x32_sign1(const pq_sign1_w *w, int32_t expert, const float *x, float *y,
                              pq_stream stream);

/*
 * Grouped int8-MFMA tile over q8 activations (a tiled kernel for large
 * batches: Parakon Runtime README, "How it works"; an int8 prefill tile:
 * pxq_llama README, "Updates - 2026-07-19").  Arguments, layouts, epilogues
 * and outputs are those of pq_moe_matvec_ternary / _grid1 / _sign1, and so
 * is the arithmetic: one v_mfma_i32_16x16x32_i8 per q8 block gives the same
 * exact int32 block sums (dbg->isums equal the mat-vec's bit for bit),
 * scaled in fp32 as sum over 256-blocks of d * (sum over 32-blocks of
 * xd * isum).  Sub-scaled signs enter the MFMA as int8 weights sign * sc
 * (|w| <= 15), so its block sums are the per-16 sums times their
 * sub-scales, and the row's anchor is d for every 256-block.  Only the fp32
 * summation order differs, within the tolerance of the fp32 result.  Every active expert is processed in chunks of up to
 * 32 assignments (batches of at most 2048 assignments) or 64 (larger
 * batches), and tiles of 64 weight rows (32 gate + 32 up rows for
 * PQ_EPI_SWIGLU_Q8).  cols % 256 == 0 (any such cols); rows >= 1 (rows % 32
 * == 0 for PQ_EPI_SWIGLU_Q8).
 *
 * pq_moe_matvec_* use this kernel by themselves, per expert, when the batch
 * has more assignments than experts and at least 8 tokens: experts holding
 * at least 8 assignments then run here, the others on the mat-vec (two
 * launches on the stream).
 */
pq_status pq_moe_tile_q8_ternary(const pq_ternary_w *w, const pq_ternary_w *w_up,
                                 const pq_groups *g, const int8_t *xq, const float *xd,
                                 int32_t act_by_token, int32_t epilogue, void *out0,
                                 void *out1, const pq_debug *dbg, pq_stream stream);
pq_status pq_moe_tile_q8_grid1(const pq_grid1_w *w, const pq_grid1_w *w_up,
                               const pq_groups *g, const int8_t *xq, const float *xd,
                               int32_t act_by_token, int32_t epilogue, void *out0,
                               void *out1, const pq_debug *dbg, pq_stream stream);
pq_status pq_moe_tile_q8_sign1(const pq_sign1_w *w, const pq_sign1_w *w_up,
                               const pq_groups *g, const int8_t *xq, const float *xd,
                               int32_t act_by_token, int32_t epilogue, void *out0,
                               void *out1, const pq_debug *dbg, pq_stream stream);

/*
 * Tile layout of the packed planes that the prefill GEMM reads (the same
 * bytes, reordered; Parakon Runtime README, "How it works": the packed blocks
 * are consumed tile by tile and never expanded).  Rows are taken in groups,
 * and for every 256-column block (every 512-column pair for sub-scales) the
 * group's bytes of that block lie back to back as one 128-byte line:
 *   grid1 qs     [E][rows/4][cols/256][4][32]  bytes
 *   grid1 qh     [E][rows/8][cols/256][8][8]   uint16
 *   sign1 signs  [E][rows/4][cols/256][4][32]  bytes
 *   sign1 sc     [E][rows/8][cols/512][8][16]  bytes
 * (row n of a group sits at its position n % 4 or n % 8 in the line).  The d
 * planes and the grid keep their own layout.
 *
 * pq_tile_layout_grid1 writes w's qs and qh in the tile layout to qs_tiled
 * (same size as w->qs) and qh_tiled (same size as w->qh);
 * pq_tile_layout_sign1 does the same for signs and sc.  rows % 8 == 0, cols
 * % 256 == 0 (grid1) or % 512 == 0 (sign1); every plane 16-byte aligned; no
 * output may overlap an input or the other output (PQ_ERR_SHAPE).  The
 * caller owns all buffers; the call only enqueues kernels on `stream`.
 */
pq_status pq_tile_layout_grid1(const pq_grid1_w *w, uint8_t *qs_tiled, uint16_t *qh_tiled,
                               pq_stream stream);
pq_status pq_tile_layout_sign1(const pq_sign1_w *w, uint8_t *signs_tiled, uint8_t *sc_tiled,
                               pq_stream stream);

/*
 * Prefill: grouped dequant-per-tile GEMM over grid1 weights with bf16
 * activations on MFMA (Parakon Runtime README, "How it works": prompt
 * processing at large batch sizes uses a dequant-per-tile GEMM path).  Packed
 * blocks are decoded to bf16 {-1,0,+1} on chip only; the exact products are
 * accumulated in fp32 and each 256-column block's fp16 scale is applied in
 * fp32 (to one running accumulator per output, rescaled by the ratio of
 * consecutive nonzero block scales: within about 3e-6 * sum|terms| of
 * scaling each block sum on its own, inside the fp32 tolerance).
 *   w, w_up: qs and qh in the tile layout (pq_tile_layout_grid1), d and grid
 *            as in pq_grid1_w.  rows % 8 == 0 (PQ_ERR_SHAPE otherwise).
 *   x: bf16 bits, [n_tokens][cols] if act_by_token else [A][cols]; 16-byte aligned.
 *   PQ_EPI_F32:         out0 float [A][rows]; out1 unused (may be NULL).
 *   PQ_EPI_SWIGLU_BF16: needs w_up; out0 bf16 bits [A][rows] of
 *                       round_to_nearest_even(silu(g) * u); rows % 32 == 0;
 *                       out1 unused.
 *   PQ_EPI_F32_COMBINE: the weighted combine (pq_moe_combine) fused into the
 *                       GEMM: out0 float y [n_tokens][rows] receives
 *                       y[a/top_k][n] += topk_w[a] * out[a][n] by fp32 atomic
 *                       adds (y must hold zeros; the order of the top_k
 *                       additions is unspecified, so the last bits can differ
 *                       between runs); out1 = topk_w float [n_tokens][top_k].
 *                       Saves writing and re-reading the [A][rows] outputs.
 * cols % 256 == 0.  dbg may be NULL (g, u, h fields honoured; with the fused
 * combine, g receives the per-assignment outputs out[a][n]).
 */
pq_status pq_moe_gemm_dequant_tile(const pq_grid1_w *w, const pq_grid1_w *w_up,
                                   const pq_groups *g, const uint16_t *x,
                                   int32_t act_by_token, int32_t epilogue, void *out0,
                                   void *out1, const pq_debug *dbg, pq_stream stream);

/*
 * The same GEMM over sub-scaled sign weights (pq_sign1_w; pxq_llama README,
 * "What's PXQ?", PXQ1): each weight is decoded on chip to the bf16 of
 * sign * sc (exact, |w| <= 15) and the fp32 sum over the row is scaled by the
 * row's fp16 anchor (the scale of every block), so out = sum_b d[n] *
 * sum_{k in b} x[k] * sign * sc, within the fp32 tolerance of the definition.  signs and sc in the tile
 * layout (pq_tile_layout_sign1), d as in pq_sign1_w.  cols % 512 == 0; signs
 * and sc 16-byte aligned; otherwise as pq_moe_gemm_dequant_tile.
 */
pq_status pq_moe_gemm_dequant_tile_sign1(const pq_sign1_w *w, const pq_sign1_w *w_up,
                                         const pq_groups *g, const uint16_t *x,
                                         int32_t act_by_token, int32_t epilogue, void *out0,
                                         void *out1, const pq_debug *dbg, pq_stream stream);

/*
 * Weighted combine of the per-assignment expert outputs (the scatter of the
 * pxq_llama README, "Run"): y[t][n] = sum_{j<top_k} topk_w[t][j] *
 * out_assign[t*top_k+j][n], summed in slot order j = 0..top_k-1 (deterministic).
 * out_assign float [n_tokens*top_k][rows]; y float [n_tokens][rows].
 */
pq_status pq_moe_combine(const float *out_assign, const float *topk_w, int32_t n_tokens,
                         int32_t top_k, int32_t rows, float *y, pq_stream stream);

/*
 * One-token gate/up with its own routing (the fused decode path of the
 * Parakon Runtime README, "How it works", at batch 1; gate/up fusion with
 * SiLU: pxq_llama README, "Updates - 2026-07-28").  Every workgroup computes
 * the top-k routing of `logits` and the q8 of `x` itself, so the launch
 * waits for no earlier one; then the gate/up mat-vec with the SwiGLU + q8
 * epilogue.  Outputs equal, bit for bit, those of pq_moe_decode_prep (routing
 * and grouping; no xq/xd) followed by pq_moe_matvec_*(gate, up,
 * act_by_token = 1, PQ_EPI_SWIGLU_Q8) on the same inputs:
 *   topk_ids int32 [top_k], topk_w float [top_k] (rank order);
 *   expert_offsets [n_experts+1], sorted_assign [top_k], active_experts
 *   [top_k], n_active [1]: the grouping of those ids, ready for the down
 *   mat-vec (e.g. pq_moe_matvec_*(down, ..., PQ_EPI_F32_COMBINE));
 *   hq int8 [top_k][I], hd float [top_k][I/32];
 *   y_zero (may be NULL): float [H] set to zero for that fused combine.
 * x float [H] (16-byte aligned), logits float [n_experts], gate and up
 * [n_experts][I][H] (grid1: gate's codebook serves both, as in the mat-vec
 * with w_up; sign1: sc 4-byte aligned); H as the mat-vec accepts
 * for cols, I % 32 == 0; n_experts <= 1024, 1 <= top_k <= min(16,
 * n_experts).  Inputs finite.
 */
pq_status pq_moe_decode1_gate_up_ternary(const float *x, const float *logits, int32_t n_experts,
                                         int32_t top_k, const pq_ternary_w *gate,
                                         const pq_ternary_w *up, int32_t *topk_ids, float *topk_w,
                                         int32_t *expert_offsets, int32_t *sorted_assign,
                                         int32_t *active_experts, int32_t *n_active, int8_t *hq,
                                         float *hd, float *y_zero, pq_stream stream);
pq_status pq_moe_decode1_gate_up_grid1(const float *x, const float *logits, int32_t n_experts,
                                       int32_t top_k, const pq_grid1_w *gate, const pq_grid1_w *up,
                                       int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                                       int32_t *sorted_assign, int32_t *active_experts,
                                       int32_t *n_active, int8_t *hq, float *hd, float *y_zero,
                                       pq_stream stream);
pq_status pq_moe_decode1_gate_up_sign1(const float *x, const float *logits, int32_t n_experts,
                                       int32_t top_k, const pq_sign1_w *gate, const pq_sign1_w *up,
                                       int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                                       int32_t *sorted_assign, int32_t *active_experts,
                                       int32_t *n_active, int8_t *hq, float *hd, float *y_zero,
                                       pq_stream stream);

/*
 * Load-time check of a ternary tensor: *n_bad (a device int32) receives the
 * number of 2-bit codes equal to 3 in w->qs (an invalid code: the format has
 * 0 -> 0, 1 -> +1, 2 -> -1 only, and the kernels' output on code 3 is
 * unspecified).  One workgroup streams the whole plane (meant for load time,
 * not the hot path); qs 16-byte aligned.  A check of packed codes before the
 * fused path trusts them, as the pxq_llama README ("Updates - 2026-07-30")
 * does with its one-shot self-check of the 1-bit sign book.
 */
pq_status pq_validate_ternary(const pq_ternary_w *w, int32_t *n_bad, pq_stream stream);

/*
 * Known-answer self test of every kernel (the runtime self test the Parallax
 * 8B kappa article runs after building its runtime, "Which runtime is
 * needed"; the one-shot self-check the pxq_llama README, "Updates -
 * 2026-07-30", runs before trusting its fused 1-bit path) on tiny inputs
 * whose results follow in closed form: q8 blocks with max|x| = 127 (scale exactly 1), routing of
 * increasing logits, grouping of a fixed id list, the ternary, grid1 and
 * sub-scaled sign mat-vecs, the int8-MFMA tile in all three formats and the
 * prefill GEMM (grid1 and sub-scaled signs) with all-(+1) weights and unit
 * scales (each output is the exact sum of its activations), the fused prep
 * and combine.  Unlike
 * every other entry point it allocates device memory and synchronizes
 * `stream`; not for the hot path.  PQ_OK, PQ_ERR_SELFTEST on a wrong answer,
 * PQ_ERR_HIP on a runtime failure.
 */
pq_status pq_selftest(pq_stream stream);

/*
 * Which kernels an entry point of family `call` (PQ_CALL_*) launches for
 * weights of format `fmt` (PQ_FMT_*) with these sizes, as PQ_PLAN_* flags: the
 * same decision the entry point itself takes (the pages choose between a
 * mat-vec and a tiled kernel by batch size: Parakon Runtime README, "How it
 * works"; the pxq_llama README, "Updates - 2026-07-28", reports a decode
 * kernel that silently never ran at a large batch, which a test of the
 * dispatch catches).  `debug` != 0 plans a call with dbg != NULL.  Host only:
 * no HIP call, nothing enqueued.  Returns 0 when the call launches nothing
 * (n_tokens == 0) and -PQ_ERR_SHAPE / -PQ_ERR_UNSUPPORTED for arguments the
 * entry point rejects for their sizes alone.
 */
int32_t pq_plan(int32_t call, int32_t fmt, int32_t n_tokens, int32_t top_k, int32_t n_experts,
                int32_t rows, int32_t cols, int32_t epilogue, int32_t debug);

/*
 * Measurement aids, not on the hot path: the achievable rates of the device,
 * used as second denominators next to the nominal 8 TB/s HBM and 2.5 PFLOP/s
 * dense bf16 peaks when expert-kernel rates are quoted as roofline fractions.
 *
 * pq_peak_read: streams `bytes` (a multiple of 16, buf 16-byte aligned) of
 * device memory with 16-byte loads and discards them; `sink` is a device
 * uint32 [1024] the kernel may write (it never does for real data).
 *
 * pq_peak_mfma_bf16: `workgroups` workgroups of *waves_per_workgroup waves,
 * each wave issuing iters * (*chains) v_mfma_f32_16x16x32_bf16 on register
 * operands (16*16*32*2 flops each) and nothing else; `sink` is a device float
 * [1024] as above.  waves_per_workgroup and chains may be NULL.
 */
pq_status pq_peak_read(const void *buf, int64_t bytes, uint32_t *sink, pq_stream stream);
pq_status pq_peak_mfma_bf16(int32_t workgroups, int32_t iters, float *sink, int32_t *waves_per_workgroup,
                            int32_t *chains, pq_stream stream);

/* Human-readable name of a status code (static storage). */
const char *pq_status_str(pq_status status);

/* PQ_ABI_VERSION of the built library. */
int32_t pq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PQ_H */
