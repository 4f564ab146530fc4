// Grouped int8-MFMA tile kernel over packed 1-bit-class expert weights against
// q8 activations: the arithmetic of the decode mat-vec (per-32 int32 block
// sums, fp32 scale application) for experts that hold many assignments, as
// in prefill.  The pages switch large batches from the mat-vec to a tiled
// kernel on their own (Parakon Runtime README, "How it works"), and add an
// int8 dot-product prefill tile for cards without fast fp16 products
// (pxq_llama README, "Updates - 2026-07-19"); this kernel is such a tile on
// the matrix cores, fed q8 activations so that the block sums stay exact.
//
// One v_mfma_i32_16x16x32_i8 covers K = 32, exactly one q8 block: its int32
// results are the block sums sum_k w[n][k] * xq[t][k] of 16 weight rows x 16
// assignments, bit-exact for any order of the 32 products.  Then, in fp32,
//   blk[n][t] += xd[t][b] * isum      (8 blocks of a 256-weight scale block)
//   tot[n][t] += d[n][B] * blk[n][t]  (once per scale block),
// both as explicit fused multiply-adds, so every build of the kernel (with
// or without its debug outputs) rounds the same way.
//
// Work item: (expert, chunk of up to 64 of its assignments (32 for small
// batches), tile of 64 physical weight rows: 32 gate + 32 up rows for the
// SwiGLU epilogue, else 64 rows).  Wave w owns 16 of the 64 rows (the A
// operand) and all live 16-column assignment subtiles (the B operand).  The K loop runs over 256-weight
// slabs: each lane loads its own weight row's packed slab straight into
// registers one slab ahead, while the workgroup stages the chunk's q8
// activations and scales for the next slab into LDS.
//
// Operand layouts (lane l: r = l % 16, lane group g = l / 16; A row r and B
// column r carry the K slots 8g..8g+7; the result rows are 4g..4g+3 of
// column r):
//  - ternary: K slot j of lane group g is weight 4j + g of the block's first
//    16 and slot 4 + j weight 16 + 4j + g, i.e. code field g of each byte of
//    the block's two code dwords, so the A fragment is two byte lookups
//    (v_perm_b32) with no byte shuffling, and the activations are staged
//    byte-transposed to match;
//  - grid1: lane group g takes group g of the block (8 weights in natural
//    order): its 11-bit index selects one 8-byte codebook row in LDS, which
//    is exactly the A fragment;
//  - sub-scaled signs: lane group g takes weights 8g..8g+7 of the block as
//    int8 sign * sc (sc the 4-bit sub-scale of their 16-weight half), built
//    by two v_perm_b32 choosing byte by byte between sc and -sc, with the
//    selectors (the sign byte's bits as 0/1 bytes) from a 256-entry LDS
//    table; the MFMA block sums are then the sub-scaled sums, and the row's
//    anchor takes the place of the per-256 scale.
//
// Items are chosen on the device from the grouping (offsets / active): an
// expert takes part when it holds at least `heavy_min` assignments, so the
// decode mat-vec can take the others in a launch of its own.
// (Included by k_tile_q8.hip, which launches it, and by k_matvec.hip, whose
// skewed-decode launch runs the heavy experts' tile items in its first
// workgroups.)
#pragma once

#include <type_traits>

#include "pq_device.hpp"
#include "pq_internal.hpp"

namespace pqk {

namespace {

namespace tq8 {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kSub = 16;          // assignments per MFMA column subtile
constexpr int kSlabK = 256;       // weights per slab: one weight-scale block
constexpr int kSlabBlocks = kSlabK / 32;
constexpr int kRows = 64;         // physical weight rows per item, 16 per wave
// Chunks of up to 64 assignments (four column subtiles) at two waves per
// SIMD for large batches; of up to 32 at three waves per SIMD (fewer
// registers and LDS) when the batch is small and the few heavy experts'
// items are latency-bound.
constexpr int kSmallChunkMaxAssign = 2048;

template <int FMT>
struct TileFmt;
template <>
struct TileFmt<kTernary> {
    static constexpr int kWords = 4;   // 64 bytes of codes per row and slab
};
template <>
struct TileFmt<kGrid1> {
    static constexpr int kWords = 3;   // 32 bytes of qs, then 16 bytes of qh
};
template <>
struct TileFmt<kSign1> {
    static constexpr int kWords = 3;   // 32 sign bytes, then 8 sub-scale bytes
};
constexpr int kSignPatterns = 256;

// The kernel body for workgroup `bid` of `nblk` (its own launch, or the
// first workgroups of a launch shared with the decode mat-vec).
template <int FMT, int EPI, bool DBG, int TOK>
__device__ __forceinline__ void tile_q8_body(const ExpertArgs& p, int bid, int nblk) {
    constexpr int kTok = TOK;                 // assignments per item
    constexpr int kJMax = kTok / kSub;        // column subtiles
    // (column, block) pairs of a slab's activation staging per thread
    constexpr int kStagePairs = kTok * kSlabBlocks / kThreads;
    static_assert(kStagePairs * kThreads == kTok * kSlabBlocks, "staging covers every (column, block) pair once");
    constexpr int NMAT = (EPI == kEpiSwigluQ8) ? 2 : 1;
    constexpr int TR = kRows / NMAT;   // output rows per item
    constexpr int KW = TileFmt<FMT>::kWords;

    // B fragments of a slab: entry (column c, block q, lane group g) at
    // c * kXStride + 4q + g.  The pad of one entry per column shifts
    // consecutive columns by two banks, so a fragment read (16 columns, one
    // block and lane group) and the staging writes are free of bank
    // conflicts; block scales likewise at c * 9 + q.
    constexpr int kXStride = 4 * kSlabBlocks + 1;
    __shared__ uint2 s_x[2][kTok * kXStride];
    __shared__ float s_xd[2][kTok * (kSlabBlocks + 1)];
    __shared__ float s_d[2][kRows];
    // grid1: the codebook; sign1: per sign byte, its 8 bits as 0/1 bytes
    // (v_perm selectors between +sc and -sc)
    __shared__ uint2 s_grid[(FMT == kGrid1) ? kGridEntries : (FMT == kSign1) ? kSignPatterns : 1];
    __shared__ float s_gu[NMAT][(NMAT == 2) ? TR : 1][kTok + 1];
    __shared__ int s_pre[kMaxExperts + 1];   // first chunk number per slot
    // Small batches: per slot, expert << 21 | its first assignment (expert <
    // 1024, assignments <= 2^20), kept from the count pass so that an item's
    // routing costs no memory round trip (its items are short); a slot's
    // assignments end where the next slot's begin (experts in between hold
    // none), the last at the total.
    constexpr bool kSlotCache = kTok <= 32;
    __shared__ int s_sinfo[kSlotCache ? kMaxExperts + 1 : 1];
    static_assert(kMaxExperts <= 1024, "expert ids are packed in 10 bits");
    __shared__ int s_scan[kWaves + 1];
    __shared__ int s_asg[kTok];
    __shared__ int s_arow[kTok];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int rows = p.rows, cols = p.cols, KB = cols / kSlabK;
    const int n_active = load_uniform(p.n_active);
    const int hmin = p.heavy_min > 0 ? p.heavy_min : 1;

    if constexpr (FMT == kGrid1) {
        const uint4* src = reinterpret_cast<const uint4*>(p.grid);
        uint4* dst = reinterpret_cast<uint4*>(s_grid);
        for (int i = tid; i < kGridEntries / 2; i += kThreads) dst[i] = src[i];
    }
    if constexpr (FMT == kSign1) {
        if (tid < kSignPatterns) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lo |= ((tid >> j) & 1u) << (8 * j);
                hi |= ((tid >> (j + 4)) & 1u) << (8 * j);
            }
            s_grid[tid] = make_uint2(lo, hi);
        }
    }
    // Chunks of up to kTok assignments of the experts that take part,
    // numbered in slot order.
    int run = 0;
    for (int s0 = 0; s0 < n_active; s0 += kThreads) {
        const int s = s0 + tid;
        int nc = 0;
        if (s < n_active) {
            const int e = p.active[s];
            const int o0 = p.offsets[e], o1 = p.offsets[e + 1];
            if constexpr (kSlotCache) {
                s_sinfo[s] = (e << 21) | o0;
                if (s == n_active - 1) s_sinfo[n_active] = o1;
            }
            const int m = o1 - o0;
            nc = m >= hmin ? (m + kTok - 1) / kTok : 0;
        }
        const int ex = block_exclusive_scan(nc, s_scan);
        if (s < n_active) s_pre[s] = run + ex;
        if (tid == kThreads - 1) s_scan[kWaves] = run + ex + nc;
        __syncthreads();
        run = s_scan[kWaves];
        __syncthreads();
    }
    if (tid == 0) s_pre[n_active] = run;
    __syncthreads();   // codebook and chunk prefix visible

    const int tiles = (rows + TR - 1) / TR;
    const int n_items = run * tiles;
    const int64_t qs_row = (FMT == kTernary) ? cols / 4 : cols / 8;   // bytes
    const int64_t qh_row = cols / 32;   // grid1: uint16 qh; sign1: sub-scale bytes
    // weight scales per row: one per slab (sign1: one anchor per row)
    const int64_t d_row = (FMT == kSign1) ? 1 : cols / kSlabK;
    const int n_sub_row = cols / 32;

    // This lane's A row: physical row pr = 16 * wave + r of the item.
    const int pr_a = 16 * wave + r;
    const int mat_a = (NMAT == 2) ? (wave >> 1) : 0;   // uniform
    const int off_a = (NMAT == 2) ? (pr_a & 31) : pr_a;

    for (int item = bid; item < n_items; item += nblk) {
        const int c = item / tiles, tile = item % tiles;
        int lo = 0, hi = n_active - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_pre[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const int slot = __builtin_amdgcn_readfirstlane(lo);
        const int cbeg = (c - __builtin_amdgcn_readfirstlane(s_pre[slot])) * kTok;
        int e, beg, m;
        if constexpr (kSlotCache) {
            const int si = __builtin_amdgcn_readfirstlane(s_sinfo[slot]);
            e = si >> 21;
            beg = si & ((1 << 21) - 1);
            m = (__builtin_amdgcn_readfirstlane(s_sinfo[slot + 1]) & ((1 << 21) - 1)) - beg;
        } else {
            e = load_uniform(p.active + slot);
            beg = load_uniform(p.offsets + e);
            m = load_uniform(p.offsets + e + 1) - beg;
        }
        const int mcount = min(kTok, m - cbeg);
        const int jn = (mcount + kSub - 1) / kSub;   // live column subtiles, 1..4
        const int n0 = tile * TR;
        if (tid < kTok) {
            // columns past mcount repeat the last assignment and are never stored
            const int a = p.sorted[beg + cbeg + min(tid, mcount - 1)];
            s_asg[tid] = a;
            s_arow[tid] = p.act_by_token ? a / p.top_k : a;
        }
        __syncthreads();

        // ---- per-lane weight row (clamped past the end; never stored)
        const int na = min(n0 + off_a, rows - 1);
        const uint8_t* qsrow = (mat_a ? p.qs[1] : p.qs[0]) + (static_cast<int64_t>(e) * rows + na) * qs_row;
        const uint16_t* qhrow = nullptr;
        if constexpr (FMT == kGrid1)
            qhrow = (mat_a ? p.qh[1] : p.qh[0]) + (static_cast<int64_t>(e) * rows + na) * qh_row;
        const uint8_t* scrow = nullptr;
        if constexpr (FMT == kSign1)
            scrow = (mat_a ? p.sc[1] : p.sc[0]) + (static_cast<int64_t>(e) * rows + na) * qh_row;
        auto wload = [&](int sb, uint4 (&w)[KW]) {
            if constexpr (FMT == kTernary) {
                const uint4* src = reinterpret_cast<const uint4*>(qsrow + 64 * sb);
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = src[i];
            } else if constexpr (FMT == kSign1) {
                const uint4* src = reinterpret_cast<const uint4*>(qsrow + 32 * sb);
                w[0] = src[0];
                w[1] = src[1];
                const uint32_t* sc4 = reinterpret_cast<const uint32_t*>(scrow + 8 * sb);
                w[2] = make_uint4(sc4[0], sc4[1], 0u, 0u);
            } else {
                const uint4* src = reinterpret_cast<const uint4*>(qsrow + 32 * sb);
                w[0] = src[0];
                w[1] = src[1];
                w[2] = *reinterpret_cast<const uint4*>(qhrow + 8 * sb);
            }
        };

        // ---- staging of a slab: thread (column c, block q) for kStagePairs
        // (c, q) pairs moves the 32 activation bytes of block q and its scale; the
        // first 64 threads also move one weight scale
        uint4 xr[kStagePairs][2];
        float xdr[kStagePairs];
        uint32_t dr = 0;   // fp16 bits: converted only when stored, so that no
                           // instruction waits on the loads before the compute
        auto sload = [&](int sb) {
#pragma unroll
            for (int k = 0; k < kStagePairs; ++k) {
                const int pair = tid + kThreads * k;
                const int c = pair >> 3, q = pair & 7;
                const int64_t row = s_arow[c];
                const uint4* src = reinterpret_cast<const uint4*>(p.xq + row * cols + sb * kSlabK + q * 32);
                xr[k][0] = src[0];
                xr[k][1] = src[1];
                xdr[k] = p.xd[row * n_sub_row + sb * kSlabBlocks + q];
            }
            if (tid < kRows) {
                // (a select of the two scalar pointers: indexing p.d by a lane
                // value would load the pointer from the argument block and
                // wait for every load in flight)
                const uint16_t* dbase = (NMAT == 2 && tid >= 32) ? p.d[1] : p.d[0];
                const int nr = min(n0 + ((NMAT == 2) ? (tid & 31) : tid), rows - 1);
                dr = dbase[(static_cast<int64_t>(e) * rows + nr) * d_row + ((FMT == kSign1) ? 0 : sb)];
            }
        };
        auto sstore = [&](int sl) {
#pragma unroll
            for (int k = 0; k < kStagePairs; ++k) {
                const int pair = tid + kThreads * k;
                const int c = pair >> 3, q = pair & 7;
                uint2* dst = &s_x[sl][c * kXStride + 4 * q];
                const uint32_t lo[4] = {xr[k][0].x, xr[k][0].y, xr[k][0].z, xr[k][0].w};
                const uint32_t hi[4] = {xr[k][1].x, xr[k][1].y, xr[k][1].z, xr[k][1].w};
                if constexpr (FMT == kTernary) {
                    // dword s of the byte transpose of each 16-byte half holds
                    // the K slots of lane group s
                    uint32_t t0[4], t1[4];
                    transpose_bytes4(lo, t0);
                    transpose_bytes4(hi, t1);
#pragma unroll
                    for (int g2 = 0; g2 < 4; ++g2) dst[g2] = make_uint2(t0[g2], t1[g2]);
                } else {
                    dst[0] = make_uint2(lo[0], lo[1]);
                    dst[1] = make_uint2(lo[2], lo[3]);
                    dst[2] = make_uint2(hi[0], hi[1]);
                    dst[3] = make_uint2(hi[2], hi[3]);
                }
                s_xd[sl][c * (kSlabBlocks + 1) + q] = xdr[k];
            }
            if (tid < kRows) s_d[sl][tid] = half_bits_to_float(static_cast<uint16_t>(dr));
        };

        float tot[kJMax][4];
#pragma unroll
        for (int j = 0; j < kJMax; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[j][i] = 0.0f;

        // One slab, in two halves of 4 blocks: the A fragments of the half,
        // its 4 x JN MFMAs into their own accumulators, then their fp32
        // scaling (so the MFMAs issue back to back instead of each waiting
        // for its result).
        auto compute = [&](auto jn_c, int sl, const uint4 (&w)[KW], int sb) {
            constexpr int JN = decltype(jn_c)::value;
            uint32_t wv[4 * KW];
#pragma unroll
            for (int i = 0; i < KW; ++i) {
                wv[4 * i] = w[i].x;
                wv[4 * i + 1] = w[i].y;
                wv[4 * i + 2] = w[i].z;
                wv[4 * i + 3] = w[i].w;
            }
            float blk[JN][4];
#pragma unroll
            for (int j = 0; j < JN; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) blk[j][i] = 0.0f;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                v4i is[4][JN];
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int q = 4 * half + qq;
                    uint64_t afrag;
                    if constexpr (FMT == kTernary) {
                        const uint32_t lo = static_cast<uint32_t>(ternary_decode4((wv[2 * q] >> (2 * g)) & 0x03030303u));
                        const uint32_t hi = static_cast<uint32_t>(ternary_decode4((wv[2 * q + 1] >> (2 * g)) & 0x03030303u));
                        afrag = (static_cast<uint64_t>(hi) << 32) | lo;
                    } else if constexpr (FMT == kSign1) {
                        // weights 8g..8g+7 of block q as int8 (+-sc): the sign
                        // byte selects, byte by byte, sc or -sc of the
                        // 16-weight sub-block (sub-scale nibble g >> 1 of byte q)
                        const uint32_t sgn = (wv[q] >> (8 * g)) & 0xffu;
                        const uint32_t scb = (wv[8 + (q >> 2)] >> (8 * (q & 3))) & 0xffu;
                        const uint32_t sc = (scb >> (4 * (g >> 1))) & 15u;
                        const uint32_t pm = sc | (((0u - sc) & 0xffu) << 8);
                        const uint2 sel = s_grid[sgn];
                        const uint32_t lo = __builtin_amdgcn_perm(pm, pm, sel.x);
                        const uint32_t hi = __builtin_amdgcn_perm(pm, pm, sel.y);
                        afrag = (static_cast<uint64_t>(hi) << 32) | lo;
                    } else {
                        const uint32_t lo8 = (wv[q] >> (8 * g)) & 0xffu;
                        const uint32_t h16 = wv[8 + (q >> 1)] >> (16 * (q & 1));
                        const uint32_t hi3 = (h16 >> (3 * g)) & 7u;
                        const uint2 cb = s_grid[lo8 | (hi3 << 8)];
                        afrag = (static_cast<uint64_t>(cb.y) << 32) | cb.x;
                    }
#pragma unroll
                    for (int j = 0; j < JN; ++j) {
                        const uint2 bx = s_x[sl][(kSub * j + r) * kXStride + 4 * q + g];
                        const uint64_t bfrag = (static_cast<uint64_t>(bx.y) << 32) | bx.x;
                        is[qq][j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(
                            static_cast<long>(afrag), static_cast<long>(bfrag), v4i{0, 0, 0, 0}, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int q = 4 * half + qq;
#pragma unroll
                    for (int j = 0; j < JN; ++j) {
                        const float xdv = s_xd[sl][(kSub * j + r) * (kSlabBlocks + 1) + q];
#pragma unroll
                        for (int i = 0; i < 4; ++i) blk[j][i] = fmaf(xdv, static_cast<float>(is[qq][j][i]), blk[j][i]);
                        if constexpr (DBG) {
                            int32_t* dst = (NMAT == 2 && mat_a) ? p.dbg_isums[1] : p.dbg_isums[0];
                            const int col = kSub * j + r;
                            if (dst && col < mcount) {
                                const int a = s_asg[col];
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const int pr = 16 * wave + 4 * g + i;
                                    const int n = n0 + ((NMAT == 2) ? (pr & 31) : pr);
                                    if (n < rows)
                                        dst[(static_cast<int64_t>(a) * rows + n) * n_sub_row + sb * kSlabBlocks + q] =
                                            is[qq][j][i];
                                }
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float dsc = s_d[sl][16 * wave + 4 * g + i];
#pragma unroll
                for (int j = 0; j < JN; ++j) tot[j][i] = fmaf(dsc, blk[j][i], tot[j][i]);
            }
        };

        uint4 wc[KW], wn[KW];
        wload(0, wc);
        sload(0);
        sstore(0);
        __syncthreads();
        for (int sb = 0; sb < KB; ++sb) {
            const int sl = sb & 1;
            const bool more = sb + 1 < KB;
            if (more) {
                wload(sb + 1, wn);
                sload(sb + 1);
            }
            if constexpr (kJMax == 2) {
                if (jn == 1)
                    compute(std::integral_constant<int, 1>{}, sl, wc, sb);
                else
                    compute(std::integral_constant<int, 2>{}, sl, wc, sb);
            } else {
                switch (jn) {
                    case 1: compute(std::integral_constant<int, 1>{}, sl, wc, sb); break;
                    case 2: compute(std::integral_constant<int, 2>{}, sl, wc, sb); break;
                    case 3: compute(std::integral_constant<int, 3>{}, sl, wc, sb); break;
                    default: compute(std::integral_constant<int, 4>{}, sl, wc, sb); break;
                }
            }
            if (more) {
                sstore(sl ^ 1);
#pragma unroll
                for (int i = 0; i < KW; ++i) wc[i] = wn[i];
            }
            __syncthreads();
        }

        // ---- epilogues: lane holds physical rows 16*wave + 4g + i of
        // columns 16j + r
        if constexpr (EPI == kEpiSwigluQ8) {
#pragma unroll
            for (int j = 0; j < kJMax; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) s_gu[mat_a][16 * (wave & 1) + 4 * g + i][kSub * j + r] = tot[j][i];
            __syncthreads();
            // one 32-lane half per assignment column; lane = output row
            for (int c0 = 0; c0 < kTok; c0 += kThreads / 32) {
                const int col = c0 + (tid >> 5), i = tid & 31;
                const float gg = s_gu[0][i][col], uu = s_gu[1][i][col];
                const float h = gg / (1.0f + expf(-gg)) * uu;
                const float amax = half_wave_max(fabsf(h));
                const float dq = amax / 127.0f;
                if (col < mcount) {
                    const int a = s_asg[col];
                    const int64_t o = static_cast<int64_t>(a) * rows + n0 + i;
                    static_cast<int8_t*>(p.out0)[o] = static_cast<int8_t>(q8_value(h, dq));
                    if (i == 0)
                        static_cast<float*>(p.out1)[static_cast<int64_t>(a) * (rows / 32) + n0 / 32] = dq;
                    if constexpr (DBG) {
                        if (p.dbg_g) p.dbg_g[o] = gg;
                        if (p.dbg_u) p.dbg_u[o] = uu;
                        if (p.dbg_h) p.dbg_h[o] = h;
                    }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kJMax; ++j) {
                const int col = kSub * j + r;
                if (j < jn && col < mcount) {
                    const int a = s_asg[col];
                    const float wsel = (EPI == kEpiF32Combine) ? static_cast<const float*>(p.out1)[a] : 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int n = n0 + 16 * wave + 4 * g + i;
                        if (n < rows) {
                            if constexpr (EPI == kEpiF32) {
                                static_cast<float*>(p.out0)[static_cast<int64_t>(a) * rows + n] = tot[j][i];
                            } else {
                                atomicAdd(static_cast<float*>(p.out0) + static_cast<int64_t>(a / p.top_k) * rows + n,
                                          wsel * tot[j][i]);
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();   // s_asg, s_arow and the LDS slots are reused by the next item
    }
}

// Workgroups of a launch over the items of the experts with at least
// a.heavy_min assignments, in chunks of TOK: an upper bound of the items,
// capped at four workgroups per compute unit.
template <int EPI, int TOK>
int64_t tile_grid(const ExpertArgs& a) {
    constexpr int TR = kRows / ((EPI == kEpiSwigluQ8) ? 2 : 1);
    // sum over the taking-part experts of ceil(m / TOK) <= A / TOK + (number of such experts)
    const int64_t A = static_cast<int64_t>(a.n_tokens) * a.top_k;
    const int64_t hmin = a.heavy_min > 0 ? a.heavy_min : 1;
    int64_t heavy = A / hmin;
    if (heavy > a.n_experts) heavy = a.n_experts;
    const int64_t chunks = A / TOK + heavy + 1;
    const int64_t items = chunks * ((a.rows + TR - 1) / TR);
    const int64_t cap = static_cast<int64_t>(cu_count()) * 4;
    int64_t grid = items < cap ? items : cap;
    return grid < 1 ? 1 : grid;
}

}  // namespace tq8

}  // namespace

}  // namespace pqk
