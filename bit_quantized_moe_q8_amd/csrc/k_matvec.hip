// Grouped decode mat-vec over packed 1-bit-class expert weights against q8
// activations (Parakon Runtime README, "How it works": fused mat-vec kernels
// read the quantized blocks directly from device memory and accumulate
// against int8 activations with a 4-way int8 dot product; nothing is ever
// dequantized to memory).
//
// Work decomposition.  A work item is (active expert, tile of 32 output rows)
// and, for skewed routing, also a group of up to MT of the expert's
// assignments (so a heavily loaded expert is spread over many workgroups
// instead of serialising in one).  Items are numbered from the routing on the
// device; the launch is persistent (grid-stride over items) and never needs
// the routing on the host.  With the SwiGLU epilogue a tile holds the 32 gate
// rows and the 32 up rows of the same outputs (gate/up fusion: pxq_llama
// README, "Updates - 2026-07-28"), so h = silu(g)*u and its q8 block of 32
// are formed in the same workgroup.
//
// Lane mapping.  A row is split into LPR chunks of 16 packed bytes (ternary:
// 64 weights = 2 int8 blocks of 32; grid1: 16 groups = 128 weights = 4 blocks
// of 32).  Lane l of a wave owns chunk l % LS of row-slot l / LS for every
// row it touches, so its slice of the activation row is loaded once into
// registers and reused for all rows (the pages stage the activation vector
// on chip for the same reason: pxq_llama README, "Updates - 2026-07-28",
// 2D decode driver).  Row slots are LPR rounded up to a power of two lanes
// wide, so the partial row sums reduce with DPP lane moves (quad_perm, row
// mirrors, row_bcast) instead of LDS permutes.
//
// Streaming.  The rows of a tile are visited in row iterations (one row slot
// per wave each); the weight loads run kDepth iterations ahead of the
// arithmetic (a register ring), so every wave keeps several 16-byte loads per
// lane in flight while it computes, and the grid1 codebook reads of a row are
// all issued before their dot products.  A tile is 32, 64 or 128 output rows,
// chosen at launch so that short rows still give a long stream per item while
// leaving enough items to fill the chip; each workgroup of the persistent
// grid fetches the next item's routing metadata while the current item
// streams.
//
// Ternary arithmetic.  A dword P of 16 two-bit codes gives, for s = 0..3, the
// selector (P >> 2s) & 0x03030303 whose byte b is the code of weight 4b+s;
// one v_perm_b32 turns it into four int8 weights (0, +1, -1), and one
// v_dot4_i32_i8 against the activation bytes 4b+s (a byte transpose done
// once per activation load) accumulates four products.  The two 32-weight
// block sums are exact int32.
//
// Grid1 arithmetic.  The 2048 x 8 int8 codebook (16 KB) sits in LDS; each
// group's 11-bit index selects one 8-byte row (ds_read_b64) and two
// v_dot4_i32_i8 accumulate its products.
//
// Sub-scaled sign arithmetic (1-bit sign codes, a 4-bit sub-scale per 16
// weights and one fp16 anchor per row: pxq_llama README, "What's PXQ?",
// PXQ1).  Each sign byte selects one 8-byte row of the 256 +-1 patterns,
// built in LDS at kernel start; two v_dot4_i32_i8 per byte give the +-1 sum
// of 8 weights, and the two 16-weight sums of a q8 block combine with their
// sub-scales in integer arithmetic (sc_lo * s_lo + sc_hi * s_hi, exact), so
// the per-block int32 sums and everything after them are those of the other
// formats, with the row's anchor as the scale of every block.  The sub-scale
// multiply-add is the second scale step the pages measure against
// single-scale blocks.
//
// Scale application in fp32: partial = d_w * (sum over the lane's blocks of
// xd * isum), then the cross-lane sum.
#include "pq_device.hpp"
#include "pq_internal.hpp"
#include "k_tile_q8.hpp"

namespace pqk {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTileRows = 32;      // q8 block of the SwiGLU epilogue; tiles are 1, 2 or 4 of these
constexpr int kMaxTileShift = 2;
constexpr int kDepth = 4;          // row iterations of weight loads in flight per wave

template <int FMT>
struct FmtInfo;
template <>
struct FmtInfo<kTernary> {
    static constexpr int kChunkWeights = 64;  // 16 bytes of 2-bit codes
    static constexpr int kSubs = 2;           // int8 blocks of 32 per chunk
};
template <>
struct FmtInfo<kGrid1> {
    static constexpr int kChunkWeights = 128;  // 16 group indices (low bytes)
    static constexpr int kSubs = 4;
};
template <>
struct FmtInfo<kSign1> {
    static constexpr int kChunkWeights = 128;  // 16 sign bytes
    static constexpr int kSubs = 4;
};
constexpr int kSignPatterns = 256;

// One lane's packed weights of one row iteration.
struct WRow {
    uint4 q;      // 16 bytes of qs
    uint2 h;      // grid1: the 4 qh words of the chunk; sign1: h.x = 4 sub-scale bytes
    uint32_t d;   // fp16 scale bits
};

// Rows per workgroup row iteration for LPR chunks per row.
template <int LPR>
struct RowGeom {
    static constexpr int LS = (LPR <= 2) ? 2 : (LPR <= 4) ? 4 : (LPR <= 8) ? 8 : (LPR <= 16) ? 16
                            : (LPR <= 32) ? 32 : 64;
    static constexpr int ROWS_IT = kWaves * (kWave / LS);
};
// Tall-tile shift: the largest TS <= kMaxTileShift with at most 2*kDepth row
// iterations per tile (0 when a 32-row tile already has more).
template <int LPR, int NMAT>
constexpr int tall_shift() {
    int ts = 0;
    while (ts < kMaxTileShift &&
           ((kTileRows << (ts + 1)) * NMAT + RowGeom<LPR>::ROWS_IT - 1) / RowGeom<LPR>::ROWS_IT <= 2 * kDepth)
        ++ts;
    return ts;
}

// Waves per SIMD asked of the single-assignment grid1 variants: three
// (<= 168 VGPRs, a few spilled) measured ~8% faster on the grid1 decode
// shapes than the two their natural 171 VGPRs allow; four spills too much.
constexpr int kGrid1WavesPerSimd = 3;

// The kernel body for workgroup `bid` of `nblk` (the grouped mat-vec's own
// launch, or the workgroups after the tile's in the skewed-decode launch),
// with DEPTH row iterations of weight loads in flight per wave.
template <int FMT, int LPR, int MT, int EPI, bool SPLIT, int TS, bool DBG, int DEPTH>
__device__ __forceinline__ void matvec_body(const ExpertArgs& p, int bid, int nblk) {
    using FI = FmtInfo<FMT>;
    constexpr int LS = RowGeom<LPR>::LS;
    constexpr int RPW = kWave / LS;               // row slots per wave
    constexpr int ROWS_IT = kWaves * RPW;         // rows per workgroup iteration
    constexpr int NMAT = (EPI == kEpiSwigluQ8) ? 2 : 1;
    constexpr int TR = kTileRows << TS;                 // output rows per tile
    constexpr int P = TR * NMAT;                        // physical rows per tile
    constexpr int ITERS = (P + ROWS_IT - 1) / ROWS_IT;  // row iterations per tile
    constexpr int D = ITERS < DEPTH ? ITERS : DEPTH;
    constexpr int SUBS = FI::kSubs;
    constexpr int ACT_DW = FI::kChunkWeights / 4;  // activation dwords per chunk

    __shared__ uint2 s_grid[(FMT == kGrid1) ? kGridEntries : (FMT == kSign1) ? kSignPatterns : 1];
    __shared__ float s_gu[NMAT][MT][TR];
    __shared__ int s_apre[SPLIT ? kMaxExperts + 1 : 1];   // first group number per slot
    // SPLIT: per slot, expert << 21 | its first assignment (expert < 1024,
    // assignments <= 2^20), kept from the count pass so that an item's
    // routing costs no memory round trip; a slot's assignments end where the
    // next slot's begin (experts in between hold none), the last at the total
    __shared__ int s_sinfo[SPLIT ? kMaxExperts + 1 : 1];
    static_assert(kMaxExperts <= 1024, "expert ids are packed in 10 bits");
    __shared__ int s_scan[kWaves + 1];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int slot_row = lane / LS, chunk = lane % LS;
    const bool lane_on = chunk < LPR;

    const int rows = p.rows, cols = p.cols;
    const int tiles = (rows + TR - 1) / TR;
    const int n_active = load_uniform(p.n_active);

    if constexpr (FMT == kGrid1) {
        const uint4* src = reinterpret_cast<const uint4*>(p.grid);
        uint4* dst = reinterpret_cast<uint4*>(s_grid);
        for (int i = tid; i < kGridEntries / 2; i += kThreads) dst[i] = src[i];
    }
    if constexpr (FMT == kSign1) {
        // pattern i: byte j is -1 where bit j of i is set, else +1
        for (int i = tid; i < kSignPatterns; i += kThreads) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lo |= (((i >> j) & 1) ? 0xFFu : 0x01u) << (8 * j);
                hi |= (((i >> (j + 4)) & 1) ? 0xFFu : 0x01u) << (8 * j);
            }
            s_grid[i] = make_uint2(lo, hi);
        }
    }

    // Item count.  SPLIT: slot s owns ceil(m_s / MT) assignment groups,
    // numbered from s_apre[s]; items are (group, tile), tile fastest.
    int n_groups = n_active;
    if constexpr (SPLIT) {
        int run = 0;
        for (int s0 = 0; s0 < n_active; s0 += kThreads) {
            const int s = s0 + tid;
            int na = 0;
            if (s < n_active) {
                const int e = p.active[s];
                const int o0 = p.offsets[e], o1 = p.offsets[e + 1];
                const int cnt = o1 - o0;
                s_sinfo[s] = (e << 21) | o0;
                if (s == n_active - 1) s_sinfo[n_active] = o1;
                // experts left to the int8-MFMA tile kernel get no groups
                na = (p.heavy_min > 0 && cnt >= p.heavy_min) ? 0 : (cnt + MT - 1) / MT;
            }
            const int ex = block_exclusive_scan(na, s_scan);
            if (s < n_active) s_apre[s] = run + ex;
            if (tid == kThreads - 1) s_scan[kWaves] = run + ex + na;
            __syncthreads();
            run = s_scan[kWaves];
            __syncthreads();
        }
        if (tid == 0) s_apre[n_active] = run;
        n_groups = run;
    }
    __syncthreads();   // codebook and group prefix visible
    const int n_items = n_groups * tiles;

    const int64_t qs_row_bytes = (FMT == kTernary) ? cols / 4 : cols / 8;
    const int64_t qh_row = cols / 32;                      // grid1 qh words; sign1 sub-scale bytes
    const int64_t d_row = (FMT == kSign1) ? 1 : cols / 256;
    const int64_t qs_e = static_cast<int64_t>(rows) * qs_row_bytes;
    const int64_t qh_e = static_cast<int64_t>(rows) * qh_row;
    const int64_t d_e = static_cast<int64_t>(rows) * d_row;
    const int n_sub_row = cols / 32;

    // Rows of iteration it: the wave's RPW row slots never straddle the
    // gate/up boundary (RPW divides 32), so the matrix index is wave-uniform
    // and the weight base pointers stay scalar.  Iterations past the tile
    // (it >= NIT, only in the prefetch of short tiles) land on rows of the
    // tile again, or on clamped rows, and are never consumed.
    const int wrow0 = __builtin_amdgcn_readfirstlane(wave) * RPW;
    auto row_of = [&](int it, int n0, int& mat, int& n, bool& rok) {
        const int pr0 = it * ROWS_IT + wrow0;   // uniform
        mat = (NMAT == 2) ? (pr0 / TR) : 0;
        n = n0 + (pr0 & (TR - 1)) + slot_row;
        rok = pr0 + slot_row < P && n < rows;
    };
    auto load_row = [&](int e, int n0, int it) -> WRow {
        int mat, n;
        bool rok;
        row_of(it, n0, mat, n, rok);
        // Branch-free: idle lanes and rows past the end load a valid
        // (clamped) location whose result is never used, so the loads of
        // all iterations can be in flight together.
        (void)rok;
        const int nc = n < rows ? n : rows - 1;
        const int cc = lane_on ? chunk : LPR - 1;
        WRow w;
        // per-expert bases are uniform; lane offsets fit in 32 bits
        const uint8_t* qsb = ((NMAT == 2 && mat == 1) ? p.qs[1] : p.qs[0]) + e * qs_e;
        const uint16_t* db = ((NMAT == 2 && mat == 1) ? p.d[1] : p.d[0]) + e * d_e;
        w.q = *reinterpret_cast<const uint4*>(
            qsb + static_cast<uint32_t>(nc * static_cast<int>(qs_row_bytes) + cc * 16));
        if constexpr (FMT == kGrid1) {
            const uint16_t* qhb = ((NMAT == 2 && mat == 1) ? p.qh[1] : p.qh[0]) + e * qh_e;
            w.h = *reinterpret_cast<const uint2*>(
                qhb + static_cast<uint32_t>(nc * static_cast<int>(qh_row) + cc * 4));
            w.d = db[static_cast<uint32_t>(nc * static_cast<int>(d_row) + cc / 2)];
        } else if constexpr (FMT == kSign1) {
            const uint8_t* scb = ((NMAT == 2 && mat == 1) ? p.sc[1] : p.sc[0]) + e * qh_e;
            w.h = make_uint2(*reinterpret_cast<const uint32_t*>(
                                 scb + static_cast<uint32_t>(nc * static_cast<int>(qh_row) + cc * 4)), 0u);
            w.d = db[static_cast<uint32_t>(nc)];
        } else {
            w.h = make_uint2(0, 0);
            w.d = db[static_cast<uint32_t>(nc * static_cast<int>(d_row) + cc / 4)];
        }
        return w;
    };

    // Uniform metadata of an item, read with scalar loads (the routing arrays
    // are read-only here); the next item's is fetched while the current
    // item's weight loads are in flight.
    struct Meta {
        int e, tile, beg, m, base;
        int asg[MT];
    };
    auto fetch_meta = [&](int item, Meta& mt) {
        const int grp = item / tiles;
        mt.tile = item % tiles;
        int slot = grp, g = 0;
        if constexpr (SPLIT) {
            // last slot whose first group is <= grp
            int lo = 0, hi = n_active - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_apre[mid] <= grp) lo = mid; else hi = mid - 1;
            }
            slot = __builtin_amdgcn_readfirstlane(lo);
            g = __builtin_amdgcn_readfirstlane(grp - s_apre[lo]);
            const int si = __builtin_amdgcn_readfirstlane(s_sinfo[slot]);
            mt.e = si >> 21;
            mt.beg = si & ((1 << 21) - 1);
            mt.m = (__builtin_amdgcn_readfirstlane(s_sinfo[slot + 1]) & ((1 << 21) - 1)) - mt.beg;
        } else {
            mt.e = load_uniform(p.active + slot);
            mt.beg = load_uniform(p.offsets + mt.e);
            mt.m = load_uniform(p.offsets + mt.e + 1) - mt.beg;
        }
        mt.base = SPLIT ? g * MT : 0;
        const int mc = min(MT, mt.m - mt.base);
#pragma unroll
        for (int j = 0; j < MT; ++j) mt.asg[j] = load_uniform(p.sorted + mt.beg + mt.base + (j < mc ? j : mc - 1));
    };

    Meta cur;
    if (bid < n_items) fetch_meta(bid, cur);
    for (int item = bid; item < n_items; item += nblk) {
        const int e = cur.e, tile = cur.tile, beg = cur.beg, m = cur.m;
        const int n0 = tile * TR;
        int base = cur.base;
        int asg[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) asg[j] = cur.asg[j];

        WRow buf[D];
#pragma unroll
        for (int i = 0; i < D; ++i) buf[i] = load_row(e, n0, i);

        const int next_item = item + nblk;
        Meta nxt = cur;
        bool first_pass = true;
        for (;;) {
            const int mcount = min(MT, m - base);
            // ---- activation slices of up to MT assignments.  Rows past
            // mcount repeat the last assignment (never stored) and idle lanes
            // read chunk LPR-1, so all loads are issued before any is used.
            const int cc = lane_on ? chunk : LPR - 1;
            uint4 raw[MT][ACT_DW / 4];
            float xs[MT][SUBS];
#pragma unroll
            for (int j = 0; j < MT; ++j) {
                const int r = p.act_by_token ? asg[j] / p.top_k : asg[j];
                const uint4* xa = reinterpret_cast<const uint4*>(
                    p.xq + static_cast<int64_t>(r) * cols + cc * FI::kChunkWeights);
#pragma unroll
                for (int v = 0; v < ACT_DW / 4; ++v) raw[j][v] = xa[v];
                const float* xdp = p.xd + static_cast<int64_t>(r) * n_sub_row + cc * SUBS;
#pragma unroll
                for (int s = 0; s < SUBS; ++s) xs[j][s] = xdp[s];
            }
            if (first_pass) {
                if (next_item < n_items) fetch_meta(next_item, nxt);
                first_pass = false;
            }
            // combine weights of the pass's assignments
            float wsel[MT];
#pragma unroll
            for (int j = 0; j < MT; ++j)
                wsel[j] = (EPI == kEpiF32Combine) ? load_uniform(static_cast<const float*>(p.out1) + asg[j]) : 0.0f;
            uint32_t act[MT][ACT_DW];
#pragma unroll
            for (int j = 0; j < MT; ++j) {
#pragma unroll
                for (int v = 0; v < ACT_DW / 4; ++v) {
                    uint32_t qq[4] = {raw[j][v].x, raw[j][v].y, raw[j][v].z, raw[j][v].w};
                    if constexpr (FMT == kTernary) {
                        uint32_t t[4];
                        transpose_bytes4(qq, t);
#pragma unroll
                        for (int s = 0; s < 4; ++s) act[j][4 * v + s] = t[s];
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; ++s) act[j][4 * v + s] = qq[s];
                    }
                }
            }

#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const WRow cur = buf[it % D];
                if (it + D < ITERS) buf[it % D] = load_row(e, n0, it + D);
                int mat, n;
                bool rok;
                row_of(it, n0, mat, n, rok);

                // ---- integer block sums of the MT activation rows
                int isum[MT][SUBS];
#pragma unroll
                for (int j = 0; j < MT; ++j)
#pragma unroll
                    for (int s = 0; s < SUBS; ++s) isum[j][s] = 0;
                const uint32_t wv[4] = {cur.q.x, cur.q.y, cur.q.z, cur.q.w};
                if constexpr (FMT == kTernary) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        int wdec[4];
                        ternary_decode16(wv[i], wdec);
#pragma unroll
                        for (int s = 0; s < 4; ++s)
#pragma unroll
                            for (int j = 0; j < MT; ++j)
                                isum[j][i >> 1] = dot4(wdec[s], static_cast<int>(act[j][4 * i + s]),
                                                       isum[j][i >> 1]);
                    }
                } else if constexpr (FMT == kSign1) {
                    // per 16 weights: the +-1 sum (two sign bytes), then
                    // times its sub-scale into the q8 block's sum
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        uint2 pat[8];
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int gi = 8 * hf + q;
                            pat[q] = s_grid[(wv[gi >> 2] >> (8 * (gi & 3))) & 0xffu];
                        }
#pragma unroll
                        for (int sub = 0; sub < 4; ++sub) {   // 16-weight blocks of this half
                            const int sb16 = 4 * hf + sub;     // 0..7 in the chunk
                            const uint32_t scv = (cur.h.x >> (4 * sb16)) & 15u;
#pragma unroll
                            for (int j = 0; j < MT; ++j) {
                                int s16 = 0;
#pragma unroll
                                for (int q = 2 * sub; q < 2 * sub + 2; ++q) {
                                    const int gi = 8 * hf + q;
                                    s16 = dot4(static_cast<int>(pat[q].x), static_cast<int>(act[j][2 * gi]), s16);
                                    s16 = dot4(static_cast<int>(pat[q].y), static_cast<int>(act[j][2 * gi + 1]), s16);
                                }
                                isum[j][sb16 >> 1] += static_cast<int>(scv) * s16;
                            }
                        }
                    }
                } else {
                    const uint32_t hv[2] = {cur.h.x, cur.h.y};
                    // two halves of 8 groups: all codebook reads of a half,
                    // then its dot products
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        uint2 cb[8];
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int gi = 8 * hf + q;
                            const uint32_t lo = (wv[gi >> 2] >> (8 * (gi & 3))) & 0xffu;
                            const uint32_t hw = hv[gi >> 3] >> (16 * ((gi >> 2) & 1));
                            const uint32_t hi = (hw >> (3 * (gi & 3))) & 7u;
                            cb[q] = s_grid[lo | (hi << 8)];
                        }
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int gi = 8 * hf + q;
#pragma unroll
                            for (int j = 0; j < MT; ++j) {
                                int acc = isum[j][gi >> 2];
                                acc = dot4(static_cast<int>(cb[q].x), static_cast<int>(act[j][2 * gi]), acc);
                                acc = dot4(static_cast<int>(cb[q].y), static_cast<int>(act[j][2 * gi + 1]), acc);
                                isum[j][gi >> 2] = acc;
                            }
                        }
                    }
                }

                // ---- fp32 scale application and the sum over the row slot
                const float dw = half_bits_to_float(static_cast<uint16_t>(cur.d));
                float part[MT];
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    float f = 0.0f;
#pragma unroll
                    for (int s = 0; s < SUBS; ++s) f += xs[j][s] * static_cast<float>(isum[j][s]);
                    part[j] = seg_sum<LS>(lane_on ? mul_rounded(dw, f) : 0.0f);
                    if constexpr (DBG) {
                        int32_t* dst = p.dbg_isums[mat];
                        if (dst && lane_on && rok && j < mcount) {
                            const int64_t o = (static_cast<int64_t>(asg[j]) * rows + n) * n_sub_row +
                                              chunk * SUBS;
#pragma unroll
                            for (int s = 0; s < SUBS; ++s) dst[o + s] = isum[j][s];
                        }
                    }
                }
                // the segment sum sits in the last lane of each row slot
                if (rok && chunk == LS - 1) {
                    if constexpr (EPI == kEpiF32) {
                        float* out = static_cast<float*>(p.out0);
#pragma unroll
                        for (int j = 0; j < MT; ++j)
                            if (j < mcount) out[static_cast<int64_t>(asg[j]) * rows + n] = part[j];
                    } else if constexpr (EPI == kEpiF32Combine) {
                        float* y = static_cast<float*>(p.out0);
#pragma unroll
                        for (int j = 0; j < MT; ++j)
                            if (j < mcount)
                                atomicAdd(y + static_cast<int64_t>(asg[j] / p.top_k) * rows + n, wsel[j] * part[j]);
                    } else {
#pragma unroll
                        for (int j = 0; j < MT; ++j) s_gu[mat][j][n - n0] = part[j];
                    }
                }
            }

            // ---- SwiGLU + q8 epilogue: one 32-lane half per (assignment,
            // block of 32 outputs); every lane takes part in each round so the
            // half-wave max sees whole halves
            if constexpr (EPI == kEpiSwigluQ8) {
                __syncthreads();
                constexpr int npairs = MT << TS;
                for (int r0 = 0; r0 < npairs; r0 += kThreads / 32) {
                    const int pi = r0 + (tid >> 5), i = tid & 31;
                    const bool pv = pi < npairs;
                    const int j = pv ? (pi >> TS) : 0, blk = pv ? (pi & ((1 << TS) - 1)) : 0;
                    const float gg = pv ? s_gu[0][j][blk * 32 + i] : 0.0f;
                    const float uu = pv ? s_gu[1][j][blk * 32 + i] : 0.0f;
                    const float h = gg / (1.0f + expf(-gg)) * uu;
                    const float amax = half_wave_max(fabsf(h));
                    const float dq = amax / 127.0f;
                    const int nb = n0 + blk * 32;
                    if (pv && j < mcount && nb < rows) {
                        const int a = p.sorted[beg + base + j];   // j varies by lane here
                        const int64_t o = static_cast<int64_t>(a) * rows + nb + i;
                        static_cast<int8_t*>(p.out0)[o] = static_cast<int8_t>(q8_value(h, dq));
                        if (i == 0)
                            static_cast<float*>(p.out1)[static_cast<int64_t>(a) * (rows / kTileRows) +
                                                        nb / kTileRows] = dq;
                        if constexpr (DBG) {
                            if (p.dbg_g) p.dbg_g[o] = gg;
                            if (p.dbg_u) p.dbg_u[o] = uu;
                            if (p.dbg_h) p.dbg_h[o] = h;
                        }
                    }
                }
                __syncthreads();
            }

            base += MT;
            if (SPLIT || base >= m) break;
            // another pass over the same tile (weights come back from cache)
            const int mc = min(MT, m - base);
#pragma unroll
            for (int j = 0; j < MT; ++j) asg[j] = load_uniform(p.sorted + beg + base + (j < mc ? j : mc - 1));
#pragma unroll
            for (int i = 0; i < D; ++i) buf[i] = load_row(e, n0, i);
        }
        cur = nxt;
    }
}

template <int FMT, int LPR, int MT, int EPI, bool SPLIT, int TS, bool DBG>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu((FMT != kTernary && MT == 1 && !DBG) ? kGrid1WavesPerSimd : 1)))
void k_matvec(ExpertArgs p) {
    matvec_body<FMT, LPR, MT, EPI, SPLIT, TS, DBG, kDepth>(p, blockIdx.x, gridDim.x);
}

// Skewed decode batches (ternary): the heavy experts' int8-MFMA tile items
// (chunks of up to 32 assignments) in the first n_tile workgroups and the
// other experts' mat-vec items (pairs of assignments) in the rest, one launch
// instead of two back to back, so the tile's few long item chains run beside
// the mat-vec stream.  The tile's registers set the occupancy (three waves
// per SIMD instead of the mat-vec's five; twice the weight loads in flight
// per mat-vec wave measured no faster).

template <int LPR, int EPI, int TS, bool DBG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(DBG ? 1 : 3)))
void k_matvec_mixed(ExpertArgs p, int n_tile) {
    static_assert(kThreads == tq8::kThreads, "one workgroup shape for both parts");
    if (static_cast<int>(blockIdx.x) < n_tile)
        tq8::tile_q8_body<kTernary, EPI, DBG, 32>(p, blockIdx.x, n_tile);
    else
        matvec_body<kTernary, LPR, 2, EPI, true, TS, DBG, kDepth>(p, blockIdx.x - n_tile,
                                                                         gridDim.x - n_tile);
}

template <int FMT, int LPR, int MT, int EPI, bool SPLIT, int TS, bool DBG>
hipError_t launch_one(const ExpertArgs& a, int64_t groups, hipStream_t s) {
    auto kernel = k_matvec<FMT, LPR, MT, EPI, SPLIT, TS, DBG>;
    // Persistent grid of up to 8 workgroups per CU (more than are resident:
    // a finishing workgroup's slot is refilled by the dispatcher, which
    // measured faster than exactly the resident count or one item each).
    const int tr = kTileRows << TS;
    const int64_t max_items = groups * ((a.rows + tr - 1) / tr);
    const int64_t cap = static_cast<int64_t>(cu_count()) * 8;
    int64_t grid = max_items < cap ? max_items : cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int FMT, int LPR, int MT, int EPI, bool SPLIT, bool DBG>
hipError_t launch_ts(const ExpertArgs& a, hipStream_t s) {
    constexpr int NMAT = (EPI == kEpiSwigluQ8) ? 2 : 1;
    constexpr int TALL = tall_shift<LPR, NMAT>();
    // Upper bound of the work-item groups: every slot active, or the
    // assignment groups (sum over slots of ceil(m / MT) <= A / MT + slots).
    const int64_t A = static_cast<int64_t>(a.n_tokens) * a.top_k;
    const int64_t slots = A < a.n_experts ? A : a.n_experts;
    const int64_t groups = SPLIT ? (A + MT - 1) / MT + slots : slots;
    // Tall tiles (longer streams per item) only when they still leave a few
    // items per CU.
    if constexpr (TALL > 0) {
        const int tr = kTileRows << TALL;
        if (groups * ((a.rows + tr - 1) / tr) >= 4 * static_cast<int64_t>(cu_count()))
            return launch_one<FMT, LPR, MT, EPI, SPLIT, TALL, DBG>(a, groups, s);
    }
    return launch_one<FMT, LPR, MT, EPI, SPLIT, 0, DBG>(a, groups, s);
}

template <int FMT, int LPR, int MT, int EPI, bool SPLIT>
hipError_t launch_dbg(const ExpertArgs& a, hipStream_t s) {
    return a.debug ? launch_ts<FMT, LPR, MT, EPI, SPLIT, true>(a, s)
                   : launch_ts<FMT, LPR, MT, EPI, SPLIT, false>(a, s);
}

template <int FMT, int LPR, int MT, bool SPLIT>
hipError_t launch_epi(Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (epi == kEpiF32) return launch_dbg<FMT, LPR, MT, kEpiF32, SPLIT>(a, s);
    if (epi == kEpiF32Combine) return launch_dbg<FMT, LPR, MT, kEpiF32Combine, SPLIT>(a, s);
    if (epi == kEpiSwigluQ8) return launch_dbg<FMT, LPR, MT, kEpiSwigluQ8, SPLIT>(a, s);
    return hipErrorInvalidValue;
}

template <int FMT, int LPR>
hipError_t launch_mt(Epi epi, const ExpertArgs& a, bool pairs, hipStream_t s) {
    // One token: every expert sees one activation row.  Up to one assignment
    // per expert on average: pairs (single rows for grid1 and sign1, whose
    // table lookups already hold more registers), passes repeated for the rare
    // heavier expert.  Otherwise (`pairs`, PQ_PLAN_MATVEC_PAIRS) pairs of
    // assignments, each its own work item (measured faster than groups of
    // four or eight on the skewed 64-token decode: fewer idle dot products
    // for the many one-assignment experts).
    if (a.n_tokens <= 1) return launch_epi<FMT, LPR, 1, false>(epi, a, s);
    constexpr int kMtPair = (FMT == kTernary) ? 2 : 1;
    if (!pairs) return launch_epi<FMT, LPR, kMtPair, false>(epi, a, s);
    return launch_epi<FMT, LPR, 2, true>(epi, a, s);
}

template <int FMT>
hipError_t launch_fmt(Epi epi, const ExpertArgs& a, bool pairs, hipStream_t s) {
    switch (a.cols / FmtInfo<FMT>::kChunkWeights) {
        case 2: return launch_mt<FMT, 2>(epi, a, pairs, s);
        case 4: return launch_mt<FMT, 4>(epi, a, pairs, s);
        case 8: return launch_mt<FMT, 8>(epi, a, pairs, s);
        case 12: return launch_mt<FMT, 12>(epi, a, pairs, s);
        case 16: return launch_mt<FMT, 16>(epi, a, pairs, s);
        case 24: return launch_mt<FMT, 24>(epi, a, pairs, s);
        case 32: return launch_mt<FMT, 32>(epi, a, pairs, s);
        case 48: return launch_mt<FMT, 48>(epi, a, pairs, s);
        case 64: return launch_mt<FMT, 64>(epi, a, pairs, s);
        default: return hipErrorInvalidValue;
    }
}

// The skewed-decode launch (k_matvec_mixed): the tile's grid first (at most
// one workgroup per compute unit: its item count is only bounded on the
// host, and its spare workgroups would hold slots the mat-vec's need), then
// the mat-vec's (the same grid and tall-tile choice as its own launch).
template <int LPR, int EPI, bool DBG, int TS>
hipError_t launch_mixed_ts(const ExpertArgs& a, int64_t groups, hipStream_t s) {
    const int64_t tg = tq8::tile_grid<EPI, 32>(a), cus = cu_count();
    const int64_t n_tile = tg < cus ? tg : cus;
    const int tr = kTileRows << TS;
    const int64_t max_items = groups * ((a.rows + tr - 1) / tr);
    const int64_t cap = static_cast<int64_t>(cu_count()) * 8;
    int64_t gm = max_items < cap ? max_items : cap;
    if (gm < 1) gm = 1;
    hipLaunchKernelGGL((k_matvec_mixed<LPR, EPI, TS, DBG>), dim3(static_cast<unsigned>(n_tile + gm)), dim3(kThreads),
                       0, s, a, static_cast<int>(n_tile));
    return hipGetLastError();
}

template <int LPR, int EPI, bool DBG>
hipError_t launch_mixed_dbg(const ExpertArgs& a, hipStream_t s) {
    constexpr int NMAT = (EPI == kEpiSwigluQ8) ? 2 : 1;
    constexpr int TALL = tall_shift<LPR, NMAT>();
    const int64_t A = static_cast<int64_t>(a.n_tokens) * a.top_k;
    const int64_t slots = A < a.n_experts ? A : a.n_experts;
    const int64_t groups = (A + 1) / 2 + slots;   // pairs of assignments
    if constexpr (TALL > 0) {
        const int tr = kTileRows << TALL;
        if (groups * ((a.rows + tr - 1) / tr) >= 4 * static_cast<int64_t>(cu_count()))
            return launch_mixed_ts<LPR, EPI, DBG, TALL>(a, groups, s);
    }
    return launch_mixed_ts<LPR, EPI, DBG, 0>(a, groups, s);
}

template <int LPR>
hipError_t launch_mixed_lpr(Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (epi == kEpiF32)
        return a.debug ? launch_mixed_dbg<LPR, kEpiF32, true>(a, s) : launch_mixed_dbg<LPR, kEpiF32, false>(a, s);
    return a.debug ? launch_mixed_dbg<LPR, kEpiSwigluQ8, true>(a, s) : launch_mixed_dbg<LPR, kEpiSwigluQ8, false>(a, s);
}


hipError_t launch_mixed(Epi epi, const ExpertArgs& a, hipStream_t s) {
    switch (a.cols / FmtInfo<kTernary>::kChunkWeights) {
        case 12: return launch_mixed_lpr<12>(epi, a, s);
        case 32: return launch_mixed_lpr<32>(epi, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Whether the skewed-decode launch covers a call (ternary, fp32 or SwiGLU
// epilogue, tile chunks of 32, and the row lengths it is built for: 768 and
// 2048 weights, the down and gate/up rows of the ternary decode FFN; each
// row length is 4-8 more kernels of both bodies to compile); otherwise the
// tile and the mat-vec run as two launches.
bool mixed_planned(Fmt fmt, Epi epi, int n_tokens, int top_k, int cols) {
    const int64_t A = static_cast<int64_t>(n_tokens) * top_k;
    if (fmt != kTernary || (epi != kEpiF32 && epi != kEpiSwigluQ8) || A > tq8::kSmallChunkMaxAssign) return false;
    const int lpr = cols / FmtInfo<kTernary>::kChunkWeights;
    return cols % FmtInfo<kTernary>::kChunkWeights == 0 && (lpr == 12 || lpr == 32);
}

bool matvec_supported(Fmt fmt, int cols) {
    const int cw = (fmt == kTernary) ? 64 : 128;   // grid1 and sign1: 128
    if (cols % 256 != 0) return false;
    switch (cols / cw) {
        case 2: case 4: case 8: case 12: case 16: case 24: case 32: case 48: case 64: return true;
        default: return false;
    }
}

hipError_t launch_matvec(Fmt fmt, Epi epi, const ExpertArgs& a, hipStream_t s) {
    // Per-expert choice by load: with more assignments than experts (the
    // split grouping) an expert holding at least kHeavyMin of them runs on
    // the int8-MFMA tile kernel, the rest on the mat-vec.
    const int plan = plan_matvec(a.n_tokens, a.top_k, a.n_experts, a.cols, a.debug);
    ExpertArgs m = a;
    m.heavy_min = 0;
    if (plan & PQ_PLAN_TILE_Q8) {
        m.heavy_min = kHeavyMin;
        if ((plan & PQ_PLAN_MATVEC_PAIRS) && mixed_planned(fmt, epi, m.n_tokens, m.top_k, m.cols))
            return launch_mixed(epi, m, s);
        const hipError_t err = launch_tile_q8(fmt, epi, m, s);
        if (err != hipSuccess) return err;
    }
    const bool pairs = (plan & PQ_PLAN_MATVEC_PAIRS) != 0;
    if (fmt == kTernary) return launch_fmt<kTernary>(epi, m, pairs, s);
    if (fmt == kSign1) return launch_fmt<kSign1>(epi, m, pairs, s);
    return launch_fmt<kGrid1>(epi, m, pairs, s);
}

}  // namespace pqk
