// Single-token decode mat-vec over packed 1-bit-class expert weights against
// q8 activations (Parakon Runtime README, "How it works": the fused decode
// mat-vec reads the packed blocks directly and accumulates against int8
// activations; pxq_llama README, "Updates - 2026-07-28": gate/up fusion with
// SiLU and the activation vector kept on chip).
//
// At one token the whole expert layer is a few megabytes, so the kernel is
// bound by how many dependent memory round trips stand between launch and
// the last store, not by bandwidth.  This kernel is laid out for exactly
// that:
//  - one workgroup per (routed slot, 32-output tile): blockIdx.y is the slot
//    of the active-expert list, blockIdx.x the tile, so nothing is computed
//    from a division and no workgroup loops;
//  - the gate/up activation row is row 0 whatever the routing, so its loads
//    are issued first, before any routing metadata has arrived;
//  - the routing reads (n_active, the slot's expert, the slot's first sorted
//    assignment) are three independent scalar loads waited for together;
//    when every assignment has an expert of its own (n_active == top_k, the
//    normal case with distinct top-k experts) slot s holds exactly sorted
//    assignment s and the expert offsets are never read;
//  - every weight row of the tile is loaded at once into registers and stays
//    there; an expert listed for several assignments (a repeated id) only
//    re-reads activations for its further assignments.
// The arithmetic per row is that of the general grouped kernel: ternary
// codes decoded with one byte permute per four weights into int8 and
// accumulated with v_dot4_i32_i8 against byte-transposed activations; grid1
// groups looked up in the 2048-entry codebook held in LDS; sub-scaled signs
// (pxq_llama README, "What's PXQ?", PXQ1: 1-bit sign codes under a per-row fp16
// anchor with a 4-bit scale per 16 weights) as +-1 byte patterns from a
// 256-entry LDS table, each 16-weight sum times its sub-scale; exact int32
// sums per 32-weight block; fp32 scale application; DPP row reductions.
#include "pq_device.hpp"
#include "pq_internal.hpp"

namespace pqk {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTile = 32;   // outputs per workgroup (one q8 block of the SwiGLU epilogue)

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate (gfx9 encoding): no vector-memory operation of this
// wave outstanding; LDS and scalar counters untouched.
constexpr int kWaitVmem0 = (0x7 << 4) | (0xF << 8);

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}

// Maximum over the wave (unsigned), returned uniform: DPP steps leave it in
// lane 63 (0 from disabled rows is neutral).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<kDppQuadXor1>(v));
    v = max(v, dpp_u32<kDppQuadXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    v = max(v, dpp_u32<kDppBcast15, 0xA>(v));
    v = max(v, dpp_u32<kDppBcast31, 0xC>(v));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// q8_pack4 with the 8-lane block maximum taken by DPP moves (the same
// maximum, so the same codes and scale).
__device__ __forceinline__ uint32_t q8_pack4_dpp(float4 v, float& d) {
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, dpp_f32<kDppQuadXor1>(a));
    a = fmaxf(a, dpp_f32<kDppQuadXor2>(a));
    a = fmaxf(a, dpp_f32<kDppHalfMirror>(a));
    d = a / 127.0f;
    return (static_cast<uint32_t>(q8_value(v.x, d)) & 0xffu) |
           ((static_cast<uint32_t>(q8_value(v.y, d)) & 0xffu) << 8) |
           ((static_cast<uint32_t>(q8_value(v.z, d)) & 0xffu) << 16) |
           ((static_cast<uint32_t>(q8_value(v.w, d)) & 0xffu) << 24);
}

template <int FMT>
struct Chunk;
template <>
struct Chunk<kTernary> {
    static constexpr int kWeights = 64;   // 16 bytes of 2-bit codes
    static constexpr int kSubs = 2;       // 32-weight blocks per chunk
};
template <>
struct Chunk<kGrid1> {
    static constexpr int kWeights = 128;  // 16 group indices
    static constexpr int kSubs = 4;
};
template <>
struct Chunk<kSign1> {
    static constexpr int kWeights = 128;  // 16 sign bytes
    static constexpr int kSubs = 4;
};
constexpr int kSignPatterns = 256;

// ROUTE (gate/up with the SwiGLU epilogue only): the workgroup computes the
// routing and the q8 activations itself from the token's logits and fp32
// activations (every workgroup the same, so no earlier launch is waited for);
// workgroup (0, 0) also writes the routing, the grouping the down projection
// reads, and zeros the output row for its fused combine.
//
// KS > 1 (K split): the workgroup is KS groups of four waves, group s taking
// chunks [s*LPR/KS, (s+1)*LPR/KS) of every row of the tile, so a tile's rows
// stream with KS times the waves and a quarter (or half) of the dependent
// work per wave.  Each group's row sums go through LDS and are added in the
// pairwise order ((S0 + S1) + (S2 + S3)) that the single-group lane tree
// (seg_sum over the whole row) uses for the same chunks, so the totals are
// bit-identical to KS = 1 and to the grouped mat-vec.
//
// QX (one matrix, F32 epilogue): no routing or grouping; the workgroup
// quantizes the fp32 row ra.x itself as ROUTE does and multiplies it by
// expert p.expert0, so a single mat-vec from fp32 activations is one launch.
template <int FMT, int LPR, int EPI, bool ABT, bool ROUTE, int NK = 1, int KS = 1, bool QX = false>
__global__ __launch_bounds__(kThreads * KS) void k_matvec_tok1(ExpertArgs p, RouteArgs ra) {
    using CK = Chunk<FMT>;
    constexpr int NT = kThreads * KS;                 // threads of the workgroup
    static_assert(KS == 1 || KS == 2 || KS == 4, "K slices");
    static_assert(LPR % KS == 0 && (KS == 1 || (LPR / KS) % 4 == 0), "whole, pairwise-summed slices");
    constexpr int LPS = LPR / KS;                     // chunks of a row in one K slice
    constexpr int LS = (LPS <= 2) ? 2 : (LPS <= 4) ? 4 : (LPS <= 8) ? 8 : (LPS <= 16) ? 16
                     : (LPS <= 32) ? 32 : 64;         // lanes per row slot
    static_assert(KS == 1 || LS == LPS, "a split row fills its lane slots");
    constexpr int RPW = kWave / LS;                   // row slots per wave
    constexpr int ROWS_IT = kWaves * RPW;             // rows per iteration
    constexpr int NMAT = (EPI == kEpiSwigluQ8) ? 2 : 1;
    constexpr int P = kTile * NMAT;                   // physical rows per tile
    constexpr int ITERS = (P + ROWS_IT - 1) / ROWS_IT;
    constexpr int SUBS = CK::kSubs;
    constexpr int ACT_DW = CK::kWeights / 4;          // activation dwords per chunk
    constexpr int kMaxCols = 64 * CK::kWeights;       // widest row the launcher accepts
    static_assert(!ROUTE || (ABT && EPI == kEpiSwigluQ8), "routing only in the gate/up kernel");
    static_assert(!QX || (ABT && !ROUTE && EPI == kEpiF32), "in-kernel q8 of one matrix: F32 only");
    constexpr bool kX32 = ROUTE || QX;   // fp32 activations quantized in the kernel

    // grid1: the codebook; sign1: the 256 byte patterns of +-1
    __shared__ uint2 s_grid[(FMT == kGrid1) ? kGridEntries : (FMT == kSign1) ? kSignPatterns : 1];
    __shared__ float s_gu[NMAT][kTile];
    __shared__ float s_kp[KS > 1 ? KS : 1][KS > 1 ? kTile * NMAT : 1];   // K-slice row sums
    __shared__ uint64_t s_key64[(ROUTE && NK <= 4) ? 4 * kWave : 1];
    __shared__ int s_part[(ROUTE && NK <= 4) ? 2 : 1][(ROUTE && NK <= 4) ? 2 * kWave : 1];
    __shared__ float s_tv[ROUTE ? 16 : 1];
    __shared__ int s_ti[ROUTE ? 16 : 1];
    __shared__ uint4 s_xq[kX32 ? kMaxCols / 16 : 1];
    __shared__ float s_xd[kX32 ? kMaxCols / 32 : 1];

    const int tid = threadIdx.x;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int kslice = wave_all / kWaves;               // K slice of this wave
    const int wave = wave_all % kWaves;                 // wave within the slice
    const int slot_row = lane / LS, chunk = lane % LS;
    const bool lane_on = chunk < LPS;
    const uint32_t cc = static_cast<uint32_t>(kslice * LPS + (lane_on ? chunk : LPS - 1));
    const int slot = blockIdx.y;
    const int n0 = blockIdx.x * kTile;
    const int rows = p.rows, cols = p.cols;
    const int n_sub_row = cols / 32;

    // ---- grid1: the codebook to LDS by direct global->LDS copies
    if constexpr (FMT == kGrid1) {
        const uint4* src = reinterpret_cast<const uint4*>(p.grid);
        uint4* dst = reinterpret_cast<uint4*>(s_grid);
#pragma unroll
        for (int k = 0; k < kGridEntries / 2 / NT; ++k)
            __builtin_amdgcn_global_load_lds(src + k * NT + tid,
                                             (lds_void*)(dst + k * NT + wave_all * kWave), 16, 0, 0);
    }
    if constexpr (FMT == kSign1) {
        // pattern i: byte j is -1 where bit j of i is set, else +1
        if (tid < kSignPatterns) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lo |= (((tid >> j) & 1) ? 0xFFu : 0x01u) << (8 * j);
                hi |= (((tid >> (j + 4)) & 1) ? 0xFFu : 0x01u) << (8 * j);
            }
            s_grid[tid] = make_uint2(lo, hi);
        }
    }

    // ---- activation slice of row r (this lane's chunk)
    uint4 raw[ACT_DW / 4];
    float xs[SUBS];
    auto load_act = [&](int r) {
        const uint4* xa = reinterpret_cast<const uint4*>(p.xq + static_cast<int64_t>(r) * cols +
                                                         cc * CK::kWeights);
#pragma unroll
        for (int v = 0; v < ACT_DW / 4; ++v) raw[v] = xa[v];
        const float* xdp = p.xd + static_cast<int64_t>(r) * n_sub_row + cc * SUBS;
#pragma unroll
        for (int s = 0; s < SUBS; ++s) xs[s] = xdp[s];
    };
    int n_active, e, a0;
    constexpr int kXP = kX32 ? (kMaxCols / 4 + NT - 1) / NT : 1;   // float4 passes of the q8
    float4 xv[kXP];
    if constexpr (kX32) {
        // ---- the fp32 activations (kept for the q8 below)
        const float4* x4 = reinterpret_cast<const float4*>(ra.x);
        const int n4 = cols / 4;
#pragma unroll
        for (int u = 0; u < kXP; ++u) {
            const int i = u * NT + tid;
            xv[u] = i < n4 ? x4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    if constexpr (ROUTE) {
        // ---- the logits: expert l + 64 i in lane l, as an order-preserving
        // 32-bit key (0 = absent; no finite logit maps to 0)
        const int E = p.n_experts, k = p.top_k;
        const bool lists = blockIdx.x == 0 && blockIdx.y == 0;
        if constexpr (NK <= 4) {
            // ---- up to 256 experts: the rank of every logit in one parallel
            // pass over the 64-bit keys in LDS (rank = number of larger keys;
            // the same keys as the separate router); below 128 experts two
            // threads share a logit, each counting half of the keys
            // (keys past E are 0, below every real key, so every thread
            // scans a fixed 64-key range with all its LDS reads in flight)
            // (the first 256 threads rank; with a K split the others wait)
            const bool rk = tid < 4 * kWave;
            const float lt = tid < E ? ra.logits[tid] : 0.0f;
            if (rk) s_key64[tid] = tid < E ? route_key(lt == 0.0f ? 0.0f : lt, tid) : 0ull;   // -0 -> +0
            __syncthreads();
            const bool split = E <= 2 * kWave;
            const int i = split ? (tid & (2 * kWave - 1)) : tid;
            const int j0 = split ? ((tid >> 7) & 1) * kWave : 0;
            const int nch = split ? 1 : (E + kWave - 1) / kWave;   // 64-key chunks
            int cnt = 0;
            if (rk && i < E) {
                const uint64_t ki = s_key64[i];
                const uint4* k4 = reinterpret_cast<const uint4*>(s_key64 + j0);
                for (int c = 0; c < nch; ++c) {
#pragma unroll
                    for (int b = 0; b < kWave / 16; ++b) {
                        uint4 kk[8];
#pragma unroll
                        for (int q = 0; q < 8; ++q) kk[q] = k4[c * (kWave / 2) + b * 8 + q];
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const uint64_t a0 = (static_cast<uint64_t>(kk[q].y) << 32) | kk[q].x;
                            const uint64_t a1 = (static_cast<uint64_t>(kk[q].w) << 32) | kk[q].z;
                            cnt += (a0 > ki) ? 1 : 0;
                            cnt += (a1 > ki) ? 1 : 0;
                        }
                    }
                }
            }
            if (split) {
                if (rk && i < E) s_part[(tid >> 7) & 1][i] = cnt;
                __syncthreads();
                if (tid < E) cnt = s_part[0][tid] + s_part[1][tid];
            }
            if (tid < E && cnt < k) {
                s_ti[cnt] = tid;
                s_tv[cnt] = lt;
            }
            __syncthreads();
            e = __builtin_amdgcn_readfirstlane(s_ti[slot]);
        } else {
            // ---- more experts: k rounds of a wave-wide maximum over
            // order-preserving 32-bit keys (0 = absent; no finite logit maps
            // to 0) in every wave, equal keys to the lowest expert id (the
            // router's order); workgroup (0, 0) keeps the lists
            uint32_t kv[NK];
            float lv[NK];
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const int ee = i * kWave + lane;
                lv[i] = ee < E ? ra.logits[ee] : 0.0f;
                const float v = lv[i] == 0.0f ? 0.0f : lv[i];   // -0 -> +0
                const uint32_t u = __builtin_bit_cast(uint32_t, v);
                kv[i] = ee < E ? ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) : 0u;
            }
            const int rounds = lists ? k : slot + 1;
            e = 0;
            for (int r = 0; r < rounds; ++r) {
                uint32_t m = kv[0];
#pragma unroll
                for (int i = 1; i < NK; ++i) m = max(m, kv[i]);
                m = wave_max_u32(m);
                int win = -1;
#pragma unroll
                for (int i = 0; i < NK; ++i) {
                    const uint64_t bal = __ballot(kv[i] == m);
                    if (win < 0 && bal != 0) win = i * kWave + __ffsll(static_cast<unsigned long long>(bal)) - 1;
                }
#pragma unroll
                for (int i = 0; i < NK; ++i)
                    if (i * kWave + lane == win) kv[i] = 0u;
                if (r == slot) e = win;
                if (lists && wave_all == 0) {
                    // the winner's logit as given (not the folded key)
                    float wv = 0.0f;
#pragma unroll
                    for (int i = 0; i < NK; ++i)
                        if (i == (win >> 6))
                            wv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lv[i]), win & 63));
                    if (lane == 0) {
                        s_ti[r] = win;
                        s_tv[r] = wv;
                    }
                }
            }
        }
        // slot = rank: the grid holds exactly top_k slots
        n_active = k;
        a0 = slot;
    } else if constexpr (QX) {
        // one matrix, one assignment (its output row 0)
        n_active = 1;
        e = p.expert0;
        a0 = 0;
    } else {
        // by token at one token: every assignment reads row 0
        if constexpr (ABT) load_act(0);
        // ---- routing: three independent scalar loads
        n_active = load_uniform(p.n_active);
        e = load_uniform(p.active + slot);
        a0 = load_uniform(p.sorted + slot);
        if (slot >= n_active) return;
    }
    const bool dense = kX32 || n_active == p.top_k;

    // ---- every weight row of the tile
    const uint32_t qs_row = (FMT == kTernary) ? cols / 4 : cols / 8;
    // grid1 qh: one uint16 per 32 weights; sign1 sub-scales: one byte per
    // 32 weights, and one anchor d per row
    const uint32_t qh_row = cols / 32, d_row = (FMT == kSign1) ? 1 : cols / 256;
    const int64_t qs_e = static_cast<int64_t>(rows) * qs_row;
    const int64_t qh_e = static_cast<int64_t>(rows) * qh_row;
    const int64_t d_e = static_cast<int64_t>(rows) * d_row;
    const int wrow0 = wave * RPW;
    uint4 wq[ITERS];
    uint2 wh[ITERS];
    uint32_t wd[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int pr = it * ROWS_IT + wrow0 + slot_row;
        const int mat = (NMAT == 2) ? ((it * ROWS_IT + wrow0) / kTile) : 0;   // wave-uniform
        const int n = n0 + (pr & (kTile - 1));
        // rows past the matrix load a clamped row that is never stored
        const uint32_t nc = static_cast<uint32_t>(n < rows ? n : rows - 1);
        const uint8_t* qsb = ((NMAT == 2 && mat == 1) ? p.qs[1] : p.qs[0]) + e * qs_e;
        const uint16_t* db = ((NMAT == 2 && mat == 1) ? p.d[1] : p.d[0]) + e * d_e;
        wq[it] = *reinterpret_cast<const uint4*>(qsb + (nc * qs_row + cc * 16u));
        if constexpr (FMT == kGrid1) {
            const uint16_t* qhb = ((NMAT == 2 && mat == 1) ? p.qh[1] : p.qh[0]) + e * qh_e;
            wh[it] = *reinterpret_cast<const uint2*>(qhb + (nc * qh_row + cc * 4u));
            wd[it] = db[nc * d_row + cc / 2u];
        } else if constexpr (FMT == kSign1) {
            const uint8_t* scb = ((NMAT == 2 && mat == 1) ? p.sc[1] : p.sc[0]) + e * qh_e;
            wh[it] = make_uint2(*reinterpret_cast<const uint32_t*>(scb + (nc * qh_row + cc * 4u)), 0u);
            wd[it] = db[nc];
        } else {
            wh[it] = make_uint2(0, 0);
            wd[it] = db[nc * d_row + cc / 4u];
        }
    }

    if constexpr (kX32) {
        // ---- q8 of the activations into LDS while the weights are in flight
        const int n4 = cols / 4;
#pragma unroll
        for (int u = 0; u < kXP; ++u) {
            if (u * NT * 4 < cols) {   // uniform; 8-lane groups are whole (cols % 32 == 0)
                float d;
                const uint32_t q = q8_pack4_dpp(xv[u], d);
                const int i = u * NT + tid;
                if (i < n4) {
                    reinterpret_cast<uint32_t*>(s_xq)[i] = q;
                    if ((i & 7) == 0) s_xd[i >> 3] = d;
                }
            }
        }
        __syncthreads();   // q8 rows and (wave 0's) routing lists visible
#pragma unroll
        for (int v = 0; v < ACT_DW / 4; ++v) raw[v] = s_xq[cc * (CK::kWeights / 16) + v];
#pragma unroll
        for (int s2 = 0; s2 < SUBS; ++s2) xs[s2] = s_xd[cc * SUBS + s2];
    }

    // ---- assignments of this slot: dense -> exactly sorted[slot]
    int beg = slot, m = 1;
    if (!dense) {
        beg = load_uniform(p.offsets + e);
        m = load_uniform(p.offsets + e + 1) - beg;
    }
    int a = dense ? a0 : load_uniform(p.sorted + beg);   // (never read with ROUTE)
    if constexpr (!ABT) load_act(a);
    float wsel = (EPI == kEpiF32Combine) ? load_uniform(static_cast<const float*>(p.out1) + a) : 0.0f;

    if constexpr (FMT == kGrid1) {
        __builtin_amdgcn_s_waitcnt(kWaitVmem0);   // this wave's codebook copies landed
        __syncthreads();
    } else if constexpr (FMT == kSign1) {
        __syncthreads();   // the sign patterns
    }

    float part[ITERS];
    // row sums of the tile against the activation slice in raw/xs
    auto compute = [&]() {
        // activation dwords in the order the weight decode wants
        uint32_t act[ACT_DW];
#pragma unroll
        for (int v = 0; v < ACT_DW / 4; ++v) {
            const uint32_t qq[4] = {raw[v].x, raw[v].y, raw[v].z, raw[v].w};
            if constexpr (FMT == kTernary) {
                uint32_t t[4];
                transpose_bytes4(qq, t);
#pragma unroll
                for (int s = 0; s < 4; ++s) act[4 * v + s] = t[s];
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) act[4 * v + s] = qq[s];
            }
        }
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            int isum[SUBS];
#pragma unroll
            for (int s = 0; s < SUBS; ++s) isum[s] = 0;
            const uint32_t wv[4] = {wq[it].x, wq[it].y, wq[it].z, wq[it].w};
            if constexpr (FMT == kTernary) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int wdec[4];
                    ternary_decode16(wv[i], wdec);
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        isum[i >> 1] = dot4(wdec[s], static_cast<int>(act[4 * i + s]), isum[i >> 1]);
                }
            } else if constexpr (FMT == kSign1) {
                // per 16 weights: the +-1 sum (two sign bytes), then times
                // its 4-bit sub-scale into the q8 block's sum
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    uint2 pat[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int gi = 8 * hf + q;
                        pat[q] = s_grid[(wv[gi >> 2] >> (8 * (gi & 3))) & 0xffu];
                    }
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub) {
                        const int sb16 = 4 * hf + sub;   // 16-weight block of the chunk
                        const uint32_t scv = (wh[it].x >> (4 * sb16)) & 15u;
                        int s16 = 0;
#pragma unroll
                        for (int q = 2 * sub; q < 2 * sub + 2; ++q) {
                            const int gi = 8 * hf + q;
                            s16 = dot4(static_cast<int>(pat[q].x), static_cast<int>(act[2 * gi]), s16);
                            s16 = dot4(static_cast<int>(pat[q].y), static_cast<int>(act[2 * gi + 1]), s16);
                        }
                        isum[sb16 >> 1] += static_cast<int>(scv) * s16;
                    }
                }
            } else {
                const uint32_t hv[2] = {wh[it].x, wh[it].y};
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
                        int acc = isum[gi >> 2];
                        acc = dot4(static_cast<int>(cb[q].x), static_cast<int>(act[2 * gi]), acc);
                        acc = dot4(static_cast<int>(cb[q].y), static_cast<int>(act[2 * gi + 1]), acc);
                        isum[gi >> 2] = acc;
                    }
                }
            }
            float f = 0.0f;
#pragma unroll
            for (int s = 0; s < SUBS; ++s) f += xs[s] * static_cast<float>(isum[s]);
            const float dw = half_bits_to_float(static_cast<uint16_t>(wd[it]));
            part[it] = seg_sum<LS>(lane_on ? mul_rounded(dw, f) : 0.0f);
        }
    };

    // outputs of assignment a (the row sums sit in each slot's last lane)
    auto store = [&](int a, float wsel) {
        if constexpr (KS > 1) {
            // the K slices' row sums, added in the lane tree's pairwise order
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const int pr = it * ROWS_IT + wrow0 + slot_row;
                if (pr < P && chunk == LS - 1) s_kp[kslice][pr] = part[it];
            }
            __syncthreads();
            if (tid < P) {
                float t;
                if constexpr (KS == 2) t = s_kp[0][tid] + s_kp[1][tid];
                else t = (s_kp[0][tid] + s_kp[1][tid]) + (s_kp[2][tid] + s_kp[3][tid]);
                const int n = n0 + (tid & (kTile - 1));
                if constexpr (EPI == kEpiF32) {
                    if (n < rows) static_cast<float*>(p.out0)[static_cast<int64_t>(a) * rows + n] = t;
                } else if constexpr (EPI == kEpiF32Combine) {
                    if (n < rows)
                        atomicAdd(static_cast<float*>(p.out0) + static_cast<int64_t>(a / p.top_k) * rows + n,
                                  wsel * t);
                } else {
                    s_gu[tid / kTile][tid & (kTile - 1)] = t;
                }
            }
            if constexpr (EPI != kEpiSwigluQ8) __syncthreads();   // s_kp is reused by a repeated expert
        }
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            if constexpr (KS > 1) break;
            const int pr0 = it * ROWS_IT + wrow0;
            const int pr = pr0 + slot_row;
            const int n = n0 + (pr & (kTile - 1));
            const bool rok = pr < P && n < rows && chunk == LS - 1;
            if (!rok) continue;
            if constexpr (EPI == kEpiF32) {
                static_cast<float*>(p.out0)[static_cast<int64_t>(a) * rows + n] = part[it];
            } else if constexpr (EPI == kEpiF32Combine) {
                atomicAdd(static_cast<float*>(p.out0) + static_cast<int64_t>(a / p.top_k) * rows + n,
                          wsel * part[it]);
            } else {
                s_gu[(NMAT == 2) ? pr0 / kTile : 0][pr & (kTile - 1)] = part[it];
            }
        }
        if constexpr (EPI == kEpiSwigluQ8) {
            // h = silu(g) * u and its q8 block: wave 0, one lane per output
            __syncthreads();
            if (wave_all == 0) {
                const int i = lane & 31;
                const bool valid = lane < 32 && n0 + i < rows;
                const float gg = s_gu[0][i], uu = s_gu[1][i];
                const float h = valid ? gg / (1.0f + expf(-gg)) * uu : 0.0f;
                const float amax = half_wave_max(fabsf(h));
                const float dq = amax / 127.0f;
                if (valid) {
                    const int64_t o = static_cast<int64_t>(a) * rows + n0 + i;
                    static_cast<int8_t*>(p.out0)[o] = static_cast<int8_t>(q8_value(h, dq));
                    if (i == 0)
                        static_cast<float*>(p.out1)[static_cast<int64_t>(a) * (rows / kTile) + n0 / kTile] = dq;
                }
            }
            __syncthreads();
        }
    };

    compute();
    store(a, wsel);
    // further assignments of a repeated expert id: by token they share the
    // activation row (same result), otherwise their own row is read
    for (int j = 1; j < m; ++j) {
        a = load_uniform(p.sorted + beg + j);
        if constexpr (EPI == kEpiF32Combine) wsel = load_uniform(static_cast<const float*>(p.out1) + a);
        if constexpr (!ABT) {
            load_act(a);
            compute();
        }
        store(a, wsel);
    }
    if (ROUTE && blockIdx.x == 0 && blockIdx.y == 0) {
        // after this workgroup's own tile (off its critical path): the
        // routing outputs (rank order), the grouping of the top_k distinct
        // experts (active list and sorted assignments in expert order,
        // offsets), and the zeroed output row
        const int k = p.top_k;
        if (wave_all == 0) route_softmax_store(s_tv, s_ti, k, lane, ra.ids, ra.w);
        if (tid < k) {
            const int et = s_ti[tid];
            int pos = 0;
            for (int q = 0; q < k; ++q) pos += (s_ti[q] < et) ? 1 : 0;
            ra.active[pos] = et;
            ra.sorted[pos] = tid;
        }
        for (int ee = tid; ee <= p.n_experts; ee += NT) {
            int below = 0;
            for (int q = 0; q < k; ++q) below += (s_ti[q] < ee) ? 1 : 0;
            ra.offsets[ee] = below;
        }
        if (tid == 0) *ra.n_active = k;
        if (ra.y)
            for (int i = tid; i < cols; i += NT) ra.y[i] = 0.0f;
    }
}

// K slices per workgroup for rows of LPR chunks: rows of 16 chunks and more
// (gate/up rows of 2048 ternary or 4096 grid1 weights) split in two or four,
// so a one-token launch (a few hundred workgroups) holds two to four waves
// per SIMD; narrower rows stay whole.
template <int LPR>
constexpr int tok1_kslices() {
    return (LPR == 16) ? 2 : (LPR == 32 || LPR == 64) ? 4 : 1;
}

template <int FMT, int LPR, int EPI, bool ABT>
hipError_t launch_one(const ExpertArgs& a, hipStream_t s) {
    const RouteArgs none{};
    constexpr int KS = tok1_kslices<LPR>();
    const unsigned tiles = static_cast<unsigned>((a.rows + kTile - 1) / kTile);
    // slots: at most top_k experts are active at one token
    const unsigned slots = static_cast<unsigned>(a.top_k < a.n_experts ? a.top_k : a.n_experts);
    hipLaunchKernelGGL((k_matvec_tok1<FMT, LPR, EPI, ABT, false, 1, KS>), dim3(tiles, slots),
                       dim3(kThreads * KS), 0, s, a, none);
    return hipGetLastError();
}

template <int FMT, int LPR, int EPI>
hipError_t launch_abt(const ExpertArgs& a, hipStream_t s) {
    return a.act_by_token ? launch_one<FMT, LPR, EPI, true>(a, s) : launch_one<FMT, LPR, EPI, false>(a, s);
}

template <int FMT, int LPR>
hipError_t launch_epi(Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (epi == kEpiF32) return launch_abt<FMT, LPR, kEpiF32>(a, s);
    if (epi == kEpiF32Combine) return launch_one<FMT, LPR, kEpiF32Combine, false>(a, s);
    if (epi == kEpiSwigluQ8) return launch_abt<FMT, LPR, kEpiSwigluQ8>(a, s);
    return hipErrorInvalidValue;
}

template <int FMT>
hipError_t launch_fmt(Epi epi, const ExpertArgs& a, hipStream_t s) {
    switch (a.cols / Chunk<FMT>::kWeights) {
        case 2: return launch_epi<FMT, 2>(epi, a, s);
        case 4: return launch_epi<FMT, 4>(epi, a, s);
        case 8: return launch_epi<FMT, 8>(epi, a, s);
        case 12: return launch_epi<FMT, 12>(epi, a, s);
        case 16: return launch_epi<FMT, 16>(epi, a, s);
        case 24: return launch_epi<FMT, 24>(epi, a, s);
        case 32: return launch_epi<FMT, 32>(epi, a, s);
        case 48: return launch_epi<FMT, 48>(epi, a, s);
        case 64: return launch_epi<FMT, 64>(epi, a, s);
        default: return hipErrorInvalidValue;
    }
}

template <int FMT, int LPR>
hipError_t launch_route_one(const ExpertArgs& a, const RouteArgs& r, hipStream_t s) {
    constexpr int KS = tok1_kslices<LPR>();   // as the unrouted kernel: the same sums
    const unsigned tiles = static_cast<unsigned>((a.rows + kTile - 1) / kTile);
    const dim3 grid(tiles, a.top_k);
    if (a.n_experts <= 2 * kWave)
        hipLaunchKernelGGL((k_matvec_tok1<FMT, LPR, kEpiSwigluQ8, true, true, 2, KS>), grid, dim3(kThreads * KS), 0,
                           s, a, r);
    else if (a.n_experts <= 4 * kWave)
        hipLaunchKernelGGL((k_matvec_tok1<FMT, LPR, kEpiSwigluQ8, true, true, 4, KS>), grid, dim3(kThreads * KS), 0,
                           s, a, r);
    else
        hipLaunchKernelGGL((k_matvec_tok1<FMT, LPR, kEpiSwigluQ8, true, true, kMaxExperts / kWave, KS>), grid,
                           dim3(kThreads * KS), 0, s, a, r);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_route_fmt(const ExpertArgs& a, const RouteArgs& r, hipStream_t s) {
    switch (a.cols / Chunk<FMT>::kWeights) {
        case 2: return launch_route_one<FMT, 2>(a, r, s);
        case 4: return launch_route_one<FMT, 4>(a, r, s);
        case 8: return launch_route_one<FMT, 8>(a, r, s);
        case 12: return launch_route_one<FMT, 12>(a, r, s);
        case 16: return launch_route_one<FMT, 16>(a, r, s);
        case 24: return launch_route_one<FMT, 24>(a, r, s);
        case 32: return launch_route_one<FMT, 32>(a, r, s);
        case 48: return launch_route_one<FMT, 48>(a, r, s);
        case 64: return launch_route_one<FMT, 64>(a, r, s);
        default: return hipErrorInvalidValue;
    }
}

template <int FMT, int LPR>
hipError_t launch_x32_one(const ExpertArgs& a, const float* x, hipStream_t s) {
    constexpr int KS = tok1_kslices<LPR>();   // as the one-token kernel: the same sums
    RouteArgs ra{};
    ra.x = x;
    const unsigned tiles = static_cast<unsigned>((a.rows + kTile - 1) / kTile);
    hipLaunchKernelGGL((k_matvec_tok1<FMT, LPR, kEpiF32, true, false, 1, KS, true>), dim3(tiles, 1),
                       dim3(kThreads * KS), 0, s, a, ra);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_x32_fmt(const ExpertArgs& a, const float* x, hipStream_t s) {
    switch (a.cols / Chunk<FMT>::kWeights) {
        case 2: return launch_x32_one<FMT, 2>(a, x, s);
        case 4: return launch_x32_one<FMT, 4>(a, x, s);
        case 8: return launch_x32_one<FMT, 8>(a, x, s);
        case 12: return launch_x32_one<FMT, 12>(a, x, s);
        case 16: return launch_x32_one<FMT, 16>(a, x, s);
        case 24: return launch_x32_one<FMT, 24>(a, x, s);
        case 32: return launch_x32_one<FMT, 32>(a, x, s);
        case 48: return launch_x32_one<FMT, 48>(a, x, s);
        case 64: return launch_x32_one<FMT, 64>(a, x, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_matvec_x32(Fmt fmt, const ExpertArgs& a, const float* x, hipStream_t s) {
    if (fmt == kTernary) return launch_x32_fmt<kTernary>(a, x, s);
    if (fmt == kSign1) return launch_x32_fmt<kSign1>(a, x, s);
    return launch_x32_fmt<kGrid1>(a, x, s);
}

hipError_t launch_decode1_gate_up(Fmt fmt, const ExpertArgs& a, const RouteArgs& r, hipStream_t s) {
    if (fmt == kTernary) return launch_route_fmt<kTernary>(a, r, s);
    if (fmt == kSign1) return launch_route_fmt<kSign1>(a, r, s);
    return launch_route_fmt<kGrid1>(a, r, s);
}

hipError_t launch_matvec_tok1(Fmt fmt, Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (fmt == kTernary) return launch_fmt<kTernary>(epi, a, s);
    if (fmt == kSign1) return launch_fmt<kSign1>(epi, a, s);
    return launch_fmt<kGrid1>(epi, a, s);
}

}  // namespace pqk
