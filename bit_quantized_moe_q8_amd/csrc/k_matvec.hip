// Grouped decode mat-vec over packed 1-bit-class expert weights against q8
// activations (Parakon Runtime README, "How it works": fused mat-vec kernels
// read the quantized blocks directly from device memory and accumulate
// against int8 activations with a 4-way int8 dot product; nothing is ever
// dequantized to memory).
//
// Work decomposition.  A work item is (active expert, tile of 32 output rows);
// items are numbered slot-major, so the first n_active*tiles items are real
// and the launch (persistent, grid-stride over items) never needs the
// routing on the host.  With the SwiGLU epilogue a tile holds the 32 gate rows
// and the 32 up rows of the same outputs (gate/up fusion: pxq_llama README,
// "Updates - 2026-07-28"), so h = silu(g)*u and its q8 block of 32 are formed
// in the same workgroup.
//
// Lane mapping.  A row is split into LPR chunks of 16 packed bytes (ternary:
// 64 weights = 2 int8 blocks of 32; grid1: 16 groups = 128 weights = 4 blocks
// of 32).  Lane l of a wave owns chunk l % LS of row-slot l / LS for every
// row it touches, so its slice of the activation row is loaded once into
// registers and reused for all rows (the pages stage the activation vector
// on chip for the same reason: pxq_llama README, "Updates - 2026-07-28",
// 2D decode driver).  Each lane issues all of its 16-byte weight loads for
// the tile before consuming any, so a wave keeps ITERS x 16 B per lane in
// flight.  Row slots are LPR rounded up to a power of two lanes wide (a 12-chunk
// row uses 12 of 16 lanes), so the partial row sums reduce with DPP lane moves
// (quad_perm, row mirrors, row_bcast) instead of LDS permutes.
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
// Scale application in fp32: partial = d_w * (sum over the lane's blocks of
// xd * isum), then the cross-lane sum.
#include "pq_device.hpp"
#include "pq_internal.hpp"

namespace pqk {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTileRows = 32;

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

template <int FMT, int LPR, int MT, int EPI, bool DBG>
__global__ __launch_bounds__(kThreads) void k_matvec(ExpertArgs p) {
    using FI = FmtInfo<FMT>;
    // Row slots are LS lanes wide (LPR rounded up to a power of two, so that
    // the row sums are DPP segment reductions); lanes chunk >= LPR idle.
    constexpr int LS = (LPR <= 2) ? 2 : (LPR <= 4) ? 4 : (LPR <= 8) ? 8 : (LPR <= 16) ? 16
                     : (LPR <= 32) ? 32 : 64;
    constexpr int RPW = kWave / LS;               // row slots per wave
    constexpr int ROWS_IT = kWaves * RPW;         // rows per workgroup iteration
    constexpr int NMAT = (EPI == kEpiF32) ? 1 : 2;
    constexpr int P = kTileRows * NMAT;           // physical rows per tile
    constexpr int ITERS = (P + ROWS_IT - 1) / ROWS_IT;
    constexpr int SUBS = FI::kSubs;
    constexpr int ACT_DW = FI::kChunkWeights / 4;  // activation dwords per chunk

    __shared__ uint2 s_grid[(FMT == kGrid1) ? kGridEntries : 1];
    __shared__ float s_gu[NMAT][MT][kTileRows];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int slot_row = lane / LS, chunk = lane % LS;
    const bool lane_on = chunk < LPR;

    const int rows = p.rows, cols = p.cols;
    const int tiles = (rows + kTileRows - 1) / kTileRows;
    const int n_items = *p.n_active * tiles;
    if (static_cast<int>(blockIdx.x) >= n_items) return;

    if constexpr (FMT == kGrid1) {
        const uint4* src = reinterpret_cast<const uint4*>(p.grid);
        uint4* dst = reinterpret_cast<uint4*>(s_grid);
        for (int i = tid; i < kGridEntries / 2; i += kThreads) dst[i] = src[i];
        __syncthreads();
    }

    const int64_t qs_row_bytes = (FMT == kTernary) ? cols / 4 : cols / 8;
    const int64_t qh_row = cols / 32;
    const int64_t d_row = cols / 256;
    const int64_t qs_e = static_cast<int64_t>(rows) * qs_row_bytes;
    const int64_t qh_e = static_cast<int64_t>(rows) * qh_row;
    const int64_t d_e = static_cast<int64_t>(rows) * d_row;
    const int n_sub_row = cols / 32;

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int slot = item / tiles, tile = item % tiles;
        const int e = p.active[slot];
        const int beg = p.offsets[e];
        const int m = p.offsets[e + 1] - beg;
        const int n0 = tile * kTileRows;

        // ---- issue every weight load of this lane for the tile
        uint4 wq[ITERS];
        uint2 wh[ITERS];
        float dw[ITERS];
        bool rv[ITERS], rok[ITERS];  // lane loads for this row / row exists
        int rn[ITERS], rm[ITERS];
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int pr = it * ROWS_IT + wave * RPW + slot_row;
            const int mat = (NMAT == 2) ? (pr / kTileRows) : 0;
            const int n = n0 + pr % kTileRows;
            rok[it] = pr < P && n < rows;
            rv[it] = lane_on && rok[it];
            rn[it] = n;
            rm[it] = mat;
            wq[it] = make_uint4(0, 0, 0, 0);
            wh[it] = make_uint2(0, 0);
            dw[it] = 0.0f;
            if (rv[it]) {
                const uint8_t* qs = p.qs[mat] + e * qs_e + n * qs_row_bytes + chunk * 16;
                wq[it] = *reinterpret_cast<const uint4*>(qs);
                if constexpr (FMT == kGrid1) {
                    const uint16_t* qh = p.qh[mat] + e * qh_e + n * qh_row + chunk * 4;
                    wh[it] = *reinterpret_cast<const uint2*>(qh);
                    dw[it] = half_bits_to_float(p.d[mat][e * d_e + n * d_row + chunk / 2]);
                } else {
                    dw[it] = half_bits_to_float(p.d[mat][e * d_e + n * d_row + chunk / 4]);
                }
            }
        }

        for (int base = 0; base < m; base += MT) {
            const int mcount = min(MT, m - base);
            // ---- activation slices of up to MT assignments
            uint32_t act[MT][ACT_DW];
            float xs[MT][SUBS];
            int asg[MT];
#pragma unroll
            for (int j = 0; j < MT; ++j) {
                asg[j] = 0;
#pragma unroll
                for (int i = 0; i < ACT_DW; ++i) act[j][i] = 0;
#pragma unroll
                for (int s = 0; s < SUBS; ++s) xs[j][s] = 0.0f;
                if (j < mcount) {
                    const int a = p.sorted[beg + base + j];
                    asg[j] = a;
                    const int r = p.act_by_token ? a / p.top_k : a;
                    const uint4* xa = reinterpret_cast<const uint4*>(
                        p.xq + static_cast<int64_t>(r) * cols + chunk * FI::kChunkWeights);
                    if (lane_on) {
#pragma unroll
                        for (int v = 0; v < ACT_DW / 4; ++v) {
                            uint4 q = xa[v];
                            uint32_t qq[4] = {q.x, q.y, q.z, q.w};
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
                        const float* xdp = p.xd + static_cast<int64_t>(r) * n_sub_row + chunk * SUBS;
#pragma unroll
                        for (int s = 0; s < SUBS; ++s) xs[j][s] = xdp[s];
                    }
                }
            }

            // ---- integer block sums, fp32 scale application
            float part[ITERS][MT];
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                int isum[MT][SUBS];
#pragma unroll
                for (int j = 0; j < MT; ++j)
#pragma unroll
                    for (int s = 0; s < SUBS; ++s) isum[j][s] = 0;
                const uint32_t wv[4] = {wq[it].x, wq[it].y, wq[it].z, wq[it].w};
                if constexpr (FMT == kTernary) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            const int wdec = ternary_decode4((wv[i] >> (2 * s)) & 0x03030303u);
#pragma unroll
                            for (int j = 0; j < MT; ++j)
                                isum[j][i >> 1] = dot4(wdec, static_cast<int>(act[j][4 * i + s]),
                                                       isum[j][i >> 1]);
                        }
                    }
                } else {
                    const uint32_t hv[2] = {wh[it].x, wh[it].y};
#pragma unroll
                    for (int g = 0; g < 16; ++g) {
                        const uint32_t lo = (wv[g >> 2] >> (8 * (g & 3))) & 0xffu;
                        const uint32_t hw = hv[g >> 3] >> (16 * ((g >> 2) & 1));
                        const uint32_t hi = (hw >> (3 * (g & 3))) & 7u;
                        const uint2 cb = s_grid[lo | (hi << 8)];
#pragma unroll
                        for (int j = 0; j < MT; ++j) {
                            int acc = isum[j][g >> 2];
                            acc = dot4(static_cast<int>(cb.x), static_cast<int>(act[j][2 * g]), acc);
                            acc = dot4(static_cast<int>(cb.y), static_cast<int>(act[j][2 * g + 1]), acc);
                            isum[j][g >> 2] = acc;
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < MT; ++j) {
                    float f = 0.0f;
#pragma unroll
                    for (int s = 0; s < SUBS; ++s) f += xs[j][s] * static_cast<float>(isum[j][s]);
                    part[it][j] = dw[it] * f;
                    if constexpr (DBG) {
                        int32_t* dst = p.dbg_isums[rm[it]];
                        if (dst && rv[it] && j < mcount) {
                            const int64_t o = (static_cast<int64_t>(asg[j]) * rows + rn[it]) * n_sub_row +
                                              chunk * SUBS;
#pragma unroll
                            for (int s = 0; s < SUBS; ++s) dst[o + s] = isum[j][s];
                        }
                    }
                }
            }

            // ---- sum over the lanes of each row slot (result in its last lane)
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
#pragma unroll
                for (int j = 0; j < MT; ++j) part[it][j] = seg_sum<LS>(lane_on ? part[it][j] : 0.0f);
            }
            const bool out_lane = chunk == LS - 1;

            // ---- epilogue
            if constexpr (EPI == kEpiF32) {
                float* out = static_cast<float*>(p.out0);
#pragma unroll
                for (int it = 0; it < ITERS; ++it) {
                    if (rok[it] && out_lane) {
#pragma unroll
                        for (int j = 0; j < MT; ++j)
                            if (j < mcount)
                                out[static_cast<int64_t>(asg[j]) * rows + rn[it]] = part[it][j];
                    }
                }
            } else {
#pragma unroll
                for (int it = 0; it < ITERS; ++it) {
                    if (rok[it] && out_lane) {
#pragma unroll
                        for (int j = 0; j < MT; ++j) s_gu[rm[it]][j][rn[it] - n0] = part[it][j];
                    }
                }
                __syncthreads();
                if (wave < (MT * kTileRows + kWave - 1) / kWave) {
                    const int j = tid / kTileRows, i = tid % kTileRows;
                    const bool jv = j < MT;
                    const float g = jv ? s_gu[0][j][i] : 0.0f, u = jv ? s_gu[1][j][i] : 0.0f;
                    const float h = g / (1.0f + expf(-g)) * u;
                    const float amax = half_wave_max(fabsf(h));
                    const float d = amax / 127.0f;
                    if (jv && j < mcount) {
                        const int a = p.sorted[beg + base + j];
                        const int64_t o = static_cast<int64_t>(a) * rows + n0 + i;
                        static_cast<int8_t*>(p.out0)[o] = static_cast<int8_t>(q8_value(h, d));
                        if (i == 0)
                            static_cast<float*>(p.out1)[static_cast<int64_t>(a) * (rows / kTileRows) +
                                                        tile] = d;
                        if constexpr (DBG) {
                            if (p.dbg_g) p.dbg_g[o] = g;
                            if (p.dbg_u) p.dbg_u[o] = u;
                            if (p.dbg_h) p.dbg_h[o] = h;
                        }
                    }
                }
                __syncthreads();
            }
        }
    }
}

template <int FMT, int LPR, int MT, int EPI, bool DBG>
hipError_t launch_one(const ExpertArgs& a, hipStream_t s) {
    const int tiles = (a.rows + kTileRows - 1) / kTileRows;
    const int64_t max_items = static_cast<int64_t>(a.n_experts) * tiles;
    const int64_t cap = static_cast<int64_t>(cu_count()) * 8;
    const unsigned grid = static_cast<unsigned>(max_items < cap ? max_items : cap);
    hipLaunchKernelGGL((k_matvec<FMT, LPR, MT, EPI, DBG>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int FMT, int LPR, int MT, int EPI>
hipError_t launch_dbg(const ExpertArgs& a, hipStream_t s) {
    return a.debug ? launch_one<FMT, LPR, MT, EPI, true>(a, s)
                   : launch_one<FMT, LPR, MT, EPI, false>(a, s);
}

template <int FMT, int LPR, int MT>
hipError_t launch_epi(Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (epi == kEpiF32) return launch_dbg<FMT, LPR, MT, kEpiF32>(a, s);
    if (epi == kEpiSwigluQ8) return launch_dbg<FMT, LPR, MT, kEpiSwigluQ8>(a, s);
    return hipErrorInvalidValue;
}

template <int FMT, int LPR>
hipError_t launch_mt(Epi epi, const ExpertArgs& a, hipStream_t s) {
    // Tokens held per pass: one when every expert sees at most one activation
    // row, otherwise a few (the assignment-per-expert mean decides).
    const int64_t A = static_cast<int64_t>(a.n_tokens) * a.top_k;
    if (a.n_tokens <= 1) return launch_epi<FMT, LPR, 1>(epi, a, s);
    if (A <= a.n_experts) return launch_epi<FMT, LPR, 2>(epi, a, s);
    return launch_epi<FMT, LPR, 4>(epi, a, s);
}

template <int FMT>
hipError_t launch_fmt(Epi epi, const ExpertArgs& a, hipStream_t s) {
    switch (a.cols / FmtInfo<FMT>::kChunkWeights) {
        case 2: return launch_mt<FMT, 2>(epi, a, s);
        case 4: return launch_mt<FMT, 4>(epi, a, s);
        case 8: return launch_mt<FMT, 8>(epi, a, s);
        case 12: return launch_mt<FMT, 12>(epi, a, s);
        case 16: return launch_mt<FMT, 16>(epi, a, s);
        case 32: return launch_mt<FMT, 32>(epi, a, s);
        case 64: return launch_mt<FMT, 64>(epi, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool matvec_supported(Fmt fmt, int cols) {
    const int cw = (fmt == kTernary) ? 64 : 128;
    if (cols % 256 != 0) return false;
    switch (cols / cw) {
        case 2: case 4: case 8: case 12: case 16: case 32: case 64: return true;
        default: return false;
    }
}

hipError_t launch_matvec(Fmt fmt, Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (fmt == kTernary) return launch_fmt<kTernary>(epi, a, s);
    return launch_fmt<kGrid1>(epi, a, s);
}

}  // namespace pqk
