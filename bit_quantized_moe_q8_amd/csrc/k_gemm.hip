// Prefill: grouped dequant-per-tile GEMM over grid1 expert weights with bf16
// activations on MFMA (Parakon Runtime README, "How it works": prompt
// processing at large batch sizes uses a dequant-per-tile GEMM path; the
// packed blocks are never expanded in memory).
//
// out[a][n] = sum_b d[e][n][b] * sum_{k in block b} x[r(a)][k] * w[e][n][k]
//
// Work item: (chunk of up to 64 rows of one expert's group, tile of output
// columns).  Four waves; each wave owns NW 16-column subtiles of every matrix
// (gate and up for the SwiGLU epilogue, so h = silu(g) * u is formed in
// registers) and all M subtiles of the chunk, i.e. MS x NMAT x NW
// v_mfma_f32_16x16x32_bf16 tiles.
//
// K loop, one 256-wide scale block at a time:
//  - A (activations, gathered by assignment) is copied global -> LDS with
//    global_load_lds_dwordx4, already in MFMA fragment order (fragment
//    (ms, ks) = 64 lanes x 16 bytes), double-buffered so the next block's copy
//    overlaps this block's MFMAs; every fragment read is conflict-free.
//  - B (weights) is decoded on chip only: lane l of a wave takes column
//    l % 16 and, in K step ks, the grid group 8*(l/16) + ks of the block; its
//    11-bit index selects a 16-byte bf16 row of the codebook in LDS, which is
//    exactly the lane's B fragment (8 consecutive weights of one column).  A
//    fragments use the same K assignment (lane group g holds k = 64g + 8ks ..
//    64g + 8ks + 7), so each MFMA sums matching products.
//  - Each block accumulates in its own fp32 MFMA accumulators (values {-1,0,1}
//    and bf16 activations are exact in the products), then the fp16 scale is
//    applied in fp32: total += d * block.  Folding the scale into bf16 weights
//    would round it to 8 significant bits.
//
// Items are ordered so that all column tiles of one row chunk run on the
// same XCD (workgroup b runs on XCD b % 8 and the grid is a multiple of 8), so
// the chunk's activation rows are fetched into one L2.
#include "pq_device.hpp"
#include "pq_internal.hpp"

namespace pqk {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kMsMax = 4;                 // 16-row M subtiles per chunk
constexpr int kChunkRows = 16 * kMsMax;   // 64
constexpr int kKs = 8;                    // 32-wide K steps per 256 block
constexpr int kMaxExperts = 1024;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void copy16_to_lds(const void* g, uint4* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_wave_base), 16, 0, 0);
}

__device__ __forceinline__ int block_exclusive_scan256(int v, int* tmp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wave; ++i) base += tmp[i];
    __syncthreads();
    return base + incl - v;
}

template <int EPI, bool DBG>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(ExpertArgs p) {
    constexpr int NMAT = (EPI == kEpiF32) ? 1 : 2;
    constexpr int NW = (NMAT == 2) ? 2 : 4;       // 16-col subtiles per wave per matrix
    constexpr int TILE_N = kWaves * NW * 16;      // 128 (gate/up) or 256 (down)

    __shared__ uint4 s_a[2][kMsMax][kKs][64];
    __shared__ uint4 s_cb[kGridEntries];
    __shared__ int s_cstart[kMaxExperts + 1];
    __shared__ int s_row[kChunkRows];
    __shared__ int s_asg[kChunkRows];
    __shared__ int s_tmp[kWaves];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int E = p.n_experts, N = p.rows, K = p.cols;
    const int KB = K / 256;

    // bf16 codebook: entry i = 8 values in {-1,0,1} -> 8 bf16 (exact).
    for (int i = tid; i < kGridEntries; i += kThreads) {
        const uint2 raw = reinterpret_cast<const uint2*>(p.grid)[i];
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t wv = (j < 2) ? raw.x : raw.y;
            const int v0 = static_cast<int8_t>((wv >> (16 * (j & 1))) & 0xffu);
            const int v1 = static_cast<int8_t>((wv >> (16 * (j & 1) + 8)) & 0xffu);
            const uint32_t b0 = __builtin_bit_cast(uint32_t, static_cast<float>(v0)) >> 16;
            const uint32_t b1 = __builtin_bit_cast(uint32_t, static_cast<float>(v1)) >> 16;
            o[j] = b0 | (b1 << 16);
        }
        s_cb[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    // Chunks of up to 64 rows per expert; s_cstart = exclusive prefix.
    {
        int cnt[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid * 4 + j;
            cnt[j] = 0;
            if (e < E) {
                const int m = p.offsets[e + 1] - p.offsets[e];
                cnt[j] = (m + kChunkRows - 1) / kChunkRows;
            }
            sum += cnt[j];
        }
        int base = block_exclusive_scan256(sum, s_tmp);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid * 4 + j;
            if (e < E) s_cstart[e] = base;
            base += cnt[j];
        }
        if (tid == kThreads - 1) s_cstart[E] = base;   // total number of chunks
    }
    __syncthreads();

    const int C = s_cstart[E];
    const int NT = (N + TILE_N - 1) / TILE_N;
    const int per_xcd = ((C + 7) / 8) * NT;
    const int n_items = 8 * per_xcd;

    const int64_t qs_row = K / 8, qh_row = K / 32, d_row = K / 256;
    const int64_t qs_e = static_cast<int64_t>(N) * qs_row;
    const int64_t qh_e = static_cast<int64_t>(N) * qh_row;
    const int64_t d_e = static_cast<int64_t>(N) * d_row;
    const int lg = lane >> 4;      // lane group: K range 64*lg .. 64*lg+63 of a block
    const int lc = lane & 15;      // column inside a 16-col subtile / row inside an M subtile

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int xcd = item & 7, j = item >> 3;
        const int c = xcd + 8 * (j / NT), nt = j % NT;
        if (c >= C) continue;   // uniform over the workgroup
        // expert owning chunk c: the last e with s_cstart[e] <= c
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_cstart[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int cbeg = p.offsets[e] + (c - s_cstart[e]) * kChunkRows;
        const int mrows = min(kChunkRows, p.offsets[e + 1] - cbeg);
        const int MS = (mrows + 15) >> 4;
        if (tid < kChunkRows) {
            const int r = tid < mrows ? tid : 0;
            const int a = p.sorted[cbeg + r];
            s_asg[tid] = a;
            s_row[tid] = p.act_by_token ? a / p.top_k : a;
        }
        __syncthreads();

        // this lane's columns (clamped for the loads; outputs past N are dropped)
        int ncol[NW], nrow[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int n = nt * TILE_N + (wave * NW + w) * 16 + lc;
            ncol[w] = n;
            nrow[w] = n < N ? n : N - 1;
        }
        const uint8_t* qsb[NMAT];
        const uint16_t* qhb[NMAT];
        const uint16_t* db[NMAT];
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
            qsb[m] = p.qs[m] + e * qs_e + 8 * lg;
            qhb[m] = p.qh[m] + e * qh_e + 2 * lg;
            db[m] = p.d[m] + e * d_e;
        }

        auto issue_a = [&](int kb, uint4 (*dst)[kKs][64]) {
            for (int f = wave; f < MS * kKs; f += kWaves) {
                const int ms = f / kKs, ks = f % kKs;
                const int row = s_row[ms * 16 + lc];
                const uint16_t* src = p.xb + static_cast<int64_t>(row) * K + kb * 256 + (8 * lg + ks) * 8;
                copy16_to_lds(src, &dst[ms][ks][0]);
            }
        };
        uint2 bq[NMAT][NW];
        uint32_t bh[NMAT][NW];
        float bd[NMAT][NW];
        auto load_b = [&](int kb) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    bq[m][w] = *reinterpret_cast<const uint2*>(qsb[m] + nrow[w] * static_cast<int>(qs_row) + kb * 32);
                    bh[m][w] = *reinterpret_cast<const uint32_t*>(qhb[m] + nrow[w] * static_cast<int>(qh_row) + kb * 8);
                    bd[m][w] = half_bits_to_float(db[m][nrow[w] * static_cast<int>(d_row) + kb]);
                }
        };

        f32x4 tot[kMsMax][NMAT][NW];
        f32x4 blk[kMsMax][NMAT][NW];
#pragma unroll
        for (int ms = 0; ms < kMsMax; ++ms)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int w = 0; w < NW; ++w) tot[ms][m][w] = f32x4{0.f, 0.f, 0.f, 0.f};

        issue_a(0, s_a[0]);
        load_b(0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        for (int kb = 0; kb < KB; ++kb) {
            uint2 cq[NMAT][NW];
            uint32_t ch[NMAT][NW];
            float cd[NMAT][NW];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    cq[m][w] = bq[m][w];
                    ch[m][w] = bh[m][w];
                    cd[m][w] = bd[m][w];
                }
            if (kb + 1 < KB) {
                issue_a(kb + 1, s_a[(kb + 1) & 1]);
                load_b(kb + 1);
            }
            {
                uint4 (*src)[kKs][64] = s_a[kb & 1];
#pragma unroll
                for (int ks = 0; ks < kKs; ++ks) {
                    bf16x8 bf[NMAT][NW];
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int w = 0; w < NW; ++w) {
                            const uint32_t qword = (ks < 4) ? cq[m][w].x : cq[m][w].y;
                            const uint32_t lo8 = (qword >> (8 * (ks & 3))) & 0xffu;
                            const uint32_t hi3 = (ch[m][w] >> (16 * (ks >> 2) + 3 * (ks & 3))) & 7u;
                            bf[m][w] = __builtin_bit_cast(bf16x8, s_cb[lo8 | (hi3 << 8)]);
                        }
#pragma unroll
                    for (int ms = 0; ms < kMsMax; ++ms) {
                        if (ms < MS) {
                            const bf16x8 af = __builtin_bit_cast(bf16x8, src[ms][ks][lane]);
#pragma unroll
                            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                                for (int w = 0; w < NW; ++w)
                                    blk[ms][m][w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                        af, bf[m][w], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : blk[ms][m][w], 0, 0, 0);
                        }
                    }
                }
            }
#pragma unroll
            for (int ms = 0; ms < kMsMax; ++ms) {
                if (ms < MS) {
#pragma unroll
                    for (int m = 0; m < NMAT; ++m)
#pragma unroll
                        for (int w = 0; w < NW; ++w)
#pragma unroll
                            for (int i = 0; i < 4; ++i) tot[ms][m][w][i] += cd[m][w] * blk[ms][m][w][i];
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }

        // epilogue: lane holds rows 16*ms + 4*lg + i of column ncol[w]
#pragma unroll
        for (int ms = 0; ms < kMsMax; ++ms) {
            if (ms >= MS) continue;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int n = ncol[w];
                if (n >= N) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = ms * 16 + lg * 4 + i;
                    if (r >= mrows) continue;
                    const int64_t o = static_cast<int64_t>(s_asg[r]) * N + n;
                    if constexpr (EPI == kEpiF32) {
                        static_cast<float*>(p.out0)[o] = tot[ms][0][w][i];
                        if constexpr (DBG) {
                            if (p.dbg_g) p.dbg_g[o] = tot[ms][0][w][i];
                        }
                    } else {
                        const float g = tot[ms][0][w][i], u = tot[ms][1][w][i];
                        const float h = g / (1.0f + expf(-g)) * u;
                        static_cast<uint16_t*>(p.out0)[o] = float_to_bf16_bits(h);
                        if constexpr (DBG) {
                            if (p.dbg_g) p.dbg_g[o] = g;
                            if (p.dbg_u) p.dbg_u[o] = u;
                            if (p.dbg_h) p.dbg_h[o] = h;
                        }
                    }
                }
            }
        }
        __syncthreads();   // s_row / s_asg / A buffers are reused by the next item
    }
}

template <int EPI, bool DBG>
hipError_t launch_one(const ExpertArgs& a, hipStream_t s) {
    // persistent: one workgroup per compute unit, a multiple of 8 (XCDs)
    int grid = cu_count();
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL((k_gemm<EPI, DBG>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool gemm_supported(int rows, int cols, int epi) {
    if (cols % 256 != 0 || rows < 1) return false;
    return epi == kEpiF32 || epi == kEpiSwigluBf16;
}

hipError_t launch_gemm(Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (epi == kEpiF32) return a.debug ? launch_one<kEpiF32, true>(a, s) : launch_one<kEpiF32, false>(a, s);
    if (epi == kEpiSwigluBf16)
        return a.debug ? launch_one<kEpiSwigluBf16, true>(a, s) : launch_one<kEpiSwigluBf16, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace pqk
