// Prefill: grouped dequant-per-tile GEMM over grid1 (or sub-scaled sign)
// expert weights with bf16 activations on MFMA (Parakon Runtime README, "How
// it works": prompt processing at large batch sizes uses a dequant-per-tile
// GEMM path; the packed blocks are never expanded in memory).  Sub-scaled
// signs (pxq_llama README, "What's PXQ?", PXQ1) take the same path: a lane's
// 8 weights are the bf16 of their 4-bit sub-scale (exact) with the sign bits
// of their sign byte ORed in from a 256-entry mask table in LDS, and the
// row's fp16 anchor is the scale of every block.
//
// out[a][n] = sum_b d[e][n][b] * sum_{k in block b} x[r(a)][k] * w[e][n][k]
//
// Work item: (chunk of up to 64 rows of one expert's group, tile of output
// columns: 256 of gate and of up, or 512 of down).  Eight waves; each wave
// owns NW 16-column subtiles of every matrix
// (gate and up for the SwiGLU epilogue, so h = silu(g) * u is formed in
// registers) and all M subtiles of the chunk, i.e. MS x NMAT x NW
// v_mfma_f32_16x16x32_bf16 tiles.
//
// K loop, one 256-wide scale block at a time:
//  - A (activations, gathered by assignment) is copied global -> LDS with
//    global_load_lds_dwordx4, two whole 512-byte row segments per
//    instruction, one block ahead of the MFMAs; 16-byte slots are
//    XOR-swizzled by row so every fragment read (16 rows x one 16-byte
//    column) is conflict-free.
//  - The weight planes come in the tile layout (rows grouped so that one K
//    block of a group is one 128-byte line: 4 rows of 32 index bytes, 8 rows
//    of 16 high-bit bytes, 8 rows of 16 sub-scale bytes per block pair), so
//    every copy into the ring moves whole lines; with rows kept whole, a line
//    would serve four to eight blocks and leave the L2 before the later
//    blocks read it.
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

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kMsMax = 4;                 // 16-row M subtiles per chunk
constexpr int kChunkRows = 16 * kMsMax;   // 64
constexpr int kKs = 8;                    // 32-wide K steps per 256 block

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory
// operations of this wave are outstanding, without waiting on LDS or exports.
constexpr int waitcnt_vm(int n) {
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}
// The same, also waiting for every outstanding LDS operation of the wave.
constexpr int waitcnt_vm_lgkm0(int n) {
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4);
}

__device__ __forceinline__ void copy16_to_lds(const void* g, uint4* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void*)(lds_wave_base), 16, 0, 0);
}

// LDS rings, one K block ahead of the MFMAs: A (activations) 2 slots and the
// weight group indices 2 slots, both copied global -> LDS (16-byte form
// only: the narrow forms write one dword per lane).  The slots are separate
// LDS arrays used alternately by an unrolled pair of steps, so the compiler
// can tell the slots being copied into from the slots being read.  Block
// scales are plain loads issued at the start of the block that uses them.
// Eight waves (two per SIMD) each cover 64 rows x 32 columns of each matrix,
// so one block is 256 MFMAs per SIMD (about 1.7 us at the MFMA rate) of
// latency cover, and the two waves of a SIMD hide each other's LDS latency.
constexpr int kASlotUnits = kMsMax * kKs * 64;   // 16-byte units per A slot (32 KB)
constexpr int kPairs = 512;                        // (matrix, column) pairs per tile
constexpr int kBQsUnits = kPairs * 2;              // 32 qs bytes per pair and block
constexpr int kBQhUnits = kPairs;                  // 16 qh bytes per pair and block

// Scheduling groups of one K block, K step KS onwards: vector-memory reads
// (the NV scale loads with the first step, one copy per step while NC
// copies last), then the step's NM MFMAs.
template <int KS, int NC, int NV, int NM>
__device__ __forceinline__ void order_block() {
    if constexpr (KS < kKs) {
        __builtin_amdgcn_sched_group_barrier(0x0020, (KS == 0 ? NV : 0) + (KS < NC ? 1 : 0), 0);
        __builtin_amdgcn_sched_group_barrier(0x0008, NM, 0);
        order_block<KS + 1, NC, NV, NM>();
    }
}
// Copies of the next block issued per K step by the gate/up item (two:
// measured 2-4 % faster than one per step or four, 4 % faster than all at
// the start of the block).
constexpr int kCopiesPerStep = 2;
// The same with the step's ND LDS reads (NQ more with the first step: the
// block's group indices) issued together between the copies and the MFMAs,
// so a wave waits once per step instead of once per fragment.
template <int KS, int NC, int NV, int NM, int ND, int NQ>
__device__ __forceinline__ void order_block_lds() {
    if constexpr (KS < kKs) {
        constexpr int left = NC - KS * kCopiesPerStep;
        constexpr int nc = left < 0 ? 0 : left > kCopiesPerStep ? kCopiesPerStep : left;
        __builtin_amdgcn_sched_group_barrier(0x0020, (KS == 0 ? NV : 0) + nc, 0);
        __builtin_amdgcn_sched_group_barrier(0x0100, ND + (KS == 0 ? NQ : 0), 0);
        __builtin_amdgcn_sched_group_barrier(0x0008, NM, 0);
        order_block_lds<KS + 1, NC, NV, NM, ND, NQ>();
    }
}

template <int NMAT, int NW>
struct BCur {
    uint2 q[NMAT][NW];
    uint32_t h[NMAT][NW];
};

// One row chunk x one column tile, all K blocks, MS = 16-row subtiles in the
// chunk (compile-time, so the inner loops have no branches).
// Sub-scaled signs: a column's sub-scale row has K/32 bytes, 8 per block;
// block kb's bytes are staged with its neighbour's as the 16-byte unit at
// byte 8 * (kb & ~1) of the row (K % 512 == 0, so every unit is 16-byte
// aligned and inside the row), in half kb & 1 of it.

template <int FMT, int EPI, bool DBG, int MS>
__device__ __forceinline__ void gemm_item(const ExpertArgs& p, uint4* __restrict__ a0,
                                          uint4* __restrict__ a1, uint4* __restrict__ q0,
                                          uint4* __restrict__ q1, uint4* __restrict__ h0,
                                          uint4* __restrict__ h1, const uint4* __restrict__ s_cb,
                                          const int* __restrict__ s_row,
                                          const int* __restrict__ s_asg, int e, int mrows, int nt) {
    constexpr int NMAT = (EPI == kEpiSwigluBf16) ? 2 : 1;
    constexpr int NW = (NMAT == 2) ? 2 : 4;
    constexpr int TILE_N = kWaves * NW * 16;
    static_assert(NMAT * TILE_N == kPairs, "tile / ring size mismatch");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keep it scalar
    const int lg = lane >> 4, lc = lane & 15;
    const int N = p.rows, K = p.cols, KB = K / 256;
    // grid1: qh uint16 per 32 weights and one scale per 256; sign1: one
    // sub-scale byte per 32 weights and one anchor per row
    const int d_row = (FMT == kSign1) ? 1 : K / 256;

    // activation row of each A copy this lane issues (fixed for the item)
    constexpr int ACOPIES = MS * 8 / kWaves;   // A copies per wave per block
    int arow[ACOPIES];
#pragma unroll
    for (int ii = 0; ii < ACOPIES; ++ii) arow[ii] = s_row[2 * (wave + kWaves * ii) + (lane >> 5)];

    int ncol[NW];
    uint32_t doff[NW];   // scale row of each of this lane's columns (element offset)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        ncol[w] = nt * TILE_N + (wave * NW + w) * 16 + lc;
        const int nn = ncol[w] < N ? ncol[w] : N - 1;
        doff[w] = static_cast<uint32_t>((e * N + nn) * d_row);
    }

    // A block -> slot: copy instruction i moves chunk rows 2i, 2i+1 whole
    // (2 x 512 contiguous bytes); lane l takes row 2i + l/32 and 16-byte
    // column c = (l % 32) ^ (row % 16), so LDS unit (row, c) sits at
    // 64*(row/2) + 32*(row%2) + (c ^ (row%16)).
    auto issue_a = [&](int kb, uint4* dst) {
#pragma unroll
        for (int ii = 0; ii < ACOPIES; ++ii) {   // MS*8 copies over the waves
            const int i = wave + kWaves * ii;
            const int row = 2 * i + (lane >> 5);
            const int c = (lane & 31) ^ (row & 15);
            const uint16_t* src = p.xb + static_cast<int64_t>(arow[ii]) * K + kb * 256 + c * 8;
            copy16_to_lds(src, dst + 64 * i);
        }
    };
    // Weight group indices of block kb for the tile's kPairs (matrix, column)
    // pairs: pair pi = m * TILE_N + column offset; qs 2 x 16 bytes and qh 16
    // bytes per pair: kQsCopies + kQhCopies copies per wave.
    constexpr int kQsCopies = kBQsUnits / 64 / kWaves;
    constexpr int kQhCopies = kBQhUnits / 64 / kWaves;
    auto issue_qs = [&](int r, int kb, uint4* dq, int ee, int ntt) {
        const int u0 = (wave * kQsCopies + r) * 64;   // uniform
        const int m = (u0 >> 1) / TILE_N;              // 32 pairs per copy
        const int pi = (u0 + lane) >> 1, half = lane & 1;
        int n = ntt * TILE_N + (pi % TILE_N);
        n = n < N ? n : N - 1;
        const uint8_t* base = (NMAT == 1 || m == 0) ? p.qs[0] : p.qs[1];
        // tile layout: block kb of rows 4g..4g+3 is the 128 bytes at group
        // line (g, kb), row n at 32 * (n % 4) in it
        copy16_to_lds(base + ((static_cast<int64_t>(ee) * (N / 4) + n / 4) * KB + kb) * 128 + (n % 4) * 32 +
                          half * 16,
                      dq + u0);
    };
    auto issue_qh = [&](int r, int kb, uint4* dh, int ee, int ntt) {
        const int u0 = (wave * kQhCopies + r) * 64;   // uniform
        const int m = u0 / TILE_N;                     // 64 pairs per copy
        const int pi = u0 + lane;
        int n = ntt * TILE_N + (pi % TILE_N);
        n = n < N ? n : N - 1;
        // tile layout, groups of 8 rows: the 16 bytes of row n sit at
        // 16 * (n % 8) of group line (g, kb) (high bits) or (g, kb / 2)
        // (sub-scales of a block pair)
        if constexpr (FMT == kSign1) {
            const uint8_t* base = (NMAT == 1 || m == 0) ? p.sc[0] : p.sc[1];
            copy16_to_lds(base + ((static_cast<int64_t>(ee) * (N / 8) + n / 8) * (KB / 2) + kb / 2) * 128 +
                              (n % 8) * 16,
                          dh + u0);
        } else {
            const uint8_t* base = reinterpret_cast<const uint8_t*>((NMAT == 1 || m == 0) ? p.qh[0] : p.qh[1]);
            copy16_to_lds(base + ((static_cast<int64_t>(ee) * (N / 8) + n / 8) * KB + kb) * 128 + (n % 8) * 16,
                          dh + u0);
        }
    };
    auto issue_b = [&](int kb, uint4* dq, uint4* dh) {
#pragma unroll
        for (int r = 0; r < kQsCopies; ++r) issue_qs(r, kb, dq, e, nt);
#pragma unroll
        for (int r = 0; r < kQhCopies; ++r) issue_qh(r, kb, dh, e, nt);
    };
    auto issue_a_row = [&](int ii, int kb, uint4* an, int row_src) {
        const int i = wave + kWaves * ii;
        const int row = 2 * i + (lane >> 5);
        const int cc = (lane & 31) ^ (row & 15);
        copy16_to_lds(p.xb + static_cast<int64_t>(row_src) * K + kb * 256 + cc * 8, an + 64 * i);
    };
    // Copy c of the next block (weights first: they come from HBM, the
    // activations mostly from L2).
    constexpr int NCOPIES = kQsCopies + kQhCopies + ACOPIES;
    static_assert(NCOPIES <= kKs, "one copy per K step");
    auto issue_copy = [&](int c, int kb, uint4* an, uint4* dq, uint4* dh) {
        if (c < kQsCopies) {
            issue_qs(c, kb, dq, e, nt);
        } else if (c < kQsCopies + kQhCopies) {
            issue_qh(c - kQsCopies, kb, dh, e, nt);
        } else {
            const int ii = c - kQsCopies - kQhCopies;
            issue_a_row(ii, kb, an, arow[ii]);
        }
    };

    f32x4 tot[MS][NMAT][NW];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int w = 0; w < NW; ++w) tot[ms][m][w] = f32x4{0.f, 0.f, 0.f, 0.f};

    issue_a(0, a0);
    issue_b(0, q0, h0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // One K block: scales of block kb (plain loads), then block kb's MFMAs
    // from `ac`, `qc`, `hc` with the copies of block kb+1 into the other
    // slots spread over the K steps (clamped to the last block, so the
    // instruction stream is the same every block): issued all at once after
    // the barrier, the eight waves' copies queue up in the address unit while
    // no MFMA runs.
    auto step = [&](int kb, const uint4* __restrict__ ac, uint4* __restrict__ an,
                    const uint4* __restrict__ qc, uint4* __restrict__ qn,
                    const uint4* __restrict__ hc, uint4* __restrict__ hn) {
        uint16_t dbits[NMAT][NW];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int w = 0; w < NW; ++w) dbits[m][w] = p.d[m][doff[w] + ((FMT == kSign1) ? 0 : kb)];
        const int kp = kb + 1 < KB ? kb + 1 : KB - 1;

        BCur<NMAT, NW> cur;
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int pi = m * TILE_N + (wave * NW + w) * 16 + lc;
                cur.q[m][w] = reinterpret_cast<const uint2*>(qc)[pi * 4 + lg];
                if constexpr (FMT == kSign1) {
                    // the two sub-scale bytes of lane group lg's 64 weights, in
                    // the half of the staged unit that holds block kb
                    cur.h[m][w] = reinterpret_cast<const uint16_t*>(hc)[pi * 8 + 4 * (kb & 1) + lg];
                } else {
                    cur.h[m][w] = reinterpret_cast<const uint32_t*>(hc)[pi * 4 + lg];
                }
            }

        auto frag_b = [&](int ks, bf16x8 (&bf)[NMAT][NW]) {
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const uint32_t qword = (ks < 4) ? cur.q[m][w].x : cur.q[m][w].y;
                    const uint32_t lo8 = (qword >> (8 * (ks & 3))) & 0xffu;
                    if constexpr (FMT == kSign1) {
                        // 8 weights: bf16 of their sub-scale (exact), with the
                        // sign bits of their sign byte from the mask table
                        const uint32_t sc = (cur.h[m][w] >> (8 * (ks >> 2) + 4 * ((ks >> 1) & 1))) & 15u;
                        const uint32_t sb = __builtin_bit_cast(uint32_t, static_cast<float>(sc)) >> 16;
                        const uint32_t pr = sb | (sb << 16);
                        const uint4 mk = s_cb[lo8];
                        bf[m][w] = __builtin_bit_cast(bf16x8, make_uint4(pr | mk.x, pr | mk.y, pr | mk.z, pr | mk.w));
                    } else {
                        const uint32_t hi3 = (cur.h[m][w] >> (16 * (ks >> 2) + 3 * (ks & 3))) & 7u;
                        bf[m][w] = __builtin_bit_cast(bf16x8, s_cb[lo8 | (hi3 << 8)]);
                    }
                }
        };
        auto frag_a = [&](int ks, bf16x8 (&af)[MS]) {
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const int row = ms * 16 + lc;
                const int c = 8 * lg + ks;
                af[ms] = __builtin_bit_cast(
                    bf16x8, ac[64 * (row >> 1) + 32 * (row & 1) + (c ^ (row & 15))]);
            }
        };

        // (two waves per SIMD hide each other's LDS latency, so fragments
        // are not double-buffered in registers)
        f32x4 blk[MS][NMAT][NW];
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
            // copies of block kb+1: one per step (down), kCopiesPerStep per
            // step (gate/up)
            constexpr int CPS = (NMAT == 2) ? kCopiesPerStep : 1;
#pragma unroll
            for (int c = ks * CPS; c < (ks + 1) * CPS; ++c)
                if (c < NCOPIES) issue_copy(c, kp, an, qn, hn);
            bf16x8 a_cur[MS];
            bf16x8 b_cur[NMAT][NW];
            frag_a(ks, a_cur);
            frag_b(ks, b_cur);
#pragma unroll
            for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int w = 0; w < NW; ++w)
                        blk[ms][m][w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            a_cur[ms], b_cur[m][w], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : blk[ms][m][w], 0, 0, 0);
        }
        // Instruction order of the block: the scale loads and the first copy,
        // then one K step of MFMAs, one more copy, and so on (the scheduler
        // would otherwise sink all copies to the end of the block).
        if constexpr (NMAT == 2)
            order_block_lds<0, NCOPIES, NMAT * NW, MS * NMAT * NW, MS + NMAT * NW, 2 * NMAT * NW>();
        else
            order_block<0, NCOPIES, NMAT * NW, MS * NMAT * NW>();
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float dsc = half_bits_to_float(dbits[m][w]);
#pragma unroll
                for (int ms = 0; ms < MS; ++ms)
#pragma unroll
                    for (int i = 0; i < 4; ++i) tot[ms][m][w][i] += dsc * blk[ms][m][w][i];
            }
        // Block kb+1's copies must have landed for every wave, and this
        // wave's LDS reads of the current slots must be complete before the
        // barrier lets the next block's copies overwrite them.  (The scales
        // were consumed above.)  A __syncthreads() would add a release fence;
        // the acquire fence after the raw barrier keeps the next block's LDS
        // reads from moving above it.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    for (int kb0 = 0; kb0 < KB; kb0 += 2) {
        step(kb0, a0, a1, q0, q1, h0, h1);
        if (kb0 + 1 < KB) step(kb0 + 1, a1, a0, q1, q0, h1, h0);
    }

    // epilogue: lane holds rows 16*ms + 4*lg + i of column ncol[w]
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
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
                } else if constexpr (EPI == kEpiF32Combine) {
                    // weighted combine: y[token][n] += topk_w[a] * out[a][n]
                    const int a = s_asg[r];
                    const float wa = static_cast<const float*>(p.out1)[a];
                    atomicAdd(static_cast<float*>(p.out0) + static_cast<int64_t>(a / p.top_k) * N + n,
                              wa * tot[ms][0][w][i]);
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
}

template <int FMT, int EPI, bool DBG>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(ExpertArgs p) {
    constexpr int NMAT = (EPI == kEpiSwigluBf16) ? 2 : 1;
    constexpr int NW = (NMAT == 2) ? 2 : 4;       // 16-col subtiles per wave per matrix
    constexpr int TILE_N = kWaves * NW * 16;      // 256 (gate/up) or 512 (down)

    __shared__ uint4 s_a0[kASlotUnits];
    __shared__ uint4 s_a1[kASlotUnits];
    __shared__ uint4 s_q0[kBQsUnits], s_q1[kBQsUnits];
    __shared__ uint4 s_h0[kBQhUnits], s_h1[kBQhUnits];
    __shared__ uint4 s_cb[kGridEntries];
    __shared__ int s_row[kChunkRows];
    __shared__ int s_asg[kChunkRows];
    __shared__ int s_info[kWaves];            // scan scratch (one per wave)
    __shared__ int s_misc[2];                 // scan carry, then the item's expert
    __shared__ int s_off[kMaxExperts + 1];    // expert_offsets
    __shared__ int s_cpre[kMaxExperts + 1];   // first chunk number of each expert
    static_assert(kMaxExperts == 2 * kThreads, "expert scan covers two experts per thread");

    const int tid = threadIdx.x;
    const int E = p.n_experts, N = p.rows;

    // grid1: bf16 codebook, entry i = 8 values in {-1,0,1} -> 8 bf16 (exact);
    // sign1: entry i = the bf16 sign bits (0x8000 where bit j of i is set) of
    // the 8 weights of sign byte i
    if constexpr (FMT == kSign1) {
        if (tid < 256) {
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j] = (((tid >> (2 * j)) & 1) ? 0x8000u : 0u) | (((tid >> (2 * j + 1)) & 1) ? 0x80000000u : 0u);
            s_cb[tid] = make_uint4(o[0], o[1], o[2], o[3]);
        }
    } else {
    for (int i = tid; i < kGridEntries; i += kThreads) {
        const uint2 raw = reinterpret_cast<const uint2*>(p.grid)[i];
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t wv = (j < 2) ? raw.x : raw.y;
            const int v0 = static_cast<int8_t>((wv >> (16 * (j & 1))) & 0xffu);
            const int v1 = static_cast<int8_t>((wv >> (16 * (j & 1) + 8)) & 0xffu);
            const uint32_t c0 = __builtin_bit_cast(uint32_t, static_cast<float>(v0)) >> 16;
            const uint32_t c1 = __builtin_bit_cast(uint32_t, static_cast<float>(v1)) >> 16;
            o[j] = c0 | (c1 << 16);
        }
        s_cb[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    }
    // Chunks of up to 64 rows are numbered in expert order; s_cpre[e] is the
    // number of expert e's first chunk (exclusive scan of the chunk counts),
    // s_cpre[E] the total.
    {
        int run = 0;
        for (int half = 0; half < 2; ++half) {
            const int e = tid + half * kThreads;
            int nch = 0;
            if (e < E) {
                const int o0 = p.offsets[e], o1 = p.offsets[e + 1];
                s_off[e] = o0;
                nch = (o1 - o0 + kChunkRows - 1) / kChunkRows;
            }
            const int ex = block_exclusive_scan(nch, s_info);
            if (e < E) s_cpre[e] = run + ex;
            if (tid == kThreads - 1) s_misc[0] = run + ex + nch;
            __syncthreads();
            run = s_misc[0];
            __syncthreads();
        }
        if (tid == 0) {
            s_cpre[E] = run;
            s_off[E] = p.offsets[E];
        }
    }
    __syncthreads();

    const int C = s_cpre[E];
    const int NT = (N + TILE_N - 1) / TILE_N;
    const int per_xcd = ((C + 7) / 8) * NT;
    const int n_items = 8 * per_xcd;

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int xcd = item & 7, j = item >> 3;
        const int c = xcd + 8 * (j / NT), nt = j % NT;
        if (c >= C) continue;   // uniform over the workgroup
        // Exactly one expert has s_cpre[e] <= c < s_cpre[e + 1] (experts
        // without rows have an empty range).
        for (int e = tid; e < E; e += kThreads)
            if (s_cpre[e] <= c && c < s_cpre[e + 1]) s_misc[1] = e;
        __syncthreads();
        const int e = s_misc[1];
        const int cbeg = s_off[e] + (c - s_cpre[e]) * kChunkRows;
        const int mrows = min(kChunkRows, s_off[e + 1] - cbeg);
        if (tid < kChunkRows) {
            const int r = tid < mrows ? tid : 0;
            const int a = p.sorted[cbeg + r];
            s_asg[tid] = a;
            s_row[tid] = p.act_by_token ? a / p.top_k : a;
        }
        __syncthreads();
        switch ((mrows + 15) >> 4) {
            case 1: gemm_item<FMT, EPI, DBG, 1>(p, s_a0, s_a1, s_q0, s_q1, s_h0, s_h1, s_cb, s_row, s_asg, e, mrows, nt); break;
            case 2: gemm_item<FMT, EPI, DBG, 2>(p, s_a0, s_a1, s_q0, s_q1, s_h0, s_h1, s_cb, s_row, s_asg, e, mrows, nt); break;
            case 3: gemm_item<FMT, EPI, DBG, 3>(p, s_a0, s_a1, s_q0, s_q1, s_h0, s_h1, s_cb, s_row, s_asg, e, mrows, nt); break;
            default: gemm_item<FMT, EPI, DBG, 4>(p, s_a0, s_a1, s_q0, s_q1, s_h0, s_h1, s_cb, s_row, s_asg, e, mrows, nt); break;
        }
        __syncthreads();   // s_row / s_asg / rings are reused by the next item
    }
}

template <int FMT, int EPI, bool DBG>
hipError_t launch_one(const ExpertArgs& a, hipStream_t s) {
    // persistent: one workgroup per compute unit, a multiple of 8 (XCDs)
    int grid = cu_count();
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL((k_gemm<FMT, EPI, DBG>), dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool gemm_supported(Fmt fmt, int rows, int cols, int epi) {
    if (cols % 256 != 0 || rows < 1 || rows % kTileRows != 0) return false;
    if (fmt == kSign1 && cols % 512 != 0) return false;   // whole 16-byte sub-scale units
    if (fmt != kGrid1 && fmt != kSign1) return false;
    return epi == kEpiF32 || epi == kEpiSwigluBf16 || epi == kEpiF32Combine;
}

template <int FMT>
hipError_t launch_fmt(Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (epi == kEpiF32) return a.debug ? launch_one<FMT, kEpiF32, true>(a, s) : launch_one<FMT, kEpiF32, false>(a, s);
    if (epi == kEpiSwigluBf16)
        return a.debug ? launch_one<FMT, kEpiSwigluBf16, true>(a, s) : launch_one<FMT, kEpiSwigluBf16, false>(a, s);
    if (epi == kEpiF32Combine)
        return a.debug ? launch_one<FMT, kEpiF32Combine, true>(a, s) : launch_one<FMT, kEpiF32Combine, false>(a, s);
    return hipErrorInvalidValue;
}

hipError_t launch_gemm(Fmt fmt, Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (fmt == kSign1) return launch_fmt<kSign1>(epi, a, s);
    if (fmt == kGrid1) return launch_fmt<kGrid1>(epi, a, s);
    return hipErrorInvalidValue;
}

}  // namespace pqk
