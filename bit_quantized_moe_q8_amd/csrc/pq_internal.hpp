// Internal interface between the C-ABI layer (pq_api.cpp) and the kernel
// translation units.  Not installed; the public interface is include/pq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pq.h"

namespace pqk {

constexpr int kGridEntries = 2048;  // grid1 codebook entries of 8 int8 values
constexpr int kMaxExperts = 1024;   // experts per layer accepted by every entry point
constexpr int kTileRows = 8;        // rows of the tile layout's largest row group
// Assignments from which an expert of a large decode batch goes to the
// int8-MFMA tile kernel (measured on the skewed 64-token decode: 6 and 8
// best, 4 and 16 slower); also the least token count for that split.
constexpr int kHeavyMin = 8;

// Number of compute units of the current device (cached per device).
int cu_count();

hipError_t launch_quantize_q8(const float* x, int64_t n_blocks, int8_t* xq, float* xd,
                              hipStream_t s);

hipError_t launch_route_topk(const float* logits, int n_tokens, int n_experts, int top_k,
                             int32_t* ids, float* w, hipStream_t s);

hipError_t launch_group(const int32_t* ids, int n_assign, int n_experts, int32_t* offsets,
                        int32_t* sorted, int32_t* active, int32_t* n_active, hipStream_t s);

// q8 + route + group: one workgroup for up to 16 tokens (the sizes
// decode_prep_one_launch accepts), else q8 and routing in one launch and the
// grouping in a second.
hipError_t launch_decode_prep(const float* x, const float* logits, int n_tokens, int hidden,
                              int n_experts, int top_k, int8_t* xq, float* xd, int32_t* ids,
                              float* w, int32_t* offsets, int32_t* sorted, int32_t* active,
                              int32_t* n_active, float* y_zero, hipStream_t s);
bool decode_prep_one_launch(int n_tokens, int n_experts, int top_k);

// Count of 2-bit codes equal to 3 in n_bytes of ternary qs (one workgroup).
hipError_t launch_validate_ternary(const uint8_t* qs, int64_t n_bytes, int32_t* n_bad, hipStream_t s);

hipError_t launch_combine(const float* out, const float* w, int n_tokens, int top_k, int rows,
                          float* y, hipStream_t s);

enum Fmt { kTernary = 0, kGrid1 = 1, kSign1 = 2 };
enum Epi { kEpiF32 = 0, kEpiSwigluQ8 = 1, kEpiSwigluBf16 = 2, kEpiF32Combine = 3 };

// Everything an expert kernel needs; index 0 is `w`, index 1 is `w_up`.
struct ExpertArgs {
    const uint8_t* qs[2];
    const uint16_t* qh[2];
    const uint16_t* d[2];   // sign1: one anchor per row
    const uint8_t* sc[2];   // sign1: 4-bit sub-scales, two per byte
    const int8_t* grid;
    int rows, cols, n_experts;
    const int32_t* offsets;
    const int32_t* sorted;
    const int32_t* active;
    const int32_t* n_active;
    int n_tokens, top_k, act_by_token;
    const int8_t* xq;    // decode activations
    const float* xd;
    const uint16_t* xb;  // prefill activations (bf16 bits)
    void* out0;
    void* out1;
    int32_t* dbg_isums[2];
    float* dbg_g;
    float* dbg_u;
    float* dbg_h;
    bool debug;
    // Experts with at least this many assignments are left to the int8-MFMA
    // tile kernel (which takes exactly those); 0: the mat-vec takes all.
    int heavy_min;
    // The matrix of the single mat-vec from fp32 activations.
    int expert0;
};

// Kernels (PQ_PLAN_* flags) of a q8 expert call of the mat-vec family on
// argument sizes the entry point has accepted: the one decision every
// launcher of that family and pq_plan share.
int plan_matvec(int n_tokens, int top_k, int n_experts, int cols, bool debug);

// Whether a mat-vec call whose plan has PQ_PLAN_TILE_Q8 | PQ_PLAN_MATVEC_PAIRS
// runs both in one launch (PQ_PLAN_MIXED).
bool mixed_planned(Fmt fmt, Epi epi, int n_tokens, int top_k, int cols);

// Decode mat-vec; returns hipErrorInvalidValue when no kernel matches cols.
hipError_t launch_matvec(Fmt fmt, Epi epi, const ExpertArgs& a, hipStream_t s);

// Decode mat-vec at one token (n_tokens == 1): one workgroup per (slot,
// tile), every weight row of the tile in flight at once.
hipError_t launch_matvec_tok1(Fmt fmt, Epi epi, const ExpertArgs& a, hipStream_t s);

// One-token gate/up with its own routing and q8 (see the one-token kernel):
// reads x [cols] and logits [n_experts]; writes ids, w [top_k], the grouping
// (offsets [n_experts+1], sorted [top_k], active [top_k], n_active) and
// zeros y [cols]; hq/hd through a.out0/out1 as the SwiGLU q8 epilogue.
struct RouteArgs {
    const float* x;
    const float* logits;
    int32_t* ids;
    float* w;
    int32_t* offsets;
    int32_t* sorted;
    int32_t* active;
    int32_t* n_active;
    float* y;
};
hipError_t launch_decode1_gate_up(Fmt fmt, const ExpertArgs& a, const RouteArgs& r, hipStream_t s);
bool matvec_supported(Fmt fmt, int cols);

// One mat-vec from fp32 activations x [cols] in one launch: the one-token
// kernel quantizing x itself (F32 epilogue into a.out0 [rows], matrix
// a.expert0).
hipError_t launch_matvec_x32(Fmt fmt, const ExpertArgs& a, const float* x, hipStream_t s);

// Grouped int8-MFMA tile over q8 activations: the mat-vec's arithmetic and
// epilogues for the experts with at least a.heavy_min (>= 1) assignments.
hipError_t launch_tile_q8(Fmt fmt, Epi epi, const ExpertArgs& a, hipStream_t s);
bool tile_q8_supported(int cols);

// Prefill dequant-per-tile GEMM (grid1 or sign1, bf16 MFMA).
hipError_t launch_gemm(Fmt fmt, Epi epi, const ExpertArgs& a, hipStream_t s);

// Tile layout of one packed plane: src [rows][nb][unit] bytes ->
// dst [rows / R][nb][R][unit] with R = 128 / unit (unit 16 or 32 bytes,
// rows % R == 0, both 16-byte aligned, no overlap).
hipError_t launch_tile_layout(const void* src, void* dst, int64_t rows, int nb, int unit, hipStream_t s);
bool gemm_supported(Fmt fmt, int rows, int cols, int epi);

// Measurement aids (k_peak.hip): a read stream over `bytes` of device memory,
// and `workgroups` x peak_mfma_waves_per_workgroup() waves each issuing
// iters x peak_mfma_chains() bf16 16x16x32 MFMAs.
hipError_t launch_peak_read(const void* p, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_peak_mfma(int workgroups, int iters, float* sink, hipStream_t s);
int peak_mfma_waves_per_workgroup();
int peak_mfma_chains();

}  // namespace pqk
