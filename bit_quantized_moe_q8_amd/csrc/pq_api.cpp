// C-ABI entry points of libpq (declared in include/pq.h): argument checks on
// the host, then kernel launches on the caller's stream.  Every check runs
// before the first HIP call; no entry point allocates or synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <type_traits>

#include "../../include/pq.h"
#include "pq_internal.hpp"

namespace pqk {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
}  // namespace

int cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        g_cu_count[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

int plan_matvec(int n_tokens, int top_k, int n_experts, int cols, bool debug) {
    if (n_tokens <= 0) return 0;
    const int dbg = debug ? PQ_PLAN_DEBUG : 0;
    // one token: the one-token kernel (its debug outputs come from the
    // grouped kernel, one assignment group per expert)
    if (n_tokens == 1) return (debug ? PQ_PLAN_MATVEC : PQ_PLAN_MATVEC_TOK1) | dbg;
    const int64_t A = int64_t(n_tokens) * top_k;
    if (A <= n_experts) return PQ_PLAN_MATVEC | dbg;
    // more assignments than experts: pairs of assignments per work item, and
    // in a batch of kHeavyMin+ tokens the experts holding kHeavyMin+
    // assignments on the int8-MFMA tile
    const bool heavy = n_tokens >= kHeavyMin && tile_q8_supported(cols);
    return PQ_PLAN_MATVEC_PAIRS | (heavy ? PQ_PLAN_TILE_Q8 : 0) | dbg;
}

}  // namespace pqk

namespace {

using pqk::kMaxExperts;
constexpr int kMaxTopK = 16;
constexpr int64_t kMaxAssign = int64_t(1) << 20;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

pq_status from_hip(hipError_t e) { return e == hipSuccess ? PQ_OK : PQ_ERR_HIP; }

hipStream_t as_stream(pq_stream s) { return reinterpret_cast<hipStream_t>(s); }

pq_status check_groups(const pq_groups* g) {
    if (!g || !g->expert_offsets || !g->sorted_assign || !g->active_experts || !g->n_active)
        return PQ_ERR_NULL;
    if (g->n_experts < 1 || g->n_experts > kMaxExperts) return PQ_ERR_SHAPE;
    if (g->top_k < 1 || g->top_k > kMaxTopK || g->top_k > g->n_experts) return PQ_ERR_SHAPE;
    if (g->n_tokens < 0 || int64_t(g->n_tokens) * g->top_k > kMaxAssign) return PQ_ERR_SHAPE;
    return PQ_OK;
}

pq_status check_dims(int n_experts, int rows, int cols, const pq_groups* g) {
    if (n_experts != g->n_experts) return PQ_ERR_SHAPE;
    if (rows < 1 || cols < 256 || cols % 256 != 0) return PQ_ERR_SHAPE;
    if (int64_t(rows) * cols > (int64_t(1) << 31)) return PQ_ERR_SHAPE;
    return PQ_OK;
}

void fill_groups(pqk::ExpertArgs& a, const pq_groups* g) {
    a.offsets = g->expert_offsets;
    a.sorted = g->sorted_assign;
    a.active = g->active_experts;
    a.n_active = g->n_active;
    a.n_tokens = g->n_tokens;
    a.top_k = g->top_k;
    a.n_experts = g->n_experts;
}

void fill_debug(pqk::ExpertArgs& a, const pq_debug* dbg) {
    a.debug = dbg != nullptr;
    a.dbg_isums[0] = dbg ? dbg->isums : nullptr;
    a.dbg_isums[1] = dbg ? dbg->isums_up : nullptr;
    a.dbg_g = dbg ? dbg->g : nullptr;
    a.dbg_u = dbg ? dbg->u : nullptr;
    a.dbg_h = dbg ? dbg->h : nullptr;
}

pq_status check_epilogue_outputs(int epilogue, const void* up, int rows, void* out0, void* out1,
                                 bool decode) {
    if (!out0) return PQ_ERR_NULL;
    if (epilogue == PQ_EPI_F32) {
        if (!aligned(out0, 4)) return PQ_ERR_ALIGN;
        return PQ_OK;
    }
    if (epilogue == PQ_EPI_F32_COMBINE) {
        if (!out1) return PQ_ERR_NULL;
        if (!aligned(out0, 4) || !aligned(out1, 4)) return PQ_ERR_ALIGN;
        return PQ_OK;
    }
    if ((decode && epilogue != PQ_EPI_SWIGLU_Q8) || (!decode && epilogue != PQ_EPI_SWIGLU_BF16))
        return PQ_ERR_UNSUPPORTED;
    if (!up) return PQ_ERR_NULL;
    if (rows % 32 != 0) return PQ_ERR_SHAPE;
    if (decode) {
        if (!out1) return PQ_ERR_NULL;
        if (!aligned(out1, 4)) return PQ_ERR_ALIGN;
    } else if (!aligned(out0, 2)) {
        return PQ_ERR_ALIGN;
    }
    return PQ_OK;
}

template <typename F>
pq_status guarded(F&& f) {
    try {
        return f();
    } catch (...) {
        return PQ_ERR_HIP;
    }
}

// The packed code plane of an expert tensor (ternary/grid1 qs, sign1 signs).
const uint8_t* codes_of(const pq_ternary_w* w) { return w->qs; }
const uint8_t* codes_of(const pq_grid1_w* w) { return w->qs; }
const uint8_t* codes_of(const pq_sign1_w* w) { return w->signs; }

// One-token gate/up with its own routing and q8; W is pq_ternary_w,
// pq_grid1_w or pq_sign1_w.
template <typename W>
pq_status decode1_gate_up(pqk::Fmt fmt, const float* x, const float* logits, int32_t n_experts,
                          int32_t top_k, const W* gate, const W* up, int32_t* topk_ids,
                          float* topk_w, int32_t* expert_offsets, int32_t* sorted_assign,
                          int32_t* active_experts, int32_t* n_active, int8_t* hq, float* hd,
                          float* y_zero, pq_stream stream) {
    if (!x || !logits || !gate || !up || !topk_ids || !topk_w || !expert_offsets || !sorted_assign ||
        !active_experts || !n_active || !hq || !hd)
        return PQ_ERR_NULL;
    const W* ws[2] = {gate, up};
    for (const W* w : ws) {
        if (!codes_of(w) || !w->d) return PQ_ERR_NULL;
        if (!aligned(codes_of(w), 16) || !aligned(w->d, 2)) return PQ_ERR_ALIGN;
    }
    const int8_t* grid = nullptr;
    const uint16_t* qh[2] = {nullptr, nullptr};
    const uint8_t* sc[2] = {nullptr, nullptr};
    if constexpr (std::is_same<W, pq_sign1_w>::value) {
        for (int i = 0; i < 2; ++i) {
            if (!ws[i]->sc) return PQ_ERR_NULL;
            if (!aligned(ws[i]->sc, 4)) return PQ_ERR_ALIGN;
            sc[i] = ws[i]->sc;
        }
    }
    if constexpr (std::is_same<W, pq_grid1_w>::value) {
        for (int i = 0; i < 2; ++i) {
            if (!ws[i]->qh || !ws[i]->grid) return PQ_ERR_NULL;
            if (!aligned(ws[i]->qh, 8) || !aligned(ws[i]->grid, 16)) return PQ_ERR_ALIGN;
            qh[i] = ws[i]->qh;
        }
        grid = gate->grid;   // used for both, as by the mat-vec
    }
    if (n_experts < 1 || n_experts > kMaxExperts) return PQ_ERR_SHAPE;
    if (top_k < 1 || top_k > kMaxTopK || top_k > n_experts) return PQ_ERR_SHAPE;
    const int I = gate->rows, H = gate->cols;
    if (gate->n_experts != n_experts || up->n_experts != n_experts) return PQ_ERR_SHAPE;
    if (up->rows != I || up->cols != H) return PQ_ERR_SHAPE;
    if (I < 32 || I % 32 != 0 || H < 256 || H % 256 != 0) return PQ_ERR_SHAPE;
    if (int64_t(I) * H > (int64_t(1) << 31)) return PQ_ERR_SHAPE;
    if (!pqk::matvec_supported(fmt, H)) return PQ_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(hd, 4) || !aligned(topk_ids, 4) ||
        !aligned(topk_w, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_assign, 4) ||
        !aligned(active_experts, 4) || !aligned(n_active, 4) || (y_zero && !aligned(y_zero, 4)))
        return PQ_ERR_ALIGN;

    pqk::ExpertArgs a{};
    a.qs[0] = codes_of(gate);
    a.qs[1] = codes_of(up);
    a.d[0] = gate->d;
    a.d[1] = up->d;
    a.qh[0] = qh[0];
    a.qh[1] = qh[1];
    a.sc[0] = sc[0];
    a.sc[1] = sc[1];
    a.grid = grid;
    a.rows = I;
    a.cols = H;
    a.n_experts = n_experts;
    a.n_tokens = 1;
    a.top_k = top_k;
    a.act_by_token = 1;
    a.out0 = hq;
    a.out1 = hd;
    const pqk::RouteArgs ra{x, logits, topk_ids, topk_w, expert_offsets, sorted_assign,
                            active_experts, n_active, y_zero};
    return from_hip(pqk::launch_decode1_gate_up(fmt, a, ra, as_stream(stream)));
}

// Validation and argument set-up shared by the q8 expert entry points (the
// mat-vec and the int8-MFMA tile); `supported` checks the row length for the
// kernel family.  *run is false when there is nothing to launch.
template <typename Supported>
pq_status ternary_args(const pq_ternary_w* w, const pq_ternary_w* w_up, const pq_groups* g,
                       const int8_t* xq, const float* xd, int32_t act_by_token, int32_t epilogue,
                       void* out0, void* out1, const pq_debug* dbg, Supported supported,
                       pqk::ExpertArgs& a, bool* run) {
    *run = false;
    if (!w || !w->qs || !w->d) return PQ_ERR_NULL;
    pq_status st = check_groups(g);
    if (st != PQ_OK) return st;
    if ((st = check_dims(w->n_experts, w->rows, w->cols, g)) != PQ_OK) return st;
    if ((st = check_epilogue_outputs(epilogue, w_up, w->rows, out0, out1, true)) != PQ_OK)
        return st;
    if (epilogue == PQ_EPI_F32_COMBINE && act_by_token) return PQ_ERR_UNSUPPORTED;
    if (epilogue == PQ_EPI_SWIGLU_Q8) {
        if (!w_up->qs || !w_up->d) return PQ_ERR_NULL;
        if (w_up->n_experts != w->n_experts || w_up->rows != w->rows || w_up->cols != w->cols)
            return PQ_ERR_SHAPE;
        if (!aligned(w_up->qs, 16) || !aligned(w_up->d, 2)) return PQ_ERR_ALIGN;
    }
    if (!aligned(w->qs, 16) || !aligned(w->d, 2)) return PQ_ERR_ALIGN;
    if (!supported(pqk::kTernary, w->cols)) return PQ_ERR_UNSUPPORTED;
    if (g->n_tokens == 0) return PQ_OK;
    if (!xq || !xd) return PQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(xd, 4)) return PQ_ERR_ALIGN;
    a = pqk::ExpertArgs{};
    a.qs[0] = w->qs;
    a.d[0] = w->d;
    a.qs[1] = w_up ? w_up->qs : nullptr;
    a.d[1] = w_up ? w_up->d : nullptr;
    a.rows = w->rows;
    a.cols = w->cols;
    fill_groups(a, g);
    a.act_by_token = act_by_token ? 1 : 0;
    a.xq = xq;
    a.xd = xd;
    a.out0 = out0;
    a.out1 = out1;
    fill_debug(a, dbg);
    *run = true;
    return PQ_OK;
}

template <typename Supported>
pq_status grid1_args(const pq_grid1_w* w, const pq_grid1_w* w_up, const pq_groups* g,
                     const int8_t* xq, const float* xd, int32_t act_by_token, int32_t epilogue,
                     void* out0, void* out1, const pq_debug* dbg, Supported supported,
                     pqk::ExpertArgs& a, bool* run) {
    *run = false;
    if (!w || !w->qs || !w->qh || !w->d || !w->grid) return PQ_ERR_NULL;
    pq_status st = check_groups(g);
    if (st != PQ_OK) return st;
    if ((st = check_dims(w->n_experts, w->rows, w->cols, g)) != PQ_OK) return st;
    if ((st = check_epilogue_outputs(epilogue, w_up, w->rows, out0, out1, true)) != PQ_OK)
        return st;
    if (epilogue == PQ_EPI_F32_COMBINE && act_by_token) return PQ_ERR_UNSUPPORTED;
    if (epilogue == PQ_EPI_SWIGLU_Q8) {
        if (!w_up->qs || !w_up->qh || !w_up->d) return PQ_ERR_NULL;
        if (w_up->n_experts != w->n_experts || w_up->rows != w->rows || w_up->cols != w->cols)
            return PQ_ERR_SHAPE;
        if (!aligned(w_up->qs, 16) || !aligned(w_up->qh, 8) || !aligned(w_up->d, 2))
            return PQ_ERR_ALIGN;
    }
    if (!aligned(w->qs, 16) || !aligned(w->qh, 8) || !aligned(w->d, 2) || !aligned(w->grid, 16))
        return PQ_ERR_ALIGN;
    if (!supported(pqk::kGrid1, w->cols)) return PQ_ERR_UNSUPPORTED;
    if (g->n_tokens == 0) return PQ_OK;
    if (!xq || !xd) return PQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(xd, 4)) return PQ_ERR_ALIGN;
    a = pqk::ExpertArgs{};
    a.qs[0] = w->qs;
    a.qh[0] = w->qh;
    a.d[0] = w->d;
    a.qs[1] = w_up ? w_up->qs : nullptr;
    a.qh[1] = w_up ? w_up->qh : nullptr;
    a.d[1] = w_up ? w_up->d : nullptr;
    a.grid = w->grid;
    a.rows = w->rows;
    a.cols = w->cols;
    fill_groups(a, g);
    a.act_by_token = act_by_token ? 1 : 0;
    a.xq = xq;
    a.xd = xd;
    a.out0 = out0;
    a.out1 = out1;
    fill_debug(a, dbg);
    *run = true;
    return PQ_OK;
}

template <typename Supported>
pq_status sign1_args(const pq_sign1_w* w, const pq_sign1_w* w_up, const pq_groups* g,
                     const int8_t* xq, const float* xd, int32_t act_by_token, int32_t epilogue,
                     void* out0, void* out1, const pq_debug* dbg, Supported supported,
                     pqk::ExpertArgs& a, bool* run) {
    *run = false;
    if (!w || !w->signs || !w->sc || !w->d) return PQ_ERR_NULL;
    pq_status st = check_groups(g);
    if (st != PQ_OK) return st;
    if ((st = check_dims(w->n_experts, w->rows, w->cols, g)) != PQ_OK) return st;
    if ((st = check_epilogue_outputs(epilogue, w_up, w->rows, out0, out1, true)) != PQ_OK)
        return st;
    if (epilogue == PQ_EPI_F32_COMBINE && act_by_token) return PQ_ERR_UNSUPPORTED;
    if (epilogue == PQ_EPI_SWIGLU_Q8) {
        if (!w_up->signs || !w_up->sc || !w_up->d) return PQ_ERR_NULL;
        if (w_up->n_experts != w->n_experts || w_up->rows != w->rows || w_up->cols != w->cols)
            return PQ_ERR_SHAPE;
        if (!aligned(w_up->signs, 16) || !aligned(w_up->sc, 4) || !aligned(w_up->d, 2))
            return PQ_ERR_ALIGN;
    }
    if (!aligned(w->signs, 16) || !aligned(w->sc, 4) || !aligned(w->d, 2)) return PQ_ERR_ALIGN;
    if (!supported(pqk::kSign1, w->cols)) return PQ_ERR_UNSUPPORTED;
    if (g->n_tokens == 0) return PQ_OK;
    if (!xq || !xd) return PQ_ERR_NULL;
    if (!aligned(xq, 16) || !aligned(xd, 4)) return PQ_ERR_ALIGN;
    a = pqk::ExpertArgs{};
    a.qs[0] = w->signs;
    a.sc[0] = w->sc;
    a.d[0] = w->d;
    a.qs[1] = w_up ? w_up->signs : nullptr;
    a.sc[1] = w_up ? w_up->sc : nullptr;
    a.d[1] = w_up ? w_up->d : nullptr;
    a.rows = w->rows;
    a.cols = w->cols;
    fill_groups(a, g);
    a.act_by_token = act_by_token ? 1 : 0;
    a.xq = xq;
    a.xd = xd;
    a.out0 = out0;
    a.out1 = out1;
    fill_debug(a, dbg);
    *run = true;
    return PQ_OK;
}

pq_status launch_matvec_any(pqk::Fmt fmt, int32_t epilogue, const pqk::ExpertArgs& a,
                            const pq_debug* dbg, pq_stream stream) {
    const int plan = pqk::plan_matvec(a.n_tokens, a.top_k, a.n_experts, a.cols, dbg != nullptr);
    if (plan & PQ_PLAN_MATVEC_TOK1)
        return from_hip(pqk::launch_matvec_tok1(fmt, static_cast<pqk::Epi>(epilogue), a, as_stream(stream)));
    return from_hip(pqk::launch_matvec(fmt, static_cast<pqk::Epi>(epilogue), a, as_stream(stream)));
}

pq_status launch_tile_all(pqk::Fmt fmt, int32_t epilogue, pqk::ExpertArgs& a, pq_stream stream) {
    a.heavy_min = 1;   // every active expert
    return from_hip(pqk::launch_tile_q8(fmt, static_cast<pqk::Epi>(epilogue), a, as_stream(stream)));
}

}  // namespace

extern "C" {

int32_t pq_abi_version(void) { return PQ_ABI_VERSION; }

const char* pq_status_str(pq_status s) {
    switch (s) {
        case PQ_OK: return "ok";
        case PQ_ERR_NULL: return "null pointer argument";
        case PQ_ERR_SHAPE: return "size out of range or inconsistent";
        case PQ_ERR_ALIGN: return "misaligned pointer";
        case PQ_ERR_UNSUPPORTED: return "no kernel for these (valid) arguments";
        case PQ_ERR_HIP: return "HIP runtime or launch failure";
        case PQ_ERR_SELFTEST: return "self test: a known answer did not come out";
    }
    return "unknown status";
}

pq_status pq_quantize_act_q8(const float* x, int32_t n_rows, int32_t cols, int8_t* xq, float* xd,
                             pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (n_rows < 0 || cols < 32 || cols % 32 != 0) return PQ_ERR_SHAPE;
        if (n_rows == 0) return PQ_OK;
        if (!x || !xq || !xd) return PQ_ERR_NULL;
        if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xd, 4)) return PQ_ERR_ALIGN;
        const int64_t n_blocks = int64_t(n_rows) * (cols / 32);
        return from_hip(pqk::launch_quantize_q8(x, n_blocks, xq, xd, as_stream(stream)));
    });
}

pq_status pq_moe_route_topk(const float* logits, int32_t n_tokens, int32_t n_experts,
                            int32_t top_k, int32_t* topk_ids, float* topk_w, pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (n_tokens < 0 || n_experts < 1 || n_experts > kMaxExperts) return PQ_ERR_SHAPE;
        if (top_k < 1 || top_k > kMaxTopK || top_k > n_experts) return PQ_ERR_SHAPE;
        if (n_tokens == 0) return PQ_OK;
        if (!logits || !topk_ids || !topk_w) return PQ_ERR_NULL;
        if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return PQ_ERR_ALIGN;
        return from_hip(pqk::launch_route_topk(logits, n_tokens, n_experts, top_k, topk_ids,
                                               topk_w, as_stream(stream)));
    });
}

pq_status pq_group_tokens_by_expert(const int32_t* topk_ids, int32_t n_tokens, int32_t top_k,
                                    int32_t n_experts, int32_t* expert_offsets,
                                    int32_t* sorted_assign, int32_t* active_experts,
                                    int32_t* n_active, pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (n_tokens < 0 || n_experts < 1 || n_experts > kMaxExperts) return PQ_ERR_SHAPE;
        if (top_k < 1 || top_k > kMaxTopK || top_k > n_experts) return PQ_ERR_SHAPE;
        const int64_t A = int64_t(n_tokens) * top_k;
        if (A > kMaxAssign) return PQ_ERR_SHAPE;
        if (!expert_offsets || !active_experts || !n_active) return PQ_ERR_NULL;
        if (A > 0 && (!topk_ids || !sorted_assign)) return PQ_ERR_NULL;
        if (!aligned(expert_offsets, 4) || !aligned(active_experts, 4) || !aligned(n_active, 4) ||
            !aligned(topk_ids, 4) || !aligned(sorted_assign, 4))
            return PQ_ERR_ALIGN;
        return from_hip(pqk::launch_group(topk_ids, int(A), n_experts, expert_offsets,
                                          sorted_assign, active_experts, n_active,
                                          as_stream(stream)));
    });
}

pq_status pq_moe_decode_prep(const float* x, const float* logits, int32_t n_tokens,
                             int32_t hidden, int32_t n_experts, int32_t top_k, int8_t* xq,
                             float* xd, int32_t* topk_ids, float* topk_w,
                             int32_t* expert_offsets, int32_t* sorted_assign,
                             int32_t* active_experts, int32_t* n_active, float* y_zero,
                             pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (n_tokens < 0 || hidden < 0 || hidden % 32 != 0) return PQ_ERR_SHAPE;
        if (n_experts < 1 || n_experts > kMaxExperts) return PQ_ERR_SHAPE;
        if (top_k < 1 || top_k > kMaxTopK || top_k > n_experts) return PQ_ERR_SHAPE;
        if (int64_t(n_tokens) * top_k > kMaxAssign) return PQ_ERR_SHAPE;
        if (!expert_offsets || !active_experts || !n_active) return PQ_ERR_NULL;
        if (n_tokens > 0 && (!x || !logits || !xq || !xd || !topk_ids || !topk_w || !sorted_assign))
            return PQ_ERR_NULL;
        if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(logits, 4) ||
            !aligned(topk_ids, 4) || !aligned(topk_w, 4) || !aligned(expert_offsets, 4) ||
            !aligned(sorted_assign, 4) || !aligned(active_experts, 4) || !aligned(n_active, 4) ||
            !aligned(y_zero, 4))
            return PQ_ERR_ALIGN;
        return from_hip(pqk::launch_decode_prep(x, logits, n_tokens, hidden, n_experts, top_k, xq,
                                                xd, topk_ids, topk_w, expert_offsets,
                                                sorted_assign, active_experts, n_active, y_zero,
                                                as_stream(stream)));
    });
}

pq_status pq_moe_matvec_ternary(const pq_ternary_w* w, const pq_ternary_w* w_up,
                                const pq_groups* g, const int8_t* xq, const float* xd,
                                int32_t act_by_token, int32_t epilogue, void* out0, void* out1,
                                const pq_debug* dbg, pq_stream stream) {
    return guarded([&]() -> pq_status {
        pqk::ExpertArgs a;
        bool run;
        const pq_status st = ternary_args(w, w_up, g, xq, xd, act_by_token, epilogue, out0, out1, dbg,
                                          pqk::matvec_supported, a, &run);
        if (st != PQ_OK || !run) return st;
        return launch_matvec_any(pqk::kTernary, epilogue, a, dbg, stream);
    });
}

// The single mat-vec from fp32 activations: checks shared by the formats
// (the weights' own pointers are checked by the caller).
pq_status x32_check(int32_t n_experts, int32_t rows, int32_t cols, int32_t expert, const float* x, float* y,
                    pqk::Fmt fmt) {
    if (!x || !y) return PQ_ERR_NULL;
    if (n_experts < 1 || expert < 0 || expert >= n_experts) return PQ_ERR_SHAPE;
    if (rows < 1 || cols < 256 || cols % 256 != 0) return PQ_ERR_SHAPE;
    if (int64_t(rows) * cols > (int64_t(1) << 31)) return PQ_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(y, 4)) return PQ_ERR_ALIGN;
    if (!pqk::matvec_supported(fmt, cols)) return PQ_ERR_UNSUPPORTED;
    return PQ_OK;
}

pqk::ExpertArgs x32_args(int32_t n_experts, int32_t rows, int32_t cols, int32_t expert, float* y) {
    pqk::ExpertArgs a{};
    a.rows = rows;
    a.cols = cols;
    a.n_experts = n_experts;
    a.n_tokens = 1;
    a.top_k = 1;
    a.act_by_token = 1;
    a.expert0 = expert;
    a.out0 = y;
    return a;
}

pq_status pq_moe_matvec_grid1(const pq_grid1_w* w, const pq_grid1_w* w_up, const pq_groups* g,
                              const int8_t* xq, const float* xd, int32_t act_by_token,
                              int32_t epilogue, void* out0, void* out1, const pq_debug* dbg,
                              pq_stream stream) {
    return guarded([&]() -> pq_status {
        pqk::ExpertArgs a;
        bool run;
        const pq_status st = grid1_args(w, w_up, g, xq, xd, act_by_token, epilogue, out0, out1, dbg,
                                        pqk::matvec_supported, a, &run);
        if (st != PQ_OK || !run) return st;
        return launch_matvec_any(pqk::kGrid1, epilogue, a, dbg, stream);
    });
}

pq_status pq_moe_matvec_sign1(const pq_sign1_w* w, const pq_sign1_w* w_up, const pq_groups* g,
                              const int8_t* xq, const float* xd, int32_t act_by_token,
                              int32_t epilogue, void* out0, void* out1, const pq_debug* dbg,
                              pq_stream stream) {
    return guarded([&]() -> pq_status {
        pqk::ExpertArgs a;
        bool run;
        const pq_status st = sign1_args(w, w_up, g, xq, xd, act_by_token, epilogue, out0, out1, dbg,
                                        pqk::matvec_supported, a, &run);
        if (st != PQ_OK || !run) return st;
        return launch_matvec_any(pqk::kSign1, epilogue, a, dbg, stream);
    });
}

pq_status pq_matvec_x32_ternary(const pq_ternary_w* w, int32_t expert, const float* x, float* y,
                                pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (!w || !w->qs || !w->d) return PQ_ERR_NULL;
        const pq_status st = x32_check(w->n_experts, w->rows, w->cols, expert, x, y, pqk::kTernary);
        if (st != PQ_OK) return st;
        if (!aligned(w->qs, 16) || !aligned(w->d, 2)) return PQ_ERR_ALIGN;
        pqk::ExpertArgs a = x32_args(w->n_experts, w->rows, w->cols, expert, y);
        a.qs[0] = w->qs;
        a.d[0] = w->d;
        return from_hip(pqk::launch_matvec_x32(pqk::kTernary, a, x, as_stream(stream)));
    });
}

pq_status pq_matvec_x32_grid1(const pq_grid1_w* w, int32_t expert, const float* x, float* y,
                              pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (!w || !w->qs || !w->qh || !w->d || !w->grid) return PQ_ERR_NULL;
        const pq_status st = x32_check(w->n_experts, w->rows, w->cols, expert, x, y, pqk::kGrid1);
        if (st != PQ_OK) return st;
        if (!aligned(w->qs, 16) || !aligned(w->qh, 8) || !aligned(w->d, 2) || !aligned(w->grid, 16))
            return PQ_ERR_ALIGN;
        pqk::ExpertArgs a = x32_args(w->n_experts, w->rows, w->cols, expert, y);
        a.qs[0] = w->qs;
        a.qh[0] = w->qh;
        a.d[0] = w->d;
        a.grid = w->grid;
        return from_hip(pqk::launch_matvec_x32(pqk::kGrid1, a, x, as_stream(stream)));
    });
}

pq_status pq_matvec_x32_sign1(const pq_sign1_w* w, int32_t expert, const float* x, float* y,
                              pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (!w || !w->signs || !w->sc || !w->d) return PQ_ERR_NULL;
        const pq_status st = x32_check(w->n_experts, w->rows, w->cols, expert, x, y, pqk::kSign1);
        if (st != PQ_OK) return st;
        if (!aligned(w->signs, 16) || !aligned(w->sc, 4) || !aligned(w->d, 2)) return PQ_ERR_ALIGN;
        pqk::ExpertArgs a = x32_args(w->n_experts, w->rows, w->cols, expert, y);
        a.qs[0] = w->signs;
        a.sc[0] = w->sc;
        a.d[0] = w->d;
        return from_hip(pqk::launch_matvec_x32(pqk::kSign1, a, x, as_stream(stream)));
    });
}

pq_status pq_moe_tile_q8_ternary(const pq_ternary_w* w, const pq_ternary_w* w_up,
                                 const pq_groups* g, const int8_t* xq, const float* xd,
                                 int32_t act_by_token, int32_t epilogue, void* out0, void* out1,
                                 const pq_debug* dbg, pq_stream stream) {
    return guarded([&]() -> pq_status {
        pqk::ExpertArgs a;
        bool run;
        const pq_status st = ternary_args(w, w_up, g, xq, xd, act_by_token, epilogue, out0, out1, dbg,
                                          [](pqk::Fmt, int cols) { return pqk::tile_q8_supported(cols); },
                                          a, &run);
        if (st != PQ_OK || !run) return st;
        return launch_tile_all(pqk::kTernary, epilogue, a, stream);
    });
}

pq_status pq_moe_tile_q8_grid1(const pq_grid1_w* w, const pq_grid1_w* w_up, const pq_groups* g,
                               const int8_t* xq, const float* xd, int32_t act_by_token,
                               int32_t epilogue, void* out0, void* out1, const pq_debug* dbg,
                               pq_stream stream) {
    return guarded([&]() -> pq_status {
        pqk::ExpertArgs a;
        bool run;
        const pq_status st = grid1_args(w, w_up, g, xq, xd, act_by_token, epilogue, out0, out1, dbg,
                                        [](pqk::Fmt, int cols) { return pqk::tile_q8_supported(cols); },
                                        a, &run);
        if (st != PQ_OK || !run) return st;
        return launch_tile_all(pqk::kGrid1, epilogue, a, stream);
    });
}

pq_status pq_moe_tile_q8_sign1(const pq_sign1_w* w, const pq_sign1_w* w_up, const pq_groups* g,
                               const int8_t* xq, const float* xd, int32_t act_by_token,
                               int32_t epilogue, void* out0, void* out1, const pq_debug* dbg,
                               pq_stream stream) {
    return guarded([&]() -> pq_status {
        pqk::ExpertArgs a;
        bool run;
        const pq_status st = sign1_args(w, w_up, g, xq, xd, act_by_token, epilogue, out0, out1, dbg,
                                        [](pqk::Fmt, int cols) { return pqk::tile_q8_supported(cols); },
                                        a, &run);
        if (st != PQ_OK || !run) return st;
        return launch_tile_all(pqk::kSign1, epilogue, a, stream);
    });
}

pq_status pq_moe_gemm_dequant_tile(const pq_grid1_w* w, const pq_grid1_w* w_up,
                                   const pq_groups* g, const uint16_t* x, int32_t act_by_token,
                                   int32_t epilogue, void* out0, void* out1, const pq_debug* dbg,
                                   pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (!w || !w->qs || !w->qh || !w->d || !w->grid) return PQ_ERR_NULL;
        pq_status st = check_groups(g);
        if (st != PQ_OK) return st;
        if ((st = check_dims(w->n_experts, w->rows, w->cols, g)) != PQ_OK) return st;
        if ((st = check_epilogue_outputs(epilogue, w_up, w->rows, out0, out1, false)) != PQ_OK)
            return st;
        if (epilogue == PQ_EPI_SWIGLU_BF16) {
            if (!w_up->qs || !w_up->qh || !w_up->d) return PQ_ERR_NULL;
            if (w_up->n_experts != w->n_experts || w_up->rows != w->rows || w_up->cols != w->cols)
                return PQ_ERR_SHAPE;
            if (!aligned(w_up->qs, 16) || !aligned(w_up->qh, 8) || !aligned(w_up->d, 2))
                return PQ_ERR_ALIGN;
        }
        if (!aligned(w->qs, 16) || !aligned(w->qh, 8) || !aligned(w->d, 2) ||
            !aligned(w->grid, 16))
            return PQ_ERR_ALIGN;
        if (w->rows % pqk::kTileRows != 0) return PQ_ERR_SHAPE;
        if (!pqk::gemm_supported(pqk::kGrid1, w->rows, w->cols, epilogue)) return PQ_ERR_UNSUPPORTED;
        if (g->n_tokens == 0) return PQ_OK;
        if (!x) return PQ_ERR_NULL;
        if (!aligned(x, 16)) return PQ_ERR_ALIGN;
        pqk::ExpertArgs a{};
        a.qs[0] = w->qs;
        a.qh[0] = w->qh;
        a.d[0] = w->d;
        a.qs[1] = w_up ? w_up->qs : nullptr;
        a.qh[1] = w_up ? w_up->qh : nullptr;
        a.d[1] = w_up ? w_up->d : nullptr;
        a.grid = w->grid;
        a.rows = w->rows;
        a.cols = w->cols;
        fill_groups(a, g);
        a.act_by_token = act_by_token ? 1 : 0;
        a.xb = x;
        a.out0 = out0;
        a.out1 = out1;
        fill_debug(a, dbg);
        return from_hip(pqk::launch_gemm(pqk::kGrid1, static_cast<pqk::Epi>(epilogue), a, as_stream(stream)));
    });
}

pq_status pq_moe_gemm_dequant_tile_sign1(const pq_sign1_w* w, const pq_sign1_w* w_up,
                                         const pq_groups* g, const uint16_t* x, int32_t act_by_token,
                                         int32_t epilogue, void* out0, void* out1, const pq_debug* dbg,
                                         pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (!w || !w->signs || !w->sc || !w->d) return PQ_ERR_NULL;
        pq_status st = check_groups(g);
        if (st != PQ_OK) return st;
        if ((st = check_dims(w->n_experts, w->rows, w->cols, g)) != PQ_OK) return st;
        if ((st = check_epilogue_outputs(epilogue, w_up, w->rows, out0, out1, false)) != PQ_OK)
            return st;
        if (epilogue == PQ_EPI_SWIGLU_BF16) {
            if (!w_up->signs || !w_up->sc || !w_up->d) return PQ_ERR_NULL;
            if (w_up->n_experts != w->n_experts || w_up->rows != w->rows || w_up->cols != w->cols)
                return PQ_ERR_SHAPE;
            if (!aligned(w_up->signs, 16) || !aligned(w_up->sc, 16) || !aligned(w_up->d, 2))
                return PQ_ERR_ALIGN;
        }
        if (!aligned(w->signs, 16) || !aligned(w->sc, 16) || !aligned(w->d, 2)) return PQ_ERR_ALIGN;
        if (w->rows % pqk::kTileRows != 0) return PQ_ERR_SHAPE;
        if (!pqk::gemm_supported(pqk::kSign1, w->rows, w->cols, epilogue)) return PQ_ERR_UNSUPPORTED;
        if (g->n_tokens == 0) return PQ_OK;
        if (!x) return PQ_ERR_NULL;
        if (!aligned(x, 16)) return PQ_ERR_ALIGN;
        pqk::ExpertArgs a{};
        a.qs[0] = w->signs;
        a.sc[0] = w->sc;
        a.d[0] = w->d;
        a.qs[1] = w_up ? w_up->signs : nullptr;
        a.sc[1] = w_up ? w_up->sc : nullptr;
        a.d[1] = w_up ? w_up->d : nullptr;
        a.rows = w->rows;
        a.cols = w->cols;
        fill_groups(a, g);
        a.act_by_token = act_by_token ? 1 : 0;
        a.xb = x;
        a.out0 = out0;
        a.out1 = out1;
        fill_debug(a, dbg);
        return from_hip(pqk::launch_gemm(pqk::kSign1, static_cast<pqk::Epi>(epilogue), a, as_stream(stream)));
    });
}

namespace {

// [a, a + na) and [b, b + nb) share a byte
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

// no destination plane shares a byte with any plane of the call
bool planes_overlap(const void* s0, int64_t n0, const void* s1, int64_t n1, const void* d0, const void* d1) {
    return overlap(d0, n0, s0, n0) || overlap(d0, n0, s1, n1) || overlap(d1, n1, s0, n0) ||
           overlap(d1, n1, s1, n1) || overlap(d0, n0, d1, n1);
}

pq_status check_tile_dims(int32_t n_experts, int32_t rows, int32_t cols, int32_t col_mult) {
    if (n_experts < 1 || n_experts > kMaxExperts) return PQ_ERR_SHAPE;
    if (rows < 1 || rows % pqk::kTileRows != 0) return PQ_ERR_SHAPE;
    if (cols < col_mult || cols % col_mult != 0) return PQ_ERR_SHAPE;
    if (int64_t(rows) * cols > (int64_t(1) << 31)) return PQ_ERR_SHAPE;
    return PQ_OK;
}

}  // namespace

pq_status pq_tile_layout_grid1(const pq_grid1_w* w, uint8_t* qs_tiled, uint16_t* qh_tiled,
                               pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (!w || !w->qs || !w->qh || !qs_tiled || !qh_tiled) return PQ_ERR_NULL;
        pq_status st = check_tile_dims(w->n_experts, w->rows, w->cols, 256);
        if (st != PQ_OK) return st;
        if (!aligned(w->qs, 16) || !aligned(w->qh, 16) || !aligned(qs_tiled, 16) || !aligned(qh_tiled, 16))
            return PQ_ERR_ALIGN;
        const int64_t rows = int64_t(w->n_experts) * w->rows;
        const int64_t qs_bytes = rows * (w->cols / 8), qh_bytes = rows * (w->cols / 32) * 2;
        if (planes_overlap(w->qs, qs_bytes, w->qh, qh_bytes, qs_tiled, qh_tiled)) return PQ_ERR_SHAPE;
        const int nb = w->cols / 256;
        hipError_t e = pqk::launch_tile_layout(w->qs, qs_tiled, rows, nb, 32, as_stream(stream));
        if (e == hipSuccess) e = pqk::launch_tile_layout(w->qh, qh_tiled, rows, nb, 16, as_stream(stream));
        return from_hip(e);
    });
}

pq_status pq_tile_layout_sign1(const pq_sign1_w* w, uint8_t* signs_tiled, uint8_t* sc_tiled,
                               pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (!w || !w->signs || !w->sc || !signs_tiled || !sc_tiled) return PQ_ERR_NULL;
        pq_status st = check_tile_dims(w->n_experts, w->rows, w->cols, 512);
        if (st != PQ_OK) return st;
        if (!aligned(w->signs, 16) || !aligned(w->sc, 16) || !aligned(signs_tiled, 16) || !aligned(sc_tiled, 16))
            return PQ_ERR_ALIGN;
        const int64_t rows = int64_t(w->n_experts) * w->rows;
        const int64_t s_bytes = rows * (w->cols / 8), c_bytes = rows * (w->cols / 32);
        if (planes_overlap(w->signs, s_bytes, w->sc, c_bytes, signs_tiled, sc_tiled)) return PQ_ERR_SHAPE;
        hipError_t e = pqk::launch_tile_layout(w->signs, signs_tiled, rows, w->cols / 256, 32, as_stream(stream));
        if (e == hipSuccess) e = pqk::launch_tile_layout(w->sc, sc_tiled, rows, w->cols / 512, 16, as_stream(stream));
        return from_hip(e);
    });
}

pq_status pq_moe_combine(const float* out_assign, const float* topk_w, int32_t n_tokens,
                         int32_t top_k, int32_t rows, float* y, pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (n_tokens < 0 || top_k < 1 || top_k > kMaxTopK || rows < 1) return PQ_ERR_SHAPE;
        if (int64_t(n_tokens) * top_k * rows > (int64_t(1) << 40)) return PQ_ERR_SHAPE;
        if (n_tokens == 0) return PQ_OK;
        if (!out_assign || !topk_w || !y) return PQ_ERR_NULL;
        if (!aligned(out_assign, 4) || !aligned(topk_w, 4) || !aligned(y, 4)) return PQ_ERR_ALIGN;
        return from_hip(
            pqk::launch_combine(out_assign, topk_w, n_tokens, top_k, rows, y, as_stream(stream)));
    });
}

pq_status pq_moe_decode1_gate_up_ternary(const float* x, const float* logits, int32_t n_experts,
                                         int32_t top_k, const pq_ternary_w* gate,
                                         const pq_ternary_w* up, int32_t* topk_ids, float* topk_w,
                                         int32_t* expert_offsets, int32_t* sorted_assign,
                                         int32_t* active_experts, int32_t* n_active, int8_t* hq,
                                         float* hd, float* y_zero, pq_stream stream) {
    return guarded([&]() -> pq_status {
        return decode1_gate_up(pqk::kTernary, x, logits, n_experts, top_k, gate, up, topk_ids, topk_w,
                               expert_offsets, sorted_assign, active_experts, n_active, hq, hd,
                               y_zero, stream);
    });
}

pq_status pq_moe_decode1_gate_up_grid1(const float* x, const float* logits, int32_t n_experts,
                                       int32_t top_k, const pq_grid1_w* gate, const pq_grid1_w* up,
                                       int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                       int32_t* sorted_assign, int32_t* active_experts,
                                       int32_t* n_active, int8_t* hq, float* hd, float* y_zero,
                                       pq_stream stream) {
    return guarded([&]() -> pq_status {
        return decode1_gate_up(pqk::kGrid1, x, logits, n_experts, top_k, gate, up, topk_ids, topk_w,
                               expert_offsets, sorted_assign, active_experts, n_active, hq, hd,
                               y_zero, stream);
    });
}

pq_status pq_moe_decode1_gate_up_sign1(const float* x, const float* logits, int32_t n_experts,
                                       int32_t top_k, const pq_sign1_w* gate, const pq_sign1_w* up,
                                       int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                       int32_t* sorted_assign, int32_t* active_experts,
                                       int32_t* n_active, int8_t* hq, float* hd, float* y_zero,
                                       pq_stream stream) {
    return guarded([&]() -> pq_status {
        return decode1_gate_up(pqk::kSign1, x, logits, n_experts, top_k, gate, up, topk_ids, topk_w,
                               expert_offsets, sorted_assign, active_experts, n_active, hq, hd,
                               y_zero, stream);
    });
}

int32_t pq_plan(int32_t call, int32_t fmt, int32_t n_tokens, int32_t top_k, int32_t n_experts,
                int32_t rows, int32_t cols, int32_t epilogue, int32_t debug) {
    try {
        if (fmt < PQ_FMT_TERNARY || fmt > PQ_FMT_SIGN1) return -PQ_ERR_UNSUPPORTED;
        const pqk::Fmt f = static_cast<pqk::Fmt>(fmt);
        if (n_tokens < 0 || n_experts < 1 || n_experts > kMaxExperts) return -PQ_ERR_SHAPE;
        if (top_k < 1 || top_k > kMaxTopK || top_k > n_experts) return -PQ_ERR_SHAPE;
        if (int64_t(n_tokens) * top_k > kMaxAssign) return -PQ_ERR_SHAPE;
        if (rows < 1 || cols < 256 || cols % 256 != 0) return -PQ_ERR_SHAPE;
        const int dbg = debug ? PQ_PLAN_DEBUG : 0;
        switch (call) {
            case PQ_CALL_MATVEC: {
                if (!pqk::matvec_supported(f, cols)) return -PQ_ERR_UNSUPPORTED;
                int p = pqk::plan_matvec(n_tokens, top_k, n_experts, cols, debug != 0);
                if ((p & PQ_PLAN_TILE_Q8) && (p & PQ_PLAN_MATVEC_PAIRS) &&
                    pqk::mixed_planned(f, static_cast<pqk::Epi>(epilogue), n_tokens, top_k, cols))
                    p |= PQ_PLAN_MIXED;
                return p;
            }
            case PQ_CALL_TILE_Q8:
                if (!pqk::tile_q8_supported(cols)) return -PQ_ERR_UNSUPPORTED;
                return n_tokens ? (PQ_PLAN_TILE_Q8 | dbg) : 0;
            case PQ_CALL_GEMM:
                if (!pqk::gemm_supported(f, rows, cols, epilogue)) return -PQ_ERR_UNSUPPORTED;
                return n_tokens ? (PQ_PLAN_GEMM | dbg) : 0;
            case PQ_CALL_DECODE1_GATE_UP:
                if (debug) return -PQ_ERR_UNSUPPORTED;
                if (!pqk::matvec_supported(f, cols) || rows % 32 != 0) return -PQ_ERR_UNSUPPORTED;
                return PQ_PLAN_DECODE1_ROUTED;
            default:
                return -PQ_ERR_UNSUPPORTED;
        }
    } catch (...) {
        return -PQ_ERR_HIP;
    }
}

pq_status pq_peak_read(const void* buf, int64_t bytes, uint32_t* sink, pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (bytes < 16 || bytes % 16 != 0) return PQ_ERR_SHAPE;
        if (!buf || !sink) return PQ_ERR_NULL;
        if (!aligned(buf, 16) || !aligned(sink, 4)) return PQ_ERR_ALIGN;
        return from_hip(pqk::launch_peak_read(buf, bytes, sink, as_stream(stream)));
    });
}

pq_status pq_peak_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, int32_t* waves_per_workgroup,
                            int32_t* chains, pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (workgroups < 1 || iters < 1) return PQ_ERR_SHAPE;
        if (!sink) return PQ_ERR_NULL;
        if (!aligned(sink, 4)) return PQ_ERR_ALIGN;
        if (waves_per_workgroup) *waves_per_workgroup = pqk::peak_mfma_waves_per_workgroup();
        if (chains) *chains = pqk::peak_mfma_chains();
        return from_hip(pqk::launch_peak_mfma(workgroups, iters, sink, as_stream(stream)));
    });
}

pq_status pq_validate_ternary(const pq_ternary_w* w, int32_t* n_bad, pq_stream stream) {
    return guarded([&]() -> pq_status {
        if (!w || !w->qs || !n_bad) return PQ_ERR_NULL;
        if (w->n_experts < 1 || w->rows < 1 || w->cols < 256 || w->cols % 256 != 0)
            return PQ_ERR_SHAPE;
        if (!aligned(w->qs, 16) || !aligned(n_bad, 4)) return PQ_ERR_ALIGN;
        const int64_t n_bytes = int64_t(w->n_experts) * w->rows * (w->cols / 4);
        return from_hip(pqk::launch_validate_ternary(w->qs, n_bytes, n_bad, as_stream(stream)));
    });
}

}  // extern "C"
