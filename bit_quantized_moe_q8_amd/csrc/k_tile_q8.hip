// Launches of the grouped int8-MFMA tile kernel (k_tile_q8.hpp).
#include "k_tile_q8.hpp"

namespace pqk {

namespace {

template <int FMT, int EPI, bool DBG, int TOK>
__global__ __launch_bounds__(tq8::kThreads) __attribute__((amdgpu_waves_per_eu((TOK == 32 && !DBG) ? 3 : 1)))
void k_tile_q8(ExpertArgs p) {
    tq8::tile_q8_body<FMT, EPI, DBG, TOK>(p, blockIdx.x, gridDim.x);
}

template <int FMT, int EPI, bool DBG, int TOK>
hipError_t launch_one(const ExpertArgs& a, hipStream_t s) {
    const int64_t grid = tq8::tile_grid<EPI, TOK>(a);
    hipLaunchKernelGGL((k_tile_q8<FMT, EPI, DBG, TOK>), dim3(static_cast<unsigned>(grid)), dim3(tq8::kThreads), 0, s, a);
    return hipGetLastError();
}

template <int FMT, int EPI>
hipError_t launch_dbg(const ExpertArgs& a, hipStream_t s) {
    const int64_t A = static_cast<int64_t>(a.n_tokens) * a.top_k;
    if (A <= tq8::kSmallChunkMaxAssign)
        return a.debug ? launch_one<FMT, EPI, true, 32>(a, s) : launch_one<FMT, EPI, false, 32>(a, s);
    return a.debug ? launch_one<FMT, EPI, true, 64>(a, s) : launch_one<FMT, EPI, false, 64>(a, s);
}

template <int FMT>
hipError_t launch_fmt(Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (epi == kEpiF32) return launch_dbg<FMT, kEpiF32>(a, s);
    if (epi == kEpiF32Combine) return launch_dbg<FMT, kEpiF32Combine>(a, s);
    if (epi == kEpiSwigluQ8) return launch_dbg<FMT, kEpiSwigluQ8>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

bool tile_q8_supported(int cols) { return cols >= tq8::kSlabK && cols % tq8::kSlabK == 0; }

hipError_t launch_tile_q8(Fmt fmt, Epi epi, const ExpertArgs& a, hipStream_t s) {
    if (!tile_q8_supported(a.cols)) return hipErrorInvalidValue;
    if (fmt == kTernary) return launch_fmt<kTernary>(epi, a, s);
    if (fmt == kSign1) return launch_fmt<kSign1>(epi, a, s);
    return launch_fmt<kGrid1>(epi, a, s);
}

}  // namespace pqk
