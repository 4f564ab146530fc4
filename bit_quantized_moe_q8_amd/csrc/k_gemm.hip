// Prefill dequant-per-tile GEMM (grid1 weights, bf16 activations, MFMA).
#include "pq_device.hpp"
#include "pq_internal.hpp"

namespace pqk {

bool gemm_supported(int, int, int) { return false; }

hipError_t launch_gemm(Epi, const ExpertArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace pqk
