// Measurement aids: the achievable HBM read rate and bf16 MFMA rate of the
// device the library runs on, as second denominators for the roofline
// fractions of the expert kernels (which are quoted against the nominal
// 8 TB/s and 2.5 PFLOP/s as well).  Not on the hot path.
#include "pq_device.hpp"
#include "pq_internal.hpp"

namespace pqk {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;   // 16-byte loads in flight per lane

// Streams n16 16-byte words with coalesced wave-wide loads, kReadUnroll per
// lane in flight, grid-stride over the buffer; the XOR of everything read
// decides a store that never happens for real data (so no load is dropped).
__global__ __launch_bounds__(kReadThreads) void k_peak_read(const uint4* __restrict__ p, int64_t n16,
                                                            uint32_t* __restrict__ sink) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kReadThreads * kReadUnroll;
    uint32_t acc = 0;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kReadThreads * kReadUnroll + threadIdx.x;
         base < n16; base += stride) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t i = base + static_cast<int64_t>(u) * kReadThreads;
            v[u] = i < n16 ? p[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x & 1023] = acc;
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kMfmaThreads = 256;
constexpr int kChains = 8;   // independent accumulators per wave

// iters x kChains back-to-back v_mfma_f32_16x16x32_bf16 per wave on register
// operands (16 * 16 * 32 * 2 flops each); the operands come from the lane id
// so the compiler cannot fold them, and the sum decides a store that does not
// happen (so no product is dropped).
__global__ void k_peak_mfma(int iters, float* __restrict__ sink) {
    const uint32_t l = threadIdx.x;
    const uint32_t ha = 0x3F80u | (l & 7u), hb = 0x3F80u | ((l >> 3) & 7u);   // bf16 1.0 .. 1.05
    const uint32_t wa = ha | (ha << 16), wb = hb | (hb << 16);
    bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(wa, wa, wa, wa));
    bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(wb, wb, wb, wb));
    f32x4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][3];
    if (s == -1.0f) sink[blockIdx.x & 1023] = s;
}

}  // namespace

hipError_t launch_peak_read(const void* p, int64_t bytes, uint32_t* sink, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    const int64_t per_wg = static_cast<int64_t>(kReadThreads) * kReadUnroll;
    int64_t grid = static_cast<int64_t>(cu_count()) * 8;
    if (grid > (n16 + per_wg - 1) / per_wg) grid = (n16 + per_wg - 1) / per_wg;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_peak_read, dim3(static_cast<unsigned>(grid)), dim3(kReadThreads), 0, s,
                       static_cast<const uint4*>(p), n16, sink);
    return hipGetLastError();
}

hipError_t launch_peak_mfma(int workgroups, int iters, float* sink, hipStream_t s) {
    hipLaunchKernelGGL(k_peak_mfma, dim3(static_cast<unsigned>(workgroups)), dim3(kMfmaThreads), 0, s, iters,
                       sink);
    return hipGetLastError();
}

int peak_mfma_waves_per_workgroup() { return kMfmaThreads / kWave; }
int peak_mfma_chains() { return kChains; }

}  // namespace pqk
