// Device helpers shared by the libpq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pqk {

constexpr int kWave = 64;

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Round a finite float to bf16, nearest with ties to even.
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Load through the scalar data cache (s_load).  Only for addresses that are
// uniform over the wave and data that nothing writes while the kernel runs
// (routing arrays, counts).
template <typename T>
__device__ __forceinline__ T load_uniform(const T* ptr) {
    return *(const __attribute__((address_space(4))) T*)(ptr);
}

// v_dot4_i32_i8: acc + sum of the four signed byte products of a and b.
__device__ __forceinline__ int dot4(int a, int b, int acc) {
    return __builtin_amdgcn_sdot4(a, b, acc, false);
}

// v_perm_b32: byte i of the result is byte sel.byte(i) of the 8-byte value
// {hi, lo} (selectors 0..3 pick lo, 4..7 pick hi).
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Ternary decode of four 2-bit codes held in the low bits of each byte of
// `sel` (values 0, 1, 2) into four int8 weights 0, +1, -1: a byte lookup in
// the constant 0x00FF0100 (bytes 00 01 FF 00).
__device__ __forceinline__ int ternary_decode4(uint32_t sel) {
    return static_cast<int>(byte_perm(0u, 0x00FF0100u, sel));
}

// The same for codes held in bits 2..3 of each byte of `sel` (values 0, 4,
// 8): selector 0 picks byte 0 of the low word (0x00), 4 byte 0 of the high
// word (0x01), and 8 replicates bit 7 of byte 1 of the low word (0x80 ->
// 0xFF), so the field needs no shift.
__device__ __forceinline__ int ternary_decode4_hi(uint32_t sel) {
    return static_cast<int>(byte_perm(0x00000001u, 0x00008000u, sel));
}

// Four ternary int8 weight words from one dword P of 16 two-bit codes: word
// s holds the codes of fields s of the four bytes (weights 4b+s), as the
// byte-transposed activations expect.
__device__ __forceinline__ void ternary_decode16(uint32_t P, int w[4]) {
    const uint32_t P4 = P >> 4;
    w[0] = ternary_decode4(P & 0x03030303u);
    w[1] = ternary_decode4_hi(P & 0x0C0C0C0Cu);
    w[2] = ternary_decode4(P4 & 0x03030303u);
    w[3] = ternary_decode4_hi(P4 & 0x0C0C0C0Cu);
}

// Activation bytes permuted for ternary decoding: given four dwords q[0..3]
// holding 16 consecutive int8 activations, returns t[s] whose byte b is
// activation 4b+s, i.e. a 4x4 byte transpose.
__device__ __forceinline__ void transpose_bytes4(const uint32_t q[4], uint32_t t[4]) {
    uint32_t t0 = byte_perm(q[1], q[0], 0x05010400u);
    uint32_t t1 = byte_perm(q[1], q[0], 0x07030602u);
    uint32_t u0 = byte_perm(q[3], q[2], 0x05010400u);
    uint32_t u1 = byte_perm(q[3], q[2], 0x07030602u);
    t[0] = byte_perm(u0, t0, 0x05040100u);
    t[1] = byte_perm(u0, t0, 0x07060302u);
    t[2] = byte_perm(u1, t1, 0x05040100u);
    t[3] = byte_perm(u1, t1, 0x07060302u);
}

// DPP lane exchange: lanes of the 16-lane rows enabled in ROW_MASK read `v`
// from the lane selected by CTRL; lanes of other rows get 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each 16
constexpr int kDppBcast15 = 0x142;    // lane 15 of a row -> next row
constexpr int kDppBcast31 = 0x143;    // lane 31 -> rows 2 and 3

// a * b rounded on its own, never fused into a following add: the lanes of a
// row sum then add rounded products, so the sum has the same bits in every
// kernel and instantiation that forms it (a fused multiply-add of one lane's
// product with its partner's rounded one differs in the last bit, and the
// compiler fuses or not depending on the surrounding code).
__device__ __forceinline__ float mul_rounded(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}

// Sum over aligned segments of LS lanes (LS a power of two, <= 64) with DPP
// moves only.  The full segment sum ends up in the last lane of each segment
// (for LS <= 16 in every lane of it).
template <int LS>
__device__ __forceinline__ float seg_sum(float v) {
    if constexpr (LS >= 2) v += dpp_f32<kDppQuadXor1>(v);
    if constexpr (LS >= 4) v += dpp_f32<kDppQuadXor2>(v);
    if constexpr (LS >= 8) v += dpp_f32<kDppHalfMirror>(v);
    if constexpr (LS >= 16) v += dpp_f32<kDppMirror>(v);
    if constexpr (LS >= 32) v += dpp_f32<kDppBcast15, 0xA>(v);
    if constexpr (LS >= 64) v += dpp_f32<kDppBcast31, 0xC>(v);
    return v;
}

// Maximum over each 32-lane half of the wave, returned in every lane of it.
__device__ __forceinline__ float half_wave_max(float v) {
    v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    // rows 1 and 3 now combine with rows 0 and 2 (values are >= 0 here, so
    // the 0 returned to disabled rows is neutral)
    v = fmaxf(v, dpp_f32<kDppBcast15, 0xA>(v));
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    return (__lane_id() < 32) ? lo : hi;
}

// q8 of one value given the fp32 block max |x|: round half away from zero of
// x / (amax / 127), clamped to [-127, 127]; amax == 0 gives 0.
__device__ __forceinline__ int q8_value(float x, float d) {
    if (d == 0.0f) return 0;
    float r = roundf(x / d);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int>(r);
}

// q8 of a 32-value block held by 8 consecutive lanes, 4 values each (lanes
// 8g..8g+7 form a group; every lane of the group must call): the block
// scale d = max|x| / 127 and this lane's four codes round_half_away(x / d),
// packed little-endian.
__device__ __forceinline__ uint32_t q8_pack4(float4 v, float& d) {
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    d = a / 127.0f;
    return (static_cast<uint32_t>(q8_value(v.x, d)) & 0xffu) |
           ((static_cast<uint32_t>(q8_value(v.y, d)) & 0xffu) << 8) |
           ((static_cast<uint32_t>(q8_value(v.z, d)) & 0xffu) << 16) |
           ((static_cast<uint32_t>(q8_value(v.w, d)) & 0xffu) << 24);
}

// Routing key of logit v of expert e: the order-preserving bits of v, then
// the complement of e, so that a larger key is a larger logit or an equal
// logit with a lower expert id.  -0.0 must be folded to +0.0 by the caller.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}

// Softmax over the k selected logits (s_val in rank order), by the lanes of
// one wave (lane < k holds selection `lane`); writes ids and weights.
__device__ __forceinline__ void route_softmax_store(const float* s_val, const int* s_idx, int k,
                                                    int lane, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
    const bool on = lane < k;
    const float v = on ? s_val[lane] : 0.0f;
    const float ex = on ? expf(v - s_val[0]) : 0.0f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    if (on) {
        ids[lane] = s_idx[lane];
        w[lane] = ex / sum;
    }
}

// Exclusive scan of one int per thread over the workgroup; `tmp` holds one
// int per wave.  Every thread of the workgroup must call.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp) {
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

}  // namespace pqk
