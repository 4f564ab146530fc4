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

__device__ __forceinline__ float wave_sum32(float v) {
    // sum over the 32-lane half of the wave that holds this lane
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float wave_max32(float v) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// q8 of one value given the fp32 block max |x|: round half away from zero of
// x / (amax / 127), clamped to [-127, 127]; amax == 0 gives 0.
__device__ __forceinline__ int q8_value(float x, float d) {
    if (d == 0.0f) return 0;
    float r = roundf(x / d);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int>(r);
}

}  // namespace pqk
