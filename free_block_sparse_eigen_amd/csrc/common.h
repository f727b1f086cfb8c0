// Shared device helpers for the SparsePR HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace spr {

typedef uint16_t bf16_t;                                   // bf16 storage
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef bf16x2 bf16x2_ones_t;

constexpr int kWave = 64;

__host__ __device__ inline float bf16_to_f32(bf16_t b) {
    union { uint32_t u; float f; } v;
    v.u = static_cast<uint32_t>(b) << 16;
    return v.f;
}

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__host__ __device__ inline bf16_t f32_to_bf16(float f) {
    union { uint32_t u; float f; } v;
    v.f = f;
    uint32_t u = v.u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

// Two fp32 -> packed bf16 pair (low half = a), round to nearest even.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate.
// Lane l supplies A[row l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][col l%32];
// the result element (row, col) sits in lane col + 32*((row/4)%2), register
// (row%4) + 4*(row/8).
__device__ inline f32x16 mfma32x32x16(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ inline bf16x2 ones_bf16x2() { return __builtin_bit_cast(bf16x2, 0x3F803F80u); }

// acc + lo(packed) + hi(packed), the bf16 pair summed in fp32
__device__ inline float dot2_bf16(uint32_t packed, bf16x2 ones, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), ones, acc, false);
}

template <typename T>
__device__ inline T wave_max(T v) {
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}

template <typename T>
__device__ inline T wave_sum(T v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace spr
