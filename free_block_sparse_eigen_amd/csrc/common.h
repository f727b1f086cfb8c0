// Shared device helpers for the SparsePR HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <cmath>
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

typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even (finite inputs): the hardware
// conversion on the device, the same rounding written out on the host.
__host__ __device__ inline bf16_t f32_to_bf16(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
#else
    union { uint32_t u; float f; } v;
    v.f = f;
    uint32_t u = v.u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
#endif
}

// Two fp32 -> packed bf16 pair (low half = a), round to nearest even (one instruction).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 2^x with the hardware instruction (results below 2^-126 flush to zero).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// LDS row swizzle for tiles of 16-byte chunks: chunk c of row r is stored at c ^ swz(r).
// With 16 chunks per row, swz rotates r's low 4 bits by two ((r & 3) << 2 | (r >> 2) & 3):
// 16-byte reads of one logical chunk by 32 consecutive rows, and the transposed 8-byte
// reads of 4 consecutive rows x 4 adjacent chunks, then run without bank conflicts on
// gfx950 (checked with the LDS bank-conflict counter). With 8 chunks per row it is a
// bit permutation of r's low 3 bits (bits 0,1 -> 1,2; bit 2 -> 0).
template <int CH>
__host__ __device__ inline int swz(int r) {
    if (CH >= 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    return ((r & 3) << 1) | ((r >> 2) & 1);
}

// Buffer resource over `bytes` bytes from base (loads past the end return zero); word 3
// (0x00020000) selects the 32-bit data format that untyped buffer loads need on gfx950.
// Global-to-LDS loads go through buffer resources rather than global addresses because
// the compiler then tracks them on the vector-memory counter alone: the global-address
// form also marks the LDS counter as out of order, which turns every wait on an LDS read
// into a wait for all of them.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// 16 bytes per lane from byte offset off (per lane) of r into LDS at s + 16 * lane
// (s is the same for the whole wave)
__device__ inline void lds_load16(rsrc_t r, void* s, int off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)s, 16, off,
                                             0, 0, 0);
}

// ---- FP8 E4M3 operands (the fp8-logit experiment) ----
typedef int i32x8 __attribute__((ext_vector_type(8)));

// D = A(32x64) * B(64x32) + C with FP8 E4M3 inputs and fp32 accumulation: lane l supplies
// row l%32 of A and column l%32 of B, 32 bytes each, for the depth half l/32. A and B
// take their depth bytes in the same order, so the sum over the depth does not depend on
// which order the instruction pairs them in.
__device__ inline f32x16 mfma32x32x64_f8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// four fp32 -> four E4M3 bytes (round to nearest even), a in the low byte; the callers'
// values are at most 448 in magnitude
__device__ inline uint32_t pack_e4m3x4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// ---- fp16 operands of the P.V products ----
// V is stored group-major in fp16, scaled per head by an exact power of two 2^e chosen from
// the head's largest |v| (so the scaled values sit below 2^15 and bf16 values convert
// without rounding); P is rounded to fp16 (11 significant bits against bf16's 8).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ inline f32x16 mfma32x32x16_f16(uint4 a, uint4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 -> packed fp16 pair (low half = a), round to nearest even (one instruction).
__device__ inline uint32_t pack_f16x2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ inline float f16_to_f32(uint32_t h16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h16)));
}

__device__ inline f16x2 ones_f16x2() { return __builtin_bit_cast(f16x2, 0x3C003C00u); }

// acc + lo(packed) + hi(packed), the fp16 pair summed in fp32
__device__ inline float dot2_f16(uint32_t packed, f16x2 ones, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), ones, acc, false);
}

// Exponent e of the per-head V scale from the head's largest bf16 magnitude bits: the
// largest scaled value lies in [2^14, 2^15). Zero, non-finite or absurdly small heads keep
// e within [-64, 64] (0 for a zero or non-finite head).
__host__ __device__ inline int v_scale_exp(uint32_t max_bf16_bits) {
    const int ef = (int)((max_bf16_bits >> 7) & 0xFF);
    if (max_bf16_bits == 0 || ef == 0xFF) return 0;
    int lg;                                            // floor(log2(max))
    if (ef == 0) {                                     // bf16 subnormal: 7 fraction bits
        int top = 6;
        while (top > 0 && !((max_bf16_bits >> top) & 1u)) --top;
        lg = -133 + top;
    } else {
        lg = ef - 127;
    }
    const int e = 14 - lg;
    return e < -64 ? -64 : (e > 64 ? 64 : e);
}

// Exponent e of a per-head FP8 E4M3 scale from the head's largest bf16 magnitude bits: the
// largest e with max 2^e <= 448 (the largest E4M3 magnitude), kept within [-120, 120]; 0
// for a zero or non-finite head. Scaling by 2^e is exact, so only the rounding to E4M3
// changes the values.
__host__ __device__ inline int f8_scale_exp(uint32_t max_bf16_bits) {
    const int ef = (int)((max_bf16_bits >> 7) & 0xFF);
    if (max_bf16_bits == 0 || ef == 0xFF) return 0;
    const float a = __builtin_bit_cast(float, max_bf16_bits << 16);
    int ex;
    const float f = frexpf(a, &ex);                    // a = f 2^ex, f in [0.5, 1)
    const int e = (2.f * f <= 1.75f) ? 9 - ex : 8 - ex;   // 448 = 1.75 2^8
    return e < -120 ? -120 : (e > 120 ? 120 : e);
}

// P offset for fp16: the lazily raised running max lets P reach 2^8, so exp2(x + 7) stays
// below 2^15 (fp16 max 65504) and keeps small weights 2^7 further from fp16 subnormals.
constexpr float kP16Offset = 7.0f;

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
