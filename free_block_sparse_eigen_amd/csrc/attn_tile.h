// Shared pieces of the attention and probe kernels: 64-key K/V tiles in LDS filled by
// direct buffer loads, the S^T = K Q^T and O^T += V^T P^T fragments of the 32x32x16 bf16
// matrix instruction, and the cross-half reductions of a query column.
#pragma once
#include "kernels.h"

#include <cmath>

namespace spr {

// internal linkage, as for functions local to each kernel file
namespace {

constexpr int KT = kKeyTile;
constexpr float kLazy = 8.0f;  // raise the running max only when a tile exceeds it by 2^8

__device__ inline uint4 ldg16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Key tiles live in LDS row-major for both K and V: row r (a key), 16-byte chunk c
// (dims 8c..8c+7) at slot r * CH + (c ^ swz(r)). They are filled by direct
// global-to-LDS loads (no VGPR staging): one 16-byte load per lane lands at
// LDS base + 16 * lane, so the swizzle is applied to the global addresses instead.
// Buffer resource over one head's [n][D] bf16 rows.
__device__ inline rsrc_t head_rsrc(const bf16_t* base, int n, int d) {
    return make_rsrc(base, (uint32_t)n * d * 2);
}

template <int D, int NT = 256>
struct Tile {
    static constexpr int CH = D / 8;
    static constexpr int SLOTS = KT * CH;           // 16-byte slots per tensor per tile
    static constexpr int PER_WAVE = SLOTS / NT;     // load instructions per wave per tensor

    // byte offset of this lane's 16-byte piece of load m (row phys[r], swizzled chunk)
    __device__ static int offset(const int* __restrict__ phys, int w, int lane, int m, int& first) {
        first = (w * PER_WAVE + m) * 64;
        const int slot = first + lane;
        const int r = slot / CH, pc = slot % CH;
        return (phys[r] * D + ((pc ^ swz<CH>(r)) * 8)) * 2;
    }
    // phys[] holds a valid row for every key of the tile (keys past the end of the
    // union repeat a real row and are masked out of the softmax).
    __device__ static void issue(rsrc_t rk, rsrc_t rv, const int* __restrict__ phys, uint4* sk,
                                 uint4* sv, int w, int lane) {
#pragma unroll
        for (int m = 0; m < PER_WAVE; ++m) {
            int first;
            const int off = offset(phys, w, lane, m, first);
            lds_load16(rk, sk + first, off);
            lds_load16(rv, sv + first, off);
        }
    }
    // rows row0 .. row0 + KT - 1 of both tensors (a contiguous tile)
    __device__ static void issue_rows(rsrc_t rk, rsrc_t rv, int row0, uint4* sk, uint4* sv, int w,
                                      int lane) {
#pragma unroll
        for (int m = 0; m < PER_WAVE; ++m) {
            const int first = (w * PER_WAVE + m) * 64;
            const int slot = first + lane;
            const int r = slot / CH, pc = slot % CH;
            const int off = ((row0 + r) * D + ((pc ^ swz<CH>(r)) * 8)) * 2;
            lds_load16(rk, sk + first, off);
            lds_load16(rv, sv + first, off);
        }
    }
    // rows row0 .. row0 + KT - 1 of one tensor (a contiguous tile)
    __device__ static void issue_rows_one(rsrc_t r, int row0, uint4* s, int w, int lane) {
#pragma unroll
        for (int m = 0; m < PER_WAVE; ++m) {
            const int first = (w * PER_WAVE + m) * 64;
            const int slot = first + lane;
            const int rr = slot / CH, pc = slot % CH;
            lds_load16(r, s + first, ((row0 + rr) * D + ((pc ^ swz<CH>(rr)) * 8)) * 2);
        }
    }
    // one tensor's tile (rows phys[]) into s
    __device__ static void issue_one(rsrc_t r, const int* __restrict__ phys, uint4* s, int w,
                                     int lane) {
#pragma unroll
        for (int m = 0; m < PER_WAVE; ++m) {
            int first;
            const int off = offset(phys, w, lane, m, first);
            lds_load16(r, s + first, off);
        }
    }
};

// FP8 K tiles (the fp8-logit experiment): rows of D bytes, 16-byte chunk c of row r at slot
// r * CH + (c ^ sw(r)), filled like Tile's from a resource over one head's [n][D] bytes.
template <int D, int NT = 256>
struct Tile8 {
    static constexpr int CH = D / 16;
    static constexpr int SLOTS = KT * CH;
    static constexpr int PER_WAVE = SLOTS / NT;
    __host__ __device__ static int sw(int r) { return CH >= 8 ? swz<8>(r) : (r & (CH - 1)); }
    __device__ static void issue_one(rsrc_t r, const int* __restrict__ phys, uint4* s, int w, int lane) {
        static_assert(SLOTS % NT == 0, "an fp8 tile must split evenly over the block");
#pragma unroll
        for (int m = 0; m < PER_WAVE; ++m) {
            const int first = (w * PER_WAVE + m) * 64;
            const int slot = first + lane;
            const int row = slot / CH, pc = slot % CH;
            lds_load16(r, s + first, phys[row] * D + (pc ^ sw(row)) * 16);
        }
    }
};

// Wait for this thread's outstanding direct loads, then for every wave of the block.
__device__ inline void tile_ready() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// S^T block kb (32 keys x 32 queries) of the tile for this lane's query column.
template <int D>
__device__ inline f32x16 qk_block(const uint4* __restrict__ sk, const uint4 (&qf)[D / 16], int kb,
                                  int lane) {
    constexpr int CH = D / 8;
    f32x16 s = {};
    const int row = kb * 32 + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 a = sk[row * CH + ((2 * kk + (lane >> 5)) ^ swz<CH>(row))];
        s = mfma32x32x16(a, qf[kk], s);
    }
    return s;
}

// A operand of O^T[db] += V^T P^T for 16-key slice s4: lane l needs V^T[dim][8 keys] with
// dim = db*32 + (l & 31) and keys 16*s4 + 4*(l/32) + {0..3} (slots 0..3) and the same + 8
// (slots 4..7) -- the key order of the P^T operand taken from the S^T accumulators.
// ds_read_tr16_b64 gives lane L of a 16-lane group element (L % 4) of the 8-byte chunks
// read by lanes L/4 + 4k (k = 0..3); so lane j supplies row key(j >> 2), columns
// base + 4 (j & 3), and lane L receives dim base + L at the four keys.
template <int D>
__device__ inline uint4 vt_frag(const uint4* __restrict__ sv, int db, int s4, int lane) {
    constexpr int CH = D / 8;
    const int g = lane >> 4, j = lane & 15;
    const int col = db * 32 + 16 * (g & 1) + 4 * (j & 3);
    const int key0 = 16 * s4 + 4 * (g >> 1) + (j >> 2);
    const int key1 = key0 + 8;
    const bf16_t* base = reinterpret_cast<const bf16_t*>(sv);
    const bf16_t* p0 = base + key0 * D + (((col >> 3) ^ swz<CH>(key0)) << 3) + (col & 7);
    const bf16_t* p1 = base + key1 * D + (((col >> 3) ^ swz<CH>(key1)) << 3) + (col & 7);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
    const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    return make_uint4(ua.x, ua.y, ub.x, ub.y);
}

// The same fragment from byte offsets computed once per kernel: o0, o1 locate this lane's
// two 8-byte reads for column block db at slice 0 (vt_offsets); slice s4 lies 16 keys further
// on, which keeps each key's low four bits and so its swizzle, a constant byte offset that
// the LDS instruction takes as its immediate.
template <int D>
__device__ inline void vt_offsets(int lane, int (&o0)[D / 32], int (&o1)[D / 32]) {
    constexpr int CH = D / 8;
    const int g = lane >> 4, j = lane & 15;
    const int key0 = 4 * (g >> 1) + (j >> 2), key1 = key0 + 8;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
        const int col = db * 32 + 16 * (g & 1) + 4 * (j & 3);
        o0[db] = 2 * (key0 * D + (((col >> 3) ^ swz<CH>(key0)) << 3) + (col & 7));
        o1[db] = 2 * (key1 * D + (((col >> 3) ^ swz<CH>(key1)) << 3) + (col & 7));
    }
}
template <int D>
__device__ inline uint4 vt_frag_at(const uint4* __restrict__ sv, int o0, int o1, int s4) {
    const char* base = reinterpret_cast<const char*>(sv) + s4 * 16 * D * 2;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + o0));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + o1));
    const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
    return make_uint4(ua.x, ua.y, ub.x, ub.y);
}

// Lanes l and l ^ 32 hold the two halves of one query column.
__device__ inline float pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

}  // namespace spr
