// Variable-block-sparse attention and exact probe rows.
//
// "Partition the Support, Reconstruct the Residual" (gist.science summary), section 2C:
// tokens are in contiguous group-major order and each query group attends only to the
// union U_i of its routed key groups; the softmax is normalised over U_i alone (the
// block-selection item of "Attention Sparsity is Input-Stable ... Online QK
// Co-Clustering", papernotes.org). Unrouted key groups are never loaded or multiplied:
// a work unit walks the routed segments only (the cloud.baidu.com explainer's point that
// skipping, not computing-then-masking, is what saves work). Section 2B: probe rows get
// the exact dense output and the routed-subset output from the same logits.
//
// Work unit = (head, query group, up to 256 query rows); 8 waves x 32 rows.
//   S^T = K Q^T  : A = K tile from LDS (row-major), B = Q^T fragments held in VGPRs
//   O^T += V^T P^T: A = V^T read from the row-major V tile with the transposing LDS
//                   read, B = P^T straight from the S^T accumulators (bf16, no
//                   cross-lane traffic)
// Keys stream in 64-key tiles packed across the routed segments (only the last tile
// of the union is partial), loaded global -> LDS directly (no VGPR staging),
// double-buffered, one barrier per tile. Softmax in fp32 base-2 with a lazily raised
// running max.
#include "kernels.h"

#include <cmath>

namespace spr {

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

// Lanes l and l ^ 32 hold the two halves of one query column.
__device__ inline float pair_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work units are dealt so that the 8 XCDs work through the heads together (the head's
// keys and values stay hot in the shared last-level cache) while each XCD takes a
// contiguous eighth of every head's unit list (units of one query group stream the same
// key tiles and so share that XCD's L2). The hardware hands workgroups to the XCDs
// round-robin, so block b runs on XCD b % 8 as that XCD's (b / 8)-th workgroup.
// Returns false for blocks past the last unit. `s_cnt` is LDS scratch of 256 ints;
// every thread of the block must call this.
__device__ inline bool unit_of_block(const int32_t* __restrict__ nunits, int stride, int heads,
                                     int* s_cnt, int& h, int& ui) {
    const int lid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int x = lid & 7;
    int k = lid >> 3;
    bool found = false;
    h = 0;
    ui = 0;
    for (int h0 = 0; h0 < heads; h0 += 256) {
        const int nh = min(256, heads - h0);
        __syncthreads();
        if ((int)threadIdx.x < nh) s_cnt[threadIdx.x] = nunits[(size_t)(h0 + threadIdx.x) * stride];
        __syncthreads();
        for (int i = 0; i < nh && !found; ++i) {
            const int n = s_cnt[i], c = (n + 7) >> 3;
            const int lo = min(x * c, n), cnt = min(lo + c, n) - lo;
            if (k < cnt) {
                h = h0 + i;
                ui = lo + k;
                found = true;
            } else {
                k -= cnt;
            }
        }
    }
    __syncthreads();
    return found;
}

}  // namespace

// Block = 8 waves x 32 query rows: a unit of up to 256 rows shares every key tile.
constexpr int kVbsaThreads = 512;
template <int D, int OUTM>
__global__ __launch_bounds__(kVbsaThreads, 1) void k_vbsa(
    const bf16_t* __restrict__ qp, const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vp,
    int n, const int32_t* __restrict__ qoff, int qoff_stride, const int32_t* __restrict__ koff,
    int koff_stride, const int32_t* __restrict__ blocks, int blocks_head_stride, int kblk,
    const int2* __restrict__ units, int units_head_stride, const int32_t* __restrict__ nunits,
    int nunits_stride, int heads, float scale_log2, void* __restrict__ out) {
    using TL = Tile<D, kVbsaThreads>;
    constexpr int DB = D / 32;
    __shared__ int s_pre[kMaxGroups + 1];
    __shared__ int s_start[kMaxGroups];
    __shared__ int s_phys[2][KT];
    // distinct arrays per buffer: the compiler then knows that the loads in flight into
    // one buffer cannot alias the reads of the other (no wait before the tile math)
    __shared__ uint4 s_k0[TL::SLOTS], s_k1[TL::SLOTS];
    __shared__ uint4 s_v0[TL::SLOTS], s_v1[TL::SLOTS];

    int h, ui;
    if (!unit_of_block(nunits, nunits_stride, heads, s_start, h, ui)) return;
    h = __builtin_amdgcn_readfirstlane(h);
    ui = __builtin_amdgcn_readfirstlane(ui);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int2 un = units[(size_t)h * units_head_stride + ui];
    const int gi = un.x, row0 = un.y;
    const int32_t* qo = qoff + (size_t)h * qoff_stride;
    const int rows = min(kAttnRows, qo[gi + 1] - row0);
    const int32_t* ko = koff + (size_t)h * koff_stride;
    const int32_t* bl = blocks + (size_t)h * blocks_head_stride + (size_t)gi * kblk;
    const size_t head_row0 = (size_t)h * n;

    for (int s = tid; s < kblk; s += kVbsaThreads) {
        const int j = bl[s];
        s_start[s] = (j >= 0) ? ko[j] : 0;
        s_pre[s + 1] = (j >= 0) ? (ko[j + 1] - ko[j]) : 0;
    }
    if (tid == 0) s_pre[0] = 0;
    __syncthreads();
    if (tid == 0)
        for (int s = 1; s <= kblk; ++s) s_pre[s] += s_pre[s - 1];
    __syncthreads();
    const int U = s_pre[kblk];
    const int ntiles = (U + KT - 1) / KT;

    // rows of tile t; keys past the union repeat the tile's first row (masked later).
    // Tiles are filled in order by the first wave: each lane advances from the segment of
    // the previous tile's last key (usually zero or one step) instead of a binary search.
    int seg_carry = 0;
    auto fill_phys = [&](int t, int buf) {
        if (tid < KT) {
            const int u = (t * KT + tid < U) ? t * KT + tid : t * KT;
            int sg = seg_carry;
            while (s_pre[sg + 1] <= u) ++sg;
            s_phys[buf][tid] = s_start[sg] + (u - s_pre[sg]);
            seg_carry = __shfl(sg, KT - 1, 64);
        }
    };

    // Q^T fragments of this wave's 32 rows
    const bool active = w * 32 < rows;
    const int qrow = w * 32 + (lane & 31);
    const bool qvalid = qrow < rows;
    uint4 qf[D / 16];
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = qvalid ? ldg16(qp + (head_row0 + row0 + qrow) * D + 16 * kk + 8 * (lane >> 5))
                        : make_uint4(0, 0, 0, 0);

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const bf16x2 ones = ones_bf16x2();
    const int half = lane >> 5;

    const rsrc_t rk = head_rsrc(kp + head_row0 * D, n, D);
    const rsrc_t rv = head_rsrc(vp + head_row0 * D, n, D);
    fill_phys(0, 0);
    __syncthreads();
    TL::issue(rk, rv, s_phys[0], s_k0, s_v0, w, lane);
    if (ntiles > 1) fill_phys(1, 1);
    tile_ready();

    // one tile: loads of tile t+1 into (nk, nv) overlap the math on (sk, sv)
    auto step = [&](int t, int buf, const uint4* sk, const uint4* sv, uint4* nk, uint4* nv) {
        if (t + 1 < ntiles) TL::issue(rk, rv, s_phys[buf ^ 1], nk, nv, w, lane);
        if (active) {
            // S^T for both 32-key blocks: two independent accumulation chains, the K
            // fragments read one depth step ahead of their MFMAs
            const int rl = lane & 31, sw = swz<TL::CH>(rl);     // same swizzle for row + 32
            const uint4* k0p = sk + rl * TL::CH;
            const uint4* k1p = sk + (32 + rl) * TL::CH;
            f32x16 s0 = {}, s1 = {};
            uint4 a0 = k0p[half ^ sw], a1 = k1p[half ^ sw];
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                uint4 n0 = a0, n1 = a1;
                if (kk + 1 < D / 16) {
                    const int c = (2 * (kk + 1) + half) ^ sw;
                    n0 = k0p[c];
                    n1 = k1p[c];
                }
                s0 = mfma32x32x16(a0, qf[kk], s0);
                s1 = mfma32x32x16(a1, qf[kk], s1);
                a0 = n0;
                a1 = n1;
            }
            // V^T fragments of keys 0..31, read now so that the softmax hides their latency
            uint4 vf[2][DB];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int db = 0; db < DB; ++db) vf[sl][db] = vt_frag<D>(sv, db, sl, lane);
            const int nvk = U - t * KT;
            if (nvk < KT) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 8 * (r >> 2) + 4 * half + (r & 3);
                    s0[r] = (key < nvk) ? s0[r] : -INFINITY;
                    s1[r] = (key + 32 < nvk) ? s1[r] : -INFINITY;
                }
            }
            float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
            mx = pair_max(mx);
            const float mt = mx * scale_log2;
            if (__ballot(mt > m_run + kLazy)) {
                const float mnew = fmaxf(m_run, mt);
                const float alpha = fast_exp2(m_run - mnew);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db] *= alpha;
                m_run = mnew;
            }
            const float mneg = -m_run;
            // P^T slices 0,1 (keys 0..31)
            uint4 pb[4];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                uint32_t wv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 8 * sl + 2 * i;
                    wv[i] = pack_bf16x2(fast_exp2(fmaf(s0[r], scale_log2, mneg)),
                                        fast_exp2(fmaf(s0[r + 1], scale_log2, mneg)));
                    l_run = dot2_bf16(wv[i], ones, l_run);
                }
                pb[sl] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
            // PV of keys 0..31; each consumed fragment's registers take the fragment of
            // the slice two further on, and the exponentials of keys 32..63 run alongside
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    o[db] = mfma32x32x16(vf[sl][db], pb[sl], o[db]);
                    vf[sl][db] = vt_frag<D>(sv, db, sl + 2, lane);
                }
#pragma unroll
            for (int sl = 2; sl < 4; ++sl) {
                uint32_t wv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 8 * (sl - 2) + 2 * i;
                    wv[i] = pack_bf16x2(fast_exp2(fmaf(s1[r], scale_log2, mneg)),
                                        fast_exp2(fmaf(s1[r + 1], scale_log2, mneg)));
                    l_run = dot2_bf16(wv[i], ones, l_run);
                }
                pb[sl] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
#pragma unroll
            for (int sl = 2; sl < 4; ++sl)
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db] = mfma32x32x16(vf[sl - 2][db], pb[sl], o[db]);
        }
        if (t + 2 < ntiles) fill_phys(t + 2, buf);
        tile_ready();
    };
    for (int t = 0; t < ntiles; t += 2) {
        step(t, 0, s_k0, s_v0, s_k1, s_v1);
        if (t + 1 < ntiles) step(t + 1, 1, s_k1, s_v1, s_k0, s_v0);
    }

    if (!active) return;
    l_run = pair_sum(l_run);
    const float inv = 1.0f / l_run;
    if (!qvalid) return;
    const size_t orow = head_row0 + row0 + qrow;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dim = db * 32 + 8 * g + 4 * half;
            const float v0 = o[db][4 * g] * inv, v1 = o[db][4 * g + 1] * inv;
            const float v2 = o[db][4 * g + 2] * inv, v3 = o[db][4 * g + 3] * inv;
            if (OUTM == 0) {
                *reinterpret_cast<float4*>(static_cast<float*>(out) + orow * D + dim) =
                    make_float4(v0, v1, v2, v3);
            } else {
                *reinterpret_cast<uint2*>(static_cast<bf16_t*>(out) + orow * D + dim) =
                    make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
            }
        }
}

void launch_vbsa(const bf16_t* qp, const bf16_t* kp, const bf16_t* vp, int heads, int n, int d,
                 const int32_t* qoff, int qoff_stride, const int32_t* koff, int koff_stride,
                 const int32_t* blocks, int blocks_head_stride, int kblk, const int2* units,
                 int units_head_stride, const int32_t* nunits, int nunits_stride, int max_units,
                 void* out, int out_mode, hipStream_t st) {
    const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    // 8 XCD slots per round of units: enough blocks for every head's units at any split
    dim3 grid(8 * ((max_units + 7) / 8), heads);
#define SPR_VBSA(DD, MM)                                                                     \
    hipLaunchKernelGGL((k_vbsa<DD, MM>), grid, dim3(kVbsaThreads), 0, st, qp, kp, vp, n, qoff,        \
                       qoff_stride, koff, koff_stride, blocks, blocks_head_stride, kblk, units, \
                       units_head_stride, nunits, nunits_stride, heads, scale_log2, out)
    if (d == 128) {
        if (out_mode == 0) SPR_VBSA(128, 0); else SPR_VBSA(128, 1);
    } else {
        if (out_mode == 0) SPR_VBSA(64, 0); else SPR_VBSA(64, 1);
    }
#undef SPR_VBSA
}

// ------------------------------------------------------------------- probes ---
// Work unit = (head, 256 probe rows = 8 waves of 32, one contiguous split of the head's
// keys). Keys are in group-major order, so a split's tiles are plain row ranges and the
// routed keys of a tile are whole runs of groups found from the group offsets. Both
// accumulators share the logits: the dense one over every key, the routed one over keys
// whose group is routed for the probe's query group. P.V uses a bf16 hi/lo split of P
// (about 2^-17 relative) so that the probe outputs are near fp32 accuracy. Partial (max,
// sum, unnormalised O) per split. Two waves share each SIMD (one block per CU), so one
// wave's exponentials overlap the other's matrix products.
int probe_splits(int n, int heads, int probes) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0) != hipSuccess ||
        cus <= 0)
        cus = 256;
    const int units = heads * std::max(1, (probes + kProbeRows - 1) / kProbeRows);
    const int max_s = std::max(1, std::min(128, (n + KT - 1) / KT));
    // fewest key tiles per CU over the whole grid (one block per CU at a time), plus a
    // per-block cost of two tiles for the prologue and the partial write
    int best = 1;
    long best_cost = -1;
    for (int s = 1; s <= max_s; ++s) {
        const int chunk = ((n + s - 1) / s + KT - 1) / KT;        // tiles per block
        const long rounds = ((long)units * s + cus - 1) / cus;
        const long cost = rounds * (chunk + 2);
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = s; }
    }
    return best;
}

template <int D>
__global__ __launch_bounds__(512, 1) void k_probe(
    const bf16_t* __restrict__ qp, const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vp,
    int n, const int32_t* __restrict__ probe_pos, const int32_t* __restrict__ probe_grp,
    int probes, const int32_t* __restrict__ koff, int koff_stride, int gk,
    const int32_t* __restrict__ blocks, int gq, int kblk, int chunk, float scale_log2,
    float* __restrict__ part_ml, float* __restrict__ part_od, float* __restrict__ part_os) {
    using TL = Tile<D, 512>;
    constexpr int DB = D / 32;
    constexpr int BW = kMaxGroups / 32 + 1;                      // odd row pitch: no bank conflicts
    __shared__ uint32_t s_bits[kProbeRows][BW];
    __shared__ int s_ko[kMaxGroups + 1];
    __shared__ uint4 s_k[2][TL::SLOTS];
    __shared__ uint4 s_v[2][TL::SLOTS];

    const int h = blockIdx.z, split = blockIdx.y, splits = gridDim.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5;
    const int p0 = blockIdx.x * kProbeRows;
    const size_t head_row0 = (size_t)h * n;
    const int32_t* ko = koff + (size_t)h * koff_stride;
    const int k0 = split * chunk;
    const int k1 = min(n, k0 + chunk);
    const int ntiles = (max(0, k1 - k0) + KT - 1) / KT;
    const rsrc_t rk = head_rsrc(kp + head_row0 * D, n, D);
    const rsrc_t rv = head_rsrc(vp + head_row0 * D, n, D);
    // the first tile's loads go out before the routing bits are set up; rows past the
    // split are masked below and rows past the head read as zeros
    if (ntiles > 0) TL::issue_rows(rk, rv, k0, s_k[0], s_v[0], w, lane);
    for (int i = tid; i < kProbeRows * BW; i += 512) (&s_bits[0][0])[i] = 0u;
    for (int g = tid; g <= gk; g += 512) s_ko[g] = ko[g];
    __syncthreads();
    for (int i = tid; i < kProbeRows * kblk; i += 512) {
        const int lp = i / kblk, s = i - lp * kblk;
        const int p = p0 + lp;
        if (p < probes) {
            const int grp = probe_grp[(size_t)h * probes + p];
            const int j = blocks[((size_t)h * gq + grp) * kblk + s];
            if (j >= 0) atomicOr(&s_bits[lp][j >> 5], 1u << (j & 31));
        }
    }

    const int lp = w * 32 + (lane & 31);
    const int p = p0 + lp;
    const bool pvalid = p < probes;
    const bool active = p0 + w * 32 < probes;
    uint4 qf[D / 16];
    {
        const int qrow = pvalid ? probe_pos[(size_t)h * probes + p] : 0;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qf[kk] = pvalid ? ldg16(qp + (head_row0 + qrow) * D + 16 * kk + 8 * (lane >> 5))
                            : make_uint4(0, 0, 0, 0);
    }
    // oa: routed keys, ob: the other keys; the dense output is oa + ob. One running max
    // (of all keys, raised lazily) scales both, so each logit needs one exponential.
    f32x16 oa[DB], ob[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { oa[db] = f32x16{}; ob[db] = f32x16{}; }
    // row sums of the routed (ls) and other (lb) parts, both from the same bf16 hi + lo
    // operands as the products: with every key routed lb stays 0 and the dense and
    // routed outputs come out bit-identical
    float m_run = -INFINITY, lb = 0.f, ls = 0.f;
    const bf16x2 ones = ones_bf16x2();
    int gcur = 0;                                   // group of the current tile's first key

    tile_ready();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        const int base = k0 + t * KT;
        if (t + 1 < ntiles) TL::issue_rows(rk, rv, base + KT, s_k[buf ^ 1], s_v[buf ^ 1], w, lane);
        if (active) {
            f32x16 sv[2];
            sv[0] = qk_block<D>(s_k[buf], qf, 0, lane);
            sv[1] = qk_block<D>(s_k[buf], qf, 1, lane);
            const int nvk = min(KT, k1 - base);
            // routed keys of the tile as a bit mask, from the runs of groups it holds
            while (s_ko[gcur + 1] <= base) ++gcur;
            uint64_t mask = 0;
            for (int g = gcur; g < gk && s_ko[g] < base + nvk; ++g) {
                if ((s_bits[lp][g >> 5] >> (g & 31)) & 1u) {
                    const int lo = max(0, s_ko[g] - base), hi = min(nvk, s_ko[g + 1] - base);
                    if (hi > lo) {
                        const uint64_t upto_hi = (hi >= 64) ? ~0ull : ((1ull << hi) - 1);
                        mask |= upto_hi & ~((1ull << lo) - 1);
                    }
                }
            }
            const uint64_t mh = mask >> (4 * half);    // this lane's keys sit 4*half further on
            const uint32_t mw[2] = {(uint32_t)mh, (uint32_t)(mh >> 32)};
            // raw logits; the scale (> 0) is applied to the max and inside the exponent
            if (nvk < KT) {                             // a split's ragged last tile
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                        if (key >= nvk) sv[kb][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[kb][r]);
            mx = pair_max(mx) * scale_log2;
            if (__ballot(mx > m_run + kLazy)) {
                const float mnew = fmaxf(m_run, mx);
                const float alpha = fast_exp2(m_run - mnew);
                lb *= alpha;
                ls *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) { oa[db] *= alpha; ob[db] *= alpha; }
                m_run = mnew;
            }
            const float mneg = -m_run;
            // per 16-key slice: P as bf16 hi + lo, each split by the routed mask of its
            // two keys into the (a) and (b) operands, then the slice's products
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) {
                uint32_t a0[4], a1[4], b0[4], b1[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kb = sl >> 1, r = 8 * (sl & 1) + 2 * i;
                    const float e0 = fast_exp2(fmaf(sv[kb][r], scale_log2, mneg));
                    const float e1 = fast_exp2(fmaf(sv[kb][r + 1], scale_log2, mneg));
                    const uint32_t hi = pack_bf16x2(e0, e1);
                    const uint32_t lo = pack_bf16x2(e0 - bf16_to_f32((bf16_t)(hi & 0xFFFF)),
                                                    e1 - bf16_to_f32((bf16_t)(hi >> 16)));
                    // bits of keys r, r+1 of block kb: 0xFFFF halves where routed
                    const int b = 8 * (r >> 2) + (r & 3);
                    const uint32_t word = mw[kb];
                    const uint32_t sel = (((word >> b) & 1u) ? 0x0000FFFFu : 0u) |
                                         (((word >> (b + 1)) & 1u) ? 0xFFFF0000u : 0u);
                    a0[i] = hi & sel;
                    b0[i] = hi ^ a0[i];
                    a1[i] = lo & sel;
                    b1[i] = lo ^ a1[i];
                    ls = dot2_bf16(a0[i], ones, ls);
                    ls = dot2_bf16(a1[i], ones, ls);
                    lb = dot2_bf16(b0[i], ones, lb);
                    lb = dot2_bf16(b1[i], ones, lb);
                }
                const uint4 ah = make_uint4(a0[0], a0[1], a0[2], a0[3]);
                const uint4 al = make_uint4(a1[0], a1[1], a1[2], a1[3]);
                const uint4 bh = make_uint4(b0[0], b0[1], b0[2], b0[3]);
                const uint4 bl = make_uint4(b1[0], b1[1], b1[2], b1[3]);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint4 a = vt_frag<D>(s_v[buf], db, sl, lane);
                    oa[db] = mfma32x32x16(a, ah, oa[db]);
                    ob[db] = mfma32x32x16(a, bh, ob[db]);
                    oa[db] = mfma32x32x16(a, al, oa[db]);
                    ob[db] = mfma32x32x16(a, bl, ob[db]);
                }
            }
        }
        tile_ready();
    }
    if (!active) return;
    lb = pair_sum(lb);
    ls = pair_sum(ls);
    if (!pvalid) return;
    const size_t base = ((size_t)h * splits + split) * probes + p;
    if (lane < 32) {
        float4* ml = reinterpret_cast<float4*>(part_ml) + base;
        *ml = make_float4(m_run, ls + lb, m_run, ls);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dim = db * 32 + 8 * g + 4 * (lane >> 5);
            const f32x16& a = oa[db];
            const f32x16& b = ob[db];
            *reinterpret_cast<float4*>(part_od + base * D + dim) =
                make_float4(a[4 * g] + b[4 * g], a[4 * g + 1] + b[4 * g + 1], a[4 * g + 2] + b[4 * g + 2],
                            a[4 * g + 3] + b[4 * g + 3]);
            *reinterpret_cast<float4*>(part_os + base * D + dim) =
                make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
        }
}

void launch_probe(const bf16_t* qp, const bf16_t* kp, const bf16_t* vp, int heads, int n, int d,
                  const int32_t* probe_pos, const int32_t* probe_grp, int probes,
                  const int32_t* koff, int koff_stride, int gk, const int32_t* blocks, int gq,
                  int kblk, int splits, float* part_ml, float* part_od, float* part_os,
                  hipStream_t st) {
    if (probes == 0) return;
    int chunk = (n + splits - 1) / splits;
    chunk = (chunk + KT - 1) / KT * KT;
    const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    dim3 grid((probes + kProbeRows - 1) / kProbeRows, splits, heads);
    if (d == 128)
        hipLaunchKernelGGL(k_probe<128>, grid, dim3(512), 0, st, qp, kp, vp, n, probe_pos, probe_grp,
                           probes, koff, koff_stride, gk, blocks, gq, kblk, chunk, scale_log2,
                           part_ml, part_od, part_os);
    else
        hipLaunchKernelGGL(k_probe<64>, grid, dim3(512), 0, st, qp, kp, vp, n, probe_pos, probe_grp,
                           probes, koff, koff_stride, gk, blocks, gq, kblk, chunk, scale_log2,
                           part_ml, part_od, part_os);
}

// Merge the key splits of every probe row in split order; X = routed output,
// Y = dense - routed, and the dense output itself.
__global__ void k_probe_merge(int probes, int d, int splits, const float* __restrict__ part_ml,
                              const float* __restrict__ part_od, const float* __restrict__ part_os,
                              float* __restrict__ x, float* __restrict__ y,
                              float* __restrict__ od) {
    const int h = blockIdx.y, p = blockIdx.x, j = threadIdx.x;
    if (j >= d) return;
    const float4* ml = reinterpret_cast<const float4*>(part_ml);
    float mdx = -INFINITY, msx = -INFINITY;
    for (int s = 0; s < splits; ++s) {
        const float4 v = ml[((size_t)h * splits + s) * probes + p];
        mdx = fmaxf(mdx, v.x);
        msx = fmaxf(msx, v.z);
    }
    float sd = 0.f, ss = 0.f, nd = 0.f, ns = 0.f;
    for (int s = 0; s < splits; ++s) {
        const size_t base = ((size_t)h * splits + s) * probes + p;
        const float4 v = ml[base];
        const float wd = (v.x == -INFINITY) ? 0.f : exp2f(v.x - mdx);
        const float ws = (v.z == -INFINITY) ? 0.f : exp2f(v.z - msx);
        sd += wd * v.y;
        ss += ws * v.w;
        nd += wd * part_od[base * d + j];
        ns += ws * part_os[base * d + j];
    }
    const float vd = nd / sd, vs = ns / ss;
    const size_t o = ((size_t)h * probes + p) * d + j;
    x[o] = vs;
    y[o] = vd - vs;
    od[o] = vd;
}

void launch_probe_merge(int heads, int probes, int d, int splits, const float* part_ml,
                        const float* part_od, const float* part_os, float* x, float* y, float* od,
                        hipStream_t st) {
    if (probes == 0) return;
    hipLaunchKernelGGL(k_probe_merge, dim3(probes, heads), dim3(128), 0, st, probes, d, splits,
                       part_ml, part_od, part_os, x, y, od);
}

}  // namespace spr
