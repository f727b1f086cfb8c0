// Variable-block-sparse attention.
//
// "Partition the Support, Reconstruct the Residual" (gist.science summary), section 2C:
// tokens are in contiguous group-major order and each query group attends only to the
// union U_i of its routed key groups; the softmax is normalised over U_i alone (the
// block-selection item of "Attention Sparsity is Input-Stable ... Online QK
// Co-Clustering", papernotes.org). Unrouted key groups are never loaded or multiplied:
// a work unit walks the routed segments only (the cloud.baidu.com explainer's point that
// skipping, not computing-then-masking, is what saves work).
//
// Work unit = (head, query group, up to NW x 32 query rows); NW waves x 32 rows. The sparse
// call runs each query group's whole 256-row chunks, and a rest of more than 128 rows, as
// units of 8-wave blocks, which share each key tile over up to 256 rows and so walk the
// group's routed union once per 256 rows; a shorter rest runs in a unit of a 4-wave block,
// two per CU: those blocks wait at their tile barriers independently, so one block's waves
// keep the SIMDs busy while the other's wait. The dense baseline runs 8-wave blocks.
//   S^T = K Q^T  : A = K tile from LDS (row-major), B = Q^T fragments held in VGPRs
//   O^T += V^T P^T: A = V^T read from the row-major V tile with the transposing LDS
//                   read, B = P^T straight from the S^T accumulators (bf16, no
//                   cross-lane traffic)
// Keys stream in 64-key tiles packed across the routed segments (only the last tile
// of the union is partial), loaded global -> LDS directly (no VGPR staging),
// double-buffered, one barrier per tile. Softmax in fp32 base-2 with a lazily raised
// running max.
#include "attn_tile.h"

namespace spr {

namespace {

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
            // XCD x takes units [x n / 8, (x + 1) n / 8): eighths that differ by at most one
            // unit (ceil(n / 8) units each would leave the last XCD short on every head)
            const int n = s_cnt[i];
            const int lo = (x * n) >> 3, cnt = (((x + 1) * n) >> 3) - lo;
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

// P^T operand: two probabilities packed as fp16 (VH, V in scaled fp16) or bf16, and the
// row sum of exactly the packed values
template <bool VH>
__device__ inline uint32_t pack_p(float a, float b) {
    if constexpr (VH) return pack_f16x2(a, b);
    else return pack_bf16x2(a, b);
}
template <bool VH>
__device__ inline float sum_p(uint32_t w, float acc) {
    if constexpr (VH) return dot2_f16(w, ones_f16x2(), acc);
    else return dot2_bf16(w, ones_bf16x2(), acc);
}
template <bool VH>
__device__ inline f32x16 mfma_pv(uint4 v, uint4 p, f32x16 c) {
    if constexpr (VH) return mfma32x32x16_f16(v, p, c);
    else return mfma32x32x16(v, p, c);
}

// Block = NW waves x 32 query rows: a unit of up to NW x 32 rows shares every key tile.
// VH: V is group-major fp16 scaled per head by 2^e (vmax, see v_scale_exp), and P is
// rounded to fp16 with the 2^7 offset; otherwise V and P are bf16.
// F8 (the fp8-logit experiment, with VH): K is group-major FP8 E4M3 scaled per head by
// 2^f8_scale_exp(kmax[h]), Q rows are rounded to E4M3 on load after their own per-head
// scale (qmax), and S^T = K Q^T runs on the 32x32x64 fp8 instruction; the two scales are
// taken out of the logits with the softmax's own factor.
template <int D, int OUTM, int NW, bool VH, bool F8>
__global__ __launch_bounds__(NW * 64, 8 / NW) void k_vbsa(
    const bf16_t* __restrict__ qp, const int32_t* __restrict__ qperm, const void* __restrict__ kp,
    const bf16_t* __restrict__ vp, int n, const int32_t* __restrict__ qoff, int qoff_stride, const int32_t* __restrict__ koff,
    int koff_stride, const int32_t* __restrict__ blocks, int blocks_head_stride, int kblk,
    const int2* __restrict__ units, int units_head_stride, const int32_t* __restrict__ nunits,
    int nunits_stride, int heads, float scale_log2, const uint32_t* __restrict__ vmax,
    const uint32_t* __restrict__ qmax, const uint32_t* __restrict__ kmax, void* __restrict__ out) {
    constexpr int kVbsaThreads = NW * 64;
    using TL = Tile<D, kVbsaThreads>;
    using T8 = Tile8<D, kVbsaThreads>;
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
    const int rows = min(NW * 32, qo[gi + 1] - row0);
    const int32_t* ko = koff + (size_t)h * koff_stride;
    const int32_t* bl = blocks + (size_t)h * blocks_head_stride + (size_t)gi * kblk;
    const size_t head_row0 = (size_t)h * n;

    // routed segments: start row and length, then the exclusive prefix of the lengths
    // (one wave: each lane sums a contiguous run, then a wave scan of the run totals)
    for (int s = tid; s < kblk; s += kVbsaThreads) {
        const int j = bl[s];
        s_start[s] = (j >= 0) ? ko[j] : 0;
        s_pre[s + 1] = (j >= 0) ? (ko[j + 1] - ko[j]) : 0;
    }
    __syncthreads();
    if (w == 0) {
        const int per = (kblk + 63) / 64, b0 = min(lane * per, kblk), b1 = min(b0 + per, kblk);
        int run = 0;
        for (int s = b0; s < b1; ++s) run += s_pre[s + 1];
        int inc = run;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(inc, o, 64);
            if (lane >= o) inc += v;
        }
        int acc = inc - run;
        if (lane == 0) s_pre[0] = 0;
        for (int s = b0; s < b1; ++s) {
            acc += s_pre[s + 1];
            s_pre[s + 1] = acc;
        }
    }
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

    // Q^T fragments of this wave's 32 rows, gathered from token order through the
    // query permutation (none for the dense baseline)
    const bool active = w * 32 < rows;
    const int qrow = w * 32 + (lane & 31);
    const bool qvalid = qrow < rows;
    uint4 qf[F8 ? 1 : D / 16];
    i32x8 qf8[F8 ? D / 64 : 1];
    {
        const int src = !qvalid ? 0 : (qperm ? qperm[head_row0 + row0 + qrow] : row0 + qrow);
        if constexpr (!F8) {
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                qf[kk] = qvalid ? ldg16(qp + (head_row0 + src) * D + 16 * kk + 8 * (lane >> 5))
                                : make_uint4(0, 0, 0, 0);
        } else {
            // depth step ks: this lane's 32 dims 64 ks + 32 (lane / 32) .. +31, scaled and
            // rounded to E4M3 (the K fragments take the same 32 dims in the same order)
            const float qs = ldexpf(1.0f, f8_scale_exp(qmax[h]));
#pragma unroll
            for (int ks = 0; ks < D / 64; ++ks) {
                uint32_t wq[8];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint4 u = qvalid ? ldg16(qp + (head_row0 + src) * D + 64 * ks + 32 * (lane >> 5) + 8 * c)
                                           : make_uint4(0, 0, 0, 0);
                    const uint32_t e[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        wq[2 * c + j] = pack_e4m3x4(bf16_to_f32((bf16_t)(e[2 * j] & 0xFFFF)) * qs,
                                                    bf16_to_f32((bf16_t)(e[2 * j] >> 16)) * qs,
                                                    bf16_to_f32((bf16_t)(e[2 * j + 1] & 0xFFFF)) * qs,
                                                    bf16_to_f32((bf16_t)(e[2 * j + 1] >> 16)) * qs);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) qf8[ks][j] = (int)wq[j];
            }
        }
    }
    if constexpr (F8) scale_log2 = ldexpf(scale_log2, -(f8_scale_exp(qmax[h]) + f8_scale_exp(kmax[h])));

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const int half = lane >> 5;

    const rsrc_t rk = F8 ? make_rsrc(static_cast<const uint8_t*>(kp) + head_row0 * D, (uint32_t)n * D)
                         : head_rsrc(static_cast<const bf16_t*>(kp) + head_row0 * D, n, D);
    const rsrc_t rv = head_rsrc(vp + head_row0 * D, n, D);
    // this lane's fragment offsets inside a tile, computed once: K row (lane & 31) at each
    // depth step (row + 32 has the same swizzle, a constant offset), V^T per column block
    int kfo[F8 ? D / 32 : D / 16], vo0[DB], vo1[DB];
    {
        const int rl = lane & 31;
        if constexpr (!F8) {
            const int sw = swz<TL::CH>(rl);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) kfo[kk] = rl * TL::CH + ((2 * kk + half) ^ sw);
        } else {
            // fp8 rows of D bytes: the two 16-byte chunks 4 ks + 2 half + {0, 1} of step ks
            const int sw = T8::sw(rl);
#pragma unroll
            for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
                for (int c = 0; c < 2; ++c) kfo[2 * ks + c] = rl * T8::CH + ((4 * ks + 2 * half + c) ^ sw);
        }
        vt_offsets<D>(lane, vo0, vo1);
    }
    auto issue_tile = [&](const int* phys, uint4* sk, uint4* sv) {
        if constexpr (F8) {
            T8::issue_one(rk, phys, sk, w, lane);
            TL::issue_one(rv, phys, sv, w, lane);
        } else {
            TL::issue(rk, rv, phys, sk, sv, w, lane);
        }
    };
    fill_phys(0, 0);
    __syncthreads();
    issue_tile(s_phys[0], s_k0, s_v0);
    if (ntiles > 1) fill_phys(1, 1);
    tile_ready();

    // one tile: loads of tile t+1 into (nk, nv) overlap the math on (sk, sv)
    auto step = [&](int t, int buf, const uint4* sk, const uint4* sv, uint4* nk, uint4* nv) {
        if (t + 1 < ntiles) issue_tile(s_phys[buf ^ 1], nk, nv);
        if (active) {
            f32x16 s0 = {}, s1 = {};
            if constexpr (F8) {
                // S^T for both 32-key blocks from fp8 K and Q: D/64 depth steps each
                const uint4* k1s = sk + 32 * T8::CH;            // rows 32..63
                uint4 a0[D / 32], a1[D / 32];
#pragma unroll
                for (int i = 0; i < D / 32; ++i) {
                    a0[i] = sk[kfo[i]];
                    a1[i] = k1s[kfo[i]];
                }
#pragma unroll
                for (int ks = 0; ks < D / 64; ++ks) {
                    const i32x8 f0 = {(int)a0[2 * ks].x, (int)a0[2 * ks].y, (int)a0[2 * ks].z, (int)a0[2 * ks].w,
                                      (int)a0[2 * ks + 1].x, (int)a0[2 * ks + 1].y, (int)a0[2 * ks + 1].z,
                                      (int)a0[2 * ks + 1].w};
                    const i32x8 f1 = {(int)a1[2 * ks].x, (int)a1[2 * ks].y, (int)a1[2 * ks].z, (int)a1[2 * ks].w,
                                      (int)a1[2 * ks + 1].x, (int)a1[2 * ks + 1].y, (int)a1[2 * ks + 1].z,
                                      (int)a1[2 * ks + 1].w};
                    s0 = mfma32x32x64_f8(f0, qf8[ks], s0);
                    s1 = mfma32x32x64_f8(f1, qf8[ks], s1);
                }
            } else {
            // S^T for both 32-key blocks: two independent accumulation chains, the K
            // fragments read two depth steps ahead of their MFMAs (a ring of three)
            constexpr int KA = 2;
            const uint4* k1s = sk + 32 * TL::CH;                // rows 32..63
            uint4 a0[KA + 1], a1[KA + 1];
#pragma unroll
            for (int kk = 0; kk < KA; ++kk) {
                a0[kk] = sk[kfo[kk]];
                a1[kk] = k1s[kfo[kk]];
            }
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                if (kk + KA < D / 16) {
                    a0[(kk + KA) % (KA + 1)] = sk[kfo[kk + KA]];
                    a1[(kk + KA) % (KA + 1)] = k1s[kfo[kk + KA]];
                }
                s0 = mfma32x32x16(a0[kk % (KA + 1)], qf[kk], s0);
                s1 = mfma32x32x16(a1[kk % (KA + 1)], qf[kk], s1);
                __builtin_amdgcn_sched_barrier(0);          // keep the reads KA steps ahead
            }
            }
            // V^T fragments of keys 0..31, read now so that the softmax hides their latency
            uint4 vf[2][DB];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int db = 0; db < DB; ++db) vf[sl][db] = vt_frag_at<D>(sv, vo0[db], vo1[db], sl);
            const int nvk = U - t * KT;
            if (nvk < KT) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 8 * (r >> 2) + 4 * half + (r & 3);
                    s0[r] = (key < nvk) ? s0[r] : -INFINITY;
                    s1[r] = (key + 32 < nvk) ? s1[r] : -INFINITY;
                }
            }
            // two chains of three-input maxima (15 v_max3 + 1 v_max for the 32 logits)
            float ma = fmaxf(s0[0], s1[0]), mb = fmaxf(s0[1], s1[1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) {
                ma = fmaxf(fmaxf(ma, s0[r]), s1[r]);
                mb = fmaxf(fmaxf(mb, s0[r + 1]), s1[r + 1]);
            }
            float mx = pair_max(fmaxf(ma, mb));
            const float mt = mx * scale_log2;
            if (__ballot(mt > m_run + kLazy)) {
                const float mnew = fmaxf(m_run, mt);
                const float alpha = fast_exp2(m_run - mnew);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db] *= alpha;
                m_run = mnew;
            }
            const float mneg = VH ? kP16Offset - m_run : -m_run;
            // P^T slices 0,1 (keys 0..31)
            uint4 pb[4];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                uint32_t wv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 8 * sl + 2 * i;
                    wv[i] = pack_p<VH>(fast_exp2(fmaf(s0[r], scale_log2, mneg)),
                                       fast_exp2(fmaf(s0[r + 1], scale_log2, mneg)));
                    l_run = sum_p<VH>(wv[i], l_run);
                }
                pb[sl] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
            // PV of keys 0..31; each consumed fragment's registers take the fragment of
            // the slice two further on, and the exponentials of keys 32..63 run alongside
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    o[db] = mfma_pv<VH>(vf[sl][db], pb[sl], o[db]);
                    vf[sl][db] = vt_frag_at<D>(sv, vo0[db], vo1[db], sl + 2);
                }
#pragma unroll
            for (int sl = 2; sl < 4; ++sl) {
                uint32_t wv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 8 * (sl - 2) + 2 * i;
                    wv[i] = pack_p<VH>(fast_exp2(fmaf(s1[r], scale_log2, mneg)),
                                       fast_exp2(fmaf(s1[r + 1], scale_log2, mneg)));
                    l_run = sum_p<VH>(wv[i], l_run);
                }
                pb[sl] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
#pragma unroll
            for (int sl = 2; sl < 4; ++sl)
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db] = mfma_pv<VH>(vf[sl - 2][db], pb[sl], o[db]);
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
    float inv = 1.0f / l_run;
    if constexpr (VH) inv *= ldexpf(1.0f, -v_scale_exp(vmax[h]));      // undo the V scale
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

void launch_vbsa(const bf16_t* qp, const int32_t* qperm, const bf16_t* kp, const void* vp,
                 const uint32_t* vmax, int heads, int n, int d,
                 const int32_t* qoff, int qoff_stride, const int32_t* koff, int koff_stride,
                 const int32_t* blocks, int blocks_head_stride, int kblk, const int2* units,
                 int units_head_stride, const int32_t* nunits, int nunits_stride, int max_units,
                 int unit_rows, void* out, int out_mode, hipStream_t st, const uint8_t* kp8,
                 const uint32_t* qmax, const uint32_t* kmax) {
    const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    // 8 XCD slots per round of units: enough blocks for every head's units at any split
    dim3 grid(8 * ((max_units + 7) / 8), heads);
#define SPR_VBSA(DD, MM, NW, VH, F8, KP)                                                        \
    hipLaunchKernelGGL((k_vbsa<DD, MM, NW, VH, F8>), grid, dim3(NW * 64), 0, st, qp, qperm,      \
                       static_cast<const void*>(KP), static_cast<const bf16_t*>(vp), n, qoff,     \
                       qoff_stride, koff, koff_stride, blocks, blocks_head_stride, kblk, units,   \
                       units_head_stride, nunits, nunits_stride, heads, scale_log2, vmax, qmax,  \
                       kmax, out)
    // the sparse call: fp16 V with its per-head scale (vmax != nullptr), fp32 output, 4-wave
    // blocks for 128-row units and 8-wave blocks for 256-row units; with kp8 (128-row units
    // only) the fp8 logits. The dense baseline: 8-wave blocks, bf16 V.
    if (unit_rows == kSparseRows && vmax && kp8) {
        if (d == 128) {
            if (out_mode == 0) SPR_VBSA(128, 0, 4, true, true, kp8); else SPR_VBSA(128, 1, 4, true, true, kp8);
        } else {
            if (out_mode == 0) SPR_VBSA(64, 0, 4, true, true, kp8); else SPR_VBSA(64, 1, 4, true, true, kp8);
        }
    } else if (unit_rows == kSparseRows && vmax) {
        if (d == 128) {
            if (out_mode == 0) SPR_VBSA(128, 0, 4, true, false, kp); else SPR_VBSA(128, 1, 4, true, false, kp);
        } else {
            if (out_mode == 0) SPR_VBSA(64, 0, 4, true, false, kp); else SPR_VBSA(64, 1, 4, true, false, kp);
        }
    } else if (vmax) {
        if (d == 128) {
            if (out_mode == 0) SPR_VBSA(128, 0, 8, true, false, kp); else SPR_VBSA(128, 1, 8, true, false, kp);
        } else {
            if (out_mode == 0) SPR_VBSA(64, 0, 8, true, false, kp); else SPR_VBSA(64, 1, 8, true, false, kp);
        }
    } else {
        if (d == 128) {
            if (out_mode == 0) SPR_VBSA(128, 0, 8, false, false, kp); else SPR_VBSA(128, 1, 8, false, false, kp);
        } else {
            if (out_mode == 0) SPR_VBSA(64, 0, 8, false, false, kp); else SPR_VBSA(64, 1, 8, false, false, kp);
        }
    }
#undef SPR_VBSA
}

}  // namespace spr
