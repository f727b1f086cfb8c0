// Exact probe rows.
//
// "Partition the Support, Reconstruct the Residual" (gist.science summary), section 2B:
// for a sample of query rows the call computes the exact dense attention output and,
// from the same logits, the output restricted to the row's routed key groups; their
// difference is the residual that the probe fit learns to predict.
#include "attn_tile.h"

namespace spr {

// ------------------------------------------------------------------- probes ---
// Work unit = (head, 256 probe rows = 8 waves of 32, one contiguous split of the head's
// keys). Keys are in group-major order, so a split's tiles are plain row ranges and the
// routed keys of a tile are whole runs of groups found from the group offsets. Both
// accumulators share the logits: the dense one over every key, the routed one over keys
// whose group is routed for the probe's query group. P.V uses a bf16 hi/lo split of P
// (about 2^-17 relative) so that the probe outputs are near fp32 accuracy; V is the bf16
// input in token order, its rows gathered through the key permutation (bf16 keeps fp32's
// exponent range, so the routed weights stay exact even when the row's largest logit lies
// outside its routed groups and every routed weight is tiny). Partial (max,
// sum, unnormalised O) per split. Two waves share each SIMD (one block per CU), so one
// wave's exponentials overlap the other's matrix products.
int probe_splits(int n, int heads, int probes) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
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
    const bf16_t* __restrict__ qp, const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vtok,
    const int32_t* __restrict__ kperm, int n, const int32_t* __restrict__ probe_orig, const int32_t* __restrict__ probe_grp,
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
    __shared__ int s_vrow[2][KT];                 // token rows of a tile's keys (V gather)

    const int h = blockIdx.z, split = blockIdx.y, splits = gridDim.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5;
    const int p0 = blockIdx.x * kProbeRows;
    const size_t head_row0 = (size_t)h * n;
    const int32_t* ko = koff + (size_t)h * koff_stride;
    const int k0 = split * chunk;
    const int k1 = min(n, k0 + chunk);
    const int ntiles = (max(0, k1 - k0) + KT - 1) / KT;
    const rsrc_t rk = head_rsrc(kp + head_row0 * D, n, D);
    const rsrc_t rv = head_rsrc(vtok + head_row0 * D, n, D);
    // token row of group-major key position pos; positions past the head are clamped to a
    // real row (their logits are masked below)
    const int32_t* kpm = kperm + head_row0;
    auto vrow = [&](int pos) { return kpm[min(pos, n - 1)]; };
    if (tid < KT && ntiles > 0) s_vrow[0][tid] = vrow(k0 + tid);
    if (tid >= KT && tid < 2 * KT && ntiles > 1) s_vrow[1][tid - KT] = vrow(k0 + tid);
    for (int i = tid; i < kProbeRows * BW; i += 512) (&s_bits[0][0])[i] = 0u;
    for (int g = tid; g <= gk; g += 512) s_ko[g] = ko[g];
    __syncthreads();
    // the first tile's loads go out before the routing bits are set up; K rows past the
    // split are masked below and rows past the head read as zeros
    if (ntiles > 0) {
        TL::issue_rows_one(rk, k0, s_k[0], w, lane);
        TL::issue_one(rv, s_vrow[0], s_v[0], w, lane);
    }
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
        const int qrow = pvalid ? probe_orig[(size_t)h * probes + p] : 0;   // token order
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
        if (t + 1 < ntiles) {
            TL::issue_rows_one(rk, base + KT, s_k[buf ^ 1], w, lane);
            TL::issue_one(rv, s_vrow[buf ^ 1], s_v[buf ^ 1], w, lane);
        }
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
            // two chains of three-input maxima (15 v_max3 + 1 v_max for the 32 logits)
            float ma = fmaxf(sv[0][0], sv[1][0]), mb = fmaxf(sv[0][1], sv[1][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) {
                ma = fmaxf(fmaxf(ma, sv[0][r]), sv[1][r]);
                mb = fmaxf(fmaxf(mb, sv[0][r + 1]), sv[1][r + 1]);
            }
            const float mx = pair_max(fmaxf(ma, mb)) * scale_log2;
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
        // V rows of tile t + 2 into the row buffer that tile t's loads have finished with
        if (t + 2 < ntiles && tid < KT) s_vrow[buf][tid] = vrow(base + 2 * KT + tid);
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

void launch_probe(const bf16_t* qp, const bf16_t* kp, const bf16_t* vtok, const int32_t* kperm,
                  int heads, int n, int d,
                  const int32_t* probe_orig, const int32_t* probe_grp, int probes,
                  const int32_t* koff, int koff_stride, int gk, const int32_t* blocks, int gq,
                  int kblk, int splits, float* part_ml, float* part_od, float* part_os,
                  hipStream_t st) {
    if (probes == 0) return;
    int chunk = (n + splits - 1) / splits;
    chunk = (chunk + KT - 1) / KT * KT;
    const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    dim3 grid((probes + kProbeRows - 1) / kProbeRows, splits, heads);
    if (d == 128)
        hipLaunchKernelGGL(k_probe<128>, grid, dim3(512), 0, st, qp, kp, vtok, kperm, n, probe_orig, probe_grp,
                           probes, koff, koff_stride, gk, blocks, gq, kblk, chunk, scale_log2,
                           part_ml, part_od, part_os);
    else
        hipLaunchKernelGGL(k_probe<64>, grid, dim3(512), 0, st, qp, kp, vtok, kperm, n, probe_orig, probe_grp,
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
