// Partition-stage kernels: response-coupled partition of "Partition the Support,
// Reconstruct the Residual" (gist.science summary), section 2A.
//
//  * metric      M_K = Q_s^T Q_s / M_s over Weyl-sampled queries (fp64 sums of exact
//                bf16 products)
//  * metric spaces: keys use L = W (the scaled leading eigenvectors of M_K), queries
//                L with L L^T = C_K^T C_K / d (their logit-profile metric)
//  * assign      nearest centroid screened on MFMA with a certified margin; uncertified
//                points are queued and resolved in fp64 by `recheck` (lowest index on ties)
//  * counting sort (histogram, scan, stable scatter) and fp64 group means: the
//                centroid update and, after the last round, the group-major permutation
#include "kernels.h"

#include <cmath>

namespace spr {

// ------------------------------------------------------------------ generic ---
__global__ void k_to_bf16(const float* __restrict__ in, bf16_t* __restrict__ out, size_t count) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        out[i] = f32_to_bf16(in[i]);
}

template <typename T>
__global__ void k_fill(T* p, T value, size_t count) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < count;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = value;
}

static int grid_for(size_t count, int block) {
    size_t g = (count + block - 1) / block;
    if (g > 65535 * 4) g = 65535 * 4;
    if (g < 1) g = 1;
    return static_cast<int>(g);
}

void launch_to_bf16(const float* in, bf16_t* out, size_t count, hipStream_t st) {
    hipLaunchKernelGGL(k_to_bf16, dim3(grid_for(count, 256)), dim3(256), 0, st, in, out, count);
}
void launch_fill_i32(int32_t* p, int32_t value, size_t count, hipStream_t st) {
    hipLaunchKernelGGL(k_fill<int32_t>, dim3(grid_for(count, 256)), dim3(256), 0, st, p, value, count);
}
void launch_fill_i64(int64_t* p, int64_t value, size_t count, hipStream_t st) {
    hipLaunchKernelGGL(k_fill<int64_t>, dim3(grid_for(count, 256)), dim3(256), 0, st, p, value, count);
}

// ------------------------------------------------------------------- metric ---
// grid (d, H), block d: thread j of block i sums q[s][i] q[s][j] over the sample.
__global__ void k_metric(const bf16_t* __restrict__ q, int n, int d, int ms, int64_t a,
                         double* __restrict__ mk) {
    const int h = blockIdx.y, i = blockIdx.x, j = threadIdx.x;
    const bf16_t* qh = q + (size_t)h * n * d;
    double s = 0.0;
    for (int t = 0; t < ms; ++t) {
        const int64_t idx = ((int64_t)t * a) % n;
        const bf16_t* row = qh + idx * d;
        s += (double)bf16_to_f32(row[i]) * (double)bf16_to_f32(row[j]);
    }
    mk[((size_t)h * d + i) * d + j] = s / ms;
}

void launch_metric(const bf16_t* q, int heads, int n, int d, int n_sample, int64_t a, double* mk,
                   hipStream_t st) {
    hipLaunchKernelGGL(k_metric, dim3(d, heads), dim3(d), 0, st, q, n, d, n_sample, a, mk);
}

// --------------------------------------------------------- centroid finish ---
// For a raw-space centroid mean m (fp64, in LDS), with the metric factor L [d][D]:
//   projected centroid   c = m L          (fp64, used by the fp64 recheck)
//   screening vector     C' = L c^T       (d-dim; x . C' = (x L) . c for any point x)
//   split of C' into bf16 hi + lo parts   (the MFMA operand; |C' - hi - lo| <= 2^-17 |C'|)
//   |c|^2 (fp32, nearest) and |C'| (fp32, rounded up) for the screening score and bound
// The block needs blockDim >= max(d, D).
__device__ void finish_centroid(const double* __restrict__ mean, double* __restrict__ cp_lds,
                                const double* __restrict__ lh, int d, int dout, int groups,
                                int h, int g, double* __restrict__ c64, bf16_t* __restrict__ cpart,
                                float* __restrict__ cn2, float* __restrict__ cpn,
                                double* __restrict__ red) {
    const int tid = threadIdx.x;
    double cv = 0.0;
    if (tid < dout) {
        for (int i = 0; i < d; ++i) cv += mean[i] * lh[(size_t)i * dout + tid];
        cp_lds[tid] = cv;
        c64[((size_t)h * groups + g) * dout + tid] = cv;
    }
    __syncthreads();
    double sv = 0.0;
    if (tid < d) {
        for (int j = 0; j < dout; ++j) sv += lh[(size_t)tid * dout + j] * cp_lds[j];
        const float hi = bf16_to_f32(f32_to_bf16((float)sv));
        const bf16_t lo = f32_to_bf16((float)(sv - (double)hi));
        cpart[((size_t)(h * 2 + 0) * groups + g) * d + tid] = f32_to_bf16((float)sv);
        cpart[((size_t)(h * 2 + 1) * groups + g) * d + tid] = lo;
    }
    // norms: thread-strided partial sums, fixed-order reduction by thread 0
    red[tid] = (tid < dout) ? cv * cv : 0.0;
    red[blockDim.x + tid] = (tid < d) ? sv * sv : 0.0;
    __syncthreads();
    if (tid == 0) {
        double a = 0.0, b = 0.0;
        for (int i = 0; i < (int)blockDim.x; ++i) {
            a += red[i];
            b += red[blockDim.x + i];
        }
        cn2[(size_t)h * groups + g] = (float)a;                      // nearest: enters the score
        cpn[(size_t)h * groups + g] = (float)(sqrt(b) * (1.0 + 1e-6));  // rounded up: bound only
    }
}

// ------------------------------------------------------------------- seeds ---
// Seed centroid g is the point at Weyl index (g a) mod n.
__global__ __launch_bounds__(128) void k_seed(const bf16_t* __restrict__ x, int n, int d,
                                              const double* __restrict__ l64, int dout, int groups,
                                              int64_t a, double* __restrict__ c64,
                                              bf16_t* __restrict__ cpart, float* __restrict__ cn2,
                                              float* __restrict__ cpn) {
    __shared__ double mean[128];
    __shared__ double cp[128];
    __shared__ double red[256];
    const int h = blockIdx.y, g = blockIdx.x, j = threadIdx.x;
    const int64_t idx = ((int64_t)g * a) % n;
    const bf16_t* row = x + ((size_t)h * n + idx) * d;
    if (j < d) mean[j] = (double)bf16_to_f32(row[j]);
    __syncthreads();
    finish_centroid(mean, cp, l64 + (size_t)h * d * dout, d, dout, groups, h, g, c64, cpart, cn2,
                    cpn, red);
}

void launch_seed_centroids(const bf16_t* x, int heads, int n, int d, const double* l64, int dout,
                           int groups, int64_t a, double* c64, bf16_t* cpart, float* cn2,
                           float* cpn, hipStream_t st) {
    hipLaunchKernelGGL(k_seed, dim3(groups, heads), dim3(128), 0, st, x, n, d, l64, dout, groups, a,
                       c64, cpart, cn2, cpn);
}

// ------------------------------------------------------------------ assign ---
// Nearest centroid in the metric space, screened on MFMA. With y = x L the point's
// coordinates, |y - c_g|^2 = |y|^2 + s_g with s_g = |c_g|^2 - 2 x . C'_g; |y|^2 is the
// same for every g, so the argmin of s_g is the label. x . C'_g runs as a bf16 GEMM of
// the raw rows (exact bf16) against the hi/lo split of C' with fp32 accumulation:
//   |computed - exact| <= kappa |x| |C'_g|,  kappa = 2 d u (1 + 2^-8) + 2^-17  (u = 2^-24)
// and the score s~_g = fl(|c_g|^2 - 2 S~_g) is within
//   eps_g = 1.1 [2 kappa |x| |C'_g| + u |c_g|^2 + u |s~_g|]
// of the exact s_g. The label is certified when every other centroid's lower end
// s~_g - eps_g exceeds the best's upper end s~_best + eps_best; otherwise the point is
// queued for the fp64 recheck (which also settles exact ties by the lowest index).
//
// Block = 4 waves x 64 points; centroids stream through LDS in tiles of 64 (hi and lo
// parts), 16-byte chunk c of centroid row r stored at c ^ swz(r).
template <int D>
__global__ __launch_bounds__(256) void k_assign(const bf16_t* __restrict__ x, int n,
                                                const bf16_t* __restrict__ cpart,
                                                const float* __restrict__ cn2,
                                                const float* __restrict__ cpn, int groups,
                                                int32_t* __restrict__ labels,
                                                int32_t* __restrict__ flag_count,
                                                int32_t* __restrict__ flag_list) {
    constexpr int CH = D / 8;
    constexpr int TG = 64;
    constexpr float kU = 5.9604644775390625e-08f;
    constexpr float kappa = 2.f * D * kU * 1.00390625f + 7.62939453125e-06f;
    __shared__ uint4 s_c[2][TG * CH];
    __shared__ float s_cn2[kMaxGroups];
    __shared__ float s_cpn[kMaxGroups];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5;
    for (int g = tid; g < groups; g += 256) {
        s_cn2[g] = cn2[(size_t)h * groups + g];
        s_cpn[g] = cpn[(size_t)h * groups + g];
    }
    const int p_base = blockIdx.x * 256 + w * 64;
    uint4 xf[2][D / 16];
    float kx[2];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
        const int pt = p_base + 32 * pb + (lane & 31);
        const bool valid = pt < n;
        float ss = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            const uint4 v = valid ? *reinterpret_cast<const uint4*>(x + ((size_t)h * n + pt) * D +
                                                                  16 * kk + 8 * half)
                                  : make_uint4(0, 0, 0, 0);
            xf[pb][kk] = v;
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = bf16_to_f32((bf16_t)(wd[e] & 0xFFFF));
                const float hi = bf16_to_f32((bf16_t)(wd[e] >> 16));
                ss = fmaf(lo, lo, fmaf(hi, hi, ss));
            }
        }
        ss += __shfl_xor(ss, 32, 64);
        kx[pb] = 1.1f * 2.f * kappa * sqrtf(ss) * 1.000001f;
    }
    constexpr float ku = 1.1f * kU;
    float best[2] = {INFINITY, INFINITY}, eb[2] = {0.f, 0.f}, low2[2] = {INFINITY, INFINITY};
    int bg[2] = {0x7fffffff, 0x7fffffff};
    for (int g0 = 0; g0 < groups; g0 += TG) {
        __syncthreads();
        for (int i = tid; i < 2 * TG * CH; i += 256) {
            const int part = i / (TG * CH), rem = i % (TG * CH);
            const int row = rem / CH, c = rem % CH;
            const int g = g0 + row;
            s_c[part][row * CH + (c ^ swz<CH>(row))] =
                (g < groups) ? *reinterpret_cast<const uint4*>(
                                   cpart + ((size_t)(h * 2 + part) * groups + g) * D + c * 8)
                             : make_uint4(0, 0, 0, 0);
        }
        __syncthreads();
#pragma unroll
        for (int sub = 0; sub < TG / 32; ++sub) {
            const int gb = g0 + 32 * sub;
            if (gb >= groups) break;
            f32x16 acc[2] = {};
#pragma unroll
            for (int part = 0; part < 2; ++part)
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    const uint4 a =
                        s_c[part][(32 * sub + (lane & 31)) * CH + ((2 * kk + half) ^ swz<CH>(lane & 31))];
                    acc[0] = mfma32x32x16(a, xf[0][kk], acc[0]);
                    acc[1] = mfma32x32x16(a, xf[1][kk], acc[1]);
                }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int g = gb + 8 * (r >> 2) + 4 * half + (r & 3);
                if (g < groups) {
                    const float c2 = s_cn2[g], cp = s_cpn[g];
#pragma unroll
                    for (int pb = 0; pb < 2; ++pb) {
                        const float v = fmaf(-2.f, acc[pb][r], c2);
                        const float e = fmaf(kx[pb], cp, ku * (c2 + fabsf(v))) + 1e-30f;
                        if (v < best[pb]) {
                            low2[pb] = fminf(low2[pb], best[pb] - eb[pb]);
                            best[pb] = v;
                            eb[pb] = e;
                            bg[pb] = g;
                        } else {
                            low2[pb] = fminf(low2[pb], v - e);
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
        // merge the two lane halves: best by (value, index); the other best joins low2
        const float ob = __shfl_xor(best[pb], 32, 64);
        const float oe = __shfl_xor(eb[pb], 32, 64);
        const float ol = __shfl_xor(low2[pb], 32, 64);
        const int og = __shfl_xor(bg[pb], 32, 64);
        float b = best[pb], e = eb[pb], l2 = fminf(low2[pb], ol);
        int gsel = bg[pb];
        if (ob < b || (ob == b && og < gsel)) {
            l2 = fminf(l2, b - e);
            b = ob;
            e = oe;
            gsel = og;
        } else {
            l2 = fminf(l2, ob - oe);
        }
        const int pt = p_base + 32 * pb + lane;
        if (lane < 32 && pt < n) {
            labels[(size_t)h * n + pt] = gsel;
            if (groups > 1 && !(l2 > b + e)) {
                const int slot = atomicAdd(&flag_count[h], 1);
                flag_list[(size_t)h * n + slot] = pt;
            }
        }
    }
}

void launch_assign(const bf16_t* x, int heads, int n, int d, const bf16_t* cpart, const float* cn2,
                   const float* cpn, int groups, int32_t* labels, int32_t* flag_count,
                   int32_t* flag_list, hipStream_t st) {
    dim3 grid((n + 255) / 256, heads);
    if (d == 128)
        hipLaunchKernelGGL(k_assign<128>, grid, dim3(256), 0, st, x, n, cpart, cn2, cpn, groups,
                           labels, flag_count, flag_list);
    else
        hipLaunchKernelGGL(k_assign<64>, grid, dim3(256), 0, st, x, n, cpart, cn2, cpn, groups,
                           labels, flag_count, flag_list);
}

// ----------------------------------------------------------------- recheck ---
// One wave per queued point: exact-input fp64 coordinates y = x L64, fp64 distances
// to every fp64 centroid, argmin with the lowest index on ties.
__global__ __launch_bounds__(64) void k_recheck(const bf16_t* __restrict__ x, int n, int d,
                                                const double* __restrict__ l64, int dim,
                                                const double* __restrict__ c64, int groups,
                                                const int32_t* __restrict__ flag_count,
                                                const int32_t* __restrict__ flag_list,
                                                int32_t* __restrict__ labels) {
    __shared__ double xs[128];
    __shared__ double ys[128];
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int count = flag_count[h];
    const double* lh = l64 + (size_t)h * d * dim;
    const double* ch = c64 + (size_t)h * groups * dim;
    for (int idx = blockIdx.x; idx < count; idx += gridDim.x) {
        const int p = flag_list[(size_t)h * n + idx];
        const bf16_t* row = x + ((size_t)h * n + p) * d;
        for (int i = lane; i < d; i += 64) xs[i] = (double)bf16_to_f32(row[i]);
        __syncthreads();
        for (int j = lane; j < dim; j += 64) {
            double s = 0.0;
            for (int i = 0; i < d; ++i) s += xs[i] * lh[(size_t)i * dim + j];
            ys[j] = s;
        }
        __syncthreads();
        double best = INFINITY;
        int bg = 0x7fffffff;
        for (int g = lane; g < groups; g += 64) {
            const double* c = ch + (size_t)g * dim;
            double dist = 0.0;
            for (int j = 0; j < dim; ++j) {
                const double t = ys[j] - c[j];
                dist += t * t;
            }
            if (dist < best) { best = dist; bg = g; }
        }
        for (int o = 32; o > 0; o >>= 1) {
            const double ob = __shfl_xor(best, o, 64);
            const int og = __shfl_xor(bg, o, 64);
            if (ob < best || (ob == best && og < bg)) { best = ob; bg = og; }
        }
        if (lane == 0) labels[(size_t)h * n + p] = bg;
        __syncthreads();
    }
}

void launch_recheck(const bf16_t* x, int heads, int n, int d, const double* l64, int dim,
                    const double* c64, int groups, const int32_t* flag_count,
                    const int32_t* flag_list, int32_t* labels, hipStream_t st) {
    int blocks = (n + 63) / 64;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(k_recheck, dim3(blocks, heads), dim3(64), 0, st, x, n, d, l64, dim, c64,
                       groups, flag_count, flag_list, labels);
}

// ---------------------------------------------------------- counting sort ---
__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ labels, int n, int groups,
                                              int32_t* __restrict__ blkhist) {
    __shared__ int hist[kMaxGroups];
    const int h = blockIdx.y, b = blockIdx.x, tid = threadIdx.x;
    for (int g = tid; g < groups; g += 256) hist[g] = 0;
    __syncthreads();
    const int base = b * kSortChunk;
    for (int i = tid; i < kSortChunk; i += 256) {
        const int p = base + i;
        if (p < n) atomicAdd(&hist[labels[(size_t)h * n + p]], 1);
    }
    __syncthreads();
    int32_t* out = blkhist + ((size_t)h * gridDim.x + b) * groups;
    for (int g = tid; g < groups; g += 256) out[g] = hist[g];
}

// per head: group totals, exclusive scan over groups, then per-block bases in block order
__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ blkhist, int nblk,
                                               int groups, int n, int32_t* __restrict__ blkoff,
                                               int32_t* __restrict__ off) {
    __shared__ int tot[kMaxGroups];
    const int h = blockIdx.x, g = threadIdx.x;
    const int32_t* hh = blkhist + (size_t)h * nblk * groups;
    if (g < groups) {
        int s = 0;
        for (int b = 0; b < nblk; ++b) s += hh[(size_t)b * groups + g];
        tot[g] = s;
    }
    __syncthreads();
    if (g == 0) {
        int run = 0;
        for (int i = 0; i < groups; ++i) {
            const int c = tot[i];
            tot[i] = run;
            run += c;
        }
    }
    __syncthreads();
    if (g < groups) {
        int run = tot[g];
        off[(size_t)h * (groups + 1) + g] = run;
        int32_t* bo = blkoff + (size_t)h * nblk * groups;
        for (int b = 0; b < nblk; ++b) {
            bo[(size_t)b * groups + g] = run;
            run += hh[(size_t)b * groups + g];
        }
    }
    if (g == 0) off[(size_t)h * (groups + 1) + groups] = n;
}

// Stable scatter: the rank of a point among equal labels follows the point order.
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ labels, int n,
                                                 int groups, const int32_t* __restrict__ blkoff,
                                                 int32_t* __restrict__ sorted) {
    __shared__ int cnt[kMaxGroups];
    const int h = blockIdx.y, b = blockIdx.x, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    for (int g = tid; g < groups; g += 256) cnt[g] = 0;
    __syncthreads();
    const int32_t* bo = blkoff + ((size_t)h * gridDim.x + b) * groups;
    for (int round = 0; round < kSortChunk / 256; ++round) {
        const int p = b * kSortChunk + round * 256 + tid;
        const bool valid = p < n;
        const int lab = valid ? labels[(size_t)h * n + p] : -1;
        // peers: lanes of this wave holding the same label
        uint64_t peers = 0;
        uint64_t todo = __ballot(valid);
        while (todo) {
            const int leader = __ffsll((unsigned long long)todo) - 1;
            const int l = __shfl(lab, leader, 64);
            const uint64_t m = __ballot(valid && lab == l);
            if (valid && lab == l) peers = m;
            todo &= ~m;
        }
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        const int prefix = __popcll(peers & below);
        const int total = __popcll(peers);
        for (int w = 0; w < 4; ++w) {
            int basev = 0;
            if (wave == w && valid) basev = cnt[lab];
            __syncthreads();
            if (wave == w && valid) {
                if (prefix == 0) cnt[lab] = basev + total;
                sorted[(size_t)h * n + bo[lab] + basev + prefix] = p;
            }
            __syncthreads();
        }
    }
}

void launch_counting_sort(const int32_t* labels, int heads, int n, int groups, int32_t* blkhist,
                          int32_t* blkoff, int32_t* sorted, int32_t* off, hipStream_t st) {
    const int nblk = (n + kSortChunk - 1) / kSortChunk;
    hipLaunchKernelGGL(k_hist, dim3(nblk, heads), dim3(256), 0, st, labels, n, groups, blkhist);
    hipLaunchKernelGGL(k_scan, dim3(heads), dim3(1024), 0, st, blkhist, nblk, groups, n, blkoff, off);
    hipLaunchKernelGGL(k_scatter, dim3(nblk, heads), dim3(256), 0, st, labels, n, groups, blkoff,
                       sorted);
}

// -------------------------------------------------------------- group means ---
// Block per (group, head): fp64 sum of the members' raw rows in sorted order (fixed
// split over row lanes, fixed-order reduction), mean = sum / count (zero if empty).
// With l64 given, a non-empty group also gets its projected centroid, screening vector
// and norms (an empty group keeps its previous centroid).
__global__ __launch_bounds__(256) void k_group_means(
    const bf16_t* __restrict__ x, int n, int d, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ off, int groups, double* __restrict__ mean_raw,
    const double* __restrict__ l64, int dout, double* __restrict__ c64,
    bf16_t* __restrict__ cpart, float* __restrict__ cn2, float* __restrict__ cpn) {
    __shared__ double red[256 * 8];
    __shared__ double mean[128];
    __shared__ double cp[128];
    const int h = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
    const int chunks = d / 8;
    const int lanes = 256 / chunks;
    const int c = tid % chunks, rl = tid / chunks;
    const int32_t* oh = off + (size_t)h * (groups + 1);
    const int beg = oh[g], end = oh[g + 1];
    const int cnt = end - beg;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    const int32_t* sh = sorted + (size_t)h * n;
    const bf16_t* xh = x + (size_t)h * n * d;
    for (int m = beg + rl; m < end; m += lanes) {
        const uint4 v = *reinterpret_cast<const uint4*>(xh + (size_t)sh[m] * d + c * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)bf16_to_f32((bf16_t)(w[e] & 0xFFFF));
            acc[2 * e + 1] += (double)bf16_to_f32((bf16_t)(w[e] >> 16));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[(size_t)rl * d + c * 8 + e] = acc[e];
    __syncthreads();
    if (tid < d) {
        double s = 0.0;
        for (int r = 0; r < lanes; ++r) s += red[(size_t)r * d + tid];
        const double mv = (cnt > 0) ? s / cnt : 0.0;
        mean[tid] = mv;
        mean_raw[((size_t)h * groups + g) * d + tid] = mv;
    }
    __syncthreads();
    if (l64 == nullptr || cnt == 0) return;           // empty: keep the previous centroid
    finish_centroid(mean, cp, l64 + (size_t)h * d * dout, d, dout, groups, h, g, c64, cpart, cn2,
                    cpn, red);
}

void launch_group_means(const bf16_t* x, int heads, int n, int d, const int32_t* sorted,
                        const int32_t* off, int groups, double* mean_raw, const double* l64,
                        int dout, double* c64, bf16_t* cpart, float* cn2, float* cpn,
                        hipStream_t st) {
    hipLaunchKernelGGL(k_group_means, dim3(groups, heads), dim3(256), 0, st, x, n, d, sorted, off,
                       groups, mean_raw, l64, dout, c64, cpart, cn2, cpn);
}

}  // namespace spr
