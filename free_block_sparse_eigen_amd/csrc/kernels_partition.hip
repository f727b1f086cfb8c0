// Partition-stage kernels: response-coupled partition of "Partition the Support,
// Reconstruct the Residual" (gist.science summary), section 2A.
//
//  * metric      M_K = Q_s^T Q_s / M_s over Weyl-sampled queries (fp64 sums of exact
//                bf16 products)
//  * project     Y = X L in fp32 (keys: L = W, the scaled leading eigenvectors of M_K;
//                queries: L L^T = C_K^T C_K / d), plus a per-row forward error bound
//  * assign      nearest centroid in fp32 with a certified margin; uncertified points
//                are queued and resolved in fp64 by `recheck` (lowest index on ties)
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

// ------------------------------------------------------------------ project ---
// y[h][r][0..dout) = x[h][r][:] . L[h] (fp32, i ascending), for 64 rows per block.
// yerr[h][r] bounds |y_fp32 - y_exact|_2 by (d + 4) u |x_r| |L|_F (u = 2^-24), which
// covers the fp32 rounding of L and the length-d fp32 dot products.
constexpr int kProjRows = 64;

__global__ __launch_bounds__(256) void k_project(const bf16_t* __restrict__ x, int n, int d,
                                                 const float* __restrict__ l32, int dout,
                                                 const float* __restrict__ lfro,
                                                 float* __restrict__ y, float* __restrict__ yerr) {
    __shared__ float smem[128 * 128 + kProjRows * 128];
    float* ls = smem;                                  // [d][dout]
    float* xs = smem + d * dout;                       // [64][d]
    const int h = blockIdx.y;
    const int r0 = blockIdx.x * kProjRows;
    const int tid = threadIdx.x;
    const float* lh = l32 + (size_t)h * d * dout;
    for (int i = tid; i < d * dout; i += 256) ls[i] = lh[i];
    const bf16_t* xh = x + (size_t)h * n * d;
    for (int i = tid; i < kProjRows * d; i += 256) {
        const int r = r0 + i / d;
        xs[i] = (r < n) ? bf16_to_f32(xh[(size_t)r * d + (i % d)]) : 0.f;
    }
    __syncthreads();
    const int r = tid >> 2, part = tid & 3;
    float acc[32];
#pragma unroll
    for (int m = 0; m < 32; ++m) acc[m] = 0.f;
    const float* xr = xs + r * d;
    for (int i = 0; i < d; ++i) {
        const float xv = xr[i];
        const float* li = ls + i * dout;
#pragma unroll
        for (int m = 0; m < 32; ++m) {
            const int j = part + 4 * m;
            if (j < dout) acc[m] = fmaf(xv, li[j], acc[m]);
        }
    }
    const int row = r0 + r;
    if (row < n) {
        float* yr = y + ((size_t)h * n + row) * dout;
#pragma unroll
        for (int m = 0; m < 32; ++m) {
            const int j = part + 4 * m;
            if (j < dout) yr[j] = acc[m];
        }
        if (part == 0) {
            double s = 0.0;
            for (int i = 0; i < d; ++i) s += (double)xr[i] * xr[i];
            const double e = (d + 4) * 5.9604644775390625e-08 * sqrt(s) * (double)lfro[h];
            yerr[(size_t)h * n + row] = (float)(e * 1.0625);
        }
    }
}

void launch_project(const bf16_t* x, int heads, int n, int d, const float* l32, int dout,
                    const float* lfro, float* y, float* yerr, hipStream_t st) {
    hipLaunchKernelGGL(k_project, dim3((n + kProjRows - 1) / kProjRows, heads), dim3(256), 0, st,
                       x, n, d, l32, dout, lfro, y, yerr);
}

// ------------------------------------------------------------------- seeds ---
// c[h][g] = x[h][(g a) mod n] . L64[h] in fp64 (the seed point's exact coordinates).
__global__ void k_seed(const bf16_t* __restrict__ x, int n, int d, const double* __restrict__ l64,
                       int dout, int64_t a, double* __restrict__ c64, float* __restrict__ c32,
                       float* __restrict__ cnorm) {
    __shared__ double xs[128];
    __shared__ double red[128];
    const int h = blockIdx.y, g = blockIdx.x, j = threadIdx.x;
    const int64_t idx = ((int64_t)g * a) % n;
    const bf16_t* row = x + ((size_t)h * n + idx) * d;
    if (j < d) xs[j] = (double)bf16_to_f32(row[j]);
    __syncthreads();
    double s = 0.0;
    if (j < dout) {
        const double* lh = l64 + (size_t)h * d * dout;
        for (int i = 0; i < d; ++i) s += xs[i] * lh[(size_t)i * dout + j];
        c64[((size_t)h * gridDim.x + g) * dout + j] = s;
        c32[((size_t)h * gridDim.x + g) * dout + j] = (float)s;
    }
    const float f = (j < dout) ? (float)s : 0.f;
    red[j] = (double)f * f;
    __syncthreads();
    if (j == 0) {
        double t = 0.0;
        for (int i = 0; i < 128; ++i) t += red[i];
        cnorm[(size_t)h * gridDim.x + g] = (float)(sqrt(t) * 1.0000002);
    }
}

void launch_seed_centroids(const bf16_t* x, int heads, int n, int d, const double* l64, int dout,
                           int groups, int64_t a, double* c64, float* c32, float* cnorm,
                           hipStream_t st) {
    hipLaunchKernelGGL(k_seed, dim3(groups, heads), dim3(128), 0, st, x, n, d, l64, dout, a, c64,
                       c32, cnorm);
}

// ------------------------------------------------------------------ assign ---
// One point per thread; centroids staged through LDS in tiles. Distances are
// sum_j (y_j - c_j)^2 in fp32 (DP = padded dimension, zero-filled). The point is
// certified when the two smallest distances are separated by more than their
// error bounds (see eps below); otherwise it is queued for the fp64 recheck.
constexpr float kU32 = 5.9604644775390625e-08f;  // 2^-24

template <int DP>
__global__ __launch_bounds__(256) void k_assign(const float* __restrict__ y,
                                                const float* __restrict__ yerr, int n, int dim,
                                                const float* __restrict__ c32,
                                                const float* __restrict__ cnorm, int groups,
                                                int32_t* __restrict__ labels,
                                                int32_t* __restrict__ flag_count,
                                                int32_t* __restrict__ flag_list) {
    constexpr int kTileBytes = 32768;
    constexpr int GT = kTileBytes / (DP * 4);       // centroids per LDS tile
    __shared__ float4 cs[GT * DP / 4];
    __shared__ float red[256];
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int p = blockIdx.x * 256 + tid;
    const bool valid = p < n;
    // largest centroid norm of this head (bound term)
    float cm = 0.f;
    for (int g = tid; g < groups; g += 256) cm = fmaxf(cm, cnorm[(size_t)h * groups + g]);
    red[tid] = cm;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
        __syncthreads();
    }
    const float cmax = red[0];
    float yv[DP];
    const float* yp = y + ((size_t)h * n + (valid ? p : 0)) * dim;
#pragma unroll
    for (int j = 0; j < DP; ++j) yv[j] = (valid && j < dim) ? yp[j] : 0.f;
    float best = INFINITY, second = INFINITY;
    int bg = 0;
    const float* ch = c32 + (size_t)h * groups * dim;
    for (int g0 = 0; g0 < groups; g0 += GT) {
        const int gt = min(GT, groups - g0);
        __syncthreads();
        float* csf = reinterpret_cast<float*>(cs);
        for (int i = tid; i < GT * DP; i += 256) {
            const int g = i / DP, j = i % DP;
            csf[i] = (g < gt && j < dim) ? ch[(size_t)(g0 + g) * dim + j] : 0.f;
        }
        __syncthreads();
        for (int g = 0; g < gt; ++g) {
            float dist = 0.f;
#pragma unroll
            for (int j4 = 0; j4 < DP / 4; ++j4) {
                const float4 c = cs[g * (DP / 4) + j4];
                const float d0 = yv[4 * j4 + 0] - c.x, d1 = yv[4 * j4 + 1] - c.y;
                const float d2 = yv[4 * j4 + 2] - c.z, d3 = yv[4 * j4 + 3] - c.w;
                dist = fmaf(d0, d0, dist);
                dist = fmaf(d1, d1, dist);
                dist = fmaf(d2, d2, dist);
                dist = fmaf(d3, d3, dist);
            }
            if (dist < best) {
                second = best;
                best = dist;
                bg = g0 + g;
            } else if (dist < second) {
                second = dist;
            }
        }
    }
    if (!valid) return;
    labels[(size_t)h * n + p] = bg;
    // |computed - exact| <= eps(x) for a computed distance x:
    //   F = E + u |c|max + 2u sqrt(x) bounds |a_computed - a_exact|_2 (a = y - c),
    //   eps = 1.1 [ (dim + 2) u x + F (2 sqrt(x) + F) ].
    // x - eps(x) is increasing once x >= 4 F^2, so checking the runner-up suffices.
    bool certified = false;
    if (groups == 1) {
        certified = true;
    } else if (isfinite(second)) {
        const float e = yerr[(size_t)h * n + p];
        auto eps = [&](float x, float& fx) {
            const float sx = sqrtf(x);
            fx = e + kU32 * cmax + 2.f * kU32 * sx;
            return 1.1f * ((dim + 2) * kU32 * x + fx * (2.f * sx + fx)) + 1e-30f;
        };
        float f1, f2;
        const float e1 = eps(best, f1), e2 = eps(second, f2);
        certified = (second - e2 > best + e1) && (second >= 4.f * f2 * f2);
    }
    if (!certified) {
        const int slot = atomicAdd(&flag_count[h], 1);
        flag_list[(size_t)h * n + slot] = p;
    }
}

void launch_assign(const float* y, const float* yerr, int heads, int n, int dim, const float* c32,
                   const float* cnorm, int groups, int32_t* labels, int32_t* flag_count,
                   int32_t* flag_list, hipStream_t st) {
    dim3 grid((n + 255) / 256, heads);
    if (dim <= 32)
        hipLaunchKernelGGL(k_assign<32>, grid, dim3(256), 0, st, y, yerr, n, dim, c32, cnorm, groups,
                           labels, flag_count, flag_list);
    else if (dim <= 64)
        hipLaunchKernelGGL(k_assign<64>, grid, dim3(256), 0, st, y, yerr, n, dim, c32, cnorm, groups,
                           labels, flag_count, flag_list);
    else
        hipLaunchKernelGGL(k_assign<128>, grid, dim3(256), 0, st, y, yerr, n, dim, c32, cnorm,
                           groups, labels, flag_count, flag_list);
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
// With l64 given, a non-empty group also gets its projected centroid c = mean . L64.
__global__ __launch_bounds__(256) void k_group_means(
    const bf16_t* __restrict__ x, int n, int d, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ off, int groups, double* __restrict__ mean_raw,
    const double* __restrict__ l64, int dout, double* __restrict__ c64, float* __restrict__ c32,
    float* __restrict__ cnorm) {
    __shared__ double red[256 * 8];
    __shared__ double mean[128];
    __shared__ double nrm[128];
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
    double cv = 0.0;
    if (tid < dout) {
        const double* lh = l64 + (size_t)h * d * dout;
        for (int i = 0; i < d; ++i) cv += mean[i] * lh[(size_t)i * dout + tid];
        c64[((size_t)h * groups + g) * dout + tid] = cv;
        c32[((size_t)h * groups + g) * dout + tid] = (float)cv;
    }
    if (tid < 128) {
        const float f = (tid < dout) ? (float)cv : 0.f;
        nrm[tid] = (double)f * f;
    }
    __syncthreads();
    if (tid == 0) {
        double t = 0.0;
        for (int i = 0; i < 128; ++i) t += nrm[i];
        cnorm[(size_t)h * groups + g] = (float)(sqrt(t) * 1.0000002);
    }
}

void launch_group_means(const bf16_t* x, int heads, int n, int d, const int32_t* sorted,
                        const int32_t* off, int groups, double* mean_raw, const double* l64,
                        int dout, double* c64, float* c32, float* cnorm, hipStream_t st) {
    hipLaunchKernelGGL(k_group_means, dim3(groups, heads), dim3(256), 0, st, x, n, d, sorted, off,
                       groups, mean_raw, l64, dout, c64, c32, cnorm);
}

}  // namespace spr
