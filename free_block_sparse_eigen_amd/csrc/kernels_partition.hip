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

#include <algorithm>
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

// Non-finite values of x (bf16 or fp32, `count` elements) added to *counter.
template <typename T>
__global__ __launch_bounds__(256) void k_count_nonfinite(const T* __restrict__ x, size_t count,
                                                         unsigned long long* __restrict__ counter) {
    unsigned c = 0;
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < count; i += (size_t)gridDim.x * 256) {
        if constexpr (sizeof(T) == 2) c += ((x[i] & 0x7F80u) == 0x7F80u) ? 1u : 0u;
        else c += ((__float_as_uint(x[i]) & 0x7F800000u) == 0x7F800000u) ? 1u : 0u;
    }
    c = wave_sum(c);
    if ((threadIdx.x & 63) == 0 && c) atomicAdd(counter, (unsigned long long)c);
}

void launch_count_nonfinite(const void* x, size_t count, int is_f32, unsigned long long* counter,
                            hipStream_t st) {
    const int grid = std::min(grid_for(count, 256), 2048);
    if (is_f32)
        hipLaunchKernelGGL(k_count_nonfinite<float>, dim3(grid), dim3(256), 0, st,
                           static_cast<const float*>(x), count, counter);
    else
        hipLaunchKernelGGL(k_count_nonfinite<bf16_t>, dim3(grid), dim3(256), 0, st,
                           static_cast<const bf16_t*>(x), count, counter);
}

// ------------------------------------------------------------------- metric ---
// grid (d, H), block d: thread j of block i sums q[s][i] q[s][j] over the sample.
__global__ void k_metric(const bf16_t* __restrict__ q, int n, int d, int ms, int64_t a,
                         double* __restrict__ mk) {
    const int h = blockIdx.y, i = blockIdx.x, j = threadIdx.x;
    const bf16_t* qh = q + (size_t)h * n * d;
    double s = 0.0;
    int64_t idx = 0;                           // (t a) mod n, stepped (0 <= a < n)
    const int64_t am = a % n;
#pragma unroll 8
    for (int t = 0; t < ms; ++t) {
        const bf16_t* row = qh + idx * d;
        s += (double)bf16_to_f32(row[i]) * (double)bf16_to_f32(row[j]);
        idx += am;
        if (idx >= n) idx -= n;
    }
    mk[((size_t)h * d + i) * d + j] = s / ms;
}

void launch_metric(const bf16_t* q, int heads, int n, int d, int n_sample, int64_t a, double* mk,
                   hipStream_t st) {
    hipLaunchKernelGGL(k_metric, dim3(d, heads), dim3(d), 0, st, q, n, d, n_sample, a, mk);
}

// --------------------------------------------------------- centroid finish ---
// For raw-space centroid means m (fp64), with the metric given either as a factor
// L [d][D] (metric L L^T) or, with dout == 0, as the full metric M [d][d]:
//   factor:  projected centroid c = m L (fp64, used by the fp64 recheck; stored
//            coordinate-major, [dim][G], so that the recheck's reads coalesce),
//            screening vector C' = L c^T (d-dim; x . C' = (x L) . c for any point x)
//   metric:  screening vector C' = M m (its fp64 copy, coordinate-major, is what the
//            recheck uses) and
//            |c|^2 = m . C' (also kept in fp64)
//   split of C' into bf16 hi + lo parts   (the MFMA operand; |C' - hi - lo| <= 2^-17 |C'|)
//   |c|^2 (fp32, nearest) and |C'| (fp32, rounded up) for the screening score and bound
// Block = 16 centroids of one head. A thread owns one output coordinate for all 16 of
// them (each element of L it reads from L2 serves 16 accumulators, 16 loads in flight at
// a time) over a contiguous range of the summed index; the ranges' partial sums are added
// in range order. The work is latency-bound: a thread's sum has at most 64 terms. With
// `off` given, empty groups are skipped (they keep their previous centroid).
constexpr int kFinG = 16;

// fixed-order sum of v over the 64 lanes (butterfly; identical on every lane)
__device__ inline double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__global__ __launch_bounds__(256) void k_finish(const double* __restrict__ mean_raw, int d,
                                                const double* __restrict__ l64, int dout, int groups,
                                                const int32_t* __restrict__ off,
                                                double* __restrict__ c64, bf16_t* __restrict__ cpart,
                                                float* __restrict__ cn2, float* __restrict__ cpn,
                                                double* __restrict__ c2_64, double* __restrict__ crow,
                                                int coords) {
    constexpr int G = kFinG;
    const bool full = dout == 0;                 // full metric M [d][d]
    __shared__ double s_m[G][129];               // means (padded rows)
    __shared__ double s_c[G][129];               // projected centroids
    __shared__ double s_s[G][129];               // screening vectors
    __shared__ double s_part[256 * G];           // partial sums [range][g][coordinate]
    const int h = blockIdx.y, g0 = blockIdx.x * G, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    if (full) dout = d;
    const double* lh = l64 + (size_t)h * d * dout;
    for (int o = tid; o < G * d; o += 256) {
        const int gs = o / d, i = o % d, g = g0 + gs;
        s_m[gs][i] = (g < groups) ? mean_raw[((size_t)h * groups + g) * d + i] : 0.0;
    }
    __syncthreads();
    // c[gs][j] = sum_i m[gs][i] L[i][j]: thread (range r, coordinate j) sums i over its
    // range for all G centroids (lanes along j: coalesced rows of L); with the full metric
    // this is C' = M m itself (M is symmetric)
    {
        const int nr = 256 / dout;                       // dout divides 256 (d and r_K are)
        const int j = tid % dout, r = tid / dout;
        const int len = (d + nr - 1) / nr, i0 = min(r * len, d), i1 = min(i0 + len, d);
        double acc[G];
#pragma unroll
        for (int gs = 0; gs < G; ++gs) acc[gs] = 0.0;
        if (r < nr) {
            int i = i0;
            for (; i + 16 <= i1; i += 16) {
                double lv[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) lv[u] = lh[(size_t)(i + u) * dout + j];
#pragma unroll
                for (int u = 0; u < 16; ++u)
#pragma unroll
                    for (int gs = 0; gs < G; ++gs) acc[gs] += s_m[gs][i + u] * lv[u];
            }
            for (; i < i1; ++i) {
                const double l = lh[(size_t)i * dout + j];
#pragma unroll
                for (int gs = 0; gs < G; ++gs) acc[gs] += s_m[gs][i] * l;
            }
#pragma unroll
            for (int gs = 0; gs < G; ++gs) s_part[(r * G + gs) * dout + j] = acc[gs];
        }
        __syncthreads();
        for (int o = tid; o < G * dout; o += 256) {
            const int gs = o / dout, jj = o % dout;
            double c = 0.0;
            for (int rr = 0; rr < nr; ++rr) c += s_part[(rr * G + gs) * dout + jj];
            s_c[gs][jj] = c;
        }
        __syncthreads();
    }
    // C'[gs][i] = sum_j L[i][j] c[gs][j]: thread (range r, coordinate i) over its j range
    // (not needed when the assignment screens in the coordinates themselves)
    if (!full && !coords) {
        const int nr = 256 / d;                          // d = 64 or 128
        const int i = tid % d, r = tid / d;
        const int len = (dout + nr - 1) / nr, j0 = min(r * len, dout), j1 = min(j0 + len, dout);
        double acc[G];
#pragma unroll
        for (int gs = 0; gs < G; ++gs) acc[gs] = 0.0;
        if (r < nr) {
            int j = j0;
            for (; j + 16 <= j1; j += 16) {
                double lv[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) lv[u] = lh[(size_t)i * dout + j + u];
#pragma unroll
                for (int u = 0; u < 16; ++u)
#pragma unroll
                    for (int gs = 0; gs < G; ++gs) acc[gs] += lv[u] * s_c[gs][j + u];
            }
            for (; j < j1; ++j) {
                const double l = lh[(size_t)i * dout + j];
#pragma unroll
                for (int gs = 0; gs < G; ++gs) acc[gs] += l * s_c[gs][j];
            }
#pragma unroll
            for (int gs = 0; gs < G; ++gs) s_part[(r * G + gs) * d + i] = acc[gs];
        }
        __syncthreads();
        for (int o = tid; o < G * d; o += 256) {
            const int gs = o / d, ii = o % d;
            double c = 0.0;
            for (int rr = 0; rr < nr; ++rr) c += s_part[(rr * G + gs) * d + ii];
            s_s[gs][ii] = c;
        }
        __syncthreads();
    }
    // one wave per centroid: stores and norms
    for (int gs = w; gs < G; gs += 4) {
        const int g = g0 + gs;
        if (g >= groups) break;
        if (off != nullptr && off[(size_t)h * (groups + 1) + g + 1] == off[(size_t)h * (groups + 1) + g])
            continue;                                   // empty: keep the previous centroid
        double a = 0.0, b = 0.0;
        for (int j = lane; j < dout; j += 64) {
            const double cv = s_c[gs][j];
            c64[((size_t)h * dout + j) * groups + g] = cv;          // coordinate-major
            if (crow && !full) crow[((size_t)h * groups + g) * dout + j] = cv;   // row-major copy
            a += full ? s_m[gs][j] * cv : cv * cv;
            if (coords) {           // screened in the key coordinates: c itself, split
                const bf16_t hi = f32_to_bf16((float)cv);
                cpart[((size_t)(h * 2 + 0) * groups + g) * dout + j] = hi;
                cpart[((size_t)(h * 2 + 1) * groups + g) * dout + j] = f32_to_bf16((float)(cv - (double)bf16_to_f32(hi)));
                b += cv * cv;
            }
        }
        for (int i = coords ? d : lane; i < d; i += 64) {
            const double sv = full ? s_c[gs][i] : s_s[gs][i];
            if (crow && full) crow[((size_t)h * groups + g) * d + i] = sv;       // row-major copy
            const bf16_t hi = f32_to_bf16((float)sv);
            cpart[((size_t)(h * 2 + 0) * groups + g) * d + i] = hi;
            cpart[((size_t)(h * 2 + 1) * groups + g) * d + i] = f32_to_bf16((float)(sv - (double)bf16_to_f32(hi)));
            b += sv * sv;
        }
        a = wave_sum_f64(a);
        b = wave_sum_f64(b);
        if (lane == 0) {
            cn2[(size_t)h * groups + g] = (float)a;                          // nearest: enters the score
            cpn[(size_t)h * groups + g] = (float)(sqrt(b) * (1.0 + 1e-6));   // rounded up: bound only
            c2_64[(size_t)h * groups + g] = a;
        }
    }
}

static void launch_finish(const double* mean_raw, int heads, int d, const double* l64, int dout,
                          int groups, const int32_t* off, double* c64, bf16_t* cpart, float* cn2,
                          float* cpn, double* c2_64, hipStream_t st, double* crow, int coords = 0) {
    hipLaunchKernelGGL(k_finish, dim3((groups + kFinG - 1) / kFinG, heads), dim3(256), 0, st, mean_raw,
                       d, l64, dout, groups, off, c64, cpart, cn2, cpn, c2_64, crow, coords);
}

// ------------------------------------------------------------------- seeds ---
// Seed centroid g is the point at Weyl index (g a) mod n (written as the raw mean).
__global__ __launch_bounds__(128) void k_seed(const bf16_t* __restrict__ x, int n, int d, int groups,
                                              int64_t a, double* __restrict__ mean_raw) {
    const int h = blockIdx.y, g = blockIdx.x, j = threadIdx.x;
    const int64_t idx = ((int64_t)g * a) % n;
    if (j < d) mean_raw[((size_t)h * groups + g) * d + j] = (double)bf16_to_f32(x[((size_t)h * n + idx) * d + j]);
}

void launch_seed_raw(const bf16_t* x, int heads, int n, int d, int groups, int64_t a, double* mean_raw,
                     hipStream_t st) {
    hipLaunchKernelGGL(k_seed, dim3(groups, heads), dim3(128), 0, st, x, n, d, groups, a, mean_raw);
}

void launch_finish_all(const double* mean_raw, int heads, int d, const double* l64, int dout, int groups,
                       double* c64, bf16_t* cpart, float* cn2, float* cpn, double* c2_64, hipStream_t st,
                       double* crow) {
    launch_finish(mean_raw, heads, d, l64, dout, groups, nullptr, c64, cpart, cn2, cpn, c2_64, st, crow);
}

void launch_seed_centroids(const bf16_t* x, int heads, int n, int d, const double* l64, int dout,
                           int groups, int64_t a, double* mean_raw, double* c64, bf16_t* cpart,
                           float* cn2, float* cpn, double* c2_64, hipStream_t st,
                           double* crow, int coords) {
    hipLaunchKernelGGL(k_seed, dim3(groups, heads), dim3(128), 0, st, x, n, d, groups, a, mean_raw);
    launch_finish(mean_raw, heads, d, l64, dout, groups, nullptr, c64, cpart, cn2, cpn, c2_64, st, crow, coords);
}

// ------------------------------------------------------------------ assign ---
// Nearest centroid in the metric space, screened on MFMA. With y = x L the point's
// coordinates, |y - c_g|^2 = |y|^2 + s_g with s_g = |c_g|^2 - 2 x . C'_g; |y|^2 is the
// same for every g, so the argmin of s_g is the label. x . C'_g runs as a bf16 GEMM of
// the raw rows (exact bf16) against the hi/lo split of C' with fp32 accumulation:
//   |computed - exact| <= kappa |x| |C'_g|,  kappa = 2 d u (1 + 2^-8) + 2^-17  (u = 2^-24)
// and the score s~_g = fl(|c_g|^2 - 2 S~_g) is within
//   e_g = 1.1 [2 kappa |x| |C'_g| + u |c_g|^2 + u |s~_g|] <= 1.1 [A + u |s~_g|],
//   A = 2 kappa |x| max_g |C'_g| + u max_g |c_g|^2
// of the exact s_g. Since s - 1.1 u |s| grows with s, every other centroid's lower end
// is at least that of the runner-up, so the label is certified when
//   s~_2nd - s~_best > 2.2 A + 1.1 u (|s~_2nd| + |s~_best|)
// (checked with a further margin for the fp32 evaluation of the test itself);
// otherwise the point is queued for the fp64 recheck, which also settles exact ties by
// the lowest index. Each lane tracks only the best and runner-up scores.
//
// The scores are compared with the accumulator slot (0..15) of their centroid written
// into their four low mantissa bits, so one min tracks value and slot together. That
// moves each score by at most 15 ulp <= 2^-19 |s~|, and the test above gets a further
// 2^-18 (|s~_2nd| + |s~_best|) for the two compared scores.
//
// Centroid tiles of 64 (hi and lo parts, 16-byte chunk c of centroid row r at c ^ swz(r))
// sit in LDS; a wave scores 64 points (two MFMA column blocks of 32) against them. Two
// kernels share the per-wave steps: k_assign_res keeps every centroid of a head resident
// in LDS (2 G D 2 bytes <= 128 KB) and lets each wave walk its points with no barriers;
// k_assign (larger G) streams the tiles, double-buffered. Padding centroids score
// kPadScore, a finite value no real score reaches (finite, so the slot bits can be
// written into it).
constexpr int kAssignTG = 64;
constexpr int kAssignResBytes = 128 * 1024;
constexpr int kMaxCand = kMaxCandidates;          // candidate centroids listed per queued point
constexpr int kCandMaxDim = kCandidateMaxDim;     // largest factor width the candidate recheck takes
constexpr float kPadScore = 3.0e38f;

// a score with accumulator slot r (0..15) in its four low mantissa bits
__device__ __attribute__((always_inline)) inline float with_slot(float v, int r) {
    return __uint_as_float((__float_as_uint(v) & ~15u) | (uint32_t)r);
}

// Z: the points are the key coordinates z = x W (depth D = r_K, written by k_zcoords),
// split into bf16 hi + lo like the centroids, and a score takes all four products (hi.hi,
// hi.lo, lo.hi, lo.lo). The bound's per-point coefficient k_p (|computed - exact| <= k_p |c|
// for the dot product) then comes with the coordinates instead of kappa |x|.
template <int D, bool Z = false>
struct AssignWave {
    static constexpr int CH = D / 8;
    static constexpr int TG = kAssignTG;
    static constexpr int SLOTS = 2 * TG * CH;   // 16-byte slots per tile (hi and lo)
    static constexpr float kU = 5.9604644775390625e-08f;
    static constexpr float kappa = 2.f * D * kU * 1.00390625f + 7.62939453125e-06f;
    // tile layout in LDS: rows of 128 or 256 bytes hold chunk c of row r at c ^ swz(r) within
    // the row; narrower rows (CH <= 4, the key coordinates) are stored chunk-major instead
    // (chunk c of row r at c TG + r), since 32 rows of 64 bytes read by 32 lanes would share
    // bank groups whatever the order within a row
    static constexpr bool CM = CH <= 4;
    __host__ __device__ static int sw(int r) { return CM ? 0 : swz<CH>(r); }
    // 16-byte slot (within one part's TG CH slots) of row r's chunk c
    __host__ __device__ static int slot_of(int r, int c) { return CM ? c * TG + r : r * CH + (c ^ sw(r)); }

    uint4 xf[2][D / 16];                        // the points (Z: their hi parts)
    uint4 xl[Z ? 2 : 1][Z ? D / 16 : 1];        // Z: their lo parts
    float xk[2];                                // kappa |x| (Z: k_p), rounded up
    float best[2], second[2];
    int bg[2];

    // this wave's 64 points as MFMA B fragments (an invalid point reads the last point
    // and is zeroed), then their norms
    __device__ __attribute__((always_inline)) void load(const bf16_t* __restrict__ x, int n,
                                                        int h, int p_base, int lane) {
        const int half = lane >> 5;
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            const int pt = min(p_base + 32 * pb + (lane & 31), n - 1);
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                xf[pb][kk] = *reinterpret_cast<const uint4*>(x + ((size_t)h * n + pt) * D + 16 * kk + 8 * half);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            const bool valid = p_base + 32 * pb + (lane & 31) < n;
            float ss = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                if (!valid) xf[pb][kk] = make_uint4(0, 0, 0, 0);
                const uint4 v = xf[pb][kk];
                const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf16_to_f32((bf16_t)(wd[e] & 0xFFFF));
                    const float hi = bf16_to_f32((bf16_t)(wd[e] >> 16));
                    ss = fmaf(lo, lo, fmaf(hi, hi, ss));
                }
            }
            ss += __shfl_xor(ss, 32, 64);
            xk[pb] = kappa * (sqrtf(ss) * 1.000001f);
            best[pb] = INFINITY;
            second[pb] = INFINITY;
            bg[pb] = 0x7fffffff;
        }
    }

    // Z: this wave's 64 points from their split coordinates (row of a point: D hi values
    // then D lo values) and their bound coefficients kb [n]
    __device__ __attribute__((always_inline)) void load_z(const bf16_t* __restrict__ zhl,
                                                          const float* __restrict__ kb, int n,
                                                          int h, int p_base, int lane) {
        const int half = lane >> 5;
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            const int pt = min(p_base + 32 * pb + (lane & 31), n - 1);
            const bf16_t* zr = zhl + ((size_t)h * n + pt) * 2 * D;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                xf[pb][kk] = *reinterpret_cast<const uint4*>(zr + 16 * kk + 8 * half);
                xl[pb][kk] = *reinterpret_cast<const uint4*>(zr + D + 16 * kk + 8 * half);
            }
            xk[pb] = kb[(size_t)h * n + pt];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            if (p_base + 32 * pb + (lane & 31) >= n) {
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    xf[pb][kk] = make_uint4(0, 0, 0, 0);
                    xl[pb][kk] = make_uint4(0, 0, 0, 0);
                }
            }
            best[pb] = INFINITY;
            second[pb] = INFINITY;
            bg[pb] = 0x7fffffff;
        }
    }

    // as load, for the queued points q_base .. q_base + 63 of the head's queue fl (count
    // entries; a lane past the end reads the last queued point and is zeroed)
    __device__ __attribute__((always_inline)) void load_queued(const bf16_t* __restrict__ x, int n, int h,
                                                               const int32_t* __restrict__ fl, int q_base,
                                                               int count, int lane) {
        const int half = lane >> 5;
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            const int pt = fl[min(q_base + 32 * pb + (lane & 31), count - 1)];
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
                xf[pb][kk] = *reinterpret_cast<const uint4*>(x + ((size_t)h * n + pt) * D + 16 * kk + 8 * half);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            const bool valid = q_base + 32 * pb + (lane & 31) < count;
            float ss = 0.f;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                if (!valid) xf[pb][kk] = make_uint4(0, 0, 0, 0);
                const uint4 v = xf[pb][kk];
                const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf16_to_f32((bf16_t)(wd[e] & 0xFFFF));
                    const float hi = bf16_to_f32((bf16_t)(wd[e] >> 16));
                    ss = fmaf(lo, lo, fmaf(hi, hi, ss));
                }
            }
            ss += __shfl_xor(ss, 32, 64);
            xk[pb] = kappa * (sqrtf(ss) * 1.000001f);
            best[pb] = INFINITY;
            second[pb] = INFINITY;
            bg[pb] = 0x7fffffff;
        }
    }

    // Z: as load_z, for the queued points q_base .. q_base + 63 of the head's queue fl (count
    // entries; a lane past the end reads the last queued point and is zeroed)
    __device__ __attribute__((always_inline)) void load_queued_z(const bf16_t* __restrict__ zhl,
                                                                 const float* __restrict__ kb, int n, int h,
                                                                 const int32_t* __restrict__ fl, int q_base,
                                                                 int count, int lane) {
        const int half = lane >> 5;
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            const int pt = fl[min(q_base + 32 * pb + (lane & 31), count - 1)];
            const bf16_t* zr = zhl + ((size_t)h * n + pt) * 2 * D;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk) {
                xf[pb][kk] = *reinterpret_cast<const uint4*>(zr + 16 * kk + 8 * half);
                xl[pb][kk] = *reinterpret_cast<const uint4*>(zr + D + 16 * kk + 8 * half);
            }
            xk[pb] = kb[(size_t)h * n + pt];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            if (q_base + 32 * pb + (lane & 31) >= count) {
#pragma unroll
                for (int kk = 0; kk < D / 16; ++kk) {
                    xf[pb][kk] = make_uint4(0, 0, 0, 0);
                    xl[pb][kk] = make_uint4(0, 0, 0, 0);
                }
            }
            best[pb] = INFINITY;
            second[pb] = INFINITY;
            bg[pb] = 0x7fffffff;
        }
    }

    // After the scores: the window [.., thr] of screened scores that can hold the exact
    // argmin. A centroid whose screened score s passes the certification test against the
    // best b (s - b > the test's margin at (s, b)) is certifiably worse than the best, so
    // only s <= b + W (1 + c) can win, with W the margin at s2 = b and c its coefficient of
    // |s2|, which covers the larger |s|; thr = b + 1.25 W keeps a wide safety factor
    // (both halves of the wave get the same value).
    __device__ __attribute__((always_inline)) float window(int pb, float c2max, float cpmax) const {
        const float b = fminf(best[pb], __shfl_xor(best[pb], 32, 64));
        const float A = fmaf(2.f * xk[pb], cpmax, kU * c2max);
        const float W = 2.4f * A + (2.4f * kU + 3.814697265625e-06f) * (2.f * fabsf(b)) + 1e-30f;
        return b + 1.25f * W;
    }

    // scores against centroid tile t held at buf: the products of both 32-centroid
    // sub-tiles run together (four independent accumulator chains), each sub-tile's
    // sums in the same order (hi then lo over the depth); then the scores in sub-tile
    // order
    __device__ __attribute__((always_inline)) void tile(int t, const uint4* buf, int groups,
                                                        const float* s_cn2, int lane) {
        const int half = lane >> 5;
        tile_with(t, buf, groups, lane, [&](const f32x16 (&acc)[2], int gb) __attribute__((always_inline)) {
            scores(acc, gb, s_cn2, half);
        });
    }

    // the products of tile t, then epi(acc, gb) for each 32-centroid sub-tile holding groups
    template <typename EPI>
    __device__ __attribute__((always_inline)) void tile_with(int t, const uint4* buf, int groups,
                                                             int lane, EPI&& epi) {
        const int half = lane >> 5;
        constexpr int KS = D / 16, PF = 2;
        const uint4* cr0 = buf + (CM ? (lane & 31) : (lane & 31) * CH);
        const uint4* cr1 = buf + (CM ? 32 + (lane & 31) : (32 + (lane & 31)) * CH);
        const int sw0 = sw(lane & 31), sw1 = sw(32 + (lane & 31));
        auto frag = [&](const uint4* cr, int swr, int i) __attribute__((always_inline)) {
            const int c = 2 * (i % KS) + half;
            return cr[(i / KS) * TG * CH + (CM ? c * TG : (c ^ swr))];
        };
        f32x16 acc[2][2];
        if constexpr (Z) {
            // each depth step: both sub-tiles' hi and lo fragments against the points' hi and
            // lo parts, the four products of each accumulator in the same order every step
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const uint4 a[2][2] = {{frag(cr0, sw0, kk), frag(cr0, sw0, KS + kk)},
                                       {frag(cr1, sw1, kk), frag(cr1, sw1, KS + kk)}};
#pragma unroll
                for (int pr = 0; pr < 4; ++pr)
#pragma unroll
                    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                        for (int pb = 0; pb < 2; ++pb) {
                            const uint4 b = (pr & 1) ? xl[pb][kk] : xf[pb][kk];
                            acc[sub][pb] = mfma32x32x16(a[sub][pr >> 1], b,
                                                        (kk == 0 && pr == 0) ? f32x16{} : acc[sub][pb]);
                        }
            }
#pragma unroll
            for (int sub = 0; sub < TG / 32; ++sub) {
                const int gb = t * TG + 32 * sub;
                if (gb >= groups) break;
                epi(acc[sub], gb);
            }
            return;
        }
        uint4 f0[PF], f1[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            f0[i] = frag(cr0, sw0, i);
            f1[i] = frag(cr1, sw1, i);
        }
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) {
            const uint4 a0 = f0[i % PF], a1 = f1[i % PF];
            if (i + PF < 2 * KS) {
                f0[i % PF] = frag(cr0, sw0, i + PF);
                f1[i % PF] = frag(cr1, sw1, i + PF);
            }
            if (i == 0) {
                acc[0][0] = mfma32x32x16(a0, xf[0][0], f32x16{});
                acc[0][1] = mfma32x32x16(a0, xf[1][0], f32x16{});
                acc[1][0] = mfma32x32x16(a1, xf[0][0], f32x16{});
                acc[1][1] = mfma32x32x16(a1, xf[1][0], f32x16{});
            } else {
                acc[0][0] = mfma32x32x16(a0, xf[0][i % KS], acc[0][0]);
                acc[0][1] = mfma32x32x16(a0, xf[1][i % KS], acc[0][1]);
                acc[1][0] = mfma32x32x16(a1, xf[0][i % KS], acc[1][0]);
                acc[1][1] = mfma32x32x16(a1, xf[1][i % KS], acc[1][1]);
            }
            __builtin_amdgcn_sched_barrier(0);     // keep the reads PF steps ahead
        }
#pragma unroll
        for (int sub = 0; sub < TG / 32; ++sub) {
            const int gb = t * TG + 32 * sub;
            if (gb >= groups) break;
            epi(acc[sub], gb);
        }
    }

    // one 32-centroid sub-tile's scores (column blocks pb = 0, 1) into best / runner-up:
    // with best <= second, the new runner-up is the median of (best, v, second); the
    // slot-marked best changes only when this sub-tile holds a new best, whose slot then
    // gives its centroid index
    __device__ __attribute__((always_inline)) void scores(const f32x16 (&acc)[2], int gb,
                                                          const float* s_cn2, int half) {
        const float b0[2] = {best[0], best[1]};
        // med3 with -inf is the min; an fminf would first quiet its slot-marked operand
        // (one more instruction per score), so -inf comes from an opaque scalar move
        uint32_t ninf_bits;
        asm("s_mov_b32 %0, 0xff800000" : "=s"(ninf_bits));
        const float ninf = __uint_as_float(ninf_bits);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float c2 = s_cn2[gb + 8 * (r >> 2) + 4 * half + (r & 3)];
#pragma unroll
            for (int pb = 0; pb < 2; ++pb) {
                const float v = with_slot(fmaf(-2.f, acc[pb][r], c2), r);
                second[pb] = __builtin_amdgcn_fmed3f(best[pb], v, second[pb]);
                best[pb] = __builtin_amdgcn_fmed3f(best[pb], v, ninf);     // the min
            }
        }
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            const int r = (int)(__float_as_uint(best[pb]) & 15u);
            if (best[pb] != b0[pb]) bg[pb] = gb + 8 * (r >> 2) + 4 * half + (r & 3);
        }
    }

    // labels, and the points whose label is not certified appended to the recheck queue
    __device__ __attribute__((always_inline)) void finish(int n, int h, int groups, int p_base,
                                                          int lane, float c2max, float cpmax,
                                                          int32_t* __restrict__ labels,
                                                          int32_t* __restrict__ flag_count,
                                                          int32_t* __restrict__ flag_list) {
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
            // merge the two lane halves: best by (value, index); the other best joins second
            const float ob = __shfl_xor(best[pb], 32, 64);
            const float os = __shfl_xor(second[pb], 32, 64);
            const int og = __shfl_xor(bg[pb], 32, 64);
            float b = best[pb];
            int gsel = bg[pb];
            const float s2 = fminf(fminf(second[pb], os), fmaxf(b, ob));
            if (ob < b || (ob == b && og < gsel)) {
                b = ob;
                gsel = og;
            }
            const float A = fmaf(2.f * xk[pb], cpmax, kU * c2max);
            const float bound = 2.4f * A + (2.4f * kU + 3.814697265625e-06f) * (fabsf(s2) + fabsf(b)) + 1e-30f;
            const int pt = p_base + 32 * pb + lane;
            if (lane < 32 && pt < n) {
                // a padding centroid (only if no real score is finite) is never certified
                const bool real = gsel < groups;
                labels[(size_t)h * n + pt] = real ? gsel : 0;
                if (!(s2 - b > bound) || !real) {
                    const int slot = atomicAdd(&flag_count[h], 1);
                    flag_list[(size_t)h * n + slot] = pt;
                }
            }
        }
    }
};

// |c|^2 of every centroid tile slot into s_cn2 (+inf past the last group), and the head's
// max |c|^2 and max |C'| for the bound; every thread of the block must call this.
template <int NT>
__device__ inline void assign_norms(const float* __restrict__ cn2, const float* __restrict__ cpn,
                                    int h, int groups, int ntiles, float* s_cn2, float* s_red,
                                    float& c2max, float& cpmax) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int NW = NT / 64;
    float c2m = 0.f, cpm = 0.f;
    for (int g = tid; g < ntiles * kAssignTG; g += NT) {
        float c2 = kPadScore;
        if (g < groups) {
            c2 = cn2[(size_t)h * groups + g];
            c2m = fmaxf(c2m, c2);
            cpm = fmaxf(cpm, cpn[(size_t)h * groups + g]);
        }
        s_cn2[g] = c2;
    }
    c2m = wave_max(c2m);
    cpm = wave_max(cpm);
    if (lane == 0) {
        s_red[w] = c2m;
        s_red[NW + w] = cpm;
    }
    __syncthreads();
    c2max = s_red[0];
    cpmax = s_red[NW];
    for (int k = 1; k < NW; ++k) {
        c2max = fmaxf(c2max, s_red[k]);
        cpmax = fmaxf(cpmax, s_red[NW + k]);
    }
}

// Block = 8 waves over a contiguous range of 64-point items in head-major order (equal
// ranges per block, one block per CU); where the range enters a new head the block loads
// that head's centroids (all tiles) into LDS once, then its waves take the head's items
// round-robin.
template <int D, bool Z>
__global__ __launch_bounds__(512, 1) void k_assign_res(const bf16_t* __restrict__ x, int n,
                                                       int heads, const bf16_t* __restrict__ cpart,
                                                       const float* __restrict__ cn2,
                                                       const float* __restrict__ cpn, int groups,
                                                       int items_per_block,
                                                       int32_t* __restrict__ labels,
                                                       int32_t* __restrict__ flag_count,
                                                       int32_t* __restrict__ flag_list,
                                                       const float* __restrict__ kb) {
    using AW = AssignWave<D, Z>;
    constexpr int CH = AW::CH, TG = kAssignTG, SLOTS = AW::SLOTS;
    __shared__ uint4 s_c[kAssignResBytes / 16];
    __shared__ float s_cn2[kAssignResBytes / (4 * D) + TG];
    __shared__ float s_red[16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ntiles = (groups + TG - 1) / TG;
    const int ipw = (n + 63) / 64;                 // items per head
    const int total = heads * ipw;
    int it = blockIdx.x * items_per_block;
    const int end = min(total, it + items_per_block);
    AW aw;
    while (it < end) {
        const int h = it / ipw;
        const int seg_end = min(end, (h + 1) * ipw);
        __syncthreads();                           // the previous head's tiles are done
        const rsrc_t rc = make_rsrc(cpart + (size_t)h * 2 * groups * D, (uint32_t)(2 * groups * D * 2));
        for (int slot = tid; slot < ntiles * SLOTS; slot += 512) {
            // lanes of a wave take consecutive slots, so each load lands at LDS base + 16 lane
            const int t = slot / SLOTS, rem0 = slot % SLOTS;
            const int part = rem0 / (TG * CH), rem = rem0 % (TG * CH);
            // the row and chunk whose 16 bytes this slot holds (AW::slot_of inverted)
            const int row = AW::CM ? rem % TG : rem / CH;
            const int ch = AW::CM ? rem / TG : (rem % CH) ^ AW::sw(row);
            const int g = min(t * TG + row, groups - 1);
            lds_load16(rc, s_c + (slot - lane), ((part * groups + g) * D + ch * 8) * 2);
        }
        float c2max, cpmax;
        assign_norms<512>(cn2, cpn, h, groups, ntiles, s_cn2, s_red, c2max, cpmax);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int k = it + w; k < seg_end; k += 8) {
            const int p_base = (k - h * ipw) * 64;
            if constexpr (Z) aw.load_z(x, kb, n, h, p_base, lane);
            else aw.load(x, n, h, p_base, lane);
            for (int t = 0; t < ntiles; ++t) aw.tile(t, s_c + t * SLOTS, groups, s_cn2, lane);
            aw.finish(n, h, groups, p_base, lane, c2max, cpmax, labels, flag_count, flag_list);
        }
        it = seg_end;
    }
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_assign(const bf16_t* __restrict__ x, int n,
                                                   const bf16_t* __restrict__ cpart,
                                                   const float* __restrict__ cn2,
                                                   const float* __restrict__ cpn, int groups,
                                                   int32_t* __restrict__ labels,
                                                   int32_t* __restrict__ flag_count,
                                                   int32_t* __restrict__ flag_list) {
    using AW = AssignWave<D>;
    constexpr int CH = AW::CH, TG = kAssignTG, SLOTS = AW::SLOTS;
    constexpr int PER = SLOTS / 256;           // direct loads per thread per tile
    __shared__ uint4 s_c0[SLOTS];
    __shared__ uint4 s_c1[SLOTS];
    __shared__ float s_cn2[kMaxGroups + TG];
    __shared__ float s_red[8];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int ntiles = (groups + TG - 1) / TG;
    const rsrc_t rc = make_rsrc(cpart + (size_t)h * 2 * groups * D, (uint32_t)(2 * groups * D * 2));
    auto issue = [&](int t, uint4* buf) {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int first = (w * PER + m) * 64;
            const int slot = first + lane;
            const int part = slot / (TG * CH), rem = slot % (TG * CH);
            const int row = rem / CH, pc = rem % CH;
            const int g = min(t * TG + row, groups - 1);
            lds_load16(rc, buf + first, ((part * groups + g) * D + ((pc ^ AW::sw(row)) * 8)) * 2);
        }
    };
    issue(0, s_c0);
    const int p_base = blockIdx.x * 256 + w * 64;
    AW aw;
    aw.load(x, n, h, p_base, lane);
    float c2max, cpmax;
    assign_norms<256>(cn2, cpn, h, groups, ntiles, s_cn2, s_red, c2max, cpmax);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
        if (t + 1 < ntiles) issue(t + 1, s_c1);
        aw.tile(t, s_c0, groups, s_cn2, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 1 >= ntiles) break;
        if (t + 2 < ntiles) issue(t + 2, s_c0);
        aw.tile(t + 1, s_c1, groups, s_cn2, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    aw.finish(n, h, groups, p_base, lane, c2max, cpmax, labels, flag_count, flag_list);
}

// ------------------------------------------------------------- candidates ---
// For a long recheck queue (large G, the full metric): the queued points are screened again
// (same MFMA products and error bound as k_assign) in two passes over the centroid tiles,
// the first for each point's best score and window, the second listing the centroids whose
// screened score lies in the window; the exact argmin is among them, so the fp64 recheck
// (k_recheck_cand) needs only those. A point with more than kMaxCand goes to a second queue
// (ovf_list) for the full recheck. The lists take 32 KB of LDS beside the two 32 KB centroid
// tiles, so one block runs per CU.
// Z: the keys screened in their split coordinates (x = zhl, D = r_K, bound coefficients kb)
// against the centroids' split coordinates, with the same products and bound as the
// resident screen in the coordinates.
template <int D, bool Z = false>
__global__ __launch_bounds__(256, 1) void k_candidates(const bf16_t* __restrict__ x, int n,
                                                       const bf16_t* __restrict__ cpart,
                                                       const float* __restrict__ cn2,
                                                       const float* __restrict__ cpn, int groups,
                                                       const int32_t* __restrict__ flag_count,
                                                       const int32_t* __restrict__ flag_list,
                                                       int32_t* __restrict__ cand,
                                                       int32_t* __restrict__ ncand,
                                                       int32_t* __restrict__ ovf_count,
                                                       int32_t* __restrict__ ovf_list,
                                                       const float* __restrict__ kb) {
    using AW = AssignWave<D, Z>;
    constexpr int CH = AW::CH, TG = kAssignTG, SLOTS = AW::SLOTS;
    constexpr int PER = SLOTS / 256;
    static_assert(SLOTS % 256 == 0, "a tile must split evenly over the block");
    __shared__ uint4 s_c0[SLOTS];
    __shared__ uint4 s_c1[SLOTS];
    __shared__ float s_cn2[kMaxGroups + TG];
    __shared__ float s_red[8];
    __shared__ int s_nc[4][64];
    __shared__ int s_cd[4][64][kMaxCand];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int count = flag_count[h];
    if ((int)blockIdx.x * 256 >= count) return;       // the whole block: no queued point
    const int ntiles = (groups + TG - 1) / TG;
    const rsrc_t rc = make_rsrc(cpart + (size_t)h * 2 * groups * D, (uint32_t)(2 * groups * D * 2));
    auto issue = [&](int t, uint4* buf) {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int first = (w * PER + m) * 64;
            const int slot = first + lane;
            const int part = slot / (TG * CH), rem = slot % (TG * CH);
            // the row and chunk whose 16 bytes this slot holds (AW::slot_of inverted)
            const int row = AW::CM ? rem % TG : rem / CH;
            const int ch = AW::CM ? rem / TG : (rem % CH) ^ AW::sw(row);
            const int g = min(t * TG + row, groups - 1);
            lds_load16(rc, buf + first, ((part * groups + g) * D + ch * 8) * 2);
        }
    };
    const int q_base = blockIdx.x * 256 + w * 64;
    const int32_t* fl = flag_list + (size_t)h * n;
    s_nc[w][lane] = 0;
    issue(0, s_c0);
    AW aw;
    if constexpr (Z) aw.load_queued_z(x, kb, n, h, fl, q_base, count, lane);
    else aw.load_queued(x, n, h, fl, q_base, count, lane);
    float c2max, cpmax;
    assign_norms<256>(cn2, cpn, h, groups, ntiles, s_cn2, s_red, c2max, cpmax);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int half = lane >> 5;
    float thr[2] = {0.f, 0.f};
    // pass 0: best scores; pass 1: the window's centroids (tile 0 is reloaded between them)
    for (int pass = 0; pass < 2; ++pass) {
        auto run = [&](int t, const uint4* buf) {
            if (pass == 0) {
                aw.tile(t, buf, groups, s_cn2, lane);
            } else {
                aw.tile_with(t, buf, groups, lane, [&](const f32x16 (&acc)[2], int gb) __attribute__((always_inline)) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int g = gb + 8 * (r >> 2) + 4 * half + (r & 3);
                        const float c2 = s_cn2[g];
#pragma unroll
                        for (int pb = 0; pb < 2; ++pb) {
                            if (fmaf(-2.f, acc[pb][r], c2) <= thr[pb]) {
                                const int p = 32 * pb + (lane & 31);
                                const int slot = atomicAdd(&s_nc[w][p], 1);
                                if (slot < kMaxCand) s_cd[w][p][slot] = g;
                            }
                        }
                    }
                });
            }
        };
        for (int t = 0; t < ntiles; t += 2) {
            if (t + 1 < ntiles) issue(t + 1, s_c1);
            run(t, s_c0);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (t + 1 >= ntiles) break;
            if (t + 2 < ntiles) issue(t + 2, s_c0);
            run(t + 1, s_c1);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        if (pass == 0) {
#pragma unroll
            for (int pb = 0; pb < 2; ++pb) thr[pb] = aw.window(pb, c2max, cpmax);
            issue(0, s_c0);                           // every wave is past its last tile read
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }
    // the lists of this wave's points, by queue position
    const int qi = q_base + lane;
    if (qi < count) {
        const int nc = s_nc[w][lane];
        const bool listed = nc >= 1 && nc <= kMaxCand;
        ncand[(size_t)h * n + qi] = listed ? nc : -1;
        for (int c = 0; c < min(nc, kMaxCand); ++c) cand[((size_t)h * n + qi) * kMaxCand + c] = s_cd[w][lane][c];
        if (!listed) {                                // to the full recheck
            const int slot = atomicAdd(&ovf_count[h], 1);
            ovf_list[(size_t)h * n + slot] = fl[qi];
        }
    }
}

// The fp64 recheck of a queued point over its candidate list: the same products, in the
// same order, as k_recheck, so that both give the same distances. With the full metric
// (dim 0) |c|^2 - 2 x . C'; with a factor L [D][dim] the point's coordinates y = x L (the
// two halves of the depth summed separately, then added) and |y - c|^2. crow holds the
// screening vectors C' (full) or the centroid coordinates (factor) row by row, so each
// candidate is one contiguous row. The lowest index wins among equal distances.
template <int D>
__global__ __launch_bounds__(256) void k_recheck_cand(const bf16_t* __restrict__ x, int n,
                                                      const double* __restrict__ l64, int dim,
                                                      const double* __restrict__ crow,
                                                      const double* __restrict__ c2_64, int groups,
                                                      const int32_t* __restrict__ flag_count,
                                                      const int32_t* __restrict__ flag_list,
                                                      const int32_t* __restrict__ cand,
                                                      const int32_t* __restrict__ ncand,
                                                      const double* __restrict__ ycoord,
                                                      int32_t* __restrict__ labels) {
    const int h = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= flag_count[h]) return;
    const int nc = ncand[(size_t)h * n + i];
    if (nc < 0) return;                               // in the full recheck's queue
    const int p = flag_list[(size_t)h * n + i];
    const bf16_t* xr = x + ((size_t)h * n + p) * D;
    const bool full = dim == 0;
    const int cdim = full ? D : dim;
    const double* ch = crow + (size_t)h * groups * cdim;
    uint32_t xw[D / 2];                               // the point, two bf16 per word
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
        const uint4 u = *reinterpret_cast<const uint4*>(xr + 8 * c);
        xw[4 * c] = u.x;
        xw[4 * c + 1] = u.y;
        xw[4 * c + 2] = u.z;
        xw[4 * c + 3] = u.w;
    }
    auto xv = [&](int ii) __attribute__((always_inline)) {
        const uint32_t wd = xw[ii >> 1];
        return (double)bf16_to_f32((bf16_t)((ii & 1) ? (wd >> 16) : (wd & 0xFFFF)));
    };
    // the factor's coordinates y = x L: each half of the depth summed in order on its own,
    // then the two halves added (as k_recheck does)
    double y[kCandMaxDim];
    if (!full && ycoord) {                            // computed for every point beforehand
        const double* yr = ycoord + ((size_t)h * n + p) * dim;
#pragma unroll
        for (int jj = 0; jj < kCandMaxDim; ++jj) y[jj] = jj < dim ? yr[jj] : 0.0;
    } else if (!full) {
        const double* lh = l64 + (size_t)h * D * dim;
        double y1[kCandMaxDim];
#pragma unroll
        for (int jj = 0; jj < kCandMaxDim; ++jj) y[jj] = y1[jj] = 0.0;
#pragma unroll 2
        for (int ii = 0; ii < D / 2; ++ii) {
            const double xi = (double)bf16_to_f32(xr[ii]);
            const double* lr = lh + (size_t)ii * dim;
#pragma unroll
            for (int jj = 0; jj < kCandMaxDim; ++jj)
                if (jj < dim) y[jj] = fma(xi, lr[jj], y[jj]);
        }
#pragma unroll 2
        for (int ii = D / 2; ii < D; ++ii) {
            const double xi = (double)bf16_to_f32(xr[ii]);
            const double* lr = lh + (size_t)ii * dim;
#pragma unroll
            for (int jj = 0; jj < kCandMaxDim; ++jj)
                if (jj < dim) y1[jj] = fma(xi, lr[jj], y1[jj]);
        }
#pragma unroll
        for (int jj = 0; jj < kCandMaxDim; ++jj) y[jj] = y[jj] + y1[jj];
    }
    double best = INFINITY;
    int bg = 0x7fffffff;
    for (int c = 0; c < nc; ++c) {
        const int g = cand[((size_t)h * n + i) * kMaxCand + c];
        if (g >= groups) continue;
        const double* cg = ch + (size_t)g * cdim;
        double dist;
        if (full) {
            double acc = 0.0;
#pragma unroll
            for (int j0 = 0; j0 < D; j0 += 16) {      // loads 16 at a time, sums in order
                double cv[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) cv[u] = cg[j0 + u];
#pragma unroll
                for (int u = 0; u < 16; ++u) acc = fma(xv(j0 + u), cv[u], acc);
            }
            dist = fma(-2.0, acc, c2_64[(size_t)h * groups + g]);
        } else {
            double acc = 0.0;
#pragma unroll
            for (int jj = 0; jj < kCandMaxDim; ++jj) {
                if (jj < dim) {
                    const double t = y[jj] - cg[jj];
                    acc = fma(t, t, acc);
                }
            }
            dist = acc;
        }
        if (dist < best || (dist == best && g < bg)) {
            best = dist;
            bg = g;
        }
    }
    labels[(size_t)h * n + p] = bg < groups ? bg : 0;
}

void launch_candidates(const bf16_t* x, int heads, int n, int d, const bf16_t* cpart, const float* cn2,
                       const float* cpn, int groups, const int32_t* flag_count, const int32_t* flag_list,
                       int32_t* cand, int32_t* ncand, int32_t* ovf_count, int32_t* ovf_list, hipStream_t st,
                       const bf16_t* zhl, const float* kb, int dz) {
    launch_fill_i32(ovf_count, 0, heads, st);
    dim3 grid((n + 255) / 256, heads);
    if (zhl != nullptr && dz == 32)
        hipLaunchKernelGGL((k_candidates<32, true>), grid, dim3(256), 0, st, zhl, n, cpart, cn2, cpn, groups,
                           flag_count, flag_list, cand, ncand, ovf_count, ovf_list, kb);
    else if (zhl != nullptr)
        hipLaunchKernelGGL((k_candidates<16, true>), grid, dim3(256), 0, st, zhl, n, cpart, cn2, cpn, groups,
                           flag_count, flag_list, cand, ncand, ovf_count, ovf_list, kb);
    else if (d == 128)
        hipLaunchKernelGGL((k_candidates<128>), grid, dim3(256), 0, st, x, n, cpart, cn2, cpn, groups,
                           flag_count, flag_list, cand, ncand, ovf_count, ovf_list, nullptr);
    else
        hipLaunchKernelGGL((k_candidates<64>), grid, dim3(256), 0, st, x, n, cpart, cn2, cpn, groups,
                           flag_count, flag_list, cand, ncand, ovf_count, ovf_list, nullptr);
}

void launch_recheck_cand(const bf16_t* x, int heads, int n, int d, const double* l64, int dim,
                         const double* crow, const double* c2_64, int groups, const int32_t* flag_count,
                         const int32_t* flag_list, const int32_t* cand, const int32_t* ncand,
                         const double* ycoord, int32_t* labels, hipStream_t st) {
    const dim3 grid((n + 255) / 256, heads);
    if (d == 128)
        hipLaunchKernelGGL(k_recheck_cand<128>, grid, dim3(256), 0, st, x, n, l64, dim, crow, c2_64, groups,
                           flag_count, flag_list, cand, ncand, ycoord, labels);
    else
        hipLaunchKernelGGL(k_recheck_cand<64>, grid, dim3(256), 0, st, x, n, l64, dim, crow, c2_64, groups,
                           flag_count, flag_list, cand, ncand, ycoord, labels);
}

// Every point's coordinates y = x L [n][dim], each half of the depth summed in order, then
// the halves added: the values k_recheck forms for a queued point, once per call instead of
// once per queued point and round. A thread per point keeps its row in registers and reads
// the rows of L (staged in LDS, the same row for every lane) as it goes.
template <int D>
__global__ __launch_bounds__(256, 1) void k_coords(const bf16_t* __restrict__ x, int n,
                                                const double* __restrict__ l64, int dim,
                                                double* __restrict__ y) {
    constexpr int M = kCandMaxDim;
    __shared__ __attribute__((aligned(16))) double s_l[D * M];
    const int h = blockIdx.y, tid = threadIdx.x;
    const double* lh = l64 + (size_t)h * D * dim;
    for (int e = tid; e < D * M; e += 256) {
        const int ii = e / M, jj = e % M;
        s_l[e] = jj < dim ? lh[(size_t)ii * dim + jj] : 0.0;
    }
    __syncthreads();
    const int p = blockIdx.x * 256 + tid;
    if (p >= n) return;
    const bf16_t* xr = x + ((size_t)h * n + p) * D;
    double part[2][M];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int jj = 0; jj < M; ++jj) part[hf][jj] = 0.0;
        // eight depth entries (one 16-byte load of the row) at a time, in order
#pragma unroll 1
        for (int i0 = hf * (D / 2); i0 < (hf + 1) * (D / 2); i0 += 8) {
            const uint4 u = *reinterpret_cast<const uint4*>(xr + i0);
            const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double xi = (double)bf16_to_f32((bf16_t)((e & 1) ? (wd[e >> 1] >> 16) : (wd[e >> 1] & 0xFFFF)));
                const double2* lr = reinterpret_cast<const double2*>(s_l + (i0 + e) * M);
#pragma unroll
                for (int jj = 0; jj < M; jj += 2) {
                    const double2 l2 = lr[jj / 2];
                    part[hf][jj] = fma(xi, l2.x, part[hf][jj]);
                    part[hf][jj + 1] = fma(xi, l2.y, part[hf][jj + 1]);
                }
            }
        }
    }
    double* yr = y + ((size_t)h * n + p) * dim;
#pragma unroll
    for (int jj = 0; jj < M; ++jj)
        if (jj < dim) yr[jj] = part[0][jj] + part[1][jj];
}

void launch_coords(const bf16_t* x, int heads, int n, int d, const double* l64, int dim, double* y,
                   hipStream_t st) {
    const dim3 grid((unsigned)((n + 255) / 256), heads);
    if (d == 128)
        hipLaunchKernelGGL(k_coords<128>, grid, dim3(256), 0, st, x, n, l64, dim, y);
    else
        hipLaunchKernelGGL(k_coords<64>, grid, dim3(256), 0, st, x, n, l64, dim, y);
}

// v = p0 + p1 + p2 + r in bf16 parts, each the nearest to what is left (through fp32), with
// |r| <= 2^-25 (1 + 2^-14) |v| (every difference below is exact in fp64)
__device__ inline void split3_bf16(double v, uint32_t& p0, uint32_t& p1, uint32_t& p2) {
    const bf16_t a = f32_to_bf16((float)v);
    const double r1 = v - (double)bf16_to_f32(a);
    const bf16_t b = f32_to_bf16((float)r1);
    p0 = a;
    p1 = b;
    p2 = f32_to_bf16((float)(r1 - (double)bf16_to_f32(b)));
}

// The key coordinates z = x W for the assignment's screen in those coordinates, on MFMA:
// W's columns split into three bf16 parts (A operand, held by each wave for all its tiles),
// the points' rows as they are (exact bf16, B operand). The top part's products are summed
// per 16-deep step (one instruction from zero) and the steps added in fp64; the two smaller
// parts share one fp32 chain over the whole depth. Against the exact x W this leaves, per
// coordinate, |z - x W|_j <= 20 u a_j with a_j = sum_i |x_i| |W_ij| (16 u (1 + 2^-8) for the
// top part, about u for the chain, u / 2 for the parts' residual), and |a| <= |x| |W|_F.
// Each point's row holds z split into bf16 hi then lo (residual <= 2^-17 (1 + 2^-16) |z_j|,
// by the exponent of what the hi part leaves), and kb its bound coefficient for the screen:
// a score takes 4 dim exact products of the parts in one fp32 chain (<= 4 dim u (1 + 2^-7)^2
// |z| |c|, as |hi| + |lo| <= (1 + 2^-7) |z_j|), the two splits' residuals add
// 2^-16 (1 + 2^-15) |z| |c|, and the coordinates' own error 20 u |x| |W|_F |c|:
//   kb = (4 dim u (1 + 2^-7)^2 + 2^-16 (1 + 2^-15)) |z| + 20 u |x| |W|_F   (rounded up).
// The block stages W's split fragments in LDS once; a wave then takes tiles of 32 points,
// and lane (point j, half) ends with the 16 coordinates 8 q + 4 half + (0..3), q = 0..3,
// of its point.
template <int D>
__global__ __launch_bounds__(256, 3) void k_zcoords(const bf16_t* __restrict__ x, int n,
                                                 const double* __restrict__ l64, int dim,
                                                 int tiles_per_wave, bf16_t* __restrict__ zhl,
                                                 float* __restrict__ kb) {
    constexpr int KS = D / 16;
    constexpr double kUd = 5.9604644775390625e-08;
    __shared__ uint4 s_a[3 * KS * 64];          // [part][kk][lane]: the A fragment of that lane
    __shared__ double s_red[4];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5;
    const int col = lane & 31;
    const double* lh = l64 + (size_t)h * D * dim;
    // A of lane ln: row ln % 32 of W^T (column of W; zero past dim), depth 16 kk + 8 (ln / 32) + 0..7
    double wf = 0.0;
    for (int f = tid; f < KS * 64; f += 256) {
        const int kk = f / 64, ln = f % 64, cj = ln & 31;
        uint32_t pk[3][4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int i = 16 * kk + 8 * (ln >> 5) + e;
            const double w0 = cj < dim ? lh[(size_t)i * dim + cj] : 0.0;
            const double w1 = cj < dim ? lh[(size_t)(i + 1) * dim + cj] : 0.0;
            wf = fma(w0, w0, fma(w1, w1, wf));
            uint32_t x0, x1, x2, y0, y1, y2;
            split3_bf16(w0, x0, x1, x2);
            split3_bf16(w1, y0, y1, y2);
            pk[0][e / 2] = x0 | (y0 << 16);
            pk[1][e / 2] = x1 | (y1 << 16);
            pk[2][e / 2] = x2 | (y2 << 16);
        }
#pragma unroll
        for (int pt = 0; pt < 3; ++pt)
            s_a[(pt * KS + kk) * 64 + ln] = make_uint4(pk[pt][0], pk[pt][1], pk[pt][2], pk[pt][3]);
    }
    wf = wave_sum_f64(wf);
    if (lane == 0) s_red[w] = wf;
    __syncthreads();
    const double wfro = sqrt(s_red[0] + s_red[1] + s_red[2] + s_red[3]);    // |W|_F
    const int tiles = (n + 31) / 32;
    const int t0 = (blockIdx.x * 4 + w) * tiles_per_wave, t1 = min(tiles, t0 + tiles_per_wave);
    const double kz = 4.0 * dim * kUd * 1.0158 + 1.5260e-05;
    for (int t = t0; t < t1; ++t) {
        asm volatile("" ::: "memory");          // re-read the fragments per tile (no hoisting)
        const int p = t * 32 + col;
        const bf16_t* xr = x + ((size_t)h * n + min(p, n - 1)) * D + 8 * half;
        uint4 b[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) b[kk] = *reinterpret_cast<const uint4*>(xr + 16 * kk);
        double z[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.0;
        f32x16 ml = {};
        float xs = 0.f;
        // step kk's top-part products are added while step kk + 1's run (two in flight)
        f32x16 hp = mfma32x32x16(s_a[lane], b[0], f32x16{});
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            f32x16 hn = hp;
            if (kk + 1 < KS) hn = mfma32x32x16(s_a[(kk + 1) * 64 + lane], b[kk + 1], f32x16{});
            ml = mfma32x32x16(s_a[(KS + kk) * 64 + lane], b[kk], ml);
            ml = mfma32x32x16(s_a[(2 * KS + kk) * 64 + lane], b[kk], ml);
            const uint32_t wd[4] = {b[kk].x, b[kk].y, b[kk].z, b[kk].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = bf16_to_f32((bf16_t)(wd[e] & 0xFFFF));
                const float hi = bf16_to_f32((bf16_t)(wd[e] >> 16));
                xs = fmaf(lo, lo, fmaf(hi, hi, xs));
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) z[r] += (double)hp[r];
            hp = hn;
            __builtin_amdgcn_sched_barrier(0);
        }
        xs += __shfl_xor(xs, 32, 64);
        double zz = 0.0;
        bf16_t* zr = zhl + ((size_t)h * n + p) * 2 * dim;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j0 = 8 * q + 4 * half;
            uint32_t hw[2], lw[2];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const double v = z[4 * q + e] + (double)ml[4 * q + e];
                zz = fma(v, v, zz);
                const bf16_t hi = f32_to_bf16((float)v);
                const bf16_t lo = f32_to_bf16((float)(v - (double)bf16_to_f32(hi)));
                if (e & 1) {
                    hw[e >> 1] |= (uint32_t)hi << 16;
                    lw[e >> 1] |= (uint32_t)lo << 16;
                } else {
                    hw[e >> 1] = hi;
                    lw[e >> 1] = lo;
                }
            }
            if (p < n && j0 < dim) {
                *reinterpret_cast<uint2*>(zr + j0) = make_uint2(hw[0], hw[1]);
                *reinterpret_cast<uint2*>(zr + dim + j0) = make_uint2(lw[0], lw[1]);
            }
        }
        zz += __shfl_xor(zz, 32, 64);
        if (half == 0 && p < n) {
            const double xn = sqrt((double)xs) * 1.0001;
            kb[(size_t)h * n + p] = (float)((kz * sqrt(zz) + 20.0 * kUd * xn * wfro) * 1.0001);
        }
    }
}

void launch_zcoords(const bf16_t* x, int heads, int n, int d, const double* l64, int dim, bf16_t* zhl,
                    float* kb, hipStream_t st) {
    const int tiles = (n + 31) / 32;
    const int tpw = std::max(4, (int)(((size_t)tiles * heads + 2047) / 2048));
    const dim3 grid((unsigned)((tiles + 4 * tpw - 1) / (4 * tpw)), heads);
    if (d == 128)
        hipLaunchKernelGGL(k_zcoords<128>, grid, dim3(256), 0, st, x, n, l64, dim, tpw, zhl, kb);
    else
        hipLaunchKernelGGL(k_zcoords<64>, grid, dim3(256), 0, st, x, n, l64, dim, tpw, zhl, kb);
}

bool assign_streams(int groups, int d) {
    const int ntiles = (groups + kAssignTG - 1) / kAssignTG;
    return (size_t)ntiles * kAssignTG * 2 * d * 2 > (size_t)kAssignResBytes;
}

void launch_assign(const bf16_t* x, int heads, int n, int d, const bf16_t* cpart, const float* cn2,
                   const float* cpn, int groups, int32_t* labels, int32_t* flag_count,
                   int32_t* flag_list, hipStream_t st, const bf16_t* zhl, const float* kb, int dz) {
    const int ntiles = (groups + kAssignTG - 1) / kAssignTG;
    if (zhl != nullptr || (size_t)ntiles * kAssignTG * 2 * d * 2 <= (size_t)kAssignResBytes) {
        static int cus = 0;
        if (cus <= 0) {
            int dev = 0;
            if (hipGetDevice(&dev) != hipSuccess ||
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                cus <= 0)
                cus = 256;
        }
        const int total = heads * ((n + 63) / 64);
        const int blocks = std::max(1, std::min(total, cus));
        const int ipb = (total + blocks - 1) / blocks;
        const int nb = (total + ipb - 1) / ipb;
        if (zhl != nullptr && dz == 32)
            hipLaunchKernelGGL((k_assign_res<32, true>), dim3(nb), dim3(512), 0, st, zhl, n, heads, cpart, cn2,
                               cpn, groups, ipb, labels, flag_count, flag_list, kb);
        else if (zhl != nullptr)
            hipLaunchKernelGGL((k_assign_res<16, true>), dim3(nb), dim3(512), 0, st, zhl, n, heads, cpart, cn2,
                               cpn, groups, ipb, labels, flag_count, flag_list, kb);
        else if (d == 128)
            hipLaunchKernelGGL((k_assign_res<128, false>), dim3(nb), dim3(512), 0, st, x, n, heads, cpart, cn2,
                               cpn, groups, ipb, labels, flag_count, flag_list, nullptr);
        else
            hipLaunchKernelGGL((k_assign_res<64, false>), dim3(nb), dim3(512), 0, st, x, n, heads, cpart, cn2,
                               cpn, groups, ipb, labels, flag_count, flag_list, nullptr);
        return;
    }
    dim3 grid((n + 255) / 256, heads);
    if (d == 128)
        hipLaunchKernelGGL(k_assign<128>, grid, dim3(256), 0, st, x, n, cpart, cn2, cpn, groups,
                           labels, flag_count, flag_list);
    else
        hipLaunchKernelGGL(k_assign<64>, grid, dim3(256), 0, st, x, n, cpart, cn2, cpn, groups,
                           labels, flag_count, flag_list);
}

// ----------------------------------------------------------------- recheck ---
// A block per batch of 8 queued points, each exact-input point in fp64 against every fp64
// centroid, argmin with the lowest index on ties. With a factor L [d][dim]: coordinates
// y = x L (two halves of the depth summed in a fixed order) and |y - c|^2. With the full
// metric (dim == 0): |c|^2 - 2 x . C', which differs from the metric distance by x^T M x,
// the same for every centroid. A thread per centroid; each centroid coordinate read serves
// the whole batch, and every point's sums run in the same order whatever its batch.
constexpr int kRecheckBatch = 8;

__global__ __launch_bounds__(256) void k_recheck(const bf16_t* __restrict__ x, int n, int d,
                                                 const double* __restrict__ l64, int dim,
                                                 const double* __restrict__ c64,
                                                 const double* __restrict__ c2_64, int groups,
                                                 const int32_t* __restrict__ flag_count,
                                                 const int32_t* __restrict__ flag_list,
                                                 int32_t* __restrict__ labels) {
    constexpr int RB = kRecheckBatch;
    __shared__ double xs[128][RB];                 // [coordinate][point of the batch]
    __shared__ double part[2][128][RB];
    __shared__ double ys[128][RB];
    __shared__ double wbest[4][RB];
    __shared__ int wbg[4][RB];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool full = dim == 0;
    const int cdim = full ? d : dim;
    const int count = flag_count[h];
    const double* lh = l64 + (size_t)h * d * dim;
    const double* ch = c64 + (size_t)h * groups * cdim;
    const int32_t* fl = flag_list + (size_t)h * n;
    const int dh = d / 2;
    for (int b0 = blockIdx.x * RB; b0 < count; b0 += gridDim.x * RB) {
        const int nb = min(RB, count - b0);
        // a short batch repeats its first point; those results are dropped
        for (int i = tid; i < RB * d; i += 256) {
            const int b = i / d, j = i - b * d;
            const int p = fl[b0 + (b < nb ? b : 0)];
            xs[j][b] = (double)bf16_to_f32(x[((size_t)h * n + p) * d + j]);
        }
        __syncthreads();
        if (!full) {
            const int j = tid & 127, hf = tid >> 7;
            if (j < dim) {
                const int i0 = hf * dh, i1 = hf ? d : dh;
                double s[RB];
#pragma unroll
                for (int b = 0; b < RB; ++b) s[b] = 0.0;
                int i = i0;
                for (; i + 16 <= i1; i += 16) {          // loads 16 at a time, sums in order
                    double lv[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u) lv[u] = lh[(size_t)(i + u) * dim + j];
#pragma unroll
                    for (int u = 0; u < 16; ++u)
#pragma unroll
                        for (int b = 0; b < RB; ++b) s[b] = fma(xs[i + u][b], lv[u], s[b]);
                }
                for (; i < i1; ++i) {
                    const double l = lh[(size_t)i * dim + j];
#pragma unroll
                    for (int b = 0; b < RB; ++b) s[b] = fma(xs[i][b], l, s[b]);
                }
#pragma unroll
                for (int b = 0; b < RB; ++b) part[hf][j][b] = s[b];
            }
            __syncthreads();
            for (int i = tid; i < dim * RB; i += 256) {
                const int j = i / RB, b = i % RB;
                ys[j][b] = part[0][j][b] + part[1][j][b];
            }
            __syncthreads();
        }
        double best[RB];
        int bg[RB];
#pragma unroll
        for (int b = 0; b < RB; ++b) { best[b] = INFINITY; bg[b] = 0x7fffffff; }
        for (int g = tid; g < groups; g += 256) {
            const double* c = ch + g;                  // coordinate j of centroid g at c[j * groups]
            double acc[RB];
#pragma unroll
            for (int b = 0; b < RB; ++b) acc[b] = 0.0;
            if (full) {
                int j = 0;
                for (; j + 16 <= d; j += 16) {           // loads 16 at a time, sums in order
                    double cv[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u) cv[u] = c[(size_t)(j + u) * groups];
#pragma unroll
                    for (int u = 0; u < 16; ++u)
#pragma unroll
                        for (int b = 0; b < RB; ++b) acc[b] = fma(xs[j + u][b], cv[u], acc[b]);
                }
                for (; j < d; ++j) {
                    const double cj = c[(size_t)j * groups];
#pragma unroll
                    for (int b = 0; b < RB; ++b) acc[b] = fma(xs[j][b], cj, acc[b]);
                }
                const double c2 = c2_64[(size_t)h * groups + g];
#pragma unroll
                for (int b = 0; b < RB; ++b) acc[b] = fma(-2.0, acc[b], c2);
            } else {
                int j = 0;
                for (; j + 16 <= dim; j += 16) {
                    double cv[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u) cv[u] = c[(size_t)(j + u) * groups];
#pragma unroll
                    for (int u = 0; u < 16; ++u)
#pragma unroll
                        for (int b = 0; b < RB; ++b) {
                            const double t = ys[j + u][b] - cv[u];
                            acc[b] = fma(t, t, acc[b]);
                        }
                }
                for (; j < dim; ++j) {
                    const double cj = c[(size_t)j * groups];
#pragma unroll
                    for (int b = 0; b < RB; ++b) {
                        const double t = ys[j][b] - cj;
                        acc[b] = fma(t, t, acc[b]);
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < RB; ++b)
                if (acc[b] < best[b]) { best[b] = acc[b]; bg[b] = g; }
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            for (int o = 32; o > 0; o >>= 1) {
                const double ob = __shfl_xor(best[b], o, 64);
                const int og = __shfl_xor(bg[b], o, 64);
                if (ob < best[b] || (ob == best[b] && og < bg[b])) { best[b] = ob; bg[b] = og; }
            }
            if (lane == 0) {
                wbest[w][b] = best[b];
                wbg[w][b] = bg[b];
            }
        }
        __syncthreads();
        if (tid < nb) {
            double bb = wbest[0][tid];
            int g = wbg[0][tid];
            for (int k = 1; k < 4; ++k)
                if (wbest[k][tid] < bb || (wbest[k][tid] == bb && wbg[k][tid] < g)) {
                    bb = wbest[k][tid];
                    g = wbg[k][tid];
                }
            // no finite distance (non-finite coordinates): the lowest index, so a label is
            // always a group
            labels[(size_t)h * n + fl[b0 + tid]] = g < groups ? g : 0;
        }
        __syncthreads();
    }
}

void launch_recheck(const bf16_t* x, int heads, int n, int d, const double* l64, int dim,
                    const double* c64, const double* c2_64, int groups, const int32_t* flag_count,
                    const int32_t* flag_list, int32_t* labels, hipStream_t st) {
    int blocks = (n + kRecheckBatch - 1) / kRecheckBatch;
    if (blocks > 64) blocks = 64;
    hipLaunchKernelGGL(k_recheck, dim3(blocks, heads), dim3(256), 0, st, x, n, d, l64, dim, c64, c2_64,
                       groups, flag_count, flag_list, labels);
}

// ---------------------------------------------------------- counting sort ---
// A label outside [0, groups) counts as group 0 in both passes, so the sort stays a
// permutation whatever the labels hold.
__device__ inline int group_of(int32_t label, int groups) {
    return (uint32_t)label < (uint32_t)groups ? label : 0;
}

__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ labels, int n, int groups,
                                              int32_t* __restrict__ blkhist) {
    __shared__ int hist[kMaxGroups];
    const int h = blockIdx.y, b = blockIdx.x, tid = threadIdx.x;
    for (int g = tid; g < groups; g += 256) hist[g] = 0;
    __syncthreads();
    const int base = b * kSortChunk;
    for (int i = tid; i < kSortChunk; i += 256) {
        const int p = base + i;
        if (p < n) atomicAdd(&hist[group_of(labels[(size_t)h * n + p], groups)], 1);
    }
    __syncthreads();
    int32_t* out = blkhist + ((size_t)h * gridDim.x + b) * groups;
    for (int g = tid; g < groups; g += 256) out[g] = hist[g];
}

// per head: group totals, exclusive scan over groups (wave scans + a scan of the wave
// totals), then per-block bases in block order. Each group's blocks are split into
// contiguous ranges over several threads (1024 / groups of them, a power of two).
__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ blkhist, int nblk,
                                               int groups, int n, int32_t* __restrict__ blkoff,
                                               int32_t* __restrict__ off) {
    __shared__ int wtot[16];
    __shared__ int part[1024];                 // [range][group] partial counts, then bases
    __shared__ int gbase[kMaxGroups];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int tpg = 1;
    while (tpg * 2 * groups <= 1024) tpg *= 2;
    const int chunk = (nblk + tpg - 1) / tpg;
    const int32_t* hh = blkhist + (size_t)h * nblk * groups;
    const int gq = tid % groups, q = tid / groups;       // group, block range
    const bool mine = q < tpg;
    const int b0 = mine ? min(nblk, q * chunk) : 0, b1 = mine ? min(nblk, b0 + chunk) : 0;
    if (mine) {
        int t = 0;
#pragma unroll 8
        for (int b = b0; b < b1; ++b) t += hh[(size_t)b * groups + gq];
        part[q * groups + gq] = t;
    }
    __syncthreads();
    const int g = tid;
    int tot = 0;
    if (g < groups)
        for (int r = 0; r < tpg; ++r) tot += part[r * groups + g];
    // inclusive scan inside the wave
    int inc = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    int base = 0;
    for (int k = 0; k < w; ++k) base += wtot[k];
    if (g < groups) {
        const int run = base + inc - tot;      // exclusive prefix
        off[(size_t)h * (groups + 1) + g] = run;
        gbase[g] = run;
    }
    if (g == 0) off[(size_t)h * (groups + 1) + groups] = n;
    __syncthreads();
    if (mine) {
        int run = gbase[gq];
        for (int r = 0; r < q; ++r) run += part[r * groups + gq];
        int32_t* bo = blkoff + (size_t)h * nblk * groups;
        for (int b = b0; b < b1; ++b) {
            bo[(size_t)b * groups + gq] = run;
            run += hh[(size_t)b * groups + gq];
        }
    }
}

// A wave's points pw0 + 64 r + lane (label lab[r], -1 past the end) to sorted[base + rank],
// base from the wave's running bases wb (advanced here): in each round the lanes holding the
// same label are found from one ballot per label bit, and rank among them follows the lane.
template <int R>
__device__ inline void scatter_ranked(const int (&lab)[R], int* wb, int groups, int pw0, int lane,
                                      int32_t* __restrict__ sorted) {
    int nbits = 0;
    while ((1 << nbits) < groups) ++nbits;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int l = lab[r];
        const bool valid = l >= 0;
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = valid && ((l >> bit) & 1);
            const uint64_t m = __ballot(on);
            peers &= on ? m : ~m;
        }
        if (valid) {
            const int prefix = __popcll(peers & below);
            const int basev = wb[l];
            sorted[basev + prefix] = pw0 + r * 64 + lane;
            if (prefix == 0) wb[l] = basev + __popcll(peers);
        }
    }
}

// Stable scatter: the rank of a point among equal labels follows the point order. Wave w
// takes the block's points [256 w, 256 w + 256) in 4 rounds of 64: per-wave label counts
// give each wave its own base per label (block base + the counts of the waves before it);
// in a round, the lanes holding the same label are found from one ballot per label bit.
__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ labels, int n,
                                                 int groups, const int32_t* __restrict__ blkoff,
                                                 int32_t* __restrict__ sorted) {
    __shared__ int cnt[4][kMaxGroups];
    const int h = blockIdx.y, b = blockIdx.x, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < 4 * groups; i += 256) cnt[i / groups][i % groups] = 0;
    __syncthreads();
    constexpr int PW = kSortChunk / 4;           // points per wave
    const int pw0 = b * kSortChunk + wave * PW;
    int lab[PW / 64];
#pragma unroll
    for (int r = 0; r < PW / 64; ++r) {
        const int p = pw0 + r * 64 + lane;
        lab[r] = (p < n) ? group_of(labels[(size_t)h * n + p], groups) : -1;
        if (lab[r] >= 0) atomicAdd(&cnt[wave][lab[r]], 1);
    }
    __syncthreads();
    const int32_t* bo = blkoff + ((size_t)h * gridDim.x + b) * groups;
    for (int g = tid; g < groups; g += 256) {
        int run = bo[g];
        for (int w = 0; w < 4; ++w) {
            const int c = cnt[w][g];
            cnt[w][g] = run;
            run += c;
        }
    }
    __syncthreads();
    scatter_ranked(lab, cnt[wave], groups, pw0, lane, sorted + (size_t)h * n);
}

// k_scatter with the scan folded in, for heads of at most kFusedScanBlocks blocks: each
// block sums its head's block histograms itself (every group's total, and its count in the
// blocks before this one, both in block order), scans the totals over the groups, and block
// 0 also writes the group offsets. The bases are k_scan's; one launch fewer per sort, for
// nblk reads per group and block (a few microseconds of cached reads at these sizes).
constexpr int kFusedScanBlocks = 256;
__global__ __launch_bounds__(256) void k_scatter_scan(const int32_t* __restrict__ labels, int n,
                                                      int groups, const int32_t* __restrict__ blkhist,
                                                      int32_t* __restrict__ off,
                                                      int32_t* __restrict__ sorted) {
    __shared__ int cnt[4][kMaxGroups];
    __shared__ int s_tot[kMaxGroups];          // group totals, then their exclusive prefix
    __shared__ int s_pre[kMaxGroups];          // counts in the blocks before this one
    __shared__ int s_wt[4];
    const int h = blockIdx.y, b = blockIdx.x, nblk = gridDim.x, tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int32_t* hh = blkhist + (size_t)h * nblk * groups;
    for (int g = tid; g < groups; g += 256) {
        int pre = 0, tot = 0;
#pragma unroll 8
        for (int bb = 0; bb < nblk; ++bb) {
            const int c = hh[(size_t)bb * groups + g];
            pre += bb < b ? c : 0;
            tot += c;
        }
        s_pre[g] = pre;
        s_tot[g] = tot;
    }
    for (int i = tid; i < 4 * groups; i += 256) cnt[i / groups][i % groups] = 0;
    __syncthreads();
    // exclusive scan of the totals: thread t takes groups 4t .. 4t+3 (groups <= 1024), a
    // wave scan of the thread sums, then the wave totals
    const int g0 = 4 * tid;
    int loc[4], run = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        loc[e] = (g0 + e < groups) ? s_tot[g0 + e] : 0;
        run += loc[e];
    }
    int inc = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    if (lane == 63) s_wt[wave] = inc;
    __syncthreads();
    int acc = inc - run;
    for (int k = 0; k < wave; ++k) acc += s_wt[k];
    int32_t* oh = off + (size_t)h * (groups + 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (g0 + e < groups) {                 // only this thread reads these entries
            s_tot[g0 + e] = acc;
            if (b == 0) oh[g0 + e] = acc;
            acc += loc[e];
        }
    }
    if (b == 0 && tid == 0) oh[groups] = n;
    // the points of this block, counted per wave
    constexpr int PW = kSortChunk / 4;
    const int pw0 = b * kSortChunk + wave * PW;
    int lab[PW / 64];
#pragma unroll
    for (int r = 0; r < PW / 64; ++r) {
        const int p = pw0 + r * 64 + lane;
        lab[r] = (p < n) ? group_of(labels[(size_t)h * n + p], groups) : -1;
        if (lab[r] >= 0) atomicAdd(&cnt[wave][lab[r]], 1);
    }
    __syncthreads();
    for (int g = tid; g < groups; g += 256) {
        int base = s_tot[g] + s_pre[g];
        for (int w = 0; w < 4; ++w) {
            const int c = cnt[w][g];
            cnt[w][g] = base;
            base += c;
        }
    }
    __syncthreads();
    scatter_ranked(lab, cnt[wave], groups, pw0, lane, sorted + (size_t)h * n);
}

void launch_counting_sort(const int32_t* labels, int heads, int n, int groups, int32_t* blkhist,
                          int32_t* blkoff, int32_t* sorted, int32_t* off, hipStream_t st) {
    const int nblk = (n + kSortChunk - 1) / kSortChunk;
    hipLaunchKernelGGL(k_hist, dim3(nblk, heads), dim3(256), 0, st, labels, n, groups, blkhist);
    if (nblk <= kFusedScanBlocks) {
        hipLaunchKernelGGL(k_scatter_scan, dim3(nblk, heads), dim3(256), 0, st, labels, n, groups, blkhist,
                           off, sorted);
        return;
    }
    hipLaunchKernelGGL(k_scan, dim3(heads), dim3(1024), 0, st, blkhist, nblk, groups, n, blkoff, off);
    hipLaunchKernelGGL(k_scatter, dim3(nblk, heads), dim3(256), 0, st, labels, n, groups, blkoff,
                       sorted);
}

// -------------------------------------------------------------- group means ---
// Block per (group, head): fp64 sum of the members' raw rows in sorted order, over a
// fixed split of rows to row lanes (four rows in flight per lane) and a fixed-order
// reduction; mean = sum / count (zero if empty). With l64 given, the non-empty groups
// then get their projected centroid, screening vector and norms (k_finish).
template <int D>
__global__ __launch_bounds__(512) void k_group_sum(const bf16_t* __restrict__ x, int n,
                                                   const int32_t* __restrict__ sorted,
                                                   const int32_t* __restrict__ off, int groups,
                                                   double* __restrict__ mean_raw) {
    constexpr int CH = D / 8;          // 16-byte chunks per row
    constexpr int RL = 512 / CH;       // row lanes
    constexpr int IDX = 2048;          // member indices staged per pass
    __shared__ double red[RL][D + 1];
    __shared__ int s_idx[IDX];
    const int h = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
    const int c = tid % CH, rl = tid / CH;
    const int32_t* oh = off + (size_t)h * (groups + 1);
    const int beg = oh[g], end = oh[g + 1];
    const int cnt = end - beg;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    const int32_t* sh = sorted + (size_t)h * n;
    const bf16_t* xh = x + (size_t)h * n * D + c * 8;
    auto add = [&](const uint4 v) {
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)bf16_to_f32((bf16_t)(wd[e] & 0xFFFF));
            acc[2 * e + 1] += (double)bf16_to_f32((bf16_t)(wd[e] >> 16));
        }
    };
    // members in passes of IDX: indices staged in LDS with coalesced loads, then eight
    // rows in flight per row lane; member m always goes to row lane m % RL (fixed order)
    for (int p0 = 0; p0 < cnt; p0 += IDX) {
        const int np = min(IDX, cnt - p0);
        __syncthreads();
        for (int i = tid; i < np; i += 512) s_idx[i] = sh[beg + p0 + i];
        __syncthreads();
        int m = rl;
        for (; m + 7 * RL < np; m += 8 * RL) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint4*>(xh + (size_t)s_idx[m + u * RL] * D);
#pragma unroll
            for (int u = 0; u < 8; ++u) add(v[u]);
        }
        for (; m < np; m += RL) add(*reinterpret_cast<const uint4*>(xh + (size_t)s_idx[m] * D));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rl][c * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        double s = 0.0;
#pragma unroll
        for (int r = 0; r < RL; ++r) s += red[r][tid];
        mean_raw[((size_t)h * groups + g) * D + tid] = (cnt > 0) ? s / cnt : 0.0;
    }
}

void launch_group_means(const bf16_t* x, int heads, int n, int d, const int32_t* sorted,
                        const int32_t* off, int groups, double* mean_raw, const double* l64,
                        int dout, double* c64, bf16_t* cpart, float* cn2, float* cpn,
                        double* c2_64, hipStream_t st, double* crow, int coords) {
    if (d == 128)
        hipLaunchKernelGGL(k_group_sum<128>, dim3(groups, heads), dim3(512), 0, st, x, n, sorted, off,
                           groups, mean_raw);
    else
        hipLaunchKernelGGL(k_group_sum<64>, dim3(groups, heads), dim3(512), 0, st, x, n, sorted, off,
                           groups, mean_raw);
    if (l64 != nullptr)
        launch_finish(mean_raw, heads, d, l64, dout, groups, off, c64, cpart, cn2, cpn, c2_64, st, crow, coords);
}

}  // namespace spr
