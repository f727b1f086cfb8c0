// Correction stage: "Partition the Support, Reconstruct the Residual" (gist.science
// summary), section 2B -- the fitted residual b' + x B' is added to every unprobed
// row's sparse output x; probe rows keep their exact dense output; rows go back to the
// original token order. Output rounded once (bf16 nearest-even or fp32).
#include "kernels.h"

namespace spr {

// Correction GEMM on MFMA: for 32 rows x per wave, C^T = B'^T X^T with
//   A = B'^T (rows = output column j, depth = i), held in LDS as bf16 hi/lo parts,
//   B = X^T  (depth = i, columns = rows), X's fp32 rows split into bf16 hi/lo in VGPRs,
// three products hi.hi + hi.lo + lo.hi (relative error about 2^-16 of |X||B'|, so the
// correction stays accurate when |B'| is large). Each lane then owns one row: it adds
// X and b', or takes the exact dense output for a probe row, and stores the row at its
// original token index.
template <int D>
__global__ __launch_bounds__(256) void k_correct(const float* __restrict__ o_s,
                                                 const float* __restrict__ bmat,
                                                 const float* __restrict__ bvec,
                                                 const float* __restrict__ od,
                                                 const int32_t* __restrict__ probe_of,
                                                 const int32_t* __restrict__ qperm, int n,
                                                 int probes, void* __restrict__ out, int out_f32) {
    constexpr int CH = D / 8;          // 16-byte chunks per bf16 row of B'^T
    constexpr int JB = D / 32;         // 32-column output blocks
    __shared__ uint4 s_b[2][D * CH];   // B'^T hi / lo: row j, chunk c at c ^ swz(j)
    __shared__ float s_bv[D];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5;
    const float* bh = bmat + (size_t)h * D * D;
    // stage B'^T as bf16 hi/lo: thread item = (j, chunk c) -> 8 consecutive i
    for (int it = tid; it < D * CH; it += 256) {
        const int j = it / CH, c = it % CH;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = bh[(size_t)(c * 8 + 2 * e) * D + j];
            const float v1 = bh[(size_t)(c * 8 + 2 * e + 1) * D + j];
            const bf16_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
            hw[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lw[e] = pack_bf16x2(v0 - bf16_to_f32(h0), v1 - bf16_to_f32(h1));
        }
        const int pc = c ^ swz<CH>(j);
        s_b[0][j * CH + pc] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        s_b[1][j * CH + pc] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    for (int j = tid; j < D; j += 256) s_bv[j] = bvec[(size_t)h * D + j];
    __syncthreads();
    const int row = blockIdx.x * 128 + w * 32 + (lane & 31);
    const bool valid = row < n;
    const float* xr = o_s + ((size_t)h * n + (valid ? row : 0)) * D;
    f32x16 acc[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) acc[jb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        float xv[8];
        const float4 a0 = valid ? *reinterpret_cast<const float4*>(xr + 16 * kk + 8 * half)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 a1 = valid ? *reinterpret_cast<const float4*>(xr + 16 * kk + 8 * half + 4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        xv[0] = a0.x; xv[1] = a0.y; xv[2] = a0.z; xv[3] = a0.w;
        xv[4] = a1.x; xv[5] = a1.y; xv[6] = a1.z; xv[7] = a1.w;
        uint32_t xh[4], xl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16_t h0 = f32_to_bf16(xv[2 * e]), h1 = f32_to_bf16(xv[2 * e + 1]);
            xh[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            xl[e] = pack_bf16x2(xv[2 * e] - bf16_to_f32(h0), xv[2 * e + 1] - bf16_to_f32(h1));
        }
        const uint4 bhi = make_uint4(xh[0], xh[1], xh[2], xh[3]);
        const uint4 blo = make_uint4(xl[0], xl[1], xl[2], xl[3]);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
            const int j = jb * 32 + (lane & 31);
            const int pc = (2 * kk + half) ^ swz<CH>(j);
            const uint4 ahi = s_b[0][j * CH + pc];
            const uint4 alo = s_b[1][j * CH + pc];
            acc[jb] = mfma32x32x16(ahi, bhi, acc[jb]);
            acc[jb] = mfma32x32x16(ahi, blo, acc[jb]);
            acc[jb] = mfma32x32x16(alo, bhi, acc[jb]);
        }
    }
    if (!valid) return;
    // this lane: row `row`, columns j = jb*32 + 8g + 4*half + 0..3
    const int pi = probe_of[(size_t)h * n + row];
    const size_t dst = ((size_t)h * n + qperm[(size_t)h * n + row]) * D;
    const float* src = (pi >= 0) ? od + ((size_t)h * probes + pi) * D : xr;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int j = jb * 32 + 8 * g + 4 * half;
            const float4 xv = *reinterpret_cast<const float4*>(src + j);
            float v[4] = {xv.x, xv.y, xv.z, xv.w};
            if (pi < 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (v[e] + s_bv[j + e]) + acc[jb][4 * g + e];
            }
            if (out_f32) {
                *reinterpret_cast<float4*>(static_cast<float*>(out) + dst + j) =
                    make_float4(v[0], v[1], v[2], v[3]);
            } else {
                *reinterpret_cast<uint2*>(static_cast<bf16_t*>(out) + dst + j) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        }
}

void launch_correct(const float* o_s, const float* bmat, const float* bvec, const float* od,
                    const int32_t* probe_of, const int32_t* qperm, int heads, int n, int d,
                    int probes, void* o, int out_f32, hipStream_t st) {
    dim3 grid((n + 127) / 128, heads);
    if (d == 128)
        hipLaunchKernelGGL(k_correct<128>, grid, dim3(256), 0, st, o_s, bmat, bvec, od, probe_of, qperm,
                           n, probes, o, out_f32);
    else
        hipLaunchKernelGGL(k_correct<64>, grid, dim3(256), 0, st, o_s, bmat, bvec, od, probe_of, qperm,
                           n, probes, o, out_f32);
}

}  // namespace spr

namespace spr {

// ------------------------------------------------------------- fit Grams ---
// Column means of a [H][p][d] (fixed summation order).
template <typename T>
__global__ void k_col_means(const T* __restrict__ a, int p, int d, double* __restrict__ mean) {
    const int h = blockIdx.x, j = threadIdx.x;
    if (j >= d) return;
    double s = 0.0;
    for (int r = 0; r < p; ++r) s += (double)a[((size_t)h * p + r) * d + j];
    mean[(size_t)h * d + j] = (p > 0) ? s / p : 0.0;
}

// out[h][i][j] = scale * sum_r (a[r][i] - ma[i]) (b[r][j] - mb[j]); ma / mb may be null.
template <typename T>
__global__ void k_gram(const T* __restrict__ a, const T* __restrict__ b,
                       const double* __restrict__ ma, const double* __restrict__ mb, int p, int d,
                       double scale, double* __restrict__ out) {
    const int h = blockIdx.y, i = blockIdx.x, j = threadIdx.x;
    if (j >= d) return;
    const double ai0 = ma ? ma[(size_t)h * d + i] : 0.0;
    const double bj0 = mb ? mb[(size_t)h * d + j] : 0.0;
    double s = 0.0;
    for (int r = 0; r < p; ++r) {
        const size_t row = ((size_t)h * p + r) * d;
        s += ((double)a[row + i] - ai0) * ((double)b[row + j] - bj0);
    }
    out[((size_t)h * d + i) * d + j] = s * scale;
}

void launch_col_means_f32(const float* a, int heads, int p, int d, double* mean, hipStream_t st) {
    hipLaunchKernelGGL(k_col_means<float>, dim3(heads), dim3(128), 0, st, a, p, d, mean);
}

void launch_gram_f32(const float* a, const float* b, const double* ma, const double* mb, int heads,
                     int p, int d, double* out, hipStream_t st) {
    hipLaunchKernelGGL(k_gram<float>, dim3(d, heads), dim3(128), 0, st, a, b, ma, mb, p, d, 1.0, out);
}

void launch_gram_f64(const double* a, int heads, int p, int d, double scale, double* out,
                     hipStream_t st) {
    hipLaunchKernelGGL(k_gram<double>, dim3(d, heads), dim3(128), 0, st, a, a, nullptr, nullptr, p,
                       d, scale, out);
}

}  // namespace spr
