// Correction stage: "Partition the Support, Reconstruct the Residual" (gist.science
// summary), section 2B -- the fitted residual b' + x B' is added to every unprobed
// row's sparse output x; probe rows keep their exact dense output; rows go back to the
// original token order. Output rounded once (bf16 nearest-even or fp32).
#include "kernels.h"

namespace spr {

// Correction GEMM on MFMA: for 32 rows x per wave, C^T = B'^T X^T with
//   A = B'^T (rows = output column j, depth = i), bf16 hi and lo parts prepared by the
//       host, staged in LDS with coalesced loads,
//   B = X^T  (depth = i, columns = rows), X's fp32 rows split into bf16 hi/lo in VGPRs,
// three products hi.hi + hi.lo + lo.hi (relative error about 2^-16 of |X||B'|, so the
// correction stays accurate when |B'| is large). Each lane then owns one row: it adds
// X and b', or takes the exact dense output for a probe row. The finished rows go
// through LDS (reusing the B' tile) so that each output row is stored whole, at its
// original token index.
template <int D>
__global__ __launch_bounds__(256) void k_correct(const float* __restrict__ o_s,
                                                 const bf16_t* __restrict__ bt16,
                                                 const float* __restrict__ bvec,
                                                 const float* __restrict__ od,
                                                 const int32_t* __restrict__ probe_of,
                                                 const int32_t* __restrict__ qperm, int n,
                                                 int probes, void* __restrict__ out, int out_f32) {
    constexpr int CH = D / 8;          // 16-byte chunks per bf16 row of B'^T
    constexpr int JB = D / 32;         // 32-column output blocks
    constexpr int SB = 2 * D * CH;                 // B'^T hi / lo tiles (16-byte slots)
    constexpr int SO = 4 * 32 * D * 4 / 16;        // output staging, 4 waves x 32 rows (fp32)
    __shared__ uint4 s_raw[SB > SO ? SB : SO];
    uint4(*s_b)[D * CH] = reinterpret_cast<uint4(*)[D * CH]>(s_raw);   // row j, chunk c at c ^ swz(j)
    __shared__ float s_bv[D];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5;
    const uint4* bsrc = reinterpret_cast<const uint4*>(bt16 + (size_t)h * 2 * D * D);
    for (int it = tid; it < 2 * D * CH; it += 256) {
        const int part = it / (D * CH), rem = it % (D * CH);
        const int j = rem / CH, c = rem % CH;
        s_b[part][j * CH + (c ^ swz<CH>(j))] = bsrc[it];
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
    // this lane: row `row`, columns j = jb*32 + 8g + 4*half + 0..3, finished in registers
    const int pi = valid ? probe_of[(size_t)h * n + row] : -1;
    const float* src = (pi >= 0) ? od + ((size_t)h * probes + pi) * D : xr;
    float res[JB][16];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int j = jb * 32 + 8 * g + 4 * half;
            const float4 xv = valid ? *reinterpret_cast<const float4*>(src + j) : make_float4(0.f, 0.f, 0.f, 0.f);
            const float v[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                res[jb][4 * g + e] = (pi < 0) ? (v[e] + s_bv[j + e]) + acc[jb][4 * g + e] : v[e];
        }
    // stage the wave's 32 finished rows in LDS (over the B' tile), then store whole rows
    __syncthreads();
    const int esz = out_f32 ? 4 : 2;
    char* stage = reinterpret_cast<char*>(s_raw) + (size_t)w * 32 * D * 4;   // 32 rows x D x 4 B
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int j = jb * 32 + 8 * g + 4 * half;
            char* dst = stage + ((size_t)(lane & 31) * D + j) * esz;
            if (out_f32)
                *reinterpret_cast<float4*>(dst) = make_float4(res[jb][4 * g], res[jb][4 * g + 1],
                                                              res[jb][4 * g + 2], res[jb][4 * g + 3]);
            else
                *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(res[jb][4 * g], res[jb][4 * g + 1]),
                                                            pack_bf16x2(res[jb][4 * g + 2], res[jb][4 * g + 3]));
        }
    __syncthreads();
    // row-contiguous stores: 16-byte pieces, consecutive lanes along a row
    const int pieces = D * esz / 16;                   // per row
    const int row_base = blockIdx.x * 128 + w * 32;
    for (int it = lane; it < 32 * pieces; it += 64) {
        const int r = it / pieces, pc = it % pieces;
        const int gr = row_base + r;
        if (gr >= n) continue;
        const size_t drow = (size_t)h * n + qperm[(size_t)h * n + gr];
        const uint4 v = *reinterpret_cast<const uint4*>(stage + (size_t)r * D * esz + pc * 16);
        *reinterpret_cast<uint4*>(static_cast<char*>(out) + drow * D * esz + pc * 16) = v;
    }
}

void launch_correct(const float* o_s, const bf16_t* bt16, const float* bvec, const float* od,
                    const int32_t* probe_of, const int32_t* qperm, int heads, int n, int d,
                    int probes, void* o, int out_f32, hipStream_t st) {
    dim3 grid((n + 127) / 128, heads);
    if (d == 128)
        hipLaunchKernelGGL(k_correct<128>, grid, dim3(256), 0, st, o_s, bt16, bvec, od, probe_of, qperm,
                           n, probes, o, out_f32);
    else
        hipLaunchKernelGGL(k_correct<64>, grid, dim3(256), 0, st, o_s, bt16, bvec, od, probe_of, qperm,
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
