// Correction stage: "Partition the Support, Reconstruct the Residual" (gist.science
// summary), section 2B -- the fitted residual b' + x B' is added to every unprobed
// row's sparse output x; probe rows keep their exact dense output; rows go back to the
// original token order. Output rounded once (bf16 nearest-even or fp32).
#include "kernels.h"

namespace spr {

// Correction GEMM on MFMA: for 32 rows x per wave, C^T = B'^T X^T with
//   A = B'^T (rows = output column j, depth = i), bf16 hi and lo parts prepared by the
//       host, staged in LDS once per block with coalesced loads,
//   B = X^T  (depth = i, columns = rows), X's fp32 rows split into bf16 hi/lo in VGPRs,
// three products hi.hi + hi.lo + lo.hi (relative error about 2^-16 of |X||B'|, so the
// correction stays accurate when |B'| is large). Each lane then owns one row and adds X
// and b' to its columns; the X values it needs there come from its own and its partner
// lane's (l ^ 32) fragments through one lane-half swap per value, not a second read. The
// finished rows go through LDS so that each output row is stored whole, at its original
// token index. Probe rows are overwritten with their exact dense output afterwards
// (k_probe_rows). Blocks (8 waves) are persistent within a head: each stages B' once and
// walks tiles of 256 rows, the next tile's rows loaded while the current one is computed.
constexpr int kCorrWaves = 8;
constexpr int kCorrRows = 32 * kCorrWaves;

template <int D>
__global__ __launch_bounds__(64 * kCorrWaves, 1) void k_correct(const float* __restrict__ o_s,
                                                    const bf16_t* __restrict__ bt16,
                                                    const float* __restrict__ bvec,
                                                    const int32_t* __restrict__ qperm, int n,
                                                    void* __restrict__ out, int out_f32) {
    constexpr int CH = D / 8;          // 16-byte chunks per bf16 row of B'^T
    constexpr int JB = D / 32;         // 32-column output blocks
    constexpr int KS = D / 16;         // depth steps
    __shared__ uint4 s_b[2][D * CH];   // B'^T hi / lo: row j, chunk c at c ^ swz(j)
    constexpr int SROW = D * 2 + 16;                 // staged row pitch in bytes (padded)
    __shared__ uint4 s_out[kCorrWaves][32 * SROW / 16];   // per wave: 32 bf16 rows (16 fp32 rows)
    __shared__ float s_bv[D];
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int half = lane >> 5;
    const uint4* bsrc = reinterpret_cast<const uint4*>(bt16 + (size_t)h * 2 * D * D);
    for (int it = tid; it < 2 * D * CH; it += 64 * kCorrWaves) {
        const int part = it / (D * CH), rem = it % (D * CH);
        const int j = rem / CH, c = rem % CH;
        s_b[part][j * CH + (c ^ swz<CH>(j))] = bsrc[it];
    }
    for (int j = tid; j < D; j += 64 * kCorrWaves) s_bv[j] = bvec[(size_t)h * D + j];
    __syncthreads();
    const int esz = out_f32 ? 4 : 2;
    const int pieces = D * esz / 16;                  // 16-byte pieces per output row
    const int pass_rows = out_f32 ? 16 : 32;          // rows per staging pass
    const int pitch = out_f32 ? 2 * SROW - 16 : SROW; // bytes per staged row (16 B of padding)
    char* stage = reinterpret_cast<char*>(&s_out[w][0]);
    const int ntile = (n + kCorrRows - 1) / kCorrRows;

    // a tile's rows for this lane: X fragments (an invalid row reads row 0) and the
    // original token index
    float4 xa[KS][2];
    int dst_row = 0;
    auto load_tile = [&](int tile, float4 (&x)[KS][2], int& dr) {
        const int row = tile * kCorrRows + w * 32 + (lane & 31);
        const bool valid = row < n;
        const float* xr = o_s + ((size_t)h * n + (valid ? row : 0)) * D;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            x[kk][0] = *reinterpret_cast<const float4*>(xr + 16 * kk + 8 * half);
            x[kk][1] = *reinterpret_cast<const float4*>(xr + 16 * kk + 8 * half + 4);
        }
        dr = valid ? qperm[(size_t)h * n + row] : 0;
    };
    if (blockIdx.x < ntile) load_tile(blockIdx.x, xa, dst_row);
    for (int tile = blockIdx.x; tile < ntile; tile += gridDim.x) {
        const int row_base = tile * kCorrRows + w * 32;
        const bool valid = row_base + (lane & 31) < n;
        float4 xn[KS][2];
        int dn = 0;
        if (tile + (int)gridDim.x < ntile) load_tile(tile + gridDim.x, xn, dn);
        __builtin_amdgcn_sched_barrier(0);      // the next tile's loads go out first
        f32x16 acc[JB];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) acc[jb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const float zf = valid ? 1.f : 0.f;
            float xv[8] = {xa[kk][0].x * zf, xa[kk][0].y * zf, xa[kk][0].z * zf, xa[kk][0].w * zf,
                           xa[kk][1].x * zf, xa[kk][1].y * zf, xa[kk][1].z * zf, xa[kk][1].w * zf};
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
        // this lane: row `row`, columns j = jb*32 + 8g + 4*half + 0..3, i.e. depth step
        // kk = 2jb + g/2 at offset 8(g%2) + 4*half. It holds offsets 8*half + 0..7 of every
        // step; swapping fragment 0 of the low lane half with fragment 1 of the high half
        // leaves offsets 4*half + 0..3 (g even) in xa[kk][0] and 8 + 4*half + 0..3 (g odd)
        // in xa[kk][1] on every lane.
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float* f0 = reinterpret_cast<float*>(&xa[kk][0]);
            float* f1 = reinterpret_cast<float*>(&xa[kk][1]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(f0[e]),
                                                                __float_as_uint(f1[e]), false, false);
                f0[e] = __uint_as_float(r[0]);
                f1[e] = __uint_as_float(r[1]);
            }
        }
        float res[JB][16];
#pragma unroll
        for (int jb = 0; jb < JB; ++jb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int j = jb * 32 + 8 * g + 4 * half;
                const float4 xv = xa[2 * jb + (g >> 1)][g & 1];
                const float v[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) res[jb][4 * g + e] = (v[e] + s_bv[j + e]) + acc[jb][4 * g + e];
            }
        // stage finished rows in the wave's own LDS area (a wave-level barrier suffices),
        // then store whole rows: 16-byte pieces, consecutive lanes along a row
        for (int r0 = 0; r0 < 32; r0 += pass_rows) {
            const int lr = (lane & 31) - r0;
            if (lr >= 0 && lr < pass_rows) {
#pragma unroll
                for (int jb = 0; jb < JB; ++jb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int j = jb * 32 + 8 * g + 4 * half;
                        char* dst = stage + (size_t)lr * pitch + (size_t)j * esz;
                        const float* rr = &res[jb][4 * g];
                        if (out_f32)
                            *reinterpret_cast<float4*>(dst) = make_float4(rr[0], rr[1], rr[2], rr[3]);
                        else
                            *reinterpret_cast<uint2*>(dst) =
                                make_uint2(pack_bf16x2(rr[0], rr[1]), pack_bf16x2(rr[2], rr[3]));
                    }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            for (int it = lane; it < pass_rows * pieces; it += 64) {
                const int r = it / pieces, pc = it % pieces;
                const int drow_r = __shfl(dst_row, r0 + r, 64);       // lane r0 + r owns row r0 + r
                if (row_base + r0 + r >= n) continue;
                const size_t drow = (size_t)h * n + drow_r;
                const uint4 v = *reinterpret_cast<const uint4*>(stage + (size_t)r * pitch + pc * 16);
                *reinterpret_cast<uint4*>(static_cast<char*>(out) + drow * D * esz + pc * 16) = v;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            xa[kk][0] = xn[kk][0];
            xa[kk][1] = xn[kk][1];
        }
        dst_row = dn;
    }
}

// Probe rows take their exact dense output: out[h][probe_orig[p]] = od[h][p] (after
// k_correct, same stream). Block per (probe, head), one thread per column.
__global__ void k_probe_rows(const float* __restrict__ od, const int32_t* __restrict__ probe_orig,
                             int n, int d, int probes, void* __restrict__ out, int out_f32) {
    const int p = blockIdx.x, h = blockIdx.y, j = threadIdx.x;
    if (j >= d) return;
    const float v = od[((size_t)h * probes + p) * d + j];
    const size_t o = ((size_t)h * n + probe_orig[(size_t)h * probes + p]) * d + j;
    if (out_f32) static_cast<float*>(out)[o] = v;
    else static_cast<bf16_t*>(out)[o] = f32_to_bf16(v);
}

void launch_correct(const float* o_s, const bf16_t* bt16, const float* bvec, const float* od,
                    const int32_t* probe_orig, const int32_t* qperm, int heads, int n, int d,
                    int probes, void* o, int out_f32, hipStream_t st) {
    const int ntile = (n + kCorrRows - 1) / kCorrRows;
    // one resident block per CU (a block fills a CU): rounding the share per head down
    // keeps the grid within one round of blocks
    static int cus = 0;
    if (cus <= 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
    }
    int per_head = cus / heads;
    if (per_head > ntile) per_head = ntile;
    if (per_head < 1) per_head = 1;
    dim3 grid(per_head, heads);
    if (d == 128)
        hipLaunchKernelGGL(k_correct<128>, grid, dim3(64 * kCorrWaves), 0, st, o_s, bt16, bvec, qperm,
                           n, o, out_f32);
    else
        hipLaunchKernelGGL(k_correct<64>, grid, dim3(64 * kCorrWaves), 0, st, o_s, bt16, bvec, qperm,
                           n, o, out_f32);
    if (probes > 0)
        hipLaunchKernelGGL(k_probe_rows, dim3(probes, heads), dim3(d), 0, st, od, probe_orig, n, d,
                           probes, o, out_f32);
}

}  // namespace spr

namespace spr {

// ------------------------------------------------------------- fit Grams ---
// Column means of a [H][p][d]: block per (head, 32 columns), 8 row partitions per column
// (rows r = part, part + 8, ...), combined in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void k_col_means(const T* __restrict__ a, int p, int d,
                                                   double* __restrict__ mean) {
    __shared__ double red[8][32];
    const int h = blockIdx.y, j = blockIdx.x * 32 + (threadIdx.x & 31), part = threadIdx.x >> 5;
    double s = 0.0;
    for (int r = part; r < p; r += 8) s += (double)a[((size_t)h * p + r) * d + j];
    red[part][threadIdx.x & 31] = s;
    __syncthreads();
    if (part == 0) {
        double t = red[0][j & 31];
#pragma unroll
        for (int q = 1; q < 8; ++q) t += red[q][j & 31];
        mean[(size_t)h * d + j] = (p > 0) ? t / p : 0.0;
    }
}

// out[h][i][j] = scale * sum_r (a[r][i] - ma[i]) (b[r][j] - mb[j]); ma / mb may be null.
// Block per (head, 32 x 32 output tile): rows staged through LDS 32 at a time, each thread
// accumulating 4 outputs over ascending r in fp64 (fixed order).
template <typename T>
__global__ __launch_bounds__(256) void k_gram(const T* __restrict__ a, const T* __restrict__ b,
                                              const double* __restrict__ ma,
                                              const double* __restrict__ mb, int p, int d,
                                              double scale, double* __restrict__ out) {
    __shared__ double sa[32][33], sb[32][33];
    const int h = blockIdx.z, ti = blockIdx.y * 32, tj = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    const double ca = ma ? ma[(size_t)h * d + ti + tx] : 0.0;
    const double cb = mb ? mb[(size_t)h * d + tj + tx] : 0.0;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int r0 = 0; r0 < p; r0 += 32) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rr = ty + 8 * q, r = r0 + rr;
            double va = 0.0, vb = 0.0;
            if (r < p) {
                const size_t row = ((size_t)h * p + r) * d;
                va = (double)a[row + ti + tx] - ca;
                vb = (double)b[row + tj + tx] - cb;
            }
            sa[rr][tx] = va;
            sb[rr][tx] = vb;
        }
        __syncthreads();
#pragma unroll 8
        for (int rr = 0; rr < 32; ++rr) {
            const double bj = sb[rr][tx];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[q] += sa[rr][ty + 8 * q] * bj;
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) out[((size_t)h * d + ti + ty + 8 * q) * d + tj + tx] = acc[q] * scale;
}

void launch_col_means_f32(const float* a, int heads, int p, int d, double* mean, hipStream_t st) {
    hipLaunchKernelGGL(k_col_means<float>, dim3(d / 32, heads), dim3(256), 0, st, a, p, d, mean);
}

void launch_gram_f32(const float* a, const float* b, const double* ma, const double* mb, int heads,
                     int p, int d, double* out, hipStream_t st) {
    hipLaunchKernelGGL(k_gram<float>, dim3(d / 32, d / 32, heads), dim3(256), 0, st, a, b, ma, mb,
                       p, d, 1.0, out);
}

void launch_gram_f64(const double* a, int heads, int p, int d, double scale, double* out,
                     hipStream_t st) {
    hipLaunchKernelGGL(k_gram<double>, dim3(d / 32, d / 32, heads), dim3(256), 0, st, a, a, nullptr,
                       nullptr, p, d, scale, out);
}

}  // namespace spr
