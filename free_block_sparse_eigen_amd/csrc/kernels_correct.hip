// Correction stage: "Partition the Support, Reconstruct the Residual" (gist.science
// summary), section 2B -- the fitted residual b' + x B' is added to every unprobed
// row's sparse output x; probe rows keep their exact dense output; rows go back to the
// original token order. fp32 arithmetic, output rounded once (bf16 nearest-even or fp32).
#include "kernels.h"

namespace spr {

template <int D>
__global__ __launch_bounds__(256) void k_correct(const float* __restrict__ o_s,
                                                 const float* __restrict__ bmat,
                                                 const float* __restrict__ bvec,
                                                 const float* __restrict__ od,
                                                 const int32_t* __restrict__ probe_of,
                                                 const int32_t* __restrict__ qperm, int n,
                                                 int probes, void* __restrict__ out, int out_f32) {
    constexpr int R = 32;                 // rows per block
    constexpr int XS = D + 1;             // padded row stride
    constexpr int PER = D / 8;            // outputs per thread
    __shared__ float bs[D * D];
    __shared__ float xs[R * XS];
    __shared__ float bv[D];
    const int h = blockIdx.y, tid = threadIdx.x;
    const int r0 = blockIdx.x * R;
    const float* bh = bmat + (size_t)h * D * D;
    for (int i = tid; i < D * D; i += 256) bs[i] = bh[i];
    for (int i = tid; i < D; i += 256) bv[i] = bvec[(size_t)h * D + i];
    for (int i = tid; i < R * D; i += 256) {
        const int r = i / D, j = i % D;
        xs[r * XS + j] = (r0 + r < n) ? o_s[((size_t)h * n + r0 + r) * D + j] : 0.f;
    }
    __syncthreads();
    const int r = tid >> 3, part = tid & 7;
    const int row = r0 + r;
    if (row >= n) return;
    float acc[PER];
#pragma unroll
    for (int m = 0; m < PER; ++m) acc[m] = 0.f;
    const float* xr = xs + r * XS;
    for (int i = 0; i < D; ++i) {
        const float xv = xr[i];
#pragma unroll
        for (int m = 0; m < PER; ++m) acc[m] = fmaf(xv, bs[i * D + part + 8 * m], acc[m]);
    }
    const int pi = probe_of[(size_t)h * n + row];
    const size_t dst = ((size_t)h * n + qperm[(size_t)h * n + row]) * D;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
        const int j = part + 8 * m;
        const float v = (pi >= 0) ? od[((size_t)h * probes + pi) * D + j] : (xr[j] + bv[j]) + acc[m];
        if (out_f32)
            static_cast<float*>(out)[dst + j] = v;
        else
            static_cast<bf16_t*>(out)[dst + j] = f32_to_bf16(v);
    }
}

void launch_correct(const float* o_s, const float* bmat, const float* bvec, const float* od,
                    const int32_t* probe_of, const int32_t* qperm, int heads, int n, int d,
                    int probes, void* o, int out_f32, hipStream_t st) {
    dim3 grid((n + 31) / 32, heads);
    if (d == 128)
        hipLaunchKernelGGL(k_correct<128>, grid, dim3(256), 0, st, o_s, bmat, bvec, od, probe_of, qperm,
                           n, probes, o, out_f32);
    else
        hipLaunchKernelGGL(k_correct<64>, grid, dim3(256), 0, st, o_s, bmat, bvec, od, probe_of, qperm,
                           n, probes, o, out_f32);
}

}  // namespace spr
