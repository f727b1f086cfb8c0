// Route-stage kernels.
//  * permute: contiguous group-major layout of Q/K/V ("Partition the Support,
//    Reconstruct the Residual", gist.science summary, section 2C), 16-byte row chunks
//  * route: centroid-logit top-k key groups per query group (block selection of
//    "Attention Sparsity is Input-Stable ... Online QK Co-Clustering", papernotes.org)
//  * probes: stratified probe rows across query groups (section 2B)
//  * units: query tiles of the attention kernel, one list per head
#include "kernels.h"

#include <algorithm>
#include <cmath>

namespace spr {

__global__ __launch_bounds__(256) void k_permute(const bf16_t* __restrict__ src,
                                                 const int32_t* __restrict__ perm, int n, int d,
                                                 bf16_t* __restrict__ dst) {
    const int h = blockIdx.y;
    const int chunks = d / 8;
    const size_t i = blockIdx.x * (size_t)256 + threadIdx.x;
    if (i >= (size_t)n * chunks) return;
    const int row = (int)(i / chunks), c = (int)(i % chunks);
    const int from = perm[(size_t)h * n + row];
    const uint4 v = *reinterpret_cast<const uint4*>(src + ((size_t)h * n + from) * d + c * 8);
    *reinterpret_cast<uint4*>(dst + ((size_t)h * n + row) * d + c * 8) = v;
}

void launch_permute(const bf16_t* src, const int32_t* perm, int heads, int n, int d, bf16_t* dst,
                    hipStream_t st) {
    const size_t total = (size_t)n * (d / 8);
    hipLaunchKernelGGL(k_permute, dim3((unsigned)((total + 255) / 256), heads), dim3(256), 0, st,
                       src, perm, n, d, dst);
}

// Largest |v| of each head as bf16 magnitude bits (vmax[h] must start at 0). Magnitude
// bits order like the magnitudes, so an integer maximum suffices.
__global__ __launch_bounds__(256) void k_absmax_bits(const bf16_t* __restrict__ src, size_t per_head,
                                                     uint32_t* __restrict__ vmax) {
    const int h = blockIdx.y;
    const uint4* p = reinterpret_cast<const uint4*>(src + (size_t)h * per_head);
    const size_t chunks = per_head / 8;
    uint32_t m = 0;
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < chunks; i += (size_t)gridDim.x * 256) {
        const uint4 v = p[i];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    }
    m = wave_max(m);
    __shared__ uint32_t s_m[4];
    if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) atomicMax(vmax + h, max(max(s_m[0], s_m[1]), max(s_m[2], s_m[3])));
}

// Group-major permute of V into fp16 scaled by 2^e(head) (exact for the scaled bf16 values
// above 2^-14; see v_scale_exp).
__global__ __launch_bounds__(256) void k_permute_f16(const bf16_t* __restrict__ src,
                                                     const int32_t* __restrict__ perm, int n, int d,
                                                     const uint32_t* __restrict__ vmax,
                                                     uint16_t* __restrict__ dst) {
    const int h = blockIdx.y;
    const int chunks = d / 8;
    const size_t i = blockIdx.x * (size_t)256 + threadIdx.x;
    if (i >= (size_t)n * chunks) return;
    const float scale = ldexpf(1.0f, v_scale_exp(vmax[h]));
    const int row = (int)(i / chunks), c = (int)(i % chunks);
    const int from = perm[(size_t)h * n + row];
    const uint4 v = *reinterpret_cast<const uint4*>(src + ((size_t)h * n + from) * d + c * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = pack_f16x2(bf16_to_f32((bf16_t)(w[j] & 0xFFFF)) * scale, bf16_to_f32((bf16_t)(w[j] >> 16)) * scale);
    *reinterpret_cast<uint4*>(dst + ((size_t)h * n + row) * d + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

// Group-major permute of K into FP8 E4M3 scaled by 2^e(head) (f8_scale_exp of the head's
// largest |k|): 16 values per thread, one 16-byte store.
__global__ __launch_bounds__(256) void k_permute_f8(const bf16_t* __restrict__ src,
                                                    const int32_t* __restrict__ perm, int n, int d,
                                                    const uint32_t* __restrict__ kmax,
                                                    uint8_t* __restrict__ dst) {
    const int h = blockIdx.y;
    const int chunks = d / 16;
    const size_t i = blockIdx.x * (size_t)256 + threadIdx.x;
    if (i >= (size_t)n * chunks) return;
    const float scale = ldexpf(1.0f, f8_scale_exp(kmax[h]));
    const int row = (int)(i / chunks), c = (int)(i % chunks);
    const int from = perm[(size_t)h * n + row];
    const bf16_t* s = src + ((size_t)h * n + from) * d + c * 16;
    const uint4 a = *reinterpret_cast<const uint4*>(s), b = *reinterpret_cast<const uint4*>(s + 8);
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        o[j] = pack_e4m3x4(bf16_to_f32((bf16_t)(w[2 * j] & 0xFFFF)) * scale,
                           bf16_to_f32((bf16_t)(w[2 * j] >> 16)) * scale,
                           bf16_to_f32((bf16_t)(w[2 * j + 1] & 0xFFFF)) * scale,
                           bf16_to_f32((bf16_t)(w[2 * j + 1] >> 16)) * scale);
    *reinterpret_cast<uint4*>(dst + ((size_t)h * n + row) * d + c * 16) = make_uint4(o[0], o[1], o[2], o[3]);
}

void launch_permute_k8(const bf16_t* src, const int32_t* perm, int heads, int n, int d, const uint32_t* kmax,
                       uint8_t* dst, hipStream_t st) {
    const size_t total = (size_t)n * (d / 16);
    hipLaunchKernelGGL(k_permute_f8, dim3((unsigned)((total + 255) / 256), heads), dim3(256), 0, st,
                       src, perm, n, d, kmax, dst);
}

void launch_absmax_v(const bf16_t* src, int heads, int n, int d, uint32_t* vmax, hipStream_t st) {
    launch_fill_i32(reinterpret_cast<int32_t*>(vmax), 0, heads, st);
    const size_t per_head = (size_t)n * d;
    const unsigned blocks = (unsigned)std::min<size_t>((per_head / 8 + 255) / 256, 256);
    hipLaunchKernelGGL(k_absmax_bits, dim3(blocks, heads), dim3(256), 0, st, src, per_head, vmax);
}

void launch_permute_f16(const bf16_t* src, const int32_t* perm, int heads, int n, int d,
                        const uint32_t* vmax, uint16_t* dst, hipStream_t st) {
    const size_t total = (size_t)n * (d / 8);
    hipLaunchKernelGGL(k_permute_f16, dim3((unsigned)((total + 255) / 256), heads), dim3(256), 0, st,
                       src, perm, n, d, vmax, dst);
}

void launch_permute_v16(const bf16_t* src, const int32_t* perm, int heads, int n, int d,
                        uint32_t* vmax, uint16_t* dst, hipStream_t st) {
    launch_absmax_v(src, heads, n, d, vmax, st);
    launch_permute_f16(src, perm, heads, n, d, vmax, dst, st);
}

// Coordinate-major copy [heads][d][g] of row-major fp64 rows [heads][g][d].
__global__ void k_transpose_f64(const double* __restrict__ src, int g, int d,
                                double* __restrict__ dst) {
    __shared__ double tile[32][33];
    const int h = blockIdx.z, r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;     // 32 x 8 threads
    const double* sh = src + (size_t)h * g * d;
    double* dh = dst + (size_t)h * d * g;
    for (int y = ty; y < 32; y += 8) {
        const int r = r0 + y, c = c0 + tx;
        tile[y][tx] = (r < g && c < d) ? sh[(size_t)r * d + c] : 0.0;
    }
    __syncthreads();
    for (int y = ty; y < 32; y += 8) {
        const int c = c0 + y, r = r0 + tx;                        // dst row c, column r
        if (c < d && r < g) dh[(size_t)c * g + r] = tile[tx][y];
    }
}

// Block per (kRouteGroups query groups, head). S_ij = c^Q_i . c^K_j / sqrt(d) in fp64 (a
// thread per key group, each query group's sum over the d coordinates in ascending order,
// reading the coordinate-major copy of the key centroids so that the lanes' loads coalesce,
// 16 at a time, each load serving all the block's query groups); key group j is kept when
// it is non-empty and fewer than k non-empty groups rank above it by (score descending,
// index ascending). Kept groups are written in ascending order (ballot compaction), and the
// union size is a block reduction.
constexpr int kRouteGroups = 4;

__global__ __launch_bounds__(256) void k_route(const double* __restrict__ cq,
                                               const double* __restrict__ ckt,
                                               const int32_t* __restrict__ qoff,
                                               const int32_t* __restrict__ koff, int gq, int gk,
                                               int d, int k, int32_t* __restrict__ blocks,
                                               int32_t* __restrict__ ucount,
                                               int64_t* __restrict__ pairs) {
    constexpr int QG = kRouteGroups;
    __shared__ double cs[QG][128];
    static_assert(QG % 2 == 0, "logits are read in pairs");
    __shared__ __align__(16) double sc[kMaxGroups][QG];     // a key group's logits side by side
    __shared__ int ne[kMaxGroups];
    __shared__ int wcnt[QG][4];
    __shared__ long long wsz[QG][4];
    const int h = blockIdx.y, i0 = blockIdx.x * QG, tid = threadIdx.x, lane = tid & 63,
              w = tid >> 6;
    const int nq = min(QG, gq - i0);
    for (int t = tid; t < QG * d; t += 256) {
        const int q = t / d, c = t - q * d;
        cs[q][c] = q < nq ? cq[((size_t)h * gq + i0 + q) * d + c] : 0.0;
    }
    __syncthreads();
    const int32_t* ko = koff + (size_t)h * (gk + 1);
    const double rs = sqrt((double)d);
    for (int j = tid; j < gk; j += 256) {
        const double* cj = ckt + (size_t)h * d * gk + j;          // coordinate t at cj[t * gk]
        double s[QG];
#pragma unroll
        for (int q = 0; q < QG; ++q) s[q] = 0.0;
        int t = 0;
        for (; t + 16 <= d; t += 16) {
            double cv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) cv[u] = cj[(size_t)(t + u) * gk];
#pragma unroll
            for (int u = 0; u < 16; ++u)
#pragma unroll
                for (int q = 0; q < QG; ++q) s[q] += cs[q][t + u] * cv[u];
        }
        for (; t < d; ++t) {
            const double cv = cj[(size_t)t * gk];
#pragma unroll
            for (int q = 0; q < QG; ++q) s[q] += cs[q][t] * cv;
        }
        // a NaN logit (non-finite centroids) ranks as -inf, so (score, index) stays a total
        // order and exactly min(k, non-empty) groups are kept
#pragma unroll
        for (int q = 0; q < QG; ++q) sc[j][q] = isnan(s[q]) ? -INFINITY : s[q] / rs;
        ne[j] = (ko[j + 1] > ko[j]) ? 1 : 0;
    }
    __syncthreads();
    // The block's query groups are ranked together: one pass over t serves all of them.
    int base[QG];
    long long u[QG];
#pragma unroll
    for (int q = 0; q < QG; ++q) {
        base[q] = 0;
        u[q] = 0;
    }
    for (int j0 = 0; j0 < gk; j0 += 256) {
        const int j = j0 + tid;
        bool keep[QG];
#pragma unroll
        for (int q = 0; q < QG; ++q) keep[q] = false;
        if (j < gk && ne[j]) {
            double sj[QG];
            int rank[QG];
#pragma unroll
            for (int q = 0; q < QG; ++q) {
                sj[q] = sc[j][q];
                rank[q] = 0;
            }
            for (int t = 0; t < gk; ++t) {
                if (!ne[t]) continue;
#pragma unroll
                for (int q = 0; q < QG; q += 2) {
                    const double2 st = *reinterpret_cast<const double2*>(&sc[t][q]);
                    rank[q] += (st.x > sj[q] || (st.x == sj[q] && t < j)) ? 1 : 0;
                    rank[q + 1] += (st.y > sj[q + 1] || (st.y == sj[q + 1] && t < j)) ? 1 : 0;
                }
            }
#pragma unroll
            for (int q = 0; q < QG; ++q) keep[q] = rank[q] < k;
        }
        const int nk = (j < gk) ? ko[j + 1] - ko[j] : 0;
        uint64_t m[QG];
#pragma unroll
        for (int q = 0; q < QG; ++q) {
            if (keep[q]) u[q] += nk;
            m[q] = __ballot(keep[q]);
            if (lane == 0) wcnt[q][w] = __popcll(m[q]);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < QG; ++q) {
            int before = 0, total = 0;
            for (int r = 0; r < 4; ++r) {
                before += (r < w) ? wcnt[q][r] : 0;
                total += wcnt[q][r];
            }
            if (keep[q] && q < nq)
                blocks[((size_t)h * gq + i0 + q) * k + base[q] + before +
                       __popcll(m[q] & ((1ull << lane) - 1))] = j;
            base[q] += total;
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < QG; ++q) {
        if (q < nq)
            for (int p = base[q] + tid; p < k; p += 256) blocks[((size_t)h * gq + i0 + q) * k + p] = -1;
        for (int o = 32; o > 0; o >>= 1) u[q] += __shfl_xor(u[q], o, 64);
        if (lane == 0) wsz[q][w] = u[q];
    }
    __syncthreads();
    if (tid < nq) {
        const int i = i0 + tid;
        const long long us = wsz[tid][0] + wsz[tid][1] + wsz[tid][2] + wsz[tid][3];
        const int32_t* qo = qoff + (size_t)h * (gq + 1);
        ucount[(size_t)h * gq + i] = (int32_t)us;
        atomicAdd(reinterpret_cast<unsigned long long*>(&pairs[h]),
                  (unsigned long long)(us * (int64_t)(qo[i + 1] - qo[i])));
    }
}

void launch_route(const double* cq, const double* ck, double* ck_t, const int32_t* qoff,
                  const int32_t* koff, int heads, int gq, int gk, int d, int k, int32_t* blocks,
                  int32_t* ucount, int64_t* pairs, hipStream_t st) {
    hipLaunchKernelGGL(k_transpose_f64, dim3((d + 31) / 32, (gk + 31) / 32, heads), dim3(256), 0, st,
                       ck, gk, d, ck_t);
    hipLaunchKernelGGL(k_route, dim3((gq + kRouteGroups - 1) / kRouteGroups, heads), dim3(256), 0,
                       st, cq, ck_t, qoff, koff, gq, gk, d, k, blocks, ucount, pairs);
}

// Block per head. m_i = floor(P n_i / N); the leftover P - sum m_i go one each to the
// groups of largest remainder (P n_i mod N), lower index first; the probes of group i
// sit at ranks floor((2t + 1) n_i / (2 m_i)), t < m_i.
__global__ __launch_bounds__(1024) void k_probes(const int32_t* __restrict__ qoff,
                                                 const int32_t* __restrict__ qperm, int n, int gq,
                                                 int probes, int32_t* __restrict__ probe_pos,
                                                 int32_t* __restrict__ probe_orig,
                                                 int32_t* __restrict__ probe_grp,
                                                 int32_t* __restrict__ probe_of) {
    __shared__ int64_t rem[kMaxGroups];
    __shared__ int m[kMaxGroups];
    __shared__ int base[kMaxGroups];
    __shared__ int wtot[16];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    // exclusive prefix of v over the block's threads (gq <= 1024 = blockDim); all threads
    auto block_scan = [&](int v, int& total) {
        int inc = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(inc, o, 64);
            if (lane >= o) inc += t;
        }
        __syncthreads();
        if (lane == 63) wtot[w] = inc;
        __syncthreads();
        int wb = 0;
        total = 0;
        for (int k = 0; k < 16; ++k) {
            wb += (k < w) ? wtot[k] : 0;
            total += wtot[k];
        }
        return wb + inc - v;
    };
    const int32_t* qo = qoff + (size_t)h * (gq + 1);
    if (probes == 0) return;
    for (int i = tid; i < gq; i += 1024) {
        const int64_t ni = qo[i + 1] - qo[i];
        m[i] = (int)((probes * ni) / n);
        rem[i] = (probes * ni) % n;
    }
    __syncthreads();
    int msum;
    (void)block_scan(tid < gq ? m[tid] : 0, msum);
    const int left = probes - msum;
    for (int i = tid; i < gq; i += 1024) {
        int rank = 0;
        const int64_t ri = rem[i];
        for (int t = 0; t < gq; ++t) rank += (rem[t] > ri || (rem[t] == ri && t < i)) ? 1 : 0;
        if (rank < left) m[i] += 1;
    }
    __syncthreads();
    int mtot;
    const int b0 = block_scan(tid < gq ? m[tid] : 0, mtot);
    if (tid < gq) base[tid] = b0;
    __syncthreads();
    for (int i = tid; i < gq; i += 1024) {
        const int64_t ni = qo[i + 1] - qo[i];
        const int mi = m[i];
        for (int t = 0; t < mi; ++t) {
            const int pos = qo[i] + (int)(((2 * (int64_t)t + 1) * ni) / (2 * (int64_t)mi));
            const int idx = base[i] + t;
            probe_pos[(size_t)h * probes + idx] = pos;
            probe_orig[(size_t)h * probes + idx] = qperm[(size_t)h * n + pos];
            probe_grp[(size_t)h * probes + idx] = i;
            probe_of[(size_t)h * n + pos] = idx;
        }
    }
}

void launch_probes(const int32_t* qoff, const int32_t* qperm, int heads, int n, int gq, int probes,
                   int32_t* probe_pos, int32_t* probe_orig, int32_t* probe_grp, int32_t* probe_of,
                   hipStream_t st) {
    hipLaunchKernelGGL(k_probes, dim3(heads), dim3(1024), 0, st, qoff, qperm, n, gq, probes,
                       probe_pos, probe_orig, probe_grp, probe_of);
}

// Block per head: query tiles of `rows_per_unit` rows inside each query group.
// exclusive prefix over the block of one count per thread (wave scans, then a scan of the
// wave totals); `wtot` holds 16 ints, `total` gets the block's sum
__device__ inline int block_exclusive_scan(int cnt, int* wtot, int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    __syncthreads();                                  // earlier readers of wtot are done
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    int wb = 0;
    total = 0;
    for (int k = 0; k < 16; ++k) {
        wb += (k < w) ? wtot[k] : 0;
        total += wtot[k];
    }
    return wb + inc - cnt;
}

// Work units of the attention kernels: (query group, first row). With big_rows > 0 every
// whole big_rows-row chunk of a group is one unit of the big list, and so is a rest of more
// than rows_per_unit rows (a partial unit: it fills as many wave slots as the two small units
// it replaces, and walks the group's routed keys once instead of twice); a shorter rest is
// one unit of the other list. With big_rows = 0 the whole group is cut into
// rows_per_unit-row units. Units of one group are consecutive in each list.
__global__ __launch_bounds__(1024) void k_units(const int32_t* __restrict__ qoff, int gq,
                                                int rows_per_unit, int max_units,
                                                int2* __restrict__ units,
                                                int32_t* __restrict__ nunits, int big_rows,
                                                int max_big, int2* __restrict__ units_big,
                                                int32_t* __restrict__ nunits_big) {
    __shared__ int wtot[16];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int32_t* qo = qoff + (size_t)h * (gq + 1);
    // gq <= 1024 = blockDim: one group per thread
    const int rows = (tid < gq) ? qo[tid + 1] - qo[tid] : 0;
    int nb = big_rows > 0 ? rows / big_rows : 0;
    int rest = rows - nb * big_rows;
    if (big_rows > 0 && rest > rows_per_unit) {
        ++nb;
        rest = 0;
    }
    const int ns = (rest + rows_per_unit - 1) / rows_per_unit;
    int tot_s = 0, tot_b = 0;
    const int bs = block_exclusive_scan(ns, wtot, tot_s);
    const int bb = block_exclusive_scan(nb, wtot, tot_b);
    if (tid == 0) {
        nunits[h] = tot_s;
        if (big_rows > 0) nunits_big[h] = tot_b;
    }
    if (tid < gq) {
        for (int t = 0; t < nb; ++t)
            units_big[(size_t)h * max_big + bb + t] = make_int2(tid, qo[tid] + t * big_rows);
        const int r0 = qo[tid] + rows - rest;
        for (int t = 0; t < ns; ++t)
            units[(size_t)h * max_units + bs + t] = make_int2(tid, r0 + t * rows_per_unit);
    }
}

void launch_units(const int32_t* qoff, int heads, int gq, int rows_per_unit, int max_units,
                  int2* units, int32_t* nunits, hipStream_t st, int big_rows, int max_big,
                  int2* units_big, int32_t* nunits_big) {
    hipLaunchKernelGGL(k_units, dim3(heads), dim3(1024), 0, st, qoff, gq, rows_per_unit, max_units,
                       units, nunits, big_rows, max_big, units_big, nunits_big);
}

}  // namespace spr
