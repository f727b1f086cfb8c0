// Leading eigenpairs of the key metric on the device (fp64), for the key coordinates
// W = U_r diag(sqrt(lambda_r)) of "Partition the Support, Reconstruct the Residual"
// (gist.science summary), section 2A: keys are clustered on the leading eigenvectors of
// M_K = Q_s^T Q_s / M_s. Every head is independent; nothing leaves the device.
//
//   k_tridiag     Householder reduction A = Q T Q^T, one 1024-thread block per head. The
//                 matrix stays in registers (eight lanes hold the 128 columns of a row, 16
//                 each), and the row that holds the column being reduced builds the
//                 reflector itself, so a step needs two barriers and eight-lane reductions.
//   k_tri_eigpair one block per (eigenvalue, head): bisection on Sturm counts at 256 points
//                 a round (eight bits a round); for the leading r also the eigenvector of T
//                 from one twisted factorisation of T - lambda I (Parlett and Dhillon's
//                 single-vector step of the MRRR method; two lanes, one pass each).
//   k_eig_finish  one block per head: later members of a cluster of near-equal eigenvalues
//                 by inverse iteration against the earlier ones, the reflectors applied back
//                 to give eigenvectors of M_K, W and the gap lambda_r / lambda_{r+1}.
// Latency, not arithmetic, bounds all three (in k_tridiag also the LDS reads of v and p by
// every lane), hence the barrier-light forms and the skipped dead rows and columns.
#include "kernels.h"

#include <cfloat>

namespace spr {

namespace {

constexpr int kTriThreads = 1024;      // k_tridiag: eight lanes per row of a 128-wide matrix
constexpr int kEigThreads = 256;       // k_tri_eigpair: bisection points per round

// Sum / min / max over the block; every thread gets the same value (the per-wave partials
// are combined in wave order). `red` holds one double per wave.
template <int NT, int OP>
__device__ inline double block_reduce(double v, double* red) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double u = __shfl_xor(v, o, 64);
        v = OP == 0 ? v + u : (OP == 1 ? fmin(v, u) : fmax(v, u));
    }
    __syncthreads();                                  // earlier readers of red are done
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = red[0];
    for (int w = 1; w < NT / 64; ++w) s = OP == 0 ? s + red[w] : (OP == 1 ? fmin(s, red[w]) : fmax(s, red[w]));
    return s;
}

// Data-parallel lane moves of a double (two 32-bit DPP moves).
template <int CTRL>
__device__ inline double dpp_move(double v) {
    int2 p = __builtin_bit_cast(int2, v);
    p.x = __builtin_amdgcn_mov_dpp(p.x, CTRL, 0xF, 0xF, false);
    p.y = __builtin_amdgcn_mov_dpp(p.y, CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, p);
}
// sum over the four lanes of a quad (lanes 4q .. 4q+3), the same in every lane
__device__ inline double quad_sum(double v) {
    v += dpp_move<0xB1>(v);                          // quad_perm [1,0,3,2]
    return v + dpp_move<0x4E>(v);                    // quad_perm [2,3,0,1]
}
// v_l + v_(l^W) (W = 16: permlane16 swap, W = 32: permlane32 swap): the swap returns the
// pair {v_l, v_(l^W)} in some order, and the sum is the same in both lanes
template <int W>
__device__ inline double lane_pair_sum(double v) {
    const uint2 u = __builtin_bit_cast(uint2, v);
    uint2 a0, a1;
    if constexpr (W == 16) {
        const auto lo = __builtin_amdgcn_permlane16_swap(u.x, u.x, false, false);
        const auto hi = __builtin_amdgcn_permlane16_swap(u.y, u.y, false, false);
        a0 = make_uint2(lo[0], hi[0]);
        a1 = make_uint2(lo[1], hi[1]);
    } else {
        const auto lo = __builtin_amdgcn_permlane32_swap(u.x, u.x, false, false);
        const auto hi = __builtin_amdgcn_permlane32_swap(u.y, u.y, false, false);
        a0 = make_uint2(lo[0], hi[0]);
        a1 = make_uint2(lo[1], hi[1]);
    }
    return __builtin_bit_cast(double, a0) + __builtin_bit_cast(double, a1);
}
// sum over the 64 lanes of the wave, the same in every lane
__device__ inline double wave_sum_f64(double v) {
    v = quad_sum(v);
    v += dpp_move<0x141>(v);                         // row_half_mirror: the other quad of 8
    v += dpp_move<0x140>(v);                         // row_mirror: the other 8 of 16
    v = lane_pair_sum<16>(v);                         // the other row of 16 in each 32
    return lane_pair_sum<32>(v);                      // the other half of the wave
}

// 1/q to about one ulp: the hardware reciprocal refined by two Newton steps
__device__ inline double recip(double q) {
    double r = __builtin_amdgcn_rcp(q);
    double e = fma(-q, r, 1.0);
    r = fma(r, e, r);
    e = fma(-q, r, 1.0);
    return fma(r, e, r);
}
// 1/q to about 2^-46 relative (one Newton step): enough for a Sturm count, whose
// perturbation then equals a relative change of about 2^-46 in the off-diagonal squares
__device__ inline double recip_sturm(double q) {
    const double r = __builtin_amdgcn_rcp(q);
    return fma(r, fma(-q, r, 1.0), r);
}
// sum of squares of s[0 .. n) in four partial sums (the loads batch)
__device__ inline double sumsq(const double* s, int n) {
    double t[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int i = 0; i < n; ++i) t[i & 3] = fma(s[i], s[i], t[i & 3]);
    return (t[0] + t[1]) + (t[2] + t[3]);
}

// ------------------------------------------------------------- tridiagonal ---
// H_k = I - beta_k v_k v_k^T acts on rows k+1 .. n-1 (v_k in hv[k][0 .. n-k-2]); beta_k = 0
// marks a column that needed no reflection. Rows and columns past n are zero padding.
//
// Step k reduces column k, which (A symmetric) is row k past the diagonal. The eight lanes
// of row k publish v_k (and beta_k) to LDS as the last act of step k - 1, right after their
// own update, so each step is: barrier, A v, barrier, the rank-two update.
namespace {
constexpr int kTriLanes = 8;                    // lanes per matrix row
constexpr int kTriCols = kEigMaxN / kTriLanes;  // columns per lane

struct RowPub {
    double beta, off;            // beta_k, T[k+1][k]
};

// sum over the eight lanes of a row group (lanes 8q .. 8q+7), the same in every lane
__device__ inline double oct_sum(double v) {
    v = quad_sum(v);
    return v + dpp_move<0x141>(v);                   // row_half_mirror: the other quad of 8
}

// The lanes of row k: v_k = (0 .. 0, u0 at k+1, the row past k+1) into x, the scalars into
// pub. raw (kEigMaxN doubles) takes the row as it stands, so that its entry at k+1 is one
// LDS read away (the row's lanes share a wave: their LDS writes precede the read).
__device__ inline void publish_row(const double (&a)[kTriCols], int c0, int k, int n, double* x,
                                   double* raw, RowPub* pub, bool lead) {
    const int o = k + 1;
#pragma unroll
    for (int j = 0; j < kTriCols; j += 2)
        *reinterpret_cast<double2*>(&raw[c0 + j]) = make_double2(a[j], a[j + 1]);
    // bit j: column c0 + j lies past k+1 (in the reflector's tail)
    const int sh = o + 1 - c0;
    const uint32_t tailm = sh <= 0 ? 0xFFFFu : (sh >= kTriCols ? 0u : (0xFFFFu << sh) & 0xFFFFu);
    double t[4] = {0.0, 0.0, 0.0, 0.0}, v[kTriCols];
#pragma unroll
    for (int j = 0; j < kTriCols; ++j) {
        v[j] = ((tailm >> j) & 1u) ? a[j] : 0.0;
        t[j & 3] = fma(v[j], v[j], t[j & 3]);
    }
#pragma unroll
    for (int j = 0; j < kTriCols; j += 2)
        *reinterpret_cast<double2*>(&x[c0 + j]) = make_double2(v[j], v[j + 1]);
    const double tail2 = oct_sum((t[0] + t[1]) + (t[2] + t[3]));
    __builtin_amdgcn_s_waitcnt(0xc07f);               // lgkmcnt(0): this wave's raw row is in LDS
    const double v0 = raw[o];
    double u0 = v0, beta = 0.0, offk = v0;
    if (tail2 > 0.0) {
        const double sigma = sqrt(v0 * v0 + tail2);
        const double alpha = (v0 >= 0.0) ? -sigma : sigma;
        u0 = v0 - alpha;
        beta = 2.0 / (tail2 + u0 * u0);
        offk = alpha;
    }
    if (o >= c0 && o < c0 + kTriCols) x[o] = u0;     // after this lane's tail stores
    if (lead) *pub = RowPub{beta, offk};
}
}  // namespace

__global__ __launch_bounds__(kTriThreads) void k_tridiag(const double* __restrict__ mk, int n,
                                                         double* __restrict__ diag,
                                                         double* __restrict__ off,
                                                         double* __restrict__ hv,
                                                         double* __restrict__ hbeta) {
    constexpr int CW = kTriCols;
    __shared__ __attribute__((aligned(16))) double s_v[2][kEigMaxN];    // v_k, by step parity
    __shared__ __attribute__((aligned(16))) double s_p[2][kEigMaxN];
    __shared__ RowPub s_pub[2];
    __shared__ __attribute__((aligned(16))) double s_raw[kEigMaxN];       // the publishing row as is
    // reflectors, betas and off-diagonal kept in LDS until the end (a barrier also waits for
    // a thread's outstanding global stores, so none are issued inside the loop)
    __shared__ double s_hv[kEigMaxN * kEigMaxN];
    __shared__ double s_hb[kEigMaxN], s_of[kEigMaxN];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int R = tid / kTriLanes, c0 = (tid % kTriLanes) * CW;
    const bool lead = (tid % kTriLanes) == 0;
    const double* m = mk + (size_t)h * n * n;
    double* dg = diag + (size_t)h * n;
    double a[CW];
#pragma unroll
    for (int j = 0; j < CW; ++j) a[j] = (R < n && c0 + j < n) ? m[(size_t)R * n + c0 + j] : 0.0;
    for (int i = tid; i < 2 * kEigMaxN; i += kTriThreads) s_p[i / kEigMaxN][i % kEigMaxN] = 0.0;
    __syncthreads();
    if (R == 0 && n > 2) publish_row(a, c0, 0, n, s_v[0], s_raw, &s_pub[0], lead);
    for (int k = 0; k + 2 < n; ++k) {
        const int o = k + 1, buf = k & 1;
        __syncthreads();                              // v_k and its scalars are published
        const RowPub pub = s_pub[buf];
        if (tid < kEigMaxN) {                         // the reflector and T's entries (off the chain)
            if (tid >= o && tid < n) s_hv[k * n + (tid - o)] = s_v[buf][tid];
            if (tid == 0) {
                s_hb[k] = pub.beta;
                s_of[k] = pub.off;
            }
        }
        const bool live = R > k && R < n;             // rows of the trailing block
        // A wave whose eight rows are all at or above row k sits the step out, and a lane
        // whose sixteen columns are all at or left of column k reads nothing: v and p vanish
        // there, and the LDS traffic of the two vector reads is what bounds a step.
        const bool wave_live = (8 * (tid >> 6) + 7 > k) && (8 * (tid >> 6) < n);
        const bool cols_live = c0 + CW > o;
        if (pub.beta != 0.0) {
            double v[CW];
            double p4[4] = {0.0, 0.0, 0.0, 0.0}, pr = 0.0;
            if (wave_live) {
#pragma unroll
                for (int j = 0; j < CW; ++j) v[j] = 0.0;
                if (cols_live) {
#pragma unroll
                    for (int j = 0; j < CW; j += 2) {
                        const double2 t = *reinterpret_cast<const double2*>(&s_v[buf][c0 + j]);
                        v[j] = t.x;
                        v[j + 1] = t.y;
                    }
                }
                // p_R = beta (A v)_R, the row's eight lanes summed
                if (live && cols_live) {
#pragma unroll
                    for (int j = 0; j < CW; ++j) p4[j & 3] = fma(a[j], v[j], p4[j & 3]);
                }
                pr = oct_sum((p4[0] + p4[1]) + (p4[2] + p4[3])) * pub.beta;
                if (lead && R < kEigMaxN) s_p[buf][R] = pr;
            }
            __syncthreads();
            // the wave of row k+1 is the step's critical path: it issues first on its SIMD
            if ((tid >> 6) == ((k + 1) >> 3)) __builtin_amdgcn_s_setprio(3);
            // kk = beta/2 v.p (each live row's lanes sum all 128 terms), w = p - kk v,
            // A -= v w^T + w v^T (v and w vanish outside the trailing block; p is zero at
            // rows at or above k, which either wrote zero or hold a finite earlier value in
            // a column whose v is zero)
            if (live) {
                double pc[CW], q4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int j = 0; j < CW; ++j) pc[j] = 0.0;
                if (cols_live) {
#pragma unroll
                    for (int j = 0; j < CW; j += 2) {
                        const double2 t = *reinterpret_cast<const double2*>(&s_p[buf][c0 + j]);
                        pc[j] = t.x;
                        pc[j + 1] = t.y;
                    }
                }
#pragma unroll
                for (int j = 0; j < CW; ++j) q4[j & 3] = fma(v[j], pc[j], q4[j & 3]);
                const double kk = 0.5 * pub.beta * oct_sum((q4[0] + q4[1]) + (q4[2] + q4[3]));
                const double vR = s_v[buf][R];
                // a - vR (p_c - kk v_c) - (p_R - kk vR) v_c = a - vR p_c + (2 kk vR - p_R) v_c
                const double g = 2.0 * kk * vR - pr;
#pragma unroll
                for (int j = 0; j < CW; ++j) a[j] = fma(g, v[j], fma(-vR, pc[j], a[j]));
            }
        }
        // row k+1 publishes v_{k+1} for the next step (into the other buffers)
        if (R == k + 1 && k + 3 < n) publish_row(a, c0, k + 1, n, s_v[buf ^ 1], s_raw, &s_pub[buf ^ 1], lead);
        __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    if (tid == 0) {                                   // entries no step writes
        s_of[n - 1] = 0.0;
        for (int k = n - 2 > 0 ? n - 2 : 0; k < n; ++k) s_hb[k] = 0.0;
    }
#pragma unroll
    for (int j = 0; j < CW; ++j) {
        if (R < n && c0 + j == R) dg[R] = a[j];
        if (n >= 2 && R == n - 1 && c0 + j == n - 2) s_of[n - 2] = a[j];
    }
    __syncthreads();
    double* of = off + (size_t)h * n;
    double* hb = hbeta + (size_t)h * n;
    double* hvh = hv + (size_t)h * n * n;
    for (int i = tid; i < n; i += kTriThreads) {
        of[i] = s_of[i];
        hb[i] = s_hb[i];
    }
    // reflector k has n - k - 1 entries (rows past it are never read)
    for (int e = tid; e < (n - 2) * n; e += kTriThreads) hvh[e] = s_hv[e];
}

// ----------------------------------------------------------- eigenpairs of T ---
// Block (j, h): the j-th largest eigenvalue of head h's T (ascending rank n-1-j); for j < r
// also its eigenvector of T, from the twisted factorisation of T - lambda I (the vector is
// z_t = 1 at the twist t where |gamma_t| is least, the rest by the two pivot ratios). tnorm[h]
// (block j = 0) is the Gershgorin bound on |T|.
__global__ __launch_bounds__(kEigThreads) void k_tri_eigpair(const double* __restrict__ diag,
                                                             const double* __restrict__ off,
                                                             int n, int r, int ne,
                                                             double* __restrict__ lam_out,
                                                             double* __restrict__ vec_out,
                                                             double* __restrict__ tnorm_out) {
    constexpr int NT = kEigThreads;
    __shared__ double s_d[kEigMaxN], s_e[kEigMaxN], s_e2[kEigMaxN];
    __shared__ double s_dp[kEigMaxN], s_dm[kEigMaxN];      // pivots of L D L^T, U D U^T
    __shared__ double s_rp[kEigMaxN], s_rm[kEigMaxN];      // -e_i / D+_i, -e_i / D-_{i+1}
    __shared__ double s_z[kEigMaxN];
    __shared__ double s_red[NT / 64];
    __shared__ int s_first[NT / 64];
    __shared__ int s_twist;
    const int j = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    for (int i = tid; i < n; i += NT) {
        s_d[i] = diag[(size_t)h * n + i];
        s_e[i] = (i + 1 < n) ? off[(size_t)h * n + i] : 0.0;
    }
    __syncthreads();
    double glo = INFINITY, ghi = -INFINITY, tn = 0.0;
    for (int i = tid; i < n; i += NT) {
        s_e2[i] = (i > 0) ? s_e[i - 1] * s_e[i - 1] : 0.0;
        const double rad = (i > 0 ? fabs(s_e[i - 1]) : 0.0) + fabs(s_e[i]);
        glo = fmin(glo, s_d[i] - rad);
        ghi = fmax(ghi, s_d[i] + rad);
        tn = fmax(tn, fabs(s_d[i]) + rad);
    }
    glo = block_reduce<NT, 1>(glo, s_red);
    ghi = block_reduce<NT, 2>(ghi, s_red);
    tn = block_reduce<NT, 2>(tn, s_red);
    if (tid == 0 && j == 0) tnorm_out[h] = tn;
    double* vec = vec_out + ((size_t)h * r + j) * n;
    if (!(tn > 0.0)) {                                // zero matrix: unit vectors
        if (tid == 0) lam_out[(size_t)h * ne + j] = 0.0;
        if (j < r)
            for (int i = tid; i < n; i += NT) vec[i] = (i == j) ? 1.0 : 0.0;
        return;
    }
    const double pivmin = DBL_MIN * fmax(1.0, tn * tn);
    const double pad = 2.0 * DBL_EPSILON * tn * n + pivmin;
    double lo = glo - pad, hi = ghi + pad;
    const int rank = n - 1 - j;                       // count(lo) <= rank < count(hi)
    // point t of a round sits at lo + (hi - lo) t / (NT + 1); the same product gives the
    // new ends, so the new interval is exactly two adjacent points of the old one
    constexpr double kStep = 1.0 / (NT + 1);
    const double my_frac = (double)(tid + 1) * kStep;
    for (int round = 0; round < 12; ++round) {
        const double x = lo + (hi - lo) * my_frac;
        double q = s_d[0] - x;
        if (fabs(q) < pivmin) q = -pivmin;
        int c = q < 0.0 ? 1 : 0;
        for (int i = 1; i < n; ++i) {
            q = (s_d[i] - x) - s_e2[i] * recip_sturm(q);
            if (fabs(q) < pivmin) q = -pivmin;
            c += q < 0.0 ? 1 : 0;
        }
        const unsigned long long b = __ballot(c > rank);
        __syncthreads();                              // earlier readers of s_first are done
        if ((tid & 63) == 0) s_first[tid >> 6] = b ? (tid + __ffsll(b) - 1) : NT;
        __syncthreads();
        int first = NT;
        for (int w = 0; w < NT / 64; ++w) first = min(first, s_first[w]);
        const double nlo = first > 0 ? lo + (hi - lo) * ((double)first * kStep) : lo;
        const double nhi = first < NT ? lo + (hi - lo) * ((double)(first + 1) * kStep) : hi;
        lo = nlo;
        hi = nhi;
        if (hi - lo <= 2.0 * DBL_EPSILON * fmax(fabs(lo), fabs(hi)) + pivmin) break;
    }
    const double lam = 0.5 * (lo + hi);
    if (tid == 0) lam_out[(size_t)h * ne + j] = lam;
    if (j >= r) return;
    // pivots of T - lam I = L+ D+ L+^T (lane 0, downward) and U- D- U-^T (lane 1, upward), the
    // ratios the vector needs, and gamma_t = D+_t + D-_t - (d_t - lam)
    if (tid == 0) {
        double dp = s_d[0] - lam;
        if (fabs(dp) < pivmin) dp = -pivmin;
        s_dp[0] = dp;
        double e0 = s_e[0], d1 = (n > 1 ? s_d[1] : 0.0) - lam;
        for (int i = 0; i + 1 < n; ++i) {
            const double e1 = s_e[i + 1], d2 = (i + 2 < n ? s_d[i + 2] : 0.0) - lam;   // next step's
            const double rp = recip(dp);
            s_rp[i] = -e0 * rp;
            dp = d1 - e0 * e0 * rp;
            if (fabs(dp) < pivmin) dp = -pivmin;
            s_dp[i + 1] = dp;
            e0 = e1;
            d1 = d2;
        }
    } else if (tid == 1) {
        double dm = s_d[n - 1] - lam;
        if (fabs(dm) < pivmin) dm = -pivmin;
        s_dm[n - 1] = dm;
        double e0 = n > 1 ? s_e[n - 2] : 0.0, d1 = (n > 1 ? s_d[n - 2] : 0.0) - lam;
        for (int i = n - 2; i >= 0; --i) {
            const double e1 = i > 0 ? s_e[i - 1] : 0.0, d2 = (i > 0 ? s_d[i - 1] : 0.0) - lam;
            const double rm = recip(dm);
            s_rm[i] = -e0 * rm;                       // z_{i+1} = s_rm[i] z_i
            dm = d1 - e0 * e0 * rm;
            if (fabs(dm) < pivmin) dm = -pivmin;
            s_dm[i] = dm;
            e0 = e1;
            d1 = d2;
        }
    }
    __syncthreads();
    if (tid < 64) {                                   // the twist: least |gamma_t|, lowest t on ties
        int best = n;
        double gbest = INFINITY;
        for (int t = tid; t < n; t += 64) {
            const double g = fabs(s_dp[t] + s_dm[t] - (s_d[t] - lam));
            if (g < gbest || best == n) {
                gbest = g;
                best = t;
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const double og = __shfl_xor(gbest, o, 64);
            const int ob = __shfl_xor(best, o, 64);
            if (og < gbest || (og == gbest && ob < best)) {
                gbest = og;
                best = ob;
            }
        }
        if (tid == 0) s_twist = best < n ? best : 0;
    }
    __syncthreads();
    const int tw = s_twist;
    if (tid == 0) {                                   // z_i = (-e_i / D+_i) z_{i+1} above the twist
        double z = 1.0;
        s_z[tw] = 1.0;
        for (int i = tw - 1; i >= 0; --i) {
            z *= s_rp[i];
            s_z[i] = z;
        }
    } else if (tid == 1) {                            // z_{i+1} = (-e_i / D-_{i+1}) z_i below it
        double z = 1.0;
        for (int i = tw; i + 1 < n; ++i) {
            z *= s_rm[i];
            s_z[i + 1] = z;
        }
    }
    __syncthreads();
    if (tid < 64) {
        double sq = 0.0;
        for (int i = tid; i < n; i += 64) sq = fma(s_z[i], s_z[i], sq);
        const double inv = 1.0 / sqrt(wave_sum_f64(sq));
        for (int i = tid; i < n; i += 64) vec[i] = s_z[i] * inv;
    }
}

// ------------------------------------------------------------------ finish ---
// Eigenvalues closer than 1e-7 |T| form a cluster. The twisted vector of a later member can
// repeat an earlier member's (a multiple eigenvalue of a split T), so a later member is
// taken instead by inverse iteration (two solves with T - lambda I, LU with partial
// pivoting) from a fixed pseudo-random start, orthogonalised against the earlier members
// (Gram-Schmidt, twice) before each solve and after the last. Outside a cluster the twisted
// vectors are orthogonal to about eps |T| / gap along a direction whose weight in W W^T
// differs by the gap itself, so W W^T is off by about eps |T|. Then the reflectors are
// applied back (X = H_0 (H_1 (... H_{n-3} Y))): sixteen lanes carry two vectors, eight
// rows per lane, reflectors staged in LDS sixteen at a time.
// Finally W = X diag(sqrt(max(lambda, 0))) and the gap.
constexpr int kFinThreads = 1024;      // r <= 64 needs 512 lanes for the back-transform
constexpr int kReflStage = 16;

// a fixed start vector entry in [-1, 1) (an integer hash of the row and the vector)
__device__ inline double start_entry(int i, int jj) {
    uint32_t x = (uint32_t)(i + 1) * 0x9E3779B1u ^ (uint32_t)(jj + 1) * 0x85EBCA77u;
    x ^= x >> 15;
    x *= 0x2C1B3C6Du;
    x ^= x >> 12;
    x *= 0x297A2D39u;
    x ^= x >> 15;
    return (double)(x >> 8) * 0x1p-23 - 1.0;
}

__global__ __launch_bounds__(kFinThreads) void k_eig_finish(const double* __restrict__ diag,
                                                            const double* __restrict__ off,
                                                            const double* __restrict__ hv,
                                                            const double* __restrict__ hbeta,
                                                            const double* __restrict__ lam,
                                                            const double* __restrict__ vec,
                                                            const double* __restrict__ tnorm,
                                                            int n, int r, int ne,
                                                            double* __restrict__ w_out,
                                                            double* __restrict__ gap_out) {
    constexpr int NT = kFinThreads;
    constexpr int RPL = kEigMaxN / 16;                // rows per lane
    __shared__ double s_x[kEigMaxN * kEigMaxR];       // [i][j], pitch r
    __shared__ double s_hv[kReflStage][kEigMaxN];
    __shared__ double s_hb[kReflStage];
    __shared__ double s_dot[kEigMaxR];
    __shared__ double s_lam[kEigMaxR + 1];
    __shared__ double s_red[NT / 64];
    __shared__ double s_d[kEigMaxN], s_e[kEigMaxN];
    __shared__ double s_u0[kEigMaxN], s_u1[kEigMaxN], s_u2[kEigMaxN];
    const int h = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < n * r; e += NT) {
        const int jj = e / n, i = e - jj * n;
        s_x[i * r + jj] = vec[((size_t)h * r + jj) * n + i];
    }
    for (int jj = tid; jj < ne; jj += NT) s_lam[jj] = lam[(size_t)h * ne + jj];
    for (int i = tid; i < n; i += NT) {
        s_d[i] = diag[(size_t)h * n + i];
        s_e[i] = (i + 1 < n) ? off[(size_t)h * n + i] : 0.0;
    }
    __syncthreads();
    const double tn = tnorm[h];
    const double ctol = 1e-7 * tn;
    for (int jj = 1; jj < r; ++jj) {
        int c0 = jj;
        while (c0 > 0 && fabs(s_lam[c0 - 1] - s_lam[jj]) < ctol) --c0;
        if (c0 == jj) continue;
        const int nc = jj - c0;
        for (int i = tid; i < n; i += NT) s_x[i * r + jj] = start_entry(i, jj);
        __syncthreads();
        for (int it = 0;; ++it) {
            for (int pass = 0; pass < 2; ++pass) {
                const int c = tid >> 2, part = tid & 3;   // 4 lanes per earlier vector
                double s = 0.0;
                if (c < nc)
                    for (int i = part; i < n; i += 4) s += s_x[i * r + c0 + c] * s_x[i * r + jj];
                s = quad_sum(s);
                if (c < nc && part == 0) s_dot[c] = s;
                __syncthreads();
                for (int i = tid; i < n; i += NT) {
                    double x = s_x[i * r + jj];
                    for (int cc = 0; cc < nc; ++cc) x -= s_dot[cc] * s_x[i * r + c0 + cc];
                    s_x[i * r + jj] = x;
                }
                __syncthreads();
            }
            double sq = 0.0;
            for (int i = tid; i < n; i += NT) sq += s_x[i * r + jj] * s_x[i * r + jj];
            const double nrm = sqrt(block_reduce<NT, 0>(sq, s_red));
            const double inv = nrm > 0.0 ? 1.0 / nrm : 0.0;
            for (int i = tid; i < n; i += NT) s_x[i * r + jj] *= inv;
            __syncthreads();
            if (it == 2) break;
            if (tid == 0) {                           // (T - lambda I) y = x, y over x
                const double lj = s_lam[jj], tiny = DBL_EPSILON * tn;
                double* x = s_x + jj;                 // x[i * r]
                double c0d = s_d[0] - lj, c1 = n > 1 ? s_e[0] : 0.0, rb = x[0];
                for (int i = 0; i + 1 < n; ++i) {
                    const double l0 = s_e[i], m1 = s_d[i + 1] - lj;
                    const double m2 = i + 2 < n ? s_e[i + 1] : 0.0, mb = x[(i + 1) * r];
                    if (fabs(c0d) >= fabs(l0)) {      // row i stays
                        if (fabs(c0d) < tiny) c0d = c0d < 0.0 ? -tiny : tiny;
                        const double f = l0 / c0d;
                        s_u0[i] = c0d;
                        s_u1[i] = c1;
                        s_u2[i] = 0.0;
                        x[i * r] = rb;
                        c0d = m1 - f * c1;
                        c1 = m2;
                        rb = mb - f * rb;
                    } else {                          // rows i and i+1 swap
                        const double f = c0d / l0;
                        s_u0[i] = l0;
                        s_u1[i] = m1;
                        s_u2[i] = m2;
                        x[i * r] = mb;
                        c0d = c1 - f * m1;
                        c1 = -f * m2;
                        rb = rb - f * mb;
                    }
                }
                if (fabs(c0d) < tiny) c0d = c0d < 0.0 ? -tiny : tiny;
                s_u0[n - 1] = c0d;
                s_u1[n - 1] = 0.0;
                s_u2[n - 1] = 0.0;
                x[(n - 1) * r] = rb;
                double z1 = 0.0, z2 = 0.0;            // z_{i+1}, z_{i+2}
                for (int i = n - 1; i >= 0; --i) {
                    const double z = (x[i * r] - s_u1[i] * z1 - s_u2[i] * z2) / s_u0[i];
                    x[i * r] = z;
                    z2 = z1;
                    z1 = z;
                }
            }
            __syncthreads();
        }
    }
    // this lane: vectors 2 vp and 2 vp + 1, rows l16 + 16 t
    const int vp = tid >> 4, l16 = tid & 15;
    const bool mine = 2 * vp < r;
    double x0[RPL], x1[RPL];
#pragma unroll
    for (int t = 0; t < RPL; ++t) {
        const int i = l16 + 16 * t;
        x0[t] = (mine && i < n) ? s_x[i * r + 2 * vp] : 0.0;
        x1[t] = (mine && i < n && 2 * vp + 1 < r) ? s_x[i * r + 2 * vp + 1] : 0.0;
    }
    // a batch of reflectors is fetched into registers while the one before it is applied
    constexpr int PER = kReflStage * kEigMaxN / NT;   // staged entries per thread
    static_assert(PER * NT == kReflStage * kEigMaxN, "whole batches");
    double nx[PER], nb = 0.0;
    auto fetch = [&](int kb) {
        const int cnt = min(kReflStage, kb + 1);      // reflectors kb, kb-1, ..., kb-cnt+1
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * NT, sI = e / kEigMaxN, i = e - sI * kEigMaxN, k = kb - sI;
            // entry of v_k at row i of the vector (zero above row k+1 and past row n-1, the
            // padding rows every lane carries)
            nx[u] = (sI < cnt && i > k && i < n) ? hv[((size_t)h * n + k) * n + (i - k - 1)] : 0.0;
        }
        nb = tid < cnt ? hbeta[(size_t)h * n + kb - tid] : 0.0;
    };
    if (n >= 3) fetch(n - 3);
    for (int kb = n - 3; kb >= 0; kb -= kReflStage) {
        const int cnt = min(kReflStage, kb + 1);
        __syncthreads();                              // the previous batch is used
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int e = tid + u * NT;
            s_hv[e / kEigMaxN][e % kEigMaxN] = nx[u];
        }
        if (tid < kReflStage) s_hb[tid] = nb;
        __syncthreads();
        if (kb - kReflStage >= 0) fetch(kb - kReflStage);
        if (mine) {
            for (int sI = 0; sI < cnt; ++sI) {
                const double beta = s_hb[sI];
                if (beta == 0.0) continue;
                const int k = kb - sI;
                double vv[RPL], p0[2] = {0.0, 0.0}, p1[2] = {0.0, 0.0};
#pragma unroll
                for (int t = 0; t < RPL; ++t) {
                    // rows at or above k+1 carry no entry of v_k: no read
                    vv[t] = (l16 + 16 * t > k) ? s_hv[sI][l16 + 16 * t] : 0.0;
                    p0[t & 1] = fma(vv[t], x0[t], p0[t & 1]);
                    p1[t & 1] = fma(vv[t], x1[t], p1[t & 1]);
                }
                double a0 = quad_sum(p0[0] + p0[1]);
                double a1 = quad_sum(p1[0] + p1[1]);
                a0 += dpp_move<0x141>(a0);            // the other quad of 8
                a1 += dpp_move<0x141>(a1);
                a0 += dpp_move<0x140>(a0);            // the other 8 of 16
                a1 += dpp_move<0x140>(a1);
                a0 *= beta;
                a1 *= beta;
#pragma unroll
                for (int t = 0; t < RPL; ++t) {
                    x0[t] = fma(-a0, vv[t], x0[t]);
                    x1[t] = fma(-a1, vv[t], x1[t]);
                }
            }
        }
    }
    __syncthreads();
    if (mine) {
        const double sl0 = sqrt(fmax(s_lam[2 * vp], 0.0));
        const double sl1 = 2 * vp + 1 < r ? sqrt(fmax(s_lam[2 * vp + 1], 0.0)) : 0.0;
#pragma unroll
        for (int t = 0; t < RPL; ++t) {
            const int i = l16 + 16 * t;
            if (i < n) {
                w_out[((size_t)h * n + i) * r + 2 * vp] = x0[t] * sl0;
                if (2 * vp + 1 < r) w_out[((size_t)h * n + i) * r + 2 * vp + 1] = x1[t] * sl1;
            }
        }
    }
    if (tid == 0) gap_out[h] = (r < ne && s_lam[r] > 0.0) ? s_lam[r - 1] / s_lam[r] : INFINITY;
}

}  // namespace

void launch_sym_eig_top(const double* m, int heads, int n, int r, double* diag, double* off,
                        double* hv, double* hbeta, double* lam, double* vec, double* tnorm,
                        double* w, double* gap, hipStream_t st) {
    const int ne = std::min(r + 1, n);
    hipLaunchKernelGGL(k_tridiag, dim3(heads), dim3(kTriThreads), 0, st, m, n, diag, off, hv, hbeta);
    hipLaunchKernelGGL(k_tri_eigpair, dim3(ne, heads), dim3(kEigThreads), 0, st, diag, off, n, r, ne,
                       lam, vec, tnorm);
    hipLaunchKernelGGL(k_eig_finish, dim3(heads), dim3(kFinThreads), 0, st, diag, off, hv, hbeta, lam,
                       vec, tnorm, n, r, ne, w, gap);
}

}  // namespace spr
