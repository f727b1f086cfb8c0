// Host-side fp64 small dense solves for the SparsePR path (no GPU, no LAPACK).
//
//  * top-r eigenpairs of a symmetric matrix: Householder reduction to tridiagonal
//    form, Sturm-sequence bisection for the wanted eigenvalues, inverse iteration
//    (tridiagonal LU with partial pivoting, re-orthogonalised inside clusters) for
//    their eigenvectors, then the Householder back-transform;
//  * Cholesky factorisation;
//  * the probe fit of "Partition the Support, Reconstruct the Residual" (gist.science
//    summary, section 2B): centred ridge regression for R ~ b + x B, and the projector
//    onto the leading right singular vectors of the residual matrix (from the
//    eigenpairs of its Gram matrix).
#include "host_linalg.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <vector>

namespace spr {

namespace {

constexpr double kEps = std::numeric_limits<double>::epsilon();

// The O(n^3) loops are written once (always inlined) and built twice: for AVX2 + FMA and
// for baseline x86-64; the AVX2 build runs when the CPU reports both features.
#define SPR_BODY static inline __attribute__((always_inline))
bool cpu_avx2_fma() {
    static const bool ok = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma");
    return ok;
}

struct Tridiag {
    int n = 0;
    std::vector<double> diag, off;     // off[i] couples rows i and i+1
    std::vector<double> hv;            // Householder vectors, row k holds v_k (length n-k-1)
    std::vector<double> hbeta;         // beta_k (0 = no reflection)
};

// A = Q T Q^T with Q = H_0 H_1 ... H_{n-3}, H_k = I - beta_k v_k v_k^T acting on rows k+1..n-1.
// Works on the lower triangle only (row i holds columns 0..i).
// Raw-pointer core (a is overwritten; p, w are scratch of length n).
SPR_BODY void tridiag_body(int n, double* a, double* diag, double* off, double* hv,
                           double* hbeta, double* p, double* w) {
    auto A = [&](int i, int j) -> double& { return a[static_cast<size_t>(i) * n + j]; };   // i >= j
    for (int k = 0; k + 2 < n; ++k) {
        const int m = n - k - 1, o = k + 1;
        double* v = &hv[static_cast<size_t>(k) * n];
        double sigma2 = 0.0;
        for (int i = 0; i < m; ++i) {
            v[i] = A(o + i, k);
            sigma2 += v[i] * v[i];
        }
        const double tail2 = sigma2 - v[0] * v[0];
        if (tail2 <= 0.0) {            // already tridiagonal in this column
            off[k] = v[0];
            hbeta[k] = 0.0;
            continue;
        }
        const double sigma = std::sqrt(sigma2);
        const double alpha = (v[0] >= 0.0) ? -sigma : sigma;
        v[0] -= alpha;
        const double beta = 2.0 / (tail2 + v[0] * v[0]);
        hbeta[k] = beta;
        off[k] = alpha;
        // p = beta * A22 v from the lower triangle: row i contributes a_ij v_j (j < i)
        // to p_i and a_ij v_i to p_j
        for (int i = 0; i < m; ++i) p[i] = 0.0;
        for (int i = 0; i < m; ++i) {
            const double* row = &A(o + i, o);
            const double vi = v[i];
            double s4[4] = {0.0, 0.0, 0.0, 0.0};   // fixed-order partial sums (vectorisable)
            int j = 0;
            for (; j + 4 <= i; j += 4)
                for (int e = 0; e < 4; ++e) {
                    s4[e] += row[j + e] * v[j + e];
                    p[j + e] += row[j + e] * vi;
                }
            for (; j < i; ++j) {
                s4[0] += row[j] * v[j];
                p[j] += row[j] * vi;
            }
            p[i] += ((s4[0] + s4[1]) + (s4[2] + s4[3])) + row[i] * vi;
        }
        double kk = 0.0;
        for (int i = 0; i < m; ++i) {
            p[i] *= beta;
            kk += v[i] * p[i];
        }
        kk *= 0.5 * beta;
        for (int i = 0; i < m; ++i) w[i] = p[i] - kk * v[i];
        for (int i = 0; i < m; ++i) {
            double* row = &A(o + i, o);
            const double vi = v[i], wi = w[i];
            for (int j = 0; j <= i; ++j) row[j] -= vi * w[j] + wi * v[j];
        }
    }
    for (int i = 0; i < n; ++i) diag[i] = A(i, i);
    if (n >= 2) off[n - 2] = A(n - 1, n - 2);
}

#define SPR_TWO_BUILDS(name, body, params, args)                                         \
    __attribute__((target("avx2,fma"))) void name##_avx2 params { body args; }           \
    void name##_base params { body args; }                                               \
    void name params {                                                                   \
        if (cpu_avx2_fma()) name##_avx2 args; else name##_base args;                     \
    }
SPR_TWO_BUILDS(tridiag_core, tridiag_body,
               (int n, double* a, double* diag, double* off, double* hv, double* hbeta, double* p, double* w),
               (n, a, diag, off, hv, hbeta, p, w))

void tridiagonalize(int n, const double* a_in, Tridiag& t) {
    t.n = n;
    t.diag.assign(n, 0.0);
    t.off.assign(std::max(n - 1, 1), 0.0);
    t.hv.assign(static_cast<size_t>(n) * n, 0.0);
    t.hbeta.assign(n, 0.0);
    std::vector<double> a(a_in, a_in + static_cast<size_t>(n) * n), p(n), w(n);
    tridiag_core(n, a.data(), t.diag.data(), t.off.data(), t.hv.data(), t.hbeta.data(), p.data(), w.data());
}

// Eigenvalues of ascending ranks first .. first+count-1 by bisection on Sturm counts, all
// intervals advanced together so that the per-eigenvalue recurrences interleave. Stops
// at a relative width of `rtol` (the caller polishes with Rayleigh quotients).
SPR_BODY void bisect_body(int n, const double* diag, const double* e2, int first, int count,
                          double* lo, double* hi, double* q, double* mid, int* cnt, double pivmin,
                          double rtol) {
    for (int it = 0; it < 80; ++it) {
        for (int j = 0; j < count; ++j) mid[j] = 0.5 * (lo[j] + hi[j]);
        for (int j = 0; j < count; ++j) {
            double v = diag[0] - mid[j];
            if (std::fabs(v) < pivmin) v = -pivmin;
            q[j] = v;
            cnt[j] = v < 0 ? 1 : 0;
        }
        for (int i = 1; i < n; ++i) {
            const double ei = e2[i], di = diag[i];
            for (int j = 0; j < count; ++j) {
                double v = (di - mid[j]) - ei / q[j];
                if (std::fabs(v) < pivmin) v = -pivmin;
                q[j] = v;
                cnt[j] += v < 0 ? 1 : 0;
            }
        }
        bool done = true;
        for (int j = 0; j < count; ++j) {
            if (cnt[j] > first + j) hi[j] = mid[j]; else lo[j] = mid[j];
            if (hi[j] - lo[j] > rtol * std::max(std::fabs(lo[j]), std::fabs(hi[j])) + pivmin)
                done = false;
        }
        if (done) break;
    }
}

SPR_TWO_BUILDS(bisect_core, bisect_body,
               (int n, const double* diag, const double* e2, int first, int count, double* lo, double* hi,
                double* q, double* mid, int* cnt, double pivmin, double rtol),
               (n, diag, e2, first, count, lo, hi, q, mid, cnt, pivmin, rtol))

void bisect_eigenvalues(const Tridiag& t, int first, int count, double lo0, double hi0,
                        double pivmin, double rtol, double* out) {
    std::vector<double> lo(count, lo0), hi(count, hi0), q(count), mid(count), e2(t.n, 0.0);
    std::vector<int> cnt(count);
    for (int i = 1; i < t.n; ++i) e2[i] = t.off[i - 1] * t.off[i - 1];
    bisect_core(t.n, t.diag.data(), e2.data(), first, count, lo.data(), hi.data(), q.data(),
                mid.data(), cnt.data(), pivmin, rtol);
    for (int j = 0; j < count; ++j) out[j] = 0.5 * (lo[j] + hi[j]);
}

// Back-transform X = H_0 (H_1 (... H_{n-3} Y)) for r vectors at once (x [n][r]; sv scratch [r]).
SPR_BODY void back_transform_body(int n, int r, const double* hv, const double* hbeta, double* x,
                                  double* sv) {
    for (int k = n - 3; k >= 0; --k) {
        const double beta = hbeta[k];
        if (beta == 0.0) continue;
        const double* v = &hv[static_cast<size_t>(k) * n];
        const int m = n - k - 1;
        for (int j = 0; j < r; ++j) sv[j] = 0.0;
        for (int i = 0; i < m; ++i) {
            const double vi = v[i];
            const double* xr = &x[static_cast<size_t>(k + 1 + i) * r];
            for (int j = 0; j < r; ++j) sv[j] += vi * xr[j];
        }
        for (int j = 0; j < r; ++j) sv[j] *= beta;
        for (int i = 0; i < m; ++i) {
            const double vi = v[i];
            double* xr = &x[static_cast<size_t>(k + 1 + i) * r];
            for (int j = 0; j < r; ++j) xr[j] -= sv[j] * vi;
        }
    }
}

SPR_TWO_BUILDS(back_transform_core, back_transform_body,
               (int n, int r, const double* hv, const double* hbeta, double* x, double* sv),
               (n, r, hv, hbeta, x, sv))

// LU factorisation (partial pivoting) of T - lambda I, reused for several solves; zero
// pivots are replaced by `tiny` (inverse iteration wants the near-singular solve).
struct ShiftedLU {
    std::vector<double> u0, u1, u2, mult, rinv;
    std::vector<char> swapped;
    void factor(const Tridiag& t, double lambda, double tiny) {
        const int n = t.n;
        u0.assign(n, 0.0);
        u1.assign(n, 0.0);
        u2.assign(n, 0.0);
        mult.assign(n, 0.0);
        swapped.assign(n, 0);
        double cur0 = t.diag[0] - lambda;                  // current row: col i, col i+1
        double cur1 = (n > 1) ? t.off[0] : 0.0;
        for (int i = 0; i < n - 1; ++i) {
            const double nl = t.off[i];                                   // row i+1, col i
            const double nd = t.diag[i + 1] - lambda;                      // row i+1, col i+1
            const double nc = (i + 2 < n) ? t.off[i + 1] : 0.0;           // row i+1, col i+2
            if (std::fabs(nl) > std::fabs(cur0)) {
                swapped[i] = 1;                                           // pivot row is i+1
                u0[i] = nl;
                u1[i] = nd;
                u2[i] = nc;
                const double m = cur0 / nl;
                mult[i] = m;
                cur0 = cur1 - m * nd;
                cur1 = -m * nc;
            } else {
                if (cur0 == 0.0) cur0 = tiny;
                u0[i] = cur0;
                u1[i] = cur1;
                const double m = nl / cur0;
                mult[i] = m;
                cur0 = nd - m * cur1;
                cur1 = nc;
            }
        }
        if (cur0 == 0.0) cur0 = tiny;
        u0[n - 1] = cur0;
        rinv.resize(n);
        for (int i = 0; i < n; ++i) rinv[i] = 1.0 / u0[i];
    }
    void solve(double* y, int n) const {
        for (int i = 0; i < n - 1; ++i) {
            if (swapped[i]) {
                const double a = y[i], b = y[i + 1];
                y[i] = b;
                y[i + 1] = a - mult[i] * b;
            } else {
                y[i + 1] -= mult[i] * y[i];
            }
        }
        for (int i = n - 1; i >= 0; --i) {
            double s = y[i];
            if (i + 1 < n) s -= u1[i] * y[i + 1];
            if (i + 2 < n) s -= u2[i] * y[i + 2];
            y[i] = s * rinv[i];
        }
    }
};

}  // namespace

int sym_eig_top(int n, const double* a, int r, double* lam, double* vec) {
    if (n < 1 || r < 0 || r > n) return -1;
    for (size_t i = 0; i < static_cast<size_t>(n) * n; ++i)
        if (!std::isfinite(a[i])) return -2;
    if (r == 0) return 0;
    if (n == 1) {
        lam[0] = a[0];
        vec[0] = 1.0;
        return 0;
    }
    Tridiag t;
    tridiagonalize(n, a, t);
    double tnorm = 0.0, glo = 0.0, ghi = 0.0;
    for (int i = 0; i < n; ++i) {
        const double radius = (i > 0 ? std::fabs(t.off[i - 1]) : 0.0) +
                              (i + 1 < n ? std::fabs(t.off[i]) : 0.0);
        const double lo = t.diag[i] - radius, hi = t.diag[i] + radius;
        if (i == 0 || lo < glo) glo = lo;
        if (i == 0 || hi > ghi) ghi = hi;
        tnorm = std::max(tnorm, std::fabs(t.diag[i]) + radius);
    }
    if (tnorm == 0.0) {                         // zero matrix: any orthonormal basis
        for (int j = 0; j < r; ++j) {
            lam[j] = 0.0;
            for (int i = 0; i < n; ++i) vec[static_cast<size_t>(i) * r + j] = (i == j) ? 1.0 : 0.0;
        }
        return 0;
    }
    const double pivmin = std::numeric_limits<double>::min() * std::max(1.0, tnorm * tnorm);
    const double pad = 2.0 * kEps * tnorm * n + pivmin;
    glo -= pad;
    ghi += pad;
    // eigenvalues, descending: the j-th largest is ascending rank n-1-j. Bisection to a
    // relative width of 2^-30 (the shift of inverse iteration), then each eigenvalue is
    // replaced by the Rayleigh quotient of its converged eigenvector.
    {
        std::vector<double> asc(r);
        bisect_eigenvalues(t, n - r, r, glo, ghi, pivmin, std::ldexp(1.0, -30), asc.data());
        for (int j = 0; j < r; ++j) lam[j] = asc[r - 1 - j];
    }

    // eigenvectors of T by inverse iteration (one factorisation, three solves each)
    const double tiny = kEps * tnorm;
    // shifts closer than 2^-28 of the eigenvalue's own size are split apart (relative, so
    // that eigenvalues far below |T| keep shifts of their own accuracy; the floor is the
    // rounding level n eps |T| below which eigenvalues are not resolved)
    const double noise = n * kEps * tnorm;
    const double cluster_tol = 1e-3 * tnorm;
    std::vector<double> ys(static_cast<size_t>(r) * n);
    ShiftedLU lu;
    double prev_shift = 0.0;
    for (int j = 0; j < r; ++j) {
        double shift = lam[j];
        const double sep = std::ldexp(1.0, -28) * std::max(std::fabs(lam[j]), noise);
        if (j > 0 && prev_shift - shift < sep) shift = prev_shift - sep;   // keep shifts apart
        prev_shift = shift;
        lu.factor(t, shift, tiny);
        double* y = &ys[static_cast<size_t>(j) * n];
        // deterministic start vector with all components non-zero
        for (int i = 0; i < n; ++i) {
            const uint32_t h = (static_cast<uint32_t>(i) + 1u) * 2654435761u ^ (static_cast<uint32_t>(j) + 7u) * 40503u;
            y[i] = 0.5 + static_cast<double>(h % 1000u) / 1000.0;
        }
        int first_in_cluster = j;
        while (first_in_cluster > 0 && std::fabs(lam[first_in_cluster - 1] - lam[j]) < cluster_tol)
            --first_in_cluster;
        for (int it = 0; it < 3; ++it) {
            double nb = 0.0;
            for (int i = 0; i < n; ++i) nb += y[i] * y[i];
            nb = 1.0 / std::sqrt(nb);
            for (int i = 0; i < n; ++i) y[i] *= nb;
            lu.solve(y, n);
            for (int c = first_in_cluster; c < j; ++c) {     // re-orthogonalise in the cluster
                const double* yc = &ys[static_cast<size_t>(c) * n];
                double dot = 0.0;
                for (int i = 0; i < n; ++i) dot += y[i] * yc[i];
                for (int i = 0; i < n; ++i) y[i] -= dot * yc[i];
            }
        }
        double ny = 0.0;
        for (int i = 0; i < n; ++i) ny += y[i] * y[i];
        ny = std::sqrt(ny);
        if (!(ny > 0.0) || !std::isfinite(ny)) return -3;
        for (int i = 0; i < n; ++i) y[i] /= ny;
        // Rayleigh quotient y^T T y
        double rq = 0.0;
        for (int i = 0; i < n; ++i) {
            double ty = t.diag[i] * y[i];
            if (i > 0) ty += t.off[i - 1] * y[i - 1];
            if (i + 1 < n) ty += t.off[i] * y[i + 1];
            rq += y[i] * ty;
        }
        lam[j] = rq;
    }
    // back-transform X = H_0 (H_1 (... H_{n-3} Y)) for all r vectors at once (X [n][r])
    std::vector<double> xs(static_cast<size_t>(n) * r), sv(r);
    for (int j = 0; j < r; ++j)
        for (int i = 0; i < n; ++i) xs[static_cast<size_t>(i) * r + j] = ys[static_cast<size_t>(j) * n + i];
    back_transform_core(n, r, t.hv.data(), t.hbeta.data(), xs.data(), sv.data());
    std::copy(xs.begin(), xs.end(), vec);
    return 0;
}

int cholesky_lower(int n, const double* a, double* l) {
    std::memset(l, 0, sizeof(double) * n * n);
    for (int j = 0; j < n; ++j) {
        double s = a[static_cast<size_t>(j) * n + j];
        for (int k = 0; k < j; ++k) s -= l[static_cast<size_t>(j) * n + k] * l[static_cast<size_t>(j) * n + k];
        if (!(s > 0.0) || !std::isfinite(s)) return -1;
        const double dj = std::sqrt(s);
        l[static_cast<size_t>(j) * n + j] = dj;
        for (int i = j + 1; i < n; ++i) {
            double t = a[static_cast<size_t>(i) * n + j];
            for (int k = 0; k < j; ++k) t -= l[static_cast<size_t>(i) * n + k] * l[static_cast<size_t>(j) * n + k];
            l[static_cast<size_t>(i) * n + j] = t / dj;
        }
    }
    return 0;
}

int key_projection(int d, const double* m_k, int r, double* w, double* gap) {
    const int r1 = std::min(r + 1, d);                 // one more eigenvalue for the gap
    std::vector<double> lam(r1), vec(static_cast<size_t>(d) * r1);
    const int rc = sym_eig_top(d, m_k, r1, lam.data(), vec.data());
    if (rc != 0) return rc;
    for (int j = 0; j < r; ++j) {
        const double s = std::sqrt(std::max(lam[j], 0.0));
        for (int i = 0; i < d; ++i) w[static_cast<size_t>(i) * r + j] = vec[static_cast<size_t>(i) * r1 + j] * s;
    }
    if (gap) *gap = (r1 > r && lam[r] > 0.0) ? lam[r - 1] / lam[r] : INFINITY;
    return 0;
}

// Centred Grams of X, Y [p][d] (and the uncentred Y^T Y): the same quantities the
// device computes before the host solve.
void probe_grams(int p, int d, const double* x, const double* y, double* xm, double* ym, double* gxx,
                 double* gxy, double* gyy) {
    std::fill(xm, xm + d, 0.0);
    std::fill(ym, ym + d, 0.0);
    for (int r = 0; r < p; ++r)
        for (int c = 0; c < d; ++c) {
            xm[c] += x[static_cast<size_t>(r) * d + c];
            ym[c] += y[static_cast<size_t>(r) * d + c];
        }
    for (int c = 0; c < d; ++c) { xm[c] /= p; ym[c] /= p; }
    std::fill(gxx, gxx + static_cast<size_t>(d) * d, 0.0);
    std::fill(gxy, gxy + static_cast<size_t>(d) * d, 0.0);
    std::fill(gyy, gyy + static_cast<size_t>(d) * d, 0.0);
    std::vector<double> xc(d), yc(d);
    for (int r = 0; r < p; ++r) {
        const double* xr = &x[static_cast<size_t>(r) * d];
        const double* yr = &y[static_cast<size_t>(r) * d];
        for (int c = 0; c < d; ++c) { xc[c] = xr[c] - xm[c]; yc[c] = yr[c] - ym[c]; }
        for (int i = 0; i < d; ++i) {
            double* gi = &gxx[static_cast<size_t>(i) * d];
            double* hi = &gxy[static_cast<size_t>(i) * d];
            double* ki = &gyy[static_cast<size_t>(i) * d];
            const double xi = xc[i], yi = yr[i];
            for (int j = 0; j < d; ++j) {
                gi[j] += xi * xc[j];
                hi[j] += xi * yc[j];
                ki[j] += yi * yr[j];
            }
        }
    }
}

// Fit from the Grams: with V_r the leading eigenvectors of Y^T Y (the right singular
// vectors of Y), B' = B V_r V_r^T where B V_r = (Xc^T Xc + lambda I)^-1 (Xc^T Yc V_r), and
// b' = ybar Pi - xbar B'.
int probe_fit_from_grams(int p, int d, const double* xm, const double* ym, const double* gxx_in,
                         const double* gxy, const double* gyy, double lambda, int rank,
                         double* b_mat, double* b_vec, double* sgap) {
    std::memset(b_mat, 0, sizeof(double) * d * d);
    std::memset(b_vec, 0, sizeof(double) * d);
    if (sgap) *sgap = INFINITY;
    if (p == 0) return 0;
    for (size_t i = 0; i < static_cast<size_t>(d) * d; ++i)
        if (!std::isfinite(gxx_in[i]) || !std::isfinite(gxy[i]) || !std::isfinite(gyy[i])) return -2;
    const int rmax = std::min(rank, std::min(p, d));
    if (rmax <= 0) return 0;
    // one eigenvalue past the kept rank for the singular gap (vec keeps rmax1 columns)
    const int rmax1 = std::min(rmax + 1, d);
    std::vector<double> lam(rmax1), vec(static_cast<size_t>(d) * rmax1);
    if (sym_eig_top(d, gyy, rmax1, lam.data(), vec.data()) != 0) return -3;
    // singular values from the Gram eigenvalues; values below 2^-20 sigma_1 are not
    // resolved by the Gram route and count as zero
    const double s1 = std::sqrt(std::max(lam[0], 0.0));
    int r = 0;
    if (s1 > 0.0) {
        const double thr = s1 * std::max(std::ldexp(1.0, -20), std::max(p, d) * kEps);
        while (r < rmax && std::sqrt(std::max(lam[r], 0.0)) > thr) ++r;
    }
    if (r == 0) return 0;
    if (sgap) {
        const bool beyond = r < rmax1 && r < std::min(p, d);
        const double next = beyond ? std::max(lam[r], 0.0) : 0.0;
        *sgap = next > 0.0 ? std::sqrt(std::max(lam[r - 1], 0.0) / next) : INFINITY;
    }
    // R = Xc^T Yc V_r  [d][r]
    std::vector<double> rhs(static_cast<size_t>(d) * r, 0.0), bv(static_cast<size_t>(d) * r, 0.0);
    for (int i = 0; i < d; ++i)
        for (int t = 0; t < d; ++t) {
            const double g = gxy[static_cast<size_t>(i) * d + t];
            for (int e = 0; e < r; ++e) rhs[static_cast<size_t>(i) * r + e] += g * vec[static_cast<size_t>(t) * rmax1 + e];
        }
    if (lambda > 0.0) {
        std::vector<double> gxx(gxx_in, gxx_in + static_cast<size_t>(d) * d);
        for (int i = 0; i < d; ++i) gxx[static_cast<size_t>(i) * d + i] += lambda;
        std::vector<double> l(static_cast<size_t>(d) * d);
        if (cholesky_lower(d, gxx.data(), l.data()) != 0) return -3;
        // forward then backward substitution, all r columns per row
        std::vector<double> z(static_cast<size_t>(d) * r);
        for (int i = 0; i < d; ++i) {
            double* zi = &z[static_cast<size_t>(i) * r];
            for (int e = 0; e < r; ++e) zi[e] = rhs[static_cast<size_t>(i) * r + e];
            for (int k = 0; k < i; ++k) {
                const double lik = l[static_cast<size_t>(i) * d + k];
                const double* zk = &z[static_cast<size_t>(k) * r];
                for (int e = 0; e < r; ++e) zi[e] -= lik * zk[e];
            }
            const double inv = 1.0 / l[static_cast<size_t>(i) * d + i];
            for (int e = 0; e < r; ++e) zi[e] *= inv;
        }
        for (int i = d - 1; i >= 0; --i) {
            double* bi = &bv[static_cast<size_t>(i) * r];
            for (int e = 0; e < r; ++e) bi[e] = z[static_cast<size_t>(i) * r + e];
            for (int k = i + 1; k < d; ++k) {
                const double lki = l[static_cast<size_t>(k) * d + i];
                const double* bk = &bv[static_cast<size_t>(k) * r];
                for (int e = 0; e < r; ++e) bi[e] -= lki * bk[e];
            }
            const double inv = 1.0 / l[static_cast<size_t>(i) * d + i];
            for (int e = 0; e < r; ++e) bi[e] *= inv;
        }
    } else {
        // minimum-norm least squares through the eigenpairs of Xc^T Xc
        std::vector<double> el(d), ev(static_cast<size_t>(d) * d);
        if (sym_eig_top(d, gxx_in, d, el.data(), ev.data()) != 0) return -3;
        const double thr = std::max(el[0], 0.0) * std::max(p, d) * kEps;
        for (int k = 0; k < d; ++k) {
            if (!(el[k] > thr)) continue;
            for (int e = 0; e < r; ++e) {
                double sdot = 0.0;
                for (int i = 0; i < d; ++i) sdot += ev[static_cast<size_t>(i) * d + k] * rhs[static_cast<size_t>(i) * r + e];
                sdot /= el[k];
                for (int i = 0; i < d; ++i) bv[static_cast<size_t>(i) * r + e] += ev[static_cast<size_t>(i) * d + k] * sdot;
            }
        }
    }
    // B' = (B V_r) V_r^T; b' = ybar Pi - xbar B'
    for (int i = 0; i < d; ++i) {
        const double* bi = &bv[static_cast<size_t>(i) * r];
        double* out = &b_mat[static_cast<size_t>(i) * d];
        for (int j = 0; j < d; ++j) {
            double s = 0.0;
            for (int e = 0; e < r; ++e) s += bi[e] * vec[static_cast<size_t>(j) * rmax1 + e];
            out[j] = s;
        }
    }
    std::vector<double> yv(r, 0.0);
    for (int e = 0; e < r; ++e)
        for (int t = 0; t < d; ++t) yv[e] += ym[t] * vec[static_cast<size_t>(t) * rmax1 + e];
    for (int j = 0; j < d; ++j) {
        double s = 0.0;
        for (int e = 0; e < r; ++e) s += yv[e] * vec[static_cast<size_t>(j) * rmax1 + e];
        for (int i = 0; i < d; ++i) s -= xm[i] * b_mat[static_cast<size_t>(i) * d + j];
        b_vec[j] = s;
    }
    return 0;
}

int probe_fit(int p, int d, const double* x, const double* y, double lambda, int rank,
              double* b_mat, double* b_vec) {
    if (p == 0) {
        std::memset(b_mat, 0, sizeof(double) * d * d);
        std::memset(b_vec, 0, sizeof(double) * d);
        return 0;
    }
    for (size_t i = 0; i < static_cast<size_t>(p) * d; ++i)
        if (!std::isfinite(x[i]) || !std::isfinite(y[i])) return -2;
    std::vector<double> xm(d), ym(d), gxx(static_cast<size_t>(d) * d), gxy(static_cast<size_t>(d) * d),
        gyy(static_cast<size_t>(d) * d);
    probe_grams(p, d, x, y, xm.data(), ym.data(), gxx.data(), gxy.data(), gyy.data());
    return probe_fit_from_grams(p, d, xm.data(), ym.data(), gxx.data(), gxy.data(), gyy.data(), lambda,
                                rank, b_mat, b_vec, nullptr);
}

}  // namespace spr
