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

struct Tridiag {
    int n = 0;
    std::vector<double> diag, off;     // off[i] couples rows i and i+1
    std::vector<double> hv;            // Householder vectors, row k holds v_k (length n-k-1)
    std::vector<double> hbeta;         // beta_k (0 = no reflection)
};

// A = Q T Q^T with Q = H_0 H_1 ... H_{n-3}, H_k = I - beta_k v_k v_k^T acting on rows k+1..n-1.
void tridiagonalize(int n, const double* a_in, Tridiag& t) {
    t.n = n;
    t.diag.assign(n, 0.0);
    t.off.assign(std::max(n - 1, 0), 0.0);
    t.hv.assign(static_cast<size_t>(n) * n, 0.0);
    t.hbeta.assign(n, 0.0);
    std::vector<double> a(a_in, a_in + static_cast<size_t>(n) * n);
    std::vector<double> p(n), w(n);
    for (int k = 0; k + 2 < n; ++k) {
        const int m = n - k - 1;
        double* v = &t.hv[static_cast<size_t>(k) * n];
        double sigma2 = 0.0;
        for (int i = 0; i < m; ++i) {
            v[i] = a[static_cast<size_t>(k + 1 + i) * n + k];
            sigma2 += v[i] * v[i];
        }
        double tail2 = sigma2 - v[0] * v[0];
        if (tail2 <= 0.0) {            // already tridiagonal in this column
            t.off[k] = v[0];
            t.hbeta[k] = 0.0;
            continue;
        }
        const double sigma = std::sqrt(sigma2);
        const double alpha = (v[0] >= 0.0) ? -sigma : sigma;
        v[0] -= alpha;
        const double vtv = tail2 + v[0] * v[0];
        const double beta = 2.0 / vtv;
        t.hbeta[k] = beta;
        t.off[k] = alpha;
        // p = beta * A22 v
        for (int i = 0; i < m; ++i) {
            const double* row = &a[static_cast<size_t>(k + 1 + i) * n + (k + 1)];
            double s = 0.0;
            for (int j = 0; j < m; ++j) s += row[j] * v[j];
            p[i] = beta * s;
        }
        double kk = 0.0;
        for (int i = 0; i < m; ++i) kk += v[i] * p[i];
        kk *= 0.5 * beta;
        for (int i = 0; i < m; ++i) w[i] = p[i] - kk * v[i];
        for (int i = 0; i < m; ++i) {
            double* row = &a[static_cast<size_t>(k + 1 + i) * n + (k + 1)];
            for (int j = 0; j < m; ++j) row[j] -= v[i] * w[j] + w[i] * v[j];
        }
    }
    for (int i = 0; i < n; ++i) t.diag[i] = a[static_cast<size_t>(i) * n + i];
    if (n >= 2) t.off[n - 2] = a[static_cast<size_t>(n - 1) * n + (n - 2)];
}

// Eigenvalues of ascending ranks first .. first+count-1 by bisection on Sturm counts, all
// intervals advanced together so that the per-eigenvalue recurrences interleave.
void bisect_eigenvalues(const Tridiag& t, int first, int count, double lo0, double hi0,
                        double pivmin, double* out) {
    std::vector<double> lo(count, lo0), hi(count, hi0), q(count), mid(count);
    std::vector<int> cnt(count);
    for (int it = 0; it < 80; ++it) {
        for (int j = 0; j < count; ++j) mid[j] = 0.5 * (lo[j] + hi[j]);
        for (int j = 0; j < count; ++j) {
            double v = t.diag[0] - mid[j];
            if (std::fabs(v) < pivmin) v = -pivmin;
            q[j] = v;
            cnt[j] = v < 0 ? 1 : 0;
        }
        for (int i = 1; i < t.n; ++i) {
            const double e2 = t.off[i - 1] * t.off[i - 1];
            const double di = t.diag[i];
            for (int j = 0; j < count; ++j) {
                double v = (di - mid[j]) - e2 / q[j];
                if (std::fabs(v) < pivmin) v = -pivmin;
                q[j] = v;
                cnt[j] += v < 0 ? 1 : 0;
            }
        }
        bool done = true;
        for (int j = 0; j < count; ++j) {
            if (cnt[j] > first + j) hi[j] = mid[j]; else lo[j] = mid[j];
            if (hi[j] - lo[j] > 2.0 * kEps * std::max(std::fabs(lo[j]), std::fabs(hi[j])) + pivmin)
                done = false;
        }
        if (done) break;
    }
    for (int j = 0; j < count; ++j) out[j] = 0.5 * (lo[j] + hi[j]);
}

// Solve (T - lambda I) y = b in place with Gaussian elimination and partial pivoting;
// zero pivots are replaced by `tiny` (inverse iteration wants the near-singular solve).
void tridiag_shifted_solve(const Tridiag& t, double lambda, double tiny, std::vector<double>& y) {
    const int n = t.n;
    // U has a diagonal, first and second super-diagonal; L multipliers with row swaps.
    std::vector<double> u0(n), u1(n, 0.0), u2(n, 0.0), mult(n, 0.0);
    std::vector<char> swapped(n, 0);
    // current row i content: cur0 at col i, cur1 at col i+1
    double cur0 = t.diag[0] - lambda;
    double cur1 = (n > 1) ? t.off[0] : 0.0;
    for (int i = 0; i < n - 1; ++i) {
        const double nl = t.off[i];                                   // row i+1, col i
        const double nd = t.diag[i + 1] - lambda;                      // row i+1, col i+1
        const double nc = (i + 2 < n) ? t.off[i + 1] : 0.0;           // row i+1, col i+2
        if (std::fabs(nl) > std::fabs(cur0)) {
            // swap: pivot row is row i+1
            swapped[i] = 1;
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
            u2[i] = 0.0;
            const double m = nl / cur0;
            mult[i] = m;
            cur0 = nd - m * cur1;
            cur1 = nc;
        }
    }
    if (cur0 == 0.0) cur0 = tiny;
    u0[n - 1] = cur0;
    // forward: apply the same swaps and multipliers to y
    for (int i = 0; i < n - 1; ++i) {
        if (swapped[i]) {
            const double a = y[i], b = y[i + 1];
            y[i] = b;
            y[i + 1] = a - mult[i] * b;
        } else {
            y[i + 1] -= mult[i] * y[i];
        }
    }
    // back substitution
    for (int i = n - 1; i >= 0; --i) {
        double s = y[i];
        if (i + 1 < n) s -= u1[i] * y[i + 1];
        if (i + 2 < n) s -= u2[i] * y[i + 2];
        double piv = u0[i];
        if (piv == 0.0) piv = tiny;
        y[i] = s / piv;
    }
}

double norm2(const std::vector<double>& x) {
    double s = 0.0;
    for (double v : x) s += v * v;
    return std::sqrt(s);
}

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
    // eigenvalues, descending: the j-th largest is ascending rank n-1-j
    {
        std::vector<double> asc(r);
        bisect_eigenvalues(t, n - r, r, glo, ghi, pivmin, asc.data());
        for (int j = 0; j < r; ++j) lam[j] = asc[r - 1 - j];
    }

    // eigenvectors of T by inverse iteration
    const double tiny = kEps * tnorm;
    const double cluster_tol = 1e-3 * tnorm;
    std::vector<std::vector<double>> ys(r, std::vector<double>(n));
    std::vector<double> y(n);
    double prev_shift = 0.0;
    for (int j = 0; j < r; ++j) {
        double shift = lam[j];
        if (j > 0 && std::fabs(shift - lam[j - 1]) < 10.0 * tiny) {
            shift = prev_shift - 10.0 * tiny;   // separate equal eigenvalues (descending)
        }
        prev_shift = shift;
        // deterministic start vector with all components non-zero
        for (int i = 0; i < n; ++i) {
            const uint32_t h = (static_cast<uint32_t>(i) + 1u) * 2654435761u ^ (static_cast<uint32_t>(j) + 7u) * 40503u;
            y[i] = 0.5 + static_cast<double>(h % 1000u) / 1000.0;
        }
        int first_in_cluster = j;
        while (first_in_cluster > 0 && std::fabs(lam[first_in_cluster - 1] - lam[j]) < cluster_tol)
            --first_in_cluster;
        for (int it = 0; it < 5; ++it) {
            const double nb = norm2(y);
            for (double& v : y) v /= nb;
            tridiag_shifted_solve(t, shift, tiny, y);
            for (int c = first_in_cluster; c < j; ++c) {     // re-orthogonalise in the cluster
                double dot = 0.0;
                for (int i = 0; i < n; ++i) dot += y[i] * ys[c][i];
                for (int i = 0; i < n; ++i) y[i] -= dot * ys[c][i];
            }
        }
        const double ny = norm2(y);
        if (!(ny > 0.0) || !std::isfinite(ny)) return -3;
        for (int i = 0; i < n; ++i) ys[j][i] = y[i] / ny;
    }
    // back-transform: x = H_0 (H_1 (... H_{n-3} y))
    for (int j = 0; j < r; ++j) {
        std::vector<double>& x = ys[j];
        for (int k = n - 3; k >= 0; --k) {
            const double beta = t.hbeta[k];
            if (beta == 0.0) continue;
            const double* v = &t.hv[static_cast<size_t>(k) * n];
            const int m = n - k - 1;
            double s = 0.0;
            for (int i = 0; i < m; ++i) s += v[i] * x[k + 1 + i];
            s *= beta;
            for (int i = 0; i < m; ++i) x[k + 1 + i] -= s * v[i];
        }
        for (int i = 0; i < n; ++i) vec[static_cast<size_t>(i) * r + j] = x[i];
    }
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

int key_projection(int d, const double* m_k, int r, double* w) {
    std::vector<double> lam(r), vec(static_cast<size_t>(d) * r);
    const int rc = sym_eig_top(d, m_k, r, lam.data(), vec.data());
    if (rc != 0) return rc;
    for (int j = 0; j < r; ++j) {
        const double s = std::sqrt(std::max(lam[j], 0.0));
        for (int i = 0; i < d; ++i) w[static_cast<size_t>(i) * r + j] = vec[static_cast<size_t>(i) * r + j] * s;
    }
    return 0;
}

int query_factor_from_metric(int d, const double* m, double* l);

int query_factor(int d, int g, const double* c, double* l, int* dims) {
    for (size_t i = 0; i < static_cast<size_t>(g) * d; ++i)
        if (!std::isfinite(c[i])) return -2;
    if (g <= d) {                               // logit profiles directly: L = C^T / sqrt(d)
        const double s = 1.0 / std::sqrt(static_cast<double>(d));
        for (int i = 0; i < d; ++i)
            for (int j = 0; j < g; ++j) l[static_cast<size_t>(i) * g + j] = c[static_cast<size_t>(j) * d + i] * s;
        *dims = g;
        return 0;
    }
    std::vector<double> m(static_cast<size_t>(d) * d, 0.0);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j <= i; ++j) {
            double s = 0.0;
            for (int t = 0; t < g; ++t) s += c[static_cast<size_t>(t) * d + i] * c[static_cast<size_t>(t) * d + j];
            m[static_cast<size_t>(i) * d + j] = m[static_cast<size_t>(j) * d + i] = s / d;
        }
    *dims = d;
    return query_factor_from_metric(d, m.data(), l);
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
                         double* b_mat, double* b_vec) {
    std::memset(b_mat, 0, sizeof(double) * d * d);
    std::memset(b_vec, 0, sizeof(double) * d);
    if (p == 0) return 0;
    for (size_t i = 0; i < static_cast<size_t>(d) * d; ++i)
        if (!std::isfinite(gxx_in[i]) || !std::isfinite(gxy[i]) || !std::isfinite(gyy[i])) return -2;
    const int rmax = std::min(rank, std::min(p, d));
    if (rmax <= 0) return 0;
    std::vector<double> lam(rmax), vec(static_cast<size_t>(d) * rmax);
    if (sym_eig_top(d, gyy, rmax, lam.data(), vec.data()) != 0) return -3;
    // singular values from the Gram eigenvalues; values below 2^-20 sigma_1 are not
    // resolved by the Gram route and count as zero
    const double s1 = std::sqrt(std::max(lam[0], 0.0));
    int r = 0;
    if (s1 > 0.0) {
        const double thr = s1 * std::max(std::ldexp(1.0, -20), std::max(p, d) * kEps);
        while (r < rmax && std::sqrt(std::max(lam[r], 0.0)) > thr) ++r;
    }
    if (r == 0) return 0;
    // R = Xc^T Yc V_r  [d][r]
    std::vector<double> rhs(static_cast<size_t>(d) * r, 0.0), bv(static_cast<size_t>(d) * r, 0.0);
    for (int i = 0; i < d; ++i)
        for (int t = 0; t < d; ++t) {
            const double g = gxy[static_cast<size_t>(i) * d + t];
            for (int e = 0; e < r; ++e) rhs[static_cast<size_t>(i) * r + e] += g * vec[static_cast<size_t>(t) * rmax + e];
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
            for (int e = 0; e < r; ++e) s += bi[e] * vec[static_cast<size_t>(j) * rmax + e];
            out[j] = s;
        }
    }
    std::vector<double> yv(r, 0.0);
    for (int e = 0; e < r; ++e)
        for (int t = 0; t < d; ++t) yv[e] += ym[t] * vec[static_cast<size_t>(t) * rmax + e];
    for (int j = 0; j < d; ++j) {
        double s = 0.0;
        for (int e = 0; e < r; ++e) s += yv[e] * vec[static_cast<size_t>(j) * rmax + e];
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
                                rank, b_mat, b_vec);
}

// L [d][dims] from the metric m = C^T C / d (d x d): Cholesky if positive definite,
// else the eigen factor U diag(sqrt(max(lambda, 0))).
int query_factor_from_metric(int d, const double* m, double* l) {
    if (cholesky_lower(d, m, l) == 0) return 0;
    return key_projection(d, m, d, l);
}

}  // namespace spr
