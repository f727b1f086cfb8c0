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

// Number of eigenvalues of T strictly below x (Sturm sequence of the LDL^T pivots).
int sturm_count(const Tridiag& t, double x, double pivmin) {
    int count = 0;
    double q = t.diag[0] - x;
    if (std::fabs(q) < pivmin) q = -pivmin;
    if (q < 0) ++count;
    for (int i = 1; i < t.n; ++i) {
        q = (t.diag[i] - x) - t.off[i - 1] * t.off[i - 1] / q;
        if (std::fabs(q) < pivmin) q = -pivmin;
        if (q < 0) ++count;
    }
    return count;
}

// Eigenvalue of rank `idx` in ascending order (0 = smallest) by bisection.
double bisect_eigenvalue(const Tridiag& t, int idx, double lo, double hi, double pivmin) {
    for (int it = 0; it < 200; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        if (sturm_count(t, mid, pivmin) > idx) hi = mid; else lo = mid;
        if (hi - lo <= 2.0 * kEps * std::max(std::fabs(lo), std::fabs(hi)) + pivmin) break;
    }
    return 0.5 * (lo + hi);
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
    for (int j = 0; j < r; ++j) lam[j] = bisect_eigenvalue(t, n - 1 - j, glo, ghi, pivmin);

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
    if (cholesky_lower(d, m.data(), l) == 0) return 0;
    // semi-definite metric: L = U diag(sqrt(max(lambda, 0)))
    return key_projection(d, m.data(), d, l);
}

int probe_fit(int p, int d, const double* x, const double* y, double lambda, int rank,
              double* b_mat, double* b_vec) {
    std::memset(b_mat, 0, sizeof(double) * d * d);
    std::memset(b_vec, 0, sizeof(double) * d);
    if (p == 0) return 0;
    for (size_t i = 0; i < static_cast<size_t>(p) * d; ++i)
        if (!std::isfinite(x[i]) || !std::isfinite(y[i])) return -2;
    // centred ridge: B = (Xc^T Xc + lambda I)^-1 Xc^T Yc, b = ybar - xbar B
    std::vector<double> xm(d, 0.0), ym(d, 0.0);
    for (int r = 0; r < p; ++r)
        for (int c = 0; c < d; ++c) {
            xm[c] += x[static_cast<size_t>(r) * d + c];
            ym[c] += y[static_cast<size_t>(r) * d + c];
        }
    for (int c = 0; c < d; ++c) { xm[c] /= p; ym[c] /= p; }
    std::vector<double> xc(static_cast<size_t>(p) * d), yc(static_cast<size_t>(p) * d);
    for (int r = 0; r < p; ++r)
        for (int c = 0; c < d; ++c) {
            xc[static_cast<size_t>(r) * d + c] = x[static_cast<size_t>(r) * d + c] - xm[c];
            yc[static_cast<size_t>(r) * d + c] = y[static_cast<size_t>(r) * d + c] - ym[c];
        }
    std::vector<double> gram(static_cast<size_t>(d) * d, 0.0), rhs(static_cast<size_t>(d) * d, 0.0);
    for (int r = 0; r < p; ++r) {
        const double* xr = &xc[static_cast<size_t>(r) * d];
        const double* yr = &yc[static_cast<size_t>(r) * d];
        for (int i = 0; i < d; ++i) {
            const double xi = xr[i];
            double* gi = &gram[static_cast<size_t>(i) * d];
            double* ri = &rhs[static_cast<size_t>(i) * d];
            for (int j = 0; j < d; ++j) { gi[j] += xi * xr[j]; ri[j] += xi * yr[j]; }
        }
    }
    std::vector<double> bfull(static_cast<size_t>(d) * d, 0.0);
    if (lambda > 0.0) {
        for (int i = 0; i < d; ++i) gram[static_cast<size_t>(i) * d + i] += lambda;
        std::vector<double> l(static_cast<size_t>(d) * d);
        if (cholesky_lower(d, gram.data(), l.data()) != 0) return -3;
        // solve L L^T B = rhs column by column
        std::vector<double> z(d);
        for (int col = 0; col < d; ++col) {
            for (int i = 0; i < d; ++i) {
                double s = rhs[static_cast<size_t>(i) * d + col];
                for (int k = 0; k < i; ++k) s -= l[static_cast<size_t>(i) * d + k] * z[k];
                z[i] = s / l[static_cast<size_t>(i) * d + i];
            }
            for (int i = d - 1; i >= 0; --i) {
                double s = z[i];
                for (int k = i + 1; k < d; ++k) s -= l[static_cast<size_t>(k) * d + i] * bfull[static_cast<size_t>(k) * d + col];
                bfull[static_cast<size_t>(i) * d + col] = s / l[static_cast<size_t>(i) * d + i];
            }
        }
    } else {
        // minimum-norm least squares through the eigenpairs of Xc^T Xc
        std::vector<double> lam(d), vec(static_cast<size_t>(d) * d);
        if (sym_eig_top(d, gram.data(), d, lam.data(), vec.data()) != 0) return -3;
        const double thr = std::max(lam[0], 0.0) * std::max(p, d) * kEps;
        std::vector<double> tmp(static_cast<size_t>(d) * d, 0.0);   // diag(1/lam) V^T rhs
        for (int e = 0; e < d; ++e) {
            if (!(lam[e] > thr)) continue;
            for (int col = 0; col < d; ++col) {
                double s = 0.0;
                for (int i = 0; i < d; ++i) s += vec[static_cast<size_t>(i) * d + e] * rhs[static_cast<size_t>(i) * d + col];
                tmp[static_cast<size_t>(e) * d + col] = s / lam[e];
            }
        }
        for (int i = 0; i < d; ++i)
            for (int col = 0; col < d; ++col) {
                double s = 0.0;
                for (int e = 0; e < d; ++e) s += vec[static_cast<size_t>(i) * d + e] * tmp[static_cast<size_t>(e) * d + col];
                bfull[static_cast<size_t>(i) * d + col] = s;
            }
    }
    std::vector<double> bv(d);
    for (int j = 0; j < d; ++j) {
        double s = ym[j];
        for (int i = 0; i < d; ++i) s -= xm[i] * bfull[static_cast<size_t>(i) * d + j];
        bv[j] = s;
    }
    // projector onto the leading right singular vectors of the uncentred Y
    const int rmax = std::min(rank, std::min(p, d));
    if (rmax <= 0) return 0;
    std::vector<double> yty(static_cast<size_t>(d) * d, 0.0);
    for (int r = 0; r < p; ++r) {
        const double* yr = &y[static_cast<size_t>(r) * d];
        for (int i = 0; i < d; ++i) {
            double* gi = &yty[static_cast<size_t>(i) * d];
            for (int j = 0; j < d; ++j) gi[j] += yr[i] * yr[j];
        }
    }
    std::vector<double> lam(rmax), vec(static_cast<size_t>(d) * rmax);
    if (sym_eig_top(d, yty.data(), rmax, lam.data(), vec.data()) != 0) return -3;
    // singular values from the Gram eigenvalues; values below 2^-20 sigma_1 are not
    // resolved by the Gram route and count as zero
    const double s1 = std::sqrt(std::max(lam[0], 0.0));
    int r_eff = 0;
    if (s1 > 0.0) {
        const double thr = s1 * std::max(std::ldexp(1.0, -20), std::max(p, d) * kEps);
        while (r_eff < rmax && std::sqrt(std::max(lam[r_eff], 0.0)) > thr) ++r_eff;
    }
    if (r_eff == 0) return 0;
    std::vector<double> pi(static_cast<size_t>(d) * d, 0.0);
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            double s = 0.0;
            for (int e = 0; e < r_eff; ++e) s += vec[static_cast<size_t>(i) * rmax + e] * vec[static_cast<size_t>(j) * rmax + e];
            pi[static_cast<size_t>(i) * d + j] = s;
        }
    for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
            double s = 0.0;
            const double* bi = &bfull[static_cast<size_t>(i) * d];
            for (int t = 0; t < d; ++t) s += bi[t] * pi[static_cast<size_t>(t) * d + j];
            b_mat[static_cast<size_t>(i) * d + j] = s;
        }
    for (int j = 0; j < d; ++j) {
        double s = 0.0;
        for (int t = 0; t < d; ++t) s += bv[t] * pi[static_cast<size_t>(t) * d + j];
        b_vec[j] = s;
    }
    return 0;
}

}  // namespace spr
