// Host-side fp64 small dense solves (no GPU). Return 0 on success, < 0 on failure.
#pragma once
#include <cstdint>

namespace spr {

// Top-r eigenpairs of symmetric a [n][n]: lam[r] descending, vec [n][r] (columns).
int sym_eig_top(int n, const double* a, int r, double* lam, double* vec);

// Lower Cholesky factor l [n][n] of a; -1 if a is not numerically positive definite.
int cholesky_lower(int n, const double* a, double* l);

// W [d][r] = U_r diag(sqrt(max(lambda_r, 0))) for the metric m_k [d][d]; *gap (if not
// null) = lambda_r / lambda_{r+1} (+inf when r = d or lambda_{r+1} <= 0).
int key_projection(int d, const double* m_k, int r, double* w, double* gap);

// Column means and centred Grams Xc^T Xc, Xc^T Yc, and Y^T Y (uncentred) of X, Y [p][d].
void probe_grams(int p, int d, const double* x, const double* y, double* xm, double* ym, double* gxx,
                 double* gxy, double* gyy);

// B' [d][d], b' [d] from the probe Grams; *sgap (if not null) = sigma_r / sigma_{r+1} of Y
// at the kept rank r (+inf when r reaches min(p, d) or sigma_{r+1} = 0).
int probe_fit_from_grams(int p, int d, const double* xm, const double* ym, const double* gxx,
                         const double* gxy, const double* gyy, double lambda, int rank,
                         double* b_mat, double* b_vec, double* sgap);

// B' [d][d], b' [d] from X, Y [p][d].
int probe_fit(int p, int d, const double* x, const double* y, double lambda, int rank,
              double* b_mat, double* b_vec);

}  // namespace spr
