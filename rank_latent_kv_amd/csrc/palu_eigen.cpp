// Symmetric eigensolver for the group fit (host side of the fit step).
//
// Householder reduction to tridiagonal form, then the implicit-shift QL
// iteration on the tridiagonal matrix (Golub & Van Loan, "Matrix
// Computations": Householder tridiagonalisation and the implicit symmetric
// QR step; the QL variant sweeps from the bottom).  D = 128 at most, so
// this is a few million flops per (tensor, group).
#include <cmath>
#include <vector>

#include "palu_internal.h"

namespace palu {

namespace {

// a (n x n, row-major, symmetric) -> Q^T a Q = tridiagonal (d, e), with
// e[i] = T[i+1][i].  q receives Q (row-major).
void tridiagonalize(double *a, int n, double *d, double *e, double *q) {
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) q[i * n + j] = (i == j) ? 1.0 : 0.0;
    std::vector<double> v(n), p(n), w(n);
    for (int k = 0; k + 2 < n; ++k) {
        const int m = n - k - 1;  // length of the column below the diagonal
        double norm2 = 0.0;
        for (int i = 0; i < m; ++i) {
            v[i] = a[(k + 1 + i) * n + k];
            norm2 += v[i] * v[i];
        }
        double alpha = std::sqrt(norm2);
        if (alpha == 0.0) continue;
        if (v[0] > 0) alpha = -alpha;  // reflect onto -sign(x0) ||x|| e1
        v[0] -= alpha;
        double vv = 0.0;
        for (int i = 0; i < m; ++i) vv += v[i] * v[i];
        if (vv == 0.0) continue;
        const double beta = 2.0 / vv;
        // p = beta * A22 v ; K = beta/2 * p.v ; w = p - K v
        double pv = 0.0;
        for (int i = 0; i < m; ++i) {
            double acc = 0.0;
            const double *row = a + (k + 1 + i) * n + (k + 1);
            for (int j = 0; j < m; ++j) acc += row[j] * v[j];
            p[i] = beta * acc;
            pv += p[i] * v[i];
        }
        const double K = 0.5 * beta * pv;
        for (int i = 0; i < m; ++i) w[i] = p[i] - K * v[i];
        // A22 <- A22 - v w^T - w v^T
        for (int i = 0; i < m; ++i) {
            double *row = a + (k + 1 + i) * n + (k + 1);
            for (int j = 0; j < m; ++j) row[j] -= v[i] * w[j] + w[i] * v[j];
        }
        // column k / row k below the diagonal become alpha e1
        a[(k + 1) * n + k] = alpha;
        a[k * n + (k + 1)] = alpha;
        for (int i = 1; i < m; ++i) {
            a[(k + 1 + i) * n + k] = 0.0;
            a[k * n + (k + 1 + i)] = 0.0;
        }
        // Q[:, k+1:] <- Q[:, k+1:] (I - beta v v^T)
        for (int r = 0; r < n; ++r) {
            double *row = q + r * n + (k + 1);
            double s = 0.0;
            for (int j = 0; j < m; ++j) s += row[j] * v[j];
            s *= beta;
            for (int j = 0; j < m; ++j) row[j] -= s * v[j];
        }
    }
    for (int i = 0; i < n; ++i) d[i] = a[i * n + i];
    for (int i = 0; i + 1 < n; ++i) e[i] = a[(i + 1) * n + i];
    if (n > 0) e[n - 1] = 0.0;
}

// Implicit-shift QL on the tridiagonal (d, e); the rotations are applied to
// the rows of zt (which enters holding Q^T, so row i is column i of Q and the
// two rows a rotation touches are contiguous).  Returns false on no
// convergence.
bool tridiagonal_ql(double *d, double *e, int n, double *zt) {
    for (int l = 0; l < n; ++l) {
        int iter = 0;
        for (;;) {
            int m = l;
            for (; m < n - 1; ++m) {
                const double scale = std::fabs(d[m]) + std::fabs(d[m + 1]);
                if (std::fabs(e[m]) <= 1e-300 + 2.2e-16 * scale) break;
            }
            if (m == l) break;
            if (++iter > 60) return false;
            // shift: eigenvalue of the leading 2x2 block closer to d[l]
            double g = (d[l + 1] - d[l]) / (2.0 * e[l]);
            double r = std::hypot(g, 1.0);
            g = d[m] - d[l] + e[l] / (g + std::copysign(r, g));
            double s = 1.0, c = 1.0, p = 0.0;
            int i = m - 1;
            bool underflow = false;
            for (; i >= l; --i) {
                const double f = s * e[i];
                const double b = c * e[i];
                r = std::hypot(f, g);
                e[i + 1] = r;
                if (r == 0.0) {  // split: restart on the smaller problem
                    d[i + 1] -= p;
                    e[m] = 0.0;
                    underflow = true;
                    break;
                }
                s = f / r;
                c = g / r;
                g = d[i + 1] - p;
                r = (d[i] - g) * s + 2.0 * c * b;
                p = s * r;
                d[i + 1] = g + p;
                g = c * r - b;
                double *zi = zt + i * n, *zj = zt + (i + 1) * n;
                for (int k = 0; k < n; ++k) {
                    const double t = zj[k];
                    zj[k] = s * zi[k] + c * t;
                    zi[k] = c * zi[k] - s * t;
                }
            }
            if (underflow) continue;
            d[l] -= p;
            e[l] = g;
            e[m] = 0.0;
        }
    }
    return true;
}

}  // namespace

bool sym_eigen(double *a, int n, double *w, double *z) {
    std::vector<double> e(n > 0 ? n : 1), zt(static_cast<size_t>(n) * n);
    tridiagonalize(a, n, w, e.data(), z);
    for (int i = 0; i < n; ++i)
        for (int k = 0; k < n; ++k) zt[static_cast<size_t>(i) * n + k] = z[static_cast<size_t>(k) * n + i];
    if (!tridiagonal_ql(w, e.data(), n, zt.data())) return false;
    for (int i = 0; i < n; ++i)
        for (int k = 0; k < n; ++k) z[static_cast<size_t>(k) * n + i] = zt[static_cast<size_t>(i) * n + k];
    return true;
}

}  // namespace palu
