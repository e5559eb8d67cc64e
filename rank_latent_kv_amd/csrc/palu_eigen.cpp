// Symmetric eigensolver for the group fit (host side of the fit step).
//
// Householder reduction to tridiagonal form, then the implicit-shift QL
// iteration on the tridiagonal matrix (Golub & Van Loan, "Matrix
// Computations": Householder tridiagonalisation and the implicit symmetric
// QR step; the QL variant sweeps from the bottom).  D = 128 at most, so
// this is a few million flops per (tensor, group).
//
// The fit needs every eigenvalue (for the energy rule and sigma) but only
// the eigenvectors of the r largest, so it runs in two steps: reduction and
// eigenvalues (QL without vectors), then, for the r largest eigenvalues,
// inverse iteration on the tridiagonal matrix (Gaussian elimination with
// partial pivoting, zero pivots replaced by eps |T|; each iterate
// re-orthogonalised against the vectors already found) and the
// back-transformation through the stored Householder reflectors (Golub &
// Van Loan, inverse iteration for symmetric tridiagonal matrices).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "palu_internal.h"

namespace palu {

namespace {

// sqrt(f^2 + g^2): directly when the squares can neither overflow nor
// lose the smaller operand to underflow, else with the larger magnitude
// factored out.  The rotations of a QL sweep form one dependency chain, so
// this (and one reciprocal per rotation instead of two divisions) sets the
// sweep's speed; std::hypot took most of it.
inline double pythag(double f, double g) {
    const double af = std::fabs(f), ag = std::fabs(g);
    const double a = std::max(af, ag);
    if (a > 1e-150 && a < 1e150) return std::sqrt(f * f + g * g);
    if (a == 0.0) return 0.0;
    const double q = std::min(af, ag) / a;
    return a * std::sqrt(1.0 + q * q);
}

// Implicit-shift QL on the tridiagonal (d, e); the rotations are applied to
// the rows of zt (which enters holding Q^T, so row i is column i of Q and the
// two rows a rotation touches are contiguous), or to nothing when zt is
// null (eigenvalues only).  An off-diagonal element is dropped once it is
// negligible next to its two diagonal neighbours or to the whole matrix
// (max |d_i| + |e_i|, as in the classic tql2): without the latter, clusters
// of eigenvalues at rounding level (a rank-deficient Gram matrix) need not
// converge.  Returns false on no convergence.
bool tridiagonal_ql(double *d, double *e, int n, double *zt) {
    double tnorm = 0.0;
    for (int i = 0; i < n; ++i) tnorm = std::max(tnorm, std::fabs(d[i]) + std::fabs(e[i]));
    for (int l = 0; l < n; ++l) {
        int iter = 0;
        for (;;) {
            int m = l;
            for (; m < n - 1; ++m) {
                const double scale = std::max(std::fabs(d[m]) + std::fabs(d[m + 1]), tnorm);
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
                r = pythag(f, g);
                e[i + 1] = r;
                if (r == 0.0) {  // split: restart on the smaller problem
                    d[i + 1] -= p;
                    e[m] = 0.0;
                    underflow = true;
                    break;
                }
                const double inv = 1.0 / r;
                s = f * inv;
                c = g * inv;
                g = d[i + 1] - p;
                r = (d[i] - g) * s + 2.0 * c * b;
                p = s * r;
                d[i + 1] = g + p;
                g = c * r - b;
                if (zt) {
                    double *zi = zt + i * n, *zj = zt + (i + 1) * n;
                    for (int k = 0; k < n; ++k) {
                        const double t = zj[k];
                        zj[k] = s * zi[k] + c * t;
                        zi[k] = c * zi[k] - s * t;
                    }
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

// a (n x n, row-major, symmetric) -> Q^T a Q = tridiagonal (d, e), with
// e[i] = T[i+1][i], Q = H_0 H_1 ... H_{n-3}.  Step k's reflector
// H_k = I - beta[k] v v^T (v of length n - k - 1, acting on indices k + 1 ..)
// is kept in hv[k * n ..] (beta[k] = 0 for a skipped step).
void reduce_keep(double *a, int n, double *d, double *e, double *hv, double *beta) {
    std::vector<double> p(n), w(n);
    for (int k = 0; k < n; ++k) beta[k] = 0.0;
    for (int k = 0; k + 2 < n; ++k) {
        const int m = n - k - 1;
        double *v = hv + static_cast<size_t>(k) * n;
        double norm2 = 0.0;
        for (int i = 0; i < m; ++i) {
            v[i] = a[(k + 1 + i) * n + k];
            norm2 += v[i] * v[i];
        }
        double alpha = std::sqrt(norm2);
        if (alpha == 0.0) continue;
        if (v[0] > 0) alpha = -alpha;
        v[0] -= alpha;
        double vv = 0.0;
        for (int i = 0; i < m; ++i) vv += v[i] * v[i];
        if (vv == 0.0) continue;
        const double bt = 2.0 / vv;
        // p = bt A v over the trailing block, as a sum of its rows (the
        // block is exactly symmetric: the rank-2 updates below keep it so),
        // so that the inner loop runs over independent entries of p and
        // vectorises; each p[i] still sums its terms in order j = 0 .. m-1
        for (int i = 0; i < m; ++i) p[i] = 0.0;
        for (int j = 0; j < m; ++j) {
            const double vj = v[j];
            const double *row = a + (k + 1 + j) * n + (k + 1);
            for (int i = 0; i < m; ++i) p[i] += row[i] * vj;
        }
        double pv = 0.0;
        for (int i = 0; i < m; ++i) {
            p[i] *= bt;
            pv += p[i] * v[i];
        }
        const double K = 0.5 * bt * pv;
        for (int i = 0; i < m; ++i) w[i] = p[i] - K * v[i];
        for (int i = 0; i < m; ++i) {
            double *row = a + (k + 1 + i) * n + (k + 1);
            for (int j = 0; j < m; ++j) row[j] -= v[i] * w[j] + w[i] * v[j];
        }
        a[(k + 1) * n + k] = alpha;
        a[k * n + (k + 1)] = alpha;
        for (int i = 1; i < m; ++i) {
            a[(k + 1 + i) * n + k] = 0.0;
            a[k * n + (k + 1 + i)] = 0.0;
        }
        beta[k] = bt;
    }
    for (int i = 0; i < n; ++i) d[i] = a[i * n + i];
    for (int i = 0; i + 1 < n; ++i) e[i] = a[(i + 1) * n + i];
    if (n > 0) e[n - 1] = 0.0;
}

// LU factors of T - lambda I (T tridiagonal: diagonal d, subdiagonal e) by
// Gaussian elimination with row interchanges: row i of U holds columns i,
// i + 1, i + 2 in u0, u1, u2; piv[i] tells whether rows i and i + 1 were
// swapped before eliminating with multiplier mult[i].  Pivots smaller than
// tiny in magnitude become +-tiny.
struct TriLU {
    std::vector<double> u0, u1, u2, mult;
    std::vector<char> piv;
};

void tri_factor(const double *d, const double *e, int n, double lambda, double tiny, TriLU &f) {
    f.u0.assign(n, 0.0);
    f.u1.assign(n, 0.0);
    f.u2.assign(n, 0.0);
    f.mult.assign(n, 0.0);
    f.piv.assign(n, 0);
    double a0 = d[0] - lambda, a1 = n > 1 ? e[0] : 0.0, a2 = 0.0;   // current row, columns i .. i + 2
    for (int i = 0; i + 1 < n; ++i) {
        const double b0 = e[i], b1 = d[i + 1] - lambda, b2 = i + 2 < n ? e[i + 1] : 0.0;
        if (std::fabs(a0) >= std::fabs(b0)) {
            if (std::fabs(a0) < tiny) a0 = a0 < 0.0 ? -tiny : tiny;
            const double m = b0 / a0;
            f.u0[i] = a0;
            f.u1[i] = a1;
            f.u2[i] = a2;
            f.mult[i] = m;
            a0 = b1 - m * a1;
            a1 = b2 - m * a2;
        } else {
            const double m = a0 / b0;
            f.piv[i] = 1;
            f.u0[i] = b0;
            f.u1[i] = b1;
            f.u2[i] = b2;
            f.mult[i] = m;
            a0 = a1 - m * b1;
            a1 = a2 - m * b2;
        }
        a2 = 0.0;
    }
    if (std::fabs(a0) < tiny) a0 = a0 < 0.0 ? -tiny : tiny;
    f.u0[n - 1] = a0;
}

// x <- (T - lambda I)^-1 x with the factors of tri_factor
void tri_solve(const TriLU &f, int n, double *x) {
    for (int i = 0; i + 1 < n; ++i) {
        if (f.piv[i]) std::swap(x[i], x[i + 1]);
        x[i + 1] -= f.mult[i] * x[i];
    }
    for (int i = n - 1; i >= 0; --i) {
        double v = x[i];
        if (i + 1 < n) v -= f.u1[i] * x[i + 1];
        if (i + 2 < n) v -= f.u2[i] * x[i + 2];
        x[i] = v / f.u0[i];
    }
}

}  // namespace

bool sym_eigenvalues(double *a, int n, SymEigen &s) {
    s.n = n;
    s.hv.assign(static_cast<size_t>(n) * n, 0.0);
    s.beta.assign(n, 0.0);
    s.d.assign(n, 0.0);
    s.e.assign(n > 0 ? n : 1, 0.0);
    reduce_keep(a, n, s.d.data(), s.e.data(), s.hv.data(), s.beta.data());
    s.w = s.d;
    std::vector<double> e = s.e;
    if (!tridiagonal_ql(s.w.data(), e.data(), n, nullptr)) return false;
    std::sort(s.w.begin(), s.w.end(), [](double x, double y) { return x > y; });
    return true;
}

void sym_top_vectors(const SymEigen &s, int k, double *z) {
    const int n = s.n;
    double norm = 0.0;   // max absolute row sum of T
    for (int i = 0; i < n; ++i) {
        double r = std::fabs(s.d[i]);
        if (i > 0) r += std::fabs(s.e[i - 1]);
        if (i + 1 < n) r += std::fabs(s.e[i]);
        norm = std::max(norm, r);
    }
    const double tiny = norm > 0.0 ? 2.2e-16 * norm : 1e-300;
    std::vector<double> xs(static_cast<size_t>(k) * n), x(n);
    TriLU f;
    for (int j = 0; j < k; ++j) {
        tri_factor(s.d.data(), s.e.data(), n, s.w[j], tiny, f);
        // deterministic start vector with no special structure
        uint32_t st = 2654435761u * static_cast<uint32_t>(j + 1);
        for (int i = 0; i < n; ++i) {
            st = st * 1664525u + 1013904223u;
            x[i] = static_cast<double>(st >> 8) / 16777216.0 - 0.5;
        }
        for (int it = 0; it < 3; ++it) {
            tri_solve(f, n, x.data());
            for (int p = 0; p < j; ++p) {   // orthogonal to the vectors already found
                const double *y = xs.data() + static_cast<size_t>(p) * n;
                double dot = 0.0;
                for (int i = 0; i < n; ++i) dot += y[i] * x[i];
                for (int i = 0; i < n; ++i) x[i] -= dot * y[i];
            }
            double nr = 0.0;
            for (int i = 0; i < n; ++i) nr += x[i] * x[i];
            nr = std::sqrt(nr);
            if (nr == 0.0) {                // degenerate start: a unit vector orthogonal to the rest
                x.assign(n, 0.0);
                x[j % n] = 1.0;
                nr = 1.0;
            }
            for (int i = 0; i < n; ++i) x[i] /= nr;
        }
        std::copy(x.begin(), x.end(), xs.begin() + static_cast<size_t>(j) * n);
    }
    // z = Q x: reflectors applied last to first
    for (int j = 0; j < k; ++j) {
        double *y = xs.data() + static_cast<size_t>(j) * n;
        for (int kk = n - 3; kk >= 0; --kk) {
            const double bt = s.beta[kk];
            if (bt == 0.0) continue;
            const double *v = s.hv.data() + static_cast<size_t>(kk) * n;
            const int m = n - kk - 1;
            double dot = 0.0;
            for (int i = 0; i < m; ++i) dot += v[i] * y[kk + 1 + i];
            dot *= bt;
            for (int i = 0; i < m; ++i) y[kk + 1 + i] -= dot * v[i];
        }
        for (int i = 0; i < n; ++i) z[static_cast<size_t>(i) * k + j] = y[i];
    }
}

}  // namespace palu
