// Winograd F(m x m, 3 x 3) transform matrices, built at compile time from the
// Cook-Toom construction (m = 2 or 6).  With alpha = m + 2 interpolation
// points (one may be "infinity", which evaluates a polynomial to its leading
// coefficient), V_n evaluates an n-coefficient polynomial at the points;
// linear convolution is V^-1 [(V_3 g) * (V_m u)] and correlation is its
// transpose, so A^T = V_m^T, G = V_3, B^T = V^-T and
//   Y = A^T [ (G g G^T) * (B^T d B) ] A   over alpha x alpha input tiles d.
// Points: {0, 1, -1, inf} for m = 2; {0, +-1, +-2, +-1/2, inf} for m = 6.
#pragma once

namespace cfwd {
namespace wg {

template <int M> struct Mats {
    static constexpr int A = M + 2;
    double at[M][A] = {};
    double g[A][3] = {};
    double bt[A][A] = {};
};

constexpr double kInf = 1e300;  // marks the point at infinity

template <int M>
constexpr Mats<M> build_mats() {
    constexpr int A = M + 2;
    double pts[A] = {};
    if (M == 2) {
        const double p[4] = {0.0, 1.0, -1.0, kInf};
        for (int i = 0; i < 4; ++i) pts[i] = p[i];
    } else {
        const double p[8] = {0.0, 1.0, -1.0, 2.0, -2.0, 0.5, -0.5, kInf};
        for (int i = 0; i < 8; ++i) pts[i] = p[i];
    }
    // evaluation matrices
    double v[A][A] = {};
    for (int i = 0; i < A; ++i)
        for (int j = 0; j < A; ++j) {
            if (pts[i] == kInf) {
                v[i][j] = (j == A - 1) ? 1.0 : 0.0;
            } else {
                double x = 1.0;
                for (int e = 0; e < j; ++e) x *= pts[i];
                v[i][j] = x;
            }
        }
    Mats<M> r{};
    for (int i = 0; i < A; ++i) {
        for (int j = 0; j < M; ++j) {
            double x = 1.0;
            if (pts[i] == kInf) {
                x = (j == M - 1) ? 1.0 : 0.0;
            } else {
                for (int e = 0; e < j; ++e) x *= pts[i];
            }
            r.at[j][i] = x;  // A^T = V_m^T
        }
        for (int j = 0; j < 3; ++j) {
            double x = 1.0;
            if (pts[i] == kInf) {
                x = (j == 2) ? 1.0 : 0.0;
            } else {
                for (int e = 0; e < j; ++e) x *= pts[i];
            }
            r.g[i][j] = x;  // G = V_3
        }
    }
    // V^-1 by Gauss-Jordan with partial pivoting
    double aug[A][2 * A] = {};
    for (int i = 0; i < A; ++i)
        for (int j = 0; j < A; ++j) {
            aug[i][j] = v[i][j];
            aug[i][A + j] = (i == j) ? 1.0 : 0.0;
        }
    for (int col = 0; col < A; ++col) {
        int piv = col;
        for (int rr = col + 1; rr < A; ++rr) {
            const double a = aug[rr][col] < 0 ? -aug[rr][col] : aug[rr][col];
            const double b = aug[piv][col] < 0 ? -aug[piv][col] : aug[piv][col];
            if (a > b) piv = rr;
        }
        for (int j = 0; j < 2 * A; ++j) {
            const double t = aug[col][j];
            aug[col][j] = aug[piv][j];
            aug[piv][j] = t;
        }
        const double inv = 1.0 / aug[col][col];
        for (int j = 0; j < 2 * A; ++j) aug[col][j] *= inv;
        for (int rr = 0; rr < A; ++rr) {
            if (rr == col) continue;
            const double f = aug[rr][col];
            if (f == 0.0) continue;
            for (int j = 0; j < 2 * A; ++j) aug[rr][j] -= f * aug[col][j];
        }
    }
    for (int i = 0; i < A; ++i)
        for (int j = 0; j < A; ++j) r.bt[i][j] = aug[j][A + i];  // B^T = (V^-1)^T
    return r;
}

template <int M> struct MatsF {
    static constexpr Mats<M> d = build_mats<M>();
};

}  // namespace wg
}  // namespace cfwd
