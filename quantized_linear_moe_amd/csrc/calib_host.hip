// Host side of the calibration statistic that follows the co-occurrence counts:
// frequency order of the channels, the NPMI similarity, the normalized-Laplacian
// spectral embedding and K-Means.  Plain C++ (no device code): this runs once per layer
// at calibration time on matrices of N_r * k channels (256 with the pages' settings).
//
// MCISLAB DeepRead summary of "Quant Experts", section "Method": channels ordered by
// selection frequency (the first k token-independent, the next N_r * k token-dependent);
// similarity of the token-dependent channels by NPMI, spectral clustering on the
// normalized Laplacian, K-Means into N_r clusters.  PaperDaily post
// "西交大提出Quant Experts：token级量化补偿", section "核心设计": p(i), p(i, j), NPMI in
// [-1, 1], weak pairs removed by a threshold such as 0.2.
//
// Readings where the pages stop short: NPMI is -1 for pairs never seen together and +1
// for pairs present in every token; pairs below the threshold get similarity 0; the
// spectral step is the algorithm of Ng, Jordan and Weiss (eigenvectors of the smallest
// eigenvalues of I - D^-1/2 S D^-1/2, rows scaled to unit length); K-Means is Lloyd's
// iteration seeded by farthest-point selection from row 0, ties to the lower index, and
// the labels are numbered in order of each cluster's lowest member.

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <numeric>
#include <vector>

#include "qe_calib.h"

namespace qe {

void frequency_order(const uint32_t* hist, int d_in, int32_t* order) {
    std::vector<int32_t> idx(d_in);
    std::iota(idx.begin(), idx.end(), 0);
    // stable: equal counts keep ascending channel order
    std::stable_sort(idx.begin(), idx.end(), [hist](int32_t a, int32_t b) { return hist[a] > hist[b]; });
    std::copy(idx.begin(), idx.end(), order);
}

// Symmetric eigendecomposition in two textbook stages (Golub and Van Loan, "Matrix
// Computations", sections 8.3.1 and 8.3.3): Householder reduction to tridiagonal form with
// the reflections accumulated, then implicit-shift QR steps (Wilkinson shift, bulge
// chasing with Givens rotations) with deflation of negligible off-diagonal entries.
int symmetric_eigen(double* A, int n, double* eigvals, double* V) {
    std::vector<double> Q((size_t)n * n, 0.0);
    for (int i = 0; i < n; ++i) Q[(size_t)i * n + i] = 1.0;
    auto a = [A, n](int i, int j) -> double& { return A[(size_t)i * n + j]; };

    std::vector<double> v(n), p(n), q(n);
    for (int k = 0; k + 2 < n; ++k) {
        double norm2 = 0.0;
        for (int i = k + 1; i < n; ++i) norm2 += a(i, k) * a(i, k);
        const double x0 = a(k + 1, k);
        const double alpha = -std::copysign(std::sqrt(norm2), x0);
        const double vnorm2 = norm2 - x0 * x0 + (x0 - alpha) * (x0 - alpha);
        if (!(vnorm2 > 0.0)) continue;  // the column is already reduced
        const double inv = 1.0 / std::sqrt(vnorm2);
        for (int i = k + 1; i < n; ++i) v[i] = a(i, k) * inv;
        v[k + 1] = (x0 - alpha) * inv;
        // H A22 H with H = I - 2 v v^T:  A22 - 2 (v w^T + w v^T), w = A22 v - (v^T A22 v) v
        double kv = 0.0;
        for (int i = k + 1; i < n; ++i) {
            double s = 0.0;
            for (int j = k + 1; j < n; ++j) s += a(i, j) * v[j];
            p[i] = s;
            kv += v[i] * s;
        }
        for (int i = k + 1; i < n; ++i) q[i] = p[i] - kv * v[i];
        for (int i = k + 1; i < n; ++i)
            for (int j = k + 1; j < n; ++j) a(i, j) -= 2.0 * (v[i] * q[j] + q[i] * v[j]);
        a(k + 1, k) = a(k, k + 1) = alpha;
        for (int i = k + 2; i < n; ++i) a(i, k) = a(k, i) = 0.0;
        // Q <- Q H on columns k+1 .. n-1
        for (int r = 0; r < n; ++r) {
            double* qr = &Q[(size_t)r * n];
            double s = 0.0;
            for (int j = k + 1; j < n; ++j) s += qr[j] * v[j];
            for (int j = k + 1; j < n; ++j) qr[j] -= 2.0 * s * v[j];
        }
    }

    std::vector<double> d(n), e(n, 0.0);
    for (int i = 0; i < n; ++i) d[i] = a(i, i);
    for (int i = 0; i + 1 < n; ++i) e[i] = a(i + 1, i);
    auto negligible = [&](int i) {  // e[i] couples i and i+1
        return std::fabs(e[i]) <= DBL_EPSILON * (std::fabs(d[i]) + std::fabs(d[i + 1])) ||
               std::fabs(e[i]) < DBL_MIN;
    };

    int hi = n - 1, iter = 0;
    while (hi > 0) {
        if (negligible(hi - 1)) {
            e[hi - 1] = 0.0;
            --hi;
            iter = 0;
            continue;
        }
        if (++iter > 64) return -1;
        int lo = hi - 1;
        while (lo > 0 && !negligible(lo - 1)) --lo;
        if (lo > 0) e[lo - 1] = 0.0;
        // Wilkinson shift: the eigenvalue of the trailing 2 x 2 block nearer to d[hi]
        const double delta = 0.5 * (d[hi - 1] - d[hi]);
        const double b = e[hi - 1];
        const double mu = d[hi] - b * b / (delta + std::copysign(std::hypot(delta, b), delta));
        double x = d[lo] - mu, z = e[lo];
        for (int k = lo; k < hi; ++k) {
            const double r = std::hypot(x, z);
            const double c = r > 0.0 ? x / r : 1.0, s = r > 0.0 ? z / r : 0.0;
            if (k > lo) e[k - 1] = r;
            const double dk = d[k], dk1 = d[k + 1], ek = e[k];
            d[k] = c * c * dk + 2.0 * c * s * ek + s * s * dk1;
            d[k + 1] = s * s * dk - 2.0 * c * s * ek + c * c * dk1;
            e[k] = c * s * (dk1 - dk) + (c * c - s * s) * ek;
            if (k + 1 < hi) {  // the rotation pushes a bulge to (k, k + 2)
                z = s * e[k + 1];
                e[k + 1] *= c;
                x = e[k];
            }
            for (int r2 = 0; r2 < n; ++r2) {
                double* qr = &Q[(size_t)r2 * n];
                const double qa = qr[k], qb = qr[k + 1];
                qr[k] = c * qa + s * qb;
                qr[k + 1] = -s * qa + c * qb;
            }
        }
    }

    std::vector<int> order(n);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&d](int x1, int x2) { return d[x1] < d[x2]; });
    for (int m = 0; m < n; ++m) {
        eigvals[m] = d[order[m]];
        for (int r = 0; r < n; ++r) V[(size_t)r * n + m] = Q[(size_t)r * n + order[m]];
    }
    return 0;
}

namespace {

double npmi(uint32_t cij, uint32_t cii, uint32_t cjj, int64_t T) {
    if (cij == 0) return -1.0;
    if ((int64_t)cij == T) return 1.0;
    const double pij = (double)cij / (double)T;
    const double pi = (double)cii / (double)T, pj = (double)cjj / (double)T;
    return std::log(pij / (pi * pj)) / -std::log(pij);
}

double sqdist(const double* x, const double* y, int m) {
    double s = 0.0;
    for (int c = 0; c < m; ++c) s += (x[c] - y[c]) * (x[c] - y[c]);
    return s;
}

// Lloyd's K-Means on n points of dimension m (row-major U), K clusters.
void kmeans(const std::vector<double>& U, int n, int m, int K, int32_t* labels) {
    std::vector<double> cent((size_t)K * m);
    std::vector<double> dmin(n);
    std::copy(U.begin(), U.begin() + m, cent.begin());
    for (int i = 0; i < n; ++i) dmin[i] = sqdist(&U[(size_t)i * m], &cent[0], m);
    for (int c = 1; c < K; ++c) {
        int far = 0;
        for (int i = 1; i < n; ++i)
            if (dmin[i] > dmin[far]) far = i;
        std::copy(U.begin() + (size_t)far * m, U.begin() + (size_t)far * m + m, cent.begin() + (size_t)c * m);
        for (int i = 0; i < n; ++i) dmin[i] = std::min(dmin[i], sqdist(&U[(size_t)i * m], &cent[(size_t)c * m], m));
    }
    std::vector<int> lab(n, -1), cnt(K);
    std::vector<double> sum((size_t)K * m);
    for (int it = 0; it < 300; ++it) {
        bool moved = false;
        for (int i = 0; i < n; ++i) {
            int best = 0;
            double bd = sqdist(&U[(size_t)i * m], &cent[0], m);
            for (int c = 1; c < K; ++c) {
                const double dc = sqdist(&U[(size_t)i * m], &cent[(size_t)c * m], m);
                if (dc < bd) {
                    bd = dc;
                    best = c;
                }
            }
            moved |= lab[i] != best;
            lab[i] = best;
        }
        if (!moved) break;
        std::fill(sum.begin(), sum.end(), 0.0);
        std::fill(cnt.begin(), cnt.end(), 0);
        for (int i = 0; i < n; ++i) {
            ++cnt[lab[i]];
            for (int c = 0; c < m; ++c) sum[(size_t)lab[i] * m + c] += U[(size_t)i * m + c];
        }
        for (int c = 0; c < K; ++c)
            if (cnt[c] > 0)
                for (int q = 0; q < m; ++q) cent[(size_t)c * m + q] = sum[(size_t)c * m + q] / cnt[c];
    }
    std::vector<int> rename(K, -1);
    int next = 0;
    for (int i = 0; i < n; ++i) {
        if (rename[lab[i]] < 0) rename[lab[i]] = next++;
        labels[i] = rename[lab[i]];
    }
}

}  // namespace

int spectral_cluster(const uint32_t* cooc, int n, int64_t T, int n_clusters, double threshold, int32_t* labels,
                     double* similarity, double* eigvals, double* embedding) {
    std::vector<double> S((size_t)n * n);
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) {
            const double v = npmi(cooc[(size_t)i * n + j], cooc[(size_t)i * n + i], cooc[(size_t)j * n + j], T);
            S[(size_t)i * n + j] = v >= threshold ? v : 0.0;
        }
    if (similarity) std::copy(S.begin(), S.end(), similarity);

    std::vector<double> inv(n, 0.0);
    for (int i = 0; i < n; ++i) {
        double deg = 0.0;
        for (int j = 0; j < n; ++j) deg += S[(size_t)i * n + j];
        if (deg > 0.0) inv[i] = 1.0 / std::sqrt(deg);
    }
    std::vector<double> L((size_t)n * n);
    for (int i = 0; i < n; ++i)
        for (int j = 0; j < n; ++j) L[(size_t)i * n + j] = (i == j ? 1.0 : 0.0) - inv[i] * S[(size_t)i * n + j] * inv[j];

    std::vector<double> w(n), V((size_t)n * n);
    if (symmetric_eigen(L.data(), n, w.data(), V.data()) != 0) return -1;

    const int m = n_clusters;
    std::vector<double> U((size_t)n * m);
    for (int i = 0; i < n; ++i) {
        double nrm = 0.0;
        for (int c = 0; c < m; ++c) nrm += V[(size_t)i * n + c] * V[(size_t)i * n + c];
        nrm = std::sqrt(nrm);
        for (int c = 0; c < m; ++c) U[(size_t)i * m + c] = nrm > 0.0 ? V[(size_t)i * n + c] / nrm : 0.0;
    }
    if (eigvals) std::copy(w.begin(), w.begin() + m, eigvals);
    if (embedding) std::copy(U.begin(), U.end(), embedding);
    kmeans(U, n, m, n_clusters, labels);
    return 0;
}

}  // namespace qe
