// Host-side helpers for the offline weight side of KroQuant: factor inverses,
// dense blocks, and folding T^-1 into a weight matrix.
//
// The abstract (mlsanity.com page for arXiv 2607.21446) applies the transform
// to the activations and its inverse to the weights, so the layer output is
// unchanged: (X T)(T^-1 W^T) = X W^T.  The pith.science verdict record
// (pith_extraction.key_machinery) folds that inverse into the weights offline;
// since every block is a Kronecker product of 2x2 factors, its inverse is the
// Kronecker product of the 2x2 inverses.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "../../include/kroquant.h"

namespace {

// 2x2 inverse by the adjugate, in double.  Rejects |det| < 1e-30 and
// non-finite entries.
bool inv2x2(const float *a, double *out)
{
    for (int i = 0; i < 4; ++i)
        if (!std::isfinite(a[i]))
            return false;
    const double det = (double)a[0] * a[3] - (double)a[1] * a[2];
    if (!(std::fabs(det) >= 1e-30) || !std::isfinite(det))
        return false;
    out[0] = a[3] / det;
    out[1] = -a[1] / det;
    out[2] = -a[2] / det;
    out[3] = a[0] / det;
    return true;
}

// Dense 32x32 Kronecker product of five 2x2 matrices g[k] (row-major,
// double), built factor by factor: P <- P (x) g[k].
void kron5(const double g[5][4], double *K)
{
    double P[1024], Q[1024];
    P[0] = 1.0;
    int n = 1;
    for (int k = 0; k < 5; ++k) {
        const int n2 = 2 * n;
        for (int r = 0; r < n; ++r)
            for (int c = 0; c < n; ++c)
                for (int a = 0; a < 2; ++a)
                    for (int b = 0; b < 2; ++b)
                        Q[(2 * r + a) * n2 + (2 * c + b)] = P[r * n + c] * g[k][a * 2 + b];
        std::memcpy(P, Q, sizeof(double) * n2 * n2);
        n = n2;
    }
    std::memcpy(K, P, sizeof(double) * 1024);
}

bool sets_inverse(const float *factors, int64_t t, double g[5][4])
{
    for (int k = 0; k < 5; ++k)
        if (!inv2x2(factors + t * 20 + k * 4, g[k]))
            return false;
    return true;
}

} // namespace

extern "C" {

int kq_factor_inverse(const float *factors, int64_t nT, float *inv)
{
    if (!factors || !inv || nT <= 0)
        return KQ_ERR_ARG;
    for (int64_t t = 0; t < nT; ++t) {
        double g[5][4];
        if (!sets_inverse(factors, t, g))
            return KQ_ERR_SINGULAR;
        for (int k = 0; k < 5; ++k)
            for (int i = 0; i < 4; ++i)
                inv[t * 20 + k * 4 + i] = (float)g[k][i];
    }
    return KQ_OK;
}

int kq_lu_factors(const float *lu, int64_t nT, float *factors)
{
    if (!lu || !factors || nT <= 0)
        return KQ_ERR_ARG;
    for (int64_t t = 0; t < nT; ++t) {
        for (int k = 0; k < 5; ++k) {
            const float a = lu[t * 15 + 3 * k], b = lu[t * 15 + 3 * k + 1], c = lu[t * 15 + 3 * k + 2];
            if (!(a != 0.0f) || !std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c))
                return KQ_ERR_SINGULAR;
            // the kernel's fp32 sequence: correctly rounded 1/a, c*a, fma(c, b, -1/a)
            const float r = 1.0f / a;
            const float g10 = c * a;
            const float g11 = std::fmaf(c, b, -r);
            if (!std::isfinite(r) || !std::isfinite(g10) || !std::isfinite(g11))
                return KQ_ERR_SINGULAR;
            float *g = factors + t * 20 + 4 * k;
            g[0] = a;
            g[1] = b;
            g[2] = g10;
            g[3] = g11;
        }
    }
    return KQ_OK;
}

int kq_block_matrix(const float *factors, int64_t nT, float *K)
{
    if (!factors || !K || nT <= 0)
        return KQ_ERR_ARG;
    for (int64_t t = 0; t < nT; ++t) {
        double g[5][4], D[1024];
        for (int k = 0; k < 5; ++k)
            for (int i = 0; i < 4; ++i)
                g[k][i] = factors[t * 20 + k * 4 + i];
        kron5(g, D);
        for (int i = 0; i < 1024; ++i)
            K[t * 1024 + i] = (float)D[i];
    }
    return KQ_OK;
}

int kq_block_inverse(const float *factors, int64_t nT, float *Kinv)
{
    if (!factors || !Kinv || nT <= 0)
        return KQ_ERR_ARG;
    for (int64_t t = 0; t < nT; ++t) {
        double g[5][4], D[1024];
        if (!sets_inverse(factors, t, g))
            return KQ_ERR_SINGULAR;
        kron5(g, D);
        for (int i = 0; i < 1024; ++i)
            Kinv[t * 1024 + i] = (float)D[i];
    }
    return KQ_OK;
}

int kq_fold_weight(const float *W, int64_t N, int64_t d, const float *factors, int64_t nT, float *W_out)
{
    if (!W || !W_out || !factors || N < 0 || d <= 0)
        return KQ_ERR_ARG;
    if (d % 32 != 0 || (nT != 1 && nT != d / 32))
        return KQ_ERR_SHAPE;
    const int64_t nB = d / 32;
    std::vector<double> inv((size_t)nT * 1024);
    for (int64_t t = 0; t < nT; ++t) {
        double g[5][4];
        if (!sets_inverse(factors, t, g))
            return KQ_ERR_SINGULAR;
        kron5(g, inv.data() + t * 1024);
    }
    // W_out[n, 32j + c] = sum_r W[n, 32j + r] * Kinv_j[c][r]
    double wrow[32];
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < nB; ++j) {
            const double *Ki = inv.data() + (nT == 1 ? 0 : j) * 1024;
            const float *w = W + n * d + j * 32;
            for (int r = 0; r < 32; ++r)
                wrow[r] = w[r];
            for (int c = 0; c < 32; ++c) {
                double acc = 0.0;
                for (int r = 0; r < 32; ++r)
                    acc += wrow[r] * Ki[c * 32 + r];
                W_out[n * d + j * 32 + c] = (float)acc;
            }
        }
    }
    return KQ_OK;
}

} // extern "C"
