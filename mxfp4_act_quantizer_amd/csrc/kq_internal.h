// Internal launch interface between the C ABI (kq_capi.hip) and the kernels
// (kq_kernels.hip).  Arguments are already validated when these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// Launch tuning knobs (chosen on MI355X measurements; see the launch code).
struct Tuning {
    int mfma_tiles_per_wave;  // 0 = automatic
    int bfly_rows_per_wave;   // 0 = automatic
    int stream_rows_per_wave; // 0 = automatic
    int mfma_interleave;      // 0 = automatic, 1 = contiguous token groups, 2 = interleaved groups
    int mfma_strip;           // 0 = automatic, 8 or 16 blocks per workgroup
    int mfma_order;           // 0 = automatic, 1 = XCD-grouped workgroups, 2 = flat order
    int adaln_blocks_per_wave;    // 0 = automatic: row blocks per wave of the AdaLN front-end's second pass
    int gemm_variant;         // 0 = automatic, 1 = per-tile kernel, 2 / 3 = persistent, k chunks of 256 / 128
    int adaln_pass;           // 0 = automatic, 1 = matrix-core second pass, 2 = butterfly second pass
    int adaln_strip;          // 0 = automatic, 4 or 8 blocks per workgroup of the matrix-core second pass
};
Tuning &tuning();

// factors: [nT,5,2,2] 2x2 factors (lu = 0) or [nT,5,3] LU scalars (lu = 1)
hipError_t launch_kq_mfma(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                          uint8_t *s, float *y, int lu, hipStream_t stream);
hipError_t launch_kq_butterfly(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT,
                               uint8_t *q, uint8_t *s, float *y, hipStream_t stream);
// 16-element blocks, four factors per set [nT, 4, 2, 2] (nT = 1 or d/16):
// quantize into q [M, d/2], s [M, d/16] (y null) or export y
hipError_t launch_kq16(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                       uint8_t *s, float *y, hipStream_t stream);
hipError_t launch_sq(const uint16_t *x, int64_t M, int64_t d, const float *scale, uint8_t *q, uint8_t *s,
                     hipStream_t stream);
hipError_t launch_mx_f32(const float *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, hipStream_t stream);
// W4A4 product of two MXFP4 matrices in the quantizer's layout: out[M, N]
// (float32, or bf16 when bf16 != 0) = A[M, K] . B[N, K]^T
hipError_t launch_mx_gemm(const uint8_t *qa, const uint8_t *sa, int64_t M, const uint8_t *qb, const uint8_t *sb,
                          int64_t N, int64_t K, void *out, int bf16, hipStream_t stream);
// AdaLN front-end: row statistics (mean, 1/sqrt(var + eps), fp64) into the
// workspace stats [M, 2], then x = LayerNorm(h) (1 + scale[m / T]) +
// shift[m / T] rounded to bf16 and either (x null) the transform and MXFP4
// into q, s (the matrix-core second pass, or the butterfly one when the
// tuning selects it), or (x given) x written out.  Two launches on `stream`.
hipError_t launch_adaln(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale, int64_t T,
                        float eps, const float *factors, int64_t nT, double *stats, uint8_t *q, uint8_t *s,
                        uint16_t *x, hipStream_t stream);
// Second pass of the AdaLN front-end on the matrix cores: h normalised with
// the statistics workspace and modulated while it is staged, then the MFMA
// transform and MXFP4 into q, s.  One launch on `stream`.
hipError_t launch_adaln_mfma(const uint16_t *h, int64_t M, int64_t d, const double *stats, const float *shift,
                             const float *scale, int64_t T, const float *factors, int64_t nT, uint8_t *q, uint8_t *s,
                             hipStream_t stream);
// normalised Walsh-Hadamard-32 comparison: quantize (y null) or export y
hipError_t launch_fwht(const uint16_t *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, float *y, hipStream_t stream);

// Largest row count / width the launchers accept (grid and 32-bit lane math).
constexpr int64_t kMaxD = (int64_t)1 << 20;
constexpr int64_t kMaxBlocksTotal = (int64_t)1 << 40;

} // namespace kq
