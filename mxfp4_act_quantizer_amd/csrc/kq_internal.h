// Internal launch interface between the C ABI (kq_capi.hip) and the kernels
// (kq_kernels.hip, kq_adaln.hip, kq_gemm.hip).  Arguments are already
// validated when these are called.  Every launcher takes its launch-shape
// overrides as an argument (kq_tuning from the public header; all fields 0
// means the automatic choices the product entry points use), so no launch
// reads mutable process state.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kroquant.h"

namespace kq {

using Tuning = kq_tuning;

// Thread-safe per-device queries, filled once per (device, kernel) under a lock.
int device_cus();                                  // compute units of the current device
int occupancy_per_cu(const void *fn, int threads); // resident workgroups per CU of fn on the current device
hipError_t allow_dynamic_lds(const void *fn, int bytes); // raise fn's dynamic LDS limit (once per device)

// Launch shape the MFMA quantizer picks for (M, d): strip width, tiles per
// workgroup, interleaved token groups, flat workgroup order, grid.  The
// transform export (y) uses the same shape as the quantizer.
struct MfmaShape {
    int strip;
    int tiles_per_wg;
    int interleave;
    int flat;
    int64_t grid;
    int nt_codes; // 1 when the code stores are nontemporal
    int ring;     // register ring depth in tiles (2 or 4)
};
hipError_t mfma_launch_shape(int64_t M, int64_t d, const Tuning &tn, bool adaln, MfmaShape &out);

// Launch shape of the flat form (one shared factor set): register ring depth
// in units of 32 blocks, workgroups of 4 waves, nontemporal code stores.
// kq_quantize / kq_transform_f32 / the LU calls take this form when nT = 1
// and no strip-kernel override is set (flat_form); kq_quantize16 and
// kq_transform16_f32 with nT = 1 take its 16-element form (b16).
struct FlatShape {
    int ring;
    int64_t wgs;
    int nt_codes;
};
bool flat_form(int64_t nT, const Tuning &tn);
// b16: 16-element blocks (one scale byte per 16 elements in the footprint)
void flat_launch_shape(int64_t M, int64_t d, const Tuning &tn, FlatShape &out, bool b16 = false);

// factors: [nT,5,2,2] 2x2 factors (lu = 0) or [nT,5,3] LU scalars (lu = 1)
hipError_t launch_kq_mfma(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                          uint8_t *s, float *y, int lu, const Tuning &tn, hipStream_t stream);
hipError_t launch_kq_butterfly(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT,
                               uint8_t *q, uint8_t *s, float *y, const Tuning &tn, hipStream_t stream);
// 16-element blocks, four factors per set [nT, 4, 2, 2] (nT = 1 or d/16):
// quantize into q [M, d/2], s [M, d/16] (y null) or export y
hipError_t launch_kq16(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                       uint8_t *s, float *y, const Tuning &tn, hipStream_t stream);
hipError_t launch_sq(const uint16_t *x, int64_t M, int64_t d, const float *scale, uint8_t *q, uint8_t *s,
                     const Tuning &tn, hipStream_t stream);
hipError_t launch_mx_f32(const float *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, const Tuning &tn,
                         hipStream_t stream);
// W4A4 product of two MXFP4 matrices in the quantizer's layout: out[M, N]
// (float32, or bf16 when bf16 != 0) = A[M, K] . B[N, K]^T
hipError_t launch_mx_gemm(const uint8_t *qa, const uint8_t *sa, int64_t M, const uint8_t *qb, const uint8_t *sb,
                          int64_t N, int64_t K, void *out, int bf16, const Tuning &tn, hipStream_t stream);
// AdaLN front-end: row statistics (mean, 1/sqrt(var + eps), fp64) into the
// workspace stats [M, 2], then x = LayerNorm(h) (1 + scale[m / T]) +
// shift[m / T] rounded to bf16 and either (x null) the transform and MXFP4
// into q, s (the matrix-core second pass, or the butterfly one when the
// tuning selects it), or (x given) x written out.  Two launches on `stream`,
// or one (x null) when the tuning selects the one-launch form.
hipError_t launch_adaln(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale, int64_t T,
                        float eps, const float *factors, int64_t nT, double *stats, uint8_t *q, uint8_t *s,
                        uint16_t *x, const Tuning &tn, hipStream_t stream);
// The AdaLN front-end in one launch (x null only): workgroups own whole token
// rows, R at a time, held in LDS (statistics, normalisation, transform and
// MXFP4 from there; stats written as by the two-launch form).  LDS layout of a
// workgroup: x rows (pitch xrow), staged codes at qoff (pitch qrow), scale
// bytes at soff (pitch srow), per-row (mean, 1/sqrt(var + eps)) at toff, the
// factor sets at foff, and at moff the shift rows then (mbytes later) the
// scale rows of up to nmod samples.
struct AdRowsLayout {
    int xrow, qrow, srow;
    int qoff, soff, toff, foff, moff, mbytes, nmod, bytes;
};
struct AdRowsShape {
    int R, nmod, bytes;
    int64_t grid;
};
// Rows per tile, staged samples and grid of the one-launch form for (M, d,
// nT); false when too few rows fit the LDS (the two-launch form then runs).
bool adaln_rows_shape(int64_t M, int64_t d, int64_t nT, AdRowsShape &sh);
hipError_t launch_adaln_rows(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                             int64_t T, float eps, const float *factors, int64_t nT, double *stats, uint8_t *q,
                             uint8_t *s, hipStream_t stream);
// Second pass of the AdaLN front-end on the matrix cores: h normalised with
// the statistics workspace and modulated while it is staged, then the MFMA
// transform and MXFP4 into q, s.  One launch on `stream`.
hipError_t launch_adaln_mfma(const uint16_t *h, int64_t M, int64_t d, const double *stats, const float *shift,
                             const float *scale, int64_t T, const float *factors, int64_t nT, uint8_t *q, uint8_t *s,
                             const Tuning &tn, hipStream_t stream);
// normalised Walsh-Hadamard-32 comparison: quantize (y null) or export y
hipError_t launch_fwht(const uint16_t *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, float *y, const Tuning &tn,
                       hipStream_t stream);

// Largest row count / width the launchers accept (grid and 32-bit lane math).
constexpr int64_t kMaxD = (int64_t)1 << 20;
constexpr int64_t kMaxBlocksTotal = (int64_t)1 << 40;

} // namespace kq
