// AdaLN front-end of the KroQuant quantizer, fused (pages describing arXiv
// 2607.21446: the abstract on the mlsanity.com paper page says the
// normalisation layers between transformer blocks force the transform to run
// online at every step; the pith.science verdict record's
// referee_report.summary names AdaLN as what prevents absorbing it offline).
//
// Per token row m (sample b = m / T):
//   x_c = (h_c - mean) / sqrt(var + eps) * (1 + scale[b][c]) + shift[b][c]
// (LayerNorm without affine, biased variance), rounded to bf16, then the
// Kronecker transform of every 32-channel block and MXFP4 - in one pass over
// h, so the normalised x never goes to memory.
//
// Structure: a workgroup spans whole rows (one wave per 512 channels, up to
// 16 waves, so d <= 8192: the hidden widths AdaLN normalises) and walks a run
// of rows, two at a time.  Each lane keeps its 8 channels for the whole run:
// its butterfly factors and the current sample's modulation stay in
// registers.  Row statistics: each lane sums its values and squares in fp64,
// the wave reduces, the waves meet in LDS, and every wave adds the partials
// in the same order, so all waves (and the x-writing variant) see identical
// mean and 1/sqrt(var + eps).  The per-element arithmetic is fp64 and the
// bf16 rounding is taken from the double value.  The transform is the
// butterfly (five DPP / in-lane 2x2 stages) shared with kq_quantize_ex's
// butterfly variant, and the encoding is the shared MX step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_device.h"
#include "kq_internal.h"

namespace kq {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kU = 2;      // rows per step
constexpr int kMaxW = 16;  // waves per workgroup: 16 x 512 channels = the widest row
constexpr int kAuxNTa = 2; // nontemporal loads: h is read once

// bf16 bits of (h - mu) * (rstd * g) + t, computed in double and rounded once
// to the nearest bf16 (ties to even).  The double -> float conversion rounds
// to nearest even; only when that lands exactly on a bf16 midpoint can the
// second rounding differ from a direct one, and then the sign of the (exact)
// remainder v - f decides.
__device__ __forceinline__ unsigned adaln_bf16(float h, double mu, double rstd, double g, double t)
{
    const double v = __builtin_fma((double)h - mu, rstd * g, t);
    const float f = (float)v;
    const double r = v - (double)f;
    const unsigned b = __float_as_uint(f);
    if ((b & 0xFFFFu) == 0x8000u && r != 0.0)
        return ((r > 0.0) == (f > 0.0)) ? (b + 0x8000u) >> 16 : b >> 16;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

struct HRows {
    u32x4 v[kU]; // the lane's 8 channels of kU rows
};

// rows mr .. mr + kU - 1 of the run (relative to its first row); rows past the
// run and lanes past the row end fall outside the range: zeros, no access
__device__ __forceinline__ void load_h(HRows &in, __amdgpu_buffer_rsrc_t rh, int mr, int d, unsigned lane_off)
{
#pragma unroll
    for (int u = 0; u < kU; ++u)
        in.v[u] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, (int)((unsigned)((mr + u) * d * 2) + lane_off), 0, kAuxNTa));
}

struct Modulation {
    float g[8], t[8]; // scale and shift of the lane's channels for the current sample
    int64_t next;     // first row of the next sample
};

__device__ __forceinline__ void load_modulation(Modulation &md, const float *__restrict__ shift,
                                                const float *__restrict__ scale, int64_t b, int64_t T, int d, int octc)
{
    md.next = (b + 1) * T;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        md.g[e] = scale[b * d + octc * 8 + e];
        md.t[e] = shift[b * d + octc * 8 + e];
    }
}

// One step of kU rows: statistics, then normalise, modulate, round to bf16
// and either write x (kQuant false) or transform and quantize.
template <bool kQuant>
__device__ __forceinline__ void adaln_rows(const HRows &in, double (&part)[kU][kMaxW][2], int64_t m, int64_t m0,
                                           int64_t m1, int d, int nW, int wave, int lane, float eps, int64_t T,
                                           const float *__restrict__ shift, const float *__restrict__ scale,
                                           Modulation &md, int oct, int octc, bool cok, const Bfly &B,
                                           __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs,
                                           __amdgpu_buffer_rsrc_t rxo)
{
    const int nB = d >> 5;
    const int qp = lane & 3;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        double s1 = 0.0, s2 = 0.0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double a = (double)bf16lo(in.v[u][i]), c = (double)bf16hi(in.v[u][i]);
            s1 += a;
            s2 = __builtin_fma(a, a, s2);
            s1 += c;
            s2 = __builtin_fma(c, c, s2);
        }
        s1 = wave_sum(s1);
        s2 = wave_sum(s2);
        if (lane == 0) {
            part[u][wave][0] = s1;
            part[u][wave][1] = s2;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t mm = m + u;
        if (mm >= m1)
            break; // uniform over the workgroup
        double s1 = 0.0, s2 = 0.0;
        for (int w = 0; w < nW; ++w) {
            s1 += part[u][w][0];
            s2 += part[u][w][1];
        }
        const double mu = s1 / (double)d;
        double var = s2 / (double)d - mu * mu;
        var = var > 0.0 ? var : 0.0;
        const double rstd = 1.0 / sqrt(var + (double)eps);
        if (mm >= md.next)
            load_modulation(md, shift, scale, mm / T, T, d, octc);
        unsigned xb[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xb[2 * i] = adaln_bf16(bf16lo(in.v[u][i]), mu, rstd, 1.0 + (double)md.g[2 * i], (double)md.t[2 * i]);
            xb[2 * i + 1] =
                adaln_bf16(bf16hi(in.v[u][i]), mu, rstd, 1.0 + (double)md.g[2 * i + 1], (double)md.t[2 * i + 1]);
        }
        const int mr = (int)(mm - m0);
        const unsigned drop = (unsigned)(cok ? 0 : 1) << 31;
        if constexpr (kQuant) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = __uint_as_float(xb[e] << 16);
            bfly_stages(v, B);
            unsigned b;
            const unsigned w = mx_encode_quad(v, b);
            const unsigned drop_s = drop | ((unsigned)(qp != 0) << 31);
            __builtin_amdgcn_raw_buffer_store_b32(w, rq, (int)((unsigned)(mr * (d >> 1) + oct * 4) | drop), 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b, rs, (int)((unsigned)(mr * nB + (oct >> 2)) | drop_s), 0,
                                                 0);
        } else {
            const u32x4 o = {xb[0] | xb[1] << 16, xb[2] | xb[3] << 16, xb[4] | xb[5] << 16, xb[6] | xb[7] << 16};
            __builtin_amdgcn_raw_buffer_store_b128(o, rxo, (int)((unsigned)(mr * d * 2 + oct * 16) | drop), 0, 0);
        }
    }
}

// Workgroup: nW waves over whole rows (wave w owns channels 512 w ..
// 512 w + 511), rows [m0, m0 + rows_per_wg).
template <bool kQuant>
__global__ __launch_bounds__(64 * kMaxW) void adaln_kernel(const uint16_t *__restrict__ h, int64_t M, int d,
                                                           const float *__restrict__ shift,
                                                           const float *__restrict__ scale, int64_t T, float eps,
                                                           const float *__restrict__ factors, int per_block,
                                                           uint8_t *__restrict__ q, uint8_t *__restrict__ s,
                                                           uint16_t *__restrict__ xo, int rows_per_wg)
{
    __shared__ double part[2][kU][kMaxW][2]; // [step parity][row of the step][wave][sum, sum of squares]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nW = blockDim.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t m1 = (m0 + rows_per_wg < M) ? m0 + rows_per_wg : M; // m0 < M: the grid covers M exactly
    const int nOct = d >> 3;
    const int oct = wave * 64 + lane;
    const bool cok = oct < nOct;
    const int octc = cok ? oct : nOct - 1; // parameter index for lanes past the row end (nothing stored)
    const unsigned lane_off = (unsigned)(oct * 16) | ((unsigned)(cok ? 0 : 1) << 31);
    const __amdgpu_buffer_rsrc_t rh = out_buffer((void *)(h + m0 * d), (m1 - m0) * d * 2);
    const __amdgpu_buffer_rsrc_t rq = out_buffer(kQuant ? q + m0 * (d >> 1) : nullptr, kQuant ? (m1 - m0) * (d >> 1) : 0);
    const __amdgpu_buffer_rsrc_t rs = out_buffer(kQuant ? s + m0 * (d >> 5) : nullptr, kQuant ? (m1 - m0) * (d >> 5) : 0);
    const __amdgpu_buffer_rsrc_t rxo = out_buffer(kQuant ? nullptr : xo + m0 * d, kQuant ? 0 : (m1 - m0) * d * 2);

    HRows bufA, bufB;
    load_h(bufA, rh, 0, d, lane_off);
    Bfly B;
    if constexpr (kQuant)
        bfly_setup(B, factors + (int64_t)(per_block ? (octc >> 2) : 0) * 20, lane & 3);
    Modulation md;
    load_modulation(md, shift, scale, m0 / T, T, d, octc);

    // two-step pipeline; a prefetch past the run falls outside the range and fetches nothing
    for (int64_t m = m0; m < m1; m += 2 * kU) {
        load_h(bufB, rh, (int)(m + kU - m0), d, lane_off);
        adaln_rows<kQuant>(bufA, part[0], m, m0, m1, d, nW, wave, lane, eps, T, shift, scale, md, oct, octc, cok, B,
                           rq, rs, rxo);
        if (m + kU >= m1)
            break; // uniform
        load_h(bufA, rh, (int)(m + 2 * kU - m0), d, lane_off);
        adaln_rows<kQuant>(bufB, part[1], m + kU, m0, m1, d, nW, wave, lane, eps, T, shift, scale, md, oct, octc, cok,
                           B, rq, rs, rxo);
    }
}

} // namespace

hipError_t launch_adaln(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale, int64_t T,
                        float eps, const float *factors, int64_t nT, uint8_t *q, uint8_t *s, uint16_t *x,
                        hipStream_t stream)
{
    const int nW = (int)((d / 8 + 63) / 64); // waves: 512 channels each
    int R = tuning().adaln_rows_per_wg;
    if (R <= 0)
        R = 8;
    const int64_t grid = (M + R - 1) / R;
    if (grid > 0x7FFFFFFF || nW > kMaxW)
        return hipErrorInvalidConfiguration;
    int di = (int)d;
    int per_block = nT > 1 ? 1 : 0;
    void *args[] = {(void *)&h, (void *)&M,   (void *)&di,      (void *)&shift,     (void *)&scale,
                    (void *)&T, (void *)&eps, (void *)&factors, (void *)&per_block, (void *)&q,
                    (void *)&s, (void *)&x,   (void *)&R};
    const void *fn = x == nullptr ? (const void *)adaln_kernel<true> : (const void *)adaln_kernel<false>;
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64 * nW), args, 0, stream);
}

} // namespace kq
