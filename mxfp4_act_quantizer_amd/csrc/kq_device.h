// Device helpers shared by the quantizer kernels (kq_kernels.hip) and the
// AdaLN front-end (kq_adaln.hip): the MX encoding step, DPP exchanges inside
// a quad of lanes, buffer descriptors, the butterfly form of the Kronecker
// transform, and the AdaLN normalisation of eight channels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kq {

// ---------------------------------------------------------------------------
// MX step pieces
// ---------------------------------------------------------------------------
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float amax_step(float m, float a) { return vmax(m, __builtin_fabsf(a)); }

// E8M0 byte of a block whose |max| is amax (amax >= 0 or NaN):
// E = floor(log2 amax) - 2 = expfield - 129, clamped below at -127 (byte 0);
// amax = 0 and fp32 subnormals land on byte 0; NaN / Inf give 0xFF.
__device__ __forceinline__ unsigned e8m0_byte(float amax)
{
    unsigned e = (__float_as_uint(amax) >> 23) & 0xFFu;
    unsigned b = (e < 2u ? 2u : e) - 2u;
    return e == 0xFFu ? 0xFFu : b;
}

// The convert instruction takes 2^E from the exponent field of a float.
__device__ __forceinline__ float scale_operand(unsigned byte) { return __uint_as_float(byte << 23); }

// Eight values -> one dword of packed FP4 (value 2k in bits 8k..8k+3).
__device__ __forceinline__ unsigned cvt8(float v0, float v1, float v2, float v3, float v4, float v5, float v6,
                                         float v7, float sc)
{
    unsigned w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v0, v1, sc, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v2, v3, sc, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v4, v5, sc, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v6, v7, sc, 3);
    return w;
}

// Raw buffer resources for the outputs.  Stores whose offset is at or past
// num_records are dropped by the hardware range check, which masks lanes
// (tail rows, a missing block) without a branch in the hot loop.
constexpr unsigned kBufWord3 = 0x00020000u; // gfx9-family raw buffer descriptor flags

__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_buffer(void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kBufWord3);
}

__device__ __forceinline__ float bf16lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// DPP quad permutes: partner lane^1 and lane^2.
__device__ __forceinline__ float dpp_xor1(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Per-lane constants of the butterfly for its block's factor set.
// The lane's channels are 8*qp + e of the block (qp = lane%4): index bits 4
// and 3 are the lane's quad position, bits 2..0 are e.
struct Bfly {
    float a3[4], a4[4], a5[4]; // full 2x2 factors for the in-lane stages
    float s1, o1, s2, o2;      // cross-lane stages: coefficient on own / partner value
};

__device__ __forceinline__ void bfly_setup(Bfly &B, const float *__restrict__ F, int qp)
{
    const int b4 = (qp >> 1) & 1, b3 = qp & 1;
    // stage on index bit 4 (A1) and bit 3 (A2): new(self) = A[b][b] self + A[1-b][b] other
    B.s1 = F[0 + b4 * 2 + b4];
    B.o1 = F[0 + (1 - b4) * 2 + b4];
    B.s2 = F[4 + b3 * 2 + b3];
    B.o2 = F[4 + (1 - b3) * 2 + b3];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        B.a3[k] = F[8 + k];
        B.a4[k] = F[12 + k];
        B.a5[k] = F[16 + k];
    }
}

// In-lane stage on index bit (stride st): pairs (u at bit 0, w at bit 1):
// u' = A00 u + A10 w, w' = A01 u + A11 w.  The last stage starts each sum
// from +0 so no result is -0.
template <int ST, bool kLast>
__device__ __forceinline__ void bfly_inlane(float (&v)[8], const float (&A)[4])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i & ST)
            continue;
        const float u = v[i], w = v[i + ST];
        if (kLast) {
            v[i] = __builtin_fmaf(A[0], u, __builtin_fmaf(A[2], w, 0.0f));
            v[i + ST] = __builtin_fmaf(A[1], u, __builtin_fmaf(A[3], w, 0.0f));
        } else {
            v[i] = __builtin_fmaf(A[0], u, A[2] * w);
            v[i + ST] = __builtin_fmaf(A[1], u, A[3] * w);
        }
    }
}

// The five butterfly stages of y = x K on one lane's 8 channels (channels
// 8 qp + e of a block, qp = lane % 4): the cross-lane stages first (index
// bits 4 and 3, partners in the quad), then the in-lane bits 2, 1, 0.
__device__ __forceinline__ void bfly_stages(float (&v)[8], const Bfly &B)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float other = dpp_xor2(v[i]);
        v[i] = __builtin_fmaf(B.o1, other, B.s1 * v[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float other = dpp_xor1(v[i]);
        v[i] = __builtin_fmaf(B.o2, other, B.s2 * v[i]);
    }
    bfly_inlane<4, false>(v, B.a3);
    bfly_inlane<2, false>(v, B.a4);
    bfly_inlane<1, true>(v, B.a5);
}

// MX encoding of a 32-element block held by a quad of lanes (8 values each):
// NaN-propagating amax over the quad, E8M0 byte b, and this lane's 8 packed
// FP4 codes (all zero for a NaN/Inf block).
__device__ __forceinline__ unsigned mx_encode_quad(const float (&v)[8], unsigned &b)
{
    float am = __builtin_fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i)
        am = amax_step(am, v[i]);
    am = vmax(am, dpp_xor1(am));
    am = vmax(am, dpp_xor2(am));
    b = e8m0_byte(am);
    const float sc = scale_operand(b);
    unsigned w = cvt8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], sc);
    if (b == 0xFFu)
        w = 0u;
    return w;
}

// ---- 16-element blocks with four factors (two lanes per block) ------------
// The lane's channels are 8 qp + e of its 16-element block (qp = lane % 2):
// index bit 3 is the lane's position in the pair, bits 2..0 are e.
struct Bfly16 {
    float a2[4], a3[4], a4[4]; // full 2x2 factors for the in-lane stages
    float s1, o1;              // cross-lane stage (A1): coefficient on own / partner value
};

__device__ __forceinline__ void bfly16_setup(Bfly16 &B, const float *__restrict__ F, int qp)
{
    const int b3 = qp & 1;
    // stage on index bit 3 (A1): new(self) = A[b][b] self + A[1-b][b] other
    B.s1 = F[b3 * 2 + b3];
    B.o1 = F[(1 - b3) * 2 + b3];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        B.a2[k] = F[4 + k];
        B.a3[k] = F[8 + k];
        B.a4[k] = F[12 + k];
    }
}

// The four stages of y = x K16 on one lane's 8 channels: the cross-lane
// stage (index bit 3, partner lane ^ 1), then the in-lane bits 2, 1, 0.
__device__ __forceinline__ void bfly16_stages(float (&v)[8], const Bfly16 &B)
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float other = dpp_xor1(v[i]);
        v[i] = __builtin_fmaf(B.o1, other, B.s1 * v[i]);
    }
    bfly_inlane<4, false>(v, B.a2);
    bfly_inlane<2, false>(v, B.a3);
    bfly_inlane<1, true>(v, B.a4);
}

// MX encoding of a 16-element block held by a pair of lanes: amax over the
// pair, E8M0 byte b, and this lane's 8 packed FP4 codes.
__device__ __forceinline__ unsigned mx_encode_pair(const float (&v)[8], unsigned &b)
{
    float am = __builtin_fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i)
        am = amax_step(am, v[i]);
    am = vmax(am, dpp_xor1(am));
    b = e8m0_byte(am);
    const float sc = scale_operand(b);
    unsigned w = cvt8(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], sc);
    if (b == 0xFFu)
        w = 0u;
    return w;
}

// ---------------------------------------------------------------------------
// AdaLN normalisation (LayerNorm without affine, then the per-sample
// modulation of the adaptive-norm block) of eight consecutive channels.
// ---------------------------------------------------------------------------
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// c + a b in double into a fresh register (the accumulating form of the
// instruction would first copy the addend, which stays live across rows)
__device__ __forceinline__ double fma_f64(double a, double b, double c)
{
    double r;
    asm("v_fma_f64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// x = (h - mu) * (rstd * g) + t in double for 8 channels, rounded once to the
// nearest bf16 (ties to even) and packed two per dword.  The double -> float
// conversion rounds to nearest even and the hardware bf16 convert rounds the
// float to nearest even; the two steps differ from one direct rounding only
// when the float lands exactly on a bf16 midpoint (low 16 bits 0x8000) while
// the double is not the float: then the sign of the exact remainder v - f
// decides.  That case is rare; the wave takes the fix-up path when any of its
// lanes has one.
__device__ __forceinline__ void adaln_bf16x8(const u32x4 &hv, double mu, double rstd, const double (&g)[8],
                                             const double (&t)[8], unsigned (&xw)[4])
{
    double v[8];
    float f[8];
    uint64_t tie = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float hf = (e & 1) ? bf16hi(hv[e >> 1]) : bf16lo(hv[e >> 1]);
        v[e] = fma_f64((double)hf - mu, rstd * g[e], t[e]);
        f[e] = (float)v[e];
        tie |= __builtin_amdgcn_ballot_w64((__float_as_uint(f[e]) & 0xFFFFu) == 0x8000u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
        xw[i] = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){f[2 * i], f[2 * i + 1]}, bf16x2));
    if (tie) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const unsigned b = __float_as_uint(f[e]);
            const double r = v[e] - (double)f[e];
            if ((b & 0xFFFFu) == 0x8000u && r != 0.0) {
                const unsigned x16 = ((r > 0.0) == (f[e] > 0.0)) ? (b + 0x8000u) >> 16 : b >> 16;
                const int sh = 16 * (e & 1);
                xw[e >> 1] = (xw[e >> 1] & ~(0xFFFFu << sh)) | (x16 << sh);
            }
        }
    }
}

// Row statistics of the AdaLN front-end, one wave per row.  Lane l sums the
// row's 16-byte pieces l, l + 64, l + 128, ... in increasing order (each
// piece's eight values in order), the sum and the sum of squares in fp64
// (bf16 values and their squares are exact in double), kChunks pieces in
// flight per lane; pieces past the row end (bit 31 of their offset) read as
// zeros and add nothing.  Then a butterfly reduction over the 64 lanes.
// Every kernel that needs the statistics sums through adaln_piece_sums in
// this order and ends in adaln_row_finish, so they agree bit for bit whatever
// their launch shape or where the row is read from.
__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 64);
    return v;
}

// One 16-byte piece (eight bf16 values, in order) into a lane's running sums.
__device__ __forceinline__ void adaln_piece_sums(const u32x4 &v, double &s1, double &s2)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double a = (double)bf16lo(v[i]), e = (double)bf16hi(v[i]);
        s1 += a;
        s2 = __builtin_fma(a, a, s2);
        s1 += e;
        s2 = __builtin_fma(e, e, s2);
    }
}

// The wave reduction of the lanes' sums, then mean and 1/sqrt(var + eps)
// (biased variance, clamped at 0).  Every lane of the wave takes part.
__device__ __forceinline__ void adaln_row_finish(double s1, double s2, int d, float eps, double &mu, double &rstd)
{
    const double t1 = wave_sum_f64(s1), t2 = wave_sum_f64(s2);
    mu = t1 / (double)d;
    double var = t2 / (double)d - mu * mu;
    var = var > 0.0 ? var : 0.0;
    rstd = 1.0 / sqrt(var + (double)eps);
}

// adaln_row_finish of two rows at once, their reductions interleaved; each
// row's values are those adaln_row_finish gives it alone.
__device__ __forceinline__ void adaln_row_finish2(const double (&s1)[2], const double (&s2)[2], int d, float eps,
                                                  double (&mu)[2], double (&rstd)[2])
{
    double t1[2] = {s1[0], s1[1]}, t2[2] = {s2[0], s2[1]};
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            t1[k] += __shfl_xor(t1[k], m, 64);
            t2[k] += __shfl_xor(t2[k], m, 64);
        }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        mu[k] = t1[k] / (double)d;
        double var = t2[k] / (double)d - mu[k] * mu[k];
        var = var > 0.0 ? var : 0.0;
        rstd[k] = 1.0 / sqrt(var + (double)eps);
    }
}

// kRows rows at once (their loads in flight together), row r at byte offset
// row_off[r] of the buffer; every row is summed exactly as a row alone.
template <int kRows, int kChunks>
__device__ __forceinline__ void adaln_row_stats(__amdgpu_buffer_rsrc_t rh, const unsigned (&row_off)[kRows], int d,
                                                float eps, int lane, double (&mu)[kRows], double (&rstd)[kRows])
{
    const int nOct = d >> 3;
    double s1[kRows], s2[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
        s1[r] = s2[r] = 0.0;
    for (int base = 0; base < nOct; base += 64 * kChunks) {
        u32x4 v[kRows][kChunks];
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                const int o = base + 64 * c + lane;
                const unsigned drop = (unsigned)(o >= nOct) << 31;
                v[r][c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rh, (int)((row_off[r] + (unsigned)o * 16u) | drop), 0, 0));
            }
#pragma unroll
        for (int r = 0; r < kRows; ++r)
#pragma unroll
            for (int c = 0; c < kChunks; ++c)
                adaln_piece_sums(v[r][c], s1[r], s2[r]);
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r)
        adaln_row_finish(s1[r], s2[r], d, eps, mu[r], rstd[r]);
}

struct Modulation {
    double g[8], t[8]; // 1 + scale and shift of the lane's channels for the current sample
    int64_t next;      // first row of the next sample
};

__device__ __forceinline__ void load_modulation(Modulation &md, const float *__restrict__ shift,
                                                const float *__restrict__ scale, int64_t b, int64_t T, int d, int octc)
{
    md.next = (b + 1) * T;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        md.g[e] = 1.0 + (double)scale[b * d + octc * 8 + e];
        md.t[e] = (double)shift[b * d + octc * 8 + e];
    }
}

} // namespace kq
