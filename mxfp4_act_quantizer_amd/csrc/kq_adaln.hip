// AdaLN front-end of the KroQuant quantizer (pages describing arXiv
// 2607.21446: the abstract on the mlsanity.com paper page says the
// normalisation layers between transformer blocks force the transform to run
// online at every step; the pith.science verdict record's
// referee_report.summary names AdaLN as what prevents absorbing it offline).
//
// Per token row m (sample b = m / T):
//   x_c = (h_c - mean) / sqrt(var + eps) * (1 + scale[b][c]) + shift[b][c]
// (LayerNorm without affine, biased variance), rounded to bf16, then the
// Kronecker transform of every 32-channel block and MXFP4.  The normalised x
// never goes to memory.
//
// The statistics kernel, then one of two second passes:
//   - by default the MFMA quantizer kernel in its AdaLN form
//     (kq_kernels.hip): h is normalised and modulated by adaln_bf16x8 as it
//     is staged for the matrix cores, so the result equals kq_quantize of
//     the x that adaln_modulate writes, bit for bit;
//   - adaln_stream_kernel below, which also writes x for adaln_modulate.
// Streaming kernels of this file, no barriers:
//   adaln_stats_kernel   one wave per row: the sum and the
//                        sum of squares of h in fp64 (lane-strided over the
//                        row, then a wave reduction), mean and
//                        1/sqrt(var + eps) in fp64 into a 16-byte record.
//                        h is read with the default cache policy so that the
//                        second pass finds it in the caches.
//   adaln_stream_kernel  one lane per 8 channels in flat row blocks (every
//                        lane busy at any width; see adaln_stage): the row
//                        records arrive by per-lane loads, the lane's
//                        modulation and butterfly factors stay in registers;
//                        per element fp64 normalisation,
//                        bf16 rounding from the double value, then the
//                        butterfly transform and MX step shared with
//                        kq_quantize_ex's butterfly variant (kQuant), or the
//                        bf16 x written out (the unfused front-end).
// Both modes read the same records, so the butterfly form of the fused
// result equals the butterfly quantizer applied to the written x bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_device.h"
#include "kq_internal.h"

namespace kq {
namespace {

constexpr int kAuxNTa = 2;   // nontemporal: the second pass reads h for the last time
constexpr int kU = 4;        // row blocks per pipeline stage of the streaming pass

// ---------------------------------------------------------------------------
// Row statistics: one row per wave (adaln_row_stats), kChunks 16-byte pieces
// per lane loaded at a time, 3 for rows of up to 192 pieces (d <= 1536) and 6
// above (measured against two rows per wave and 4 pieces: 17.9 / 12.8 / 23.3
// us against 18.8 / 13.9 / 25.3 for the whole front-end at d 1152 / 2240 /
// 3072).  A lane sums its pieces in increasing order whatever kChunks is, so
// the statistics do not depend on it.
// ---------------------------------------------------------------------------
template <int kChunks>
__global__ __launch_bounds__(256) void adaln_stats_kernel(const uint16_t *__restrict__ h, int64_t M, int d, float eps,
                                                          double *__restrict__ stats)
{
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M)
        return; // wave-uniform; no barrier in this kernel
    const __amdgpu_buffer_rsrc_t rh = out_buffer((void *)(h + m * d), (int64_t)d * 2);
    const unsigned off[1] = {0u};
    double mu[1], rstd[1];
    adaln_row_stats<1, kChunks>(rh, off, d, eps, lane, mu, rstd);
    if (lane == 0) {
        stats[2 * m] = mu[0];
        stats[2 * m + 1] = rstd[0];
    }
}

// ---------------------------------------------------------------------------
// Second pass: normalise, modulate, round to bf16, then transform + MXFP4 or
// write x.
// ---------------------------------------------------------------------------
struct HRows {
    u32x4 v[kU];
};

// Flat row blocks.  Rb = 64 / gcd(nOct, 64) rows of nOct octets (8 channels
// each) are a whole number Wb = Rb nOct / 64 of waves with every lane busy
// (a 512-channel column tile per wave would leave lanes idle at d = 1152).
// Lane l of wave wb of a block takes the block's flat octet f = 64 wb + l:
// row f / nOct of the block, octet f % nOct, the same octet in every block,
// so the lane's factors and modulation stay in registers.  A wave walks the
// kIt blocks of its group, kU blocks per pipeline stage; a wave's loads and
// code stores cover 64 consecutive octets of memory.
template <bool kQuant>
__device__ __forceinline__ void adaln_stage(const HRows &in, int64_t rb0, int ro, int Rb, int64_t M, int64_t mlo,
                                            int d, int oct, int qp, const double *__restrict__ stats,
                                            const float *__restrict__ shift, const float *__restrict__ scale,
                                            int64_t T, Modulation &md, const Bfly &B, __amdgpu_buffer_rsrc_t rq,
                                            __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rxo)
{
    const int nB = d >> 5;
    // the stage's row records, all requested before any is used (rows past M
    // read the last record; nothing of theirs is stored)
    double mus[kU], rstds[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t m = rb0 + (int64_t)u * Rb + ro;
        const int64_t mc = m < M ? m : M - 1;
        mus[u] = stats[2 * mc];
        rstds[u] = stats[2 * mc + 1];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t m = rb0 + (int64_t)u * Rb + ro;
        if (m >= md.next)
            load_modulation(md, shift, scale, (m < M ? m : M - 1) / T, T, d, oct);
        unsigned xw[4];
        adaln_bf16x8(in.v[u], mus[u], rstds[u], md.g, md.t, xw);
        // rows past M fall outside the output ranges, which end at row M
        const int mr = (int)(m - mlo);
        if constexpr (kQuant) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = (e & 1) ? bf16hi(xw[e >> 1]) : bf16lo(xw[e >> 1]);
            bfly_stages(v, B);
            unsigned b;
            const unsigned w = mx_encode_quad(v, b);
            const unsigned drop_s = (unsigned)(qp != 0) << 31;
            __builtin_amdgcn_raw_buffer_store_b32(w, rq, mr * (d >> 1) + oct * 4, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b, rs, (int)((unsigned)(mr * nB + (oct >> 2)) | drop_s), 0,
                                                 0);
        } else {
            const u32x4 o = {xw[0], xw[1], xw[2], xw[3]};
            __builtin_amdgcn_raw_buffer_store_b128(o, rxo, mr * d * 2 + oct * 16, 0, 0);
        }
    }
}

template <bool kQuant>
__global__ __launch_bounds__(256) void adaln_stream_kernel(const uint16_t *__restrict__ h, int64_t M, int d,
                                                           const double *__restrict__ stats,
                                                           const float *__restrict__ shift,
                                                           const float *__restrict__ scale, int64_t T,
                                                           const float *__restrict__ factors, int per_block,
                                                           uint8_t *__restrict__ q, uint8_t *__restrict__ s,
                                                           uint16_t *__restrict__ xo, int Rb, int Wb, int kIt)
{
    const int lane = threadIdx.x & 63;
    // groups go to the XCDs in turn (blockIdx % 8), all waves of a group on
    // one XCD: the XCDs stream one compact band of rows together, and the
    // partial lines of a group's scale rows merge in one L2
    const unsigned xcd = blockIdx.x % 8u;
    const unsigned j = (blockIdx.x / 8u) * 4u + (threadIdx.x >> 6); // wave of this XCD (32-bit: the
    const unsigned jg = j / (unsigned)Wb;                            // divisions run once per short-lived wave)
    const int64_t grp = (int64_t)jg * 8 + xcd;
    const int wb = (int)(j - jg * (unsigned)Wb);
    const int64_t mlo = grp * kIt * Rb; // first row of the group
    if (mlo >= M)
        return; // wave-uniform; no barrier in this kernel
    const int64_t mhi = (mlo + (int64_t)kIt * Rb < M) ? mlo + (int64_t)kIt * Rb : M;
    const int nOct = d >> 3;
    const int f = wb * 64 + lane;
    const int ro = (int)((unsigned)f / (unsigned)nOct); // row within a block
    const int oct = f - ro * nOct;
    const int qp = lane & 3;  // == oct & 3: 64 wb is a multiple of 4
    const __amdgpu_buffer_rsrc_t rh = out_buffer((void *)(h + mlo * d), (mhi - mlo) * d * 2);
    const __amdgpu_buffer_rsrc_t rq = out_buffer(kQuant ? q + mlo * (d >> 1) : nullptr, kQuant ? (mhi - mlo) * (d >> 1) : 0);
    const __amdgpu_buffer_rsrc_t rs = out_buffer(kQuant ? s + mlo * (d >> 5) : nullptr, kQuant ? (mhi - mlo) * (d >> 5) : 0);
    const __amdgpu_buffer_rsrc_t rxo = out_buffer(kQuant ? nullptr : xo + mlo * d, kQuant ? 0 : (mhi - mlo) * d * 2);
    // row (block k, lane row ro) of the group starts at byte (k Rb + ro) d 2 of
    // rh; rows past M fall outside its range and read as zeros
    const unsigned lane_off = (unsigned)((ro * d + oct * 8) * 2);
    const unsigned blk_bytes = (unsigned)(Rb * d * 2);
    auto load_stage = [&](HRows &in, int k0) {
#pragma unroll
        for (int u = 0; u < kU; ++u)
            in.v[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rh, (int)(lane_off + (unsigned)(k0 + u) * blk_bytes), 0, kAuxNTa));
    };
    Bfly B;
    if constexpr (kQuant)
        bfly_setup(B, factors + (int64_t)(per_block ? (oct >> 2) : 0) * 20, qp);
    Modulation md;
    {
        const int64_t m = mlo + ro;
        load_modulation(md, shift, scale, (m < M ? m : M - 1) / T, T, d, oct);
    }

    // two-stage pipeline over the group's blocks; loads past the group fall
    // outside the range and fetch nothing
    HRows bufA, bufB;
    load_stage(bufA, 0);
    int k = 0;
    for (; k + kU < kIt; k += 2 * kU) {
        load_stage(bufB, k + kU);
        adaln_stage<kQuant>(bufA, mlo + (int64_t)k * Rb, ro, Rb, M, mlo, d, oct, qp, stats, shift, scale, T, md, B,
                            rq, rs, rxo);
        load_stage(bufA, k + 2 * kU);
        adaln_stage<kQuant>(bufB, mlo + (int64_t)(k + kU) * Rb, ro, Rb, M, mlo, d, oct, qp, stats, shift, scale, T,
                            md, B, rq, rs, rxo);
    }
    if (k < kIt)
        adaln_stage<kQuant>(bufA, mlo + (int64_t)k * Rb, ro, Rb, M, mlo, d, oct, qp, stats, shift, scale, T, md, B,
                            rq, rs, rxo);
}

} // namespace

hipError_t launch_adaln(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale, int64_t T,
                        float eps, const float *factors, int64_t nT, double *stats, uint8_t *q, uint8_t *s,
                        uint16_t *x, const Tuning &tn, hipStream_t stream)
{
    // the one-launch form when the tuning selects it (measured slower than the
    // two launches at every width tried, so never chosen by itself)
    if (x == nullptr && tn.adaln_pass == 3)
        return launch_adaln_rows(h, M, d, shift, scale, T, eps, factors, nT, stats, q, s, stream);
    // pass 1: row statistics, one row per wave
    const int64_t grid1 = (M + 3) / 4;
    // pass 2: flat row blocks of Rb rows = Wb full waves; kIt blocks per wave
    const int nOct = (int)(d / 8);
    int g = 64;
    while (nOct % g)
        g >>= 1; // gcd(nOct, 64): nOct is a multiple of 4
    const int Rb = 64 / g;
    const int Wb = Rb * nOct / 64;
    int kIt = tn.adaln_blocks_per_wave;
    if (kIt <= 0)
        kIt = kU; // blocks per wave: one pipeline stage (measured best of 4..16 on MI355X)
    kIt = (kIt + kU - 1) / kU * kU;
    // a group's byte offsets, the prefetch past it included, stay below 2^31
    while (kIt > kU && (int64_t)(kIt + 2 * kU) * Rb * d * 2 >= ((int64_t)1 << 31))
        kIt -= kU;
    const int64_t nGroups = (M + (int64_t)kIt * Rb - 1) / ((int64_t)kIt * Rb);
    const int64_t wavesPerXcd = (nGroups + 7) / 8 * Wb;
    const int64_t grid2 = (wavesPerXcd + 3) / 4 * 8;
    if (grid1 > 0x7FFFFFFF || grid2 > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    int di = (int)d;
    void *args1[] = {(void *)&h, (void *)&M, (void *)&di, (void *)&eps, (void *)&stats};
    const void *fs = nOct <= 192 ? (const void *)adaln_stats_kernel<3> : (const void *)adaln_stats_kernel<6>;
    hipError_t e = hipLaunchKernel(fs, dim3((unsigned)grid1), dim3(256), args1, 0, stream);
    if (e != hipSuccess)
        return e;
    if (x == nullptr && tn.adaln_pass != 2)
        return launch_adaln_mfma(h, M, d, stats, shift, scale, T, factors, nT, q, s, tn, stream);
    int per_block = nT > 1 ? 1 : 0;
    const double *cst = stats;
    int rb = Rb, wbn = Wb, kit = kIt;
    void *args2[] = {(void *)&h,     (void *)&M, (void *)&di,      (void *)&cst,       (void *)&shift,
                     (void *)&scale, (void *)&T, (void *)&factors, (void *)&per_block, (void *)&q,
                     (void *)&s,     (void *)&x, (void *)&rb,      (void *)&wbn,       (void *)&kit};
    const void *fn = x == nullptr ? (const void *)adaln_stream_kernel<true> : (const void *)adaln_stream_kernel<false>;
    return hipLaunchKernel(fn, dim3((unsigned)grid2), dim3(256), args2, 0, stream);
}

} // namespace kq
