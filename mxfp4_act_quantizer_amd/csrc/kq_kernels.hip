// KroQuant activation quantizer kernels for MI355X (gfx950, CDNA4).
//
// Method (pages describing arXiv 2607.21446, "KroQuant: Kronecker-Structured
// Block Transforms for Efficient Post-Training Quantization of Diffusion
// Transformers"): the abstract (mlsanity.com paper page) applies a learned
// Kronecker-structured invertible transform to every 32-element block of an
// activation row and quantizes the result to MXFP4 in the same pass; the
// pith.science verdict record (pith_extraction.key_machinery) gives the block
// as K = A1 (x) A2 (x) A3 (x) A4 (x) A5 of 2x2 factors; its
// skeptic_critique.load_bearing_attack (paper Section 3.2, Eq. 4) fixes the
// block-diagonal 32x32 structure aligned with the MX blocks.  Encodings: OCP MX
// v1.0 (E2M1 elements, E8M0 scale E = floor(log2 amax) - 2).
//
// Kernels
//   kq_mfma_kernel   dense 32x32 block on bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//                    K is held as an exact 3-term bf16 split (hi + mid + lo == K
//                    in fp32), so bf16 x times each term is exact and the
//                    accumulation is fp32.  The pages run the block as small
//                    GEMMs on the matrix units; here the GEMM is
//                    Y^T = K^T X^T so one token's 32 outputs land in 2 lanes x
//                    16 accumulators.  The strip kernel: 32-token tiles of a
//                    strip of blocks staged in LDS (a factor set per block).
//   kq_flat_kernel   the same products with 32 consecutive blocks of the
//                    flattened input as the MFMA columns (one shared set; also
//                    16-element blocks): contiguous 1 KB loads and 512-byte
//                    code stores, no LDS.
//   stream_kernel    one lane per 8 consecutive channels, 4 lanes per block,
//                    used for: the butterfly transform (five 2x2 stages, the
//                    two cross-lane stages via DPP quad permutes), SmoothQuant
//                    per-channel scaling, and plain MXFP4 of fp32 input.
// All variants end in the same MX step: NaN-propagating block amax
// (v_maximum3_f32), E8M0 byte from the amax exponent field, and the gfx950
// scaled FP4 convert (v_cvt_scalef32_pk_fp4_f32), which rounds to nearest even,
// saturates at 6 and reads only the exponent field of its scale operand.
// Values handed to the convert are never -0 (it would set the sign bit): every
// path ends in an add of +0 or an MFMA accumulation started at +0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

#include "kq_device.h"
#include "kq_internal.h"

namespace kq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// MFMA variant
// ---------------------------------------------------------------------------
constexpr unsigned kXcds = 8; // MI355X: 8 accelerator dies, workgroups dealt round-robin
constexpr int kTileT = 32; // tokens per wave tile

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ unsigned short bf16_rne(float f)
{
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(unsigned short, b);
}
__device__ __forceinline__ float bf16_val(unsigned short h) { return __uint_as_float((unsigned)h << 16); }

// MFMA A operands of one wave for its block, built in registers.
// The 32x32 block enters the MFMA as A = K^T with rows permuted (output
// channel order) so that accumulator v of a lane in half h is channel 16h+v:
// A row i holds output channel pi(i) = 16*((i>>2)&1) + 4*(i>>3) + (i&3).
// Lane l of MFMA j holds A[i = l%32][k = 8h + e] = K[16j + 8h + e][pi(i)]
// (h = l/32), i.e. input index bits (r4 r3 r2 r1 r0) = (j, h, e2, e1, e0).
// Each entry K = A1[r4][c4] A2[r3][c3] A3[r2][c2] A4[r1][c1] A5[r0][c0] is
// formed in fp32 and split exactly into hi + mid + lo bf16 terms (each step
// keeps the next 8 significant bits, so the third remainder fits bf16).
//
// With lu set, F holds the set as 15 LU scalars (a, b, c) per factor and each
// factor is rebuilt first as G = [[1, 0], [c, 1]] [[a, b], [0, -1/a]] =
// [[a, b], [c a, c b - 1/a]], in fp32 with the operations kq_lu_factors
// performs on the host (correctly rounded 1/a, c*a, fma(c, b, -1/a)).
__device__ __forceinline__ void build_a_operands(bf16x8 (&A)[3][2], const float *__restrict__ F, int lu, int lane)
{
    // the set is the same for the whole wave: scalar loads, then per-lane selects
    float f[20];
    if (lu) {
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            const float a = F[3 * k], b = F[3 * k + 1], c = F[3 * k + 2];
            const float r = __fdiv_rn(1.0f, a);
            f[4 * k] = a;
            f[4 * k + 1] = b;
            f[4 * k + 2] = c * a;
            f[4 * k + 3] = __builtin_fmaf(c, b, -r);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 20; ++i)
            f[i] = F[i];
    }
    const int h = lane >> 5;
    const int i = lane & 31;
    const int c = 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
    const bool c4 = (c >> 4) & 1, c3 = (c >> 3) & 1, c2 = (c >> 2) & 1, c1 = (c >> 1) & 1, c0 = c & 1;
    // f[k*4 + r*2 + col] is entry (r, col) of factor A_{k+1}
    const float a2 = h ? (c3 ? f[7] : f[6]) : (c3 ? f[5] : f[4]);
    const float a3_0 = c2 ? f[9] : f[8], a3_1 = c2 ? f[11] : f[10];
    const float a4_0 = c1 ? f[13] : f[12], a4_1 = c1 ? f[15] : f[14];
    const float a5_0 = c0 ? f[17] : f[16], a5_1 = c0 ? f[19] : f[18];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float p = (j ? (c4 ? f[3] : f[2]) : (c4 ? f[1] : f[0])) * a2;
        bf16x8 hi, mid, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float k = ((p * ((e & 4) ? a3_1 : a3_0)) * ((e & 2) ? a4_1 : a4_0)) * ((e & 1) ? a5_1 : a5_0);
            const unsigned short bh = bf16_rne(k);
            const float r1 = k - bf16_val(bh);
            const unsigned short bm = bf16_rne(r1);
            const float r2 = r1 - bf16_val(bm);
            hi[e] = __builtin_bit_cast(__bf16, bh);
            mid[e] = __builtin_bit_cast(__bf16, bm);
            lo[e] = __builtin_bit_cast(__bf16, bf16_rne(r2));
        }
        A[0][j] = lo;
        A[1][j] = mid;
        A[2][j] = hi;
    }
}

// The A operands for two 16-element blocks (four factors per set, K16 = A1
// (x) A2 (x) A3 (x) A4 with A1 on the most significant bit of the 4-bit in-block
// index): the 32 x 32 block diag(K16 of set F0, K16 of set F1), so input half
// j (k-step j) belongs to set j and feeds only output half j; with F0 == F1
// it is I (x) K16.  Same lane layout, product order ((A1 A2) A3) A4 and exact
// three-term split as build_a_operands.
__device__ __forceinline__ void build_a_operands16(bf16x8 (&A)[3][2], const float *__restrict__ F0,
                                                   const float *__restrict__ F1, int lane)
{
    const int h = lane >> 5;
    const int i = lane & 31;
    const int c = 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
    const int c4 = (c >> 4) & 1;
    const bool c3 = (c >> 3) & 1, c2 = (c >> 2) & 1, c1 = (c >> 1) & 1, c0 = c & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float *F = j ? F1 : F0;
        float f[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
            f[k] = F[k];
        // f[4k + 2r + col] is entry (r, col) of factor A_{k+1} of the set
        const float a1 = h ? (c3 ? f[3] : f[2]) : (c3 ? f[1] : f[0]);
        const float a2_0 = c2 ? f[5] : f[4], a2_1 = c2 ? f[7] : f[6];
        const float a3_0 = c1 ? f[9] : f[8], a3_1 = c1 ? f[11] : f[10];
        const float a4_0 = c0 ? f[13] : f[12], a4_1 = c0 ? f[15] : f[14];
        const float p = c4 == j ? a1 : 0.0f;
        bf16x8 hi, mid, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float k = ((p * ((e & 4) ? a2_1 : a2_0)) * ((e & 2) ? a3_1 : a3_0)) * ((e & 1) ? a4_1 : a4_0);
            const unsigned short bh = bf16_rne(k);
            const float r1 = k - bf16_val(bh);
            const unsigned short bm = bf16_rne(r1);
            const float r2 = r1 - bf16_val(bm);
            hi[e] = __builtin_bit_cast(__bf16, bh);
            mid[e] = __builtin_bit_cast(__bf16, bm);
            lo[e] = __builtin_bit_cast(__bf16, bf16_rne(r2));
        }
        A[0][j] = lo;
        A[1][j] = mid;
        A[2][j] = hi;
    }
}

// ---- workgroup tile of the MFMA variant ----------------------------------
// A workgroup of kW waves owns a strip of kW adjacent blocks (kW * 32
// channels, kW * 64 bytes of a token row: 512 bytes for kW = 8, 1 KB for
// kW = 16) and walks 32-token tiles.  x arrives with contiguous loads (16
// bytes per lane; each wave instruction covers whole row strips), goes through
// a padded LDS tile, and is read back in the MFMA operand layout.
template <int kW>
struct Strip {
    static constexpr int kBytes = kW * 64;        // bytes of x per token row and workgroup
    static constexpr int kXRow = kBytes + 16;     // padded LDS row: 16 consecutive tokens hit distinct banks
    static constexpr int kQRow = kW * 16 + 16;    // padded LDS row of staged codes
    static constexpr int kLanesPerRow = kW * 4;   // 16-byte chunks per row strip
    static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
    static constexpr int kRowsPerWave = kTileT / kW;
    static_assert(kRowsPerWave == 2 * kRowsPerLoad, "two load instructions per wave and tile");
};

// kB16: 16-element blocks, two scale bytes per 32-element block of the strip
template <int kW, bool kB16 = false>
struct __align__(16) WgStage {
    unsigned char x[2][kTileT][Strip<kW>::kXRow];    // x tile, double-buffered by tile parity
    unsigned char q[2][kTileT][Strip<kW>::kQRow];    // staged codes
    unsigned char s[2][kTileT][kB16 ? 2 * kW : kW]; // staged scale bytes
};

// Raw x of one tile for one wave: two load instructions, rows
// kRowsPerWave * wave + kRowsPerLoad * k + lane / kLanesPerRow, 16-byte chunk
// lane % kLanesPerRow of the row strip.
struct XIn {
    u32x4 v[2];
};

// Load this wave's share of the tile at token row r0 through a buffer range
// that holds exactly the tile's rows below M (none when `valid` is false, for
// the look-ahead steps past a workgroup's last tile).  Rows past M and chunks
// of blocks past the row end (bit 31 set in their offsets) fall outside the
// range: the hardware returns zeros for them without touching memory, and no
// such value is ever stored.  x is read exactly once, so the loads are marked
// nontemporal (streamed past the caches rather than kept there).
constexpr int kAuxNT = 2; // buffer instruction cache policy: nontemporal

template <int kW>
__device__ __forceinline__ void load_x(XIn &in, const uint16_t *__restrict__ x, int64_t M, int d, int bg, int nB,
                                       int64_t r0, bool valid, int wave, int lane)
{
    using S = Strip<kW>;
    const int chunk = lane % S::kLanesPerRow;
    const int blk = bg * kW + (chunk >> 2);
    const int64_t rows = valid ? ((M - r0) < kTileT ? (M - r0) : kTileT) : 0;
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc((void *)(x + r0 * d), 0, (int)(rows * d * 2), kBufWord3);
    const unsigned drop = (unsigned)(blk >= nB) << 31;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int row = S::kRowsPerWave * wave + S::kRowsPerLoad * k + lane / S::kLanesPerRow;
        const unsigned off = (unsigned)((row * d + bg * (S::kBytes / 2) + chunk * 8) * 2) | drop;
        in.v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, kAuxNT));
    }
}

template <int kW, bool kB16>
__device__ __forceinline__ void stage_x(WgStage<kW, kB16> &st, int par, const XIn &in, int wave, int lane)
{
    using S = Strip<kW>;
#pragma unroll
    for (int k = 0; k < 2; ++k)
        *(u32x4 *)&st.x[par][S::kRowsPerWave * wave + S::kRowsPerLoad * k + lane / S::kLanesPerRow]
                         [(lane % S::kLanesPerRow) * 16] = in.v[k];
}

// The transform of one 32 x 32 MFMA tile: Y^T = K^T X^T with K^T in its three
// exact bf16 terms, smallest first (lo, mid, hi), two k-steps of 16 each.
// bv[j] holds, in lane (column c = l % 32, half h = l / 32), input channels
// 16j + 8h .. +7 of column c's block.
__device__ __forceinline__ f32x16 block_product(const bf16x8 (&A)[3][2], const bf16x8 (&bv)[2])
{
    f32x16 acc = {};
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[sp][j], bv[j], acc, 0, 0, 0);
    return acc;
}

// MX step of one MFMA tile: acc holds output channels 16h .. 16h+15 of the
// lane's column block (h = l / 32), the other 16 sit in lane l ^ 32.  Returns
// the block's E8M0 byte; w0, w1 receive the lane's 8 code bytes (all zero
// for a NaN/Inf block).
__device__ __forceinline__ unsigned mx_tile(const f32x16 &acc, unsigned &w0, unsigned &w1)
{
    float m = __builtin_fabsf(acc[0]);
#pragma unroll
    for (int v = 1; v < 16; ++v)
        m = amax_step(m, acc[v]);
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    m = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
    const unsigned b = e8m0_byte(m);
    const float sc = scale_operand(b);
    w0 = cvt8(acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7], sc);
    w1 = cvt8(acc[8], acc[9], acc[10], acc[11], acc[12], acc[13], acc[14], acc[15], sc);
    if (b == 0xFFu)
        w0 = w1 = 0u;
    return b;
}

// The same for I (x) K16 (16-element blocks): half h of a column (output
// channels 16h .. 16h+15) depends only on its own 16 inputs, taken by k-step
// h, so each half accumulates its own step alone and the lane keeps its
// half's sums.  A NaN or Inf input then reaches only its own 16-element
// block, where a single sum over both steps would have spread it through the
// zero entries of the other half.
__device__ __forceinline__ f32x16 block_product16(const bf16x8 (&A)[3][2], const bf16x8 (&bv)[2], int h)
{
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int sp = 0; sp < 3; ++sp) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[sp][0], bv[0], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[sp][1], bv[1], acc1, 0, 0, 0);
    }
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v)
        acc[v] = h ? acc1[v] : acc0[v];
    return acc;
}

// MX step of one half column (16-element blocks): the lane's 16 accumulators
// are one block; no exchange between lanes.
__device__ __forceinline__ unsigned mx_tile16(const f32x16 &acc, unsigned &w0, unsigned &w1)
{
    float m = __builtin_fabsf(acc[0]);
#pragma unroll
    for (int v = 1; v < 16; ++v)
        m = amax_step(m, acc[v]);
    const unsigned b = e8m0_byte(m);
    const float sc = scale_operand(b);
    w0 = cvt8(acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7], sc);
    w1 = cvt8(acc[8], acc[9], acc[10], acc[11], acc[12], acc[13], acc[14], acc[15], sc);
    if (b == 0xFFu)
        w0 = w1 = 0u;
    return b;
}

// Transform one tile on the matrix cores; quantize into the staging buffer
// (or write y directly).  Lane l takes token l%32 and, for MFMA j, channels
// 16j + 8h .. +7 of block `wave` of the strip (h = l/32).
template <bool kQuant, int kW, bool kB16>
__device__ __forceinline__ void transform_tile(const WgStage<kW, kB16> &stc, WgStage<kW, kB16> &st, int par,
                                               const bf16x8 (&A)[3][2], int64_t t, int64_t M, int d, int jb,
                                               bool jb_valid, int h, int wave, int tl, float *__restrict__ y)
{
    bf16x8 bv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        bv[j] = *(const bf16x8 *)&stc.x[par][tl][wave * 64 + 32 * j + 16 * h];
    const f32x16 acc = kB16 ? block_product16(A, bv, h) : block_product(A, bv);
    if constexpr (kQuant) {
        unsigned w0, w1;
        const unsigned b = kB16 ? mx_tile16(acc, w0, w1) : mx_tile(acc, w0, w1);
        // lane half h holds q bytes 8h..8h+7 of block `wave` of the strip (and
        // with kB16 the scale byte of 16-element block 2 wave + h)
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        *(u32x2 *)&st.q[par][tl][wave * 16 + 8 * h] = u32x2{w0, w1};
        if constexpr (kB16)
            st.s[par][tl][2 * wave + h] = (unsigned char)b;
        else if (h == 0)
            st.s[par][tl][wave] = (unsigned char)b;
    } else {
        // waves past the row end computed a stand-in block: nothing to write
        if (t < M && jb_valid) {
            f32x4 *o = (f32x4 *)(y + t * d + jb * 32 + 16 * h);
            o[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
            o[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
            o[2] = f32x4{acc[8], acc[9], acc[10], acc[11]};
            o[3] = f32x4{acc[12], acc[13], acc[14], acc[15]};
        }
    }
}

// Store one staged tile.  Every wave issues the same two stores, with no
// branch (so the compiler's memory-counter waits stay exact): 8 code bytes
// per lane, 2*kW lanes per token (one contiguous 16*kW-byte segment per token
// row), and one scale byte per lane for the first 32*kW lanes of the
// workgroup (kW consecutive bytes per token).  rq and rs cover the tile's own
// rows, so rows past M fall outside them; blocks past the row end, the spare
// scale lanes, and every lane when `valid` is false set bit 31 of their
// offsets, which the range check drops.  With kNT the code stores are
// nontemporal (streamed past the caches), otherwise they keep the default
// cache policy; the launcher takes nontemporal stores when the launch's whole
// footprint exceeds the last-level cache, so that codes a following W4A4
// product could still read from the caches keep the default policy: at the
// DiT qkv shape (8192 x 1152 by 3456) nontemporal code stores made the
// quantizer alone 3-6% faster but quantize-then-product 8% slower (41.7
// against 38.4 us).  Scale bytes always keep the default policy.
template <int kW, bool kNT, bool kB16>
__device__ __forceinline__ void store_tile(const WgStage<kW, kB16> &st, int par, bool valid, int bg, int nB, int d,
                                           int wave, int lane, __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs)
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    constexpr int kLQ = 2 * kW; // lanes per token for the codes
    const int tq = wave * (64 / kLQ) + lane / kLQ;
    const int c8 = lane % kLQ;
    const unsigned drop_q = (unsigned)(bg * kW + (c8 >> 1) >= nB || !valid) << 31;
    const u32x2 v = *(const u32x2 *)&st.q[par][tq][c8 * 8];
    __builtin_amdgcn_raw_buffer_store_b64(v, rq, (int)((unsigned)(tq * (d >> 1) + bg * kW * 16 + c8 * 8) | drop_q), 0,
                                          kNT ? kAuxNT : 0);
    const int f = wave * 64 + lane; // flat lane of the workgroup
    if constexpr (kB16) {
        // two scale bytes per 32-element block: every lane stores one
        const int ts = f / (2 * kW);
        const int cs = f % (2 * kW);
        const int nB16 = 2 * nB;
        const unsigned drop_s = (unsigned)(2 * bg * kW + cs >= nB16 || !valid) << 31;
        __builtin_amdgcn_raw_buffer_store_b8(st.s[par][ts][cs], rs,
                                             (int)((unsigned)(ts * nB16 + 2 * bg * kW + cs) | drop_s), 0, 0);
    } else {
        const int ts = (f / kW) % kTileT;
        const int cs = f % kW;
        const unsigned drop_s = (unsigned)(bg * kW + cs >= nB || !valid || f >= kTileT * kW) << 31;
        __builtin_amdgcn_raw_buffer_store_b8(st.s[par][ts][cs], rs, (int)((unsigned)(ts * nB + bg * kW + cs) | drop_s),
                                             0, 0);
    }
}

// One workgroup: a strip of kW blocks (one per wave for the transform) and
// a sequence of 32-token tiles the eight waves walk together: tiles
// tile0, tile0 + stride, tile0 + 2*stride, ...  With stride 1 a workgroup owns
// a contiguous run of rows; with stride = number of token groups the groups
// interleave, so the workgroups resident at one time cover one compact band
// of rows (as a grid-stride copy does).  Per tile, in order: issue the loads
// of the tile kRing-1 ahead, stage this tile's x (loaded kRing-1 steps
// earlier) in LDS, barrier, store the previous tile's staged codes, transform
// this tile from LDS into the staging buffer.  One barrier per tile orders all of it
// (the LDS buffers alternate by tile parity).  Every load instruction is
// issued unconditionally; those of look-ahead steps past the last tile have
// an empty range and fetch nothing.  kRing: tiles in the register ring of a
// wave, kRing - 1 of them in flight ahead of the one being staged (the
// launcher picks 2 or 4).

// With kAd the kernel is the second pass of the AdaLN front-end: x holds h,
// and each lane normalises and modulates its two 16-byte pieces of a tile in
// registers (adaln_bf16x8, the same arithmetic as the front-end's own
// streaming pass) before they are staged, so the transform sees the bf16 x
// that adaln_modulate would write.  The row statistics come from the
// workspace the statistics kernel filled; a lane's record loads ride in the
// ring with the tile's loads.
struct AdArgs {
    const double *stats;       // [M, 2]: mean, 1/sqrt(var + eps)
    const float *shift, *scale; // [ceil(M / T), d]
    int64_t T;                 // tokens per sample
};
// The AdaLN form needs about 180 VGPRs: two waves per SIMD (at three the
// compiler spills, and that measured no faster).
constexpr int kAdOcc = 2;

// kB16: 16-element blocks with four factors per set (a pair of sets per
// 32-element block of the strip, build_a_operands16); s has d / 16 bytes per
// row.
template <bool kQuant, int kW, bool kAd = false, bool kNT = false, int kRing = 4, bool kB16 = false>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(kAd ? kAdOcc : 4))) void kq_mfma_kernel(
    const uint16_t *__restrict__ x, int64_t M, int d, const float *__restrict__ factors, int per_block,
    uint8_t *__restrict__ q, uint8_t *__restrict__ s, float *__restrict__ y, int nBG, int tiles_per_wg,
    int order, int lu, AdArgs ad)
{
    __shared__ WgStage<kW, kB16> st;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // order bit 0: interleaved token groups (else contiguous runs of tiles).
    // order bit 1: flat workgroup order, strips fastest.  Otherwise XCD-grouped:
    // workgroups go round-robin to the 8 XCDs (blockIdx % 8) and all strips of
    // one token group run on the same XCD, one after another, so partial lines
    // written into the same q and s rows merge in that L2.
    const bool interleave = order & 1;
    int bg;
    int64_t group;
    if (order & 2) {
        bg = (int)(blockIdx.x % (unsigned)nBG);
        group = blockIdx.x / (unsigned)nBG;
    } else {
        const unsigned xcd = blockIdx.x % kXcds;
        const unsigned slot = blockIdx.x / kXcds;
        bg = (int)(slot % (unsigned)nBG);
        group = (int64_t)(slot / (unsigned)nBG) * kXcds + xcd;
    }
    const int nB = d >> 5;
    const int64_t nTiles = (M + kTileT - 1) / kTileT;
    const int64_t nG = (nTiles + tiles_per_wg - 1) / tiles_per_wg;
    if (group >= nG)
        return; // padding workgroup: uniform over the workgroup, before any barrier
    const int64_t tile0 = interleave ? group : group * tiles_per_wg;
    const int64_t stride = interleave ? nG : 1;
    const int64_t left = (nTiles - tile0 + stride - 1) / stride;
    const int n = (int)(left < tiles_per_wg ? left : tiles_per_wg);
    const int jb_raw = bg * kW + wave;
    // waves past the row end take part in loads and barriers and transform block
    // nB-1 (their results are never stored)
    const int jb = jb_raw < nB ? jb_raw : nB - 1;
    const int h = lane >> 5;
    const int tl = lane & 31;
    // first token row of step k (steps past the last tile name it again; their
    // loads are empty)
    auto trow = [&](int k) -> int64_t { return (tile0 + (int64_t)(k < n ? k : n - 1) * stride) * kTileT; };

    // register ring of kRing tiles: tile k lives in ring[k % kRing] from its
    // load (kRing - 1 steps ahead) until it is staged in LDS
    XIn ring[kRing];
    // kAd: statistics records, lane l holding the one of its row for load
    // k = l & 1 (its partner l ^ 1 holds the other)
    u32x4 sring[kAd ? kRing : 1];
    using S = Strip<kW>;
    auto load_stat = [&](u32x4 &rec, int kk) {
        const int64_t m = trow(kk) + S::kRowsPerWave * wave + S::kRowsPerLoad * (lane & 1) + lane / S::kLanesPerRow;
        rec = *(const u32x4 *)(ad.stats + 2 * (m < M ? m : M - 1));
    };
    Modulation md;
    int oct = 0; // kAd: the lane's octet (8 channels) of the row; blocks past the row end use the last one
    if constexpr (kAd) {
        const int chunk = lane % S::kLanesPerRow;
        const int blk = bg * kW + (chunk >> 2);
        oct = (blk < nB ? blk : nB - 1) * 4 + (chunk & 3);
        const int64_t m = trow(0) + S::kRowsPerWave * wave + lane / S::kLanesPerRow;
        load_modulation(md, ad.shift, ad.scale, (m < M ? m : M - 1) / ad.T, ad.T, d, oct);
    }
    // normalise the two pieces of step kk in place (rows past M: any finite
    // stand-in, never stored)
    auto normalize = [&](XIn &in, const u32x4 &rec, int kk) {
        u32x4 oth;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            oth[i] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)rec[i], 0xB1, 0xF, 0xF, false);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const u32x4 r = (lane & 1) == k ? rec : oth;
            const double mu = __builtin_bit_cast(double, ((uint64_t)r[1] << 32) | r[0]);
            const double rstd = __builtin_bit_cast(double, ((uint64_t)r[3] << 32) | r[2]);
            const int64_t m = trow(kk) + S::kRowsPerWave * wave + S::kRowsPerLoad * k + lane / S::kLanesPerRow;
            if (m >= md.next)
                load_modulation(md, ad.shift, ad.scale, (m < M ? m : M - 1) / ad.T, ad.T, d, oct);
            unsigned xw[4];
            adaln_bf16x8(in.v[k], mu, rstd, md.g, md.t, xw);
            in.v[k] = u32x4{xw[0], xw[1], xw[2], xw[3]};
        }
    };
    // output ranges of one tile's rows
    auto store_prev = [&](int kp) {
        const int64_t r0 = trow(kp < 0 ? 0 : kp);
        const int64_t rows = (M - r0) < kTileT ? (M - r0) : kTileT;
        const int sB = kB16 ? 2 * nB : nB; // scale bytes per row
        store_tile<kW, kNT, kB16>(st, kp & 1, kp >= 0, bg, nB, d, wave, lane,
                                  out_buffer(q + r0 * (d >> 1), rows * (d >> 1)), out_buffer(s + r0 * sB, rows * sB));
    };
    // Each prologue load is followed by a store pair with every lane dropped
    // (no memory access), so the memory counter holds the same sequence on
    // entry to the loop as after a loop step, and the compiler's waits inside
    // the loop stay exact rather than falling back to the prologue's shorter
    // sequence.
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k) {
        if constexpr (kAd)
            load_stat(sring[k], k);
        load_x<kW>(ring[k], x, M, d, bg, nB, trow(k), k < n, wave, lane);
        if (kQuant)
            store_prev(-1);
    }

    bf16x8 A[3][2];
    if constexpr (kB16)
        build_a_operands16(A, factors + (int64_t)(per_block ? 2 * jb : 0) * 16,
                           factors + (int64_t)(per_block ? 2 * jb + 1 : 0) * 16, lane);
    else
        build_a_operands(A, factors + (int64_t)(per_block ? jb : 0) * (lu ? 15 : 20), lu, lane);

    auto step = [&](XIn &cur, XIn &ld, const u32x4 &rcur, u32x4 &rld, int kk) {
        if constexpr (kAd)
            load_stat(rld, kk + kRing - 1);
        load_x<kW>(ld, x, M, d, bg, nB, trow(kk + kRing - 1), kk + kRing - 1 < n, wave, lane);
        if constexpr (kAd)
            normalize(cur, rcur, kk);
        stage_x(st, kk & 1, cur, wave, lane);
        __syncthreads();
        if (kQuant)
            store_prev(kk - 1);
        transform_tile<kQuant, kW, kB16>(st, st, kk & 1, A, trow(kk) + tl, M, d, jb, jb_raw < nB, h, wave, tl, y);
    };

    int it = 0;
    for (; it + kRing - 1 < n; it += kRing) {
#pragma unroll
        for (int k = 0; k < kRing; ++k)
            step(ring[k], ring[(k + kRing - 1) % kRing], sring[kAd ? k : 0], sring[kAd ? (k + kRing - 1) % kRing : 0],
                 it + k);
    }
    // fewer than kRing tiles left, already in ring[0 ..]; their look-ahead loads are empty
#pragma unroll
    for (int k = 0; k < kRing - 1; ++k)
        if (it + k < n)
            step(ring[k], ring[kRing - 1], sring[kAd ? k : 0], sring[kAd ? kRing - 1 : 0], it + k);
    if (kQuant) {
        __syncthreads();
        store_prev(n - 1);
    }
}

// ---------------------------------------------------------------------------
// Flat form of the MFMA quantizer, for one factor set shared by every block.
//
// With a single set every block goes through the same transform, so the row
// structure plays no part: x is one flat run of M*d/32 blocks of 64 bytes, q
// one of 16-byte code blocks and s one of scale bytes (block b at byte 64b,
// 16b and b).  The 32 columns of an MFMA tile are 32 consecutive blocks, a
// unit: per unit a wave reads 2 KB of contiguous x and writes 512 contiguous
// code bytes and 32 scale bytes, with no LDS and no barrier.  The A operand,
// the products and the MX step are those of kq_mfma_kernel (build_a_operands,
// block_product, mx_tile), each column of a tile being computed alone, so the
// two kernels give the same values bit for bit.
//
// Loads.  Step j of the product wants, in lane (column c = l % 32, half h =
// l / 32), input channels 16j + 8h .. +7 of column c's block.  Load i (i = 0,
// 1) reads 1 KB of contiguous x, blocks 16i .. 16i + 15 of the unit: lane
// (c, h) takes the 16 bytes at 32 (c / 16) + 16h of block 16i + c % 16.  So
// lanes with c < 16 receive step 0 of block 16i + c, lanes with c >= 16 step 1
// of block 16i + c - 16.  One permlane16 swap per register (the odd 16-lane
// rows of load 0 with the even rows of load 1) leaves load 0 holding step 0
// and load 1 step 1 of block c, for every column c.
//
// Work split: wave g of G walks units g, g + G, g + 2G, ...: the waves keep
// one compact band of x in flight, and the 4 units whose scale bytes share a
// 128-byte line run on the 4 waves of one workgroup.  A register ring of kFR
// units keeps kFR - 1 units of loads in flight while one is transformed (the
// launcher picks kFR and G; few bytes in flight per CU measured fastest).
// Buffer ranges hold exactly a unit's blocks below the end, so the missing
// blocks of the last unit and the look-ahead past a wave's last unit fetch
// and store nothing; every load and store instruction is issued
// unconditionally (exact memory-counter waits, as in kq_mfma_kernel).
//
// With kB16 the kernel runs 16-element blocks with one shared set of four
// factors: the 32 x 32 block is I (x) K16 (build_a_operands16), each half
// column sums only its own k-step (block_product16) and is one 16-element
// block with its own scale byte (mx_tile16; 64 scale bytes per unit).  nelem
// is M * d, a multiple of 16 with kB16 and of 32 otherwise; a unit is 1024
// elements either way.
// ---------------------------------------------------------------------------
constexpr int kFlatWaves = 4; // waves per workgroup

template <bool kQuant, bool kNT, int kFR, bool kB16 = false>
__global__ __launch_bounds__(64 * kFlatWaves) void kq_flat_kernel(const uint16_t *__restrict__ x, int64_t nelem,
                                                                  const float *__restrict__ factors, int lu,
                                                                  uint8_t *__restrict__ q, uint8_t *__restrict__ s,
                                                                  float *__restrict__ y)
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const int lane = threadIdx.x & 63;
    const int64_t G = (int64_t)gridDim.x * kFlatWaves;
    const int64_t g = (int64_t)blockIdx.x * kFlatWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nunits = (nelem + 1023) / 1024;
    if (g >= nunits)
        return; // wave-uniform; this kernel has no barrier
    const int n = (int)((nunits - g + G - 1) / G); // units of this wave
    const int col = lane & 31, h = lane >> 5;
    const unsigned xoff = (unsigned)(64 * (col & 15) + 32 * (col >> 4) + 16 * h);

    // the wave's k-th unit (steps past its last unit name that unit again)
    // and its elements below the end (none past the last unit)
    auto unit_of = [&](int k) -> int64_t { return g + (int64_t)(k < n ? k : n - 1) * G; };
    auto elems_of = [&](int k) -> int {
        const int64_t left = nelem - unit_of(k) * 1024;
        return k < n ? (int)(left < 1024 ? left : 1024) : 0;
    };
    auto load_unit = [&](XIn &in, int k) {
        const __amdgpu_buffer_rsrc_t rx =
            __builtin_amdgcn_make_buffer_rsrc((void *)(x + unit_of(k) * 1024), 0, elems_of(k) * 2, kBufWord3);
        in.v[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)xoff, 0, kAuxNT));
        in.v[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xoff + 1024), 0, kAuxNT));
    };
    // outputs of unit u with ne elements (ne = 0 drops every lane): lane (c, h)
    // holds code bytes 8h .. 8h+7 of column c's 32 elements and either (32-
    // element blocks) the block's scale byte, stored by lanes h = 0, or
    // (16-element blocks, kB16) the scale byte of its own 16 elements, block
    // 2c + h of the unit; or (y) output channels 16h .. 16h+15 of column c
    auto emit_q = [&](unsigned w0, unsigned w1, unsigned b, int64_t u, int ne) {
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{w0, w1}, out_buffer(q + u * 512, ne / 2), 16 * col + 8 * h, 0,
                                              kNT ? kAuxNT : 0);
        if constexpr (kB16)
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b, out_buffer(s + u * 64, ne / 16), 2 * col + h, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b, out_buffer(s + u * 32, ne / 32),
                                                 (int)((unsigned)col | ((unsigned)h << 31)), 0, 0);
    };
    auto emit_y = [&](const f32x16 &acc, int64_t u, int ne) {
        const __amdgpu_buffer_rsrc_t ry = out_buffer(y + u * 1024, ne * 4);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, f32x4{acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]}), ry,
                128 * col + 64 * h + 16 * v, 0, 0);
    };

    // Each prologue load is followed by the step's stores with every lane
    // dropped, so the memory counter holds the same sequence on entry to the
    // loop as after a loop step.
    XIn ring[kFR];
#pragma unroll
    for (int k = 0; k < kFR - 1; ++k) {
        load_unit(ring[k], k);
        if constexpr (kQuant)
            emit_q(0u, 0u, 0u, 0, 0);
        else
            emit_y(f32x16{}, 0, 0);
    }
    bf16x8 A[3][2];
    if constexpr (kB16)
        build_a_operands16(A, factors, factors, lane);
    else
        build_a_operands(A, factors, lu, lane);

    // The scheduling barriers keep each step's work after its look-ahead load
    // and before the next step's: hoisting the swaps of later units would
    // move their memory-counter waits up and drain the ring.
    auto step = [&](XIn &cur, XIn &ld, int kk) {
        load_unit(ld, kk + kFR - 1);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 b0, b1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto r = __builtin_amdgcn_permlane16_swap(cur.v[0][i], cur.v[1][i], false, false);
            b0[i] = r[0];
            b1[i] = r[1];
        }
        const bf16x8 bv[2] = {__builtin_bit_cast(bf16x8, b0), __builtin_bit_cast(bf16x8, b1)};
        const f32x16 acc = kB16 ? block_product16(A, bv, h) : block_product(A, bv);
        const int64_t u = g + (int64_t)kk * G;
        const int64_t left = nelem - u * 1024;
        const int ne = (int)(left < 1024 ? left : 1024);
        if constexpr (kQuant) {
            unsigned w0, w1;
            const unsigned b = kB16 ? mx_tile16(acc, w0, w1) : mx_tile(acc, w0, w1);
            emit_q(w0, w1, b, u, ne);
        } else {
            emit_y(acc, u, ne);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    int it = 0;
    for (; it + kFR - 1 < n; it += kFR) {
#pragma unroll
        for (int k = 0; k < kFR; ++k)
            step(ring[k], ring[(k + kFR - 1) % kFR], it + k);
    }
    // fewer than kFR units left, already in ring[0 ..]; their look-ahead loads are empty
#pragma unroll
    for (int k = 0; k < kFR - 1; ++k)
        if (it + k < n)
            step(ring[k], ring[kFR - 1], it + k);
}

// ---------------------------------------------------------------------------
// AdaLN front-end in one launch, for rows that fit the LDS (selected by the
// tuning; the two-launch form is the default).  A workgroup of kRowsWaves waves
// owns R <= 32 whole token rows at a time (one matrix-core tile of tokens), so
// h is read from HBM once:
//   0. the factor sets go into LDS once; each tile's rows of h, and the
//      modulation rows of its samples when there are at most nmod of them,
//      go into LDS by LDS-DMA loads (padded rows: a 16-byte read at the same
//      column of 16 consecutive rows hits every bank once);
//   1. each wave computes the statistics of two rows from LDS at a time,
//      summing a row's pieces in the statistics kernel's order
//      (adaln_piece_sums, adaln_row_finish2), so the values agree with it bit
//      for bit; they go to `stats` and to LDS;
//   2. the waves walk the row's blocks: lane (h, t) normalises and modulates
//      its 8 channels of token t from LDS (adaln_bf16x8, per lane, since a
//      tile can straddle two samples), the block is transformed on the matrix
//      cores exactly as in kq_mfma_kernel and quantized into an LDS staging
//      tile;
//   3. the codes and scales leave as whole rows, 16 bytes per lane, while the
//      next tile's loads are in flight.
// Lanes of tokens past the tile's last row compute on a copy of that row and
// store nothing.  With one tile per workgroup nothing overlaps the load, the
// statistics and the blocks of a tile, and the two-launch form, whose many
// workgroups per CU overlap them, measured faster at every width.
// ---------------------------------------------------------------------------
constexpr int kRowsWaves = 16;

// LDS layout for R rows of width d, nsets staged factor sets and the
// modulation rows of up to nmod samples (shift, then scale, fp32).  Regions
// filled by LDS-DMA are whole 1 KB instructions long, so the lanes past their
// data (which write zeros) stay inside them.
__host__ __device__ inline AdRowsLayout adaln_rows_layout(int R, int d, int nsets, int nmod)
{
    AdRowsLayout L;
    L.xrow = 2 * d + 16;
    L.qrow = d / 2 + 16;
    L.srow = (d / 32 + 15) / 16 * 16;
    const int round = 1024 * kRowsWaves; // one DMA instruction of every wave
    L.qoff = (R * L.xrow + round - 1) / round * round;
    L.soff = L.qoff + R * L.qrow;
    L.toff = L.soff + R * L.srow;
    L.foff = (L.toff + R * 16 + 1023) / 1024 * 1024;
    L.moff = L.foff + (nsets * 80 + 1023) / 1024 * 1024;
    L.nmod = nmod;
    L.mbytes = (nmod * d * 4 + 1023) / 1024 * 1024;
    L.bytes = L.moff + 2 * L.mbytes;
    return L;
}

// bytes (a multiple of 16) from rsrc into LDS at dst by 16-byte LDS-DMA loads,
// 1 KB per instruction, instructions dealt to the waves in turn
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t rsrc, unsigned char *dst, int bytes, int wave,
                                           int lane)
{
    const int n = (bytes + 1023) >> 10;
    for (int k = wave; k < n; k += kRowsWaves) {
        const int o = (k << 10) + lane * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void *)(dst + (k << 10)), 16,
            (int)(o < bytes ? (unsigned)o : 0x80000000u), 0, 0, 0);
    }
}

__global__ __launch_bounds__(64 * kRowsWaves) void adaln_rows_kernel(
    const uint16_t *__restrict__ h, int64_t M, int d, const float *__restrict__ shift,
    const float *__restrict__ scale, int64_t T, float eps, const float *__restrict__ factors, int per_block,
    double *__restrict__ stats, uint8_t *__restrict__ q, uint8_t *__restrict__ s, int R, int nmod)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int nB = d >> 5, nOct = d >> 3;
    const AdRowsLayout L = adaln_rows_layout(R, d, per_block ? nB : 1, nmod);
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int slots = nOct + 1; // 16-byte slots of a padded LDS row
    const int h2 = lane >> 5, tl = lane & 31;
    const int64_t nTiles = (M + R - 1) / R;
    const int64_t nS = (M + T - 1) / T;
    constexpr unsigned kVm0 = 0x0F70u; // s_waitcnt vmcnt(0) alone

    // Loads of tile `tile`: its rows of h into the x region (instruction k of
    // wave w fills slots 64 (w + kRowsWaves k) .. +63; pad slots, rows past R
    // and rows past M fetch nothing and write zeros) and, when its rows span
    // at most nmod samples, those samples' modulation rows.
    auto load_tile = [&](int64_t tile) {
        const int64_t r0 = tile * R;
        const int rows = (int)((M - r0) < R ? (M - r0) : R);
        const __amdgpu_buffer_rsrc_t rh =
            __builtin_amdgcn_make_buffer_rsrc((void *)(h + r0 * d), 0, rows * d * 2, kBufWord3);
        for (int base = wave * 64; base < L.qoff / 16; base += 64 * kRowsWaves) {
            const int p = base + lane;
            const int row = p / slots, slot = p - row * slots;
            const unsigned off = (row < R && slot < nOct) ? (unsigned)(row * d + slot * 8) * 2u : 0x80000000u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (__attribute__((address_space(3))) void *)(lds + base * 16),
                                                     16, (int)off, 0, 0, 0);
        }
        const int64_t b0 = r0 / T, ns = (r0 + rows - 1) / T - b0 + 1;
        if (ns <= nmod) {
            const int bytes = (int)ns * d * 4;
            dma_to_lds(__builtin_amdgcn_make_buffer_rsrc((void *)(shift + b0 * d), 0, bytes, kBufWord3),
                       lds + L.moff, bytes, wave, lane);
            dma_to_lds(__builtin_amdgcn_make_buffer_rsrc((void *)(scale + b0 * d), 0, bytes, kBufWord3),
                       lds + L.moff + L.mbytes, bytes, wave, lane);
        }
    };

    // the factor sets, staged once
    const int fbytes = (per_block ? nB : 1) * 80;
    dma_to_lds(__builtin_amdgcn_make_buffer_rsrc((void *)factors, 0, fbytes, kBufWord3), lds + L.foff, fbytes, wave,
               lane);
    const float *fl = (const float *)(lds + L.foff);
    bf16x8 A[3][2];
    if ((int64_t)blockIdx.x < nTiles)
        load_tile(blockIdx.x);
    bool built = false;
    for (int64_t tile = blockIdx.x; tile < nTiles; tile += gridDim.x) {
        const int64_t r0 = tile * R;
        const int rows = (int)((M - r0) < R ? (M - r0) : R);
        // this wave's loads (and earlier stores) done, then everyone's
        __builtin_amdgcn_s_waitcnt(kVm0);
        __syncthreads();
        asm volatile("" ::: "memory");
        if (!per_block && !built) {
            build_a_operands(A, fl, 0, lane);
            built = true;
        }

        // statistics: wave w takes rows w and w + kRowsWaves together (their
        // reductions interleave), each summed as a row alone
        for (int r = wave; r < rows; r += 2 * kRowsWaves) {
            const bool two = r + kRowsWaves < rows;
            const unsigned char *xa = lds + r * L.xrow;
            const unsigned char *xb = lds + (two ? r + kRowsWaves : r) * L.xrow;
            double s1[2] = {0.0, 0.0}, s2[2] = {0.0, 0.0};
            for (int o = lane; o < nOct; o += 64) {
                adaln_piece_sums(*(const u32x4 *)(xa + o * 16), s1[0], s2[0]);
                adaln_piece_sums(*(const u32x4 *)(xb + o * 16), s1[1], s2[1]);
            }
            double mu[2], rstd[2];
            adaln_row_finish2(s1, s2, d, eps, mu, rstd);
            if (lane < (two ? 2 : 1)) {
                const int rr = r + lane * kRowsWaves;
                const double m = lane ? mu[1] : mu[0], rs = lane ? rstd[1] : rstd[0];
                *(double *)(lds + L.toff + rr * 16) = m;
                *(double *)(lds + L.toff + rr * 16 + 8) = rs;
                stats[2 * (r0 + rr)] = m;
                stats[2 * (r0 + rr) + 1] = rs;
            }
        }
        __syncthreads();

        // blocks: normalise, transform, quantize into the staging tile
        const int tr = tl < rows ? tl : rows - 1; // the lane's row (a copy of the last for tokens past it)
        const double mu = *(const double *)(lds + L.toff + tr * 16);
        const double rstd = *(const double *)(lds + L.toff + tr * 16 + 8);
        const int64_t b0 = r0 / T;
        const bool staged = (r0 + rows - 1) / T - b0 + 1 <= nmod;
        const int64_t b = (r0 + tr) / T; // the lane's sample
        const float *msh = staged ? (const float *)(lds + L.moff) + (b - b0) * d : shift + (b < nS ? b : nS - 1) * d;
        const float *msc =
            staged ? (const float *)(lds + L.moff + L.mbytes) + (b - b0) * d : scale + (b < nS ? b : nS - 1) * d;
        const unsigned char *xrow = lds + tr * L.xrow;
        for (int jb = wave; jb < nB; jb += kRowsWaves) {
            if (per_block)
                build_a_operands(A, fl + jb * 20, 0, lane);
            bf16x8 bv[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int oct = jb * 4 + 2 * j + h2; // channels 32 jb + 16 j + 8 h .. +7
                double g[8], sh[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    g[e] = 1.0 + (double)msc[oct * 8 + e];
                    sh[e] = (double)msh[oct * 8 + e];
                }
                unsigned xw[4];
                adaln_bf16x8(*(const u32x4 *)(xrow + oct * 16), mu, rstd, g, sh, xw);
                bv[j] = __builtin_bit_cast(bf16x8, u32x4{xw[0], xw[1], xw[2], xw[3]});
            }
            const f32x16 acc = block_product(A, bv);
            unsigned w0, w1;
            const unsigned bs = mx_tile(acc, w0, w1);
            if (tl < rows) {
                typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
                *(u32x2 *)(lds + L.qoff + tl * L.qrow + jb * 16 + 8 * h2) = u32x2{w0, w1};
                if (h2 == 0)
                    lds[L.soff + tl * L.srow + jb] = (unsigned char)bs;
            }
        }
        __syncthreads();

        // the next tile's loads go out while this tile's codes and scales leave
        if (tile + gridDim.x < nTiles)
            load_tile(tile + gridDim.x);
        const int pieces = d >> 5; // 16-byte code pieces per row
        const __amdgpu_buffer_rsrc_t rq = out_buffer(q + r0 * (d >> 1), (int64_t)rows * (d >> 1));
        for (int c = t; c < rows * pieces; c += 64 * kRowsWaves) {
            const int row = c / pieces, pc = c - row * pieces;
            const u32x4 v = *(const u32x4 *)(lds + L.qoff + row * L.qrow + pc * 16);
            __builtin_amdgcn_raw_buffer_store_b128(v, rq, row * (d >> 1) + pc * 16, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t rs = out_buffer(s + r0 * nB, (int64_t)rows * nB);
        for (int c = t; c < rows * nB; c += 64 * kRowsWaves) {
            const int row = c / nB, k = c - row * nB;
            __builtin_amdgcn_raw_buffer_store_b8(lds[L.soff + row * L.srow + k], rs, row * nB + k, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Streaming variants: one lane per 8 channels, a wave covers 512 channels
// (16 blocks) of U rows at a time and walks a run of rows.
// ---------------------------------------------------------------------------
enum StreamMode { kSQ = 0, kMXF32 = 1, kBflyQ = 2, kBflyT = 3, kFwhtQ = 4, kFwhtT = 5, kBfly16Q = 6, kBfly16T = 7 };

// Unnormalised Walsh-Hadamard stage on an in-lane index bit (stride ST):
// pairs (u at bit 0, w at bit 1) become (u + w, u - w).
template <int ST>
__device__ __forceinline__ void wht_inlane(float (&v)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i & ST)
            continue;
        const float u = v[i], w = v[i + ST];
        v[i] = u + w;
        v[i + ST] = u - w;
    }
}

constexpr float kInvSqrt32 = 0.17677669529663688f; // fl32(1 / sqrt(32))

constexpr int kStreamU = 4; // rows per pipeline stage of the streaming kernels

// Raw loads of U rows of one lane's 8 channels, through a buffer range that
// holds exactly the wave's rows [m0, m1).  Rows past m1 and lanes past the
// row end (bit 31 of lane_off) fall outside it: the hardware returns zeros
// without touching memory, and no such value is stored.  Nontemporal: x is
// read once.
template <int kMode>
struct RowsIn {
    u32x4 v[kStreamU][kMode == kMXF32 ? 2 : 1];
};

template <int kMode>
__device__ __forceinline__ void load_rows(RowsIn<kMode> &in, __amdgpu_buffer_rsrc_t rx, int mr, int d,
                                          unsigned lane_off)
{
    constexpr int kES = kMode == kMXF32 ? 4 : 2; // bytes per input element
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
        const unsigned off = (unsigned)((mr + u) * d * kES) + lane_off;
        in.v[u][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, kAuxNT));
        if constexpr (kMode == kMXF32)
            in.v[u][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(off + 16), 0, kAuxNT));
    }
}

template <int kMode>
__device__ __forceinline__ void process_rows(const RowsIn<kMode> &in, int64_t m, int64_t m0, int64_t m1, int d, int nB,
                                             int oct, bool cok, int qp, const float (&r)[8], const Bfly &B,
                                             const Bfly16 &B16,
                                             __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs,
                                             float *__restrict__ y)
{
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
        float v[8];
        if constexpr (kMode == kMXF32) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = __uint_as_float(in.v[u][0][i]) + 0.0f; // -0 -> +0
                v[4 + i] = __uint_as_float(in.v[u][1][i]) + 0.0f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = bf16lo(in.v[u][0][i]);
                v[2 * i + 1] = bf16hi(in.v[u][0][i]);
            }
        }
        if constexpr (kMode == kSQ) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = __builtin_fmaf(v[i], r[i], 0.0f); // one rounding; -0 -> +0
        }
        if constexpr (kMode == kBflyQ || kMode == kBflyT)
            bfly_stages(v, B);
        if constexpr (kMode == kBfly16Q || kMode == kBfly16T)
            bfly16_stages(v, B16);
        if constexpr (kMode == kFwhtQ || kMode == kFwhtT) {
            // Walsh-Hadamard comparison transform: the same five stages with
            // fixed +-1 coefficients.  Cross-lane bits 4 and 3: a lane at bit
            // value b keeps own + other (b = 0) or other - own (b = 1); then the
            // in-lane bits 2, 1, 0; then one multiply by fl32(1/sqrt 32),
            // started from +0 so no result is -0.
            const float s4 = (qp & 2) ? -1.0f : 1.0f, s3 = (qp & 1) ? -1.0f : 1.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = __builtin_fmaf(s4, v[i], dpp_xor2(v[i]));
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = __builtin_fmaf(s3, v[i], dpp_xor1(v[i]));
            wht_inlane<4>(v);
            wht_inlane<2>(v);
            wht_inlane<1>(v);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = __builtin_fmaf(v[i], kInvSqrt32, 0.0f);
        }
        const int64_t mm = m + u;
        if constexpr (kMode == kBflyT || kMode == kFwhtT || kMode == kBfly16T) {
            if (mm < m1 && cok) {
                f32x4 *o = (f32x4 *)(y + mm * d + (int64_t)oct * 8);
                o[0] = f32x4{v[0], v[1], v[2], v[3]};
                o[1] = f32x4{v[4], v[5], v[6], v[7]};
            }
        } else {
            // 32-element blocks span a quad of lanes, 16-element blocks a pair
            constexpr bool k16 = kMode == kBfly16Q;
            unsigned b;
            const unsigned w = k16 ? mx_encode_pair(v, b) : mx_encode_quad(v, b);
            // rows past the run fall outside the wave's ranges; lanes past the row
            // end (and all lanes of a block but the first for s) set bit 31 of their offset
            const int mr = (int)(mm - m0);
            const unsigned drop_q = (unsigned)(cok ? 0 : 1) << 31;
            const unsigned drop_s = drop_q | ((unsigned)((qp & (k16 ? 1 : 3)) != 0) << 31);
            __builtin_amdgcn_raw_buffer_store_b32(w, rq, (int)((unsigned)(mr * (d >> 1) + oct * 4) | drop_q), 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)b, rs,
                                                 (int)((unsigned)(mr * nB + (oct >> (k16 ? 1 : 2))) | drop_s), 0, 0);
        }
    }
}

template <int kMode>
__global__ __launch_bounds__(256) void stream_kernel(const void *__restrict__ xin, int64_t M, int d,
                                                     const float *__restrict__ aux, int per_block,
                                                     uint8_t *__restrict__ q, uint8_t *__restrict__ s,
                                                     float *__restrict__ y, int rows_per_wave, int nCT)
{
    const int lane = threadIdx.x & 63;
    // A workgroup covers four column tiles of one row group.  All column groups
    // of a row group run on the same XCD back to back (blockIdx % 8 picks the
    // XCD), so the partial lines of q and s rows merge in one L2.
    const int nCG = (nCT + 3) / 4;
    const unsigned xcd = blockIdx.x % kXcds;
    const unsigned slot = blockIdx.x / kXcds;
    const int cg = (int)(slot % (unsigned)nCG);
    const int64_t rg = (int64_t)(slot / (unsigned)nCG) * kXcds + xcd;
    const int ct = cg * 4 + (threadIdx.x >> 6);
    const int64_t m0 = rg * rows_per_wave;
    if (m0 >= M || ct >= nCT)
        return; // wave-uniform; this kernel has no barrier
    const int64_t m1 = (m0 + rows_per_wave < M) ? m0 + rows_per_wave : M;
    const int nOct = d >> 3;
    constexpr bool k16 = kMode == kBfly16Q || kMode == kBfly16T;
    const int nB = k16 ? d >> 4 : d >> 5; // scale blocks per row
    const int oct = ct * 64 + lane;
    const bool cok = oct < nOct;
    const int octc = cok ? oct : nOct - 1; // parameter index for lanes past the row end (results not stored)
    const int qp = lane & 3;
    constexpr int kES = kMode == kMXF32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const unsigned char *)xin + m0 * d * kES), 0, (int)((m1 - m0) * d * kES), kBufWord3);
    const unsigned lane_off = (unsigned)(oct * 8 * kES) | ((unsigned)(cok ? 0 : 1) << 31);

    RowsIn<kMode> bufA, bufB;
    load_rows<kMode>(bufA, rx, 0, d, lane_off);
    const bool quant = (kMode != kBflyT && kMode != kFwhtT && kMode != kBfly16T);
    __amdgpu_buffer_rsrc_t rq = out_buffer(quant ? q + m0 * (d >> 1) : nullptr, quant ? (m1 - m0) * (d >> 1) : 0);
    __amdgpu_buffer_rsrc_t rs = out_buffer(quant ? s + m0 * nB : nullptr, quant ? (m1 - m0) * nB : 0);

    float r[8];
    Bfly B;
    if constexpr (kMode == kSQ) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r[i] = (float)(1.0 / (double)aux[octc * 8 + i]); // correctly rounded fp32 reciprocal
    }
    if constexpr (kMode == kBflyQ || kMode == kBflyT) {
        const int set = per_block ? (octc >> 2) : 0;
        bfly_setup(B, aux + (int64_t)set * 20, qp);
    }
    Bfly16 B16;
    if constexpr (k16) {
        const int set = per_block ? (octc >> 1) : 0;
        bfly16_setup(B16, aux + (int64_t)set * 16, lane & 1);
    }

    // two-stage pipeline; a prefetch past the run falls outside the range and fetches nothing
    int64_t m = m0;
    for (; m + kStreamU < m1; m += 2 * kStreamU) {
        load_rows<kMode>(bufB, rx, (int)(m + kStreamU - m0), d, lane_off);
        __builtin_amdgcn_sched_barrier(0); // keep the prefetch ahead of these rows' stores
        process_rows<kMode>(bufA, m, m0, m1, d, nB, oct, cok, qp, r, B, B16, rq, rs, y);
        __builtin_amdgcn_sched_barrier(0);
        load_rows<kMode>(bufA, rx, (int)(m + 2 * kStreamU - m0), d, lane_off);
        __builtin_amdgcn_sched_barrier(0);
        process_rows<kMode>(bufB, m + kStreamU, m0, m1, d, nB, oct, cok, qp, r, B, B16, rq, rs, y);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (m < m1)
        process_rows<kMode>(bufA, m, m0, m1, d, nB, oct, cok, qp, r, B, B16, rq, rs, y);
}


// ---------------------------------------------------------------------------
// device queries (thread-safe, cached per device and kernel)
// ---------------------------------------------------------------------------
namespace {
std::mutex g_info_mu;
std::map<int, int> g_cus;
std::map<std::pair<int, const void *>, int> g_occ;

int current_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        dev = 0;
    return dev;
}
} // namespace

int device_cus()
{
    const int dev = current_device();
    std::lock_guard<std::mutex> lock(g_info_mu);
    const auto it = g_cus.find(dev);
    if (it != g_cus.end())
        return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    g_cus[dev] = n;
    return n;
}

int occupancy_per_cu(const void *fn, int threads)
{
    const int dev = current_device();
    std::lock_guard<std::mutex> lock(g_info_mu);
    const auto key = std::make_pair(dev, fn);
    const auto it = g_occ.find(key);
    if (it != g_occ.end())
        return it->second;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    g_occ[key] = per_cu;
    return per_cu;
}

namespace {
std::map<std::pair<int, const void *>, hipError_t> g_lds_attr;
} // namespace

// Raise fn's dynamic LDS limit to `bytes` on the current device, once per
// (device, kernel); later calls return the first call's result.
hipError_t allow_dynamic_lds(const void *fn, int bytes)
{
    const int dev = current_device();
    std::lock_guard<std::mutex> lock(g_info_mu);
    const auto key = std::make_pair(dev, fn);
    const auto it = g_lds_attr.find(key);
    if (it != g_lds_attr.end())
        return it->second;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    g_lds_attr[key] = e;
    return e;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
namespace {

// Resident workgroups per XCD of an MFMA quantizer instance (at least 1).
int64_t mfma_wgs_per_xcd(const void *fn, int threads)
{
    const int64_t v = (int64_t)occupancy_per_cu(fn, threads) * device_cus() / (int64_t)kXcds;
    return v < 1 ? 1 : v;
}

// The quantizing instance of a strip width and ring depth: the launch shape of
// every form (quantizer, transform export, nontemporal stores) is taken from
// its occupancy.
const void *mfma_shape_fn(int w, bool adaln, int ring)
{
    if (ring == 2) {
        if (adaln)
            return w == 4 ? (const void *)kq_mfma_kernel<true, 4, true, false, 2>
                          : (const void *)kq_mfma_kernel<true, 8, true, false, 2>;
        if (w == 4)
            return (const void *)kq_mfma_kernel<true, 4, false, false, 2>;
        return w == 16 ? (const void *)kq_mfma_kernel<true, 16, false, false, 2>
                       : (const void *)kq_mfma_kernel<true, 8, false, false, 2>;
    }
    if (adaln)
        return w == 4 ? (const void *)kq_mfma_kernel<true, 4, true> : (const void *)kq_mfma_kernel<true, 8, true>;
    if (w == 4)
        return (const void *)kq_mfma_kernel<true, 4>;
    return w == 16 ? (const void *)kq_mfma_kernel<true, 16> : (const void *)kq_mfma_kernel<true, 8>;
}

// The last-level cache (MALL) of MI355X.  A launch whose x, q and s together
// exceed it streams its codes past the caches (nontemporal stores): no later
// kernel could find them there anyway.
constexpr int64_t kMallBytes = (int64_t)256 << 20;

// Token grouping for strip width w: tiles per workgroup, interleaved or
// contiguous groups, flat or XCD-grouped order.
void mfma_groups(int64_t M, int64_t d, int w, bool adaln, int ring, const Tuning &tn, MfmaShape &sh)
{
    const int64_t nB = d / 32;
    const int64_t nBG = (nB + w - 1) / w;
    const int64_t nTiles = (M + kTileT - 1) / kTileT;
    const int64_t resident = mfma_wgs_per_xcd(mfma_shape_fn(w, adaln, ring), 64 * w);
    int64_t tpw = tn.mfma_tiles_per_wg;
    int interleave = tn.mfma_groups == 2 ? 1 : 0;
    bool flat = tn.mfma_order == 2;
    if (tpw <= 0 && tn.mfma_order == 0 && tn.mfma_groups != 1) {
        // When XCD-grouped token groups would fill under 80% of the resident
        // workgroup slots (strips per row not a good divisor of the slots per
        // XCD: e.g. 35 strips against 64 slots), deal (group, strip) pairs in
        // flat order instead and cover the rows in one interleaved round
        // (measured: 2048 x 8960 from 14.6 to 13.0 us, 4608 x 12288 from 30.1
        // to 28.1 us).
        const int64_t gx = resident / nBG;
        const int64_t groups_f = resident * kXcds / nBG;
        if (groups_f >= 1 && 5 * (gx < 1 ? 1 : gx) * nBG < 4 * resident) {
            const int64_t t1f = (nTiles + groups_f - 1) / groups_f;
            if (t1f >= 3 && t1f <= 16) {
                tpw = t1f;
                interleave = 1;
                flat = true;
            }
        }
    }
    if (tpw <= 0) {
        // Launch shape, from measurements on MI355X (HBM time of one launch
        // against tiles per workgroup, for M = 2048..65536 and d = 1152..12288):
        // workgroups resident at the same time should cover one compact band
        // of rows, and each should walk enough tiles to hide its start-up.
        //  - If one resident round of interleaved token groups covers the rows
        //    with 3..12 tiles per workgroup, use it.
        //  - Fewer tiles than that: contiguous groups of 3 tiles.
        //  - Otherwise contiguous groups of 4 tiles once that makes at least
        //    four rounds of resident workgroups, else of 6.
        //  - At exactly 3 tiles per interleaved group, contiguous groups of 6
        //    tiles are faster while they still give 90% of the CUs a
        //    workgroup: half as many workgroups start, each with a longer
        //    pipeline (measured at 8192 x 1152 on three MI355X machines: 8.3 us against
        //    8.5-9.2).
        int64_t gx = resident / nBG; // token groups per XCD in one round
        if (gx < 1)
            gx = 1;
        const int64_t t1 = (nTiles + gx * kXcds - 1) / (gx * kXcds);
        const int64_t wgs6 = ((nTiles + 5) / 6 + kXcds - 1) / kXcds * kXcds * nBG;
        if (tn.mfma_groups != 1 && t1 == 3 && 10 * wgs6 >= 9 * (int64_t)device_cus()) {
            tpw = 6;
            interleave = 0;
        } else if (tn.mfma_groups != 1 && t1 >= 3 && t1 <= 12) {
            tpw = t1;
            interleave = 1;
        } else if (t1 < 3) {
            tpw = 3;
            interleave = 0;
        } else {
            const int64_t groups4 = (nTiles + 3) / 4;
            const int64_t rounds4 = ((groups4 + kXcds - 1) / kXcds * nBG) / resident;
            tpw = rounds4 >= 4 ? 4 : 6;
            interleave = 0;
        }
        if (tn.mfma_groups == 2)
            interleave = 1;
    }
    const int64_t nG = (nTiles + tpw - 1) / tpw;
    // XCD-grouped: token groups dealt to the XCDs in turn, padded to a multiple of 8
    const int64_t nGpad = flat ? nG : (nG + kXcds - 1) / kXcds * kXcds;
    sh.strip = w;
    sh.tiles_per_wg = (int)tpw;
    sh.interleave = interleave;
    sh.flat = flat ? 1 : 0;
    sh.grid = nGpad * nBG;
}

template <int kW, bool kAd, bool kNT, int kRing, bool kB16 = false>
hipError_t launch_mfma_instance(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT,
                                uint8_t *q, uint8_t *s, float *y, int lu, const MfmaShape &sh, hipStream_t stream,
                                AdArgs ad)
{
    if (sh.grid > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    const void *fn;
    if constexpr (kAd)
        fn = (const void *)kq_mfma_kernel<true, kW, true, false, kRing>;
    else
        fn = y ? (const void *)kq_mfma_kernel<false, kW, false, false, kRing, kB16>
               : (const void *)kq_mfma_kernel<true, kW, false, kNT, kRing, kB16>;
    int di = (int)d;
    int per_block = nT > 1 ? 1 : 0;
    int nbg = (int)((d / 32 + kW - 1) / kW);
    int tpw = sh.tiles_per_wg;
    int order = (sh.interleave ? 1 : 0) | (sh.flat ? 2 : 0);
    void *args[] = {(void *)&x,   (void *)&M,   (void *)&di,  (void *)&factors, (void *)&per_block, (void *)&q,
                    (void *)&s,   (void *)&y,   (void *)&nbg, (void *)&tpw,     (void *)&order,     (void *)&lu,
                    (void *)&ad};
    return hipLaunchKernel(fn, dim3((unsigned)sh.grid), dim3(64 * kW), args, 0, stream);
}

} // namespace

// Long runs: one resident round of persistent workgroups.  Token groups
// interleave (tile = group + k * groups) and (group, strip) pairs are dealt in
// flat order, so the workgroups walk one compact band of rows down the matrix
// and each pays its start-up once.  Strips of 16 blocks when they divide the
// row (measured on one MI355X, 65536 x 12288: 329 us against 381 for contiguous
// groups of 4 tiles in strips of 8; 16384 x 12288: 87.2 against 97.5).
// Taken when that round needs more than 16 tiles per workgroup and fills at
// least 80% of the resident slots; false otherwise.
bool mfma_long_run(int64_t M, int64_t d, MfmaShape &sh)
{
    const int64_t nB = d / 32;
    const int w = nB % 16 == 0 ? 16 : 8;
    const int64_t nBG = (nB + w - 1) / w;
    const int64_t nTiles = (M + kTileT - 1) / kTileT;
    const int64_t slots = mfma_wgs_per_xcd(mfma_shape_fn(w, false, 2), 64 * w) * kXcds;
    const int64_t groups = slots / nBG;
    if (groups < 1 || 5 * groups * nBG < 4 * slots)
        return false;
    const int64_t tpw = (nTiles + groups - 1) / groups;
    if (tpw <= 16 || tpw > 0x7FFFFFFF)
        return false;
    sh.strip = w;
    sh.tiles_per_wg = (int)tpw;
    sh.interleave = 1;
    sh.flat = 1;
    sh.grid = (nTiles + tpw - 1) / tpw * nBG;
    return true;
}

// Mid-size runs: one resident round of at most one workgroup per CU, whose
// interleaved token groups (flat order) each walk 6..16 tiles.  Of strips of
// 16 and 8 blocks (whichever divide the row) the one that gives the longer
// runs inside that range is taken.  Used when the shape above would put more
// than one workgroup on a CU or walk fewer than 8 tiles per workgroup
// (measured on two MI355X machines against that shape: 4608 x 3072 10.1 against 11.2
// us, 2048 x 8960 12.0 against 12.8, 4608 x 12288 27.3 against 29.3, 4096 x
// 12288 24.7 against 25.5, 2048 x 12288 14.4 against 15.0; at 8192 x 4608,
// where that shape already is one round of 11 tiles per workgroup, this one
// was 2% slower, so it is not taken there).  Leaves sh unchanged when no
// strip gives such a round.
void mfma_one_per_cu(int64_t M, int64_t d, MfmaShape &sh)
{
    const int64_t nB = d / 32;
    const int64_t nTiles = (M + kTileT - 1) / kTileT;
    const int64_t cus = device_cus();
    int best_w = 0;
    int64_t best_t = 0;
    for (const int w : {16, 8}) {
        if (nB % w != 0)
            continue;
        const int64_t groups = cus / (nB / w);
        if (groups < 1)
            continue;
        const int64_t tpw = (nTiles + groups - 1) / groups;
        if (tpw >= 6 && tpw <= 16 && tpw > best_t) {
            best_w = w;
            best_t = tpw;
        }
    }
    if (best_w == 0)
        return;
    // In strips of 16 (16-wave workgroups) the longest runs of the range, 16
    // tiles, while they still give three CUs of four a workgroup: fewer
    // loads in flight per round measured faster (with the ring of 2, two
    // machines: 4608 x 12288 26.8 against 28.1-29.9 us for 15 tiles on 240
    // workgroups; 4096 x 12288 25.5 against 27.3-29.4 for 13 tiles).
    if (best_w == 16 && best_t < 16 && 4 * ((nTiles + 15) / 16) * (nB / 16) >= 3 * cus)
        best_t = 16;
    sh.strip = best_w;
    sh.tiles_per_wg = (int)best_t;
    sh.interleave = 1;
    sh.flat = 1;
    sh.grid = (nTiles + best_t - 1) / best_t * (nB / best_w);
}

hipError_t mfma_launch_shape(int64_t M, int64_t d, const Tuning &tn, bool adaln, MfmaShape &sh)
{
    const int64_t nB = d / 32;
    const bool automatic =
        tn.mfma_strip == 0 && tn.mfma_tiles_per_wg <= 0 && tn.mfma_groups == 0 && tn.mfma_order == 0;
    const bool long_run = !adaln && automatic && mfma_long_run(M, d, sh);
    int w = sh.strip;
    if (long_run) {
        // shape complete
    } else if (adaln) {
        // The normalisation takes the registers of a lane to about 180 VGPRs
        // (two waves per SIMD), so 16-block strips (1024 threads, at most 128
        // VGPRs) are not offered.  Strips of 4 blocks when they divide the row
        // and strips of 8 do not (measured at 8192 x 1152: 18.95 against 19.83
        // us for the whole front-end; strips of 8 were as fast or faster at
        // 2048 x 2240 and 4608 x 3072).
        w = tn.adaln_strip;
        if (w != 4 && w != 8)
            w = (nB % 4 == 0 && nB % 8 != 0) ? 4 : 8;
    } else {
        // Strips of 16 blocks (16 waves, 1 KB of each row per workgroup, 85 KB
        // of LDS, one workgroup per CU) read and write HBM in longer runs than
        // strips of 8, which pays when the whole launch is one resident round
        // of interleaved token groups (measured: 8192 x 4608, 18.3 us against
        // 19.8).  Over several rounds the lone workgroup per CU leaves its CU
        // idle between workgroups, and strips of 8 (two per CU) win.  They are
        // used only when they divide the row exactly, so no wave idles.
        w = tn.mfma_strip;
        if (w != 4 && w != 8 && w != 16 && nB % 8 != 0 && nB % 4 == 0) {
            // Strips of 4 blocks when they divide the row and strips of 8 do
            // not, so no wave idles (measured at 8192 x 1152, contiguous
            // groups of 6 tiles: 7.93 against 8.23 us for strips of 8).
            w = 4;
        } else if (w != 4 && w != 8 && w != 16) {
            w = 8;
            if (nB % 16 == 0 && tn.mfma_tiles_per_wg <= 0 && tn.mfma_groups != 1) {
                int64_t gx = mfma_wgs_per_xcd(mfma_shape_fn(16, false, 2), 64 * 16) / (nB / 16);
                if (gx < 1)
                    gx = 1;
                const int64_t nTiles = (M + kTileT - 1) / kTileT;
                const int64_t t1 = (nTiles + gx * kXcds - 1) / (gx * kXcds);
                if (t1 >= 3 && t1 <= 12)
                    w = 16;
            }
        }
    }
    // Register ring: 2 tiles (one in flight ahead) except in the persistent
    // long runs and the AdaLN second pass, which keep 4.  Measured with
    // per-block factor sets, ring 2 against ring 4 in the same runs (three
    // machines): 2-8% faster at every configured shape below the long runs
    // (8192 x 1152: 7.5 against 8.0 us; 8192 x 4608: 18.6 against 19.5), at
    // 16384 x 12288 1% slower on two machines of three (85.0 against 84.0), at
    // 65536 x 12288 within the spread of identical legs.
    const int ring = tn.mfma_ring ? tn.mfma_ring : (adaln || long_run) ? 4 : 2;
    if (!long_run) {
        mfma_groups(M, d, w, adaln, ring, tn, sh);
        if (!adaln && automatic && (sh.grid > device_cus() || sh.tiles_per_wg < 8))
            mfma_one_per_cu(M, d, sh);
    }
    sh.ring = ring;
    const double footprint = (double)M * (double)d * (2.0 + 0.5 + 1.0 / 32.0);
    sh.nt_codes = !adaln && (tn.code_stores == 2 || (tn.code_stores == 0 && footprint > (double)kMallBytes));
    return sh.grid > 0x7FFFFFFF ? hipErrorInvalidConfiguration : hipSuccess;
}

template <int kRing, bool kB16 = false>
hipError_t launch_mfma_ring(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                            uint8_t *s, float *y, int lu, const MfmaShape &sh, hipStream_t stream)
{
    const AdArgs ad{};
    const bool nt = sh.nt_codes && !y;
    if (sh.strip == 16)
        return nt ? launch_mfma_instance<16, false, true, kRing, kB16>(x, M, d, factors, nT, q, s, y, lu, sh, stream, ad)
                  : launch_mfma_instance<16, false, false, kRing, kB16>(x, M, d, factors, nT, q, s, y, lu, sh, stream,
                                                                        ad);
    if (sh.strip == 4) {
        // 16-element blocks reach the ring of 4 only in the persistent long
        // runs, whose strips are 16 or 8 blocks wide; that instance (which
        // spills two registers) is not built.
        if constexpr (kB16 && kRing == 4)
            return hipErrorInvalidConfiguration;
        else
            return nt ? launch_mfma_instance<4, false, true, kRing, kB16>(x, M, d, factors, nT, q, s, y, lu, sh, stream,
                                                                          ad)
                      : launch_mfma_instance<4, false, false, kRing, kB16>(x, M, d, factors, nT, q, s, y, lu, sh,
                                                                           stream, ad);
    }
    return nt ? launch_mfma_instance<8, false, true, kRing, kB16>(x, M, d, factors, nT, q, s, y, lu, sh, stream, ad)
              : launch_mfma_instance<8, false, false, kRing, kB16>(x, M, d, factors, nT, q, s, y, lu, sh, stream, ad);
}

// Flat form (one shared factor set).  Measured on MI355X over the configured
// shapes (rotating inputs, graphs of 40 launches; ring depths 2..10 against
// 128..1024 workgroups of 4 waves): the fastest launches keep few loads in
// flight.  While x, q and s together fit the last-level cache: a ring of 2
// units and 2 workgroups per CU (8192 x 4608: 16.7 us; rings of 3-5 or 1, 3
// or 4 workgroups per CU 17.5-23.0).  Above it: a ring of 3 units and one
// workgroup per CU (65536 x 12288: 322 us; a ring of 2 at 2 per CU 379, any
// ring at 3 or 4 per CU 380-400).  Fractions of a workgroup per CU leave the
// CUs unevenly loaded and were slower at every size.
bool flat_form(int64_t nT, const Tuning &tn)
{
    if (nT != 1 || tn.shared_form == 1)
        return false;
    return tn.shared_form == 2 ||
           (tn.mfma_strip == 0 && tn.mfma_tiles_per_wg <= 0 && tn.mfma_groups == 0 && tn.mfma_order == 0);
}

void flat_launch_shape(int64_t M, int64_t d, const Tuning &tn, FlatShape &sh, bool b16)
{
    const double footprint = (double)M * (double)d * (2.0 + 0.5 + (b16 ? 1.0 / 16.0 : 1.0 / 32.0));
    const bool big = footprint > (double)kMallBytes;
    sh.nt_codes = tn.code_stores == 2 || (tn.code_stores == 0 && big);
    sh.ring = tn.flat_ring ? tn.flat_ring : (big ? 3 : 2);
    int64_t wgs = tn.flat_wgs > 0 ? tn.flat_wgs : (int64_t)(big ? 1 : 2) * device_cus();
    const int64_t nunits = (M * d + 1023) / 1024;
    const int64_t need = (nunits + kFlatWaves - 1) / kFlatWaves;
    sh.wgs = wgs < need ? wgs : need;
}

template <bool kB16>
hipError_t launch_flat_instance(const uint16_t *x, int64_t M, int64_t d, const float *factors, uint8_t *q,
                                uint8_t *s, float *y, int lu, const Tuning &tn, hipStream_t stream)
{
    FlatShape sh{};
    flat_launch_shape(M, d, tn, sh, kB16);
    const int64_t nelem = M * d;
    const void *fn;
    if (sh.ring == 3)
        fn = y ? (const void *)kq_flat_kernel<false, false, 3, kB16>
             : sh.nt_codes ? (const void *)kq_flat_kernel<true, true, 3, kB16>
                           : (const void *)kq_flat_kernel<true, false, 3, kB16>;
    else
        fn = y ? (const void *)kq_flat_kernel<false, false, 2, kB16>
             : sh.nt_codes ? (const void *)kq_flat_kernel<true, true, 2, kB16>
                           : (const void *)kq_flat_kernel<true, false, 2, kB16>;
    void *args[] = {(void *)&x, (void *)&nelem, (void *)&factors, (void *)&lu, (void *)&q, (void *)&s, (void *)&y};
    return hipLaunchKernel(fn, dim3((unsigned)sh.wgs), dim3(64 * kFlatWaves), args, 0, stream);
}

hipError_t launch_kq_flat(const uint16_t *x, int64_t M, int64_t d, const float *factors, uint8_t *q, uint8_t *s,
                          float *y, int lu, const Tuning &tn, hipStream_t stream)
{
    return launch_flat_instance<false>(x, M, d, factors, q, s, y, lu, tn, stream);
}

hipError_t launch_kq_mfma(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                          uint8_t *s, float *y, int lu, const Tuning &tn, hipStream_t stream)
{
    if (flat_form(nT, tn))
        return launch_kq_flat(x, M, d, factors, q, s, y, lu, tn, stream);
    MfmaShape sh{};
    hipError_t e = mfma_launch_shape(M, d, tn, false, sh);
    if (e != hipSuccess)
        return e;
    return sh.ring == 2 ? launch_mfma_ring<2>(x, M, d, factors, nT, q, s, y, lu, sh, stream)
                        : launch_mfma_ring<4>(x, M, d, factors, nT, q, s, y, lu, sh, stream);
}

// One-launch AdaLN form.  Rows per tile R: enough for every CU to take at most
// one tile (at most 32, one matrix-core tile of tokens), fewer (down to 8) when
// the LDS cannot hold that many.  Staged modulation: the most samples (2, 1, 0)
// whose rows still fit beside them.  Grid: one resident round.
constexpr int kAdRowsLds = 160 * 1024; // LDS of one CU (gfx950), all of it for one workgroup at most
bool adaln_rows_shape(int64_t M, int64_t d, int64_t nT, AdRowsShape &sh)
{
    if (M < 1 || d > 65536)
        return false;
    const int nsets = nT > 1 ? (int)(d / 32) : 1;
    const int64_t cus = device_cus();
    int64_t need = (M + cus - 1) / cus;
    if (need > 32)
        need = 32;
    const int floor_r = need < 8 ? (int)need : 8;
    for (int r = (int)need; r >= floor_r; --r)
        for (int nm = 2; nm >= 0; --nm) {
            const AdRowsLayout L = adaln_rows_layout(r, (int)d, nsets, nm);
            if (L.bytes > kAdRowsLds)
                continue;
            sh.R = r;
            sh.nmod = nm;
            sh.bytes = L.bytes;
            const int64_t nTiles = (M + r - 1) / r;
            int per_cu = kAdRowsLds / L.bytes;
            const int occ = occupancy_per_cu((const void *)adaln_rows_kernel, 64 * kRowsWaves);
            if (per_cu > occ)
                per_cu = occ;
            const int64_t slots = cus * (int64_t)(per_cu < 1 ? 1 : per_cu);
            sh.grid = nTiles < slots ? nTiles : slots;
            return true;
        }
    return false;
}

hipError_t launch_adaln_rows(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                             int64_t T, float eps, const float *factors, int64_t nT, double *stats, uint8_t *q,
                             uint8_t *s, hipStream_t stream)
{
    AdRowsShape sh{};
    if (!adaln_rows_shape(M, d, nT, sh))
        return hipErrorInvalidConfiguration;
    // above the default dynamic LDS limit the launch needs the attribute
    hipError_t e = allow_dynamic_lds((const void *)adaln_rows_kernel, kAdRowsLds);
    if (e != hipSuccess)
        return e;
    int di = (int)d;
    int per_block = nT > 1 ? 1 : 0;
    int R = sh.R, nmod = sh.nmod;
    void *args[] = {(void *)&h,     (void *)&M,       (void *)&di,        (void *)&shift, (void *)&scale,
                    (void *)&T,     (void *)&eps,     (void *)&factors,   (void *)&per_block,
                    (void *)&stats, (void *)&q,       (void *)&s,         (void *)&R,     (void *)&nmod};
    return hipLaunchKernel((const void *)adaln_rows_kernel, dim3((unsigned)sh.grid), dim3(64 * kRowsWaves), args,
                           (unsigned)sh.bytes, stream);
}

// Second pass of the AdaLN front-end on the matrix cores: the quantizer's
// launch shape with h in place of x, normalised at staging.
hipError_t launch_adaln_mfma(const uint16_t *h, int64_t M, int64_t d, const double *stats, const float *shift,
                             const float *scale, int64_t T, const float *factors, int64_t nT, uint8_t *q, uint8_t *s,
                             const Tuning &tn, hipStream_t stream)
{
    MfmaShape sh{};
    hipError_t e = mfma_launch_shape(M, d, tn, true, sh);
    if (e != hipSuccess)
        return e;
    const AdArgs ad{stats, shift, scale, T};
    if (sh.ring == 2)
        return sh.strip == 4
                   ? launch_mfma_instance<4, true, false, 2>(h, M, d, factors, nT, q, s, nullptr, 0, sh, stream, ad)
                   : launch_mfma_instance<8, true, false, 2>(h, M, d, factors, nT, q, s, nullptr, 0, sh, stream, ad);
    if (sh.strip == 4)
        return launch_mfma_instance<4, true, false, 4>(h, M, d, factors, nT, q, s, nullptr, 0, sh, stream, ad);
    return launch_mfma_instance<8, true, false, 4>(h, M, d, factors, nT, q, s, nullptr, 0, sh, stream, ad);
}

static hipError_t launch_stream(int mode, const void *x, int64_t M, int64_t d, const float *aux, int per_block,
                                uint8_t *q, uint8_t *s, float *y, const Tuning &tn, hipStream_t stream)
{
    const int nOct = (int)(d / 8);
    const int nCT = (nOct + 63) / 64;
    int R = tn.stream_rows_per_wave > 256 ? 256 : tn.stream_rows_per_wave;
    if (R <= 0)
        R = 4; // short-lived waves (one pipeline stage of rows each) keep the most loads in flight

    const int64_t nRG = (M + R - 1) / R;
    const int64_t nRGpad = (nRG + kXcds - 1) / kXcds * kXcds;
    const int64_t grid = nRGpad * ((nCT + 3) / 4);
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    int di = (int)d;
    void *args[] = {(void *)&x, (void *)&M, (void *)&di, (void *)&aux, (void *)&per_block, (void *)&q,
                    (void *)&s, (void *)&y, (void *)&R, (void *)&nCT};
    const void *fn = nullptr;
    switch (mode) {
    case kSQ: fn = (const void *)stream_kernel<kSQ>; break;
    case kMXF32: fn = (const void *)stream_kernel<kMXF32>; break;
    case kBflyQ: fn = (const void *)stream_kernel<kBflyQ>; break;
    case kBflyT: fn = (const void *)stream_kernel<kBflyT>; break;
    case kBfly16Q: fn = (const void *)stream_kernel<kBfly16Q>; break;
    case kBfly16T: fn = (const void *)stream_kernel<kBfly16T>; break;
    case kFwhtQ: fn = (const void *)stream_kernel<kFwhtQ>; break;
    default: fn = (const void *)stream_kernel<kFwhtT>; break;
    }
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, stream);
}

hipError_t launch_kq_butterfly(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT,
                               uint8_t *q, uint8_t *s, float *y, const Tuning &tn, hipStream_t stream)
{
    return launch_stream(y ? kBflyT : kBflyQ, x, M, d, factors, nT > 1 ? 1 : 0, q, s, y, tn, stream);
}

// One shared set: the flat matrix-core kernel with the 32 x 32 block I (x) K16;
// a set per block and rows of whole 32-element pairs: the strip kernel with
// the block diag(K16, K16') of each pair of sets, in the 32-element launch
// shape; other rows: the butterfly streaming kernel.  Both matrix-core forms
// measured faster than the butterfly at every configured shape.
hipError_t launch_kq16(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                       uint8_t *s, float *y, const Tuning &tn, hipStream_t stream)
{
    if (tn.shared_form != 1) {
        if (nT == 1)
            return launch_flat_instance<true>(x, M, d, factors, q, s, y, 0, tn, stream);
        if (d % 32 == 0) {
            MfmaShape sh{};
            hipError_t e = mfma_launch_shape(M, d, tn, false, sh);
            if (e != hipSuccess)
                return e;
            return sh.ring == 2 ? launch_mfma_ring<2, true>(x, M, d, factors, nT, q, s, y, 0, sh, stream)
                                : launch_mfma_ring<4, true>(x, M, d, factors, nT, q, s, y, 0, sh, stream);
        }
    }
    return launch_stream(y ? kBfly16T : kBfly16Q, x, M, d, factors, nT > 1 ? 1 : 0, q, s, y, tn, stream);
}

hipError_t launch_sq(const uint16_t *x, int64_t M, int64_t d, const float *scale, uint8_t *q, uint8_t *s,
                     const Tuning &tn, hipStream_t stream)
{
    return launch_stream(kSQ, x, M, d, scale, 0, q, s, nullptr, tn, stream);
}

hipError_t launch_mx_f32(const float *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, const Tuning &tn,
                         hipStream_t stream)
{
    return launch_stream(kMXF32, x, M, d, nullptr, 0, q, s, nullptr, tn, stream);
}

hipError_t launch_fwht(const uint16_t *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, float *y, const Tuning &tn,
                       hipStream_t stream)
{
    return launch_stream(y ? kFwhtT : kFwhtQ, x, M, d, nullptr, 0, q, s, y, tn, stream);
}

} // namespace kq
