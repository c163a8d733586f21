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
//                    accumulation is fp32.  The pages run the block as "small
//                    tensor-core GEMMs"; here the GEMM is Y^T = K^T X^T so one
//                    token's 32 outputs land in 2 lanes x 16 accumulators.
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

#include "kq_device.h"
#include "kq_internal.h"

namespace kq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

Tuning &tuning()
{
    static Tuning t{0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    return t;
}

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

template <int kW>
struct __align__(16) WgStage {
    unsigned char x[2][kTileT][Strip<kW>::kXRow]; // x tile, double-buffered by tile parity
    unsigned char q[2][kTileT][Strip<kW>::kQRow]; // staged codes
    unsigned char s[2][kTileT][kW];               // staged scale bytes
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

template <int kW>
__device__ __forceinline__ void stage_x(WgStage<kW> &st, int par, const XIn &in, int wave, int lane)
{
    using S = Strip<kW>;
#pragma unroll
    for (int k = 0; k < 2; ++k)
        *(u32x4 *)&st.x[par][S::kRowsPerWave * wave + S::kRowsPerLoad * k + lane / S::kLanesPerRow]
                         [(lane % S::kLanesPerRow) * 16] = in.v[k];
}

// Transform one tile on the matrix cores; quantize into the staging buffer
// (or write y directly).  Lane l takes token l%32 and, for MFMA j, channels
// 16j + 8h .. +7 of block `wave` of the strip (h = l/32).
template <bool kQuant, int kW>
__device__ __forceinline__ void transform_tile(const WgStage<kW> &stc, WgStage<kW> &st, int par, const bf16x8 (&A)[3][2],
                                               int64_t t, int64_t M, int d, int jb, bool jb_valid, int h, int wave,
                                               int tl, float *__restrict__ y)
{
    bf16x8 bv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
        bv[j] = *(const bf16x8 *)&stc.x[par][tl][wave * 64 + 32 * j + 16 * h];
    f32x16 acc = {};
    // smallest terms first: lo, mid, hi
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[sp][j], bv[j], acc, 0, 0, 0);
    if constexpr (kQuant) {
        float m = __builtin_fabsf(acc[0]);
#pragma unroll
        for (int v = 1; v < 16; ++v)
            m = amax_step(m, acc[v]);
        // the other 16 channels of the token sit in lane l^32
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        m = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
        const unsigned b = e8m0_byte(m);
        const float sc = scale_operand(b);
        unsigned w0 = cvt8(acc[0], acc[1], acc[2], acc[3], acc[4], acc[5], acc[6], acc[7], sc);
        unsigned w1 = cvt8(acc[8], acc[9], acc[10], acc[11], acc[12], acc[13], acc[14], acc[15], sc);
        if (b == 0xFFu)
            w0 = w1 = 0u;
        // lane half h holds q bytes 8h..8h+7 of block `wave` of the strip
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        *(u32x2 *)&st.q[par][tl][wave * 16 + 8 * h] = u32x2{w0, w1};
        if (h == 0)
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
// offsets, which the range check drops.  Both stores keep the default cache
// policy, so that the codes are still in the caches when the W4A4 product
// reads them right after: nontemporal code stores made the quantizer alone
// 3-6% faster but quantize-then-product at the DiT qkv shape (8192 x 1152 by
// 3456) 8% slower (41.7 against 38.4 us).
template <int kW>
__device__ __forceinline__ void store_tile(const WgStage<kW> &st, int par, bool valid, int bg, int nB, int d, int wave,
                                           int lane, __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs)
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    constexpr int kLQ = 2 * kW; // lanes per token for the codes
    const int tq = wave * (64 / kLQ) + lane / kLQ;
    const int c8 = lane % kLQ;
    const unsigned drop_q = (unsigned)(bg * kW + (c8 >> 1) >= nB || !valid) << 31;
    const u32x2 v = *(const u32x2 *)&st.q[par][tq][c8 * 8];
    __builtin_amdgcn_raw_buffer_store_b64(v, rq, (int)((unsigned)(tq * (d >> 1) + bg * kW * 16 + c8 * 8) | drop_q), 0,
                                          0);
    const int f = wave * 64 + lane; // flat lane of the workgroup
    const int ts = (f / kW) % kTileT;
    const int cs = f % kW;
    const unsigned drop_s = (unsigned)(bg * kW + cs >= nB || !valid || f >= kTileT * kW) << 31;
    __builtin_amdgcn_raw_buffer_store_b8(st.s[par][ts][cs], rs, (int)((unsigned)(ts * nB + bg * kW + cs) | drop_s), 0,
                                         0);
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
// an empty range and fetch nothing.
#ifndef KQ_RING
#define KQ_RING 4
#endif
constexpr int kRing = KQ_RING; // tiles in flight per wave: kRing - 1 ahead of the one being staged

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

template <bool kQuant, int kW, bool kAd = false>
__global__ __launch_bounds__(64 * kW) __attribute__((amdgpu_waves_per_eu(kAd ? kAdOcc : 4))) void kq_mfma_kernel(
    const uint16_t *__restrict__ x, int64_t M, int d, const float *__restrict__ factors, int per_block,
    uint8_t *__restrict__ q, uint8_t *__restrict__ s, float *__restrict__ y, int nBG, int tiles_per_wg,
    int order, int lu, AdArgs ad)
{
    __shared__ WgStage<kW> st;
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
        store_tile(st, kp & 1, kp >= 0, bg, nB, d, wave, lane, out_buffer(q + r0 * (d >> 1), rows * (d >> 1)),
                   out_buffer(s + r0 * nB, rows * nB));
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
        transform_tile<kQuant, kW>(st, st, kk & 1, A, trow(kk) + tl, M, d, jb, jb_raw < nB, h, wave, tl, y);
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
// launchers
// ---------------------------------------------------------------------------
static int num_cus()
{
    static int n = 0;
    if (!n) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
    }
    return n;
}

// Resident workgroups of an MFMA kernel per XCD (occupancy from the runtime),
// cached per kernel instance.
static int mfma_wgs_per_xcd(const void *fn, int threads)
{
    static const void *keys[4] = {nullptr, nullptr, nullptr, nullptr};
    static int vals[4] = {0, 0, 0, 0};
    for (int i = 0; i < 4; ++i)
        if (keys[i] == fn)
            return vals[i];
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess || per_cu <= 0)
        per_cu = 1;
    int v = per_cu * num_cus() / (int)kXcds;
    if (v < 1)
        v = 1;
    for (int i = 0; i < 4; ++i)
        if (!keys[i]) {
            keys[i] = fn;
            vals[i] = v;
            break;
        }
    return v;
}

template <int kW, bool kAd = false>
static hipError_t launch_kq_mfma_w(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT,
                                   uint8_t *q, uint8_t *s, float *y, int lu, hipStream_t stream, AdArgs ad = {})
{
    const int nB = (int)(d / 32);
    const int nBG = (nB + kW - 1) / kW;
    const int64_t nTiles = (M + kTileT - 1) / kTileT;
    const void *fn;
    if constexpr (kAd)
        fn = (const void *)kq_mfma_kernel<true, kW, true>;
    else
        fn = y ? (const void *)kq_mfma_kernel<false, kW> : (const void *)kq_mfma_kernel<true, kW>;
    const int64_t resident = mfma_wgs_per_xcd(fn, 64 * kW); // per XCD
    int tpw = tuning().mfma_tiles_per_wave > 256 ? 256 : tuning().mfma_tiles_per_wave;
    int interleave = tuning().mfma_interleave == 2 ? 1 : 0;
    bool flat = tuning().mfma_order == 2;
    if (tpw <= 0 && tuning().mfma_order == 0 && tuning().mfma_interleave != 1) {
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
                tpw = (int)t1f;
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
        //    pipeline (measured at 8192 x 1152 on three boxes: 8.3 us against
        //    8.5-9.2).
        int64_t gx = resident / nBG; // token groups per XCD in one round
        if (gx < 1)
            gx = 1;
        const int64_t t1 = (nTiles + gx * kXcds - 1) / (gx * kXcds);
        const int64_t wgs6 = ((nTiles + 5) / 6 + kXcds - 1) / kXcds * kXcds * nBG;
        if (tuning().mfma_interleave != 1 && t1 == 3 && 10 * wgs6 >= 9 * (int64_t)num_cus()) {
            tpw = 6;
            interleave = 0;
        } else if (tuning().mfma_interleave != 1 && t1 >= 3 && t1 <= 12) {
            tpw = (int)t1;
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
        if (tuning().mfma_interleave == 2)
            interleave = 1;
    }
    const int64_t nG = (nTiles + tpw - 1) / tpw;
    // XCD-grouped: token groups dealt to the XCDs in turn, padded to a multiple of 8
    const int64_t nGpad = flat ? nG : (nG + kXcds - 1) / kXcds * kXcds;
    const int64_t grid = nGpad * nBG;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    int di = (int)d;
    int per_block = nT > 1 ? 1 : 0;
    int nbg = nBG;
    int order = (interleave ? 1 : 0) | (flat ? 2 : 0);
    void *args_q[] = {(void *)&x,   (void *)&M,   (void *)&di,  (void *)&factors, (void *)&per_block, (void *)&q,
                      (void *)&s,   (void *)&y,   (void *)&nbg, (void *)&tpw,     (void *)&order,     (void *)&lu,
                      (void *)&ad};
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64 * kW), args_q, 0, stream);
}

hipError_t launch_kq_mfma(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                          uint8_t *s, float *y, int lu, hipStream_t stream)
{
    // Strips of 16 blocks (16 waves, 1 KB of each row per workgroup, 85 KB of
    // LDS, one workgroup per CU) read and write HBM in longer runs than strips
    // of 8, which pays when the whole launch is one resident round of
    // interleaved token groups (measured: 8192 x 4608, 18.3 us against 19.8).
    // Over several rounds the lone workgroup per CU leaves its CU idle
    // between workgroups, and strips of 8 (two per CU) win.  They are used
    // only when they divide the row exactly, so no wave idles.
    const int64_t nB = d / 32;
    int w = tuning().mfma_strip;
    if (w != 8 && w != 16) {
        w = 8;
        if (nB % 16 == 0 && tuning().mfma_tiles_per_wave <= 0 && tuning().mfma_interleave != 1) {
            const void *fn16 = y ? (const void *)kq_mfma_kernel<false, 16> : (const void *)kq_mfma_kernel<true, 16>;
            int64_t gx = mfma_wgs_per_xcd(fn16, 64 * 16) / (nB / 16);
            if (gx < 1)
                gx = 1;
            const int64_t nTiles = (M + kTileT - 1) / kTileT;
            const int64_t t1 = (nTiles + gx * kXcds - 1) / (gx * kXcds);
            if (t1 >= 3 && t1 <= 12)
                w = 16;
        }
    }
    if (w == 16)
        return launch_kq_mfma_w<16>(x, M, d, factors, nT, q, s, y, lu, stream);
    return launch_kq_mfma_w<8>(x, M, d, factors, nT, q, s, y, lu, stream);
}

// Second pass of the AdaLN front-end on the matrix cores: the quantizer's
// launch shape with h in place of x, normalised at staging.
hipError_t launch_adaln_mfma(const uint16_t *h, int64_t M, int64_t d, const double *stats, const float *shift,
                             const float *scale, int64_t T, const float *factors, int64_t nT, uint8_t *q, uint8_t *s,
                             hipStream_t stream)
{
    // The normalisation takes the registers of a lane to about 180 VGPRs (two
    // waves per SIMD), so 16-block strips (1024 threads, at most 128 VGPRs)
    // are not offered.  Strips of 4 blocks when they divide the row and
    // strips of 8 do not (measured at 8192 x 1152: 18.95 against 19.83 us for
    // the whole front-end; strips of 8 were as fast or faster at 2048 x 2240
    // and 4608 x 3072).
    const AdArgs ad{stats, shift, scale, T};
    const int64_t nB = d / 32;
    int w = tuning().adaln_strip;
    if (w != 4 && w != 8)
        w = (nB % 4 == 0 && nB % 8 != 0) ? 4 : 8;
    if (w == 4)
        return launch_kq_mfma_w<4, true>(h, M, d, factors, nT, q, s, nullptr, 0, stream, ad);
    return launch_kq_mfma_w<8, true>(h, M, d, factors, nT, q, s, nullptr, 0, stream, ad);
}

static hipError_t launch_stream(int mode, const void *x, int64_t M, int64_t d, const float *aux, int per_block,
                                uint8_t *q, uint8_t *s, float *y, int rows_knob, hipStream_t stream)
{
    const int nOct = (int)(d / 8);
    const int nCT = (nOct + 63) / 64;
    int R = rows_knob > 256 ? 256 : rows_knob;
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
                               uint8_t *q, uint8_t *s, float *y, hipStream_t stream)
{
    return launch_stream(y ? kBflyT : kBflyQ, x, M, d, factors, nT > 1 ? 1 : 0, q, s, y,
                         tuning().bfly_rows_per_wave, stream);
}

hipError_t launch_kq16(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                       uint8_t *s, float *y, hipStream_t stream)
{
    return launch_stream(y ? kBfly16T : kBfly16Q, x, M, d, factors, nT > 1 ? 1 : 0, q, s, y,
                         tuning().bfly_rows_per_wave, stream);
}

hipError_t launch_sq(const uint16_t *x, int64_t M, int64_t d, const float *scale, uint8_t *q, uint8_t *s,
                     hipStream_t stream)
{
    return launch_stream(kSQ, x, M, d, scale, 0, q, s, nullptr, tuning().stream_rows_per_wave, stream);
}

hipError_t launch_mx_f32(const float *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, hipStream_t stream)
{
    return launch_stream(kMXF32, x, M, d, nullptr, 0, q, s, nullptr, tuning().stream_rows_per_wave, stream);
}

hipError_t launch_fwht(const uint16_t *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, float *y, hipStream_t stream)
{
    return launch_stream(y ? kFwhtT : kFwhtQ, x, M, d, nullptr, 0, q, s, y, tuning().stream_rows_per_wave, stream);
}

} // namespace kq
