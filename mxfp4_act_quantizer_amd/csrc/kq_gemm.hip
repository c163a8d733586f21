// MXFP4 x MXFP4 product (W4A4) on the gfx950 block-scaled matrix cores:
// out[M, N] = A[M, K] . B[N, K]^T, where A and B are MXFP4 matrices in the
// quantizer's layout (codes [rows, K/2], element 2i in the low nibble; E8M0
// scales [rows, K/32]).  This is the consumer the quantized activations feed
// (abstract of the KroQuant paper page on mlsanity.com: W4A4 MXFP4 with the
// inverse transform folded into the weights).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1: lane l holds,
// for row l % 32 of its 32-row operand and k-block l / 32 of the 64-wide k
// step, one whole 32-element MX block (16 code bytes) and that block's scale
// byte - exactly one block of q and one byte of s.  The scale operand is a
// 32-bit register whose byte the instruction's op_sel picks.  The
// accumulator holds D[row 8(v/4) + 4(l/32) + v%4][column l % 32] in element
// v of lane l.
//
// Two kernels share that operand handling, both with 128 x 128 output tiles
// per workgroup of 4 waves (64 x 64 per wave as 2 x 2 MFMA tiles) and two
// workgroups per CU, and both send the finished tile back through LDS so
// that every store instruction writes whole 256-byte (bf16) or 512-byte
// (f32) row segments:
//  - mx_gemm_persistent (K % 128 == 0, whole 16-byte output pieces): one
//    resident round of workgroups, each streaming the k chunks of all its
//    tiles through a ring of LDS stages filled by LDS-DMA loads;
//  - mx_gemm_kernel (every other shape): one workgroup per tile, chunks of
//    256 going global -> registers (two chunks ahead) -> LDS (double
//    buffered) -> fragments.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_internal.h"

namespace kq {
namespace {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr unsigned kBufWord3G = 0x00020000; // raw buffer, 32-bit dwords
constexpr int kWM = 2, kWN = 2;              // waves along M and N
constexpr int kTX = 2, kTY = 2;              // 32 x 32 MFMA tiles per wave along M and N
constexpr int kBM = kWM * kTX * 32;          // workgroup tile: 128 x 128
constexpr int kBN = kWN * kTY * 32;
constexpr int kThreads = 64 * kWM * kWN;     // 4 waves
constexpr int kKC = 256;                     // k per LDS chunk
constexpr int kSteps = kKC / 64;             // 64-wide MFMA steps per chunk
constexpr int kPR = kKC / 32;                // 16-byte code pieces (= MX blocks) per row and chunk
constexpr int kRowB = kKC / 2 + 16;          // padded LDS row of code bytes (below)
constexpr int kPA = kBM * kPR / kThreads;    // code pieces of A per lane and chunk
constexpr int kPB = kBN * kPR / kThreads;
constexpr unsigned kGemmXcds = 8;

// Rows are padded by 16 bytes: the same 16-byte piece of 16 consecutive rows
// (one fragment read) then starts 4 dwords apart modulo 64 banks, so the 16
// lanes served together hit every bank once.
//
// Scales: a row's 8 scale bytes of a chunk (block j = byte j) are kept as two
// words, the even blocks {0, 2, 4, 6} and the odd blocks {1, 3, 5, 7}.  Lane
// (i, h) uses block 2u + h in step u, i.e. byte u of word h: one word read per
// chunk, and op_sel picks the byte in each step.
struct __align__(16) GemmStage {
    unsigned char a[2][kBM][kRowB];
    unsigned char b[2][kBN][kRowB];
    unsigned sa[2][kBM][2];
    unsigned sb[2][kBN][2];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, kBufWord3G);
}

// Raw loads of one chunk for one lane: kPA 16-byte code pieces of A and kPB
// of B (rows t / kPR + (kThreads / kPR) u, piece t % kPR of the row's chunk),
// and the chunk's 8 scale bytes of one row (A rows for the first kBM lanes, B
// rows for the next kBN).  Nothing here reads a loaded register: the loads
// stay in flight until stage_chunk, which runs after the products of an
// earlier chunk (a use right after the load would make the wave wait for
// every load of the chunk there).
struct ChunkIn {
    u32x4 a[kPA], b[kPB];
    unsigned s[8]; // scales: two dwords (whole-dword rows) or one byte per register
};

// kSAligned: K % 128 == 0, so row starts and chunk offsets in the scale
// matrix are dword aligned.  Offsets past the k range (k >= K) or the tile's
// rows fall outside the ranges or carry bit 31: the hardware returns zeros.
// A zero code is +0 and contributes nothing whatever its scale.
template <bool kSAligned>
__device__ __forceinline__ void load_chunk(ChunkIn &in, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                           __amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb, int K, int kc,
                                           int t, int wave)
{
    const int kbyte = kc / 2 + (t % kPR) * 16; // byte within the row
    const unsigned dropk = (unsigned)(kbyte >= K / 2) << 31;
#pragma unroll
    for (int u = 0; u < kPA; ++u) {
        const int row = t / kPR + (kThreads / kPR) * u;
        const unsigned off = (unsigned)(row * (K / 2) + kbyte) | dropk;
        in.a[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < kPB; ++u) {
        const int row = t / kPR + (kThreads / kPR) * u;
        const unsigned off = (unsigned)(row * (K / 2) + kbyte) | dropk;
        in.b[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)off, 0, 0));
    }
    // the first kBM lanes take A's scale rows, the next kBN lanes B's (whole
    // waves, so the descriptor choice is uniform and stays scalar)
    static_assert(kBM % 64 == 0 && kBN % 64 == 0 && kBM + kBN <= kThreads, "scale rows per wave");
    const bool on_a = wave < kBM / 64;
    const __amdgpu_buffer_rsrc_t rs = on_a ? rsa : rsb;
    const int row = on_a ? t : t - kBM;
    const int left = K / 32 - kc / 32; // scale bytes of this row still inside K (> 0)
    const unsigned base = (unsigned)(row * (K / 32) + kc / 32);
    if constexpr (kSAligned) {
        // bytes past K are read here (the next row's) and cleared at staging
        in.s[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)base, 0, 0);
        in.s[1] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(base + 4), 0, 0);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const unsigned drop = (unsigned)(j >= left) << 31;
            in.s[j] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)((base + j) | drop), 0, 0);
        }
    }
}

template <bool kSAligned>
__device__ __forceinline__ void stage_chunk(GemmStage &st, int par, const ChunkIn &in, int t, int wave, int K,
                                            int kc)
{
#pragma unroll
    for (int u = 0; u < kPA; ++u)
        *(u32x4 *)&st.a[par][t / kPR + (kThreads / kPR) * u][(t % kPR) * 16] = in.a[u];
#pragma unroll
    for (int u = 0; u < kPB; ++u)
        *(u32x4 *)&st.b[par][t / kPR + (kThreads / kPR) * u][(t % kPR) * 16] = in.b[u];
    unsigned lo, hi; // scale bytes 0-3 and 4-7 of the chunk
    if constexpr (kSAligned) {
        lo = in.s[0];
        hi = in.s[1];
    } else {
        lo = (in.s[0] & 0xFF) | (in.s[1] & 0xFF) << 8 | (in.s[2] & 0xFF) << 16 | in.s[3] << 24;
        hi = (in.s[4] & 0xFF) | (in.s[5] & 0xFF) << 8 | (in.s[6] & 0xFF) << 16 | in.s[7] << 24;
    }
    // bytes past K belong to the next row: clear them (scale 2^-127 times +0 codes)
    const int left = K / 32 - kc / 32;
    if (left < 8) {
        const unsigned long long keep = (1ull << (8 * left)) - 1;
        lo &= (unsigned)keep;
        hi &= (unsigned)(keep >> 32);
    }
    // even blocks {0, 2, 4, 6} and odd blocks {1, 3, 5, 7}
    const u32x2 eo = {__builtin_amdgcn_perm(hi, lo, 0x06040200u), __builtin_amdgcn_perm(hi, lo, 0x07050301u)};
    if (wave < kBM / 64)
        *(u32x2 *)st.sa[par][t] = eo;
    else if (wave < (kBM + kBN) / 64)
        *(u32x2 *)st.sb[par][t - kBM] = eo;
}

__device__ __forceinline__ i32x8 widen(const u32x4 v)
{
    return i32x8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
}

// Step U of a chunk for one wave: lane (i, h) takes k-block 2U + h, whose
// scale is byte U of the lane's scale words.  D = B . A^T: for n tile y and
// m tile x, lane l holds out[m = 32x + l%32][n = 32y + 8(v/4) + 4(l/32) + v%4]
// in element v, so each lane owns runs of four consecutive output columns.
template <int U>
__device__ __forceinline__ void step_mfma(f32x16 (&acc)[kTY][kTX], const GemmStage &st, int par, int wm, int wn,
                                          int i, int h, const unsigned (&sca)[kTX], const unsigned (&scb)[kTY])
{
    u32x4 fa[kTX], fb[kTY]; // the FP4 form of the instruction reads 4 of its 8 operand registers
#pragma unroll
    for (int x = 0; x < kTX; ++x)
        fa[x] = *(const u32x4 *)&st.a[par][32 * kTX * wm + 32 * x + i][16 * (2 * U + h)];
#pragma unroll
    for (int y = 0; y < kTY; ++y)
        fb[y] = *(const u32x4 *)&st.b[par][32 * kTY * wn + 32 * y + i][16 * (2 * U + h)];
#pragma unroll
    for (int y = 0; y < kTY; ++y)
#pragma unroll
        for (int x = 0; x < kTX; ++x)
            acc[y][x] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(fb[y]), widen(fa[x]), acc[y][x], 4, 4,
                                                                        U, (int)scb[y], U, (int)sca[x]);
}

// One chunk's products for one wave (kSteps = 4 steps).
__device__ __forceinline__ void compute_chunk(f32x16 (&acc)[kTY][kTX], const GemmStage &st, int par, int wm, int wn,
                                              int i, int h)
{
    static_assert(kSteps == 4, "one step call per 64-wide k step");
    unsigned sca[kTX], scb[kTY];
#pragma unroll
    for (int x = 0; x < kTX; ++x)
        sca[x] = st.sa[par][32 * kTX * wm + 32 * x + i][h];
#pragma unroll
    for (int y = 0; y < kTY; ++y)
        scb[y] = st.sb[par][32 * kTY * wn + 32 * y + i][h];
    step_mfma<0>(acc, st, par, wm, wn, i, h, sca, scb);
    step_mfma<1>(acc, st, par, wm, wn, i, h, sca, scb);
    step_mfma<2>(acc, st, par, wm, wn, i, h, sca, scb);
    step_mfma<3>(acc, st, par, wm, wn, i, h, sca, scb);
}

// One workgroup: a kBM x kBN tile of out; wave w computes rows
// 32 kTX (w / kWN) .. and columns 32 kTY (w % kWN) .. as kTX x kTY MFMA tiles.
// The LDS use (78 KB) allows two workgroups per CU; the register budget is
// set to match (256 per lane).
template <bool kBf16, bool kSAligned>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
mx_gemm_kernel(const uint8_t *__restrict__ qa, const uint8_t *__restrict__ sa, int64_t M,
               const uint8_t *__restrict__ qb, const uint8_t *__restrict__ sb, int64_t N, int K,
               void *__restrict__ out, int tilesN, int vec_out)
{
    __shared__ GemmStage st;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    // tiles dealt so that each XCD (blockIdx % 8) walks a contiguous range of
    // tiles, n fastest: consecutive workgroups of an XCD share their A rows in
    // L2 (the grid is a multiple of 8, so every (XCD, slot) pair exists)
    const unsigned per_xcd = gridDim.x / kGemmXcds;
    const unsigned tile = (blockIdx.x % kGemmXcds) * per_xcd + blockIdx.x / kGemmXcds;
    if (tile >= (unsigned)(((M + kBM - 1) / kBM) * tilesN))
        return; // uniform, before any barrier
    const int64_t m0 = (int64_t)(tile / (unsigned)tilesN) * kBM;
    const int64_t n0 = (int64_t)(tile % (unsigned)tilesN) * kBN;
    const int64_t rowsA = (M - m0) < kBM ? (M - m0) : kBM;
    const int64_t rowsB = (N - n0) < kBN ? (N - n0) : kBN;
    const __amdgpu_buffer_rsrc_t ra = rsrc(qa + m0 * (K / 2), rowsA * (K / 2));
    const __amdgpu_buffer_rsrc_t rb = rsrc(qb + n0 * (K / 2), rowsB * (K / 2));
    const __amdgpu_buffer_rsrc_t rsa = rsrc(sa + m0 * (K / 32), rowsA * (K / 32));
    const __amdgpu_buffer_rsrc_t rsb = rsrc(sb + n0 * (K / 32), rowsB * (K / 32));

    const int wm = wave / kWN, wn = wave % kWN;
    const int i = lane & 31, h = lane >> 5;
    f32x16 acc[kTY][kTX];
#pragma unroll
    for (int y = 0; y < kTY; ++y)
#pragma unroll
        for (int x = 0; x < kTX; ++x)
            acc[y][x] = f32x16{};

    // A last partial chunk runs all its steps: its codes past K were loaded as
    // zeros and its scales past K cleared, so they add exact zeros.
    const int nChunks = (K + kKC - 1) / kKC;
    if constexpr (!kSAligned) {
        // byte-wise scales: one chunk ahead (eight scale registers per chunk)
        ChunkIn in;
        load_chunk<false>(in, ra, rb, rsa, rsb, K, 0, t, wave);
        stage_chunk<false>(st, 0, in, t, wave, K, 0);
        __syncthreads();
        for (int c = 0; c < nChunks; ++c) {
            if (c + 1 < nChunks)
                load_chunk<false>(in, ra, rb, rsa, rsb, K, (c + 1) * kKC, t, wave);
            compute_chunk(acc, st, c & 1, wm, wn, i, h);
            // the other buffer was last read in the previous chunk, before the
            // previous barrier: stage into it, then one barrier before it is read
            if (c + 1 < nChunks) {
                stage_chunk<false>(st, (c & 1) ^ 1, in, t, wave, K, (c + 1) * kKC);
                __syncthreads();
            }
        }
    } else {
        // Two chunks in flight in registers ahead of the one in LDS: the loads
        // of chunk c + 2 are issued before chunk c is multiplied, so each load
        // has two chunks of products to arrive.  Chunk j lives in register set
        // j % 2; the loop is unrolled by two so that both sets are named
        // statically and stay in registers.
        ChunkIn in0, in1;
        load_chunk<true>(in0, ra, rb, rsa, rsb, K, 0, t, wave);
        if (nChunks > 1)
            load_chunk<true>(in1, ra, rb, rsa, rsb, K, kKC, t, wave);
        stage_chunk<true>(st, 0, in0, t, wave, K, 0);
        __syncthreads();
        auto chunk = [&](int c, ChunkIn &mine, ChunkIn &next) {
            if (c + 2 < nChunks)
                load_chunk<true>(mine, ra, rb, rsa, rsb, K, (c + 2) * kKC, t, wave);
            compute_chunk(acc, st, c & 1, wm, wn, i, h);
            if (c + 1 < nChunks) {
                stage_chunk<true>(st, (c & 1) ^ 1, next, t, wave, K, (c + 1) * kKC);
                __syncthreads();
            }
        };
        for (int c = 0; c < nChunks; c += 2) {
            chunk(c, in0, in1);
            if (c + 1 < nChunks)
                chunk(c + 1, in1, in0);
        }
    }

    // Epilogue through LDS: the tile is written into the (now idle) staging
    // memory in the MFMA layout, then read back by rows so that each store
    // instruction writes whole row segments of kBN columns.
    constexpr int kES = kBf16 ? 2 : 4;
    constexpr int kOP = kBf16 ? kBN * 2 + 8 : kBN * 4 + 16; // padded row pitch in bytes
    static_assert(kBM * kOP <= (int)sizeof(GemmStage), "output tile fits the staging memory");
    unsigned char *ot = (unsigned char *)&st;
    __syncthreads(); // every wave is done with the last chunk in LDS
#pragma unroll
    for (int y = 0; y < kTY; ++y)
#pragma unroll
        for (int x = 0; x < kTX; ++x) {
            const int row = 32 * kTX * wm + 32 * x + i;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * kTY * wn + 32 * y + 8 * g + 4 * h;
                const f32x16 &a = acc[y][x];
                if constexpr (kBf16) {
                    const unsigned lo = (unsigned)__builtin_bit_cast(unsigned short, (__bf16)a[4 * g]) |
                                        ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)a[4 * g + 1]) << 16);
                    const unsigned hi = (unsigned)__builtin_bit_cast(unsigned short, (__bf16)a[4 * g + 2]) |
                                        ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)a[4 * g + 3]) << 16);
                    *(u32x2 *)(ot + row * kOP + col * 2) = u32x2{lo, hi};
                } else {
                    *(u32x4 *)(ot + row * kOP + col * 4) = u32x4{__float_as_uint(a[4 * g]), __float_as_uint(a[4 * g + 1]),
                                                                 __float_as_uint(a[4 * g + 2]),
                                                                 __float_as_uint(a[4 * g + 3])};
                }
            }
        }
    __syncthreads();
    // kLR lanes cover one row (16 bytes each); rows past rowsA fall outside the
    // range and columns past N are dropped
    constexpr int kLR = kBN * kES / 16;
    constexpr int kRP = kThreads / kLR; // rows per pass
    constexpr int kEL = 16 / kES;       // elements per lane
    const __amdgpu_buffer_rsrc_t ro = rsrc((unsigned char *)out + m0 * N * kES, rowsA * N * kES);
    const int c16 = t % kLR;
    const int64_t col = n0 + c16 * kEL;
#pragma unroll 4
    for (int r = t / kLR; r < kBM; r += kRP) {
        const u32x4 v = *(const u32x4 *)(ot + r * kOP + c16 * 16);
        if (vec_out) {
            // 16-byte aligned output and N % kEL == 0: whole 16-byte pieces
            const unsigned drop = (unsigned)(col >= N) << 31;
            __builtin_amdgcn_raw_buffer_store_b128(v, ro, (int)((unsigned)((r * N + col) * kES) | drop), 0, 0);
        } else {
#pragma unroll
            for (int e = 0; e < kEL; ++e) {
                const unsigned drop = (unsigned)(col + e >= N) << 31;
                const unsigned off = (unsigned)((r * N + col + e) * kES) | drop;
                if constexpr (kBf16)
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(v[e / 2] >> (16 * (e & 1))), ro, (int)off,
                                                          0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(v[e], ro, (int)off, 0, 0);
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Persistent form, used when K % 128 == 0 and the output rows split into
// whole 16-byte pieces (every layer of the transformer shapes): each
// workgroup owns a fixed list of tiles and runs one continuous stream of k
// chunks over all of them, so the loads of the next tile are in flight while
// the last chunk of this one is multiplied and stored.  Codes and scales go straight from global memory into LDS
// (buffer_load ... lds, 16 or 4 bytes per lane) through a ring of kS stages;
// no register staging.
//
// LDS layout of a stage: the code rows of A (BM of them) then of B (BN), RB =
// KC/2 bytes each, then the scale rows of A and B (SB = KC/32 bytes each).
// One 64-lane load writes 1 KB of consecutive LDS, so the conflict-avoiding
// permutation is applied to what each lane fetches: slot s of row r holds the
// row's 16-byte piece s ^ rot(r), rot(r) = (r / (16 / PR)) % PR with PR
// pieces per row.  A fragment read (16 lanes = 16 consecutive rows, one piece)
// then covers all 64 banks once.
// ---------------------------------------------------------------------------
template <int kWM_, int kWN_, int kTX_, int kTY_, int kKC_, int kS_>
struct PGeom {
    static constexpr int WM = kWM_, WN = kWN_, TX = kTX_, TY = kTY_, KC = kKC_, S = kS_;
    static constexpr int W = WM * WN, T = 64 * W;
    static constexpr int BM = WM * TX * 32, BN = WN * TY * 32;
    static constexpr int STEPS = KC / 64;
    static constexpr int PR = KC / 32;       // 16-byte pieces (MX blocks) per row and chunk
    static constexpr int RB = KC / 2;        // code bytes per row and chunk
    static constexpr int RPI = 1024 / RB;    // rows per code load (64 lanes x 16 bytes)
    static constexpr int SB = KC / 32;       // scale bytes per row and chunk
    static constexpr int SRPI = 256 / SB;    // rows per scale load (64 lanes x 4 bytes)
    static constexpr int NCI = (BM + BN) / RPI, NSI = (BM + BN) / SRPI;
    // scale loads padded to a whole number per wave: the extra ones fetch
    // nothing and land in slack at the end of the stage
    static constexpr int NSP = (NSI + W - 1) / W * W;
    static constexpr int LC = NCI / W, LS = NSP / W, L = LC + LS; // loads per wave and chunk
    static constexpr int SOFF = (BM + BN) * RB;                  // scale rows within a stage
    static constexpr int SZ = SOFF + NSP * 256;                   // bytes per stage
    static constexpr int ROWS256 = 16 / PR;                      // rows per 256 bytes of LDS
    // workgroups per CU that the 160 KB of LDS hold, and the waves per SIMD
    // that gives (the register budget is set to match)
    static constexpr int WGS = (160 * 1024) / (S * SZ) < 1 ? 1 : (160 * 1024) / (S * SZ);
    static constexpr int OCC = WGS * W / 4 < 1 ? 1 : (WGS * W / 4 > 8 ? 8 : WGS * W / 4);
    static_assert(KC == 128 || KC == 256, "chunk of 2 or 4 MFMA steps");
    static_assert(NCI % W == 0, "the code loads split evenly over the waves");
    static_assert(BM % RPI == 0 && BM % SRPI == 0, "no load straddles A and B");
    static_assert(S >= 2 && S <= 4, "ring of 2 to 4 stages");
};

// A chunk's scale words for one wave: byte u of the word of lane half h is the
// scale of block 2u + h of the lane's row.
template <class G>
__device__ __forceinline__ void p_scales(unsigned (&sca)[G::TX], unsigned (&scb)[G::TY], const unsigned char *stg,
                                         unsigned sa_off, unsigned sb_off, unsigned scale_sel)
{
#pragma unroll
    for (int x = 0; x < G::TX; ++x) {
        if constexpr (G::SB == 8) {
            const u32x2 w = *(const u32x2 *)(stg + sa_off + x * 32 * 8);
            sca[x] = __builtin_amdgcn_perm(w[1], w[0], scale_sel);
        } else {
            const unsigned w = *(const unsigned *)(stg + sa_off + x * 32 * 4);
            sca[x] = __builtin_amdgcn_perm(w, w, scale_sel);
        }
    }
#pragma unroll
    for (int y = 0; y < G::TY; ++y) {
        if constexpr (G::SB == 8) {
            const u32x2 w = *(const u32x2 *)(stg + sb_off + y * 32 * 8);
            scb[y] = __builtin_amdgcn_perm(w[1], w[0], scale_sel);
        } else {
            const unsigned w = *(const unsigned *)(stg + sb_off + y * 32 * 4);
            scb[y] = __builtin_amdgcn_perm(w, w, scale_sel);
        }
    }
}

// Steps kU0 .. kU1 - 1 of one chunk's products for one wave from a stage (the
// last chunk of a tile whose k range ends half way runs steps 0 and 1 only).
template <class G, int kU0, int kU1>
__device__ __forceinline__ void p_compute(f32x16 (&acc)[G::TY][G::TX], const unsigned char *stg,
                                          const unsigned (&fa_off)[G::STEPS], const unsigned (&fb_off)[G::STEPS],
                                          const unsigned (&sca)[G::TX], const unsigned (&scb)[G::TY])
{
#define KQ_PSTEP(U)                                                                                                  \
    if constexpr (U >= kU0 && U < kU1) {                                                                                         \
        u32x4 fa[G::TX], fb[G::TY];                                                                                  \
        _Pragma("unroll") for (int x = 0; x < G::TX; ++x) fa[x] =                                                    \
            *(const u32x4 *)(stg + fa_off[U] + x * 32 * G::RB);                                                      \
        _Pragma("unroll") for (int y = 0; y < G::TY; ++y) fb[y] =                                                    \
            *(const u32x4 *)(stg + fb_off[U] + y * 32 * G::RB);                                                      \
        _Pragma("unroll") for (int y = 0; y < G::TY; ++y) _Pragma("unroll") for (int x = 0; x < G::TX; ++x)         \
            acc[y][x] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(fb[y]), widen(fa[x]), acc[y][x], 4, 4, \
                                                                        U, (int)scb[y], U, (int)sca[x]);             \
    }
    KQ_PSTEP(0)
    KQ_PSTEP(1)
    KQ_PSTEP(2)
    KQ_PSTEP(3)
#undef KQ_PSTEP
}

constexpr int slab_rows(int bm, int fit)
{
    int r = 32;
    while (r * 2 <= bm && r * 2 <= fit && bm % (r * 2) == 0)
        r *= 2;
    return r;
}

// LDS stores of the epilogue, written as instructions: the compiler cannot
// tell them apart from the loads still filling other stages and would wait
// for all of those first.  A store has no output register; the barrier that
// follows is preceded by an explicit lgkmcnt(0) wait.
__device__ __forceinline__ void lds_store_b64(unsigned char *p, u32x2 v)
{
    const unsigned a = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)p;
    asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store_b128(unsigned char *p, u32x4 v)
{
    const unsigned a = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)p;
    asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}

template <class G, bool kBf16>
__global__ __launch_bounds__(G::T) __attribute__((amdgpu_waves_per_eu(G::OCC, G::OCC))) void mx_gemm_persistent(const uint8_t *__restrict__ qa,
                                                           const uint8_t *__restrict__ sa, int64_t M,
                                                           const uint8_t *__restrict__ qb,
                                                           const uint8_t *__restrict__ sb, int64_t N, int K,
                                                           void *__restrict__ out, int tilesN, int tiles)
{
    __shared__ __align__(16) unsigned char lds0[G::SZ];
    __shared__ __align__(16) unsigned char lds1[G::SZ];
    __shared__ __align__(16) unsigned char lds2[G::S > 2 ? G::SZ : 16];
    __shared__ __align__(16) unsigned char lds3[G::S > 3 ? G::SZ : 16];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);

    // tiles of this workgroup: XCD x = blockIdx % 8 owns the contiguous range
    // [x T / 8, (x + 1) T / 8) of tiles (n fastest), and its g = grid / 8
    // workgroups take every g-th tile of it, so the tiles in flight on one
    // XCD at any time are neighbours sharing A rows in its L2
    const unsigned g8 = gridDim.x / kGemmXcds;
    const unsigned xcd = blockIdx.x % kGemmXcds, slot = blockIdx.x / kGemmXcds;
    const unsigned lo = (unsigned)(((uint64_t)tiles * xcd) / kGemmXcds);
    const unsigned hi = (unsigned)(((uint64_t)tiles * (xcd + 1)) / kGemmXcds);
    if (lo + slot >= hi)
        return; // uniform, before any barrier
    const int mine = (int)((hi - lo - slot + g8 - 1) / g8);
    const int nC = (K + G::KC - 1) / G::KC;
    const bool half_last = (K % G::KC) != 0; // K % 128 == 0: the last chunk has 2 of 4 steps
    const int total = mine * nC;
    const int Kh = K / 2, Ks = K / 32;

    // per-lane load offsets within a tile (the chunk offset is added per load)
    unsigned voff[G::L];
#pragma unroll
    for (int u = 0; u < G::LC; ++u) {
        const int f = wave + G::W * u; // code load index within the stage
        const int row = f * G::RPI + lane / G::PR; // stage row: A rows, then B rows
        const int rot = (row / G::ROWS256) % G::PR;
        const int mrow = row < G::BM ? row : row - G::BM;
        voff[u] = (unsigned)(mrow * Kh + (((lane % G::PR) ^ rot) << 4));
    }
#pragma unroll
    for (int u = 0; u < G::LS; ++u) {
        const int f = wave + G::W * u;
        const int row = f * G::SRPI + (G::SB == 8 ? lane / 2 : lane);
        const int mrow = row < G::BM ? row : row - G::BM;
        // a padding load (f >= NSI) carries bit 31: outside every range
        voff[G::LC + u] = f < G::NSI ? (unsigned)(mrow * Ks + (G::SB == 8 ? (lane & 1) * 4 : 0)) : 0x80000000u;
    }

    // fragment and scale read offsets within a stage
    const int wm = wave / G::WN, wn = wave % G::WN;
    const int i = lane & 31, h = lane >> 5;
    const int rot_i = (i / G::ROWS256) % G::PR;
    unsigned fa_off[G::STEPS], fb_off[G::STEPS];
#pragma unroll
    for (int u = 0; u < G::STEPS; ++u) {
        const unsigned p = (unsigned)(((2 * u + h) ^ rot_i) << 4);
        fa_off[u] = (unsigned)((32 * G::TX * wm + i) * G::RB) + p;
        fb_off[u] = (unsigned)((G::BM + 32 * G::TY * wn + i) * G::RB) + p;
    }
    const unsigned sa_off = (unsigned)(G::SOFF + (32 * G::TX * wm + i) * G::SB);
    const unsigned sb_off = (unsigned)(G::SOFF + (G::BM + 32 * G::TY * wn + i) * G::SB);
    // scale word for lane half h: byte u = the scale of block 2u + h
    const unsigned scale_sel = G::SB == 8 ? (h ? 0x07050301u : 0x06040200u) : (h ? 0x03010301u : 0x02000200u);

    // load cursor: chunk dq of the stream is chunk dkc of tile dtile.  The
    // cursors advance without branches and the descriptors are rebuilt from
    // the tile every chunk (a few scalar operations): state written on one
    // side of a branch only was merged by the compiler into a store through a
    // selected address, which kept it out of registers.
    int dq = 0, dkc = 0;
    unsigned dtile = lo + slot;
    // Loads of the next chunk of the stream into stage `stg`; past the end of
    // the stream the same loads go out with bit 31 set in the offset (outside
    // every range: nothing is fetched), so every wave always has the same
    // number of loads in flight and the wait below stays a constant.
    auto load_next = [&](unsigned char *stg) {
        const int64_t m0 = (int64_t)(dtile / (unsigned)tilesN) * G::BM;
        const int64_t n0 = (int64_t)(dtile % (unsigned)tilesN) * G::BN;
        const int64_t ra = (M - m0) < G::BM ? (M - m0) : G::BM;
        const int64_t rb = (N - n0) < G::BN ? (N - n0) : G::BN;
        const bool live = dq < total;
        const __amdgpu_buffer_rsrc_t rca = rsrc(qa + m0 * Kh, live ? ra * Kh : 0);
        const __amdgpu_buffer_rsrc_t rcb = rsrc(qb + n0 * Kh, live ? rb * Kh : 0);
        const __amdgpu_buffer_rsrc_t rsa = rsrc(sa + m0 * Ks, live ? ra * Ks : 0);
        const __amdgpu_buffer_rsrc_t rsb = rsrc(sb + n0 * Ks, live ? rb * Ks : 0);
        const unsigned addc = live ? (unsigned)(dkc * G::RB) : 0x80000000u;
        const unsigned adds = live ? (unsigned)(dkc * G::SB) : 0x80000000u;
#pragma unroll
        for (int u = 0; u < G::LC; ++u) {
            const int f = wave + G::W * u;
            const bool on_a = f * G::RPI < G::BM;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(on_a ? rca : rcb,
                                                     (__attribute__((address_space(3))) void *)(stg + f * 1024), 16,
                                                     (int)(voff[u] + addc), 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < G::LS; ++u) {
            const int f = wave + G::W * u;
            const bool on_a = f * G::SRPI < G::BM;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                on_a ? rsa : rsb, (__attribute__((address_space(3))) void *)(stg + G::SOFF + f * 256), 4,
                (int)(voff[G::LC + u] + adds), 0, 0, 0);
        }
        ++dq;
        const bool wrap = dkc == nC - 1;
        dkc = wrap ? 0 : dkc + 1;
        dtile += wrap ? g8 : 0u;
    };

    f32x16 acc[G::TY][G::TX];
#pragma unroll
    for (int y = 0; y < G::TY; ++y)
#pragma unroll
        for (int x = 0; x < G::TX; ++x)
            acc[y][x] = f32x16{};

    // store cursor: tile ctile is finished after chunk nC - 1 of it
    int ckc = 0;
    unsigned ctile = lo + slot;
    // Epilogue through LDS, in the stage just multiplied: the tile goes in
    // row slabs (all of it for bf16; two halves for f32 when a stage is
    // smaller than the tile) into the stage in the accumulator layout, and
    // leaves by rows, 16 bytes per lane and whole row segments per store
    // instruction.  The next chunk's loads target other stages, so they stay
    // in flight meanwhile; the stage itself is next filled after the barrier
    // that opens the next step.
    constexpr int kES = kBf16 ? 2 : 4;
    constexpr int kOP = kBf16 ? G::BN * 2 + 8 : G::BN * 4 + 16; // padded row pitch in bytes
    // rows per slab: the largest power-of-two multiple of 32 dividing BM whose
    // rows fit a stage
    constexpr int kSR = slab_rows(G::BM, G::SZ / kOP);
    static_assert(kSR >= 32 && G::BM % kSR == 0, "slabs of whole 32-row blocks");
    constexpr int kLR = G::BN * kES / 16; // lanes per output row
    constexpr int kRP = G::T / kLR;       // rows per pass
    constexpr int kEL = 16 / kES;         // elements per lane
    static_assert(G::T % kLR == 0 && kSR % kRP == 0, "whole rows per pass");
    constexpr unsigned kLgkm0 = 0xC07Fu;  // s_waitcnt lgkmcnt(0) alone
    auto store_tile = [&](unsigned char *stg) {
        const int64_t m0 = (int64_t)(ctile / (unsigned)tilesN) * G::BM;
        const int64_t n0 = (int64_t)(ctile % (unsigned)tilesN) * G::BN;
        const int64_t rows = (M - m0) < G::BM ? (M - m0) : G::BM;
        const __amdgpu_buffer_rsrc_t ro = rsrc((unsigned char *)out + m0 * N * kES, rows * N * kES);
        const int c16 = t % kLR;
        const int64_t col = n0 + c16 * kEL;
        const unsigned drop = (unsigned)(col >= N) << 31;
#pragma unroll
        for (int r0 = 0; r0 < G::BM; r0 += kSR) {
            // every wave is done reading the stage (products, or the slab before)
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int y = 0; y < G::TY; ++y)
#pragma unroll
                for (int x = 0; x < G::TX; ++x) {
                    const int rb = 32 * G::TX * wm + 32 * x; // uniform: the 32-row block is in or out
                    if (rb < r0 || rb >= r0 + kSR)
                        continue;
                    const int row = rb - r0 + i;
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int c = 32 * G::TY * wn + 32 * y + 8 * gq + 4 * h;
                        const f32x16 &a = acc[y][x];
                        if constexpr (kBf16) {
                            const unsigned w0 =
                                (unsigned)__builtin_bit_cast(unsigned short, (__bf16)a[4 * gq]) |
                                ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)a[4 * gq + 1]) << 16);
                            const unsigned w1 =
                                (unsigned)__builtin_bit_cast(unsigned short, (__bf16)a[4 * gq + 2]) |
                                ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)a[4 * gq + 3]) << 16);
                            lds_store_b64(stg + row * kOP + c * 2, u32x2{w0, w1});
                        } else {
                            lds_store_b128(stg + row * kOP + c * 4,
                                           u32x4{__float_as_uint(a[4 * gq]), __float_as_uint(a[4 * gq + 1]),
                                                 __float_as_uint(a[4 * gq + 2]), __float_as_uint(a[4 * gq + 3])});
                        }
                    }
                }
            __builtin_amdgcn_s_waitcnt(kLgkm0);
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int pss = 0; pss < kSR / kRP; ++pss) {
                const int rr = t / kLR + pss * kRP;
                const u32x4 v = *(const u32x4 *)(stg + rr * kOP + c16 * 16);
                __builtin_amdgcn_raw_buffer_store_b128(v, ro, (int)((unsigned)(((r0 + rr) * N + col) * kES) | drop),
                                                       0, 0);
            }
        }
#pragma unroll
        for (int y = 0; y < G::TY; ++y)
#pragma unroll
            for (int x = 0; x < G::TX; ++x)
                acc[y][x] = f32x16{};
    };

    // prologue: chunks 0 .. S-2 in flight
    load_next(lds0);
    if constexpr (G::S > 2)
        load_next(lds1);
    if constexpr (G::S > 3)
        load_next(lds2);

    // One step of the stream: wait for this wave's loads of chunk q (the
    // S - 2 later chunks may stay in flight; stores issued since only make
    // the wait longer), barrier (every wave's loads of chunk q have landed,
    // and every wave is done with chunk q - 1, whose stage takes chunk
    // q + S - 1), then multiply.  The stream is padded to a multiple of S
    // chunks so that every unrolled step runs unconditionally and names its
    // stage statically (the compiler then tracks which load filled which
    // stage); a padding step multiplies stale data into accumulators that are
    // never stored.
    constexpr int kWait = (G::S - 2) * G::L;
    static_assert(kWait < 64, "vmcnt field");
    constexpr unsigned kWaitImm = 0x0F70u | (kWait & 15) | ((kWait >> 4) << 14);
    int qq = 0;
    auto step = [&](unsigned char *cur, unsigned char *nxt) {
        // A plain s_barrier: __syncthreads() adds a workgroup release fence,
        // which counts the loads still filling later stages as pending LDS
        // writes and waits for all of them.  What the fence would order is
        // ordered here already: this wave's loads of chunk q by the wait, its
        // LDS reads of chunk q - 1 by their use in the products before it,
        // and the empty asm keeps the compiler from moving LDS accesses
        // across the barrier.
        __builtin_amdgcn_s_waitcnt(kWaitImm);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        load_next(nxt);
        const bool last = ckc == nC - 1;
        unsigned sca[G::TX], scb[G::TY];
        p_scales<G>(sca, scb, cur, sa_off, sb_off, scale_sel);
        p_compute<G, 0, 2>(acc, cur, fa_off, fb_off, sca, scb);
        if (!(half_last && last))
            p_compute<G, 2, G::STEPS>(acc, cur, fa_off, fb_off, sca, scb);
        if (last && qq < total)
            store_tile(cur);
        ckc = last ? 0 : ckc + 1;
        ctile += last ? g8 : 0u;
        ++qq;
    };
    for (int q = 0; q < total; q += G::S) {
        step(lds0, G::S == 2 ? lds1 : G::S == 3 ? lds2 : lds3);
        step(lds1, lds0);
        if constexpr (G::S > 2)
            step(lds2, lds1);
        if constexpr (G::S > 3)
            step(lds3, lds2);
    }
}

} // namespace

namespace {

template <class G>
hipError_t launch_persistent(const uint8_t *qa, const uint8_t *sa, int64_t M, const uint8_t *qb, const uint8_t *sb,
                             int64_t N, int64_t K, void *out, int bf16, hipStream_t stream)
{
    const int64_t tilesM = (M + G::BM - 1) / G::BM, tilesN = (N + G::BN - 1) / G::BN;
    const int64_t tiles = tilesM * tilesN;
    if (tiles > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    const void *fn = bf16 ? (const void *)mx_gemm_persistent<G, true> : (const void *)mx_gemm_persistent<G, false>;
    int64_t grid = (int64_t)device_cus() * occupancy_per_cu(fn, G::T);
    const int64_t tiles8 = (tiles + kGemmXcds - 1) / kGemmXcds * kGemmXcds;
    if (grid > tiles8)
        grid = tiles8;
    grid = grid / kGemmXcds * kGemmXcds;
    if (grid < (int64_t)kGemmXcds)
        grid = kGemmXcds;
    int Ki = (int)K, tn = (int)tilesN, tt = (int)tiles;
    void *args[] = {(void *)&qa, (void *)&sa, (void *)&M, (void *)&qb, (void *)&sb, (void *)&N, (void *)&Ki,
                    (void *)&out, (void *)&tn, (void *)&tt};
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(G::T), args, 0, stream);
}

// 128 x 128 tiles, 4 waves of 64 x 64, two workgroups per CU.  Measured on
// the transformer layer shapes: k chunks of 256 in a ring of 2 stages (68 KB)
// beat chunks of 128 in a ring of 4 (68 KB), and every one-workgroup-per-CU
// form (rings of 3 or 4 chunks of 256, 256 x 128 and 128 x 256 tiles), where
// a single wave per SIMD leaves the LDS and matrix-core latencies exposed.
using GemmP256 = PGeom<2, 2, 2, 2, 256, 2>;
using GemmP128 = PGeom<2, 2, 2, 2, 128, 4>;

} // namespace

hipError_t launch_mx_gemm(const uint8_t *qa, const uint8_t *sa, int64_t M, const uint8_t *qb, const uint8_t *sb,
                          int64_t N, int64_t K, void *out, int bf16, const Tuning &tune, hipStream_t stream)
{
    // the persistent form stores whole 16-byte output pieces and reads whole
    // dwords of scales
    const bool persistent = K % 128 == 0 && N % (bf16 ? 8 : 4) == 0 && (uintptr_t)out % 16 == 0 &&
                            (uintptr_t)sa % 4 == 0 && (uintptr_t)sb % 4 == 0;
    const int variant = tune.gemm_kernel;
    if (persistent && variant != 1) {
        if (variant == 3)
            return launch_persistent<GemmP128>(qa, sa, M, qb, sb, N, K, out, bf16, stream);
        return launch_persistent<GemmP256>(qa, sa, M, qb, sb, N, K, out, bf16, stream);
    }
    const int64_t tilesM = (M + kBM - 1) / kBM, tilesN = (N + kBN - 1) / kBN;
    const int64_t grid = (tilesM * tilesN + kGemmXcds - 1) / kGemmXcds * kGemmXcds;
    if (grid > 0x7FFFFFFF)
        return hipErrorInvalidConfiguration;
    int Ki = (int)K, tn = (int)tilesN;
    // 16-byte output stores need a 16-byte aligned base and whole pieces per row
    int vec = ((uintptr_t)out % 16 == 0) && N % (bf16 ? 8 : 4) == 0;
    void *args[] = {(void *)&qa, (void *)&sa, (void *)&M, (void *)&qb, (void *)&sb, (void *)&N, (void *)&Ki,
                    (void *)&out, (void *)&tn, (void *)&vec};
    const bool sal = K % 128 == 0;
    const void *fn = bf16 ? (sal ? (const void *)mx_gemm_kernel<true, true> : (const void *)mx_gemm_kernel<true, false>)
                          : (sal ? (const void *)mx_gemm_kernel<false, true> : (const void *)mx_gemm_kernel<false, false>);
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
}

} // namespace kq
