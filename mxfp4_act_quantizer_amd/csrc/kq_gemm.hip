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
// Data path: 128 x 128 output tile per workgroup of 4 waves (64 x 64 per
// wave as 2 x 2 MFMA tiles), two workgroups per CU.  k advances in chunks
// of 256 (4 MFMA steps): codes and scales of a chunk go global -> registers
// (buffer loads, two chunks ahead) -> LDS (double buffered) -> fragments.
// The finished tile goes back through LDS so that every store instruction
// writes whole 256-byte (bf16) or 512-byte (f32) row segments.
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

} // namespace

hipError_t launch_mx_gemm(const uint8_t *qa, const uint8_t *sa, int64_t M, const uint8_t *qb, const uint8_t *sb,
                          int64_t N, int64_t K, void *out, int bf16, hipStream_t stream)
{
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
