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
// byte - exactly one block of q and one byte of s.  The accumulator holds
// out[row 8(v/4) + 4(l/32) + v%4][column l % 32] in element v of lane l.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_internal.h"

namespace kq {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr unsigned kBufWord3G = 0x00020000; // raw buffer, 32-bit dwords
constexpr int kBM = 128, kBN = 128;          // workgroup tile
constexpr int kKC = 256;                     // k per LDS chunk (four 64-wide MFMA steps)
constexpr int kRowB = kKC / 2 + 16;          // padded LDS row of code bytes
constexpr int kSB = kKC / 32;                // scale bytes per row and chunk
constexpr unsigned kGemmXcds = 8;

struct __align__(16) GemmStage {
    unsigned char a[2][kBM][kRowB];
    unsigned char b[2][kBN][kRowB];
    unsigned char sa[2][kBM][kSB];
    unsigned char sb[2][kBN][kSB];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, (int)bytes, kBufWord3G);
}

// Raw loads of one chunk for one lane: four 16-byte code pieces of A and of
// B (rows t/8 + 32u, bytes 16 (t%8)), and four scale bytes of A and of B.
struct ChunkIn {
    u32x4 a[4], b[4];
    unsigned char sa[4], sb[4];
};

// Offsets past the k range (k >= K) or the tile's rows fall outside the
// ranges or carry bit 31: the hardware returns zeros.  A zero code is +0 and
// contributes nothing whatever its scale, and a zero scale byte is finite.
__device__ __forceinline__ void load_chunk(ChunkIn &in, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                           __amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb, int K, int kc,
                                           int t)
{
    const int col = (t & 7) * 16;   // byte within the chunk's 128 bytes of a row
    const int kbyte = kc / 2 + col; // byte within the row
    const unsigned dropk = (unsigned)(kbyte >= K / 2) << 31;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int row = (t >> 3) + 32 * u;
        const unsigned off = (unsigned)(row * (K / 2) + kbyte) | dropk;
        in.a[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
        in.b[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)off, 0, 0));
    }
    // scales: 128 rows x 8 bytes per operand = 1024 bytes = 4 per lane
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int f = t + 256 * u;
        const int row = f >> 3, kb = f & 7;
        const int kblk = kc / 32 + kb;
        const unsigned drop = (unsigned)(kblk >= K / 32) << 31;
        const unsigned off = (unsigned)(row * (K / 32) + kblk) | drop;
        in.sa[u] = __builtin_amdgcn_raw_buffer_load_b8(rsa, (int)off, 0, 0);
        in.sb[u] = __builtin_amdgcn_raw_buffer_load_b8(rsb, (int)off, 0, 0);
    }
}

__device__ __forceinline__ void stage_chunk(GemmStage &st, int par, const ChunkIn &in, int t)
{
    const int col = (t & 7) * 16;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int row = (t >> 3) + 32 * u;
        *(u32x4 *)&st.a[par][row][col] = in.a[u];
        *(u32x4 *)&st.b[par][row][col] = in.b[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int f = t + 256 * u;
        st.sa[par][f >> 3][f & 7] = in.sa[u];
        st.sb[par][f >> 3][f & 7] = in.sb[u];
    }
}

// One workgroup: a 128 x 128 tile of out; wave w computes rows 64 (w / 2) ..
// +63 and columns 64 (w % 2) .. +63 as 2 x 2 MFMA tiles.
template <bool kBf16>
__global__ __launch_bounds__(256) void mx_gemm_kernel(const uint8_t *__restrict__ qa, const uint8_t *__restrict__ sa,
                                                      int64_t M, const uint8_t *__restrict__ qb,
                                                      const uint8_t *__restrict__ sb, int64_t N, int K,
                                                      void *__restrict__ out, int tilesN)
{
    __shared__ GemmStage st;
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    // tiles dealt so that each XCD (blockIdx % 8) walks a contiguous range of
    // tiles, n fastest: consecutive workgroups of an XCD share their A rows in L2
    // (the grid is a multiple of 8, so every (XCD, slot) pair exists)
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

    const int wm = wave >> 1, wn = wave & 1;
    const int i = lane & 31, h = lane >> 5;
    f32x16 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
            acc[x][y] = f32x16{};

    const int nChunks = (K + kKC - 1) / kKC;
    ChunkIn in;
    load_chunk(in, ra, rb, rsa, rsb, K, 0, t);
    stage_chunk(st, 0, in, t);
    __syncthreads();
    for (int c = 0; c < nChunks; ++c) {
        const int par = c & 1;
        if (c + 1 < nChunks)
            load_chunk(in, ra, rb, rsa, rsb, K, (c + 1) * kKC, t);
        const int ksteps = (K - c * kKC) >= kKC ? 4 : (K - c * kKC + 63) / 64; // 64-wide steps left
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u >= ksteps)
                break; // uniform: the rest of the last chunk is past K
            i32x8 af[2], bf[2];
            int as[2], bs[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int ra_row = 64 * wm + 32 * x + i;
                const u32x4 va = *(const u32x4 *)&st.a[par][ra_row][32 * u + 16 * h];
                af[x] = i32x8{(int)va[0], (int)va[1], (int)va[2], (int)va[3], 0, 0, 0, 0};
                as[x] = st.sa[par][ra_row][2 * u + h];
                const int rb_row = 64 * wn + 32 * x + i;
                const u32x4 vb = *(const u32x4 *)&st.b[par][rb_row][32 * u + 16 * h];
                bf[x] = i32x8{(int)vb[0], (int)vb[1], (int)vb[2], (int)vb[3], 0, 0, 0, 0};
                bs[x] = st.sb[par][rb_row][2 * u + h];
            }
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[x], bf[y], acc[x][y], 4, 4, 0,
                                                                                as[x], 0, bs[y]);
        }
        // the other buffer was last read in the previous chunk, before the
        // previous barrier: stage into it, then one barrier before it is read
        if (c + 1 < nChunks) {
            stage_chunk(st, par ^ 1, in, t);
            __syncthreads();
        }
    }

    // out rows m0 + 64 wm + 32 x + 8 (v/4) + 4 h + v%4, columns n0 + 64 wn + 32 y + i
    constexpr int kES = kBf16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t ro = rsrc((unsigned char *)out + m0 * N * kES, rowsA * N * kES);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
            const int64_t col = n0 + 64 * wn + 32 * y + i;
            const unsigned dropc = (unsigned)(col >= N) << 31;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = 64 * wm + 32 * x + 8 * (v >> 2) + 4 * h + (v & 3);
                const unsigned off = (unsigned)((row * N + col) * kES) | dropc;
                if constexpr (kBf16) {
                    const __bf16 b = (__bf16)acc[x][y][v];
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, b), ro, (int)off, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[x][y][v]), ro, (int)off, 0, 0);
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
    void *args[] = {(void *)&qa, (void *)&sa, (void *)&M, (void *)&qb, (void *)&sb, (void *)&N, (void *)&Ki,
                    (void *)&out, (void *)&tn};
    const void *fn = bf16 ? (const void *)mx_gemm_kernel<true> : (const void *)mx_gemm_kernel<false>;
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, stream);
}

} // namespace kq
