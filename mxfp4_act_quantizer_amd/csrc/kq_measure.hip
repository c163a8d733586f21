// Measurement-only export (declared in the measurement section of
// kroquant.h): streaming copies with the quantizer's 4:1 read:write footprint
// (2 bytes read and 0.5 byte written per activation element), which the
// benchmark times next to the quantizer as the practical HBM ceiling of such
// a kernel.  Each 16-byte piece read yields one 4-byte word written (the xor of
// its four words, so no read can be optimised away).
//
// Forms (all read with nontemporal 16-byte loads; P = 16-byte pieces):
//   chunked:  wave w owns pieces [w*64*U, (w+1)*64*U): U loads of 1 KB per
//             wave in flight, then U stores of 256 B (4 bytes per lane); the
//             grid covers the input once (short-lived waves, like the
//             streaming quantizers)
//   wide:     a lane reads 4 consecutive pieces (64 bytes) per step and
//             writes one 16-byte word, so the stores are 1 KB per wave
//   stride:   grid-stride loop over 2048 workgroups, U pieces in flight per lane
//   persist:  one wave per resident slot walks chunks chunk = wave + k * waves
//   ring:     the memory instructions of the flat quantizer kernel: wave g of
//             G walks 2 KB units g, g + G, ... (two contiguous 1 KB loads, the
//             flat kernel's 16-lane row swap, one 512-byte store of 8 bytes
//             per lane), a register ring of R units (R - 1 in flight); R = 2
//             at two workgroups per CU with default-policy stores, or R = 3 at
//             one per CU with nontemporal stores, the flat kernel's two launch
//             shapes; also R = 4 at one per CU and R = 3 at two per CU, both
//             nontemporal.  Within each 64-byte group of src (4 pieces) the
//             words land in the order 0, 2, 1, 3 (the swap's order)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kroquant.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

template <bool kNT>
__device__ __forceinline__ void put(unsigned *p, unsigned v)
{
    if constexpr (kNT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// chunked / persistent: U loads of 1 KB per wave, then U stores of 256 B
template <int U, bool kNT, bool kPersist>
__global__ __launch_bounds__(256) void copy41_chunked(const u32x4 *__restrict__ in, int64_t n16,
                                                      unsigned *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t waves = kPersist ? (int64_t)gridDim.x * 4 : 1;
    const int64_t chunk = 64 * U;
    for (int64_t w = wave0; w * chunk < n16; w += waves) {
        const int64_t base = w * chunk + lane;
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = base + 64 * u;
            v[u] = p < n16 ? __builtin_nontemporal_load(&in[p]) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t p = base + 64 * u;
            if (p < n16)
                put<kNT>(&out[p], fold(v[u]));
        }
        if (!kPersist)
            break;
    }
}

// wide: lane reads pieces 4j .. 4j+3 (64 contiguous bytes) and writes word j of
// 16 bytes; U such steps per wave
template <int U>
__global__ __launch_bounds__(256) void copy41_wide(const u32x4 *__restrict__ in, int64_t n16, u32x4 *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t n64 = n16 / 4; // n16 is a multiple of 64
    u32x4 v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t j = (w * U + u) * 64 + lane;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            v[u][k] = j < n64 ? __builtin_nontemporal_load(&in[4 * j + k]) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t j = (w * U + u) * 64 + lane;
        if (j < n64)
            __builtin_nontemporal_store(u32x4{fold(v[u][0]), fold(v[u][1]), fold(v[u][2]), fold(v[u][3])}, &out[j]);
    }
}

// grid-stride: 2048 workgroups, U pieces in flight per lane
template <int U>
__global__ __launch_bounds__(256) void copy41_stride(const u32x4 *__restrict__ in, int64_t n16,
                                                     unsigned *__restrict__ out)
{
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(&in[i + u * stride]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            __builtin_nontemporal_store(fold(v[u]), &out[i + u * stride]);
    }
    for (; i < n16; i += stride)
        __builtin_nontemporal_store(fold(__builtin_nontemporal_load(&in[i])), &out[i]);
}

// ring: see the header comment; buffer ranges drop the half unit past the end
// and the look-ahead past a wave's last unit
template <int kR, bool kNT>
__global__ __launch_bounds__(256) void copy41_ring(const unsigned char *__restrict__ in, int64_t nbytes,
                                                   unsigned char *__restrict__ out)
{
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    constexpr unsigned kWord3 = 0x00020000u;
    const int lane = threadIdx.x & 63;
    const int64_t G = (int64_t)gridDim.x * 4;
    const int64_t g = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nunits = (nbytes + 2047) / 2048;
    if (g >= nunits)
        return;
    const int n = (int)((nunits - g + G - 1) / G);
    const int col = lane & 31, h = lane >> 5;
    const int off = 64 * (col & 15) + 32 * (col >> 4) + 16 * h;
    auto unit_of = [&](int k) -> int64_t { return g + (int64_t)(k < n ? k : n - 1) * G; };
    auto bytes_of = [&](int k) -> int {
        const int64_t left = nbytes - unit_of(k) * 2048;
        return k < n ? (int)(left < 2048 ? left : 2048) : 0;
    };
    u32x4 ring[kR][2];
    auto load = [&](u32x4 (&r)[2], int k) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)(in + unit_of(k) * 2048), 0,
                                                                            bytes_of(k), kWord3);
        r[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2));
        r[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 1024, 0, 2));
    };
    auto store = [&](const u32x4 (&r)[2], int k) {
        const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void *)(out + unit_of(k) * 512), 0,
                                                                            bytes_of(k) / 4, kWord3);
        // lane (c, h) holds pieces 4c + h and 4c + 2 + h after the swap
        unsigned a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto t = __builtin_amdgcn_permlane16_swap(r[0][i], r[1][i], false, false);
            a[i] = t[0];
            b[i] = t[1];
        }
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{a[0] ^ a[1] ^ a[2] ^ a[3], b[0] ^ b[1] ^ b[2] ^ b[3]}, rd,
                                              16 * col + 8 * h, 0, kNT ? 2 : 0);
    };
#pragma unroll
    for (int k = 0; k < kR - 1; ++k)
        load(ring[k], k);
    auto step = [&](u32x4 (&cur)[2], u32x4 (&ld)[2], int kk) {
        load(ld, kk + kR - 1);
        __builtin_amdgcn_sched_barrier(0);
        store(cur, kk);
        __builtin_amdgcn_sched_barrier(0);
    };
    int it = 0;
    for (; it + kR - 1 < n; it += kR) {
#pragma unroll
        for (int k = 0; k < kR; ++k)
            step(ring[k], ring[(k + kR - 1) % kR], it + k);
    }
#pragma unroll
    for (int k = 0; k < kR - 1; ++k)
        if (it + k < n)
            step(ring[k], ring[kR - 1], it + k);
}

int device_cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || n <= 0)
        n = 256;
    return n;
}

} // namespace

extern "C" {

int kq_measure_copy41(const void *src, int64_t src_bytes, void *dst, int form, void *stream)
{
    if (!src || !dst || src_bytes < 0 || src_bytes % 1024 || form < 0 || form >= KQ_COPY_FORMS)
        return KQ_ERR_ARG;
    if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
        return KQ_ERR_ALIGN;
    const uintptr_t a0 = (uintptr_t)src, a1 = a0 + (uintptr_t)src_bytes;
    const uintptr_t b0 = (uintptr_t)dst, b1 = b0 + (uintptr_t)(src_bytes / 4);
    if (src_bytes > 0 && a0 < b1 && b0 < a1)
        return KQ_ERR_OVERLAP;
    if (src_bytes == 0)
        return KQ_OK;
    const int64_t n16 = src_bytes / 16;
    const u32x4 *in = (const u32x4 *)src;
    unsigned *out = (unsigned *)dst;
    u32x4 *out16 = (u32x4 *)dst;
    hipStream_t hs = (hipStream_t)stream;
    auto waves_for = [&](int64_t pieces_per_wave) { return (n16 + pieces_per_wave - 1) / pieces_per_wave; };
    auto grid_for = [&](int64_t waves) { return (waves + 3) / 4; };
    int64_t grid = 0;
    const void *fn = nullptr;
    switch (form) {
    case 0: fn = (const void *)copy41_chunked<8, true, false>; grid = grid_for(waves_for(64 * 8)); break;
    case 1: fn = (const void *)copy41_chunked<8, false, false>; grid = grid_for(waves_for(64 * 8)); break;
    case 2: fn = (const void *)copy41_chunked<4, true, false>; grid = grid_for(waves_for(64 * 4)); break;
    case 3: fn = (const void *)copy41_wide<2>; grid = grid_for(waves_for(64 * 4 * 2)); break;
    case 4: {
        fn = (const void *)copy41_chunked<8, true, true>;
        const int64_t slots = (int64_t)device_cus() * 8; // 8 workgroups of 4 waves per CU
        const int64_t need = grid_for(waves_for(64 * 8));
        grid = need < slots ? need : slots;
        break;
    }
    case 5: {
        fn = (const void *)copy41_stride<4>;
        const int64_t need = (n16 + 255) / 256;
        grid = need < 2048 ? need : 2048;
        break;
    }
    default: {
        // ring forms: (ring depth, nontemporal stores, workgroups per CU)
        int per_cu = 1;
        switch (form) {
        case 6: fn = (const void *)copy41_ring<2, false>; per_cu = 2; break;
        case 7: fn = (const void *)copy41_ring<3, true>; break;
        case 8: fn = (const void *)copy41_ring<4, true>; break;
        default: fn = (const void *)copy41_ring<3, true>; per_cu = 2; break;
        }
        const int64_t slots = (int64_t)device_cus() * per_cu;
        const int64_t units = (src_bytes + 2047) / 2048;
        const int64_t need = (units + 3) / 4;
        grid = need < slots ? need : slots;
        break;
    }
    }
    if (grid > 0x7FFFFFFF)
        return KQ_ERR_SHAPE;
    void *args_w[] = {(void *)&in, (void *)&n16, (void *)&out16};
    void *args[] = {(void *)&in, (void *)&n16, (void *)&out};
    void *args_r[] = {(void *)&src, (void *)&src_bytes, (void *)&dst};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256),
                                         form == 3 ? args_w : form >= 6 ? args_r : args, 0, hs);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

} // extern "C"
