// Measurement-only export (not part of the quantizer API in kroquant.h): a
// plain streaming copy with the quantizer's 4:1 read:write footprint, which
// the benchmark times next to the quantizer as the practical HBM ceiling of
// a kernel that reads 2 bytes and writes 0.5 bytes per element.
//
// Each lane reads 16 bytes (nontemporal) and writes one 4-byte word (the xor
// of the four words read, nontemporal), grid-stride, four reads in flight per
// lane.  src_bytes / 4 bytes are written to dst.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kroquant.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 4;
constexpr int kGrid = 2048; // workgroups of 256 lanes (a sweep of 1024..8192 on MI355X put 2048 at the top)

__global__ __launch_bounds__(256) void copy41_kernel(const u32x4 *__restrict__ in, int64_t n16,
                                                     unsigned *__restrict__ out)
{
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            v[u] = __builtin_nontemporal_load(&in[i + u * stride]);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            __builtin_nontemporal_store(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3], &out[i + u * stride]);
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(&in[i]);
        __builtin_nontemporal_store(v[0] ^ v[1] ^ v[2] ^ v[3], &out[i]);
    }
}

} // namespace

extern "C" {

// src: device, 16-byte aligned, src_bytes a multiple of 16; dst: device,
// 4-byte aligned, src_bytes / 4 bytes, not overlapping src.  One launch on
// `stream`.  Returns KQ_OK, KQ_ERR_ARG, KQ_ERR_ALIGN, KQ_ERR_OVERLAP or KQ_ERR_HIP.
int kq_measure_copy41(const void *src, int64_t src_bytes, void *dst, void *stream)
{
    if (!src || !dst || src_bytes < 0 || src_bytes % 16)
        return KQ_ERR_ARG;
    if (((uintptr_t)src & 15) || ((uintptr_t)dst & 3))
        return KQ_ERR_ALIGN;
    const uintptr_t a0 = (uintptr_t)src, a1 = a0 + (uintptr_t)src_bytes;
    const uintptr_t b0 = (uintptr_t)dst, b1 = b0 + (uintptr_t)(src_bytes / 4);
    if (src_bytes > 0 && a0 < b1 && b0 < a1)
        return KQ_ERR_OVERLAP;
    if (src_bytes == 0)
        return KQ_OK;
    const int64_t n16 = src_bytes / 16;
    const int64_t need = (n16 + 255) / 256;
    const unsigned grid = (unsigned)(need < kGrid ? need : kGrid);
    const u32x4 *in = (const u32x4 *)src;
    unsigned *out = (unsigned *)dst;
    void *args[] = {(void *)&in, (void *)&n16, (void *)&out};
    return hipLaunchKernel((const void *)copy41_kernel, dim3(grid), dim3(256), args, 0, (hipStream_t)stream) ==
                   hipSuccess
               ? KQ_OK
               : KQ_ERR_HIP;
}

} // extern "C"
