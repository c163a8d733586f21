// extern "C" entry points of libkroquant.so: argument checks on the host, then
// one kernel launch on the caller's stream.  See include/kroquant.h for the
// contract of every function.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>

#include "../../include/kroquant.h"
#include "kq_internal.h"

// Row-statistics workspace of kq_adaln_quantize_noalloc: (mean,
// 1/sqrt(var + eps)) per row, KQ_NOALLOC_MAX_ROWS rows.  Each GPU holds its
// own copy; host code reaches it only through the device address looked up
// per device (noalloc_stats), never through this name.
static __device__ __align__(256) double scratch[2 * KQ_NOALLOC_MAX_ROWS];

namespace {

std::mutex g_scratch_mu;
std::map<int, double *> g_scratch_ptr;

// Device address of `scratch` on the current device (looked up once per
// device, with that device current).
hipError_t noalloc_stats(double **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    const auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return hipSuccess;
    }
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return e;
    if (p == nullptr)
        return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (double *)p;
    *out = (double *)p;
    return hipSuccess;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// [p, p + n) and [r, r + m) overlap?
bool overlap(const void *p, int64_t n, const void *r, int64_t m)
{
    const uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)n;
    const uintptr_t b0 = (uintptr_t)r, b1 = b0 + (uintptr_t)m;
    return n > 0 && m > 0 && a0 < b1 && b0 < a1;
}

// Shape check of a [M, d] activation with blocks of bw channels.  The block
// count M * (d / bw) is bounded by comparing M with the quotient, so no
// product is formed before the bound holds (afterwards M * d * 4 < 2^63).
int check_md_bw(int64_t M, int64_t d, int64_t bw)
{
    if (M < 0 || d <= 0)
        return KQ_ERR_ARG;
    if (d % bw != 0 || d > kq::kMaxD)
        return KQ_ERR_SHAPE;
    if (M > kq::kMaxBlocksTotal / (d / bw))
        return KQ_ERR_SHAPE;
    return KQ_OK;
}

int check_md(int64_t M, int64_t d) { return check_md_bw(M, d, 32); }

// Launch-shape overrides: NULL or every field in its documented range.
int check_tuning(const kq_tuning *t)
{
    if (!t)
        return KQ_OK;
    auto in = [](int32_t v, int32_t lo, int32_t hi) { return v == 0 || (v >= lo && v <= hi); };
    const bool ok = in(t->mfma_tiles_per_wg, 1, 256) && in(t->mfma_groups, 1, 2) &&
                    (t->mfma_strip == 0 || t->mfma_strip == 4 || t->mfma_strip == 8 || t->mfma_strip == 16) && in(t->mfma_order, 1, 2) &&
                    in(t->code_stores, 1, 2) && in(t->stream_rows_per_wave, 1, 256) && in(t->gemm_kernel, 1, 3) &&
                    in(t->adaln_pass, 1, 3) && (t->adaln_strip == 0 || t->adaln_strip == 4 || t->adaln_strip == 8) &&
                    in(t->adaln_blocks_per_wave, 1, 256) && in(t->shared_form, 1, 2) &&
                    in(t->flat_wgs, 1, 1 << 20) && in(t->flat_ring, 2, 3) &&
                    (t->mfma_ring == 0 || t->mfma_ring == 2 || t->mfma_ring == 4);
    return ok ? KQ_OK : KQ_ERR_ARG;
}

kq::Tuning tuning_of(const kq_tuning *t)
{
    kq::Tuning r{};
    if (t)
        r = *t;
    return r;
}

int check_sets(int64_t d, int64_t nT)
{
    if (nT != 1 && nT != d / 32)
        return KQ_ERR_SHAPE;
    return KQ_OK;
}

// HIP error behind the calling thread's most recent KQ_ERR_HIP return
thread_local hipError_t last_hip_error = hipSuccess;

int hip_status(hipError_t e)
{
    if (e == hipSuccess)
        return KQ_OK;
    last_hip_error = e;
    return KQ_ERR_HIP;
}

// shared checks of the quantizing entry points (x is bf16 or fp32)
int check_quant_io(const void *x, int64_t xbytes, const uint8_t *q, const uint8_t *s, int64_t M, int64_t d)
{
    if (!x || !q || !s)
        return KQ_ERR_ARG;
    if (!aligned(x, 16) || !aligned(q, 16))
        return KQ_ERR_ALIGN;
    const int64_t qbytes = M * (d / 2), sbytes = M * (d / 32);
    if (overlap(x, xbytes, q, qbytes) || overlap(x, xbytes, s, sbytes) || overlap(q, qbytes, s, sbytes))
        return KQ_ERR_OVERLAP;
    return KQ_OK;
}

int check_param(const float *p, int64_t count, const void *x, int64_t xbytes, const void *o1, int64_t n1,
                const void *o2, int64_t n2)
{
    if (!p)
        return KQ_ERR_ARG;
    if (!aligned(p, 4))
        return KQ_ERR_ALIGN;
    const int64_t pb = count * 4;
    if (overlap(p, pb, o1, n1) || overlap(p, pb, o2, n2))
        return KQ_ERR_OVERLAP;
    (void)x;
    (void)xbytes;
    return KQ_OK;
}

} // namespace

extern "C" {

int kq_quantize_tuned(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                      uint8_t *s, int variant, const kq_tuning *tuning, void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if (variant != KQ_VARIANT_AUTO && variant != KQ_VARIANT_MFMA && variant != KQ_VARIANT_BUTTERFLY)
        return KQ_ERR_ARG;
    if ((st = check_tuning(tuning)))
        return st;
    if ((st = check_sets(d, nT)))
        return st;
    if (M == 0)
        return KQ_OK;
    const int64_t xb = M * d * 2;
    if ((st = check_quant_io(x, xb, q, s, M, d)))
        return st;
    if ((st = check_param(factors, nT * 20, x, xb, q, M * (d / 2), s, M * (d / 32))))
        return st;
    hipStream_t hs = (hipStream_t)stream;
    const kq::Tuning tn = tuning_of(tuning);
    if (variant == KQ_VARIANT_BUTTERFLY)
        return hip_status(kq::launch_kq_butterfly(x, M, d, factors, nT, q, s, nullptr, tn, hs));
    return hip_status(kq::launch_kq_mfma(x, M, d, factors, nT, q, s, nullptr, 0, tn, hs));
}

int kq_quantize_ex(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                   uint8_t *s, int variant, void *stream)
{
    return kq_quantize_tuned(x, M, d, factors, nT, q, s, variant, nullptr, stream);
}

int kq_quantize(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                uint8_t *s, void *stream)
{
    return kq_quantize_tuned(x, M, d, factors, nT, q, s, KQ_VARIANT_AUTO, nullptr, stream);
}

int kq_transform_tuned(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, float *y,
                       int variant, const kq_tuning *tuning, void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if (variant != KQ_VARIANT_AUTO && variant != KQ_VARIANT_MFMA && variant != KQ_VARIANT_BUTTERFLY)
        return KQ_ERR_ARG;
    if ((st = check_tuning(tuning)))
        return st;
    if ((st = check_sets(d, nT)))
        return st;
    if (M == 0)
        return KQ_OK;
    if (!x || !y)
        return KQ_ERR_ARG;
    if (!aligned(x, 16) || !aligned(y, 16))
        return KQ_ERR_ALIGN;
    const int64_t xb = M * d * 2, yb = M * d * 4;
    if (overlap(x, xb, y, yb))
        return KQ_ERR_OVERLAP;
    if ((st = check_param(factors, nT * 20, x, xb, y, yb, nullptr, 0)))
        return st;
    hipStream_t hs = (hipStream_t)stream;
    const kq::Tuning tn = tuning_of(tuning);
    if (variant == KQ_VARIANT_BUTTERFLY)
        return hip_status(kq::launch_kq_butterfly(x, M, d, factors, nT, nullptr, nullptr, y, tn, hs));
    return hip_status(kq::launch_kq_mfma(x, M, d, factors, nT, nullptr, nullptr, y, 0, tn, hs));
}

int kq_transform_f32(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, float *y,
                     void *stream)
{
    return kq_transform_tuned(x, M, d, factors, nT, y, KQ_VARIANT_AUTO, nullptr, stream);
}

int kq_launch_shape(int64_t M, int64_t d, int adaln, const kq_tuning *tuning, int64_t shape[7])
{
    int st = check_md(M, d);
    if (st)
        return st;
    if ((adaln != 0 && adaln != 1) || !shape)
        return KQ_ERR_ARG;
    if ((st = check_tuning(tuning)))
        return st;
    kq::MfmaShape sh{};
    if ((st = hip_status(kq::mfma_launch_shape(M, d, tuning_of(tuning), adaln != 0, sh))))
        return st;
    shape[0] = sh.strip;
    shape[1] = sh.tiles_per_wg;
    shape[2] = sh.interleave;
    shape[3] = sh.flat;
    shape[4] = sh.grid;
    shape[5] = sh.nt_codes;
    shape[6] = sh.ring;
    return KQ_OK;
}

int kq_flat_launch_shape(int64_t M, int64_t d, const kq_tuning *tuning, int64_t shape[3])
{
    int st = check_md(M, d);
    if (st)
        return st;
    if (!shape)
        return KQ_ERR_ARG;
    if ((st = check_tuning(tuning)))
        return st;
    kq::FlatShape sh{};
    kq::flat_launch_shape(M, d, tuning_of(tuning), sh);
    shape[0] = sh.ring;
    shape[1] = sh.wgs;
    shape[2] = sh.nt_codes;
    return KQ_OK;
}

int kq_quantize_lu(const uint16_t *x, int64_t M, int64_t d, const float *lu, int64_t nT, uint8_t *q, uint8_t *s,
                   void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if ((st = check_sets(d, nT)))
        return st;
    if (M == 0)
        return KQ_OK;
    const int64_t xb = M * d * 2;
    if ((st = check_quant_io(x, xb, q, s, M, d)))
        return st;
    if ((st = check_param(lu, nT * 15, x, xb, q, M * (d / 2), s, M * (d / 32))))
        return st;
    return hip_status(kq::launch_kq_mfma(x, M, d, lu, nT, q, s, nullptr, 1, kq::Tuning{}, (hipStream_t)stream));
}

int kq_transform_lu_f32(const uint16_t *x, int64_t M, int64_t d, const float *lu, int64_t nT, float *y,
                        void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if ((st = check_sets(d, nT)))
        return st;
    if (M == 0)
        return KQ_OK;
    if (!x || !y)
        return KQ_ERR_ARG;
    if (!aligned(x, 16) || !aligned(y, 16))
        return KQ_ERR_ALIGN;
    const int64_t xb = M * d * 2, yb = M * d * 4;
    if (overlap(x, xb, y, yb))
        return KQ_ERR_OVERLAP;
    if ((st = check_param(lu, nT * 15, x, xb, y, yb, nullptr, 0)))
        return st;
    return hip_status(kq::launch_kq_mfma(x, M, d, lu, nT, nullptr, nullptr, y, 1, kq::Tuning{}, (hipStream_t)stream));
}

int fwht_quantize(const uint16_t *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if (M == 0)
        return KQ_OK;
    if ((st = check_quant_io(x, M * d * 2, q, s, M, d)))
        return st;
    return hip_status(kq::launch_fwht(x, M, d, q, s, nullptr, kq::Tuning{}, (hipStream_t)stream));
}

int fwht_transform_f32(const uint16_t *x, int64_t M, int64_t d, float *y, void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if (M == 0)
        return KQ_OK;
    if (!x || !y)
        return KQ_ERR_ARG;
    if (!aligned(x, 16) || !aligned(y, 16))
        return KQ_ERR_ALIGN;
    if (overlap(x, M * d * 2, y, M * d * 4))
        return KQ_ERR_OVERLAP;
    return hip_status(kq::launch_fwht(x, M, d, nullptr, nullptr, y, kq::Tuning{}, (hipStream_t)stream));
}

int sq_quantize(const uint16_t *x, int64_t M, int64_t d, const float *scale, uint8_t *q, uint8_t *s, void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if (M == 0)
        return KQ_OK;
    const int64_t xb = M * d * 2;
    if ((st = check_quant_io(x, xb, q, s, M, d)))
        return st;
    if ((st = check_param(scale, d, x, xb, q, M * (d / 2), s, M * (d / 32))))
        return st;
    return hip_status(kq::launch_sq(x, M, d, scale, q, s, kq::Tuning{}, (hipStream_t)stream));
}

int mx_quantize_f32(const float *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if (M == 0)
        return KQ_OK;
    if ((st = check_quant_io(x, M * d * 4, q, s, M, d)))
        return st;
    return hip_status(kq::launch_mx_f32(x, M, d, q, s, kq::Tuning{}, (hipStream_t)stream));
}

int mx_gemm_tuned(const uint8_t *qa, const uint8_t *sa, int64_t M, const uint8_t *qb, const uint8_t *sb, int64_t N,
                  int64_t K, void *out, int out_bf16, const kq_tuning *tuning, void *stream)
{
    if (M < 0 || N < 0 || K <= 0 || (out_bf16 != 0 && out_bf16 != 1))
        return KQ_ERR_ARG;
    int st = check_tuning(tuning);
    if (st)
        return st;
    // bounds by quotient: no product is formed before M * N <= 2^40 holds
    if (K % 32 != 0 || K > kq::kMaxD || N > ((int64_t)1 << 21) || (N > 0 && M > ((int64_t)1 << 40) / N))
        return KQ_ERR_SHAPE;
    if (M == 0 || N == 0)
        return KQ_OK;
    if (!qa || !sa || !qb || !sb || !out)
        return KQ_ERR_ARG;
    if (!aligned(qa, 16) || !aligned(qb, 16) || !aligned(out, out_bf16 ? 2 : 4))
        return KQ_ERR_ALIGN;
    const int64_t ob = M * N * (out_bf16 ? 2 : 4);
    if (overlap(out, ob, qa, M * (K / 2)) || overlap(out, ob, sa, M * (K / 32)) || overlap(out, ob, qb, N * (K / 2)) ||
        overlap(out, ob, sb, N * (K / 32)))
        return KQ_ERR_OVERLAP;
    return hip_status(
        kq::launch_mx_gemm(qa, sa, M, qb, sb, N, K, out, out_bf16, tuning_of(tuning), (hipStream_t)stream));
}

int mx_gemm(const uint8_t *qa, const uint8_t *sa, int64_t M, const uint8_t *qb, const uint8_t *sb, int64_t N,
            int64_t K, void *out, int out_bf16, void *stream)
{
    return mx_gemm_tuned(qa, sa, M, qb, sb, N, K, out, out_bf16, nullptr, stream);
}

// shape checks of the 16-element-block entry points
static int check_md16(int64_t M, int64_t d, int64_t nT)
{
    const int st = check_md_bw(M, d, 16);
    if (st)
        return st;
    if (nT != 1 && nT != d / 16)
        return KQ_ERR_SHAPE;
    return KQ_OK;
}

int kq_quantize16(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q, uint8_t *s,
                  void *stream)
{
    int st = check_md16(M, d, nT);
    if (st)
        return st;
    if (M == 0)
        return KQ_OK;
    if (!x || !q || !s)
        return KQ_ERR_ARG;
    if (!aligned(x, 16) || !aligned(q, 16))
        return KQ_ERR_ALIGN;
    const int64_t xb = M * d * 2, qb = M * (d / 2), sb = M * (d / 16);
    if (overlap(x, xb, q, qb) || overlap(x, xb, s, sb) || overlap(q, qb, s, sb))
        return KQ_ERR_OVERLAP;
    if ((st = check_param(factors, nT * 16, x, xb, q, qb, s, sb)))
        return st;
    return hip_status(kq::launch_kq16(x, M, d, factors, nT, q, s, nullptr, kq::Tuning{}, (hipStream_t)stream));
}

int kq_transform16_f32(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, float *y,
                       void *stream)
{
    int st = check_md16(M, d, nT);
    if (st)
        return st;
    if (M == 0)
        return KQ_OK;
    if (!x || !y)
        return KQ_ERR_ARG;
    if (!aligned(x, 16) || !aligned(y, 16))
        return KQ_ERR_ALIGN;
    const int64_t xb = M * d * 2, yb = M * d * 4;
    if (overlap(x, xb, y, yb))
        return KQ_ERR_OVERLAP;
    if ((st = check_param(factors, nT * 16, x, xb, y, yb, nullptr, 0)))
        return st;
    return hip_status(kq::launch_kq16(x, M, d, factors, nT, nullptr, nullptr, y, kq::Tuning{}, (hipStream_t)stream));
}

// shared checks of the AdaLN entry points (h, shift, scale, T, eps, the
// statistics workspace); out and out2 are the outputs, each with its byte count
// (own_stats: the workspace is the library's own array, so `stats` is not
// the caller's and is not checked)
static int check_adaln(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale, int64_t T,
                       float eps, const double *stats, const void *out, int64_t ob, const void *out2, int64_t ob2,
                       bool own_stats = false)
{
    if (T < 1 || !(eps > 0.0f) || eps > 3.0e38f)
        return KQ_ERR_ARG;
    if (!h || !shift || !scale || (!stats && !own_stats) || !out)
        return KQ_ERR_ARG;
    if (!aligned(h, 16) || !aligned(out, 16) || !aligned(shift, 4) || !aligned(scale, 4) || !aligned(stats, 8))
        return KQ_ERR_ALIGN;
    // samples: ceil(M / T) formed without M + T - 1 (T may be near INT64_MAX)
    const int64_t samples = M > 0 ? (M - 1) / T + 1 : 0;
    const int64_t hb = M * d * 2, pb = samples * d * 4, wb = M * 16;
    const void *in[3] = {h, shift, scale};
    const int64_t inb[3] = {hb, pb, pb};
    for (int i = 0; i < 3; ++i)
        if (overlap(out, ob, in[i], inb[i]) || overlap(out2, ob2, in[i], inb[i]) || overlap(stats, wb, in[i], inb[i]))
            return KQ_ERR_OVERLAP;
    if (overlap(out, ob, out2, ob2) || overlap(stats, wb, out, ob) || overlap(stats, wb, out2, ob2))
        return KQ_ERR_OVERLAP;
    return KQ_OK;
}

int kq_adaln_quantize_tuned(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                            int64_t tokens_per_sample, float eps, const float *factors, int64_t nT, double *stats,
                            uint8_t *q, uint8_t *s, const kq_tuning *tuning, void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if ((st = check_tuning(tuning)))
        return st;
    if ((st = check_sets(d, nT)))
        return st;
    if (M == 0)
        return KQ_OK;
    if (!s)
        return KQ_ERR_ARG;
    const int64_t qb = M * (d / 2), sb = M * (d / 32);
    if ((st = check_adaln(h, M, d, shift, scale, tokens_per_sample, eps, stats, q, qb, s, sb)))
        return st;
    if ((st = check_param(factors, nT * 20, h, M * d * 2, q, qb, s, sb)))
        return st;
    if (overlap(factors, nT * 80, stats, M * 16))
        return KQ_ERR_OVERLAP;
    return hip_status(kq::launch_adaln(h, M, d, shift, scale, tokens_per_sample, eps, factors, nT, stats, q, s,
                                       nullptr, tuning_of(tuning), (hipStream_t)stream));
}

int kq_adaln_quantize(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                      int64_t tokens_per_sample, float eps, const float *factors, int64_t nT, double *stats,
                      uint8_t *q, uint8_t *s, void *stream)
{
    return kq_adaln_quantize_tuned(h, M, d, shift, scale, tokens_per_sample, eps, factors, nT, stats, q, s, nullptr,
                                   stream);
}

int kq_adaln_quantize_noalloc(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                              int64_t tokens_per_sample, float eps, const float *factors, int64_t nT, uint8_t *q,
                              uint8_t *s, void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if ((st = check_sets(d, nT)))
        return st;
    if (M > KQ_NOALLOC_MAX_ROWS)
        return KQ_ERR_SHAPE;
    if (M == 0)
        return KQ_OK;
    if (!s)
        return KQ_ERR_ARG;
    const int64_t qb = M * (d / 2), sb = M * (d / 32);
    if ((st = check_adaln(h, M, d, shift, scale, tokens_per_sample, eps, nullptr, q, qb, s, sb, true)))
        return st;
    if ((st = check_param(factors, nT * 20, h, M * d * 2, q, qb, s, sb)))
        return st;
    double *stats = nullptr;
    if ((st = hip_status(noalloc_stats(&stats))))
        return st;
    return hip_status(kq::launch_adaln(h, M, d, shift, scale, tokens_per_sample, eps, factors, nT, stats, q, s,
                                       nullptr, kq::Tuning{}, (hipStream_t)stream));
}

int adaln_modulate(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                   int64_t tokens_per_sample, float eps, double *stats, uint16_t *x, void *stream)
{
    int st = check_md(M, d);
    if (st)
        return st;
    if (M == 0)
        return KQ_OK;
    if ((st = check_adaln(h, M, d, shift, scale, tokens_per_sample, eps, stats, x, M * d * 2, nullptr, 0)))
        return st;
    return hip_status(kq::launch_adaln(h, M, d, shift, scale, tokens_per_sample, eps, nullptr, 1, stats, nullptr,
                                       nullptr, x, kq::Tuning{}, (hipStream_t)stream));
}

const char *kq_status_string(int status)
{
    switch (status) {
    case KQ_OK: return "ok";
    case KQ_ERR_ARG: return "invalid argument (null pointer, negative size or unknown variant)";
    case KQ_ERR_SHAPE: return "invalid shape (d % 32 != 0, nT not in {1, d/32}, or too large)";
    case KQ_ERR_ALIGN: return "misaligned pointer (x, q, y need 16 bytes; factors, scale 4 bytes)";
    case KQ_ERR_SINGULAR: return "singular or non-finite 2x2 factor";
    case KQ_ERR_HIP: return "HIP runtime error at launch";
    case KQ_ERR_OVERLAP: return "an output buffer overlaps another buffer";
    default: return "unknown status";
    }
}

#ifndef KQ_SOURCE_HASH
#define KQ_SOURCE_HASH "unknown"
#endif

const char *kq_build_info(void)
{
    return "kroquant gfx950: default variant=mfma (v_mfma_f32_32x32x16_bf16, 3-term bf16 split of K), "
           "butterfly=DPP quad stages; FP4 via v_cvt_scalef32_pk_fp4_f32; sources " KQ_SOURCE_HASH;
}

int kq_last_hip_error(void) { return (int)last_hip_error; }

const char *kq_hip_error_name(int code) { return hipGetErrorName((hipError_t)code); }

} // extern "C"
