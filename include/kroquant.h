/*
 * kroquant.h - C ABI of the MI355X (gfx950) KroQuant activation quantizer.
 *
 * What the library computes (pages describing arXiv 2607.21446, "KroQuant:
 * Kronecker-Structured Block Transforms for Efficient Post-Training
 * Quantization of Diffusion Transformers"):
 *   - the abstract (mlsanity.com paper page, section "Abstract (arXiv)"): a
 *     learned Kronecker-structured invertible transform applied online to each
 *     32-element block of an activation row, its inverse folded into the
 *     weights offline, W4A4 with MXFP4 ("MXFP4e2"); per-channel scaling
 *     (SmoothQuant) is the cheap alternative it is compared with;
 *   - the pith.science verdict record for 2607.21446, field
 *     pith_extraction.key_machinery: every 32x32 block is
 *     K = A1 (x) A2 (x) A3 (x) A4 (x) A5 of five 2x2 factors, applied before
 *     the MX quantizer;
 *   - same record, skeptic_critique.load_bearing_attack (paper Section 3.2,
 *     Eq. 4): the transform is block diagonal, blocks aligned with the
 *     quantizer's 32-element blocks.
 * Element and scale encodings follow the OCP Microscaling (MX) v1.0 spec:
 * FP4 E2M1 codes (sign in bit 3), round to nearest even, saturating at +-6;
 * one E8M0 byte per 32 elements holding E + 127 with
 * E = clamp(floor(log2(max|y|)) - 2, -127, 127).
 *
 * Conventions shared by every entry point
 *   - Layouts are dense row-major.  x[M, d] is bf16 (passed as its uint16 bit
 *     patterns), q[M, d/2] holds packed codes (element 2i in bits 0-3 of byte
 *     i, element 2i+1 in bits 4-7), s[M, d/32] holds one E8M0 byte per block
 *     of 32 consecutive elements of a row.
 *   - Block b = m * (d/32) + j covers x[m, 32j .. 32j+31], q bytes
 *     [16b, 16b+16) and s byte b.
 *   - factors is float32 [nT, 5, 2, 2]: factors[t][k][r][c] is entry (r, c) of
 *     A_{k+1} of set t.  nT = 1 shares one set among all blocks; nT = d/32
 *     gives set j to block column j.  A1 acts on the most significant bit of
 *     the 5-bit in-block index (numpy kron order).  A row block x (1x32) is
 *     transformed as y = x . K, so (X T)(T^-1 W^T) = X W^T.
 *   - Sign of a code is set iff its value is < 0 (+0 and -0 give code 0).  An
 *     all-zero block has scale byte 0x00.  A block whose transformed values
 *     contain a NaN or an infinity gets scale byte 0xFF and zero codes.
 *   - "dev" pointers are device (HBM) pointers, "host" pointers are host
 *     memory.  The caller owns every buffer.  Device entry points never
 *     allocate, free or synchronise: they check their arguments on the host,
 *     enqueue kernels on `stream` (a hipStream_t; NULL is the default stream)
 *     and return.  A kernel fault surfaces at the caller's next
 *     synchronisation.  Inputs are read-only; q and s are fully overwritten.
 *   - M == 0 is a successful no-op (pointers are not inspected).
 *   - Argument errors are reported before any HIP call and launch nothing.
 *   - Every entry point is stateless and reentrant: a launch depends only on
 *     its arguments and on the device it runs on (compute-unit count and
 *     kernel occupancy, queried once per device under a lock).  Calls from
 *     several host threads, on one stream or several, need no external
 *     locking.  The library keeps no mutable settings; launch-shape overrides
 *     exist only as an argument of the measurement entry points at the end of
 *     this header.
 */
#ifndef KROQUANT_H
#define KROQUANT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define KQ_OK 0
#define KQ_ERR_ARG 1      /* null pointer, M < 0, d <= 0, bad variant */
#define KQ_ERR_SHAPE 2    /* d % 32 != 0, nT not in {1, d/32}, size too large for a launch */
#define KQ_ERR_ALIGN 3    /* x, q, y not 16-byte aligned, factors / scale not 4-byte aligned */
#define KQ_ERR_SINGULAR 4 /* host helpers: a 2x2 factor with |det| < 1e-30 or a non-finite entry */
#define KQ_ERR_HIP 5      /* the HIP runtime reported an error at launch */
#define KQ_ERR_OVERLAP 6  /* an output buffer overlaps an input or another output */

/* transform variants for kq_quantize_ex / kq_transform_f32 */
#define KQ_VARIANT_AUTO 0      /* the library's default (the faster one on MI355X) */
#define KQ_VARIANT_MFMA 1      /* dense 32x32 block on bf16 MFMA, K as an exact 3-term bf16 split */
#define KQ_VARIANT_BUTTERFLY 2 /* five 2x2 stages in fp32 registers, cross-lane stages via DPP */

/*
 * kq_quantize: KroQuant online quantizer.  For every block, y = x_blk . K_j in
 * fp32 accumulation, then MXFP4 quantization of y (abstract; key_machinery).
 * With nT = d/32 (a set per block) the strip kernel runs; with nT = 1 (one set
 * shared by every block) the flat kernel, which treats x as one run of M*d/32
 * blocks.  Both compute the same values bit for bit.
 *   x        dev, bf16 bits [M, d], 16-byte aligned
 *   factors  dev, float32 [nT, 5, 2, 2], nT = 1 or d/32, 4-byte aligned
 *   q        dev, uint8 [M, d/2], 16-byte aligned
 *   s        dev, uint8 [M, d/32], any alignment
 *   stream   hipStream_t or NULL
 * Returns KQ_OK or an error code (nothing launched on error).
 */
int kq_quantize(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                uint8_t *s, void *stream);

/* kq_quantize with an explicit transform variant (KQ_VARIANT_*). */
int kq_quantize_ex(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                   uint8_t *s, int variant, void *stream);

/*
 * kq_transform_f32: the transformed values y = x_blk . K_j (fp32) that
 * kq_quantize quantizes, written out for inspection.  Same transform code,
 * same kernel and the same launch shape (strip kernel: strip width, token
 * groups, workgroup order; flat kernel: ring depth and grid) as kq_quantize
 * for the same (M, d, nT); only the MX step is replaced by fp32 stores of y.
 * kq_transform_tuned (below) selects the butterfly variant.
 *   y  dev, float32 [M, d], 16-byte aligned
 */
int kq_transform_f32(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, float *y,
                     void *stream);

/*
 * sq_quantize: SmoothQuant-style comparison quantizer (abstract: per-channel
 * scaling).  y[m, c] = x[m, c] * fl32(1 / scale[c]) rounded once to fp32, then
 * the same MXFP4 quantization.
 *   scale  dev, float32 [d], 4-byte aligned
 */
int sq_quantize(const uint16_t *x, int64_t M, int64_t d, const float *scale, uint8_t *q, uint8_t *s,
                void *stream);

/*
 * mx_quantize_f32: plain MXFP4 quantization of an fp32 matrix (no transform).
 *   x  dev, float32 [M, d], 16-byte aligned
 */
int mx_quantize_f32(const float *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, void *stream);

/*
 * K2 form: each factor set given as 15 LU scalars and rebuilt inside the
 * kernel (pith.science record: key_machinery and core_discovery - three
 * scalars per factor through a unit-determinant LU form, 15 per block, and a
 * kernel that rebuilds the block from them on the fly; referee_report.
 * minor_comments on section 3 - U = [[a, b], [0, -1/a]], det G = -1).
 * Reading of the unstated L: L = [[1, 0], [c, 1]], so
 * G = L U = [[a, b], [c a, c b - 1/a]] (a = b = 1/sqrt(2), c = 1 gives the
 * normalised 2x2 Hadamard factor).
 *   lu  dev, float32 [nT, 5, 3]: lu[t][k] = (a, b, c) of factor A_{k+1} of set t,
 *       nT = 1 or d/32, 4-byte aligned
 * In the kernel each factor is formed in fp32 exactly as kq_lu_factors forms
 * it on the host, then the block is transformed on the matrix cores as in
 * kq_quantize (KQ_VARIANT_MFMA).  a = 0 or non-finite scalars make the
 * block's values non-finite: such blocks encode as scale 0xFF, codes 0.
 * Otherwise the same contract as kq_quantize.
 */
int kq_quantize_lu(const uint16_t *x, int64_t M, int64_t d, const float *lu, int64_t nT, uint8_t *q, uint8_t *s,
                   void *stream);

/* The transformed values of kq_quantize_lu (fp32), for inspection.
 *   y  dev, float32 [M, d], 16-byte aligned */
int kq_transform_lu_f32(const uint16_t *x, int64_t M, int64_t d, const float *lu, int64_t nT, float *y,
                        void *stream);

/*
 * fwht_quantize: the fixed-transform comparison kernel (pith.science record,
 * pith_extraction.forward_implications: the K2 kernel is compared with a fast
 * Walsh-Hadamard transform of the same 32-element blocks).  For every block,
 * y_c = (1/sqrt 32) sum_r x_r (-1)^popcount(r & c) (Sylvester order, five
 * butterfly stages of +-1 in fp32, then one multiply by fl32(1/sqrt 32)),
 * then the same MXFP4 quantization.  Same contract as sq_quantize without a
 * parameter array.
 */
int fwht_quantize(const uint16_t *x, int64_t M, int64_t d, uint8_t *q, uint8_t *s, void *stream);

/* The transformed values of fwht_quantize (fp32), for inspection.
 *   y  dev, float32 [M, d], 16-byte aligned */
int fwht_transform_f32(const uint16_t *x, int64_t M, int64_t d, float *y, void *stream);

/*
 * kq_quantize16: the same quantizer on 16-element blocks with four Kronecker
 * factors (pith.science record, pith_inferences[0], an editorial inference:
 * the construction carries over to 16-element blockwise formats by changing
 * the number of factors).  Reading: K16 = A1 (x) A2 (x) A3 (x) A4 per
 * 16-channel block (A1 on the most significant bit of the 4-bit in-block
 * index), y = x_blk . K16_j in fp32, and the MX rules applied to 16-element
 * blocks: one E8M0 scale per 16 elements, E2M1 codes, element 2i in the low
 * nibble.  The transform runs on the matrix cores as a 32 x 32 block per
 * pair of 16-element blocks: I (x) K16 with one shared set (nT = 1), and
 * diag(K16_2j, K16_2j+1) with a set per block (nT = d/16) when d % 32 == 0;
 * each half is one 16-element block summed on its own (a NaN or Inf input
 * stays in its own block).  A set per block with d % 32 == 16 runs as four
 * butterfly stages instead (one cross-lane stage over a lane pair by DPP,
 * three in-lane stages).  Both give the same results up to fp32 rounding.
 *   x        dev, bf16 [M, d], d % 16 == 0, 16-byte aligned
 *   factors  dev, float32 [nT, 4, 2, 2], nT = 1 or d/16, 4-byte aligned
 *   q        dev, u8 [M, d/2], 16-byte aligned
 *   s        dev, u8 [M, d/16] (one scale byte per 16 elements)
 * Otherwise the same contract and errors as kq_quantize (KQ_ERR_SHAPE for
 * d % 16 != 0 or nT not in {1, d/16}).
 */
int kq_quantize16(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q, uint8_t *s,
                  void *stream);

/* The transformed values of kq_quantize16 (fp32), for inspection.
 *   y  dev, float32 [M, d], 16-byte aligned */
int kq_transform16_f32(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, float *y,
                       void *stream);

/*
 * kq_adaln_quantize: the quantizer fused with the AdaLN normalisation in
 * front of it (abstract on the mlsanity.com paper page: the normalisation
 * layers between blocks make the transform run online at every step;
 * pith.science record, referee_report.summary: AdaLN is what prevents
 * absorbing it offline).  For token row m of sample b = m / tokens_per_sample:
 *   x_c = (h_c - mean) / sqrt(var + eps) * (1 + scale[b][c]) + shift[b][c]
 * (mean and biased variance over the row's d channels; LayerNorm without a
 * learned affine - a reading, the pages print no formula), x rounded to bf16
 * (nearest, ties to even) from its double value, then the Kronecker transform
 * of every 32-channel block and MXFP4 as kq_quantize.  The normalised x is
 * never written: one pass writes the row statistics into `stats`, a second
 * reads h again, normalises it while staging it for the matrix cores, and
 * quantizes (kq_adaln_quantize_tuned can select a one-launch form instead,
 * which holds whole rows in LDS; same results and statistics, bit for bit).
 * The transform is the default (KQ_VARIANT_MFMA) form; the result equals
 * kq_quantize(adaln_modulate(h), ...) bit for bit.
 *   h      dev, bf16 [M, d] (the residual stream), 16-byte aligned
 *   shift  dev, float32 [ceil(M / tokens_per_sample), d], 4-byte aligned
 *   scale  dev, float32, same shape and alignment as shift
 *   tokens_per_sample  >= 1 (rows of one sample are consecutive)
 *   eps    > 0 and finite (KQ_ERR_ARG otherwise)
 *   stats  dev, float64 [M, 2], 8-byte aligned: workspace owned by the caller
 *          (row mean and 1/sqrt(var + eps), overwritten; its contents after
 *          the call are those values, in double)
 *   factors, nT, q, s  as kq_quantize
 * Statistics and normalisation run in double.  Two launches on `stream`.
 * Outputs and the workspace may not overlap h, shift, scale, factors or each
 * other (KQ_ERR_OVERLAP).  Otherwise the same contract as kq_quantize.
 */
int kq_adaln_quantize(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                      int64_t tokens_per_sample, float eps, const float *factors, int64_t nT, double *stats,
                      uint8_t *q, uint8_t *s, void *stream);

/*
 * kq_adaln_quantize_noalloc: kq_adaln_quantize for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc).  The row-statistics workspace is a fixed
 * device array inside the library instead of the caller's `stats`:
 * KQ_NOALLOC_MAX_ROWS rows of 16 bytes (2 MiB), one copy per GPU the library
 * runs on, held until the process ends; its device address is looked up
 * once per device on the first call there.  M > KQ_NOALLOC_MAX_ROWS returns
 * KQ_ERR_SHAPE and launches nothing.  The call allocates and frees nothing.
 * Every call on one GPU shares that array and leaves its statistics in it:
 * calls that overlap in time on the same GPU (different streams, or threads
 * without ordering) race on it and must be ordered by the caller.  Calls on
 * one stream are ordered.  Arguments, results and errors are otherwise those
 * of kq_adaln_quantize.
 */
#define KQ_NOALLOC_MAX_ROWS 131072
int kq_adaln_quantize_noalloc(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                              int64_t tokens_per_sample, float eps, const float *factors, int64_t nT, uint8_t *q,
                              uint8_t *s, void *stream);

/*
 * adaln_modulate: the same normalisation alone (the unfused front-end): x as
 * kq_adaln_quantize computes it, written as bf16.
 *   x  dev, bf16 [M, d], 16-byte aligned, not overlapping h, shift, scale or stats
 * Same arguments and errors as kq_adaln_quantize otherwise.
 */
int adaln_modulate(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                   int64_t tokens_per_sample, float eps, double *stats, uint16_t *x, void *stream);

/*
 * mx_gemm: the W4A4 consumer of the quantizer's output (abstract: MXFP4 W4A4,
 * with the inverse transform folded into the weights).  out = A . B^T, where
 * A [M, K] and B [N, K] are MXFP4 matrices in the layout above: codes
 * qa [M, K/2], qb [N, K/2] and E8M0 scales sa [M, K/32], sb [N, K/32].  Every
 * element is (E2M1 value) x 2^(s - 127); a scale byte 0xFF is NaN.  Products
 * are formed on the gfx950 block-scaled FP4 matrix cores and accumulated in
 * fp32; out is float32 [M, N] (out_bf16 = 0) or bf16 [M, N] rounded to
 * nearest even from that fp32 sum (out_bf16 = 1).
 *   qa, qb     dev, 16-byte aligned        sa, sb  dev, any alignment
 *   out        dev, 4-byte (float32) or 2-byte (bf16) aligned, not overlapping
 *   K % 32 == 0, K <= 2^20, N <= 2^21 (per-tile offsets stay 32-bit).
 *   M == 0 or N == 0 is a no-op.
 * Typical use: qa, sa from kq_quantize of the activations; qb, sb from
 * mx_quantize_f32 of kq_fold_weight(W).
 */
int mx_gemm(const uint8_t *qa, const uint8_t *sa, int64_t M, const uint8_t *qb, const uint8_t *sb, int64_t N,
            int64_t K, void *out, int out_bf16, void *stream);

/* ---------------- host helpers for the offline weight side --------------- */
/* All pointers are host memory; the calls are synchronous and touch no GPU.  */

/* inv[t][k] = A_k^-1 of set t, for every set and factor (abstract: the
 * inverse goes to the weights; key_machinery: inverse of a Kronecker product
 * is the Kronecker product of the inverses).  inv: float32 [nT, 5, 2, 2]. */
int kq_factor_inverse(const float *factors, int64_t nT, float *inv);

/* K[t] = A1 (x) ... (x) A5 of set t as a dense float32 [nT, 32, 32] matrix
 * (row r = input index, column c = output index: y = x . K). */
int kq_block_matrix(const float *factors, int64_t nT, float *K);

/* Kinv[t] = A1^-1 (x) ... (x) A5^-1 = K[t]^-1, float32 [nT, 32, 32]. */
int kq_block_inverse(const float *factors, int64_t nT, float *Kinv);

/* Fold T^-1 into a weight matrix W[N, d] (float32, row-major), so that for
 * Y = X T the product Y W_out^T equals X W^T:  W_out = W T^-T, i.e. for every
 * row n and block j, W_out[n, 32j:32j+32] = W[n, 32j:32j+32] . (K_j^-1)^T.
 * Accumulates in double, rounds once to float32.  W_out may equal W. */
int kq_fold_weight(const float *W, int64_t N, int64_t d, const float *factors, int64_t nT, float *W_out);

/* The 2x2 factors [nT, 5, 2, 2] of LU-parameterised sets [nT, 5, 3], formed
 * in fp32 exactly as kq_quantize_lu forms them in the kernel: g00 = a,
 * g01 = b, g10 = fl32(c a), g11 = fma(c, b, -fl32(1/a)).  The result can be
 * passed to kq_fold_weight, kq_factor_inverse or kq_quantize.  Returns
 * KQ_ERR_SINGULAR if some a is 0 or a scalar or result is not finite. */
int kq_lu_factors(const float *lu, int64_t nT, float *factors);

/* ---------------- measurement and test interface ----------------------- */
/* Launch-shape overrides for benchmarks and for tests that pin a launch
 * shape.  A field left 0 keeps the library's automatic choice; the product
 * entry points above always use the automatic choices.  Out-of-range values
 * are rejected with KQ_ERR_ARG. */
typedef struct kq_tuning {
    int32_t mfma_tiles_per_wg;     /* MFMA quantizer: 32-token tiles per workgroup, 1..256 */
    int32_t mfma_groups;           /* 1 contiguous runs of tiles, 2 interleaved token groups */
    int32_t mfma_strip;            /* 4, 8 or 16 blocks (32-channel) per workgroup */
    int32_t mfma_order;            /* 1 XCD-grouped workgroups, 2 flat order */
    int32_t code_stores;           /* MFMA quantizer code stores: 1 default cache policy, 2 nontemporal */
    int32_t stream_rows_per_wave;  /* butterfly, SmoothQuant, fp32, FWHT, 16-element kernels: rows per wave, 1..256 */
    int32_t gemm_kernel;           /* mx_gemm: 1 per-tile, 2 persistent (k chunks of 256), 3 persistent (128) */
    int32_t adaln_pass;            /* kq_adaln_quantize form: 1 two launches, second pass on the matrix
                                      cores; 2 two launches, butterfly second pass; 3 one launch (whole
                                      rows in LDS; KQ_ERR_HIP when they do not fit) */
    int32_t adaln_strip;           /* its matrix-core strip width: 4 or 8 blocks */
    int32_t adaln_blocks_per_wave; /* butterfly / adaln_modulate pass: row blocks per wave, 1..256 */
    int32_t shared_form;           /* MFMA quantizer with one shared factor set: 1 the strip kernel, 2 the
                                      flat kernel (the default when no mfma_* field is set) */
    int32_t flat_wgs;              /* flat kernel: workgroups of 4 waves, 1..2^20 */
    int32_t flat_ring;             /* flat kernel: register ring of 2 or 3 units of 32 blocks */
    int32_t mfma_ring;             /* strip kernel (and the AdaLN second pass): register ring of 2 or 4 tiles */
} kq_tuning;

/* kq_quantize_ex / kq_transform_f32 / mx_gemm / kq_adaln_quantize with
 * launch-shape overrides (tuning may be NULL: automatic).  variant is one of
 * KQ_VARIANT_*.  Results do not depend on the launch shape: every shape
 * computes the same values bit for bit (the tests check this). */
int kq_quantize_tuned(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, uint8_t *q,
                      uint8_t *s, int variant, const kq_tuning *tuning, void *stream);
int kq_transform_tuned(const uint16_t *x, int64_t M, int64_t d, const float *factors, int64_t nT, float *y,
                       int variant, const kq_tuning *tuning, void *stream);
int mx_gemm_tuned(const uint8_t *qa, const uint8_t *sa, int64_t M, const uint8_t *qb, const uint8_t *sb, int64_t N,
                  int64_t K, void *out, int out_bf16, const kq_tuning *tuning, void *stream);
int kq_adaln_quantize_tuned(const uint16_t *h, int64_t M, int64_t d, const float *shift, const float *scale,
                            int64_t tokens_per_sample, float eps, const float *factors, int64_t nT, double *stats,
                            uint8_t *q, uint8_t *s, const kq_tuning *tuning, void *stream);

/* The launch shape the strip kernel of the MFMA quantizer (per-block factor
 * sets, or a shared set with an mfma_* override) takes for an [M, d] input on
 * the current device (adaln = 1: the AdaLN second pass), with the given
 * overrides (NULL: automatic, as kq_quantize and kq_transform_f32).  shape receives
 * {strip width in blocks, tiles per workgroup, interleaved (0/1), flat order
 * (0/1), grid size in workgroups, nontemporal code stores (0/1), register ring
 * depth in tiles}.  Queries the device (occupancy); launches nothing.  Same
 * argument errors as kq_quantize. */
int kq_launch_shape(int64_t M, int64_t d, int adaln, const kq_tuning *tuning, int64_t shape[7]);

/* The launch shape of the flat form, the MFMA quantizer's kernel for one
 * shared factor set (kq_quantize, kq_transform_f32, kq_quantize_lu and
 * kq_transform_lu_f32 with nT = 1 and no strip override), for an [M, d]
 * input on the current device with the given overrides (NULL: automatic).
 * shape receives {register ring depth in units of 32 blocks, workgroups of 4
 * waves, nontemporal code stores (0/1)}.  Queries the device; launches
 * nothing.  Same argument errors as kq_quantize. */
int kq_flat_launch_shape(int64_t M, int64_t d, const kq_tuning *tuning, int64_t shape[3]);

/* Copy kernels with the quantizer's 4:1 read:write footprint, timed by the
 * benchmark as the practical HBM ceiling: src_bytes of src are read (16-byte
 * loads) and src_bytes / 4 bytes of dst are written.  form 0 is the default
 * (the fastest form measured); other forms are the alternatives the benchmark
 * sweeps (1..KQ_COPY_FORMS-1).  src: dev, 16-byte aligned, src_bytes a
 * multiple of 1024; dst: dev, 16-byte aligned, not overlapping src.  One
 * launch on `stream`. */
#define KQ_COPY_FORMS 10
int kq_measure_copy41(const void *src, int64_t src_bytes, void *dst, int form, void *stream);

/* Text for a status code (static storage). */
const char *kq_status_string(int status);

/* Build description (target, variant defaults), static storage. */
const char *kq_build_info(void);

/* The hipError_t value behind the calling thread's most recent KQ_ERR_HIP
 * return (hipSuccess = 0 if there was none), and its name (static storage,
 * from the HIP runtime).  Neither call touches the GPU. */
int kq_last_hip_error(void);
const char *kq_hip_error_name(int code);

#ifdef __cplusplus
}
#endif

#endif /* KROQUANT_H */
