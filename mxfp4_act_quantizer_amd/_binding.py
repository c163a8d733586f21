"""ctypes binding of libkroquant.so: argument marshalling only.

Every computation runs in the library (HIP kernels on the GPU, or the C++
host helpers).  Device functions take torch tensors that already live on the
GPU and enqueue on the given stream (default: torch's current stream); they
return without synchronising.  There is no fallback: if the library is not
built, importing this module raises.
"""
import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkroquant.so")

KQ_OK = 0
KQ_ERR_ARG = 1
KQ_ERR_SHAPE = 2
KQ_ERR_ALIGN = 3
KQ_ERR_SINGULAR = 4
KQ_ERR_HIP = 5
KQ_ERR_OVERLAP = 6

KQ_VARIANT_AUTO = 0
KQ_VARIANT_MFMA = 1
KQ_VARIANT_BUTTERFLY = 2

# every symbol the public header declares
EXPORTS = (
    "kq_quantize", "kq_quantize_ex", "kq_transform_f32", "sq_quantize", "mx_quantize_f32",
    "kq_factor_inverse", "kq_block_matrix", "kq_block_inverse", "kq_fold_weight",
    "kq_quantize_lu", "kq_transform_lu_f32", "fwht_quantize", "fwht_transform_f32", "kq_lu_factors", "mx_gemm",
    "kq_adaln_quantize", "adaln_modulate", "kq_quantize16", "kq_transform16_f32", "kq_status_string",
    "kq_build_info", "kq_last_hip_error", "kq_hip_error_name",
    # measurement and test interface
    "kq_quantize_tuned", "kq_transform_tuned", "mx_gemm_tuned", "kq_adaln_quantize_tuned", "kq_launch_shape",
    "kq_flat_launch_shape",
    "kq_measure_copy41",
    # for callers that cannot allocate
    "kq_adaln_quantize_noalloc",
)
KQ_NOALLOC_MAX_ROWS = 131072
KQ_COPY_FORMS = 10

# launch-shape overrides (kq_tuning in kroquant.h); 0 keeps the automatic choice
TUNING_FIELDS = ("mfma_tiles_per_wg", "mfma_groups", "mfma_strip", "mfma_order", "code_stores",
                 "stream_rows_per_wave", "gemm_kernel", "adaln_pass", "adaln_strip", "adaln_blocks_per_wave",
                 "shared_form", "flat_wgs", "flat_ring", "mfma_ring")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python -m mxfp4_act_quantizer_amd.build` "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int


class Tuning(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in TUNING_FIELDS]


def _tuning(tuning):
    """A kq_tuning pointer from a dict of overrides (None: automatic)."""
    if not tuning:
        return None
    unknown = set(tuning) - set(TUNING_FIELDS)
    if unknown:
        raise ValueError(f"unknown tuning fields {sorted(unknown)}")
    return ctypes.byref(Tuning(**{k: int(v) for k, v in tuning.items()}))


_lib.kq_quantize.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, _P]
_lib.kq_quantize_ex.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, _INT, _P]
_lib.kq_transform_f32.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
_lib.kq_quantize_tuned.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, _INT, _P, _P]
_lib.kq_transform_tuned.argtypes = [_P, _I64, _I64, _P, _I64, _P, _INT, _P, _P]
_lib.mx_gemm_tuned.argtypes = [_P, _P, _I64, _P, _P, _I64, _I64, _P, _INT, _P, _P]
_lib.kq_adaln_quantize_tuned.argtypes = [_P, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _I64, _P, _P, _P, _P, _P]
_lib.kq_launch_shape.argtypes = [_I64, _I64, _INT, _P, _P]
_lib.kq_flat_launch_shape.argtypes = [_I64, _I64, _P, _P]
_lib.sq_quantize.argtypes = [_P, _I64, _I64, _P, _P, _P, _P]
_lib.mx_quantize_f32.argtypes = [_P, _I64, _I64, _P, _P, _P]
_lib.kq_quantize_lu.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, _P]
_lib.kq_transform_lu_f32.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
_lib.fwht_quantize.argtypes = [_P, _I64, _I64, _P, _P, _P]
_lib.fwht_transform_f32.argtypes = [_P, _I64, _I64, _P, _P]
_lib.kq_lu_factors.argtypes = [_P, _I64, _P]
_lib.mx_gemm.argtypes = [_P, _P, _I64, _P, _P, _I64, _I64, _P, _INT, _P]
_lib.kq_quantize16.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P, _P]
_lib.kq_transform16_f32.argtypes = [_P, _I64, _I64, _P, _I64, _P, _P]
_lib.kq_adaln_quantize.argtypes = [_P, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _I64, _P, _P, _P, _P]
_lib.kq_adaln_quantize_noalloc.argtypes = [_P, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _I64, _P, _P, _P]
_lib.adaln_modulate.argtypes = [_P, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _P, _P]
_lib.kq_factor_inverse.argtypes = [_P, _I64, _P]
_lib.kq_block_matrix.argtypes = [_P, _I64, _P]
_lib.kq_block_inverse.argtypes = [_P, _I64, _P]
_lib.kq_fold_weight.argtypes = [_P, _I64, _I64, _P, _I64, _P]
_lib.kq_status_string.argtypes = [_INT]
_lib.kq_status_string.restype = ctypes.c_char_p
_lib.kq_build_info.argtypes = []
_lib.kq_build_info.restype = ctypes.c_char_p
_lib.kq_last_hip_error.argtypes = []
_lib.kq_hip_error_name.argtypes = [_INT]
_lib.kq_hip_error_name.restype = ctypes.c_char_p
_lib.kq_measure_copy41.argtypes = [_P, _I64, _P, _INT, _P]
for _name in EXPORTS:
    if _name not in ("kq_status_string", "kq_build_info", "kq_hip_error_name"):
        getattr(_lib, _name).restype = _INT


class KQError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = f"{where}: {kq_status_string(status)} (status {status})"
        if status == KQ_ERR_HIP:
            self.hip_error = _lib.kq_last_hip_error()
            msg += f": {_lib.kq_hip_error_name(self.hip_error).decode()} ({self.hip_error})"
        super().__init__(msg)


def kq_status_string(status):
    return _lib.kq_status_string(int(status)).decode()


def kq_build_info():
    return _lib.kq_build_info().decode()


def lib():
    """The loaded ctypes library (raw C entry points)."""
    return _lib


def _check(st, where):
    if st != KQ_OK:
        raise KQError(st, where)


# ---------------------------------------------------------------------------
# device entry points (torch tensors on the GPU)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_handle(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtypes, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def _outputs(x, M, d, q, s):
    torch = _torch()
    if q is None:
        q = torch.empty((M, d // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((M, d // 32), dtype=torch.uint8, device=x.device)
    return q, s


def _md(x):
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, d]")
    return int(x.shape[0]), int(x.shape[1])


def _nT(factors):
    n = factors.numel()
    if n % 20:
        raise ValueError("factors must hold [nT, 5, 2, 2] float32 values")
    return n // 20


def kq_quantize(x, factors, q=None, s=None, stream=None, variant=KQ_VARIANT_AUTO, tuning=None):
    """KroQuant quantizer: returns (q [M, d/2] u8, s [M, d/32] u8).  `tuning`
    (a dict of kq_tuning fields) pins the launch shape, for measurements."""
    torch = _torch()
    M, d = _md(x)
    q, s = _outputs(x, M, d, q, s)
    args = (_dev(x, _bf16_types(), "x"), M, d, _dev(factors, (torch.float32,), "factors"), _nT(factors),
            _dev(q, (torch.uint8,), "q"), _dev(s, (torch.uint8,), "s"))
    if tuning:
        st = _lib.kq_quantize_tuned(*args, int(variant), _tuning(tuning), _stream_handle(stream))
    elif variant == KQ_VARIANT_AUTO:
        st = _lib.kq_quantize(*args, _stream_handle(stream))
    else:
        st = _lib.kq_quantize_ex(*args, int(variant), _stream_handle(stream))
    _check(st, "kq_quantize")
    return q, s


def kq_quantize_ex(x, factors, q, s, variant, stream=None):
    return kq_quantize(x, factors, q, s, stream, variant)


def kq_transform_f32(x, factors, y=None, stream=None, variant=KQ_VARIANT_AUTO, tuning=None):
    """Transformed values y = x_blk . K_j (fp32) as the quantizer computes them."""
    torch = _torch()
    M, d = _md(x)
    if y is None:
        y = torch.empty((M, d), dtype=torch.float32, device=x.device)
    args = (_dev(x, _bf16_types(), "x"), M, d, _dev(factors, (torch.float32,), "factors"), _nT(factors),
            _dev(y, (torch.float32,), "y"))
    if tuning or variant != KQ_VARIANT_AUTO:
        st = _lib.kq_transform_tuned(*args, int(variant), _tuning(tuning), _stream_handle(stream))
    else:
        st = _lib.kq_transform_f32(*args, _stream_handle(stream))
    _check(st, "kq_transform_f32")
    return y


def kq_launch_shape(M, d, adaln=False, tuning=None):
    """Launch shape of the MFMA quantizer for [M, d] on the current device:
    dict of strip, tiles_per_wg, interleave, flat, grid, nt_codes, ring."""
    out = (ctypes.c_int64 * 7)()
    _check(_lib.kq_launch_shape(int(M), int(d), 1 if adaln else 0, _tuning(tuning), out), "kq_launch_shape")
    return dict(zip(("strip", "tiles_per_wg", "interleave", "flat", "grid", "nt_codes", "ring"),
                    (int(v) for v in out)))


def kq_flat_launch_shape(M, d, tuning=None):
    """Launch shape of the flat form (one shared factor set) for [M, d] on the
    current device: dict of ring, workgroups, nt_codes."""
    out = (ctypes.c_int64 * 3)()
    _check(_lib.kq_flat_launch_shape(int(M), int(d), _tuning(tuning), out), "kq_flat_launch_shape")
    return dict(zip(("ring", "workgroups", "nt_codes"), (int(v) for v in out)))


def _nT_lu(lu):
    n = lu.numel()
    if n % 15:
        raise ValueError("lu must hold [nT, 5, 3] float32 values")
    return n // 15


def kq_quantize_lu(x, lu, q=None, s=None, stream=None):
    """K2 form of the KroQuant quantizer: factor sets as LU scalars [nT, 5, 3]."""
    torch = _torch()
    M, d = _md(x)
    q, s = _outputs(x, M, d, q, s)
    st = _lib.kq_quantize_lu(_dev(x, _bf16_types(), "x"), M, d, _dev(lu, (torch.float32,), "lu"), _nT_lu(lu),
                             _dev(q, (torch.uint8,), "q"), _dev(s, (torch.uint8,), "s"), _stream_handle(stream))
    _check(st, "kq_quantize_lu")
    return q, s


def kq_transform_lu_f32(x, lu, y=None, stream=None):
    torch = _torch()
    M, d = _md(x)
    if y is None:
        y = torch.empty((M, d), dtype=torch.float32, device=x.device)
    st = _lib.kq_transform_lu_f32(_dev(x, _bf16_types(), "x"), M, d, _dev(lu, (torch.float32,), "lu"), _nT_lu(lu),
                                  _dev(y, (torch.float32,), "y"), _stream_handle(stream))
    _check(st, "kq_transform_lu_f32")
    return y


def fwht_quantize(x, q=None, s=None, stream=None):
    """Walsh-Hadamard-32 comparison quantizer (fixed transform, then MXFP4)."""
    torch = _torch()
    M, d = _md(x)
    q, s = _outputs(x, M, d, q, s)
    st = _lib.fwht_quantize(_dev(x, _bf16_types(), "x"), M, d, _dev(q, (torch.uint8,), "q"),
                            _dev(s, (torch.uint8,), "s"), _stream_handle(stream))
    _check(st, "fwht_quantize")
    return q, s


def fwht_transform_f32(x, y=None, stream=None):
    torch = _torch()
    M, d = _md(x)
    if y is None:
        y = torch.empty((M, d), dtype=torch.float32, device=x.device)
    st = _lib.fwht_transform_f32(_dev(x, _bf16_types(), "x"), M, d, _dev(y, (torch.float32,), "y"),
                                 _stream_handle(stream))
    _check(st, "fwht_transform_f32")
    return y


def mx_gemm(qa, sa, qb, sb, out=None, out_dtype=None, stream=None, tuning=None):
    """W4A4 product out = A . B^T of two MXFP4 matrices (codes [rows, K/2] u8,
    scales [rows, K/32] u8), accumulated in fp32; out float32 or bfloat16."""
    torch = _torch()
    M, K = int(qa.shape[0]), int(qa.shape[1]) * 2
    N = int(qb.shape[0])
    if int(qb.shape[1]) * 2 != K or sa.shape != (M, K // 32) or sb.shape != (N, K // 32):
        raise ValueError("operand shapes do not match")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=qa.device)
    bf = 1 if out.dtype == torch.bfloat16 else 0
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (M, N):
        raise ValueError("out must be float32 or bfloat16 [M, N]")
    u8 = (torch.uint8,)
    args = (_dev(qa, u8, "qa"), _dev(sa, u8, "sa"), M, _dev(qb, u8, "qb"), _dev(sb, u8, "sb"), N, K,
            _dev(out, (torch.float32, torch.bfloat16), "out"), bf)
    if tuning:
        st = _lib.mx_gemm_tuned(*args, _tuning(tuning), _stream_handle(stream))
    else:
        st = _lib.mx_gemm(*args, _stream_handle(stream))
    _check(st, "mx_gemm")
    return out


def sq_quantize(x, scale, q=None, s=None, stream=None):
    """SmoothQuant comparison quantizer: y = x * fl32(1/scale_c), then MXFP4."""
    torch = _torch()
    M, d = _md(x)
    q, s = _outputs(x, M, d, q, s)
    st = _lib.sq_quantize(_dev(x, _bf16_types(), "x"), M, d, _dev(scale, (torch.float32,), "scale"),
                          _dev(q, (torch.uint8,), "q"), _dev(s, (torch.uint8,), "s"), _stream_handle(stream))
    _check(st, "sq_quantize")
    return q, s


def mx_quantize_f32(x, q=None, s=None, stream=None):
    """Plain MXFP4 quantization of an fp32 matrix."""
    torch = _torch()
    M, d = _md(x)
    q, s = _outputs(x, M, d, q, s)
    st = _lib.mx_quantize_f32(_dev(x, (torch.float32,), "x"), M, d, _dev(q, (torch.uint8,), "q"),
                              _dev(s, (torch.uint8,), "s"), _stream_handle(stream))
    _check(st, "mx_quantize_f32")
    return q, s


def _nT16(factors):
    n = factors.numel()
    if n % 16:
        raise ValueError("factors must hold [nT, 4, 2, 2] float32 values")
    return n // 16


def kq_quantize16(x, factors, q=None, s=None, stream=None):
    """16-element blocks with four factors per set [nT, 4, 2, 2]: returns
    (q [M, d/2] u8, s [M, d/16] u8)."""
    torch = _torch()
    M, d = _md(x)
    if q is None:
        q = torch.empty((M, d // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((M, d // 16), dtype=torch.uint8, device=x.device)
    st = _lib.kq_quantize16(_dev(x, _bf16_types(), "x"), M, d, _dev(factors, (torch.float32,), "factors"),
                            _nT16(factors), _dev(q, (torch.uint8,), "q"), _dev(s, (torch.uint8,), "s"),
                            _stream_handle(stream))
    _check(st, "kq_quantize16")
    return q, s


def kq_transform16_f32(x, factors, y=None, stream=None):
    """The transformed values of kq_quantize16 (fp32 [M, d])."""
    torch = _torch()
    M, d = _md(x)
    if y is None:
        y = torch.empty((M, d), dtype=torch.float32, device=x.device)
    st = _lib.kq_transform16_f32(_dev(x, _bf16_types(), "x"), M, d, _dev(factors, (torch.float32,), "factors"),
                                 _nT16(factors), _dev(y, (torch.float32,), "y"), _stream_handle(stream))
    _check(st, "kq_transform16_f32")
    return y


def _stats(h, M, stats):
    torch = _torch()
    if stats is None:
        stats = torch.empty((M, 2), dtype=torch.float64, device=h.device)
    return stats


def kq_adaln_quantize(h, shift, scale, tokens_per_sample, eps, factors, q=None, s=None, stats=None, stream=None,
                      tuning=None):
    """AdaLN front-end fused with the quantizer: x = LN(h) (1 + scale[b]) +
    shift[b] (b = row // tokens_per_sample) rounded to bf16, then the
    Kronecker transform and MXFP4.  `stats` is the [M, 2] float64 workspace
    (allocated here when not given).  Returns (q, s)."""
    torch = _torch()
    M, d = _md(h)
    q, s = _outputs(h, M, d, q, s)
    stats = _stats(h, M, stats)
    args = (_dev(h, _bf16_types(), "h"), M, d, _dev(shift, (torch.float32,), "shift"),
            _dev(scale, (torch.float32,), "scale"), int(tokens_per_sample), float(eps),
            _dev(factors, (torch.float32,), "factors"), _nT(factors), _dev(stats, (torch.float64,), "stats"),
            _dev(q, (torch.uint8,), "q"), _dev(s, (torch.uint8,), "s"))
    if tuning:
        st = _lib.kq_adaln_quantize_tuned(*args, _tuning(tuning), _stream_handle(stream))
    else:
        st = _lib.kq_adaln_quantize(*args, _stream_handle(stream))
    _check(st, "kq_adaln_quantize")
    return q, s


def kq_adaln_quantize_noalloc(h, shift, scale, tokens_per_sample, eps, factors, q, s, stream=None):
    """kq_adaln_quantize with the library's own fixed row-statistics array
    (at most KQ_NOALLOC_MAX_ROWS rows; calls overlapping in time on one GPU
    race on it): q and s are the caller's, nothing is allocated."""
    torch = _torch()
    M, d = _md(h)
    st = _lib.kq_adaln_quantize_noalloc(_dev(h, _bf16_types(), "h"), M, d, _dev(shift, (torch.float32,), "shift"),
                                        _dev(scale, (torch.float32,), "scale"), int(tokens_per_sample), float(eps),
                                        _dev(factors, (torch.float32,), "factors"), _nT(factors),
                                        _dev(q, (torch.uint8,), "q"), _dev(s, (torch.uint8,), "s"),
                                        _stream_handle(stream))
    _check(st, "kq_adaln_quantize_noalloc")
    return q, s


def adaln_modulate(h, shift, scale, tokens_per_sample, eps, x=None, stats=None, stream=None):
    """The AdaLN front-end alone: x (bf16 [M, d]) as kq_adaln_quantize computes it."""
    torch = _torch()
    M, d = _md(h)
    if x is None:
        x = torch.empty((M, d), dtype=torch.bfloat16, device=h.device)
    stats = _stats(h, M, stats)
    st = _lib.adaln_modulate(_dev(h, _bf16_types(), "h"), M, d, _dev(shift, (torch.float32,), "shift"),
                             _dev(scale, (torch.float32,), "scale"), int(tokens_per_sample), float(eps),
                             _dev(stats, (torch.float64,), "stats"), _dev(x, _bf16_types(), "x"),
                             _stream_handle(stream))
    _check(st, "adaln_modulate")
    return x


def measure_copy41(src, dst, form=0, stream=None):
    """Measurement only: a streaming copy with the quantizer's 4:1 footprint
    (reads all of src, writes src.nbytes / 4 bytes of dst), the benchmark's
    HBM ceiling; `form` picks one of the KQ_COPY_FORMS copy forms."""
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous GPU tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes // 4:
        raise ValueError("dst must hold src.nbytes / 4 bytes")
    _check(_lib.kq_measure_copy41(src.data_ptr(), nbytes, dst.data_ptr(), int(form), _stream_handle(stream)),
           "kq_measure_copy41")


# ---------------------------------------------------------------------------
# host helpers (numpy arrays, synchronous)
# ---------------------------------------------------------------------------
def _host_f32(a, name):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def kq_lu_factors(lu):
    """2x2 factors [nT, 5, 2, 2] of LU scalars [nT, 5, 3], in the kernel's fp32 arithmetic."""
    f = _host_f32(lu, "lu")
    if f.size % 15:
        raise ValueError("lu must hold [nT, 5, 3] float32 values")
    nT = f.size // 15
    out = np.empty((nT, 5, 2, 2), np.float32)
    _check(_lib.kq_lu_factors(f.ctypes.data, nT, out.ctypes.data), "kq_lu_factors")
    return out


def kq_factor_inverse(factors):
    f = _host_f32(factors, "factors")
    nT = f.size // 20
    out = np.empty((nT, 5, 2, 2), np.float32)
    _check(_lib.kq_factor_inverse(f.ctypes.data, nT, out.ctypes.data), "kq_factor_inverse")
    return out


def kq_block_matrix(factors):
    f = _host_f32(factors, "factors")
    nT = f.size // 20
    out = np.empty((nT, 32, 32), np.float32)
    _check(_lib.kq_block_matrix(f.ctypes.data, nT, out.ctypes.data), "kq_block_matrix")
    return out


def kq_block_inverse(factors):
    f = _host_f32(factors, "factors")
    nT = f.size // 20
    out = np.empty((nT, 32, 32), np.float32)
    _check(_lib.kq_block_inverse(f.ctypes.data, nT, out.ctypes.data), "kq_block_inverse")
    return out


def kq_fold_weight(W, factors):
    """W_out = W . T^-T so that (X T) W_out^T = X W^T."""
    w = _host_f32(W, "W")
    f = _host_f32(factors, "factors")
    N, d = w.shape
    out = np.empty_like(w)
    _check(_lib.kq_fold_weight(w.ctypes.data, N, d, f.ctypes.data, f.size // 20, out.ctypes.data), "kq_fold_weight")
    return out
