"""ctypes front end for the CPU oracle (``oracle/kq_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg are the only callers.  The product library never
imports this module.

Arrays are numpy arrays on the host.  bf16 activations are carried as their
raw uint16 bit patterns.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kq_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def build(force=True):
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(LIB_PATH):
        cmd = ["gcc", *GCC_FLAGS, "-o", LIB_PATH, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def bind(L):
    """Declare the C signatures on a loaded oracle library."""
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_to_double.restype = ctypes.c_double
    L.oracle_kron_block.argtypes = [P, P]
    L.oracle_kron_block.restype = None
    L.oracle_kron_block_inverse.argtypes = [P, P]
    L.oracle_kron_block_inverse.restype = ctypes.c_int
    L.oracle_e8m0_exponent.argtypes = [ctypes.c_float]
    L.oracle_e8m0_exponent.restype = ctypes.c_int
    L.oracle_fp4_code.argtypes = [ctypes.c_float, ctypes.c_int]
    L.oracle_fp4_code.restype = ctypes.c_int
    L.oracle_mx_block.argtypes = [P, P, P]
    L.oracle_mx_block.restype = None
    L.oracle_kq_transform.argtypes = [P, I64, I64, P, I64, P, P]
    L.oracle_kq_transform.restype = ctypes.c_int
    L.oracle_kq_quantize.argtypes = [P, I64, I64, P, I64, P, P, P]
    L.oracle_kq_quantize.restype = ctypes.c_int
    L.oracle_sq_quantize.argtypes = [P, I64, I64, P, P, P, P]
    L.oracle_sq_quantize.restype = ctypes.c_int
    L.oracle_mx_quantize_f32.argtypes = [P, I64, I64, P, P]
    L.oracle_mx_quantize_f32.restype = ctypes.c_int
    L.oracle_lu_factor.argtypes = [P, P]
    L.oracle_lu_factor.restype = None
    L.oracle_lu_kron_block.argtypes = [P, P]
    L.oracle_lu_kron_block.restype = None
    L.oracle_wht_block.argtypes = [P]
    L.oracle_wht_block.restype = None
    L.oracle_kq_transform_lu.argtypes = [P, I64, I64, P, I64, P, P]
    L.oracle_kq_transform_lu.restype = ctypes.c_int
    L.oracle_kq_quantize_lu.argtypes = [P, I64, I64, P, I64, P, P, P]
    L.oracle_kq_quantize_lu.restype = ctypes.c_int
    L.oracle_fwht_transform.argtypes = [P, I64, I64, P, P]
    L.oracle_fwht_transform.restype = ctypes.c_int
    L.oracle_fwht_quantize.argtypes = [P, I64, I64, P, P, P]
    L.oracle_fwht_quantize.restype = ctypes.c_int
    L.oracle_mx_value.argtypes = [ctypes.c_int, ctypes.c_int]
    L.oracle_mx_value.restype = ctypes.c_double
    L.oracle_mx_dequant.argtypes = [P, P, I64, I64, P]
    L.oracle_mx_dequant.restype = ctypes.c_int
    L.oracle_mx_gemm.argtypes = [P, P, I64, P, P, I64, I64, P, P]
    L.oracle_mx_gemm.restype = ctypes.c_int
    L.oracle_kron_block16.argtypes = [P, P]
    L.oracle_kron_block16.restype = None
    L.oracle_mx_block16.argtypes = [P, P, P]
    L.oracle_mx_block16.restype = None
    L.oracle_kq_transform16.argtypes = [P, I64, I64, P, I64, P, P]
    L.oracle_kq_transform16.restype = ctypes.c_int
    L.oracle_kq_quantize16.argtypes = [P, I64, I64, P, I64, P, P, P]
    L.oracle_kq_quantize16.restype = ctypes.c_int
    L.oracle_double_to_bf16.argtypes = [ctypes.c_double]
    L.oracle_double_to_bf16.restype = ctypes.c_uint16
    L.oracle_adaln.argtypes = [P, I64, I64, P, P, I64, ctypes.c_float, P, P, P]
    L.oracle_adaln.restype = ctypes.c_int
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = bind(ctypes.CDLL(LIB_PATH))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _u16(x):
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, "bf16 activations are passed as uint16 bit patterns"
    return x


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


class OracleError(RuntimeError):
    pass


def _check(st):
    if st != 0:
        raise OracleError(f"oracle returned status {st}")


def bf16_to_double(h):
    return lib().oracle_bf16_to_double(int(h))


def kron_block(f5):
    """Dense 32x32 block (float64) from one factor set ``f5`` of shape [5,2,2]."""
    f = _f32(f5).reshape(20)
    K = np.empty((32, 32), np.float64)
    lib().oracle_kron_block(_ptr(f), _ptr(K))
    return K


def kron_block_inverse(f5):
    f = _f32(f5).reshape(20)
    K = np.empty((32, 32), np.float64)
    _check(lib().oracle_kron_block_inverse(_ptr(f), _ptr(K)))
    return K


def e8m0_exponent(amax):
    return lib().oracle_e8m0_exponent(float(amax))


def fp4_code(y, E):
    return lib().oracle_fp4_code(float(y), int(E))


def mx_block(y32):
    y = _f32(y32).reshape(32)
    q = np.empty(16, np.uint8)
    s = np.empty(1, np.uint8)
    lib().oracle_mx_block(_ptr(y), _ptr(q), _ptr(s))
    return q, int(s[0])


def kq_transform(x_u16, factors, want_z=True):
    """Exact (float64) transformed values y and magnitudes z, both [M, d]."""
    x = _u16(x_u16)
    M, d = x.shape
    f = _f32(factors)
    nT = f.reshape(-1, 20).shape[0]
    y = np.empty((M, d), np.float64)
    z = np.empty((M, d), np.float64) if want_z else None
    _check(lib().oracle_kq_transform(_ptr(x), M, d, _ptr(f), nT, _ptr(y), _ptr(z)))
    return (y, z) if want_z else y


def kq_quantize(x_u16, factors, want_y32=False):
    x = _u16(x_u16)
    M, d = x.shape
    f = _f32(factors)
    nT = f.reshape(-1, 20).shape[0]
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 32), np.uint8)
    y32 = np.empty((M, d), np.float32) if want_y32 else None
    _check(lib().oracle_kq_quantize(_ptr(x), M, d, _ptr(f), nT, _ptr(q), _ptr(s), _ptr(y32)))
    return (q, s, y32) if want_y32 else (q, s)


def sq_quantize(x_u16, scale, want_y32=False):
    x = _u16(x_u16)
    M, d = x.shape
    sc = _f32(scale)
    assert sc.shape == (d,)
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 32), np.uint8)
    y32 = np.empty((M, d), np.float32) if want_y32 else None
    _check(lib().oracle_sq_quantize(_ptr(x), M, d, _ptr(sc), _ptr(q), _ptr(s), _ptr(y32)))
    return (q, s, y32) if want_y32 else (q, s)


def mx_quantize_f32(x_f32):
    x = _f32(x_f32)
    M, d = x.shape
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 32), np.uint8)
    _check(lib().oracle_mx_quantize_f32(_ptr(x), M, d, _ptr(q), _ptr(s)))
    return q, s


def lu_factor(abc):
    """One LU-form factor G = L U (2x2, float64) from its scalars (a, b, c)."""
    a = _f32(abc).reshape(3)
    G = np.empty((2, 2), np.float64)
    lib().oracle_lu_factor(_ptr(a), _ptr(G))
    return G


def lu_kron_block(lu5):
    """The 32x32 block (float64) of one LU-parameterised factor set [5, 3]."""
    f = _f32(lu5).reshape(15)
    K = np.empty((32, 32), np.float64)
    lib().oracle_lu_kron_block(_ptr(f), _ptr(K))
    return K


def wht_block():
    K = np.empty((32, 32), np.float64)
    lib().oracle_wht_block(_ptr(K))
    return K


def kq_transform_lu(x_u16, lu, want_z=True):
    x = _u16(x_u16)
    M, d = x.shape
    f = _f32(lu)
    nT = f.reshape(-1, 15).shape[0]
    y = np.empty((M, d), np.float64)
    z = np.empty((M, d), np.float64) if want_z else None
    _check(lib().oracle_kq_transform_lu(_ptr(x), M, d, _ptr(f), nT, _ptr(y), _ptr(z)))
    return (y, z) if want_z else y


def kq_quantize_lu(x_u16, lu, want_y32=False):
    x = _u16(x_u16)
    M, d = x.shape
    f = _f32(lu)
    nT = f.reshape(-1, 15).shape[0]
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 32), np.uint8)
    y32 = np.empty((M, d), np.float32) if want_y32 else None
    _check(lib().oracle_kq_quantize_lu(_ptr(x), M, d, _ptr(f), nT, _ptr(q), _ptr(s), _ptr(y32)))
    return (q, s, y32) if want_y32 else (q, s)


def fwht_transform(x_u16, want_z=True):
    x = _u16(x_u16)
    M, d = x.shape
    y = np.empty((M, d), np.float64)
    z = np.empty((M, d), np.float64) if want_z else None
    _check(lib().oracle_fwht_transform(_ptr(x), M, d, _ptr(y), _ptr(z)))
    return (y, z) if want_z else y


def fwht_quantize(x_u16, want_y32=False):
    x = _u16(x_u16)
    M, d = x.shape
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 32), np.uint8)
    y32 = np.empty((M, d), np.float32) if want_y32 else None
    _check(lib().oracle_fwht_quantize(_ptr(x), M, d, _ptr(q), _ptr(s), _ptr(y32)))
    return (q, s, y32) if want_y32 else (q, s)


def mx_value(code, sbyte):
    return lib().oracle_mx_value(int(code), int(sbyte))


def mx_dequant(q, s):
    """float64 values [M, K] of an MXFP4 matrix (q [M, K/2], s [M, K/32])."""
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    M, K = q.shape[0], q.shape[1] * 2
    out = np.empty((M, K), np.float64)
    _check(lib().oracle_mx_dequant(_ptr(q), _ptr(s), M, K, _ptr(out)))
    return out


def mx_gemm(qa, sa, qb, sb, want_mag=True):
    """A [M, K] times B [N, K]^T of two MXFP4 matrices, float64 (and sum |a b|)."""
    qa, sa = np.ascontiguousarray(qa, np.uint8), np.ascontiguousarray(sa, np.uint8)
    qb, sb = np.ascontiguousarray(qb, np.uint8), np.ascontiguousarray(sb, np.uint8)
    M, K = qa.shape[0], qa.shape[1] * 2
    N = qb.shape[0]
    assert qb.shape[1] * 2 == K
    out = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64) if want_mag else None
    _check(lib().oracle_mx_gemm(_ptr(qa), _ptr(sa), M, _ptr(qb), _ptr(sb), N, K, _ptr(out), _ptr(mag)))
    return (out, mag) if want_mag else out


def kron_block16(f4):
    """Dense 16x16 block (float64) from four 2x2 factors [4, 2, 2]."""
    f = _f32(f4).reshape(16)
    K = np.empty((16, 16), np.float64)
    lib().oracle_kron_block16(_ptr(f), _ptr(K))
    return K


def mx_block16(y16):
    y = _f32(y16).reshape(16)
    q = np.empty(8, np.uint8)
    s = np.empty(1, np.uint8)
    lib().oracle_mx_block16(_ptr(y), _ptr(q), _ptr(s))
    return q, int(s[0])


def kq_transform16(x_u16, factors, want_z=True):
    """16-element blocks, four factors per set [nT, 4, 2, 2]: y and z [M, d]."""
    x = _u16(x_u16)
    M, d = x.shape
    f = _f32(factors)
    nT = f.reshape(-1, 16).shape[0]
    y = np.empty((M, d), np.float64)
    z = np.empty((M, d), np.float64) if want_z else None
    _check(lib().oracle_kq_transform16(_ptr(x), M, d, _ptr(f), nT, _ptr(y), _ptr(z)))
    return (y, z) if want_z else y


def kq_quantize16(x_u16, factors, want_y32=False):
    """16-element blocks: codes [M, d/2], scales [M, d/16] (one per 16 elements)."""
    x = _u16(x_u16)
    M, d = x.shape
    f = _f32(factors)
    nT = f.reshape(-1, 16).shape[0]
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 16), np.uint8)
    y32 = np.empty((M, d), np.float32) if want_y32 else None
    _check(lib().oracle_kq_quantize16(_ptr(x), M, d, _ptr(f), nT, _ptr(q), _ptr(s), _ptr(y32)))
    return (q, s, y32) if want_y32 else (q, s)


def double_to_bf16(v):
    """bf16 bit pattern of a double, rounded to nearest, ties to even."""
    return int(lib().oracle_double_to_bf16(float(v)))


def adaln(h_u16, shift, scale, T, eps):
    """AdaLN front-end: x = LN(h) * (1 + scale[b]) + shift[b], b = m // T.
    Returns x (float64 [M, d]), x rounded to bf16 (uint16 bits) and the
    near-midpoint flags (bool [M, d])."""
    h = _u16(h_u16)
    M, d = h.shape
    sh = _f32(shift)
    sc = _f32(scale)
    nS = (M + T - 1) // T
    assert sh.shape == (max(nS, 0), d) and sc.shape == sh.shape
    x = np.empty((M, d), np.float64)
    xb = np.empty((M, d), np.uint16)
    fl = np.empty((M, d), np.uint8)
    _check(lib().oracle_adaln(_ptr(h), M, d, _ptr(sh), _ptr(sc), int(T), float(eps), _ptr(x), _ptr(xb), _ptr(fl)))
    return x, xb, fl.astype(bool)


def raw_status(fn_name, *args):
    """Call an oracle entry point with raw arguments and return its status code."""
    return getattr(lib(), fn_name)(*args)
