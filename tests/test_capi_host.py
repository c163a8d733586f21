"""CPU-side checks of the C-ABI library: it loads, exports every declared
symbol, rejects bad arguments before touching the GPU, and its host helpers
(T^-1, dense blocks, weight folding) agree with the oracle."""
import os
import re

import numpy as np
import pytest
import scipy.linalg

import mxfp4_act_quantizer_amd as K
from synth import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kroquant.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kq_\w+|sq_\w+|mx_\w+|fwht_\w+|adaln_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11, names
    L = K.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in kroquant.h but not exported"
    assert set(names) == set(K.EXPORTS)


def test_library_is_the_in_tree_build():
    assert os.path.dirname(K.LIB_PATH) == os.path.join(ROOT, "mxfp4_act_quantizer_amd")
    assert "gfx950" in K.kq_build_info()


def test_library_is_built_from_the_current_sources():
    # the library carries the hash of the sources it was compiled from; a
    # stale build (sources changed since) fails here
    from mxfp4_act_quantizer_amd import build as B
    assert K.kq_build_info().endswith("sources " + B.source_hash()), (K.kq_build_info(), B.source_hash())


def test_status_strings():
    for st in range(7):
        assert K.kq_status_string(st) != "unknown status"
    assert K.kq_status_string(99) == "unknown status"


def test_copy_ceiling_validation():
    # the benchmark's measurement copies check their arguments before any HIP call
    L = K.lib()
    assert L.kq_measure_copy41(FAKE, 0, FAKE + (1 << 30), 0, None) == K.KQ_OK
    assert L.kq_measure_copy41(None, 1024, FAKE, 0, None) == K.KQ_ERR_ARG
    assert L.kq_measure_copy41(FAKE, 1000, FAKE + (1 << 30), 0, None) == K.KQ_ERR_ARG
    assert L.kq_measure_copy41(FAKE, 1024, FAKE + (1 << 30), -1, None) == K.KQ_ERR_ARG
    assert L.kq_measure_copy41(FAKE, 1024, FAKE + (1 << 30), K.KQ_COPY_FORMS, None) == K.KQ_ERR_ARG
    assert L.kq_measure_copy41(FAKE + 4, 1024, FAKE + (1 << 30), 0, None) == K.KQ_ERR_ALIGN
    assert L.kq_measure_copy41(FAKE, 1024, FAKE + (1 << 30) + 4, 0, None) == K.KQ_ERR_ALIGN
    assert L.kq_measure_copy41(FAKE, 1024, FAKE + 32, 0, None) == K.KQ_ERR_OVERLAP


def test_hip_error_detail_without_gpu():
    # a thread that saw no KQ_ERR_HIP return reports hipSuccess; names come from the runtime
    import threading
    seen = []
    t = threading.Thread(target=lambda: seen.append(K.lib().kq_last_hip_error()))
    t.start()
    t.join()
    assert seen == [0]
    assert K.lib().kq_hip_error_name(0) == b"hipSuccess"
    assert K.lib().kq_hip_error_name(98) == b"hipErrorInvalidDeviceFunction"


# ---------------------------------------------------------------------------
# argument checks: every one returns before any HIP call
# ---------------------------------------------------------------------------
FAKE = 1 << 40  # never dereferenced: every call below fails validation first


def raw(name, *args):
    return getattr(K.lib(), name)(*args)


def test_kq_validation():
    q, s, f, x = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    assert raw("kq_quantize", x, 4, 48, f, 1, q, s, None) == K.KQ_ERR_SHAPE  # d % 32
    assert raw("kq_quantize", x, 4, 64, f, 3, q, s, None) == K.KQ_ERR_SHAPE  # nT
    assert raw("kq_quantize", x, -1, 64, f, 1, q, s, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize", x, 4, 0, f, 1, q, s, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize", None, 4, 64, f, 1, q, s, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize", x, 4, 64, None, 1, q, s, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize", x, 4, 64, f, 1, None, s, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize", x, 4, 64, f, 1, q, None, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize", x + 2, 4, 64, f, 1, q, s, None) == K.KQ_ERR_ALIGN
    assert raw("kq_quantize", x, 4, 64, f, 1, q + 8, s, None) == K.KQ_ERR_ALIGN
    assert raw("kq_quantize", x, 4, 64, f + 2, 1, q, s, None) == K.KQ_ERR_ALIGN
    assert raw("kq_quantize", x, 4, 64, f, 1, x + 64, s, None) == K.KQ_ERR_OVERLAP  # q inside x
    assert raw("kq_quantize", x, 4, 64, f, 1, q, q + 16, None) == K.KQ_ERR_OVERLAP  # s inside q
    assert raw("kq_quantize", x, 4, 64, q + 32, 1, q, s, None) == K.KQ_ERR_OVERLAP  # factors inside q
    assert raw("kq_quantize_ex", x, 4, 64, f, 1, q, s, 7, None) == K.KQ_ERR_ARG  # variant
    assert raw("kq_quantize", x, 0, 64, f, 1, q, s, None) == K.KQ_OK  # empty: no launch
    assert raw("kq_quantize", None, 0, 64, None, 1, None, None, None) == K.KQ_OK
    assert raw("kq_quantize", x, 4, 64 << 20, f, 1, q, s, None) == K.KQ_ERR_SHAPE  # too wide


def test_transform_and_sq_mx_validation():
    y, f, x, sc = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    q, s = FAKE + (4 << 30), FAKE + (5 << 30)
    assert raw("kq_transform_f32", x, 4, 64, f, 2, y + 4, None) == K.KQ_ERR_ALIGN
    assert raw("kq_transform_f32", x, 4, 64, f, 5, y, None) == K.KQ_ERR_SHAPE
    assert raw("kq_transform_f32", x, 4, 64, f, 2, x + 16, None) == K.KQ_ERR_OVERLAP
    assert raw("kq_transform_tuned", x, 4, 64, f, 2, y, 9, None, None) == K.KQ_ERR_ARG  # variant
    assert raw("kq_transform_tuned", x, 4, 64, f, 2, y + 4, 1, None, None) == K.KQ_ERR_ALIGN
    assert raw("sq_quantize", x, 4, 96, None, q, s, None) == K.KQ_ERR_ARG
    assert raw("sq_quantize", x, 4, 96, sc + 1, q, s, None) == K.KQ_ERR_ALIGN
    assert raw("sq_quantize", x, 4, 100, sc, q, s, None) == K.KQ_ERR_SHAPE
    assert raw("sq_quantize", x, 0, 96, sc, q, s, None) == K.KQ_OK
    assert raw("mx_quantize_f32", x + 8, 4, 64, q, s, None) == K.KQ_ERR_ALIGN
    assert raw("mx_quantize_f32", x, 4, 64, x + 32, s, None) == K.KQ_ERR_OVERLAP
    assert raw("mx_quantize_f32", x, -2, 64, q, s, None) == K.KQ_ERR_ARG


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        K.kq_quantize(x, torch.zeros(20))


# ---------------------------------------------------------------------------
# host helpers against the oracle
# ---------------------------------------------------------------------------
def test_block_matrix_and_inverse_match_oracle(oracle_lib):
    f = I.random_factors(4, 17)
    Kd = K.kq_block_matrix(f)
    Ki = K.kq_block_inverse(f)
    for t in range(4):
        Kref = oracle_lib.kron_block(f[t])
        Kiref = oracle_lib.kron_block_inverse(f[t])
        assert np.allclose(Kd[t], Kref, rtol=2 ** -23, atol=0)
        assert np.allclose(Ki[t], Kiref, rtol=2 ** -22, atol=1e-7 * np.abs(Kiref).max())
        cond = np.linalg.cond(Kref)
        assert np.abs(Ki[t].astype(np.float64) @ Kref - np.eye(32)).max() < 1e-6 * cond


def test_factor_inverse(oracle_lib):
    f = I.random_factors(3, 18)
    inv = K.kq_factor_inverse(f)
    for t in range(3):
        for k in range(5):
            assert np.allclose(inv[t, k].astype(np.float64) @ f[t, k].astype(np.float64), np.eye(2), atol=1e-6)


def test_singular_factor_reported():
    f = I.identity_factors(2)
    f[1, 3] = np.array([[1, 2], [2, 4]], np.float32)
    with pytest.raises(K.KQError) as e:
        K.kq_block_inverse(f)
    assert e.value.status == K.KQ_ERR_SINGULAR
    f[1, 3] = np.array([[np.nan, 0], [0, 1]], np.float32)
    with pytest.raises(K.KQError):
        K.kq_factor_inverse(f)


@pytest.mark.parametrize("shared", [True, False])
def test_fold_weight_exact_invariance(oracle_lib, shared):
    """(X T)(W_out)^T == X W^T exactly with integer unimodular factors."""
    rng = np.random.default_rng(5)
    M, d, N = 6, 160, 7
    f = I.integer_unimodular_factors(1 if shared else d // 32, 6)
    x_int = rng.integers(-4, 5, (M, d)).astype(np.float32)
    W = rng.integers(-4, 5, (N, d)).astype(np.float32)
    Wf = K.kq_fold_weight(W, f)
    y = oracle_lib.kq_transform(I.f32_to_bf16_bits(x_int), f, want_z=False)
    assert np.array_equal(y @ Wf.astype(np.float64).T, x_int.astype(np.float64) @ W.astype(np.float64).T)


def test_fold_weight_real_factors(oracle_lib):
    rng = np.random.default_rng(7)
    M, d, N = 5, 128, 9
    f = I.random_factors(d // 32, 8)
    x = I.make_activation("tiny", M=M, d=d)
    W = rng.standard_normal((N, d)).astype(np.float32)
    Wf = K.kq_fold_weight(W, f)
    y = oracle_lib.kq_transform(x, f, want_z=False)
    Tinv = scipy.linalg.block_diag(*[oracle_lib.kron_block_inverse(f[j]) for j in range(d // 32)])
    ref = W.astype(np.float64) @ Tinv.T
    assert np.allclose(Wf, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())
    lhs = y @ Wf.astype(np.float64).T
    rhs = I.bf16_bits_to_f32(x).astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-4 * np.abs(rhs).max())


def test_fold_weight_in_place():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((3, 64)).astype(np.float32)
    f = I.random_factors(2, 10)
    ref = K.kq_fold_weight(W, f)
    L = K.lib()
    Wc = W.copy()
    fc = np.ascontiguousarray(f)
    assert L.kq_fold_weight(Wc.ctypes.data, 3, 64, fc.ctypes.data, 2, Wc.ctypes.data) == 0
    assert np.array_equal(Wc, ref)


def test_fold_weight_shape_errors():
    L = K.lib()
    W = np.zeros((2, 64), np.float32)
    f = np.ascontiguousarray(I.identity_factors(3))
    assert L.kq_fold_weight(W.ctypes.data, 2, 64, f.ctypes.data, 3, W.ctypes.data) == K.KQ_ERR_SHAPE
    assert L.kq_fold_weight(W.ctypes.data, 2, 60, f.ctypes.data, 1, W.ctypes.data) == K.KQ_ERR_SHAPE
    assert L.kq_fold_weight(None, 2, 64, f.ctypes.data, 1, W.ctypes.data) == K.KQ_ERR_ARG


# ---------------------------------------------------------------------------
# K2 (LU scalars) and Walsh-Hadamard comparison entry points
# ---------------------------------------------------------------------------
def test_lu_and_fwht_validation():
    q, s, f, x = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30)
    y = FAKE + (4 << 30)
    assert raw("kq_quantize_lu", x, 4, 48, f, 1, q, s, None) == K.KQ_ERR_SHAPE
    assert raw("kq_quantize_lu", x, 4, 64, f, 3, q, s, None) == K.KQ_ERR_SHAPE
    assert raw("kq_quantize_lu", x, 4, 64, None, 1, q, s, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize_lu", x, 4, 64, f + 2, 1, q, s, None) == K.KQ_ERR_ALIGN
    assert raw("kq_quantize_lu", x, 4, 64, q + 32, 1, q, s, None) == K.KQ_ERR_OVERLAP
    assert raw("kq_quantize_lu", x, 0, 64, None, 1, None, None, None) == K.KQ_OK
    assert raw("kq_transform_lu_f32", x, 4, 64, f, 2, None, None) == K.KQ_ERR_ARG
    assert raw("kq_transform_lu_f32", x, 4, 64, f, 2, y + 4, None) == K.KQ_ERR_ALIGN
    assert raw("kq_transform_lu_f32", x, 4, 64, f, 2, x + 64, None) == K.KQ_ERR_OVERLAP
    assert raw("fwht_quantize", x, 4, 40, q, s, None) == K.KQ_ERR_SHAPE
    assert raw("fwht_quantize", None, 4, 64, q, s, None) == K.KQ_ERR_ARG
    assert raw("fwht_quantize", x + 2, 4, 64, q, s, None) == K.KQ_ERR_ALIGN
    assert raw("fwht_quantize", x, 4, 64, x + 32, s, None) == K.KQ_ERR_OVERLAP
    assert raw("fwht_quantize", x, 0, 64, None, None, None) == K.KQ_OK
    assert raw("fwht_transform_f32", x, 4, 64, None, None) == K.KQ_ERR_ARG
    assert raw("fwht_transform_f32", x, 4, 64, y + 8, None) == K.KQ_ERR_ALIGN


def test_lu_factors_match_oracle_factor(oracle_lib):
    lu = np.concatenate([I.random_lu(6, 23), I.hadamard_lu(1),
                         np.array([[[1, 2, -1], [-1, 0, 1], [1, 1, 1], [1, -1, 2], [-1, 1, 0]]], np.float32)])
    g = K.kq_lu_factors(lu)
    assert g.shape == (lu.shape[0], 5, 2, 2) and g.dtype == np.float32
    for t in range(lu.shape[0]):
        for k in range(5):
            a, b, c = (np.float32(v) for v in lu[t, k])
            G = oracle_lib.lu_factor(lu[t, k])
            # entries the fp32 sequence forms exactly: a, b and fl32(c a)
            assert g[t, k, 0, 0] == a and g[t, k, 0, 1] == b
            assert g[t, k, 1, 0] == np.float32(G[1, 0])
            # c b - fl32(1/a), rounded once: within half an fp32 ulp of the double value
            r = np.float32(1.0) / a
            exact = float(c) * float(b) - float(r)
            assert abs(float(g[t, k, 1, 1]) - exact) <= 0.5 * float(np.spacing(np.float32(abs(exact)))) + 1e-300
            # and close to the oracle's double-precision factor (differs only by fl32(1/a))
            assert abs(float(g[t, k, 1, 1]) - G[1, 1]) <= 2 ** -22 * max(1.0, abs(G[1, 1]))
    # the Hadamard initialisation gives the fp32 Hadamard factor up to one ulp of -1/sqrt 2
    h = K.kq_lu_factors(I.hadamard_lu(1))[0]
    assert np.abs(h - I.hadamard_factors(1)[0]).max() <= np.spacing(np.float32(0.70710677))


def test_lu_factors_singular():
    bad = I.hadamard_lu(2)
    bad[1, 3, 0] = 0.0
    with pytest.raises(K.KQError) as e:
        K.kq_lu_factors(bad)
    assert e.value.status == K.KQ_ERR_SINGULAR
    bad[1, 3, 0] = np.inf
    with pytest.raises(K.KQError):
        K.kq_lu_factors(bad)


def test_fold_weight_through_lu_factors(oracle_lib):
    # K2 users fold their weights with the factors kq_lu_factors forms
    rng = np.random.default_rng(29)
    M, d, N = 4, 96, 5
    lu = I.random_lu(d // 32, 31)
    f = K.kq_lu_factors(lu)
    x = I.act_gaussian_outliers(M, d, 37, 1, 10.0)[0]
    W = rng.standard_normal((N, d)).astype(np.float32)
    Wf = K.kq_fold_weight(W, f)
    y = oracle_lib.kq_transform(x, f, want_z=False)
    ref = I.bf16_bits_to_f32(x).astype(np.float64) @ W.astype(np.float64).T
    got = y @ Wf.astype(np.float64).T
    assert np.allclose(got, ref, rtol=0, atol=1e-4 * np.abs(ref).max())


def test_mx_gemm_validation():
    qa, sa, qb, sb, out = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30)
    assert raw("mx_gemm", qa, sa, 4, qb, sb, 4, 48, out, 0, None) == K.KQ_ERR_SHAPE  # K % 32
    assert raw("mx_gemm", qa, sa, 4, qb, sb, 4, 0, out, 0, None) == K.KQ_ERR_ARG
    assert raw("mx_gemm", qa, sa, -1, qb, sb, 4, 64, out, 0, None) == K.KQ_ERR_ARG
    assert raw("mx_gemm", qa, sa, 4, qb, sb, 4, 64, out, 2, None) == K.KQ_ERR_ARG  # out type
    assert raw("mx_gemm", None, sa, 4, qb, sb, 4, 64, out, 0, None) == K.KQ_ERR_ARG
    assert raw("mx_gemm", qa + 8, sa, 4, qb, sb, 4, 64, out, 0, None) == K.KQ_ERR_ALIGN
    assert raw("mx_gemm", qa, sa, 4, qb, sb, 4, 64, out + 2, 0, None) == K.KQ_ERR_ALIGN
    assert raw("mx_gemm", qa, sa, 4, qb, sb, 4, 64, qa + 2, 1, None) == K.KQ_ERR_OVERLAP  # 2-byte ok for bf16
    assert raw("mx_gemm", qa, sa, 4, qb, sb, 4, 64, qa + 16, 0, None) == K.KQ_ERR_OVERLAP
    assert raw("mx_gemm", None, None, 0, None, None, 4, 64, None, 0, None) == K.KQ_OK
    assert raw("mx_gemm", qa, sa, 4, qb, sb, (1 << 21) + 1, 64, out, 0, None) == K.KQ_ERR_SHAPE


def test_adaln_validation():
    h, sh, sc, f, q, s, x, w = (FAKE + (k << 30) for k in range(8))
    ok = dict(T=2, eps=1e-6)

    def fused(h=h, M=4, d=64, sh=sh, sc=sc, T=ok["T"], eps=ok["eps"], f=f, nT=1, w=w, q=q, s=s):
        return raw("kq_adaln_quantize", h, M, d, sh, sc, T, eps, f, nT, w, q, s, None)

    def alone(h=h, M=4, d=64, sh=sh, sc=sc, T=ok["T"], eps=ok["eps"], w=w, x=x):
        return raw("adaln_modulate", h, M, d, sh, sc, T, eps, w, x, None)

    assert fused(d=48) == K.KQ_ERR_SHAPE
    assert fused(d=(1 << 20) + 32) == K.KQ_ERR_SHAPE
    assert fused(nT=3) == K.KQ_ERR_SHAPE
    assert fused(T=0) == K.KQ_ERR_ARG
    for e in (0.0, -1.0, float("inf"), float("nan")):
        assert fused(eps=e) == K.KQ_ERR_ARG
    assert fused(M=-1) == K.KQ_ERR_ARG
    assert fused(h=None) == K.KQ_ERR_ARG
    assert fused(sc=None) == K.KQ_ERR_ARG
    assert fused(f=None) == K.KQ_ERR_ARG
    assert fused(w=None) == K.KQ_ERR_ARG
    assert fused(h=h + 2) == K.KQ_ERR_ALIGN
    assert fused(q=q + 8) == K.KQ_ERR_ALIGN
    assert fused(sh=sh + 2) == K.KQ_ERR_ALIGN
    assert fused(w=w + 4) == K.KQ_ERR_ALIGN
    assert fused(q=h + 16) == K.KQ_ERR_OVERLAP
    assert fused(s=sh + 4) == K.KQ_ERR_OVERLAP
    assert fused(s=q + 8) == K.KQ_ERR_OVERLAP
    assert fused(f=q + 16) == K.KQ_ERR_OVERLAP
    assert fused(w=q + 16) == K.KQ_ERR_OVERLAP
    assert fused(w=h + 64) == K.KQ_ERR_OVERLAP
    assert fused(w=f + 8) == K.KQ_ERR_OVERLAP
    assert fused(M=0, h=None, q=None) == K.KQ_OK
    assert alone(x=None) == K.KQ_ERR_ARG
    assert alone(w=None) == K.KQ_ERR_ARG
    assert alone(x=x + 8) == K.KQ_ERR_ALIGN
    assert alone(x=sc) == K.KQ_ERR_OVERLAP
    assert alone(x=h + 64) == K.KQ_ERR_OVERLAP
    assert alone(x=w + 16) == K.KQ_ERR_OVERLAP
    assert alone(T=-3) == K.KQ_ERR_ARG
    assert alone(M=0, x=None) == K.KQ_OK


def test_kq16_validation():
    x, f, q, s, y = (FAKE + (k << 30) for k in range(5))
    assert raw("kq_quantize16", x, 4, 24, f, 1, q, s, None) == K.KQ_ERR_SHAPE  # d % 16
    assert raw("kq_quantize16", x, 4, 48, f, 2, q, s, None) == K.KQ_ERR_SHAPE  # nT not in {1, 3}
    assert raw("kq_quantize16", x, -1, 48, f, 1, q, s, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize16", None, 4, 48, f, 3, q, s, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize16", x, 4, 48, None, 3, q, s, None) == K.KQ_ERR_ARG
    assert raw("kq_quantize16", x + 8, 4, 48, f, 3, q, s, None) == K.KQ_ERR_ALIGN
    assert raw("kq_quantize16", x, 4, 48, f + 2, 3, q, s, None) == K.KQ_ERR_ALIGN
    assert raw("kq_quantize16", x, 4, 48, f, 3, x + 32, s, None) == K.KQ_ERR_OVERLAP
    assert raw("kq_quantize16", x, 4, 48, f, 3, q, q + 95, None) == K.KQ_ERR_OVERLAP  # s overlaps q's 96 bytes
    assert raw("kq_quantize16", x, 4, 48, q, 3, q, s, None) == K.KQ_ERR_OVERLAP
    assert raw("kq_quantize16", None, 0, 48, None, 1, None, None, None) == K.KQ_OK
    assert raw("kq_transform16_f32", x, 4, 40, f, 1, y, None) == K.KQ_ERR_SHAPE
    assert raw("kq_transform16_f32", x, 4, 48, f, 3, x + 16, None) == K.KQ_ERR_OVERLAP
    assert raw("kq_transform16_f32", x, 4, 48, f, 3, y + 4, None) == K.KQ_ERR_ALIGN


def test_tuning_validation():
    # launch-shape overrides travel as an argument; out-of-range fields are
    # refused before any HIP call, and nothing is kept between calls
    import ctypes
    x, q, s, f, y = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30)
    bad = [("mfma_tiles_per_wg", 257), ("mfma_tiles_per_wg", -1), ("mfma_groups", 3), ("mfma_strip", 12), ("mfma_strip", 2),
           ("mfma_order", 3), ("code_stores", 3), ("stream_rows_per_wave", 300), ("gemm_kernel", 4),
           ("adaln_pass", 4), ("adaln_strip", 16), ("adaln_blocks_per_wave", 0x10000), ("shared_form", 3),
           ("flat_wgs", -2), ("flat_wgs", (1 << 20) + 1), ("flat_ring", 1), ("flat_ring", 4),
           ("mfma_ring", 3), ("mfma_ring", 1)]
    for field, val in bad:
        t = ctypes.byref(K.Tuning(**{field: val}))
        assert raw("kq_quantize_tuned", x, 4, 64, f, 1, q, s, 0, t, None) == K.KQ_ERR_ARG, field
        assert raw("kq_transform_tuned", x, 4, 64, f, 1, y, 0, t, None) == K.KQ_ERR_ARG, field
        assert raw("mx_gemm_tuned", q, s, 4, q, s, 4, 64, y, 0, t, None) == K.KQ_ERR_ARG, field
        shape = (ctypes.c_int64 * 7)()
        assert raw("kq_launch_shape", 4, 64, 0, t, shape) == K.KQ_ERR_ARG, field
        assert raw("kq_flat_launch_shape", 4, 64, t, shape) == K.KQ_ERR_ARG, field
    ok = ctypes.byref(K.Tuning(mfma_strip=16, code_stores=2, gemm_kernel=3))
    # a valid override still fails the other checks first (no GPU is touched)
    assert raw("kq_quantize_tuned", x + 2, 4, 64, f, 1, q, s, 0, ok, None) == K.KQ_ERR_ALIGN
    assert raw("kq_quantize_tuned", x, 0, 64, f, 1, q, s, 0, ok, None) == K.KQ_OK
    assert raw("kq_launch_shape", 4, 48, 0, None, (ctypes.c_int64 * 7)()) == K.KQ_ERR_SHAPE
    assert raw("kq_launch_shape", 4, 64, 2, None, (ctypes.c_int64 * 7)()) == K.KQ_ERR_ARG
    assert raw("kq_launch_shape", 4, 64, 0, None, None) == K.KQ_ERR_ARG
    assert raw("kq_flat_launch_shape", 4, 48, None, (ctypes.c_int64 * 3)()) == K.KQ_ERR_SHAPE
    assert raw("kq_flat_launch_shape", -1, 64, None, (ctypes.c_int64 * 3)()) == K.KQ_ERR_ARG
    assert raw("kq_flat_launch_shape", 4, 64, None, None) == K.KQ_ERR_ARG
    with pytest.raises(ValueError):
        K.kq_launch_shape(4, 64, tuning={"no_such_field": 1})
    assert not hasattr(K.lib(), "kq_set_tuning")


def test_sizes_near_int64_max_are_shape_errors():
    # block counts and byte sizes are bounded by quotient, so huge M is a shape
    # error, never a wrapped product that reaches the launch
    big = (1 << 63) - 1
    x, q, s, f, y = FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE + (4 << 30)
    for M in (big, big // 2, (1 << 40) // 36 + 1, 1 << 62):
        assert raw("kq_quantize", x, M, 1152, f, 1, q, s, None) == K.KQ_ERR_SHAPE, M
        assert raw("sq_quantize", x, M, 1152, f, q, s, None) == K.KQ_ERR_SHAPE, M
        assert raw("mx_quantize_f32", x, M, 1152, q, s, None) == K.KQ_ERR_SHAPE, M
        assert raw("kq_transform_f32", x, M, 1152, f, 1, y, None) == K.KQ_ERR_SHAPE, M
        assert raw("kq_quantize16", x, M, 1152, f, 1, q, s, None) == K.KQ_ERR_SHAPE, M
        assert raw("fwht_quantize", x, M, 1152, q, s, None) == K.KQ_ERR_SHAPE, M
        assert raw("mx_gemm", q, s, M, q, s, 64, 64, y, 0, None) == K.KQ_ERR_SHAPE, M
        assert raw("kq_adaln_quantize", x, M, 1152, f, f, 1, ctypes_float(1e-6), f, 1, y, q, s, None) \
            == K.KQ_ERR_SHAPE, M
    # the largest accepted block count still passes the shape check (it then
    # fails on the null pointer, before any HIP call)
    M = (1 << 40) // 36
    assert raw("kq_quantize", None, M, 1152, f, 1, q, s, None) == K.KQ_ERR_ARG
    # tokens_per_sample near INT64_MAX: ceil(M / T) is formed without
    # overflow, so the [1, d] modulation rows still have their true size and a
    # workspace placed inside them is caught
    h, sh, sc, q2, s2 = (FAKE + (i << 32) for i in range(5))
    assert raw("kq_adaln_quantize", h, 4, 64, sh, sc, big, ctypes_float(1e-6), f, 1, sh + 128, q2, s2,
               None) == K.KQ_ERR_OVERLAP


def ctypes_float(v):
    import ctypes
    return ctypes.c_float(v)


def test_noalloc_validation():
    # the allocation-free AdaLN entry point refuses rows beyond its fixed
    # workspace before any HIP call, and checks the other arguments as
    # kq_adaln_quantize does
    import ctypes
    h, sh, sc, f, q, s = (FAKE + (i << 32) for i in range(6))
    eps = ctypes.c_float(1e-6)
    big = K.KQ_NOALLOC_MAX_ROWS + 1
    assert raw("kq_adaln_quantize_noalloc", h, big, 64, sh, sc, 1, eps, f, 1, q, s, None) == K.KQ_ERR_SHAPE
    assert raw("kq_adaln_quantize_noalloc", h, 1 << 62, 64, sh, sc, 1, eps, f, 1, q, s, None) == K.KQ_ERR_SHAPE
    assert raw("kq_adaln_quantize_noalloc", h, 4, 48, sh, sc, 1, eps, f, 1, q, s, None) == K.KQ_ERR_SHAPE
    assert raw("kq_adaln_quantize_noalloc", h, 4, 64, sh, sc, 0, eps, f, 1, q, s, None) == K.KQ_ERR_ARG
    assert raw("kq_adaln_quantize_noalloc", h, 4, 64, sh, sc, 1, eps, f, 1, q, None, None) == K.KQ_ERR_ARG
    assert raw("kq_adaln_quantize_noalloc", h + 2, 4, 64, sh, sc, 1, eps, f, 1, q, s, None) == K.KQ_ERR_ALIGN
    assert raw("kq_adaln_quantize_noalloc", h, 4, 64, sh, sc, 1, eps, f, 1, h + 64, s, None) == K.KQ_ERR_OVERLAP
    assert raw("kq_adaln_quantize_noalloc", None, 0, 64, None, None, 1, eps, None, 1, None, None, None) == K.KQ_OK
