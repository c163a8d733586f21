"""Pins for the CPU oracle: each check ties the oracle to something other than
itself (a library routine, a closed form, a hand-derived fixture, brute force).

Sources: the abstract on the mlsanity.com page for arXiv 2607.21446 (block
transform + inverse on the weights, MXFP4), the pith.science verdict record
for the same paper (pith_extraction.key_machinery: K = G1 (x) ... (x) G5 of
2x2 factors; pith_extraction.core_discovery: Hadamard is five identical 2x2
factors; skeptic_critique.load_bearing_attack, paper Section 3.2 Eq. 4:
block-diagonal 32x32 blocks), and the OCP MX v1.0 encodings for E2M1 / E8M0.
"""
import json
import math
import os
import subprocess

import numpy as np
import pytest
import scipy.linalg

from synth import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))


def kron5(f5):
    """numpy's kron chain A1 (x) A2 (x) A3 (x) A4 (x) A5 in float64."""
    K = np.array([[1.0]])
    for k in range(5):
        K = np.kron(K, f5[k].astype(np.float64))
    return K


# ---------------------------------------------------------------------------
# bf16 decoding: every one of the 65536 patterns against numpy's bit view
# ---------------------------------------------------------------------------
def test_bf16_decode_all_patterns(oracle_lib):
    import ctypes
    L = oracle_lib.lib()
    pats = np.arange(65536, dtype=np.uint32)
    ref = (pats << 16).view(np.float32).astype(np.float64)
    got = np.array([L.oracle_bf16_to_double(ctypes.c_uint16(int(p))) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero preserved
    assert math.copysign(1.0, got[0x8000]) == -1.0


# ---------------------------------------------------------------------------
# Kronecker block: library kron, mode-wise product, inverse, det, cond
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_kron_block_equals_numpy_kron(oracle_lib, seed):
    f = I.random_factors(1, seed)[0]
    K = oracle_lib.kron_block(f)
    R = kron5(f)
    assert np.allclose(K, R, rtol=1e-15, atol=0.0)


def test_kron_bit_order_is_msb_first(oracle_lib):
    # A1 = diag(1, 2) and the rest identity: the factor 2 must land on the
    # second half of the block (index bit 4 set), as numpy's kron does.
    f = I.identity_factors(1)[0].copy()
    f[0] = np.diag([1.0, 2.0])
    K = oracle_lib.kron_block(f)
    assert np.array_equal(np.diag(K), np.array([1.0] * 16 + [2.0] * 16))
    f = I.identity_factors(1)[0].copy()
    f[4] = np.diag([1.0, 2.0])
    K = oracle_lib.kron_block(f)
    assert np.array_equal(np.diag(K), np.array([1.0, 2.0] * 16))


def test_transform_equals_modewise_product(oracle_lib):
    M, d = 7, 256
    x = I.act_gaussian_outliers(M, d, 11, 3, 30.0)[0]
    f = I.random_factors(d // 32, 12)
    y, z = oracle_lib.kq_transform(x, f)
    X = I.bf16_bits_to_f32(x).astype(np.float64).reshape(M, d // 32, 2, 2, 2, 2, 2)
    F = f.astype(np.float64)
    ref = np.einsum("mjabcde,jaA,jbB,jcC,jdD,jeE->mjABCDE", X, F[:, 0], F[:, 1], F[:, 2], F[:, 3], F[:, 4],
                    optimize=True).reshape(M, d)
    assert np.all(np.abs(y - ref) <= 1e-12 * z)
    # and the dense product x_blk @ K_j with numpy's kron
    dense = np.concatenate([X.reshape(M, d // 32, 32)[:, j] @ kron5(f[j]) for j in range(d // 32)], axis=1)
    assert np.all(np.abs(y - dense) <= 1e-12 * z)
    # z is the same contraction on magnitudes
    zref = np.concatenate([np.abs(X.reshape(M, d // 32, 32)[:, j]) @ np.abs(kron5(f[j])) for j in range(d // 32)],
                          axis=1)
    assert np.allclose(z, zref, rtol=1e-13, atol=0)


def test_shared_factor_set_applies_to_every_block(oracle_lib):
    M, d = 3, 128
    x = I.act_gaussian_outliers(M, d, 5, 2, 10.0)[0]
    f1 = I.random_factors(1, 9)
    y1 = oracle_lib.kq_transform(x, f1, want_z=False)
    y4 = oracle_lib.kq_transform(x, np.repeat(f1, d // 32, axis=0), want_z=False)
    assert np.array_equal(y1, y4)


@pytest.mark.parametrize("seed", [4, 5])
def test_inverse_is_kron_of_factor_inverses(oracle_lib, seed):
    f = I.random_factors(1, seed)[0]
    K = oracle_lib.kron_block(f)
    Kinv = oracle_lib.kron_block_inverse(f)
    cond = np.linalg.cond(K)
    assert np.abs(Kinv @ K - np.eye(32)).max() <= 1e-12 * cond
    assert np.allclose(Kinv, np.linalg.inv(K), rtol=0, atol=1e-12 * cond * np.abs(Kinv).max())
    # determinant: det(A (x) B) = det(A)^m det(B)^n, so det K = prod det(A_k)^16
    sign, logdet = np.linalg.slogdet(K)
    dets = [np.linalg.det(f[k].astype(np.float64)) for k in range(5)]
    expect = np.prod(np.array(dets) ** 16)
    assert sign > 0 and np.isclose(logdet, math.log(expect), rtol=0, atol=1e-10)
    # condition number of a Kronecker product is the product of the conditions
    conds = [np.linalg.cond(f[k].astype(np.float64)) for k in range(5)]
    assert np.isclose(cond, np.prod(conds), rtol=1e-9)


def test_lu_factors_have_det_minus_one_and_block_det_plus_one(oracle_lib):
    # G = L U with L = [[1,0],[c,1]], U = [[a,b],[0,-1/a]] has det -1 per factor;
    # five such factors give det K = (-1)^(16*5) = +1, not -1.
    rng = np.random.default_rng(3)
    f = np.empty((5, 2, 2), np.float32)
    for k in range(5):
        a, b, c = rng.uniform(0.5, 1.5), rng.uniform(-1, 1), rng.uniform(-1, 1)
        L = np.array([[1, 0], [c, 1]])
        U = np.array([[a, b], [0, -1 / a]])
        f[k] = (L @ U).astype(np.float32)
    K = oracle_lib.kron_block(f)
    dets = [np.linalg.det(f[k].astype(np.float64)) for k in range(5)]
    assert all(abs(dd + 1) < 1e-6 for dd in dets)
    assert np.isclose(np.linalg.det(K), np.prod(np.array(dets) ** 16), rtol=1e-9)
    assert np.linalg.det(K) > 0


def test_singular_factor_is_rejected(oracle_lib):
    f = I.identity_factors(1)[0].copy()
    f[2] = np.array([[1.0, 2.0], [2.0, 4.0]])
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.kron_block_inverse(f)


# ---------------------------------------------------------------------------
# exact invariance (X T)(T^-1 W^T) = X W^T with integer unimodular factors
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shared", [True, False])
def test_exact_invariance_integer_factors(oracle_lib, shared):
    rng = np.random.default_rng(21)
    M, d, N = 5, 128, 6
    nB = d // 32
    f = I.integer_unimodular_factors(1 if shared else nB, 33)
    x_int = rng.integers(-3, 4, size=(M, d)).astype(np.float32)
    w_int = rng.integers(-3, 4, size=(N, d)).astype(np.float64)
    x = I.f32_to_bf16_bits(x_int)  # small integers are exact in bf16
    y = oracle_lib.kq_transform(x, f, want_z=False)
    assert np.array_equal(y, np.round(y)), "integer factors and inputs give integer outputs"
    blocks = [oracle_lib.kron_block_inverse(f[0 if shared else j]) for j in range(nB)]
    Tinv = scipy.linalg.block_diag(*blocks)
    assert np.array_equal(Tinv, np.round(Tinv))
    lhs = y @ (Tinv @ w_int.T)
    rhs = x_int.astype(np.float64) @ w_int.T
    assert np.array_equal(lhs, rhs)


def test_invariance_real_factors(oracle_lib):
    rng = np.random.default_rng(22)
    M, d, N = 4, 96, 3
    f = I.random_factors(d // 32, 44)
    x = I.act_gaussian_outliers(M, d, 23, 2, 30.0)[0]
    w = rng.standard_normal((N, d))
    y = oracle_lib.kq_transform(x, f, want_z=False)
    Tinv = scipy.linalg.block_diag(*[oracle_lib.kron_block_inverse(f[j]) for j in range(d // 32)])
    cond = max(np.linalg.cond(oracle_lib.kron_block(f[j])) for j in range(d // 32))
    lhs = y @ (Tinv @ w.T)
    rhs = I.bf16_bits_to_f32(x).astype(np.float64) @ w.T
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-10 * cond * np.abs(rhs).max())


# ---------------------------------------------------------------------------
# special factor sets
# ---------------------------------------------------------------------------
def test_identity_factors_reduce_to_plain_mxfp4(oracle_lib):
    x, _, _ = I.act_sweep_special(64, 1024, 77, special_frac=0.02)
    q1, s1, y1 = oracle_lib.kq_quantize(x, I.identity_factors(1), want_y32=True)
    q2, s2 = oracle_lib.mx_quantize_f32(I.bf16_bits_to_f32(x))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    # the transformed values are the inputs themselves (as real numbers)
    assert np.array_equal(y1, I.bf16_bits_to_f32(x) + np.float32(0.0))
    # and SmoothQuant with unit scales is the same quantizer
    q3, s3 = oracle_lib.sq_quantize(x, np.ones(1024, np.float32))
    assert np.array_equal(q1, q3) and np.array_equal(s1, s3)


def test_hadamard_factors_give_normalised_wht32(oracle_lib):
    M, d = 9, 64
    x = I.act_gaussian_outliers(M, d, 31, 2, 30.0)[0]
    y, z = oracle_lib.kq_transform(x, I.hadamard_factors(1))
    H = scipy.linalg.hadamard(32).astype(np.float64)  # Sylvester order
    assert np.array_equal(H @ H.T, 32 * np.eye(32))
    X = I.bf16_bits_to_f32(x).astype(np.float64).reshape(M, d // 32, 32)
    c = float(np.float32(1.0 / math.sqrt(2.0))) ** 5  # the fp32 factors, exactly
    ref = (X @ H).reshape(M, d) * c
    assert np.all(np.abs(y - ref) <= 1e-12 * z)
    # against the exact normalised WHT: off only by fl32(1/sqrt 2)^5 vs 1/sqrt(32)
    ref_exact = (X @ H).reshape(M, d) / math.sqrt(32.0)
    assert np.all(np.abs(y - ref_exact) <= 5 * 2.0 ** -24 * z)


# ---------------------------------------------------------------------------
# MX quantizer: hand-derived fixtures and exhaustive element / scale sweeps
# ---------------------------------------------------------------------------
def _load_handcases():
    with open(os.path.join(HERE, "golden", "mx_handcases.json")) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _load_handcases(), ids=lambda c: c["name"])
def test_mx_block_handcases(oracle_lib, case):
    y = np.array([float.fromhex(v) if v.lower().lstrip("-").startswith("0x") else float(v) for v in case["y"]],
                 np.float32)
    q, sbyte = oracle_lib.mx_block(y)
    codes = np.array(case["codes"], np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    assert sbyte == case["scale_byte"]
    assert np.array_equal(q, packed), (q, packed)


def test_grid_and_scale_bruteforce(oracle_lib, tmp_path):
    exe = tmp_path / "grid_bruteforce"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(HERE, "pins", "grid_bruteforce.c"), "-ldl", "-lpthread", "-lm"], check=True)
    nth = str(min(16, os.cpu_count() or 1))
    args = [str(exe), oracle_lib.LIB_PATH, nth]
    if os.environ.get("KQ_PIN_FULL"):
        args.append("full")
    r = subprocess.run(args, capture_output=True, text=True, timeout=1200)
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("PASS"), r.stdout + r.stderr


# ---------------------------------------------------------------------------
# SmoothQuant reading and shape rules
# ---------------------------------------------------------------------------
def test_sq_power_of_two_scales_are_exact_division(oracle_lib):
    M, d = 6, 128
    x = I.act_gaussian_outliers(M, d, 41, 4, 30.0)[0]
    k = np.random.default_rng(5).integers(-6, 7, size=d)
    scale = np.ldexp(np.ones(d, np.float32), k).astype(np.float32)
    _, _, y = oracle_lib.sq_quantize(x, scale, want_y32=True)
    assert np.array_equal(y, np.ldexp(I.bf16_bits_to_f32(x), -k[None, :]).astype(np.float32))


def test_sq_rounds_once_per_step(oracle_lib):
    # y = fl32(x * fl32(1/s)): check against python's correctly rounded doubles
    M, d = 4, 64
    x = I.act_gaussian_outliers(M, d, 42, 2, 30.0)[0]
    scale = (1.0 + np.random.default_rng(6).random(d) * 7).astype(np.float32)
    _, _, y = oracle_lib.sq_quantize(x, scale, want_y32=True)
    xf = I.bf16_bits_to_f32(x).astype(np.float64)
    recip = np.array([np.float32(1.0 / float(s)) for s in scale], np.float64)  # 1/s correctly rounded to fp32
    # the exact product of two fp32 values fits a double, so one cast rounds it once
    assert np.array_equal(y, (xf * recip[None, :]).astype(np.float32))


def test_shape_rules(oracle_lib):
    L = oracle_lib.lib()
    x = np.zeros((2, 64), np.uint16)
    f = I.identity_factors(2)
    q = np.zeros((2, 32), np.uint8)
    s = np.zeros((2, 2), np.uint8)
    P = lambda a: a.ctypes.data  # noqa: E731
    assert L.oracle_kq_quantize(P(x), 2, 64, P(f), 2, P(q), P(s), None) == 0
    assert L.oracle_kq_quantize(P(x), 2, 64, P(f), 1, P(q), P(s), None) == 0
    assert L.oracle_kq_quantize(P(x), 2, 48, P(f), 1, P(q), P(s), None) == 2  # d % 32
    assert L.oracle_kq_quantize(P(x), 2, 64, P(f), 3, P(q), P(s), None) == 2  # nT not in {1, d/32}
    assert L.oracle_kq_quantize(P(x), -1, 64, P(f), 1, P(q), P(s), None) == 1
    assert L.oracle_kq_quantize(P(x), 0, 64, P(f), 1, P(q), P(s), None) == 0  # empty is fine


# ---------------------------------------------------------------------------
# K2 form: factors given as LU scalars (pith.science verdict record:
# referee_report.minor_comments, section 3, U = [[a, b], [0, -1/a]] and
# det G = -1; key_machinery / core_discovery: three scalars per factor,
# Hadamard initialisation).  L = [[1, 0], [c, 1]] is this build's reading.
# ---------------------------------------------------------------------------
def test_lu_factor_closed_forms(oracle_lib):
    rng = np.random.default_rng(11)
    for _ in range(200):
        a, b, c = (rng.uniform(0.3, 2.0) * rng.choice([-1, 1]), rng.normal(), rng.normal())
        abc = np.array([a, b, c], np.float32)
        a, b, c = (float(v) for v in abc)
        G = oracle_lib.lu_factor(abc)
        # row 0 of L U is row 0 of U
        assert G[0, 0] == a and G[0, 1] == b
        # unit-triangular L and det U = a * (-1/a): det G = -1
        assert abs(np.linalg.det(G) + 1.0) <= 1e-13 * max(1.0, np.abs(G).max() ** 2)
        # inverse from the closed forms U^-1 = [[1/a, b], [0, -a]], L^-1 = [[1, 0], [-c, 1]]
        Uinv = np.array([[1.0 / a, b], [0.0, -a]])
        Linv = np.array([[1.0, 0.0], [-c, 1.0]])
        assert np.allclose(G @ (Uinv @ Linv), np.eye(2), rtol=0, atol=1e-12 * max(1.0, np.abs(G).max() ** 2))


def test_lu_block_is_kron_of_its_factors(oracle_lib):
    lu = I.random_lu(3, 17)
    for t in range(3):
        K = oracle_lib.lu_kron_block(lu[t])
        ref = np.array([[1.0]])
        for k in range(5):
            ref = np.kron(ref, oracle_lib.lu_factor(lu[t, k]))
        assert np.allclose(K, ref, rtol=1e-15, atol=0)
        # det(A (x) B) = det(A)^n det(B)^m: five factors of det -1 give det K = +1
        assert abs(np.linalg.det(K) - 1.0) < 1e-9


def test_lu_hadamard_initialisation_gives_wht32(oracle_lib):
    K = oracle_lib.lu_kron_block(I.hadamard_lu(1)[0])
    H = scipy.linalg.hadamard(32).astype(np.float64) / math.sqrt(32.0)
    # exact up to the fp32 rounding of 1/sqrt(2) in a, b (and -1/a)
    assert np.abs(K - H).max() <= 8 * 2.0 ** -24


def test_wht_block_is_sylvester_hadamard(oracle_lib):
    H = scipy.linalg.hadamard(32).astype(np.float64) / math.sqrt(32.0)
    assert np.abs(oracle_lib.wht_block() - H).max() <= 1e-16


def _fwht_inplace(v):
    """Iterative fast Walsh-Hadamard transform along the last axis (natural
    order), unnormalised: the butterfly algorithm, independent of the dense
    definition the oracle uses."""
    v = v.copy()
    n = v.shape[-1]
    h = 1
    while h < n:
        v = v.reshape(v.shape[:-1] + (n // (2 * h), 2, h))
        a, b = v[..., 0, :].copy(), v[..., 1, :].copy()
        v[..., 0, :], v[..., 1, :] = a + b, a - b
        v = v.reshape(v.shape[:-3] + (n,))
        h *= 2
    return v


def test_fwht_transform_matches_fast_butterfly(oracle_lib):
    M, d = 13, 96
    x = I.act_gaussian_outliers(M, d, 41, 2, 50.0)[0]
    y, z = oracle_lib.fwht_transform(x)
    X = I.bf16_bits_to_f32(x).astype(np.float64).reshape(M, d // 32, 32)
    ref = _fwht_inplace(X).reshape(M, d) / math.sqrt(32.0)
    assert np.all(np.abs(y - ref) <= 1e-14 * z)
    assert np.allclose(z, np.abs(X).sum(axis=2).repeat(32, axis=1).reshape(M, d) / math.sqrt(32.0), rtol=1e-14)


def test_fwht_quantize_is_mx_of_its_transform(oracle_lib):
    M, d = 7, 64
    x = I.act_gaussian_outliers(M, d, 43, 2, 50.0)[0]
    q, s, y32 = oracle_lib.fwht_quantize(x, want_y32=True)
    y = oracle_lib.fwht_transform(x, want_z=False)
    assert np.array_equal(y32, y.astype(np.float32))
    qm, sm = oracle_lib.mx_quantize_f32(y32)
    assert np.array_equal(q, qm) and np.array_equal(s, sm)


def test_kq_lu_matches_factor_path_on_the_same_block(oracle_lib):
    # the LU path and the 2x2-factor path share the per-block machinery: with
    # integer scalars every factor entry is exact in fp32, so both paths see the
    # identical block and must agree bit for bit
    lu = np.array([[[1, 2, -1], [-1, 0, 1], [1, 1, 1], [1, -1, 2], [-1, 1, 0]]], np.float32)
    f = np.array([[oracle_lib.lu_factor(lu[0, k]) for k in range(5)]], np.float32)
    assert np.array_equal(f.astype(np.float64), np.array([[oracle_lib.lu_factor(lu[0, k]) for k in range(5)]]))
    M, d = 5, 96
    x = I.act_gaussian_outliers(M, d, 47, 2, 20.0)[0]
    q1, s1 = oracle_lib.kq_quantize_lu(x, lu)
    q2, s2 = oracle_lib.kq_quantize(x, f)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    for shape_lu in (np.zeros((2, 5, 3), np.float32), np.zeros((d // 32 + 1, 5, 3), np.float32)):
        with pytest.raises(Exception):
            oracle_lib.kq_quantize_lu(x, shape_lu)


# ---------------------------------------------------------------------------
# MXFP4 consumer (the abstract's W4A4 product): dequantization and GEMM
# ---------------------------------------------------------------------------
def test_mx_value_inverts_the_element_encoding(oracle_lib):
    # every code at every normal scale: encoding the value again gives the code
    # back (-0, code 8, comes back as +0: the sign bit is set only for values < 0)
    for sbyte in range(1, 255, 3):
        E = sbyte - 127
        for code in range(16):
            v = oracle_lib.mx_value(code, sbyte)
            if abs(v) > float(np.finfo(np.float32).max):
                continue  # 4 or 6 times 2^126 is past fp32: not an fp32 input to encode
            back = oracle_lib.fp4_code(np.float32(v), E)
            assert back == (0 if code == 8 else code), (code, sbyte, v, back)
    assert math.isnan(oracle_lib.mx_value(3, 0xFF))


def test_mx_dequant_requantizes_to_itself(oracle_lib):
    rng = np.random.default_rng(53)
    y = (rng.standard_normal((24, 256)) * np.exp(rng.uniform(-8, 8, (24, 1)))).astype(np.float32)
    y[3, 32:64] = 0.0
    q, s = oracle_lib.mx_quantize_f32(y)
    v = oracle_lib.mx_dequant(q, s)
    # each value is within 2^(E+1) of its input: half the widest grid step
    # (2 * 2^E, between 4 and 6), or the saturation of (6, 8) * 2^E to 6 * 2^E
    E = s.astype(np.int64).repeat(32, axis=1) - 127
    assert np.all(np.abs(v - y) <= np.ldexp(2.0, E))
    q2, s2 = oracle_lib.mx_quantize_f32(v.astype(np.float32))
    lo, hi = q & 0x0F, q >> 4
    q_pos0 = np.where(lo == 8, 0, lo) | (np.where(hi == 8, 0, hi) << 4)
    assert np.array_equal(s2, s) and np.array_equal(q2, q_pos0.astype(np.uint8))


def test_mx_gemm_matches_numpy_matmul(oracle_lib):
    rng = np.random.default_rng(59)
    M, N, K = 9, 7, 160
    ya = (rng.standard_normal((M, K)) * 3).astype(np.float32)
    yb = (rng.standard_normal((N, K)) * 0.1).astype(np.float32)
    qa, sa = oracle_lib.mx_quantize_f32(ya)
    qb, sb = oracle_lib.mx_quantize_f32(yb)
    out, mag = oracle_lib.mx_gemm(qa, sa, qb, sb)
    A, B = oracle_lib.mx_dequant(qa, sa), oracle_lib.mx_dequant(qb, sb)
    assert np.all(np.abs(out - A @ B.T) <= 1e-14 * mag)
    assert np.allclose(mag, np.abs(A) @ np.abs(B).T, rtol=1e-14, atol=0)


def test_mx_gemm_hand_case(oracle_lib):
    # one block each: A = 1.5 * 2^1 at k = 0 and -6 * 2^1 at k = 31; B = 4 * 2^-2 at
    # k = 0 and 0.5 * 2^-2 at k = 31:  3 * 1 + (-12) * 0.125 = 1.5
    qa = np.zeros((1, 16), np.uint8)
    qa[0, 0] = 0x03          # k = 0: code 3 (1.5), low nibble
    qa[0, 15] = 0xF0         # k = 31: code 15 (-6), high nibble
    qb = np.zeros((1, 16), np.uint8)
    qb[0, 0] = 0x06          # k = 0: code 6 (4)
    qb[0, 15] = 0x10         # k = 31: code 1 (0.5)
    sa = np.array([[128]], np.uint8)
    sb = np.array([[125]], np.uint8)
    out, mag = oracle_lib.mx_gemm(qa, sa, qb, sb)
    assert out[0, 0] == 1.5 and mag[0, 0] == 4.5


# ---------------------------------------------------------------------------
# AdaLN front-end (the abstract: normalisation between the blocks keeps the
# transform online; the verdict record's referee summary: AdaLN).  Reading:
# LayerNorm without affine, then x * (1 + scale[b]) + shift[b], b = m // T,
# and x rounded to bf16.
# ---------------------------------------------------------------------------
def _bf16_bits(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def _adaln_inputs(M, d, T, seed):
    rng = np.random.default_rng(seed)
    h = _bf16_bits(rng.standard_normal((M, d)) * np.exp(rng.uniform(-2, 2, (M, 1))) + rng.uniform(-3, 3, (M, 1)))
    nS = (M + T - 1) // T
    shift = (0.5 * rng.standard_normal((nS, d))).astype(np.float32)
    scale = (0.5 * rng.standard_normal((nS, d))).astype(np.float32)
    return h, shift, scale


@pytest.mark.parametrize("M,d,T", [(5, 64, 2), (7, 1152, 3), (4, 4608, 4)])
def test_adaln_matches_torch_layer_norm(oracle_lib, M, d, T):
    import torch
    h, shift, scale = _adaln_inputs(M, d, T, 700 + d)
    x, xb, fl = oracle_lib.adaln(h, shift, scale, T, 1e-6)
    hd = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ln = torch.nn.functional.layer_norm(torch.from_numpy(hd), (d,), eps=1e-6).numpy()
    b = np.arange(M) // T
    ref = ln * (1.0 + scale[b].astype(np.float64)) + shift[b].astype(np.float64)
    assert np.all(np.abs(x - ref) <= 1e-12 * (np.abs(ref) + 1.0)), float(np.abs(x - ref).max())
    assert not fl.any()


def test_adaln_hand_case(oracle_lib):
    # a row alternating a and b: mean (a+b)/2, variance ((a-b)/2)^2, so
    # x_c = +-((a-b)/2) / sqrt(((a-b)/2)^2 + eps) * (1 + scale) + shift
    M, d, T, eps = 5, 32, 2, 1e-6
    a, bv = 3.5, -1.25
    row = np.array([a, bv] * (d // 2), np.float32)
    h = _bf16_bits(np.tile(row, (M, 1)))
    shift = np.stack([np.full(d, 10.0 * k, np.float32) for k in range(3)])
    scale = np.stack([np.full(d, 0.25 * k, np.float32) for k in range(3)])
    x, _, _ = oracle_lib.adaln(h, shift, scale, T, eps)
    half = (a - bv) / 2.0
    n = half / math.sqrt(half * half + float(np.float32(eps)))
    for m in range(M):
        k = m // T
        want = np.array([n, -n] * (d // 2)) * (1.0 + 0.25 * k) + 10.0 * k
        assert np.allclose(x[m], want, rtol=1e-14, atol=1e-13)


def test_adaln_unit_moments(oracle_lib):
    # with scale = shift = 0 each row has mean 0 and mean square var / (var + eps)
    M, d, T = 6, 4608, 3
    h, shift, scale = _adaln_inputs(M, d, T, 710)
    x, _, _ = oracle_lib.adaln(h, np.zeros_like(shift), np.zeros_like(scale), T, 1e-6)
    hd = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    var = hd.var(axis=1)
    eps = float(np.float32(1e-6))
    assert np.all(np.abs(x.mean(axis=1)) <= 1e-13)
    assert np.allclose((x * x).mean(axis=1), var / (var + eps), rtol=1e-12, atol=0)


def _bf16_nearest_bruteforce(v):
    """bf16 bits of v by search: the finite bf16 values bracketing v, nearer
    wins, ties to the even bit pattern."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    sgn = 0x8000 if v < 0 else 0
    a = abs(v)
    pos = (np.arange(0x7F81, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)  # +0 .. +inf
    k = int(np.searchsorted(pos, a, side="right")) - 1  # pos[k] <= a < pos[k+1]
    lo, hi = pos[k], pos[k + 1]
    if a - lo < hi - a or (a - lo == hi - a and k % 2 == 0):
        return sgn | k
    return sgn | (k + 1)


def test_double_to_bf16_nearest_even(oracle_lib):
    # every midpoint between adjacent finite positive bf16 values (ties to the
    # even pattern), one double step either side of it, and random doubles
    pats = np.arange(0x7F7F, dtype=np.uint32)
    lo = (pats << 16).view(np.float32).astype(np.float64)
    hi = ((pats + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2.0
    for k in range(0, len(pats), 7):
        m = mid[k]
        want_tie = int(pats[k]) if pats[k] % 2 == 0 else int(pats[k]) + 1
        assert oracle_lib.double_to_bf16(m) == want_tie, hex(int(pats[k]))
        assert oracle_lib.double_to_bf16(np.nextafter(m, 0.0)) == int(pats[k])
        assert oracle_lib.double_to_bf16(np.nextafter(m, np.inf)) == int(pats[k]) + 1
        assert oracle_lib.double_to_bf16(-m) == 0x8000 | want_tie
    rng = np.random.default_rng(720)
    vals = rng.standard_normal(3000) * np.exp2(rng.integers(-140, 120, 3000))
    for v in vals:
        assert oracle_lib.double_to_bf16(v) == _bf16_nearest_bruteforce(v), v


def test_adaln_flags_a_value_on_a_midpoint(oracle_lib):
    # scale = -1 makes x = shift exactly; a shift on a bf16 midpoint must be
    # flagged (and round to even), a shift on a bf16 value must not
    M, d, T = 2, 32, 1
    h, _, _ = _adaln_inputs(M, d, T, 730)
    mid = np.float32(1.0 + 2.0 ** -8)       # between 0x3F80 and 0x3F81
    exact = np.float32(1.0 + 2.0 ** -7)     # 0x3F81 itself
    shift = np.array([np.full(d, mid), np.full(d, exact)], np.float32)
    scale = np.full((2, d), -1.0, np.float32)
    x, xb, fl = oracle_lib.adaln(h, shift, scale, T, 1e-6)
    assert np.all(x[0] == float(mid)) and np.all(xb[0] == 0x3F80) and fl[0].all()
    assert np.all(xb[1] == 0x3F81) and not fl[1].any()


def test_adaln_margin_flags_near_midpoints_only(oracle_lib):
    # Rows alternating +half and -half: n = +-half / sqrt(half^2 + eps) =
    # +-(1 - delta) with delta about eps / (2 half^2).  With scale = 0 and
    # shift = 2^-8, x = 1 + 2^-8 - delta sits delta below the bf16 midpoint
    # between 1 and 1 + 2^-7 (the other half of the row sits near -1 + 2^-8,
    # far from any midpoint).  delta = 4.8e-13 (half = 1024) is inside the
    # margin, so those elements are flagged (and round down, to 1);
    # delta = 2e-9 (half = 16) is far outside it and nothing is flagged.
    d, T, eps = 32, 1, 1e-6
    for half, flagged in ((1024.0, True), (16.0, False)):
        h = _bf16_bits(np.tile(np.array([half, -half] * (d // 2), np.float32), (1, 1)))
        shift = np.full((1, d), 2.0 ** -8, np.float32)
        scale = np.zeros((1, d), np.float32)
        x, xb, fl = oracle_lib.adaln(h, shift, scale, T, eps)
        delta = 1.0 + 2.0 ** -8 - x[0, 0]
        assert 0.0 < delta < (1e-12 if flagged else 1e-8)
        assert bool(fl[0, 0::2].all()) == flagged and not fl[0, 1::2].any()
        assert np.all(xb[0, 0::2] == 0x3F80)


def test_adaln_margin_against_high_precision(oracle_lib):
    # x recomputed in 60-digit decimal arithmetic (exact sums of the bf16
    # inputs, then one high-precision square root): the oracle's double x is
    # within its margin of it (so the margin bounds a double evaluation), and
    # every element the oracle does not flag rounds to the same bf16 from the
    # high-precision value
    import decimal
    decimal.getcontext().prec = 60
    D = decimal.Decimal
    M, d, T, eps = 24, 64, 5, 1e-6
    h, shift, scale = _adaln_inputs(M, d, T, 740)
    x, xb, fl = oracle_lib.adaln(h, shift, scale, T, eps)
    hv = (h.astype(np.uint32) << 16).view(np.float32)
    e32 = D(float(np.float32(eps)))
    worst = 0.0
    for m in range(M):
        vals = [D(float(v)) for v in hv[m]]
        mu = sum(vals) / d
        var = sum((v - mu) ** 2 for v in vals) / d
        r = 1 / (var + e32).sqrt()
        b = m // T
        for c in range(d):
            xe = (vals[c] - mu) * r * (1 + D(float(scale[b, c]))) + D(float(shift[b, c]))
            err = abs(float(D(float(x[m, c])) - xe))
            worst = max(worst, err / max(abs(float(xe)), 1e-300))
            if not fl[m, c]:
                assert oracle_lib.double_to_bf16(float(xe)) == int(xb[m, c]), (m, c)
    assert worst < 2.0 ** -40, worst


# ---------------------------------------------------------------------------
# 16-element blocks with four factors (the verdict record's pith_inferences:
# the construction carries over to 16-element blocks by changing the number of
# Kronecker factors).  Reading: K16 = A1 (x) A2 (x) A3 (x) A4, one E8M0 scale
# per 16 elements.
# ---------------------------------------------------------------------------
def kron4(f4):
    K = np.array([[1.0]])
    for k in range(4):
        K = np.kron(K, f4[k].astype(np.float64))
    return K


@pytest.mark.parametrize("seed", [21, 22])
def test_kron_block16_equals_numpy_kron(oracle_lib, seed):
    f = I.random_factors16(1, seed)[0]
    assert np.allclose(oracle_lib.kron_block16(f), kron4(f), rtol=1e-15, atol=0.0)


def test_transform16_per_block_sets_equal_modewise_product(oracle_lib):
    # each 16-element block through its own set, as four mode-wise 2x2
    # products on the block reshaped [2, 2, 2, 2] (A1 on the first mode)
    M, d = 3, 96
    nT = d // 16
    x = I.act_gaussian_outliers(M, d, 23, 2, 20.0)[0]
    f = I.random_factors16(nT, 24)
    y, z = oracle_lib.kq_transform16(x, f)
    xd = I.bf16_bits_to_f32(x).astype(np.float64)
    for j in range(nT):
        blk = xd[:, 16 * j:16 * j + 16].reshape(M, 2, 2, 2, 2)
        F = f[j].astype(np.float64)
        ref = np.einsum("mabcd,ae,bf,cg,dh->mefgh", blk, F[0], F[1], F[2], F[3]).reshape(M, 16)
        assert np.allclose(y[:, 16 * j:16 * j + 16], ref, rtol=1e-13, atol=1e-13)
    assert np.all(z >= np.abs(y))


def test_mx_block16_equals_padded_mx32(oracle_lib):
    # a 16-element block encodes exactly as the first half of a 32-element
    # block whose second half is zero (zeros change neither amax nor codes)
    rng = np.random.default_rng(25)
    for k in range(300):
        y = (rng.standard_normal(16) * np.exp2(rng.integers(-20, 20))).astype(np.float32)
        if k % 7 == 0:
            y[:] = 0.0
        q16, s16 = oracle_lib.mx_block16(y)
        q32, s32 = oracle_lib.mx_block(np.concatenate([y, np.zeros(16, np.float32)]))
        assert s16 == s32 and np.array_equal(q16, q32[:8])


def test_kq16_identity_factors_are_plain_mx16(oracle_lib):
    M, d = 4, 64
    x = I.act_gaussian_outliers(M, d, 26, 3, 30.0)[0]
    f = np.tile(np.eye(2, dtype=np.float32), (1, 4, 1, 1))
    q, s = oracle_lib.kq_quantize16(x, f)
    xf = I.bf16_bits_to_f32(x)
    for m in range(M):
        for j in range(d // 16):
            qb, sb = oracle_lib.mx_block16(xf[m, 16 * j:16 * j + 16])
            assert s[m, j] == sb and np.array_equal(q[m, 8 * j:8 * j + 8], qb)


def test_kq16_exact_integer_invariance(oracle_lib):
    # (X T16)(T16^-1 W^T) = X W^T exactly for integer unimodular factors
    M, d, N = 3, 64, 5
    rng = np.random.default_rng(27)
    X = rng.integers(-4, 5, (M, d)).astype(np.float32)
    x = I.f32_to_bf16_bits(X)
    f = I.integer_unimodular_factors16(d // 16, 28)
    y = oracle_lib.kq_transform16(x, f, want_z=False)
    W = rng.integers(-3, 4, (N, d)).astype(np.float64)
    Tinv = scipy.linalg.block_diag(*[np.round(np.linalg.inv(kron4(f[j]))) for j in range(d // 16)])
    assert np.array_equal(y @ (Tinv @ W.T), X.astype(np.float64) @ W.T)
