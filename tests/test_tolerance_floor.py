"""The absolute term of the transformed-value tolerance (tests/parity.py,
TOL_ABS), derived and checked on the CPU.

Below 2^-126 fp32 values lie on a fixed grid of spacing u = 2^-149, so a
rounding whose exact result is that small errs by up to u/2 no matter how
small the operands are; a relative bound (2e-6 z) cannot cover it.  The two
GPU transform forms round as follows:

  matrix cores: K is formed in fp32 and split exactly into three bf16 terms;
    every product of a bf16 x with a bf16 term is exact in fp32 unless it is
    below 2^-126, and sums of subnormals are exact.  At most 96 products per
    output can round: |error| <= 48 u.
  butterfly: each of the five 2x2 stages rounds twice per output (a product,
    then the fused multiply-add); an error of u made at stage k is then
    multiplied by the later stages, giving u * sum_k prod_{j>k} C_j with C_j
    the largest column abs sum of factor A_j.

The tests below emulate both summation orders in fp32 with numpy on
subnormal-range blocks and on an adversarial block built so that every
product rounds by nearly u/2 in the same direction, and check that the
emulated error stays within the derived bound and that the matrix-core bound
is nearly reached (so a smaller floor would be unsound for it).  The exact
reference comes from the oracle (float64 transform of the same inputs).
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import inputs as I
from tests import parity as P

U = P.ULP_SUB


def f32(a):
    return np.asarray(a, np.float64).astype(np.float32)


def bf16(a):
    """fp32 -> bf16 value (nearest even), as float32."""
    return I.bf16_bits_to_f32(I.f32_to_bf16_bits(f32(a)))


def fma32(a, b, c):
    """fp32 fused multiply-add: the product of two fp32 values is exact in
    float64; the sum is rounded once to float64 and then to fp32 (the double
    rounding can differ from a true fused result by one fp32 unit only when
    the float64 sum lands exactly on an fp32 midpoint, which the bounds below
    leave room for)."""
    return f32(np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64))


def kernel_block_matrix(fs):
    """K of one factor set formed in fp32 in the matrix-core kernel's order:
    ((((A1 A2) A3) A4) A5) entry products, one rounding after each."""
    F = np.asarray(fs, np.float32)
    K = np.empty((32, 32), np.float32)
    for r in range(32):
        for c in range(32):
            v = np.float32(F[0][(r >> 4) & 1][(c >> 4) & 1]) * np.float32(F[1][(r >> 3) & 1][(c >> 3) & 1])
            for k in range(2, 5):
                v = np.float32(v * np.float32(F[k][(r >> (4 - k)) & 1][(c >> (4 - k)) & 1]))
            K[r, c] = v
    return K


def split3(K):
    """Exact three-term bf16 split of fp32 K (each term keeps the next 8 bits)."""
    hi = bf16(K)
    r1 = f32(K.astype(np.float64) - hi)
    mid = bf16(r1)
    r2 = f32(r1.astype(np.float64) - mid)
    lo = bf16(r2)
    return hi, mid, lo


def mfma_emulate(xb, terms):
    """Matrix-core order: accumulator from +0, terms lo, mid, hi, each over
    input halves j = 0, 1 (16 products); every product rounded to fp32, every
    addition rounded to fp32 (the most rounding steps any such unit takes)."""
    hi, mid, lo = terms
    x = xb.astype(np.float64)
    acc = np.zeros((xb.shape[0], 32), np.float32)
    for T in (lo, mid, hi):
        for j in range(2):
            for r in range(16 * j, 16 * j + 16):
                p = f32(x[:, r:r + 1] * T[r][None, :].astype(np.float64))
                acc = f32(acc.astype(np.float64) + p)
    return acc


def butterfly_emulate(xb, fs):
    """Butterfly order: stages on index bits 4, 3 (A1, A2) then 2, 1, 0 (A3..A5);
    out = fma(A[0][c], u, fl(A[1][c] w)) for the pair (u at bit 0, w at bit 1),
    the last stage adding to an fma started from +0."""
    F = np.asarray(fs, np.float32)
    v = xb.astype(np.float32).copy()
    for k in range(5):
        bit = 4 - k
        A = F[k]
        out = np.empty_like(v)
        for i in range(32):
            b = (i >> bit) & 1
            i0, i1 = i & ~(1 << bit), i | (1 << bit)
            u, w = v[:, i0], v[:, i1]
            if k < 4:
                prod = f32(np.float64(A[1][b]) * w.astype(np.float64))
            else:
                prod = fma32(A[1][b], w, 0.0)
            out[:, i] = fma32(A[0][b], u, prod)
        v = out
    return v


def subnormal_blocks(n, seed, scale_exp=-130):
    """n blocks of 32 bf16 values N(0,1) * 2^scale_exp (bf16 subnormals, zeros
    and -0 at -130), as fp32 values and bf16 bit patterns."""
    rng = np.random.default_rng(seed)
    bits = I.f32_to_bf16_bits((rng.standard_normal((n, 32)) * 2.0 ** scale_exp).astype(np.float32))
    return I.bf16_bits_to_f32(bits), bits


def exact(bits, fs):
    y, z = O.kq_transform(bits, np.asarray(fs, np.float32)[None])
    return y, z


def test_matrix_core_floor_is_nearly_reached_adversarially():
    # x = 63 * 2^-133 (a bf16 subnormal) and all three bf16 terms equal to
    # 129 * 2^-23 (built directly as terms): each of the 96 products is
    # (63 * 129 / 128) u = 63.49 u and rounds down by 0.49 u, so the emulated
    # error approaches the bound 96 * u/2 = 48 u.
    x = np.full((1, 32), 63 * 2.0 ** -133, np.float32)
    t = np.float32(129 * 2.0 ** -23)  # 8 significant bits: a bf16 value
    T = np.full((32, 32), t, np.float32)
    acc = mfma_emulate(x, (T, T, T))
    y_exact = 96 * 63 * 129 * 2.0 ** -156
    err = np.abs(acc.astype(np.float64) - y_exact) / U
    assert err.max() == pytest.approx(96 * 63 / 128, abs=1e-9)  # 47.25 u
    assert 46 * U < err.max() * U <= P.TOL_ABS


@pytest.mark.parametrize("kind", ["random", "hadamard", "identity"])
def test_matrix_core_order_within_floor(kind):
    worst = 0.0
    for s in range(6):
        fs = {"random": I.random_factors(1, 4200 + s)[0], "hadamard": I.hadamard_factors(1)[0],
              "identity": I.identity_factors(1)[0]}[kind]
        terms = split3(kernel_block_matrix(fs))
        K = kernel_block_matrix(fs).astype(np.float64)
        assert np.array_equal(terms[0].astype(np.float64) + terms[1] + terms[2], K)  # the split is exact
        for e in (-130, -128, -126, -124):
            xv, bits = subnormal_blocks(256, 4300 + s + e, e)
            y, z = exact(bits, fs)
            got = mfma_emulate(xv, terms)
            err = np.abs(got.astype(np.float64) - y)
            # the rounding of K itself to fp32 is a relative error (inside 2e-6 z)
            assert np.all(err <= P.TOL * z + P.TOL_ABS)
            sub = z < 2.0 ** -126
            if sub.any():
                worst = max(worst, float((err[sub] / U).max()))
    print(f"matrix-core order, {kind}: worst subnormal-range error {worst:.2f} u (bound 48 u)")
    assert worst <= 48


@pytest.mark.parametrize("kind", ["random", "hadamard", "lu"])
def test_butterfly_order_within_floor(kind):
    worst, worst_bound = 0.0, 0.0
    for s in range(8):
        if kind == "random":
            fs = I.random_factors(1, 4400 + s)[0]
        elif kind == "hadamard":
            fs = I.hadamard_factors(1)[0]
        else:
            lu = I.random_lu(1, 4500 + s)[0]
            a, b, c = lu[:, 0], lu[:, 1], lu[:, 2]
            fs = np.stack([np.stack([a, b], -1), np.stack([f32(c * a), fma32(c, b, -f32(1.0 / a.astype(np.float64)))],
                                                          -1)], -2).astype(np.float32)
        bound = float(P.abs_floor_units(fs[None])[0])
        worst_bound = max(worst_bound, bound)
        for e in (-130, -128, -126, -124):
            xv, bits = subnormal_blocks(256, 4600 + s + e, e)
            y, z = exact(bits, fs)
            got = butterfly_emulate(xv, fs)
            err = np.abs(got.astype(np.float64) - y)
            assert np.all(err <= P.TOL * z + (bound + 1) * U), (kind, s, e)
            sub = z < 2.0 ** -126
            if sub.any():
                worst = max(worst, float((err[sub] / U).max()))
    print(f"butterfly order, {kind}: worst subnormal-range error {worst:.2f} u, largest bound {worst_bound:.1f} u")
    assert worst <= worst_bound + 1


def test_suite_factor_sets_within_the_floor():
    # every random factor set the suites draw (the per-block sets of every
    # workload, the test seeds) has a butterfly bound below TOL_ABS
    names = ["tiny", "dit_1152", "dit_4608", "mid_2240", "mid_8960", "dbl_3072", "dbl_12288", "sweep_4096",
             "sweep_16384", "sweep_65536"]
    worst = 0.0
    for n in names:
        worst = max(worst, P.abs_floor_units(I.make_factors(n)).max(),
                    P.abs_floor_units(I.random_factors(384, I.factor_seed(n))).max())
    for seed in range(0, 10000, 97):
        worst = max(worst, P.abs_floor_units(I.random_factors(4, seed)).max())
    worst = max(worst, P.abs_floor_units(I.hadamard_factors(1)).max(), P.abs_floor_units(I.random_factors16(256, 7)).max())
    print(f"largest butterfly bound over the suites' factor sets: {worst:.1f} u")
    assert worst * U <= P.TOL_ABS


def test_floor_catches_a_wrong_stage_order():
    # the floor is small enough that a butterfly applying A5 before A1 (a
    # transposed Kronecker order) is caught on subnormal-range blocks
    fs = I.random_factors(1, 4700)[0]
    xv, bits = subnormal_blocks(512, 4701, -120)
    y, z = exact(bits, fs)
    wrong = butterfly_emulate(xv, fs[::-1].copy())
    err = np.abs(wrong.astype(np.float64) - y)
    assert np.any(err > P.TOL * z + P.TOL_ABS)
