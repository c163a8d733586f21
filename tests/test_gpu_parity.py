"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Every case prints its name, shape and seed before it touches the GPU.
Bars (see tests/parity.py for the exact rules):
  - kq_transform_f32 values within 2e-6 * z of the exact transform;
  - kq_quantize codes/scales bit-exact except tolerance-boundary elements;
  - sq_quantize, mx_quantize_f32 and kq_quantize with identity factors fully
    bit-exact.
"""
import math
import sys

import numpy as np
import pytest

from oracle import oracle as O
from synth import inputs as I
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

VARIANTS = {"mfma": 1, "butterfly": 2}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")


@pytest.fixture(scope="module")
def K():
    _need_gpu()
    import mxfp4_act_quantizer_amd as K
    return K


@pytest.fixture(scope="module")
def K_lib(K):
    return K


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(x_bits):
    return torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def run_kq(K, x_bits, f, variant, tuning=None):
    x = dev_bf16(x_bits)
    q, s = K.kq_quantize(x, dev_f32(f), variant=variant, tuning=tuning)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def check_kq(K, name, x_bits, f, variant, exact=False, tuning=None):
    M, d = x_bits.shape
    say(f"[kq {name}] M={M} d={d} nT={f.shape[0]} variant={variant} tuning={tuning}")
    qg, sg = run_kq(K, x_bits, f, variant, tuning)
    qr, sr, y32 = O.kq_quantize(x_bits, f, want_y32=True)
    if exact:
        res = P.compare(qg, sg, qr, sr)
    else:
        _, z = O.kq_transform(x_bits, f)
        ef, bf = P.boundary_flags(z, y32)
        res = P.compare(qg, sg, qr, sr, ef, bf)
    say(f"    {res}")
    assert res["ok"], res
    return res


# ---------------------------------------------------------------------------
# transformed values
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("case", ["tiny_shared", "per_block_ragged", "student_t", "hadamard", "lu_factors"])
def test_transform_values_within_tolerance(K, variant, case):
    if case == "tiny_shared":
        x = I.make_activation("tiny")
        f = I.make_factors("tiny")
    elif case == "per_block_ragged":
        x = I.make_activation("dit_1152", M=97)
        f = I.make_factors("dit_1152")
    elif case == "student_t":
        x = I.make_activation("mid_2240", M=45)
        f = I.make_factors("mid_2240")
    elif case == "hadamard":
        x = I.make_activation("sweep_4096", M=33, d=1024)
        f = I.hadamard_factors(1)
    else:
        rng = np.random.default_rng(8)
        f = np.empty((3, 5, 2, 2), np.float32)
        for t in range(3):
            for k in range(5):
                a, b, c = rng.uniform(0.5, 1.5), rng.uniform(-1, 1), rng.uniform(-1, 1)
                f[t, k] = (np.array([[1, 0], [c, 1]]) @ np.array([[a, b], [0, -1 / a]])).astype(np.float32)
        x = I.make_activation("tiny", M=40, d=96)
    M, d = x.shape
    say(f"[transform {case}] M={M} d={d} nT={f.shape[0]} variant={variant}")
    y = K.kq_transform_f32(dev_bf16(x), dev_f32(f), variant=VARIANTS[variant])
    torch.cuda.synchronize()
    yr, z = O.kq_transform(x, f)
    worst, nbad = P.transform_error(y.cpu().numpy(), yr, z)
    say(f"    max |y_gpu - y| / z = {worst:.3e}, elements above 2e-6: {nbad}")
    assert nbad == 0


# ---------------------------------------------------------------------------
# quantized outputs, oracle-sized cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_kq_tiny_config(K, variant):
    check_kq(K, "tiny", I.make_activation("tiny"), I.make_factors("tiny"), VARIANTS[variant])


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("name,M", [("dit_1152", 130), ("dit_4608", 33), ("mid_2240", 70), ("mid_8960", 9),
                                    ("dbl_3072", 72), ("sweep_4096", 21)])
def test_kq_per_block_configs_small_rows(K, variant, name, M):
    x = I.make_activation(name, M=M)
    f = I.make_factors(name)
    check_kq(K, name, x, f, VARIANTS[variant])


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("M,d", [(1, 32), (1, 64), (31, 96), (32, 64), (33, 160), (65, 2240), (257, 32)])
def test_kq_ragged_shapes(K, variant, M, d):
    x = I.make_activation("dit_1152", M=M, d=d, seed=M * 7 + d)
    for shared in (True, False):
        f = I.random_factors(1 if shared else d // 32, M + d)
        check_kq(K, f"ragged shared={shared}", x, f, VARIANTS[variant])


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_kq_identity_is_plain_mxfp4_bit_exact(K, variant):
    x, _, sp = I.act_sweep_special(48, 1536, 5151, special_frac=0.02)
    assert len(sp) > 0
    # a block of -0 and tiny negatives: sign handling must not depend on op order
    x[0, :32] = I.f32_to_bf16_bits(-np.zeros(32, np.float32))
    x[1, 32:64] = I.f32_to_bf16_bits(np.full(32, -1e-40, np.float32))
    for nT in (1, 1536 // 32):
        check_kq(K, f"identity nT={nT}", x, I.identity_factors(nT), VARIANTS[variant], exact=True)


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_kq_hadamard(K, variant):
    x = I.make_activation("sweep_4096", M=40, d=2048)
    check_kq(K, "hadamard", x, I.hadamard_factors(1), VARIANTS[variant])


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_kq_nonfinite_blocks(K, variant):
    x = I.make_activation("tiny", M=8, d=256)
    xf = I.bf16_bits_to_f32(x).copy()
    xf[0, 3] = np.nan
    xf[2, 40] = np.inf
    xf[3, 100] = -np.inf
    x = I.f32_to_bf16_bits(xf)
    qr, sr = O.kq_quantize(x, I.random_factors(8, 3))
    assert sr[0, 0] == 0xFF and sr[2, 1] == 0xFF and sr[3, 3] == 0xFF
    check_kq(K, "nonfinite", x, I.random_factors(8, 3), VARIANTS[variant])


@pytest.mark.parametrize("variant", sorted(VARIANTS))
def test_kq_deterministic_and_no_stray_writes(K, variant):
    M, d = 77, 1152
    x = I.make_activation("dit_1152", M=M)
    f = I.make_factors("dit_1152")
    xd, fd = dev_bf16(x), dev_f32(f)
    guard = 4096
    qbuf = torch.full((M * d // 2 + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((M * d // 32 + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    q = qbuf[guard:guard + M * d // 2].view(M, d // 2)
    s = sbuf[guard:guard + M * d // 32].view(M, d // 32)
    say(f"[canary] M={M} d={d} variant={variant}")
    K.kq_quantize(xd, fd, q, s, variant=VARIANTS[variant])
    torch.cuda.synchronize()
    q1, s1 = q.cpu().numpy().copy(), s.cpu().numpy().copy()
    K.kq_quantize(xd, fd, q, s, variant=VARIANTS[variant])
    torch.cuda.synchronize()
    assert np.array_equal(q1, q.cpu().numpy()) and np.array_equal(s1, s.cpu().numpy())
    qb, sb = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert (qb[:guard] == 0xA5).all() and (qb[-guard:] == 0xA5).all()
    assert (sb[:guard] == 0x5A).all() and (sb[-guard:] == 0x5A).all()


def test_kq_variants_agree_off_boundary(K):
    x = I.make_activation("dbl_3072", M=64)
    f = I.make_factors("dbl_3072")
    qa, sa = run_kq(K, x, f, 1)
    qb, sb = run_kq(K, x, f, 2)
    _, z = O.kq_transform(x, f)
    _, _, y32 = O.kq_quantize(x, f, want_y32=True)
    ef, bf = P.boundary_flags(z, y32)
    res = P.compare(qa, sa, qb, sb, ef, bf)
    say(f"[mfma vs butterfly] {res}")
    assert res["ok"]


def test_kq_empty_is_noop(K):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s = K.kq_quantize(x, dev_f32(I.identity_factors(1)))
    assert q.shape == (0, 32) and s.shape == (0, 2)


def test_kq_misaligned_rejected(K):
    x = torch.zeros((4 * 64 + 8,), dtype=torch.bfloat16, device="cuda")
    xv = x[1:1 + 4 * 64].view(4, 64)  # 2-byte offset
    with pytest.raises(K.KQError) as e:
        K.kq_quantize(xv, dev_f32(I.identity_factors(1)))
    assert e.value.status == K.KQ_ERR_ALIGN


# ---------------------------------------------------------------------------
# SmoothQuant and fp32 MX: fully bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,M", [("tiny", 256), ("dit_4608", 41), ("mid_2240", 33), ("dbl_12288", 17),
                                    ("sweep_4096", 19)])
def test_sq_bit_exact(K, name, M):
    x = I.make_activation(name, M=M)
    scale = I.smoothquant_scale(x)
    M, d = x.shape
    say(f"[sq {name}] M={M} d={d}")
    q, s = K.sq_quantize(dev_bf16(x), dev_f32(scale))
    torch.cuda.synchronize()
    qr, sr = O.sq_quantize(x, scale)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr)
    say(f"    {res}")
    assert res["code_mismatch"] == 0 and res["scale_mismatch"] == 0


def test_sq_ragged_and_odd_scales(K):
    rng = np.random.default_rng(12)
    for M, d in [(1, 32), (5, 96), (37, 2240), (3, 544)]:
        x = I.make_activation("mid_2240", M=M, d=d, seed=M + d)
        scale = np.exp(rng.uniform(-12, 12, d)).astype(np.float32)
        scale[:3] = [1e-30, 3e30, 1.0]
        say(f"[sq ragged] M={M} d={d}")
        q, s = K.sq_quantize(dev_bf16(x), dev_f32(scale))
        torch.cuda.synchronize()
        qr, sr = O.sq_quantize(x, scale)
        res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr)
        assert res["code_mismatch"] == 0 and res["scale_mismatch"] == 0, res


def _special_f32_matrix():
    rng = np.random.default_rng(99)
    rows = []
    grid = np.array([0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7, 7.99], np.float32)
    for E in (-127, -126, -100, -3, 0, 5, 100, 125):
        v = np.resize(grid, 32).astype(np.float32) * np.float32(2.0 ** E if E > -126 else 1.0)
        if E <= -126:
            v = np.ldexp(np.resize(grid, 32).astype(np.float64), E).astype(np.float32)
        v[1::3] *= -1
        rows.append(v)
    rows.append(np.full(32, -0.0, np.float32))
    rows.append(np.ldexp(rng.standard_normal(32), -140).astype(np.float32))  # fp32 subnormals
    rows.append(np.float32(3.4028235e38) * np.sign(rng.standard_normal(32)).astype(np.float32))
    rows.append((rng.standard_normal(32) * 1e-3).astype(np.float32))
    nf = rng.standard_normal(32).astype(np.float32)
    nf[5] = np.nan
    rows.append(nf)
    inf = rng.standard_normal(32).astype(np.float32)
    inf[30] = -np.inf
    rows.append(inf)
    m = np.concatenate(rows).reshape(-1, 64)  # 2 blocks per row
    return m


def test_mx_f32_bit_exact_specials(K):
    x = _special_f32_matrix()
    M, d = x.shape
    say(f"[mx f32 specials] M={M} d={d}")
    q, s = K.mx_quantize_f32(dev_f32(x))
    torch.cuda.synchronize()
    qr, sr = O.mx_quantize_f32(x)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr)
    say(f"    {res}")
    assert res["code_mismatch"] == 0 and res["scale_mismatch"] == 0


@pytest.mark.parametrize("M,d", [(256, 1152), (67, 2240), (3, 12288)])
def test_mx_f32_bit_exact_random(K, M, d):
    rng = np.random.default_rng(M + d)
    x = (rng.standard_normal((M, d)) * np.exp(rng.uniform(-30, 30, (M, 1)))).astype(np.float32)
    say(f"[mx f32] M={M} d={d}")
    q, s = K.mx_quantize_f32(dev_f32(x))
    torch.cuda.synchronize()
    qr, sr = O.mx_quantize_f32(x)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr)
    assert res["code_mismatch"] == 0 and res["scale_mismatch"] == 0, res


def test_mx_f32_exhaustive_bf16_patterns(K):
    # every bf16 bit pattern (as fp32) once, in blocks with controlled maxima
    pats = np.arange(65536, dtype=np.uint32)
    vals = (pats << 16).view(np.float32)
    fin = vals[np.isfinite(vals)]
    rng = np.random.default_rng(4)
    fin = fin[rng.permutation(fin.size)]
    n = (fin.size // 1024) * 1024
    x = fin[:n].reshape(-1, 1024)
    say(f"[mx f32 all bf16 patterns] M={x.shape[0]} d=1024")
    q, s = K.mx_quantize_f32(dev_f32(x))
    torch.cuda.synchronize()
    qr, sr = O.mx_quantize_f32(x)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr)
    assert res["code_mismatch"] == 0 and res["scale_mismatch"] == 0, res


def test_graph_replay_matches_eager(K):
    """The benchmark launches through HIP graphs: every replay must give the
    eager result, with other eager work and synchronisation in between."""
    x = I.make_activation("dit_1152", M=300)
    f = I.make_factors("dit_1152")
    scale = I.smoothquant_scale(x)
    xd, fd, sd = dev_bf16(x), dev_f32(f), dev_f32(scale)
    q_e, s_e = K.kq_quantize(xd, fd)
    qs_e, ss_e = K.sq_quantize(xd, sd)
    torch.cuda.synchronize()
    q_e, s_e, qs_e, ss_e = (t.cpu().numpy() for t in (q_e, s_e, qs_e, ss_e))
    q = torch.empty((300, 576), dtype=torch.uint8, device="cuda")
    s = torch.empty((300, 36), dtype=torch.uint8, device="cuda")
    qs = torch.empty_like(q)
    ss = torch.empty_like(s)
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        K.kq_quantize(xd, fd, q, s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cs):
            K.kq_quantize(xd, fd, q, s, stream=cs)
            K.sq_quantize(xd, sd, qs, ss, stream=cs)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"[graph replay {rep}]")
        q.fill_(0)
        qs.fill_(0)
        s.zero_()
        ss.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), q_e) and np.array_equal(s.cpu().numpy(), s_e)
        assert np.array_equal(qs.cpu().numpy(), qs_e) and np.array_equal(ss.cpu().numpy(), ss_e)
        _ = (xd.float() * 2).sum().item()  # unrelated eager work between replays


def test_copy_ceiling_kernel_output(K):
    # the benchmark's 4:1 measurement copies, every form: word i of dst = xor
    # of the four words of src piece i (the ring forms, which mirror the flat
    # quantizer's lane layout, write each 64-byte group's words in the order
    # 0, 2, 1, 3); nothing past dst's n16 words is written
    for n16 in (64, 64 * 255, 64 * (2048 * 4 + 77)):
        rng = np.random.default_rng(n16)
        src = rng.integers(0, 2**32, size=4 * n16, dtype=np.uint32)
        s_dev = torch.from_numpy(src.view(np.int32)).cuda()
        want = np.bitwise_xor.reduce(src.reshape(n16, 4), axis=1)
        for form in range(K.KQ_COPY_FORMS):
            say(f"[copy41] pieces={n16} form={form}")
            d_dev = torch.zeros(n16 + 64, dtype=torch.int32, device="cuda")
            K.measure_copy41(s_dev, d_dev[:n16], form=form)
            torch.cuda.synchronize()
            got = d_dev.cpu().numpy().view(np.uint32)
            exp = want.reshape(-1, 4)[:, [0, 2, 1, 3]].ravel() if form >= 6 else want
            assert np.array_equal(got[:n16], exp), form
            assert not got[n16:].any(), form


@pytest.mark.parametrize("ring", [2, 4])
@pytest.mark.parametrize("strip", [4, 8, 16])
@pytest.mark.parametrize("M,d,shared", [(67, 1152, False), (33, 160, True), (130, 4608, False), (5, 544, False)])
def test_kq_mfma_strip_widths(K, strip, ring, M, d, shared):
    # every workgroup strip width and register ring depth of the strip kernel,
    # forced, on ragged shapes (blocks past the row end inside a strip, rows
    # past M inside a tile)
    x, _ = I.act_gaussian_outliers(M, d, 7000 + M + d, max(1, d // 100), 50.0)
    f = I.random_factors(1 if shared else d // 32, 7100 + d)
    tn = {"mfma_strip": strip, "mfma_ring": ring}
    sh = K.kq_launch_shape(M, d, tuning=tn)
    assert sh["strip"] == strip and sh["ring"] == ring
    check_kq(K, f"strip={strip} shared={shared}", x, f, VARIANTS["mfma"], tuning=tn)
    y = K.kq_transform_f32(dev_bf16(x), dev_f32(f), variant=VARIANTS["mfma"], tuning=tn)
    torch.cuda.synchronize()
    yr, z = O.kq_transform(x, f)
    err = np.abs(y.cpu().numpy().astype(np.float64) - yr)
    assert np.all(err <= P.TOL * z + P.TOL_ABS), float((err / (z + 1e-300)).max())


# The automatic launch shapes of the strip kernel the library documents for
# MI355X (256 CUs), so a change of the launch rules shows up here: the
# persistent round of long runs (a ring of 4 tiles; 2 elsewhere), the
# one-round-per-CU shape of mid-size runs, the XCD-grouped round
# at 8192 x 4608 and contiguous groups of 3 tiles in strips of 4 at 8192 x 1152.
AUTO_SHAPES = [((65536, 12288), dict(strip=16, tiles_per_wg=205, interleave=1, flat=1, grid=240, nt_codes=1, ring=4)),
               ((16384, 12288), dict(strip=16, tiles_per_wg=52, interleave=1, flat=1, grid=240, nt_codes=1, ring=4)),
               ((8192, 4608), dict(strip=16, tiles_per_wg=11, interleave=1, flat=0, grid=216, nt_codes=0, ring=2)),
               ((8192, 1152), dict(strip=4, tiles_per_wg=3, interleave=0, flat=0, grid=792, nt_codes=0, ring=2)),
               ((4608, 3072), dict(strip=8, tiles_per_wg=7, interleave=1, flat=1, grid=252, nt_codes=0, ring=2)),
               ((4608, 12288), dict(strip=16, tiles_per_wg=16, interleave=1, flat=1, grid=216, nt_codes=0, ring=2)),
               ((4096, 12288), dict(strip=16, tiles_per_wg=16, interleave=1, flat=1, grid=192, nt_codes=0, ring=2)),
               ((2048, 8960), dict(strip=8, tiles_per_wg=10, interleave=1, flat=1, grid=245, nt_codes=0, ring=2))]


@pytest.mark.parametrize("shape,want", AUTO_SHAPES, ids=[f"{m}x{d}" for (m, d), _ in AUTO_SHAPES])
def test_automatic_launch_shapes(K, shape, want):
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the documented shapes are those of a 256-CU MI355X")
    M, d = shape
    got = K.kq_launch_shape(M, d)
    say(f"[launch shape] {M}x{d}: {got}")
    assert got == want


# ---------------------------------------------------------------------------
# K2 form: factor sets as 15 LU scalars, rebuilt in the kernel
# ---------------------------------------------------------------------------
def _check_values(y_gpu, yr, z, what):
    err = np.abs(y_gpu.astype(np.float64) - yr)
    bad = err > P.TOL * z + P.TOL_ABS
    assert not bad.any(), f"{what}: {int(bad.sum())} values outside 2e-6*z, worst {float((err / (z + 1e-300)).max())}"


LU_CASES = [(256, 1152, True), (130, 4608, False), (67, 2240, False), (33, 160, True), (1, 32, False),
            (5, 12288, False)]


@pytest.mark.parametrize("M,d,shared", LU_CASES, ids=[f"{m}x{d}-{'shared' if s else 'perblock'}"
                                                       for m, d, s in LU_CASES])
def test_kq_lu_against_oracle(K, M, d, shared):
    x, _ = I.act_gaussian_outliers(M, d, 8000 + M + d, max(1, d // 100), 50.0)
    lu = I.random_lu(1 if shared else d // 32, 8100 + d)
    say(f"[kq_lu] M={M} d={d} nT={lu.shape[0]}")
    xd, ld = dev_bf16(x), dev_f32(lu)
    q, s = K.kq_quantize_lu(xd, ld)
    y = K.kq_transform_lu_f32(xd, ld)
    torch.cuda.synchronize()
    qr, sr, y32 = O.kq_quantize_lu(x, lu, want_y32=True)
    yr, z = O.kq_transform_lu(x, lu)
    _check_values(y.cpu().numpy(), yr, z, "kq_transform_lu_f32")
    ef, bf = P.boundary_flags(z, y32)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr, ef, bf)
    say(f"    {res}")
    assert res["ok"], res


@pytest.mark.parametrize("M,d", [(200, 1152), (96, 4608)])
def test_kq_lu_equals_factor_path_bit_exact(K, M, d):
    # the kernel forms each factor from its LU scalars with the same fp32
    # operations as kq_lu_factors on the host, so both paths see identical
    # blocks: codes, scales and transformed values agree bit for bit
    x, _ = I.act_gaussian_outliers(M, d, 8200 + d, max(1, d // 100), 50.0)
    for shared in (True, False):
        lu = I.random_lu(1 if shared else d // 32, 8300 + d + shared)
        f = K.kq_lu_factors(lu)
        say(f"[kq_lu == kq(kq_lu_factors)] M={M} d={d} nT={lu.shape[0]}")
        xd = dev_bf16(x)
        q1, s1 = K.kq_quantize_lu(xd, dev_f32(lu))
        q2, s2 = K.kq_quantize(xd, dev_f32(f), variant=VARIANTS["mfma"])
        y1 = K.kq_transform_lu_f32(xd, dev_f32(lu))
        y2 = K.kq_transform_f32(xd, dev_f32(f), variant=VARIANTS["mfma"])
        torch.cuda.synchronize()
        assert torch.equal(q1, q2) and torch.equal(s1, s2)
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_kq_lu_hadamard_init_and_nonfinite(K):
    # Hadamard initialisation: within tolerance of the oracle's K2 path;
    # a = 0 makes the set's blocks non-finite (scale 0xFF, codes 0)
    M, d = 40, 256
    x, _ = I.act_gaussian_outliers(M, d, 8400, 3, 30.0)
    check_lu = I.hadamard_lu(d // 32)
    say(f"[kq_lu hadamard] M={M} d={d}")
    q, s = K.kq_quantize_lu(dev_bf16(x), dev_f32(check_lu))
    torch.cuda.synchronize()
    qr, sr, y32 = O.kq_quantize_lu(x, check_lu, want_y32=True)
    _, z = O.kq_transform_lu(x, check_lu)
    ef, bf = P.boundary_flags(z, y32)
    assert P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr, ef, bf)["ok"]
    bad = check_lu.copy()
    bad[3, 2, 0] = 0.0  # a = 0 in factor A3 of set 3
    say(f"[kq_lu a=0] M={M} d={d}")
    q, s = K.kq_quantize_lu(dev_bf16(x), dev_f32(bad))
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    q = q.cpu().numpy()
    assert np.all(s[:, 3] == 0xFF) and np.all(q[:, 48:64] == 0)
    # every other block as the oracle gives it for the same scalars (same flags:
    # their blocks are unchanged)
    qb, sb = O.kq_quantize_lu(x, bad)
    assert np.all(sb[:, 3] == 0xFF) and np.all(qb[:, 48:64] == 0)
    assert P.compare(q, s, qb, sb, ef, bf)["ok"]


# ---------------------------------------------------------------------------
# Walsh-Hadamard-32 comparison kernel
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,d", [(256, 1152), (67, 2240), (33, 160), (1, 32), (130, 4608), (3, 12288)])
def test_fwht_against_oracle(K, M, d):
    x, _ = I.act_gaussian_outliers(M, d, 8500 + M + d, max(1, d // 100), 50.0)
    say(f"[fwht] M={M} d={d}")
    xd = dev_bf16(x)
    q, s = K.fwht_quantize(xd)
    y = K.fwht_transform_f32(xd)
    torch.cuda.synchronize()
    qr, sr, y32 = O.fwht_quantize(x, want_y32=True)
    yr, z = O.fwht_transform(x)
    _check_values(y.cpu().numpy(), yr, z, "fwht_transform_f32")
    ef, bf = P.boundary_flags(z, y32)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr, ef, bf)
    say(f"    {res}")
    assert res["ok"], res


def test_fwht_special_blocks(K):
    # all-zero, all -0, subnormal, NaN and Inf blocks; -0 must never give code 8
    M, d = 6, 192
    xf = np.zeros((M, d), np.float32)
    xf[1] = -0.0
    xf[2, :32] = np.float32(2.0 ** -130) * np.arange(1, 33, dtype=np.float32)
    xf[3, 40] = np.nan
    xf[4, 70] = np.inf
    xf[5] = np.linspace(-3, 3, d, dtype=np.float32)
    x = I.f32_to_bf16_bits(xf)
    say(f"[fwht special] M={M} d={d}")
    q, s = K.fwht_quantize(dev_bf16(x))
    torch.cuda.synchronize()
    qr, sr, y32 = O.fwht_quantize(x, want_y32=True)
    _, z = O.fwht_transform(x)
    assert sr[3, 1] == 0xFF and sr[4, 2] == 0xFF
    ef, bf = P.boundary_flags(z, y32)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr, ef, bf)
    assert res["ok"], res
    assert np.all(q.cpu().numpy()[:2] == 0) and np.all(s.cpu().numpy()[:2] == 0)


def test_lu_fwht_empty(K):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s = K.kq_quantize_lu(x, dev_f32(I.hadamard_lu(1)))
    q2, s2 = K.fwht_quantize(x)
    torch.cuda.synchronize()
    assert q.shape == (0, 32) and s2.shape == (0, 2)


# ---------------------------------------------------------------------------
# W4A4 consumer: MXFP4 x MXFP4 on the block-scaled matrix cores
# ---------------------------------------------------------------------------
def _mx_operand(rows, K, seed, scale_spread=6.0):
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal((rows, K)) * np.exp(rng.uniform(-scale_spread, scale_spread, (rows, 1)))).astype(np.float32)
    q, s = O.mx_quantize_f32(y)
    return q, s


def _gemm_tol(K, mag):
    # fp32 accumulation: one rounding per 64-wide k step, plus the last; a
    # factor 2 of margin for the order inside a step
    return (K // 64 + 2) * 2.0 ** -23 * mag


GEMM_CASES = [(128, 128, 256), (200, 72, 160), (1, 1, 32), (257, 130, 1152), (64, 300, 4608), (33, 129, 96)]


@pytest.mark.parametrize("M,N,Kd", GEMM_CASES, ids=[f"{m}x{n}x{k}" for m, n, k in GEMM_CASES])
def test_mx_gemm_against_oracle(K_lib, M, N, Kd):
    qa, sa = _mx_operand(M, Kd, 9000 + M)
    qb, sb = _mx_operand(N, Kd, 9100 + N)
    say(f"[mx_gemm] M={M} N={N} K={Kd}")
    d = [torch.from_numpy(a).cuda() for a in (qa, sa, qb, sb)]
    out = K_lib.mx_gemm(*d)
    outb = K_lib.mx_gemm(*d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, mag = O.mx_gemm(qa, sa, qb, sb)
    o = out.cpu().numpy().astype(np.float64)
    err = np.abs(o - ref)
    assert np.all(err <= _gemm_tol(Kd, mag) + 1e-300), float((err / (mag + 1e-300)).max())
    # bf16 output: round to nearest even of the same fp32 sums
    rne = torch.from_numpy(out.cpu().numpy()).to(torch.bfloat16)
    assert torch.equal(outb.cpu().view(torch.int16), rne.view(torch.int16))


# Shapes on the persistent path (K % 128 == 0, 16-byte output pieces):
# a k range ending half way through a 256-wide chunk, one chunk per tile
# (the epilogue after every chunk), ragged M and N, and more tiles than
# resident workgroups (528 tiles: some workgroups run two).
PERSIST_CASES = [(1000, 520, 384), (300, 4104, 640), (64, 64, 128), (129, 136, 256), (4160, 2048, 256)]


@pytest.mark.parametrize("M,N,Kd", PERSIST_CASES, ids=[f"{m}x{n}x{k}" for m, n, k in PERSIST_CASES])
def test_mx_gemm_persistent_against_oracle(K_lib, M, N, Kd):
    qa, sa = _mx_operand(M, Kd, 9600 + M)
    qb, sb = _mx_operand(N, Kd, 9700 + N)
    say(f"[mx_gemm persistent] M={M} N={N} K={Kd}")
    d = [torch.from_numpy(a).cuda() for a in (qa, sa, qb, sb)]
    out = K_lib.mx_gemm(*d)
    outb = K_lib.mx_gemm(*d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # the oracle on 40 sampled rows, both ends of the first and last row tiles
    rng = np.random.default_rng(9800 + M)
    rows = np.unique(np.concatenate([[0, 127 % M, M - 1, max(M - 128, 0)], rng.integers(0, M, 36)]))
    ref, mag = O.mx_gemm(qa[rows], sa[rows], qb, sb)
    o = out.cpu().numpy()[rows].astype(np.float64)
    err = np.abs(o - ref)
    assert np.all(err <= _gemm_tol(Kd, mag) + 1e-300), float((err / (mag + 1e-300)).max())
    rne = torch.from_numpy(out.cpu().numpy()).to(torch.bfloat16)
    assert torch.equal(outb.cpu().view(torch.int16), rne.view(torch.int16))


@pytest.mark.parametrize("M,N,Kd", [(8192, 3456, 1152), (1000, 520, 384), (64, 64, 128), (4160, 2048, 256)],
                         ids=["dit_qkv", "ragged", "one_chunk", "two_tiles_per_wg"])
def test_mx_gemm_kernels_agree(K_lib, M, N, Kd):
    # The persistent kernels (k chunks of 256 and of 128) and the per-tile
    # kernel accumulate the same fp32 sums in the same k order: outputs equal
    # bit for bit, in both output types.
    qa, sa = _mx_operand(M, Kd, 9900 + M)
    qb, sb = _mx_operand(N, Kd, 9901 + N)
    d = [torch.from_numpy(a).cuda() for a in (qa, sa, qb, sb)]
    for dt in (torch.float32, torch.bfloat16):
        outs = []
        for v in (1, 2, 3):
            say(f"[mx_gemm kernels] M={M} N={N} K={Kd} dtype={dt} variant={v}")
            outs.append(K_lib.mx_gemm(*d, out_dtype=dt, tuning={"gemm_kernel": v}))
        torch.cuda.synchronize()
        iv = torch.int32 if dt == torch.float32 else torch.int16
        for o in outs[1:]:
            assert torch.equal(o.view(iv), outs[0].view(iv))


def test_mx_gemm_output_alignment_and_guards(K_lib):
    # The product written into caller buffers that start 4 or 2 bytes past a
    # 16-byte boundary (element-wise stores) must equal the one written into
    # an aligned buffer (16-byte row pieces), and nothing outside [M, N] is
    # touched in either case.
    M, N, Kd = 96, 136, 320
    qa, sa = _mx_operand(M, Kd, 9400)
    qb, sb = _mx_operand(N, Kd, 9401)
    d = [torch.from_numpy(a).cuda() for a in (qa, sa, qb, sb)]
    for dt, off in ((torch.float32, 4), (torch.float32, 1), (torch.bfloat16, 8), (torch.bfloat16, 2),
                    (torch.bfloat16, 1)):
        say(f"[mx_gemm out] dtype={dt} element offset={off}")
        buf = torch.full((M * N + off + 16,), float("nan"), dtype=dt, device="cuda")
        out = buf[off:off + M * N].view(M, N)
        K_lib.mx_gemm(*d, out=out)
        ref = K_lib.mx_gemm(*d, out_dtype=dt)
        torch.cuda.synchronize()
        iv = torch.int32 if dt == torch.float32 else torch.int16
        assert torch.equal(out.cpu().view(iv), ref.cpu().view(iv))
        assert torch.isnan(buf[:off].float()).all() and torch.isnan(buf[off + M * N:].float()).all()


def test_mx_gemm_nan_scale_and_zero_blocks(K_lib):
    M, N, Kd = 64, 64, 128
    qa, sa = _mx_operand(M, Kd, 9200)
    qb, sb = _mx_operand(N, Kd, 9201)
    sa[5, 2] = 0xFF            # NaN block in row 5
    qb[7, :] = 0               # column 7 all +0 codes
    say(f"[mx_gemm special] M={M} N={N} K={Kd}")
    out = K_lib.mx_gemm(*[torch.from_numpy(a).cuda() for a in (qa, sa, qb, sb)])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    ref, mag = O.mx_gemm(qa, sa, qb, sb)
    assert np.all(np.isnan(o[5])) and np.all(np.isnan(ref[5]))
    keep = np.ones(M, bool)
    keep[5] = False
    assert np.all(o[keep, 7] == 0.0)
    assert np.all(np.abs(o[keep] - ref[keep]) <= _gemm_tol(Kd, mag[keep]) + 1e-300)


def test_w4a4_end_to_end_invariance(K_lib):
    # Y = X W^T through the quantized path: activations transformed and
    # quantized by kq_quantize, weights folded (kq_fold_weight) and quantized
    # (mx_quantize_f32), product on the matrix cores.  With outlier channels in
    # X, the Hadamard-initialised transform must beat plain MXFP4 (identity
    # factors) on output error, and every GPU product must match the oracle's
    # product of the same codes.
    M, d, N = 256, 1152, 384
    x = I.make_activation("dit_1152", M=M)
    rng = np.random.default_rng(9300)
    W = (rng.standard_normal((N, d)) / math.sqrt(d)).astype(np.float32)
    Xf = I.bf16_bits_to_f32(x).astype(np.float64)
    Y_ref = Xf @ W.astype(np.float64).T
    errs = {}
    for label, f in (("identity", I.identity_factors(1)), ("hadamard", I.hadamard_factors(d // 32)),
                     ("lu_random", K_lib.kq_lu_factors(I.random_lu(d // 32, 9301)))):
        say(f"[w4a4] {label} M={M} d={d} N={N}")
        qa, sa = K_lib.kq_quantize(dev_bf16(x), dev_f32(f))
        Wf = K_lib.kq_fold_weight(W, f)
        qb, sb = K_lib.mx_quantize_f32(torch.from_numpy(Wf).cuda())
        Y = K_lib.mx_gemm(qa, sa, qb, sb)
        torch.cuda.synchronize()
        Yn = Y.cpu().numpy().astype(np.float64)
        ref, mag = O.mx_gemm(qa.cpu().numpy(), sa.cpu().numpy(), qb.cpu().numpy(), sb.cpu().numpy())
        assert np.all(np.abs(Yn - ref) <= _gemm_tol(d, mag) + 1e-300)
        errs[label] = float(np.linalg.norm(Yn - Y_ref) / np.linalg.norm(Y_ref))
    say(f"    relative output error {errs}")
    assert all(np.isfinite(v) for v in errs.values())
    assert errs["hadamard"] < errs["identity"]
