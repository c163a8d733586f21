"""GPU parity of the flat form of the MFMA quantizer (one shared factor set):
the 32 columns of a matrix-core tile are 32 consecutive blocks of the
flattened input, so it has its own tail handling (a last unit of fewer than 32
blocks), its own load layout (two contiguous 1 KB loads and a 16-lane row swap
per unit) and its own work split (every G-th unit per wave).

Checked here: against the oracle on ragged flat lengths, with NaN/Inf blocks,
the transform export and the LU form; bit for bit against the strip kernel
(same transform, other data path) over grid sizes that give every wave from
one to many units; no writes outside q and s.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from synth import inputs as I
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FLAT = {"shared_form": 2}
STRIP = {"shared_form": 1}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    import mxfp4_act_quantizer_amd as K
    return K


def dev_bf16(x_bits):
    return torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def quantize(K, x_bits, f, tuning):
    q, s = K.kq_quantize(dev_bf16(x_bits), dev_f32(f), variant=1, tuning=tuning)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


# flat lengths M*d/32 of 1, 9, 93, 165, 257, 1920 (60 whole units), 2412 and
# 18720 blocks: single blocks, a lone partial unit, partial last units, whole units
RAGGED = [(1, 32), (3, 96), (31, 96), (33, 160), (257, 32), (5, 12288), (67, 1152), (130, 4608)]


@pytest.mark.parametrize("M,d", RAGGED, ids=[f"{m}x{d}" for m, d in RAGGED])
def test_flat_against_oracle(K, M, d):
    x, _ = I.act_gaussian_outliers(M, d, 9100 + M + d, max(1, d // 100), 50.0)
    f = I.random_factors(1, 9200 + d)
    say(f"[flat kq] M={M} d={d} blocks={M * d // 32}")
    qg, sg = quantize(K, x, f, FLAT)
    qr, sr, y32 = O.kq_quantize(x, f, want_y32=True)
    _, z = O.kq_transform(x, f)
    ef, bf = P.boundary_flags(z, y32)
    res = P.compare(qg, sg, qr, sr, ef, bf)
    say(f"    {res}")
    assert res["ok"], res
    # transform export through the same kernel
    y = K.kq_transform_f32(dev_bf16(x), dev_f32(f), variant=1, tuning=FLAT)
    torch.cuda.synchronize()
    yr, z = O.kq_transform(x, f)
    worst, nbad = P.transform_error(y.cpu().numpy(), yr, z)
    say(f"    transform: max |y_gpu - y| / z = {worst:.3e}, outside the bound: {nbad}")
    assert nbad == 0


def test_flat_identity_and_nonfinite(K):
    # identity factors: plain MXFP4 bit for bit, special blocks included
    x = I.make_activation("tiny", M=40, d=256)
    xf = I.bf16_bits_to_f32(x).copy()
    xf[0, 3] = np.nan
    xf[2, 40] = np.inf
    xf[3, 100] = -np.inf
    xf[5, 64:96] = 0.0
    xf[6, 96:128] = 1e-39  # fp32 subnormal magnitude: bf16 keeps it, the scale byte is 0
    x = I.f32_to_bf16_bits(xf)
    say("[flat identity/nonfinite] M=40 d=256")
    qg, sg = quantize(K, x, I.identity_factors(1), FLAT)
    qr, sr = O.mx_quantize_f32(I.bf16_bits_to_f32(x))
    assert np.array_equal(qg, qr) and np.array_equal(sg, sr)
    assert sg[0, 0] == 0xFF and sg[2, 1] == 0xFF and sg[3, 3] == 0xFF
    f = I.random_factors(1, 31)
    qg, sg = quantize(K, x, f, FLAT)
    qr, sr, y32 = O.kq_quantize(x, f, want_y32=True)
    _, z = O.kq_transform(x, f)
    ef, bf = P.boundary_flags(z, y32)
    res = P.compare(qg, sg, qr, sr, ef, bf)
    say(f"    random factors: {res}")
    assert res["ok"], res


def test_flat_lu_against_oracle(K):
    # the K2 form with one shared set takes the flat kernel by default
    x = I.make_activation("dit_1152", M=67)
    lu = I.random_lu(1, 9500)
    say("[flat lu] M=67 d=1152")
    q, s = K.kq_quantize_lu(dev_bf16(x), dev_f32(lu))
    y = K.kq_transform_lu_f32(dev_bf16(x), dev_f32(lu))
    torch.cuda.synchronize()
    qr, sr, y32 = O.kq_quantize_lu(x, lu, want_y32=True)
    yr, z = O.kq_transform_lu(x, lu)
    ef, bf = P.boundary_flags(z, y32)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr, ef, bf)
    say(f"    {res}")
    assert res["ok"], res
    worst, nbad = P.transform_error(y.cpu().numpy(), yr, z)
    assert nbad == 0, worst


# grid sizes (workgroups of 4 waves): one wave per unit up to many units per
# wave, so the ring's steady state and every tail length are exercised
@pytest.mark.parametrize("M,d", [(4096, 1152), (999, 2240), (2048, 12288)], ids=["4096x1152", "999x2240",
                                                                                  "2048x12288"])
def test_flat_equals_strip_kernel(K, M, d):
    x, _ = I.act_gaussian_outliers(M, d, 9300 + M, max(1, d // 100), 50.0)
    f = I.random_factors(1, 9400 + d)
    xd, fd = dev_bf16(x), dev_f32(f)
    say(f"[flat vs strip] M={M} d={d}")
    qs, ss = K.kq_quantize(xd, fd, variant=1, tuning=STRIP)
    ys = K.kq_transform_f32(xd, fd, variant=1, tuning=STRIP)
    for tn in (FLAT, dict(FLAT, flat_wgs=1), dict(FLAT, flat_wgs=3, flat_ring=3), dict(FLAT, flat_wgs=37),
               dict(FLAT, flat_ring=3), dict(FLAT, flat_ring=2, flat_wgs=256), dict(FLAT, code_stores=2),
               dict(FLAT, code_stores=2, flat_ring=3, flat_wgs=5), dict(FLAT, code_stores=1, flat_wgs=1000)):
        say(f"    tuning {tn}")
        qf, sf = K.kq_quantize(xd, fd, variant=1, tuning=tn)
        torch.cuda.synchronize()
        assert torch.equal(qf, qs) and torch.equal(sf, ss), tn
    for tn in (dict(FLAT, flat_wgs=5), dict(FLAT, flat_ring=3, flat_wgs=7)):
        yf = K.kq_transform_f32(xd, fd, variant=1, tuning=tn)
        torch.cuda.synchronize()
        assert torch.equal(yf, ys), tn


def test_flat_no_stray_writes(K):
    # a partial last unit (2412 blocks) with guard bytes around q and s
    M, d = 67, 1152
    x = I.make_activation("dit_1152", M=M)
    f = I.hadamard_factors(1)
    xd, fd = dev_bf16(x), dev_f32(f)
    guard = 4096
    qbuf = torch.full((M * d // 2 + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((M * d // 32 + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    ybuf = torch.full((M * d + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    q = qbuf[guard:guard + M * d // 2].view(M, d // 2)
    s = sbuf[guard:guard + M * d // 32].view(M, d // 32)
    y = ybuf[guard:guard + M * d].view(M, d)
    say(f"[flat canary] M={M} d={d}")
    for tn in (FLAT, dict(FLAT, flat_wgs=1), dict(FLAT, flat_wgs=2, flat_ring=3), dict(FLAT, flat_ring=3)):
        K.kq_quantize(xd, fd, q, s, variant=1, tuning=tn)
        K.kq_transform_f32(xd, fd, y, variant=1, tuning=tn)
        torch.cuda.synchronize()
        qb, sb, yb = qbuf.cpu().numpy(), sbuf.cpu().numpy(), ybuf.cpu().numpy()
        assert (qb[:guard] == 0xA5).all() and (qb[-guard:] == 0xA5).all()
        assert (sb[:guard] == 0x5A).all() and (sb[-guard:] == 0x5A).all()
        assert (yb[:guard] == 7.0).all() and (yb[-guard:] == 7.0).all()
    qr, sr = O.kq_quantize(x, f)
    _, z = O.kq_transform(x, f)
    _, _, y32 = O.kq_quantize(x, f, want_y32=True)
    ef, bf = P.boundary_flags(z, y32)
    assert P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr, ef, bf)["ok"]


# The automatic shapes the library documents for MI355X (256 CUs): a ring of 2
# units at two workgroups per CU while x, q and s fit the last-level cache, a
# ring of 3 at one per CU with nontemporal code stores above it; small inputs
# get one wave per unit.
FLAT_SHAPES = [((65536, 12288), dict(ring=3, workgroups=256, nt_codes=1)),
               ((16384, 12288), dict(ring=3, workgroups=256, nt_codes=1)),
               ((4608, 12288), dict(ring=2, workgroups=512, nt_codes=0)),
               ((8192, 4608), dict(ring=2, workgroups=512, nt_codes=0)),
               ((8192, 1152), dict(ring=2, workgroups=512, nt_codes=0)),
               ((256, 1152), dict(ring=2, workgroups=72, nt_codes=0))]


@pytest.mark.parametrize("shape,want", FLAT_SHAPES, ids=[f"{m}x{d}" for (m, d), _ in FLAT_SHAPES])
def test_flat_automatic_launch_shapes(K, shape, want):
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the documented shapes are those of a 256-CU MI355X")
    got = K.kq_flat_launch_shape(*shape)
    say(f"[flat launch shape] {shape}: {got}")
    assert got == want
