"""GPU parity of the 16-element-block quantizer (kq_quantize16,
kq_transform16_f32) against the oracle, through the C ABI.  One shared set
runs on the flat matrix-core kernel, a set per block on the strip kernel when
rows are whole 32-element blocks, the butterfly kernel otherwise.  Transformed
values within 2e-6 z + 2^-146, codes and scales bit-exact except
tolerance-boundary elements (tests/parity.py with 16-element blocks),
identity factors fully bit-exact.  Every case prints its shape and seed
before it touches the GPU."""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from synth import inputs as I
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    import mxfp4_act_quantizer_amd as K
    return K


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def check(K, x, f, label):
    xd, fd = dev_bf16(x), dev_f32(f)
    q, s = K.kq_quantize16(xd, fd)
    y = K.kq_transform16_f32(xd, fd)
    torch.cuda.synchronize()
    q, s, y = q.cpu().numpy(), s.cpu().numpy(), y.cpu().numpy()
    yr, z = O.kq_transform16(x, f)
    worst, outside = P.transform_error(y, yr, z)
    assert outside == 0, f"{label}: {outside} values outside 2e-6 z (worst {worst})"
    qr, sr, y32 = O.kq_quantize16(x, f, want_y32=True)
    ef, bf = P.boundary_flags(z, y32, bw=16)
    res = P.compare(q, s, qr, sr, ef, bf)
    say(f"    transform worst {worst:.2e}; codes {res}")
    assert res["ok"], res
    return res


CASES16 = [(1, 16), (5, 48), (37, 1152), (33, 2240), (9, 4608), (3, 12288), (66, 528)]


@pytest.mark.parametrize("M,d", CASES16, ids=[f"{m}x{d}" for m, d in CASES16])
@pytest.mark.parametrize("sets", ["per_block", "shared"])
def test_kq16_against_oracle(K, M, d, sets):
    seed = 9500 + M + d
    say(f"[kq16] M={M} d={d} sets={sets} seed={seed}")
    x = I.act_dit_lognormal(M, d, seed)[0]
    f = I.random_factors16(d // 16 if sets == "per_block" else 1, seed + 1)
    check(K, x, f, f"{M}x{d}")


def test_kq16_identity_is_bit_exact(K):
    M, d = 40, 1152
    say(f"[kq16 identity] M={M} d={d}")
    x = I.act_sweep_special(M, d, 9600)[0]
    f = np.tile(np.eye(2, dtype=np.float32), (1, 4, 1, 1))
    q, s = K.kq_quantize16(dev_bf16(x), dev_f32(f))
    torch.cuda.synchronize()
    qr, sr = O.kq_quantize16(x, f)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr)
    say(f"    {res}")
    assert res["ok"] and res["code_mismatch"] == 0 and res["scale_mismatch"] == 0


def test_kq16_special_blocks(K):
    # zero, subnormal, NaN and Inf 16-element blocks next to ordinary ones
    M, d = 6, 256
    say(f"[kq16 specials] M={M} d={d}")
    rng = np.random.default_rng(9700)
    v = rng.standard_normal((M, d)).astype(np.float32)
    v[0, 16:32] = 0.0
    v[1, 32:48] *= 2.0 ** -130
    v[2, 48 + 5] = np.nan
    v[3, 64 + 9] = np.inf
    v[4, 80:96] = -0.0
    x = I.f32_to_bf16_bits(v)
    f = I.random_factors16(d // 16, 9701)
    res = check(K, x, f, "specials")
    s = K.kq_quantize16(dev_bf16(x), dev_f32(f))[1].cpu().numpy()
    assert s[2, 3] == 0xFF and s[3, 4] == 0xFF and s[0, 1] == 0x00
    assert res["ok"]


def test_kq16_shared_special_blocks_stay_in_their_block(K):
    # one shared set takes the matrix-core kernel, whose 32 x 32 block pairs
    # two 16-element blocks (I (x) K16): a NaN or Inf in one of them must not
    # reach its partner
    M, d = 6, 256
    say(f"[kq16 shared specials] M={M} d={d}")
    rng = np.random.default_rng(9750)
    v = rng.standard_normal((M, d)).astype(np.float32)
    v[0, 16:32] = 0.0
    v[1, 32:48] *= 2.0 ** -130
    v[2, 48 + 5] = np.nan   # block 3: its partner is block 2
    v[3, 64 + 9] = np.inf   # block 4: its partner is block 5
    v[4, 80:96] = -0.0
    v[5, 0] = -np.inf       # block 0 of the last row
    x = I.f32_to_bf16_bits(v)
    f = I.random_factors16(1, 9751)
    check(K, x, f, "shared specials")
    s = K.kq_quantize16(dev_bf16(x), dev_f32(f))[1].cpu().numpy()
    assert s[2, 3] == 0xFF and s[3, 4] == 0xFF and s[5, 0] == 0xFF and s[0, 1] == 0x00
    assert s[2, 2] != 0xFF and s[3, 5] != 0xFF and s[5, 1] != 0xFF


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dit_4608", "sweep_16384"])
def test_kq16_shared_full_size_sampled_rows(K, name):
    # one shared set at full size, in both launch shapes of the matrix-core
    # kernel (below and above the last-level cache size)
    M, d, _ = I.CONFIGS[name]
    say(f"[kq16 shared full] {name} M={M} d={d}")
    x = I.make_activation(name) if name != "sweep_16384" else I.act_sweep_special(M, d, I.data_seed(name))[0]
    f = I.random_factors16(1, I.factor_seed(name) + 17)
    q, s = K.kq_quantize16(dev_bf16(x), dev_f32(f))
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    rng = np.random.default_rng(9850)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 30)]))
    qr, sr, y32 = O.kq_quantize16(x[rows], f, want_y32=True)
    _, z = O.kq_transform16(x[rows], f)
    ef, bf = P.boundary_flags(z, y32, bw=16)
    res = P.compare(q[rows], s[rows], qr, sr, ef, bf)
    say(f"    {len(rows)} rows: {res}")
    assert res["ok"], res


def test_kq16_empty(K):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s = K.kq_quantize16(x, dev_f32(I.random_factors16(1, 1)))
    torch.cuda.synchronize()
    assert q.shape == (0, 32) and s.shape == (0, 4)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dit_4608", "sweep_4096", "sweep_16384"])
def test_kq16_full_size_sampled_rows(K, name):
    # a set per block on the matrix-core kernel: one resident round of strips
    # (4608, 4096 tokens) and the persistent long runs with the ring of 4
    # (16384 tokens)
    M, d, _ = I.CONFIGS[name]
    say(f"[kq16 full] {name} M={M} d={d}")
    x = I.make_activation(name) if name != "sweep_16384" else I.act_sweep_special(M, d, I.data_seed(name))[0]
    f = I.random_factors16(d // 16, I.factor_seed(name) + 16)
    q, s = K.kq_quantize16(dev_bf16(x), dev_f32(f))
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    rng = np.random.default_rng(9800)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 30)]))
    qr, sr, y32 = O.kq_quantize16(x[rows], f, want_y32=True)
    _, z = O.kq_transform16(x[rows], f)
    ef, bf = P.boundary_flags(z, y32, bw=16)
    res = P.compare(q[rows], s[rows], qr, sr, ef, bf)
    say(f"    {len(rows)} rows: {res}")
    assert res["ok"], res


@pytest.mark.timeout(900)
def test_kq16_per_block_long_run_strips_of_8(K):
    # the persistent long runs in strips of 8 blocks (rows of 70 blocks, so
    # the last strip of each row is ragged) with the ring of 4: the first
    # token count whose automatic shape is that one
    d = 2240
    for M in (65536, 98304, 131072):
        sh = K.kq_launch_shape(M, d)
        if sh["strip"] == 8 and sh["ring"] == 4:
            break
    else:
        pytest.fail(f"no long run in strips of 8 at d={d}: {sh}")
    say(f"[kq16 long run, strips of 8] M={M} d={d} shape={sh}")
    x = I.act_dit_lognormal(M, d, 9870)[0]
    f = I.random_factors16(d // 16, 9871)
    q, s = K.kq_quantize16(dev_bf16(x), dev_f32(f))
    torch.cuda.synchronize()
    q, s = q.cpu().numpy(), s.cpu().numpy()
    rng = np.random.default_rng(9872)
    rows = np.unique(np.concatenate([[0, 31, 32, M - 1], rng.integers(0, M, 28)]))
    qr, sr, y32 = O.kq_quantize16(x[rows], f, want_y32=True)
    _, z = O.kq_transform16(x[rows], f)
    ef, bf = P.boundary_flags(z, y32, bw=16)
    res = P.compare(q[rows], s[rows], qr, sr, ef, bf)
    say(f"    {len(rows)} rows: {res}")
    assert res["ok"], res


CANARY16 = [(67, 1152, "per_block"), (45, 2240, "per_block"), (67, 1168, "per_block"), (67, 1168, "shared")]


@pytest.mark.parametrize("M,d,sets", CANARY16, ids=[f"{m}x{d}-{s}" for m, d, s in CANARY16])
def test_kq16_no_stray_writes(K, M, d, sets):
    # guard bytes around q, s and y; ragged token tiles, ragged strips
    # (d = 2240), rows with an odd number of 16-element blocks (d = 1168)
    x = I.act_dit_lognormal(M, d, 9880 + d)[0]
    f = I.random_factors16(d // 16 if sets == "per_block" else 1, 9881 + d)
    xd, fd = dev_bf16(x), dev_f32(f)
    guard = 4096
    qbuf = torch.full((M * d // 2 + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((M * d // 16 + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
    ybuf = torch.full((M * d + 2 * guard,), 7.0, dtype=torch.float32, device="cuda")
    q = qbuf[guard:guard + M * d // 2].view(M, d // 2)
    s = sbuf[guard:guard + M * d // 16].view(M, d // 16)
    y = ybuf[guard:guard + M * d].view(M, d)
    say(f"[kq16 canary] M={M} d={d} sets={sets}")
    K.kq_quantize16(xd, fd, q, s)
    K.kq_transform16_f32(xd, fd, y)
    torch.cuda.synchronize()
    qb, sb, yb = qbuf.cpu().numpy(), sbuf.cpu().numpy(), ybuf.cpu().numpy()
    assert (qb[:guard] == 0xA5).all() and (qb[-guard:] == 0xA5).all()
    assert (sb[:guard] == 0x5A).all() and (sb[-guard:] == 0x5A).all()
    assert (yb[:guard] == 7.0).all() and (yb[-guard:] == 7.0).all()
    # a second call gives the same bytes
    q2, s2 = K.kq_quantize16(xd, fd)
    torch.cuda.synchronize()
    assert torch.equal(q2, q) and torch.equal(s2, s)
    qr, sr, y32 = O.kq_quantize16(x, f, want_y32=True)
    yr, z = O.kq_transform16(x, f)
    ef, bf = P.boundary_flags(z, y32, bw=16)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr, ef, bf)
    assert res["ok"], res
    worst, outside = P.transform_error(y.cpu().numpy(), yr, z)
    assert outside == 0, worst
