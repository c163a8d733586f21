"""GPU parity of the 16-element-block quantizer (kq_quantize16,
kq_transform16_f32) against the oracle, through the C ABI: transformed
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


def test_kq16_empty(K):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s = K.kq_quantize16(x, dev_f32(I.random_factors16(1, 1)))
    torch.cuda.synchronize()
    assert q.shape == (0, 32) and s.shape == (0, 4)


@pytest.mark.parametrize("name", ["dit_4608", "sweep_4096"])
def test_kq16_full_size_sampled_rows(K, name):
    M, d, _ = I.CONFIGS[name]
    say(f"[kq16 full] {name} M={M} d={d}")
    x = I.make_activation(name)
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
