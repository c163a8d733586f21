"""GPU parity of the AdaLN front-end (kq_adaln_quantize, adaln_modulate)
against the oracle, through the C ABI.

Bars:
  - adaln_modulate's bf16 x equals the oracle's x rounded to bf16, except
    elements the oracle flags as within its margin of a bf16 rounding
    midpoint (counted; none are expected on these inputs);
  - kq_adaln_quantize's codes and scales equal the oracle's MXFP4 of the
    transform of that x under tests/parity.py's rules, with every block that
    holds a flagged x element flagged as well;
  - kq_adaln_quantize equals kq_quantize(adaln_modulate(h)) bit for bit (the
    fused kernels compute what the unfused pipeline stores and reads back),
    in the two-launch forms (the default) and in the one-launch form (whole
    rows in LDS, selected by the tuning);
    with the butterfly second pass selected it equals
    kq_quantize_ex(adaln_modulate(h), BUTTERFLY) bit for bit.
Every case prints its name, shape and seed before it touches the GPU.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from synth import inputs as I
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

EPS = 1e-6


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


def bits(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def oracle_codes(h, shift, scale, T, f):
    """The oracle's x (bf16 bits), its flags, codes, scales and the element /
    block flags for the codes."""
    x, xb, xfl = O.adaln(h, shift, scale, T, EPS)
    qr, sr, y32 = O.kq_quantize(xb, f, want_y32=True)
    _, z = O.kq_transform(xb, f)
    ef, bf = P.boundary_flags(z, y32)
    M, d = h.shape
    xblk = xfl.reshape(M, d // 32, 32).any(axis=2)
    bf = bf | xblk
    ef = ef | np.repeat(xblk, 32, axis=1)
    return xb, xfl, qr, sr, ef, bf


def run_gpu(K, h, shift, scale, T, f):
    hd, sh, sc, fd = dev_bf16(h), dev_f32(shift), dev_f32(scale), dev_f32(f)
    q, s = K.kq_adaln_quantize(hd, sh, sc, T, EPS, fd)
    x = K.adaln_modulate(hd, sh, sc, T, EPS)
    q2, s2 = K.kq_quantize(x, fd)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy(), bits(x), q2.cpu().numpy(), s2.cpu().numpy()


def check(K, h, shift, scale, T, f, label):
    M, d = h.shape
    q, s, xg, q2, s2 = run_gpu(K, h, shift, scale, T, f)
    xb, xfl, qr, sr, ef, bf = oracle_codes(h, shift, scale, T, f)
    x_mis = xg != xb
    assert not np.any(x_mis & ~xfl), f"{label}: {int((x_mis & ~xfl).sum())} unflagged x mismatches"
    res = P.compare(q, s, qr, sr, ef, bf)
    say(f"    x flagged {int(xfl.sum())}, x mismatches {int(x_mis.sum())}; codes {res}")
    assert res["ok"], res
    assert np.array_equal(q, q2) and np.array_equal(s, s2), "fused != unfused"
    return res


# (M, d, tokens per sample): ragged row counts against runs of 8 rows and
# pipeline stages of 4, samples that end inside a run, widths from one block
# to past several 512-channel column tiles
# Also samples of 32 tokens and more: sample boundaries inside 32-row tiles
# (T = 40, 35, 33), a ragged last tile, one sample for all rows, and widths
# from 96 to 12288 channels.
ADALN_CASES = [(1, 32, 1), (5, 64, 2), (37, 1152, 16), (130, 1152, 3), (67, 2240, 32), (19, 3072, 7),
               (9, 8192, 4), (24, 544, 5), (3, 8960, 2), (6, 12288, 3),
               (33, 1152, 32), (97, 1152, 40), (70, 8192, 35), (300, 96, 100), (64, 3072, 64),
               (5, 12288, 64), (130, 1152, 1000), (200, 544, 33), (161, 2240, 80)]


@pytest.mark.parametrize("M,d,T", ADALN_CASES, ids=[f"{m}x{d}_T{t}" for m, d, t in ADALN_CASES])
@pytest.mark.parametrize("sets", ["per_block", "shared"])
def test_adaln_against_oracle(K, M, d, T, sets):
    seed = 8000 + M + d
    say(f"[adaln] M={M} d={d} T={T} sets={sets} seed={seed}")
    h = I.act_dit_lognormal(M, d, seed)[0]
    shift, scale = I.adaln_modulation((M + T - 1) // T, d, seed + 1)
    f = I.random_factors(d // 32 if sets == "per_block" else 1, seed + 2)
    check(K, h, shift, scale, T, f, f"{M}x{d}")


def test_adaln_special_rows(K):
    # constant row (variance 0: x = shift exactly), zero row, a row far from
    # zero mean, subnormal inputs, a NaN and an Inf row, -0 entries
    M, d, T = 12, 1152, 3
    say(f"[adaln specials] M={M} d={d} T={T}")
    rng = np.random.default_rng(8100)
    v = rng.standard_normal((M, d)).astype(np.float32)
    v[0] = 2.5
    v[1] = 0.0
    v[2] = 1000.0 + v[2]
    v[3] = v[3] * 2.0 ** -130
    v[4, 7] = np.inf
    v[5, 100] = np.nan
    v[6, ::3] = -0.0
    h = I.f32_to_bf16_bits(v)
    shift, scale = I.adaln_modulation((M + T - 1) // T, d, 8101)
    f = I.random_factors(d // 32, 8102)
    q, s, xg, q2, s2 = run_gpu(K, h, shift, scale, T, f)
    xb, xfl, qr, sr, ef, bf = oracle_codes(h, shift, scale, T, f)
    finite = np.isfinite(v).all(axis=1)
    assert np.array_equal(xg[finite], xb[finite]) or not np.any((xg != xb)[finite] & ~xfl[finite])
    # a non-finite entry makes its whole row non-finite on both sides: every
    # block of such a row encodes as scale 0xFF, codes 0
    assert np.all(sr[~finite] == 0xFF) and np.all(s[~finite] == 0xFF) and np.all(q[~finite] == 0)
    res = P.compare(q[finite], s[finite], qr[finite], sr[finite], ef[finite], bf[finite])
    say(f"    codes {res}")
    assert res["ok"], res
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # the constant row: x = shift of its sample, exactly representable or rounded
    assert np.array_equal(xg[0], xb[0])


# launch-shape overrides of kq_adaln_quantize: two launches with the second
# pass on the matrix cores (strips of 4 or 8 blocks) or the butterfly one, or
# one launch with whole rows in LDS (every case here fits it)
PASS_FORMS = [("mfma_strip4", {"adaln_pass": 1, "adaln_strip": 4}, None),
              ("mfma_strip8", {"adaln_pass": 1, "adaln_strip": 8}, None),
              ("butterfly", {"adaln_pass": 2}, "KQ_VARIANT_BUTTERFLY"),
              ("one_launch", {"adaln_pass": 3}, None)]
FORM_CASES = [(37, 1152, 16), (130, 1152, 3), (67, 2240, 32), (9, 8192, 4), (300, 96, 1), (4100, 3072, 2048),
              (97, 1152, 40), (70, 8192, 35), (200, 544, 33)]


@pytest.mark.parametrize("form,knobs,variant", PASS_FORMS, ids=[p[0] for p in PASS_FORMS])
def test_adaln_second_pass_forms(K, form, knobs, variant):
    # every second-pass form equals the unfused pipeline through the matching
    # quantizer bit for bit, on ragged rows, sample boundaries inside tiles and
    # several widths
    if True:
        for M, d, T in FORM_CASES:
            seed = 8400 + M + d
            say(f"[adaln form {form}] M={M} d={d} T={T} seed={seed}")
            h = I.act_dit_lognormal(M, d, seed)[0]
            shift, scale = I.adaln_modulation((M + T - 1) // T, d, seed + 1)
            hd, sh, sc = dev_bf16(h), dev_f32(shift), dev_f32(scale)
            fd = dev_f32(I.random_factors(d // 32, seed + 2))
            q, s = K.kq_adaln_quantize(hd, sh, sc, T, EPS, fd, tuning=knobs)
            x = K.adaln_modulate(hd, sh, sc, T, EPS)
            if variant is None:
                q2, s2 = K.kq_quantize(x, fd)
            else:
                q2, s2 = K.kq_quantize(x, fd, variant=getattr(K, variant))
            torch.cuda.synchronize()
            assert torch.equal(q, q2) and torch.equal(s, s2), f"{form} {M}x{d}: fused != unfused"


def test_adaln_stats_agree_across_forms(K):
    # the one-launch form sums each row from LDS in the statistics kernel's
    # order, so the workspace holds the same doubles bit for bit as after the
    # two-launch form and after adaln_modulate
    for M, d, T in ((37, 1152, 16), (300, 2240, 64), (130, 3072, 40), (5, 12288, 2)):
        say(f"[adaln stats forms] M={M} d={d} T={T}")
        h = I.act_dit_lognormal(M, d, 8350 + M)[0]
        shift, scale = I.adaln_modulation((M + T - 1) // T, d, 8351 + M)
        hd, sh, sc = dev_bf16(h), dev_f32(shift), dev_f32(scale)
        fd = dev_f32(I.random_factors(d // 32, 8352 + M))
        ws = [torch.full((M, 2), float("nan"), dtype=torch.float64, device="cuda") for _ in range(3)]
        K.kq_adaln_quantize(hd, sh, sc, T, EPS, fd, stats=ws[0], tuning={"adaln_pass": 3})
        K.kq_adaln_quantize(hd, sh, sc, T, EPS, fd, stats=ws[1], tuning={"adaln_pass": 1})
        K.adaln_modulate(hd, sh, sc, T, EPS, stats=ws[2])
        torch.cuda.synchronize()
        a, b, c = (w.cpu().numpy().view(np.uint64) for w in ws)
        assert np.array_equal(a, b) and np.array_equal(a, c), f"{M}x{d}: statistics differ between forms"


def test_adaln_one_launch_too_wide(K):
    # a row too wide for the one-launch form's LDS (one row of h, its codes and
    # the staging need more than 160 KB at d = 65536): the forced form returns
    # KQ_ERR_HIP and launches nothing; the automatic form runs two launches
    M, d, T = 2, 65536, 2
    say(f"[adaln one-launch too wide] M={M} d={d}")
    h = I.act_dit_lognormal(M, d, 8360)[0]
    shift, scale = I.adaln_modulation(1, d, 8361)
    hd, sh, sc = dev_bf16(h), dev_f32(shift), dev_f32(scale)
    fd = dev_f32(I.random_factors(d // 32, 8362))
    with pytest.raises(K.KQError) as ei:
        K.kq_adaln_quantize(hd, sh, sc, T, EPS, fd, tuning={"adaln_pass": 3})
    assert ei.value.status == K.KQ_ERR_HIP
    q, s = K.kq_adaln_quantize(hd, sh, sc, T, EPS, fd)
    x = K.adaln_modulate(hd, sh, sc, T, EPS)
    q2, s2 = K.kq_quantize(x, fd)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)


def test_adaln_stats_workspace(K):
    # the caller's workspace holds each row's mean and 1/sqrt(var + eps) in
    # double after the call (numpy's float64 statistics of the same bf16 rows)
    for M, d, T in ((21, 2240, 4), (75, 1152, 40)):
        _check_stats(K, M, d, T)


def _check_stats(K, M, d, T):
    say(f"[adaln stats] M={M} d={d} T={T}")
    h = I.act_dit_lognormal(M, d, 8300)[0]
    shift, scale = I.adaln_modulation((M + T - 1) // T, d, 8301)
    w = torch.full((M, 2), float("nan"), dtype=torch.float64, device="cuda")
    K.kq_adaln_quantize(dev_bf16(h), dev_f32(shift), dev_f32(scale), T, EPS,
                        dev_f32(I.random_factors(d // 32, 8302)), stats=w)
    torch.cuda.synchronize()
    hd = I.bf16_bits_to_f32(h).astype(np.float64)
    mu = hd.mean(axis=1)
    rstd = 1.0 / np.sqrt(hd.var(axis=1) + float(np.float32(EPS)))
    got = w.cpu().numpy()
    assert np.allclose(got[:, 0], mu, rtol=1e-12, atol=1e-14 * np.abs(hd).mean())
    assert np.allclose(got[:, 1], rstd, rtol=1e-12, atol=0)


def test_adaln_empty(K):
    h = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    sh = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
    q, s = K.kq_adaln_quantize(h, sh, sh, 4, EPS, dev_f32(I.identity_factors(1)))
    x = K.adaln_modulate(h, sh, sh, 4, EPS)
    torch.cuda.synchronize()
    assert q.shape == (0, 32) and s.shape == (0, 2) and x.shape == (0, 64)


@pytest.mark.parametrize("name", ["dit_1152", "mid_2240", "dbl_3072"])
def test_adaln_full_size_sampled_rows(K, name):
    # the full workload on the GPU (the DiT / mid / double-stream hidden widths,
    # two samples of M/2 tokens); the oracle on 48 sampled rows including both
    # ends of every sample
    M, d, _ = I.CONFIGS[name]
    T = I.tokens_per_sample(name)
    say(f"[adaln full] {name} M={M} d={d} T={T}")
    h = I.make_activation(name)
    shift, scale = I.adaln_modulation((M + T - 1) // T, d, I.adaln_seed(name))
    f = I.make_factors(name)
    q, s, xg, q2, s2 = run_gpu(K, h, shift, scale, T, f)
    assert np.array_equal(q, q2) and np.array_equal(s, s2), "fused != unfused"
    rng = np.random.default_rng(8200)
    ends = [0, T - 1, T, min(2 * T, M) - 1, M - 1]
    rows = np.unique(np.concatenate([ends, rng.integers(0, M, 43)]))
    b = rows // T
    xb, xfl, qr, sr, ef, bf = oracle_codes(h[rows], shift[b], scale[b], 1, f)
    x_mis = xg[rows] != xb
    assert not np.any(x_mis & ~xfl)
    res = P.compare(q[rows], s[rows], qr, sr, ef, bf)
    say(f"    {len(rows)} rows: x flagged {int(xfl.sum())}; codes {res}")
    assert res["ok"], res
