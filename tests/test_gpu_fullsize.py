"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the library's automatic launch shapes).

Every configuration, the 16384- and 65536-row sweeps included, is compared
against the oracle on every row (the oracle runs on host threads over row
chunks).  Properties that hold at any size are checked as well: identity
factors give exactly the plain MXFP4 of the input, a replicated per-block
factor layout gives exactly the shared-set result, and the transform export
(same launch shape as the quantizer) re-encoded by the fp32 quantizer gives
exactly the quantizer's codes and scales.
"""
import sys

import numpy as np
import pytest

from oracle import oracle as O
from synth import inputs as I
from tests import oracle_mt as OM
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    import mxfp4_act_quantizer_amd as K
    return K


def to_dev(x_bits):
    return torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)


def kq_gpu(K, xd, f, variant=0):
    q, s = K.kq_quantize(xd, torch.from_numpy(np.ascontiguousarray(f)).cuda(), variant=variant)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


FULL = [("tiny", True), ("dit_1152", False), ("dit_1152", True), ("dit_4608", False), ("dit_4608", True),
        ("mid_2240", False), ("mid_8960", False), ("dbl_3072", False), ("dbl_12288", False),
        ("sweep_4096", False)]


@pytest.mark.parametrize("name,shared", FULL, ids=[f"{n}-{'shared' if s else 'perblock'}" for n, s in FULL])
def test_kq_full_config_all_rows(K, name, shared):
    x = I.make_activation(name)
    f = I.make_factors(name, shared=shared)
    M, d = x.shape
    say(f"[full kq {name}] M={M} d={d} nT={f.shape[0]}")
    qg, sg = kq_gpu(K, to_dev(x), f)
    qr, sr, y32 = OM.kq_quantize(x, f)
    z = OM.kq_z(x, f)
    ef, bf = P.boundary_flags(z, y32)
    res = P.compare(qg, sg, qr, sr, ef, bf)
    say(f"    {res}")
    if name.startswith("dbl"):
        # image rows and text rows reported separately
        m_img = (M * 8) // 9
        for lab, sl in (("image", slice(0, m_img)), ("text", slice(m_img, M))):
            r = P.compare(qg[sl], sg[sl], qr[sl], sr[sl], ef[sl], bf[sl])
            say(f"    {lab} rows: {r}")
            assert r["ok"]
    assert res["ok"], res


@pytest.mark.parametrize("name", ["tiny", "dit_4608", "mid_8960", "dbl_12288", "sweep_4096"])
def test_sq_full_config_bit_exact(K, name):
    x = I.make_activation(name)
    scale = I.smoothquant_scale(x)
    M, d = x.shape
    say(f"[full sq {name}] M={M} d={d}")
    q, s = K.sq_quantize(to_dev(x), torch.from_numpy(scale).cuda())
    torch.cuda.synchronize()
    qr, sr = OM.sq_quantize(x, scale)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr)
    say(f"    {res}")
    assert res["code_mismatch"] == 0 and res["scale_mismatch"] == 0


@pytest.mark.timeout(1800)
@pytest.mark.parametrize("name", ["sweep_4096", "sweep_16384", "sweep_65536"])
def test_sweep_identity_hadamard(K, name):
    M, d, _ = I.CONFIGS[name]
    say(f"[sweep {name}] generating M={M} d={d}")
    x, _, specials = I.act_sweep_special(M, d, I.data_seed(name))
    xd = to_dev(x)
    say(f"[sweep {name}] launch shape {K.kq_launch_shape(M, d)}")

    # identity: bit-exact plain MXFP4, against the fp32 quantizer on the GPU
    # and against the oracle on every row
    say(f"[sweep {name}] identity nT=1 and nT={d // 32}")
    qi, si = kq_gpu(K, xd, I.identity_factors(1))
    q32, s32 = K.mx_quantize_f32(xd.float())
    torch.cuda.synchronize()
    assert np.array_equal(qi, q32.cpu().numpy()) and np.array_equal(si, s32.cpu().numpy())
    del q32, s32
    torch.cuda.empty_cache()
    res = OM.compare_kq_rows(x, I.identity_factors(1), qi, si, progress=say)
    say(f"    identity, every row: {res}")
    assert res["code_mismatch"] == 0 and res["scale_mismatch"] == 0
    qb, sb = kq_gpu(K, xd, I.identity_factors(d // 32))
    assert np.array_equal(qb, qi) and np.array_equal(sb, si)
    del qb, sb, qi, si

    # normalised WHT-32 via five H2/sqrt(2) factors; replicated layout equals shared
    say(f"[sweep {name}] hadamard nT=1 and nT={d // 32}")
    h = I.hadamard_factors(1)
    qh, sh = kq_gpu(K, xd, h)
    qhb, shb = kq_gpu(K, xd, I.hadamard_factors(d // 32))
    assert np.array_equal(qh, qhb) and np.array_equal(sh, shb)
    del qhb, shb
    res = OM.compare_kq_rows(x, h, qh, sh, progress=say)
    say(f"    hadamard, every row: {res}")
    assert res["ok"], res
    del qh, sh

    # learned-style per-block factors, every row
    f = I.random_factors(d // 32, I.factor_seed(name))
    say(f"[sweep {name}] random per-block factors")
    qg, sg = kq_gpu(K, xd, f)
    res = OM.compare_kq_rows(x, f, qg, sg, progress=say)
    say(f"    per-block, every row: {res}")
    assert res["ok"], res
    del xd
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["dit_4608", "dbl_12288", "sweep_65536"])
def test_transform_export_in_timed_launch_shape(K, name):
    # kq_transform_f32 runs the quantizer's transform in the quantizer's own
    # launch shape (strip width, token groups, workgroup order: one shape
    # function serves both); its values are within tolerance of the exact
    # transform on every row (sampled rows at 65536 x 12288), and the fp32
    # quantizer applied to them gives the quantizer's codes and scales bit for bit
    M, d, _ = I.CONFIGS[name]
    if name.startswith("sweep"):
        x = I.act_sweep_special(M, d, I.data_seed(name))[0]
        f = I.hadamard_factors(1)
    else:
        x = I.make_activation(name)
        f = I.make_factors(name)
    shape = K.kq_launch_shape(M, d)
    say(f"[transform full {name}] M={M} d={d} nT={f.shape[0]} launch shape {shape}")
    xd = to_dev(x)
    fd = torch.from_numpy(f).cuda()
    y = K.kq_transform_f32(xd, fd)
    q, s = K.kq_quantize(xd, fd)
    q2, s2 = K.mx_quantize_f32(y)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2), "quantizer != MXFP4 of its own exported transform"
    del q, s, q2, s2, xd
    if name.startswith("sweep"):
        rng = np.random.default_rng(M + 1)
        rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M), rng.choice(M, 896, replace=False)]))
        yh = y[torch.from_numpy(rows).cuda()].cpu().numpy()
        xs = np.ascontiguousarray(x[rows])
        worst, bad = OM.transform_rows_error(xs, f, yh)
        say(f"    {len(rows)} sampled rows: max |y_gpu - y| / z = {worst:.3e}, outside the bound: {bad}")
    else:
        worst, bad = OM.transform_rows_error(x, f, y.cpu().numpy())
        say(f"    every row: max |y_gpu - y| / z = {worst:.3e}, outside the bound: {bad}")
    assert bad == 0
    del y
    torch.cuda.empty_cache()


def test_concurrent_host_threads_match_single_thread(K):
    # two host threads, each on its own stream, quantizing different shapes at
    # the same time (the first launches of their kernel instances included)
    # give exactly the single-thread results
    import threading
    cases = [("dit_1152", 8192, 1152), ("sweep_16384", 16384, 12288)]
    inputs = []
    for name, M, d in cases:
        x = I.make_activation(name) if not name.startswith("sweep") else \
            I.act_sweep_special(M, d, I.data_seed(name))[0]
        f = I.make_factors(name) if not name.startswith("sweep") else I.random_factors(d // 32, 9300)
        inputs.append((to_dev(x), torch.from_numpy(f).cuda()))
    say("[concurrency] two threads, two streams, 12 launches each")
    results = [None, None]
    errors = []
    barrier = threading.Barrier(2)

    def run(k):
        try:
            xd, fd = inputs[k]
            st = torch.cuda.Stream()
            barrier.wait()
            outs = []
            with torch.cuda.stream(st):
                for _ in range(12):
                    outs.append(K.kq_quantize(xd, fd, stream=st))
            st.synchronize()
            results[k] = outs
        except Exception as e:  # reported below
            errors.append(e)

    ths = [threading.Thread(target=run, args=(k,)) for k in range(2)]
    for th in ths:
        th.start()
    for th in ths:
        th.join()
    assert not errors, errors
    for k, (xd, fd) in enumerate(inputs):
        q0, s0 = K.kq_quantize(xd, fd)
        torch.cuda.synchronize()
        for q, s in results[k]:
            assert torch.equal(q, q0) and torch.equal(s, s0), cases[k]
    say("    all launches equal the single-thread result")


@pytest.mark.parametrize("name", ["dit_4608", "mid_8960", "dbl_12288"])
def test_kq_lu_and_fwht_full_config_all_rows(K, name):
    # K2 form with per-block LU scalars, and the Walsh-Hadamard comparison, on every row
    x = I.make_activation(name)
    M, d = x.shape
    lu = I.random_lu(d // 32, I.factor_seed(name) + 77)
    xd = to_dev(x)
    say(f"[full kq_lu {name}] M={M} d={d}")
    q, s = K.kq_quantize_lu(xd, torch.from_numpy(lu).cuda())
    qf, sf = K.fwht_quantize(xd)
    torch.cuda.synchronize()
    qr, sr, y32 = OM.kq_quantize_lu(x, lu)
    ef, bf = P.boundary_flags(OM.kq_z_lu(x, lu), y32)
    res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr, ef, bf)
    say(f"    {res}")
    assert res["ok"], res
    say(f"[full fwht {name}] M={M} d={d}")
    qr, sr, y32 = OM.fwht_quantize(x)
    ef, bf = P.boundary_flags(OM.fwht_z(x), y32)
    res = P.compare(qf.cpu().numpy(), sf.cpu().numpy(), qr, sr, ef, bf)
    say(f"    {res}")
    assert res["ok"], res
