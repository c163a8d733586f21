"""kq_adaln_quantize_noalloc (the entry point for callers that cannot
allocate) against kq_adaln_quantize with a caller workspace, through the raw
C ABI: equal codes and scales bit for bit on two calls in a row, the second
with a smaller input (the fixed statistics array then still holds rows of the
first call past the second's M), plus the row limit and an oracle check of
the first call."""
import ctypes
import sys

import numpy as np
import pytest

from oracle import oracle as O
from synth import inputs as I
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

EPS = 1e-6


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    import mxfp4_act_quantizer_amd as K
    return K


def raw_noalloc(K, hd, shift, scale, T, fd, q, s, M=None):
    M = hd.shape[0] if M is None else M
    d = hd.shape[1]
    return K.lib().kq_adaln_quantize_noalloc(hd.data_ptr(), M, d, shift.data_ptr(), scale.data_ptr(), T,
                                             ctypes.c_float(EPS), fd.data_ptr(), fd.numel() // 20, q.data_ptr(),
                                             s.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def inputs(M, d, T, seed, shared=False):
    h = I.act_dit_lognormal(M, d, seed)[0]
    shift, scale = I.adaln_modulation((M + T - 1) // T, d, seed + 1)
    f = I.random_factors(1 if shared else d // 32, seed + 2)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    hd = torch.from_numpy(h.view(np.int16)).cuda().view(torch.bfloat16)
    return h, shift, scale, f, hd, dev(shift), dev(scale), dev(f)


@pytest.mark.parametrize("first,second", [((8192, 1152, 4096, False), (37, 1152, 16, False)),
                                          ((4608, 3072, 2304, False), (1000, 2240, 500, True))])
def test_noalloc_equals_workspace_form_twice(K, first, second):
    for k, (M, d, T, shared) in enumerate((first, second)):
        seed = 9600 + 10 * k + M + d
        say(f"[noalloc call {k + 1}] M={M} d={d} T={T} shared={shared} seed={seed}")
        h, shift, scale, f, hd, sh, sc, fd = inputs(M, d, T, seed, shared)
        q = torch.full((M, d // 2), 0xA5, dtype=torch.uint8, device="cuda")
        s = torch.full((M, d // 32), 0x5A, dtype=torch.uint8, device="cuda")
        assert raw_noalloc(K, hd, sh, sc, T, fd, q, s) == K.KQ_OK
        qw, sw = K.kq_adaln_quantize(hd, sh, sc, T, EPS, fd)  # caller-owned workspace
        torch.cuda.synchronize()
        assert torch.equal(q, qw) and torch.equal(s, sw), f"call {k + 1}: noalloc != workspace form"
        if k == 1:
            # the smaller call against the oracle too (its rows are the array's first rows)
            x, xb, xfl = O.adaln(h, shift, scale, T, EPS)
            qr, sr, y32 = O.kq_quantize(xb, f, want_y32=True)
            _, z = O.kq_transform(xb, f)
            ef, bf = P.boundary_flags(z, y32)
            xblk = xfl.reshape(M, d // 32, 32).any(axis=2)
            res = P.compare(q.cpu().numpy(), s.cpu().numpy(), qr, sr, ef | np.repeat(xblk, 32, axis=1), bf | xblk)
            say(f"    oracle: {res}")
            assert res["ok"], res


def test_noalloc_row_limit(K):
    # one row past the limit is refused before any launch; outputs untouched
    M, d, T = K.KQ_NOALLOC_MAX_ROWS + 1, 64, 1
    say(f"[noalloc limit] M={M} d={d}")
    hd = torch.zeros((M, d), dtype=torch.bfloat16, device="cuda")
    sh = torch.zeros((M, d), dtype=torch.float32, device="cuda")
    fd = torch.from_numpy(I.identity_factors(1)).cuda()
    q = torch.full((M, d // 2), 7, dtype=torch.uint8, device="cuda")
    s = torch.full((M, d // 32), 7, dtype=torch.uint8, device="cuda")
    assert raw_noalloc(K, hd, sh, sh, T, fd, q, s) == K.KQ_ERR_SHAPE
    torch.cuda.synchronize()
    assert int(q.min()) == 7 and int(s.max()) == 7
    # exactly the limit is accepted and equals the workspace form
    Ml = K.KQ_NOALLOC_MAX_ROWS
    assert raw_noalloc(K, hd, sh, sh, T, fd, q, s, M=Ml) == K.KQ_OK
    qw, sw = K.kq_adaln_quantize(hd[:Ml], sh[:Ml], sh[:Ml], T, EPS, fd)
    torch.cuda.synchronize()
    assert torch.equal(q[:Ml], qw) and torch.equal(s[:Ml], sw)
