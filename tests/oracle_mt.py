"""Run the (single-threaded) oracle over row chunks on several host threads;
ctypes releases the GIL during each call.  Rows are independent, so the
result is the same as one call over the whole matrix."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import oracle as O
from tests import parity as P

THREADS = max(1, min(16, os.cpu_count() or 1))


def _chunks(M):
    step = max(1, (M + THREADS * 4 - 1) // (THREADS * 4))
    return [(r, min(M, r + step)) for r in range(0, M, step)]


def kq_quantize(x, f):
    M, d = x.shape
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 32), np.uint8)
    y32 = np.empty((M, d), np.float32)

    def job(rr):
        a, b = rr
        q[a:b], s[a:b], y32[a:b] = O.kq_quantize(np.ascontiguousarray(x[a:b]), f, want_y32=True)

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(job, _chunks(M)))
    return q, s, y32


def kq_z(x, f):
    M, d = x.shape
    z = np.empty((M, d), np.float64)

    def job(rr):
        a, b = rr
        z[a:b] = O.kq_transform(np.ascontiguousarray(x[a:b]), f)[1]

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(job, _chunks(M)))
    return z


def sq_quantize(x, scale):
    M, d = x.shape
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 32), np.uint8)

    def job(rr):
        a, b = rr
        q[a:b], s[a:b] = O.sq_quantize(np.ascontiguousarray(x[a:b]), scale)

    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(job, _chunks(M)))
    return q, s


def _run(M, fn):
    with ThreadPoolExecutor(THREADS) as ex:
        list(ex.map(fn, _chunks(M)))


def kq_quantize_lu(x, lu):
    M, d = x.shape
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 32), np.uint8)
    y32 = np.empty((M, d), np.float32)

    def job(rr):
        a, b = rr
        q[a:b], s[a:b], y32[a:b] = O.kq_quantize_lu(np.ascontiguousarray(x[a:b]), lu, want_y32=True)

    _run(M, job)
    return q, s, y32


def kq_z_lu(x, lu):
    M, d = x.shape
    z = np.empty((M, d), np.float64)

    def job(rr):
        a, b = rr
        z[a:b] = O.kq_transform_lu(np.ascontiguousarray(x[a:b]), lu)[1]

    _run(M, job)
    return z


def fwht_quantize(x):
    M, d = x.shape
    q = np.empty((M, d // 2), np.uint8)
    s = np.empty((M, d // 32), np.uint8)
    y32 = np.empty((M, d), np.float32)

    def job(rr):
        a, b = rr
        q[a:b], s[a:b], y32[a:b] = O.fwht_quantize(np.ascontiguousarray(x[a:b]), want_y32=True)

    _run(M, job)
    return q, s, y32


def fwht_z(x):
    M, d = x.shape
    z = np.empty((M, d), np.float64)

    def job(rr):
        a, b = rr
        z[a:b] = O.fwht_transform(np.ascontiguousarray(x[a:b]))[1]

    _run(M, job)
    return z


def compare_kq_rows(x, f, qg, sg, rows=1024, progress=None, lu=False):
    """Every row of a GPU result (qg, sg) against the oracle under the flag
    rules of tests/parity.py, in row chunks on host threads (memory stays
    bounded at any M).  Returns the summed counts of parity.compare."""
    M = x.shape[0]
    chunks = [(a, min(M, a + rows)) for a in range(0, M, rows)]
    quant = O.kq_quantize_lu if lu else O.kq_quantize
    transform = O.kq_transform_lu if lu else O.kq_transform

    def job(rr):
        a, b = rr
        xc = np.ascontiguousarray(x[a:b])
        qr, sr, y32 = quant(xc, f, want_y32=True)
        z = transform(xc, f)[1]
        ef, bf = P.boundary_flags(z, y32)
        return P.compare(qg[a:b], sg[a:b], qr, sr, ef, bf)

    tot = None
    done = 0
    with ThreadPoolExecutor(THREADS) as ex:
        for r in ex.map(job, chunks):
            if tot is None:
                tot = dict(r)
            else:
                for k, v in r.items():
                    tot[k] = (tot[k] and v) if k == "ok" else tot[k] + v
            done += 1
            if progress and done % 16 == 0:
                progress(f"    {done}/{len(chunks)} chunks")
    return tot


def transform_rows_error(x, f, y_gpu, rows=1024):
    """(max |y_gpu - y| / z, elements outside 2e-6 z + TOL_ABS) over every row,
    y the oracle's exact transform, in row chunks on host threads."""
    M = x.shape[0]
    chunks = [(a, min(M, a + rows)) for a in range(0, M, rows)]

    def job(rr):
        a, b = rr
        y, z = O.kq_transform(np.ascontiguousarray(x[a:b]), f)
        return P.transform_error(y_gpu[a:b], y, z)

    worst, bad = 0.0, 0
    with ThreadPoolExecutor(THREADS) as ex:
        for w, n in ex.map(job, chunks):
            worst, bad = max(worst, w), bad + n
    return worst, bad
