"""GPU-vs-oracle comparison rules for the quantizer outputs.

Tolerance on the transformed values: |y_gpu - y| <= 2e-6 * z + TOL_ABS
elementwise, where y is the exact (float64) transformed value and
z = sum_r |x_r| |K_rc| is its magnitude scale.  A bound relative to |y| alone
cannot hold for any fp32 accumulation under cancellation; z >= |y| is the
loosest sound reading that still catches a wrong factor, index or sign.

The absolute term covers roundings whose result falls in the fp32 subnormal
range, where values are u = 2^-149 apart and no fp32 computation resolves a
relative 2e-6.  Each such rounding errs by at most u/2; sums of subnormals are
exact; products of normal-range values are exact (bf16 x bf16).  So:
  - matrix-core path: the 32 products of each of the three bf16 terms of K
    (96 products per output) are the only roundings that can land below
    2^-126: at most 96 * u/2 = 48 u;
  - butterfly path (five 2x2 stages, two roundings per output per stage):
    a stage-k error of at most u is multiplied by the later factors, so
    u * sum_k prod_{j>k} C_j, with C_j the largest column abs sum of A_j
    (abs_floor below; at most 33.7 for every random factor set the suites
    draw, 11.2 for the Hadamard factors, 5 for identity).
TOL_ABS = 48 u covers both for those sets; tests/test_tolerance_floor.py
checks the derivation against fp32 emulations of both summation orders,
including an adversarial block where the matrix-core bound is nearly reached.

Codes and scales are compared bit for bit, except where a value within that
tolerance of the oracle's fp32 value could legitimately round the other way:
  - an element is flagged when [|y32| - delta, |y32| + delta] / 2^E contains an
    E2M1 rounding threshold (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5), or when
    |y32| <= delta (a value that close to zero may come out with either sign,
    e.g. an exact cancellation computed as a tiny negative or an underflow to -0);
  - a block (and every element in it) is flagged when the shared exponent of
    amax - delta_blk and of amax + delta_blk differ;
  with delta = 2e-6 * max(z, |y32|) + 2^-146 and delta_blk its maximum over
  the block.
Every mismatching code must be flagged, every mismatching scale byte must be
on a flagged block; both counts are reported.
"""
import numpy as np

TOL = 2e-6
ULP_SUB = 2.0 ** -149  # fp32 subnormal spacing
TOL_ABS = 48 * ULP_SUB


def abs_floor_units(factors):
    """Per factor set, the butterfly path's subnormal rounding bound in units
    of ULP_SUB: sum_k prod_{j>k} C_j over the stages in kernel order (A1 first),
    C_j = max over output index of |A_j[0][c]| + |A_j[1][c]|."""
    F = np.asarray(factors, np.float64)
    C = np.abs(F).sum(axis=-2).max(axis=-1)  # [nT, stages]
    nT, ns = C.shape
    out = np.zeros(nT)
    for k in range(ns):
        out += np.prod(C[:, k + 1:], axis=1)
    return out


THRESHOLDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def unpack_codes(q):
    q = np.asarray(q, np.uint8)
    M = q.shape[0]
    out = np.empty((M, q.shape[1] * 2), np.uint8)
    out[:, 0::2] = q & 0xF
    out[:, 1::2] = q >> 4
    return out


def shared_exponent(amax):
    """E = clamp(floor(log2 amax) - 2, -127, 127), amax = 0 -> -127 (vectorised)."""
    amax = np.asarray(amax, np.float64)
    _, e = np.frexp(amax)  # amax = f 2^e, f in [0.5, 1)
    E = (e - 1) - 2
    E = np.where(amax == 0, -127, E)
    return np.clip(E, -127, 127)


def boundary_flags(z, y32, tol=TOL, bw=32, tol_abs=TOL_ABS):
    """Flags (elements [M, d], blocks [M, d/bw]) where a tolerance-sized change
    of the transformed value may change the code or the scale (bw: elements
    per scale block)."""
    M, d = y32.shape
    nB = d // bw
    a = np.abs(y32.astype(np.float64))
    delta = tol * np.maximum(z, a) + tol_abs
    ab = a.reshape(M, nB, bw)
    db = delta.reshape(M, nB, bw)
    amax = ab.max(axis=2)
    dmax = db.max(axis=2)
    # blocks holding Inf/NaN give inf - inf here; their scale byte is 0xFF
    # either way, so the arithmetic warning carries no information
    with np.errstate(invalid="ignore"):
        E_lo = shared_exponent(np.maximum(amax - dmax, 0.0))
    E_hi = shared_exponent(amax + dmax)
    blk = E_lo != E_hi
    E = shared_exponent(amax)  # the oracle's own exponent
    scale = np.ldexp(1.0, -E)[:, :, None]
    lo = (ab - db) * scale
    hi = (ab + db) * scale
    # some threshold t with lo <= t <= hi (NaN bounds select none)
    elem = np.searchsorted(THRESHOLDS, hi, side="right") > np.searchsorted(THRESHOLDS, lo, side="left")
    # within delta of zero: the computed value may carry either sign (code 0 vs 8)
    elem |= ab <= db
    elem |= blk[:, :, None]
    return elem.reshape(M, d), blk


def compare(q_gpu, s_gpu, q_ref, s_ref, elem_flag=None, blk_flag=None):
    """Returns a dict of counts; 'ok' is True when every mismatch is flagged
    (or, with no flags given, when there is no mismatch at all)."""
    cg, cr = unpack_codes(q_gpu), unpack_codes(q_ref)
    s_gpu = np.asarray(s_gpu, np.uint8)
    s_ref = np.asarray(s_ref, np.uint8)
    code_mis = cg != cr
    scale_mis = s_gpu != s_ref
    res = {
        "elements": int(cg.size),
        "blocks": int(s_ref.size),
        "code_mismatch": int(code_mis.sum()),
        "scale_mismatch": int(scale_mis.sum()),
    }
    if elem_flag is None:
        res["flagged_elements"] = 0
        res["flagged_blocks"] = 0
        res["unflagged_code_mismatch"] = res["code_mismatch"]
        res["unflagged_scale_mismatch"] = res["scale_mismatch"]
    else:
        res["flagged_elements"] = int(elem_flag.sum())
        res["flagged_blocks"] = int(blk_flag.sum())
        res["unflagged_code_mismatch"] = int((code_mis & ~elem_flag).sum())
        res["unflagged_scale_mismatch"] = int((scale_mis & ~blk_flag).sum())
    res["ok"] = res["unflagged_code_mismatch"] == 0 and res["unflagged_scale_mismatch"] == 0
    return res


def transform_error(y_gpu, y_ref, z, tol_abs=TOL_ABS):
    """(max |y_gpu - y| / z over elements with z > 0, number of elements
    outside the bound 2e-6 z + tol_abs)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(z > 0, err / z, np.where(err == 0, 0.0, np.inf))
    outside = err > TOL * z + tol_abs
    return (float(rel.max()) if rel.size else 0.0), int(outside.sum())
