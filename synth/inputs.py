"""Seeded synthetic inputs for the KroQuant quantizer path.

This module only draws random numbers and lays them out.  It holds none of the
quantizer's arithmetic.  Both sides get the same inputs from here: the GPU
library (through the tests and the benchmark) and the CPU oracle.

The shapes and value distributions stand in for diffusion-transformer
linear-layer inputs: DiT hidden sizes, CFG-doubled token batches, outlier
channels, and a double-stream image/text split.  The pages' quality evaluation
uses real models and prompt sets (PixArt-Sigma, SANA, FLUX.1-schnell on
MJHQ-30K / SDCI).  None of those are used here.

Every generator takes an explicit integer seed and uses numpy's PCG64, so the
same seed gives the same bytes on every machine with this numpy.
bf16 activations are returned as uint16 bit patterns (fp32 -> bf16
round-to-nearest-even), and factors as float32 arrays of shape [nT, 5, 2, 2].
"""
import math

import numpy as np

# ---------------------------------------------------------------------------
# small helpers (layout / type conversion only)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(a):
    """fp32 -> bf16 bit patterns, round to nearest even (NaN kept quiet).
    Works in uint32 (no overflow for any non-NaN pattern) over row chunks."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.reshape(-1).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    step = 1 << 24
    for i in range(0, u.size, step):
        c = u[i:i + step]
        r = c + (np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1)))
        r >>= np.uint32(16)
        nan = (c & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            r[nan] = (c[nan] >> np.uint32(16)) | np.uint32(0x40)
        out[i:i + step] = r
    return out.reshape(a.shape)


def bf16_bits_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(int(seed)))


def _pick_channels(rng, d, count, exclude=None):
    """Distinct channel indices (partial Fisher-Yates via permutation)."""
    pool = np.arange(d)
    if exclude is not None and len(exclude):
        pool = np.setdiff1d(pool, np.asarray(exclude))
    return np.sort(rng.permutation(pool)[:count])


def n_outliers(d, frac):
    return int(round(frac * d))


# ---------------------------------------------------------------------------
# transform factors
# ---------------------------------------------------------------------------


def random_factors(nT, seed, sigma=0.3, cond_max=10.0):
    """nT sets of five 2x2 factors, each I + sigma*N(0,1), redrawn until its
    2-norm condition number is below cond_max."""
    rng = _rng(seed)
    out = np.empty((nT, 5, 2, 2), np.float32)
    for t in range(nT):
        for k in range(5):
            while True:
                g = (np.eye(2) + sigma * rng.standard_normal((2, 2))).astype(np.float32)
                if np.linalg.cond(g.astype(np.float64)) < cond_max:
                    break
            out[t, k] = g
    return out


def identity_factors(nT=1):
    return np.tile(np.eye(2, dtype=np.float32), (nT, 5, 1, 1))


def hadamard_factors(nT=1):
    """Five copies of [[1,1],[1,-1]]/sqrt(2) in fp32: the normalised
    Walsh-Hadamard transform of size 32 (up to fp32 rounding of 1/sqrt(2))."""
    h = np.float32(1.0 / math.sqrt(2.0))
    g = np.array([[h, h], [h, -h]], np.float32)
    return np.tile(g, (nT, 5, 1, 1))


def hadamard_lu(nT=1):
    """LU scalars (a, b, c) per factor, [nT, 5, 3] fp32, at the Hadamard
    initialisation: a = b = fl32(1/sqrt(2)), c = 1 for all five factors."""
    h = np.float32(1.0 / math.sqrt(2.0))
    return np.tile(np.array([h, h, 1.0], np.float32), (nT, 5, 1))


def random_lu(nT, seed, spread=0.3):
    """LU scalars (a, b, c) per factor, [nT, 5, 3] fp32: bounded perturbations
    of the Hadamard initialisation, a = (1/sqrt 2)(1 + spread*U(-1,1)),
    b = 1/sqrt 2 + spread*U(-1,1), c = 1 + spread*U(-1,1).  |a| stays at or
    above 0.49, so every factor is well conditioned without any test here."""
    rng = _rng(seed)
    h = 1.0 / math.sqrt(2.0)
    u = rng.uniform(-1.0, 1.0, size=(nT, 5, 3))
    out = np.empty((nT, 5, 3), np.float32)
    out[..., 0] = h * (1.0 + spread * u[..., 0])
    out[..., 1] = h + spread * u[..., 1]
    out[..., 2] = 1.0 + spread * u[..., 2]
    return out


def integer_unimodular_factors(nT, seed):
    """Integer factors with determinant +-1 (so every inverse is integer too);
    used for exact invariance checks."""
    choices = [
        [[1, 1], [0, 1]], [[1, 0], [1, 1]], [[0, 1], [1, 0]], [[2, 1], [1, 1]],
        [[1, -1], [0, 1]], [[1, 0], [-1, 1]], [[-1, 0], [0, 1]], [[1, 2], [0, -1]],
    ]
    rng = _rng(seed)
    idx = rng.integers(0, len(choices), size=(nT, 5))
    return np.array([[choices[i] for i in row] for row in idx], np.float32)


# ---------------------------------------------------------------------------
# activations
# ---------------------------------------------------------------------------


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def act_gaussian_outliers(M, d, seed, n_out, out_scale, base_scale=1.0):
    """N(0,1)*base_scale with n_out seeded outlier channels multiplied by out_scale."""
    rng = _rng(seed)
    ch = _pick_channels(rng, d, n_out)
    x = _normal(rng, (M, d))
    if base_scale != 1.0:
        x *= np.float32(base_scale)
    x[:, ch] *= np.float32(out_scale)
    return f32_to_bf16_bits(x), ch


def act_dit_lognormal(M, d, seed, out_frac=0.01, out_scale=50.0):
    """Rows N(0,1) times a per-token LogNormal(0, 0.5) magnitude, with 1% outlier
    channels x50 (the CFG-doubled DiT attention/MLP input)."""
    rng = _rng(seed)
    ch = _pick_channels(rng, d, n_outliers(d, out_frac))
    x = _normal(rng, (M, d))
    tok = np.exp(0.5 * rng.standard_normal(M)).astype(np.float32)
    x *= tok[:, None]
    x[:, ch] *= np.float32(out_scale)
    return f32_to_bf16_bits(x), ch


def act_student_t(M, d, seed, nu=3, scale=0.5, out_frac=0.02, out_scale=40.0, zero_block_frac=0.001):
    """0.5 * Student-t(nu=3), drawn as Z / sqrt(chi2_3 / 3) from four normals,
    2% outlier channels x40 and 0.1% of (row, 32-block) pairs set to +0."""
    rng = _rng(seed)
    ch = _pick_channels(rng, d, n_outliers(d, out_frac))
    z = _normal(rng, (M, d)).astype(np.float64)
    chi2 = np.zeros((M, d), np.float64)
    for _ in range(nu):
        chi2 += _normal(rng, (M, d)).astype(np.float64) ** 2
    x = (scale * z / np.sqrt(chi2 / nu)).astype(np.float32)
    x[:, ch] *= np.float32(out_scale)
    nB = d // 32
    nzero = int(round(zero_block_frac * M * nB))
    flat = rng.choice(M * nB, size=nzero, replace=False) if nzero else np.zeros(0, np.int64)
    rows, blks = flat // nB, flat % nB
    for m, j in zip(rows, blks):
        x[m, 32 * j:32 * j + 32] = 0.0
    return f32_to_bf16_bits(x), ch, np.stack([rows, blks], 1)


def act_double_stream(M_img, M_txt, d, seed, img_frac=0.01, img_scale=50.0, txt_frac=0.01, txt_scale=80.0,
                      txt_base=10.0):
    """Image rows N(0,1) with 1% outlier channels x50, then text rows 10*N(0,1)
    with a disjoint 1% outlier set x80 (a double-stream DiT joint input)."""
    rng = _rng(seed)
    ch_img = _pick_channels(rng, d, n_outliers(d, img_frac))
    ch_txt = _pick_channels(rng, d, n_outliers(d, txt_frac), exclude=ch_img)
    x = _normal(rng, (M_img + M_txt, d))
    x[:M_img][:, ch_img] *= np.float32(img_scale)
    x[M_img:] *= np.float32(txt_base)
    x[M_img:, ch_txt] *= np.float32(txt_scale)
    return f32_to_bf16_bits(x), ch_img, ch_txt


def act_sweep_special(M, d, seed, out_frac=0.01, out_scale=50.0, special_frac=0.001):
    """N(0,1) with 1% outlier channels x50, plus special 32-blocks at seeded
    positions (special_frac of all blocks each):
      kind 0  all +0
      kind 1  subnormal magnitude: N(0,1) * 2^-130 (bf16 subnormals, zeros, -0)
      kind 2  near the smallest normal: N(0,1) * 2^-124
      kind 3  exact ties: multiples of 0.25 * 2^e with block max exactly 4*2^e or 6*2^e
    Returns (bits, outlier channels, special (row, block, kind) triples)."""
    rng = _rng(seed)
    ch = _pick_channels(rng, d, n_outliers(d, out_frac))
    x = _normal(rng, (M, d))
    x[:, ch] *= np.float32(out_scale)
    nB = d // 32
    per_kind = int(round(special_frac * M * nB))
    total = 4 * per_kind
    flat = rng.choice(M * nB, size=total, replace=False) if total else np.zeros(0, np.int64)
    specials = []
    for idx, b in enumerate(flat):
        kind = idx % 4
        m, j = int(b // nB), int(b % nB)
        sl = (m, slice(32 * j, 32 * j + 32))
        if kind == 0:
            x[sl] = 0.0
        elif kind == 1:
            x[sl] = _normal(rng, 32) * np.float32(2.0 ** -130)
        elif kind == 2:
            x[sl] = _normal(rng, 32) * np.float32(2.0 ** -124)
        else:
            e = int(rng.integers(-20, 21))
            k = rng.integers(-24, 25, size=32).astype(np.float32)  # |k|*0.25 <= 6
            top = np.float32(16.0 if rng.integers(0, 2) == 0 else 24.0)  # 4*2^e or 6*2^e
            k[int(rng.integers(0, 32))] = top * (1 if rng.integers(0, 2) else -1)
            k = np.clip(k, -top, top)
            x[sl] = (k * np.float32(0.25) * np.float32(2.0 ** e)).astype(np.float32)
        specials.append((m, j, kind))
    return f32_to_bf16_bits(x), ch, np.array(specials, np.int64).reshape(-1, 3)


def smoothquant_scale(x_bits, floor=1e-5):
    """Per-channel SmoothQuant scale s_c = sqrt(max(amax_c, floor)), amax over
    all rows of the bf16 activation (calibration on the same tensor)."""
    xf = np.abs(bf16_bits_to_f32(x_bits))
    amax = xf.max(axis=0).astype(np.float64)
    return np.sqrt(np.maximum(amax, floor)).astype(np.float32)


# ---------------------------------------------------------------------------
# named workloads (the five configurations)
# ---------------------------------------------------------------------------

CONFIGS = {
    # name: (M, d, description)
    "tiny": (256, 1152, "N(0,1), 12 outlier channels x30, one shared factor set; SmoothQuant scale amax^0.5"),
    "dit_1152": (8192, 1152, "CFG 2x4096 tokens, per-token lognormal(0,0.5) rows, 1% outlier channels x50"),
    "dit_4608": (8192, 4608, "CFG 2x4096 tokens, per-token lognormal(0,0.5) rows, 1% outlier channels x50"),
    "mid_2240": (2048, 2240, "0.5*Student-t(3), 2% outlier channels x40, 0.1% zero blocks"),
    "mid_8960": (2048, 8960, "0.5*Student-t(3), 2% outlier channels x40, 0.1% zero blocks"),
    "dbl_3072": (4608, 3072, "4096 image rows N(0,1) 1% x50 + 512 text rows 10*N(0,1) disjoint 1% x80"),
    "dbl_12288": (4608, 12288, "4096 image rows N(0,1) 1% x50 + 512 text rows 10*N(0,1) disjoint 1% x80"),
    "sweep_4096": (4096, 12288, "N(0,1) 1% x50, special zero/subnormal/min-normal/tie blocks"),
    "sweep_16384": (16384, 12288, "N(0,1) 1% x50, special zero/subnormal/min-normal/tie blocks"),
    "sweep_65536": (65536, 12288, "N(0,1) 1% x50, special zero/subnormal/min-normal/tie blocks"),
}

_CFG_ID = {"tiny": 1, "dit_1152": 2, "dit_4608": 2, "mid_2240": 3, "mid_8960": 3, "dbl_3072": 4, "dbl_12288": 4,
           "sweep_4096": 5, "sweep_16384": 5, "sweep_65536": 5}
_VARIANT = {"tiny": 0, "dit_1152": 0, "dit_4608": 1, "mid_2240": 0, "mid_8960": 1, "dbl_3072": 0, "dbl_12288": 1,
            "sweep_4096": 0, "sweep_16384": 1, "sweep_65536": 2}


def data_seed(name):
    return 1000 * _CFG_ID[name] + _VARIANT[name]


def factor_seed(name):
    return 1000 * _CFG_ID[name] + 500 + _VARIANT[name]


def make_activation(name, M=None, d=None, seed=None):
    """Activation bits for a named workload; M/d/seed override the defaults
    (smaller M keeps the same distribution for oracle-sized tests)."""
    M0, d0, _ = CONFIGS[name]
    M = M0 if M is None else M
    d = d0 if d is None else d
    seed = data_seed(name) if seed is None else seed
    cid = _CFG_ID[name]
    if cid == 1:
        return act_gaussian_outliers(M, d, seed, 12, 30.0)[0]
    if cid == 2:
        return act_dit_lognormal(M, d, seed)[0]
    if cid == 3:
        return act_student_t(M, d, seed)[0]
    if cid == 4:
        m_img = (M * 8) // 9  # 4096 image + 512 text rows at M = 4608
        return act_double_stream(m_img, M - m_img, d, seed)[0]
    return act_sweep_special(M, d, seed)[0]


def make_factors(name, d=None, shared=None, seed=None):
    """Factor sets for a named workload: per-block (nT = d/32) unless the
    workload is the tiny one (shared) or `shared` says otherwise."""
    _, d0, _ = CONFIGS[name]
    d = d0 if d is None else d
    seed = factor_seed(name) if seed is None else seed
    if shared is None:
        shared = (_CFG_ID[name] == 1)
    nT = 1 if shared else d // 32
    return random_factors(nT, seed)


def adaln_modulation(n_samples, d, seed, sigma=0.5):
    """Per-sample AdaLN modulation vectors (shift, scale), fp32 [n_samples, d]
    each, drawn N(0, sigma^2) per entry (standing in for the conditioning
    projection of a diffusion transformer block)."""
    rng = _rng(seed)
    shift = (sigma * _normal(rng, (n_samples, d))).astype(np.float32)
    scale = (sigma * _normal(rng, (n_samples, d))).astype(np.float32)
    return shift, scale


def adaln_seed(name):
    return 1000 * _CFG_ID[name] + 700 + _VARIANT[name]


def tokens_per_sample(name, M=None):
    """Tokens per sample of a named workload: the CFG-doubled batches hold two
    samples (conditional and unconditional) of M / 2 tokens each; the tiny
    workload is one sample."""
    M0, _, _ = CONFIGS[name]
    M = M0 if M is None else M
    if _CFG_ID[name] == 1:
        return max(M, 1)
    return max((M + 1) // 2, 1)


def random_factors16(nT, seed, sigma=0.3, cond_max=10.0):
    """nT sets of four 2x2 factors (16-element blocks), drawn as random_factors
    draws its five."""
    return np.ascontiguousarray(random_factors(nT, seed, sigma, cond_max)[:, :4])


def integer_unimodular_factors16(nT, seed):
    return np.ascontiguousarray(integer_unimodular_factors(nT, seed)[:, :4])
