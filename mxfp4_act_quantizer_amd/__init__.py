"""MI355X (gfx950) KroQuant online activation quantizer.

bf16 activations -> per-32-block Kronecker transform (A1 (x) ... (x) A5 of 2x2
factors) -> MXFP4 (FP4 E2M1 codes + E8M0 scales), plus the SmoothQuant-style
per-channel-scale comparison quantizer.  The work runs in libkroquant.so (HIP
kernels + C++ host helpers); this package is the thin Python binding.

The binding (and with it libkroquant.so) is loaded on first use of any of the
names below, so `python -m mxfp4_act_quantizer_amd.build` works on a tree
where the library is missing or stale.  Using a name without the library
raises ImportError: there is no fallback.
"""
_BINDING_NAMES = (
    "EXPORTS", "KQ_ERR_ALIGN", "KQ_ERR_ARG", "KQ_ERR_HIP", "KQ_ERR_OVERLAP", "KQ_ERR_SHAPE", "KQ_ERR_SINGULAR",
    "KQ_OK", "KQ_VARIANT_AUTO", "KQ_VARIANT_BUTTERFLY", "KQ_VARIANT_MFMA", "LIB_PATH", "KQError",
    "kq_block_inverse", "kq_block_matrix", "kq_build_info", "kq_factor_inverse", "kq_fold_weight", "kq_quantize",
    "kq_quantize_ex", "kq_status_string", "kq_transform_f32", "lib", "mx_quantize_f32", "kq_launch_shape",
    "kq_flat_launch_shape", "Tuning", "TUNING_FIELDS", "KQ_COPY_FORMS",
    "sq_quantize", "measure_copy41", "kq_quantize_lu", "kq_transform_lu_f32", "fwht_quantize",
    "fwht_transform_f32", "kq_lu_factors", "mx_gemm", "kq_adaln_quantize", "adaln_modulate",
    "kq_quantize16", "kq_transform16_f32", "kq_adaln_quantize_noalloc", "KQ_NOALLOC_MAX_ROWS",
)
__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


def __dir__():
    return sorted(list(globals()) + list(_BINDING_NAMES))
