"""The pins must catch plausible mistakes.  Each case plants one mistake in a
copy of the oracle source (on the CPU), builds it, and checks that the pin
meant to guard that step fails against the mutated oracle."""
import ctypes
import os
import subprocess

import pytest

import tests.test_oracle_pins as pins
from oracle import oracle

SRC = os.path.join(os.path.dirname(oracle.LIB_PATH), "kq_oracle.c")

MUTATIONS = {
    # name: (original text, replacement, pin that must fail, pin arguments)
    "kron_bit_order_lsb_first": (
        "int rk = (r >> (4 - k)) & 1;\n                int ck = (c >> (4 - k)) & 1;\n                p *= (double)f",
        "int rk = (r >> k) & 1;\n                int ck = (c >> k) & 1;\n                p *= (double)f",
        "test_kron_block_equals_numpy_kron", {"seed": 1}),
    "transposed_block": (
        "acc += xb[r] * Kj[r * 32 + c];\n                    mag",
        "acc += xb[r] * Kj[c * 32 + r];\n                    mag",
        "test_transform_equals_modewise_product", {}),
    "ties_round_up": (
        "if (dist < bestd || (dist == bestd && (i & 1) == 0 && (best & 1) == 1)) {",
        "if (dist <= bestd) {",
        "test_mx_block_handcases", {"case": pins._load_handcases()[1]}),
    "scale_exponent_off_by_one": (
        "int E = (e - 1) - 2;",
        "int E = e - 2;",
        "test_mx_block_handcases", {"case": pins._load_handcases()[0]}),
    "sign_from_signbit": (
        "return best | ((y < 0.0f) ? 8 : 0);",
        "return best | (signbit(y) ? 8 : 0);",
        "test_mx_block_handcases", {"case": pins._load_handcases()[7]}),
    "zero_block_scale_one": (
        "if (amax == 0.0f)\n        return -127;",
        "if (amax == 0.0f)\n        return 0;",
        "test_mx_block_handcases", {"case": pins._load_handcases()[6]}),
    "inverse_wrong_order": (
        "p *= inv[k * 4 + rk * 2 + ck];",
        "p *= inv[k * 4 + ck * 2 + rk];",
        "test_inverse_is_kron_of_factor_inverses", {"seed": 4}),
    "sq_divides_in_double": (
        "float recip = 1.0f / scale[j * 32 + c];\n                float xf = (float)oracle_bf16_to_double(x[m * d + j * 32 + c]);\n                yb[c] = xf * recip;",
        "float recip = 1.0f / scale[j * 32 + c];\n                float xf = (float)oracle_bf16_to_double(x[m * d + j * 32 + c]);\n                yb[c] = (float)((double)xf / (double)scale[j * 32 + c]); (void)recip;",
        "test_sq_rounds_once_per_step", {}),
    "lu_upper_diagonal_sign": (
        "double u11 = -1.0 / a;",
        "double u11 = 1.0 / a;",
        "test_lu_factor_closed_forms", {}),
    "lu_product_order_u_times_l": (
        "G[0] = a;\n    G[1] = b;\n    G[2] = c * a;\n    G[3] = c * b + u11;",
        "G[0] = a + b * c;\n    G[1] = b;\n    G[2] = c * u11;\n    G[3] = u11;",
        "test_lu_factor_closed_forms", {}),
    "lu_block_factors_transposed": (
        "p *= G[k * 4 + rk * 2 + ck];",
        "p *= G[k * 4 + ck * 2 + rk];",
        "test_lu_block_is_kron_of_its_factors", {}),
    "dequant_nibble_order_swapped": (
        "int code = (k & 1) ? (byte >> 4) : (byte & 15);",
        "int code = (k & 1) ? (byte & 15) : (byte >> 4);",
        "test_mx_dequant_requantizes_to_itself", {}),
    "dequant_grid_value_wrong": (
        "{0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};\n    if (sbyte == 0xFF)",
        "{0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 4.0, 6.0};\n    if (sbyte == 0xFF)",
        "test_mx_value_inverts_the_element_encoding", {}),
    "adaln_eps_dropped": (
        "double r = 1.0 / sqrt(var + (double)eps);",
        "double r = 1.0 / sqrt(var);",
        "test_adaln_matches_torch_layer_norm", {"M": 5, "d": 64, "T": 2}),
    "adaln_unbiased_variance": (
        "double var = ss / (double)d;",
        "double var = ss / (double)(d - 1);",
        "test_adaln_matches_torch_layer_norm", {"M": 5, "d": 64, "T": 2}),
    "adaln_modulation_without_one": (
        "double g = 1.0 + (double)scale[b * d + c];",
        "double g = (double)scale[b * d + c];",
        "test_adaln_hand_case", {}),
    "adaln_sample_index_modulo": (
        "int64_t b = m / T;",
        "int64_t b = m % T;",
        "test_adaln_matches_torch_layer_norm", {"M": 7, "d": 1152, "T": 3}),
    "bf16_rounding_ties_away": (
        "if (rem > half || (rem == half && fmod(m, 2.0) == 1.0))\n        m += 1.0;\n    double r = m * ulp;",
        "if (rem >= half)\n        m += 1.0;\n    double r = m * ulp;",
        "test_double_to_bf16_nearest_even", {}),
    "kron16_bit_order_lsb_first": (
        "int rk = (r >> (3 - k)) & 1;\n                int ck = (c >> (3 - k)) & 1;",
        "int rk = (r >> k) & 1;\n                int ck = (c >> k) & 1;",
        "test_kron_block16_equals_numpy_kron", {"seed": 21}),
    "transform16_set_of_the_wrong_block": (
        "oracle_kron_block16(factors + (nT == 1 ? 0 : j) * 16, K);\n            for (int c = 0; c < 16; ++c) {\n"
        "                double acc = 0.0, mag = 0.0;",
        "oracle_kron_block16(factors + (nT == 1 ? 0 : j / 2) * 16, K);\n            for (int c = 0; c < 16; ++c) {\n"
        "                double acc = 0.0, mag = 0.0;",
        "test_transform16_per_block_sets_equal_modewise_product", {}),
    "mx16_amax_over_half_the_block": (
        "for (int i = 0; i < 16; ++i) {\n        if (!isfinite(y16[i]))",
        "for (int i = 0; i < 8; ++i) {\n        if (!isfinite(y16[i]))",
        "test_mx_block16_equals_padded_mx32", {}),
    "wht_sign_flipped": (
        "K[r * 32 + c] = par ? -scale : scale;",
        "K[r * 32 + c] = par ? scale : -scale;",
        "test_wht_block_is_sylvester_hadamard", {}),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pin_catches_planted_mistake(name, tmp_path, monkeypatch):
    old, new, pin, kwargs = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut_c = tmp_path / "kq_oracle_mut.c"
    mut_c.write_text(src.replace(old, new))
    mut_so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", str(mut_so), str(mut_c), "-lm"], check=True)
    L = oracle.bind(ctypes.CDLL(str(mut_so)))
    monkeypatch.setattr(oracle, "_lib", L)
    with pytest.raises(AssertionError):
        getattr(pins, pin)(oracle_lib=oracle, **kwargs)
