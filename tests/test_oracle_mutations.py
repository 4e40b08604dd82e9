"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of oracle.c (a flipped kernel,
a dropped term, a wrong stride / padding / dilation / group index, a
transposed weight index, a wrong error normaliser, a different rounding or
clamp), builds it with the oracle's own flags and runs the pins of
test_oracle_pins.py against it: at least one pin must fail.  The committed
oracle itself is never modified.
"""
import os

import pytest

import oracle
import tests.test_oracle_epilogue as epi_pins
import tests.test_oracle_pins as pins

MUTATIONS = {
    "kernel_flip": ("+ s * dw", "+ (S - 1 - s) * dw"),
    "stride_ignored": ("oh * sh - ph", "oh - ph"),
    "dilation_is_stride": ("r * dh", "r * sh"),
    "padding_sign": ("- ph +", "+ ph +"),
    "dropped_last_tap": ("for (int s = 0; s < S; ++s)", "for (int s = 0; s + 1 < S; ++s)"),
    "group_offset_dropped": ("const int c = g * Cg + cc;", "const int c = cc + 0 * g;"),
    "weight_index_transposed": ("* R + r) * S + s]", "* R + s) * S + r]"),
    "den_not_absolute": ("+= fabs(prod);", "+= prod;"),
    "round_half_away": ("rintf(prod)", "roundf(prod)"),
    "asymmetric_clamp": ("if (q < -127.0f)\n        return -127;", "if (q < -128.0f)\n        return -128;"),
    "exact_product": ("const float prod = a * scale;", "const float prod = (float)((double)acc * (double)scale); (void)a;"),
    # fused epilogue
    "epi_bias_dropped": ("v += bias[k];", "v += 0.0 * bias[k];"),
    "epi_bias_indexed_by_image": ("v += bias[k];", "v += bias[n % K];"),
    "epi_den_without_bias": ("d += fabs(bias[k]);", "d += 0.0;"),
    "epi_den_without_residual": ("d += fabs(res[o]);", "d += 0.0;"),
    "epi_relu_ignored": ("if (relu && v < 0.0)", "if (relu < 0 && v < 0.0)"),
    "epi_relu_before_residual": (
        "if (res) {\n                    v += res[o];\n                    d += fabs(res[o]);\n                }\n"
        "                if (relu && v < 0.0)\n                    v = 0.0;",
        "if (relu && v < 0.0)\n                    v = 0.0;\n                if (res) {\n"
        "                    v += res[o];\n                    d += fabs(res[o]);\n                }"),
    "epi_int8_bias_after_scale": ("const float a = (float)(int32_t)(acc + bias);\n    float q = a * scale;",
                                  "const float a = (float)(int32_t)acc;\n    float q = a * scale + (float)bias;"),
    "epi_int8_residual_before_scale": ("q = q + (float)res; /* one IEEE fp32 add */",
                                       "q = (a + (float)res) * scale;"),
    "epi_int8_relu_floor_ignored": ("const float lo = relu ? 0.0f : -127.0f;",
                                    "const float lo = -127.0f;\n    (void)relu;"),
}


def pin_checks():
    yield "worked_example", pins.test_worked_example_stride2
    yield "no_flip", pins.test_no_kernel_flip
    for i, case in enumerate(pins.cases(12, 1234)):
        yield "im2col_%d" % i, (lambda c=case: pins.test_vs_im2col_bruteforce(c))
    yield "groups", pins.test_groups_are_concatenated_convolutions
    yield "depthwise", pins.test_depthwise_is_per_channel_correlation
    yield "scipy", pins.test_single_channel_is_scipy_correlate2d
    yield "den", pins.test_den_properties
    yield "ties", pins.test_requant_ties_to_even
    yield "saturate", pins.test_requant_saturates_symmetrically
    yield "fp32_first", pins.test_requant_converts_acc_to_fp32_first
    yield "delta", lambda: pins.test_delta_kernel_is_identity(3, 3)
    for pin in epi_pins.PINS:
        yield pin.__name__, pin


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert old in src, "mutation pattern %r no longer matches oracle.c" % old
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(force=True, src=str(mutated), out=str(tmp_path / "liboracle_mut.so"))
    saved = oracle._default
    oracle._default = oracle.Oracle(lib)
    failed = []
    try:
        for label, check in pin_checks():
            try:
                check()
            except (AssertionError, ValueError, OverflowError):
                failed.append(label)
    finally:
        oracle._default = saved
        # the mutated library stays on disk until pytest removes tmp_path after
        # the session: a loaded library is never unloaded, and deleting its
        # file would let a later test's library reuse the inode, which the
        # dynamic loader then takes for the library it already has loaded
    assert failed, "planted mistake %r was not caught by any pin" % name
