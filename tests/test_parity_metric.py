"""CPU checks of the parity metric that every GPU parity test uses.

The metric (tests/parity.py) must pass a correctly rounded bf16 result,
fail a truncating store and a too-large fp32 error, flag non-finite output,
and its side figures must round ties to even.
"""
import numpy as np

from parity import TOL, diagnostics, parity_error, rne_bf16
from linear_spatial_propagation_amd.inputs import bf16_bits_to_f32


def test_correctly_rounded_bf16_scores_zero():
    yhat = np.random.default_rng(0).standard_normal(200_000)
    y = rne_bf16(yhat)
    assert parity_error(y, yhat, "bf16") == 0.0
    assert diagnostics(y, yhat, "bf16")["frac_not_rne"] == 0.0


def test_truncating_bf16_store_fails():
    """Rounding toward zero instead of to nearest: about one bf16 ulp of
    error on half the values, above the 2e-3 bound (the metric only forgives
    the half ulp of a correct rounding)."""
    yhat = np.random.default_rng(1).standard_normal(200_000)
    bits = yhat.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    y = bits.view(np.float32).astype(np.float64)
    assert parity_error(y, yhat, "bf16") > TOL["bf16"]


def test_fp32_bound():
    yhat = np.random.default_rng(2).standard_normal(10_000) + 3.0
    assert parity_error(yhat * (1 + 5e-5), yhat, "f32") <= TOL["f32"]
    assert parity_error(yhat * (1 + 2e-4), yhat, "f32") > TOL["f32"]


def test_near_zero_outputs_use_the_rms_floor():
    """An output that cancels to ~0 is judged against 0.1 rms, not against itself."""
    yhat = np.array([1.0, -1.0, 1e-12])
    y = yhat + np.array([0.0, 0.0, 1e-6])
    assert parity_error(y, yhat, "f32") < TOL["f32"]


def test_non_finite_output_fails():
    yhat = np.ones(8)
    y = yhat.copy()
    y[3] = np.nan
    assert parity_error(y, yhat, "f32") == float("inf")


def test_rne_ties_to_even():
    # 1 + 2^-8 lies halfway between the bf16 values 1 and 1 + 2^-7: the even
    # mantissa (1.0) wins; 1 + 3 * 2^-8 lies between 1 + 2^-7 and 1 + 2^-6:
    # the even one is 1 + 2^-6
    got = rne_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]))
    np.testing.assert_array_equal(got, [1.0, 1 + 2.0 ** -6, -1.0])
    # every bf16 value is its own rounding
    b = np.arange(0x3F00, 0x4100, dtype=np.uint16)
    v = bf16_bits_to_f32(b).astype(np.float64)
    np.testing.assert_array_equal(rne_bf16(v), v)
