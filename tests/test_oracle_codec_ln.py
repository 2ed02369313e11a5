"""Pins for the oracle's bf16 codec and its index-key LayerNorm (CPU only).

Each check ties the oracle to something other than itself: the bf16 bit-level
definition, torch's float32->bfloat16 conversion, torch's layer_norm, or closed forms.
"""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O


def test_bf16_roundtrip_all_finite_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = O.bf16_to_f64(bits)
    finite = np.isfinite(vals)
    back = O.f64_to_bf16(vals[finite])
    assert np.array_equal(back, bits[finite])
    # NaN patterns collapse to the canonical quiet NaN
    assert np.all(O.f64_to_bf16(vals[np.isnan(vals)]) == 0x7FC0)
    assert O.f64_to_bf16(np.array([np.inf, -np.inf])).tolist() == [0x7F80, 0xFF80]


def test_bf16_midpoints_round_to_even():
    # consecutive positive finite bf16 values a < b; their midpoint is exact in float64
    lo = np.arange(0x0001, 0x7F7F, dtype=np.uint32).astype(np.uint16)
    a, b = O.bf16_to_f64(lo), O.bf16_to_f64(lo + 1)
    mid = (a + b) / 2
    got = O.f64_to_bf16(mid)
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, even)
    assert np.array_equal(O.f64_to_bf16(-mid), even | np.uint16(0x8000))
    # just above / below the midpoint go to the nearer neighbour
    assert np.array_equal(O.f64_to_bf16(np.nextafter(mid, np.inf)), lo + 1)
    assert np.array_equal(O.f64_to_bf16(np.nextafter(mid, -np.inf)), lo)


def test_bf16_matches_torch_on_float32_inputs():
    g = np.random.default_rng(7)
    x = np.concatenate([
        (g.standard_normal(200000) * 10.0 ** g.integers(-40, 38, 200000)).astype(np.float32),
        np.array([3.3961e38, 3.39e38, 1e-40, -1e-45, 0.0, -0.0], np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16(x.astype(np.float64))
    finite = np.isfinite(x)
    assert np.array_equal(got[finite], ref[finite])


def test_ln_constant_row_gives_beta_exactly():
    beta = np.linspace(-1, 1, 128).astype(np.float32)
    gamma = np.full(128, 1.7, np.float32)
    raw = np.full((3, 128), 5.5, np.float32)
    y = O.layernorm_keys(raw, gamma, beta, 1e-6)
    assert np.array_equal(y, np.broadcast_to(beta.astype(np.float64), y.shape))


def test_ln_matches_torch_layer_norm_fp64():
    g = np.random.default_rng(1)
    raw = (g.standard_normal((64, 128)) * 3 + 1).astype(np.float32)
    gamma = (1 + 0.3 * g.standard_normal(128)).astype(np.float32)
    beta = (0.3 * g.standard_normal(128)).astype(np.float32)
    eps = np.float32(1e-6)
    ref = torch.nn.functional.layer_norm(
        torch.from_numpy(raw.astype(np.float64)), (128,),
        torch.from_numpy(gamma.astype(np.float64)), torch.from_numpy(beta.astype(np.float64)),
        eps=float(eps)).numpy()
    assert np.allclose(O.layernorm_keys(raw, gamma, beta, eps), ref, rtol=0, atol=1e-12)


def test_ln_alternating_row_closed_form():
    # x = +-c alternating: mean 0, biased variance c^2, so y = sign * c/sqrt(c^2+eps)*g+b
    c, eps = 2.0, 1e-6
    raw = np.tile(np.array([c, -c], np.float32), 64)[None, :]
    gamma = np.full(128, 0.5, np.float32)
    beta = np.full(128, 0.25, np.float32)
    y = O.layernorm_keys(raw, gamma, beta, eps)
    expect = np.tile([1.0, -1.0], 64) * c / np.sqrt(c * c + float(np.float32(eps))) * 0.5 + 0.25
    assert np.allclose(y[0], expect, rtol=0, atol=1e-15)


def test_ln_unit_affine_invariants_and_shift_scale_invariance():
    g = np.random.default_rng(2)
    raw = g.standard_normal((50, 128)).astype(np.float32)
    one, zero = np.ones(128, np.float32), np.zeros(128, np.float32)
    y = O.layernorm_keys(raw, one, zero, 0.0)
    assert np.allclose(y.mean(axis=1), 0, atol=1e-14)
    assert np.allclose((y * y).mean(axis=1), 1, atol=1e-12)
    # LN(a x + c) == LN(x) for a > 0 when eps = 0 (a power of two keeps fp32 inputs exact)
    y2 = O.layernorm_keys(raw * np.float32(4.0) + np.float32(0.0), one, zero, 0.0)
    assert np.allclose(y, y2, atol=1e-12)


def test_ln_bf16_output_is_correct_rounding():
    g = np.random.default_rng(3)
    raw = g.standard_normal((16, 128)).astype(np.float32)
    gamma = (1 + 0.3 * g.standard_normal(128)).astype(np.float32)
    beta = (0.3 * g.standard_normal(128)).astype(np.float32)
    y = O.layernorm_keys(raw, gamma, beta, 1e-6)
    bits = O.layernorm_keys_bf16(raw, gamma, beta, 1e-6)
    v = O.bf16_to_f64(bits)
    # the stored value is within half a bf16 spacing of the exact value
    spacing = np.ldexp(1.0, np.frexp(np.abs(v))[1] - 8)
    assert np.all(np.abs(v - y) <= spacing / 2 + 1e-300)
