"""Pins of the oracle's post-read epilogue (value up-projection and sigmoid output gate).

The pages give no formula; the reading (v_th = W_UV[h] o_th, u_th = v_th * sigmoid(g_th),
coordinatewise) follows the page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie",
section "Was ändert sich – und was nicht?" (96 heads, 128-wide value heads) and the
paragraph on the gated MLA output gate.  Each check below would fail for a plausible slip:
a transposed W_UV, a swapped head index, a sign error in the sigmoid, a gate applied per
head instead of per coordinate.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from oracle import dsa_oracle as O


def bits(x):
    """Exact bf16 patterns of values that bf16 represents exactly."""
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32) >> np.uint32(16)
    assert np.array_equal((b.astype(np.uint32) << np.uint32(16)).view(np.float32), x)
    return b.astype(np.uint16)


def test_sigmoid_against_library_and_symmetry():
    x = np.linspace(-30, 30, 1201)
    assert np.allclose(O.sigmoid(x), scipy.special.expit(x), rtol=1e-15, atol=0)
    assert O.sigmoid(0.0) == 0.5
    assert np.allclose(O.sigmoid(-x), 1.0 - O.sigmoid(x), rtol=0, atol=4e-16)  # 1 - s loses ~1 ulp of 1
    assert O.sigmoid(800.0) == 1.0 and O.sigmoid(-800.0) == 0.0  # no overflow either way


def test_open_gate_equals_exact_integer_projection():
    """Gate logits of 2^100 make sigmoid exactly 1; integer inputs make the contraction
    exact, so u must equal a brute-force rational sum."""
    g = np.random.default_rng(0)
    t, h = 2, 3
    o = g.integers(-3, 4, size=(t, h, 512))
    w = np.zeros((96, 128, 512))
    w[:h] = g.integers(-2, 3, size=(h, 128, 512))
    gate = np.full((t, 96, 128), 2.0 ** 100)
    ob = np.zeros((t, 96, 512)); ob[:, :h] = o
    u = O.value_gate(bits(ob), bits(w), bits(gate))
    for ti in range(t):
        for hi in range(h):
            for c in (0, 1, 77, 127):
                ref = sum(Fraction(int(w[hi, c, k])) * int(o[ti, hi, k]) for k in range(512))
                assert u[ti, hi, c] == float(ref)
    assert np.all(u[:, h:] == 0)


def test_identity_projection_and_half_gate():
    """W_UV[h] = [I_128 | 0] picks the first 128 latent coordinates; zero logits halve them."""
    g = np.random.default_rng(1)
    o = g.standard_normal((3, 96, 512)).astype(np.float32)
    o = (o.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # bf16-exact values
    w = np.zeros((96, 128, 512), np.float32)
    w[:, np.arange(128), np.arange(128)] = 1.0
    u = O.value_gate(bits(o), bits(w), bits(np.zeros((3, 96, 128), np.float32)))
    assert np.array_equal(u, o[:, :, :128].astype(np.float64) / 2)


def test_closed_gate_and_coordinatewise_gate():
    g = np.random.default_rng(2)
    o = bits(np.round(g.standard_normal((2, 96, 512)) * 4) / 4)
    w = bits(np.round(g.standard_normal((96, 128, 512)) * 4) / 4)
    gate = np.zeros((2, 96, 128), np.float32)
    gate[:, :, ::2] = -(2.0 ** 100)  # closed on even coordinates, half open on odd ones
    u = O.value_gate(o, w, bits(gate))
    v = O.value_gate(o, w, bits(np.full((2, 96, 128), 2.0 ** 100, np.float32)))
    assert np.all(u[:, :, ::2] == 0)
    assert np.array_equal(u[:, :, 1::2], v[:, :, 1::2] / 2)


def test_against_torch_bmm_and_head_permutation():
    g = np.random.default_rng(3)
    ob = bits((g.standard_normal((4, 96, 512)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    wb = bits((g.standard_normal((96, 128, 512)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    gb = bits((g.standard_normal((4, 96, 128)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    u = O.value_gate(ob, wb, gb)
    o64 = torch.from_numpy(O.bf16_to_f64(ob))
    w64 = torch.from_numpy(O.bf16_to_f64(wb))
    g64 = torch.from_numpy(O.bf16_to_f64(gb))
    ref = torch.bmm(w64, o64.permute(1, 2, 0).contiguous()).permute(2, 0, 1) * torch.sigmoid(g64)
    assert np.allclose(u, ref.numpy(), rtol=1e-12, atol=1e-12)
    perm = g.permutation(96)
    up = O.value_gate(ob[:, perm], wb[perm], gb[:, perm])
    assert np.array_equal(up, u[:, perm])


def test_magnitude_bounds_the_value():
    g = np.random.default_rng(4)
    ob = bits((g.standard_normal((2, 96, 512)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    wb = bits((g.standard_normal((96, 128, 512)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    gb = bits((g.standard_normal((2, 96, 128)).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32))
    assert np.all(np.abs(O.value_gate(ob, wb, gb)) <= O.value_gate_magnitude(ob, wb, gb) * (1 + 1e-12))
