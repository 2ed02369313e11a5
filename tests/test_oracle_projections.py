"""Pins of the oracle's indexer-side projections (index queries from the query latent, the
index key from the residual state followed by the key LayerNorm, the head weights from the
residual state).  Page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie", section
"Eine Query durch den Indexer verfolgen"; widths from section "Was ändert sich – und was
nicht?" (query latent 1536, residual 7168)."""
from fractions import Fraction

import numpy as np
import torch

import synth
from oracle import dsa_oracle as O

bits = synth.bf16_bits_from_f32


def test_linear_equals_exact_integer_sums():
    """Small integers: every product and sum is an integer, computed exactly by Python ints;
    the [out, in] weight convention (row n of the weight makes output n) is pinned too."""
    g = np.random.default_rng(1)
    x = g.integers(-3, 4, size=(3, 37))
    w = g.integers(-2, 3, size=(5, 37))
    got = O.linear(bits(x), bits(w))
    for t in range(3):
        for n in range(5):
            assert got[t, n] == sum(int(x[t, k]) * int(w[n, k]) for k in range(37))


def test_linear_on_rationals_against_fraction_brute_force():
    """Dyadic bf16 values: the fp64 matmul of 64 terms is exact here, as rational sums show."""
    g = np.random.default_rng(2)
    x = bits(g.standard_normal((2, 64)))
    w = bits(g.standard_normal((3, 64)))
    xf, wf = O.bf16_to_f64(x), O.bf16_to_f64(w)
    got = O.linear(x, w)
    for t in range(2):
        for n in range(3):
            exact = sum(Fraction(float(xf[t, k])) * Fraction(float(wf[n, k])) for k in range(64))
            assert abs(Fraction(float(got[t, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_index_query_head_layout_from_one_hot_weights():
    """W_qi row j = 128 head + dim picks latent coordinate perm[j]: q_idx[t, head, dim] must be
    that coordinate of c_q (the [T,32,128] reshape puts the head first)."""
    g = np.random.default_rng(3)
    t = 4
    c_q = bits(g.standard_normal((t, 1536)))
    perm = g.integers(0, 1536, size=4096)
    w_qi = np.zeros((4096, 1536), np.float32)
    w_qi[np.arange(4096), perm] = 1.0
    z128 = np.zeros((128, 7168), np.uint16)
    out = O.indexer_projections(c_q, np.zeros((t, 7168), np.uint16), bits(w_qi), z128,
                                np.zeros((32, 7168), np.uint16), np.ones(128, np.float32),
                                np.zeros(128, np.float32), 1e-6)
    assert out["q_idx"].shape == (t, 32, 128)
    for head in (0, 5, 31):
        for dim in (0, 77, 127):
            assert np.array_equal(out["q_idx"][:, head, dim], c_q[:, perm[128 * head + dim]])


def test_head_weights_from_one_hot_residual():
    """h_t = e_i gives w[t, head] = W_w[head, i] exactly (bf16 in, bf16 out)."""
    g = np.random.default_rng(4)
    idx = np.array([0, 4000, 7167])
    h = np.zeros((3, 7168), np.float32)
    h[np.arange(3), idx] = 1.0
    w_w = bits(g.standard_normal((32, 7168)) * 0.01)
    out = O.indexer_projections(np.zeros((3, 1536), np.uint16), bits(h),
                                np.zeros((4096, 1536), np.uint16), np.zeros((128, 7168), np.uint16),
                                w_w, np.ones(128, np.float32), np.zeros(128, np.float32), 1e-6)
    for t in range(3):
        assert np.array_equal(out["w"][t], w_w[:, idx[t]])


def test_key_is_layernorm_of_the_exact_projection():
    """Integer residual and key weights: the raw key is an exact integer vector, and the key is
    torch's fp64 layer_norm of it (biased variance, affine), rounded once to bf16.  A key
    normalised from a bf16-rounded projection would differ here: the raw keys exceed 2^9,
    beyond bf16's 8 significant bits (fp32 holds these integers exactly)."""
    g = np.random.default_rng(5)
    t = 6
    h = g.integers(-4, 5, size=(t, 7168))
    w_k = g.integers(-1, 2, size=(128, 7168))
    gamma = (1 + 0.3 * g.standard_normal(128)).astype(np.float32)
    beta = (0.3 * g.standard_normal(128)).astype(np.float32)
    out = O.indexer_projections(np.zeros((t, 1536), np.uint16), bits(h),
                                np.zeros((4096, 1536), np.uint16), bits(w_k),
                                np.zeros((32, 7168), np.uint16), gamma, beta, 1e-6)
    exact = (h.astype(object) @ w_k.T.astype(object)).astype(np.float64)
    assert np.array_equal(out["k_raw"], exact)
    assert np.abs(exact).max() > 2 ** 9
    ref = torch.nn.functional.layer_norm(torch.from_numpy(exact), (128,),
                                         torch.from_numpy(gamma.astype(np.float64)),
                                         torch.from_numpy(beta.astype(np.float64)),
                                         eps=float(np.float32(1e-6))).numpy()
    assert np.allclose(out["key"], ref, rtol=0, atol=1e-12)
    assert np.array_equal(out["key_bf16"], O.f64_to_bf16(ref))
    rounded = O.layernorm64(O.bf16_to_f64(O.f64_to_bf16(exact)), gamma, beta, 1e-6)
    assert not np.array_equal(O.f64_to_bf16(rounded), out["key_bf16"])


def test_projections_are_linear_and_scale_exactly():
    """Doubling the inputs doubles q_idx and w exactly (powers of two commute with rounding)
    and leaves the LayerNorm key unchanged up to the eps term."""
    lay = synth.decode_layout("pin", 6, [10] * 3)
    d = synth.inputs_np(lay, parts=("proj",))
    a = O.indexer_projections(d["c_q"], d["h"], d["w_qi"], d["w_k"], d["w_w"], d["gamma"],
                              d["beta"], 1e-6)
    two = lambda x: bits(2.0 * O.bf16_to_f64(x))
    b = O.indexer_projections(two(d["c_q"]), two(d["h"]), d["w_qi"], d["w_k"], d["w_w"],
                              d["gamma"], d["beta"], 1e-6)
    assert np.array_equal(O.bf16_to_f64(b["q_idx"]), 2.0 * O.bf16_to_f64(a["q_idx"]))
    assert np.array_equal(O.bf16_to_f64(b["w"]), 2.0 * O.bf16_to_f64(a["w"]))
    assert np.array_equal(b["k_raw"], 2.0 * a["k_raw"])
    assert np.allclose(b["key"], a["key"], rtol=0, atol=1e-5)


def test_synthetic_projections_have_the_given_inputs_statistics():
    """Unit-gain weights: projected queries ~ N(0,1) and head weights ~ N(0,1/32), as the
    indexer's given inputs are drawn; each LayerNorm key's mean stays near beta's mean."""
    lay = synth.decode_layout("stat", 7, [10] * 64)
    d = synth.inputs_np(lay, parts=("proj",))
    out = O.indexer_projections(d["c_q"], d["h"], d["w_qi"], d["w_k"], d["w_w"], d["gamma"],
                                d["beta"], 1e-6)
    q = O.bf16_to_f64(out["q_idx"])
    w = O.bf16_to_f64(out["w"])
    assert abs(q.std() - 1.0) < 0.05 and abs(q.mean()) < 0.02
    assert abs(w.std() - synth.W_STD) < 0.02
    assert np.abs(out["key"].mean(axis=1) - d["beta"].astype(np.float64).mean()).max() < 0.2


def test_magnitude_bounds_the_value():
    lay = synth.decode_layout("mag", 8, [10] * 2)
    d = synth.inputs_np(lay, parts=("proj",))
    assert np.all(O.linear_magnitude(d["h"], d["w_k"]) >= np.abs(O.linear(d["h"], d["w_k"])))
