"""Pins of the oracle's FP8 index-key cache variant: the OCP E4M3 codec, the per-row
power-of-two scale, the quantised keys and the scores over them.  Pages: "Kimi K3.1 Pro:
Sparse-Zugriffe, keine kleinere Historie", section "Warum Top-2048 keinen 2048-Token-Cache
bedeutet" (index quantisation and scale metadata) and section "Was ein Deployment validieren
muss" (cache precision as an option)."""
import numpy as np
import torch

import synth
from oracle import dsa_oracle as O

bits = synth.bf16_bits_from_f32


def test_decode_matches_torch_float8_e4m3fn_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.nanmax(got) == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_encode_round_trips_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(O.e4m3_encode(vals[fin].astype(np.float32)), codes[fin])


def test_encode_is_round_to_nearest_even_like_torch():
    """Midpoints between neighbouring codes go to the even code; everything else to the
    nearest.  torch's float32 -> float8_e4m3fn conversion is the library reference."""
    codes = np.arange(0, 0x7F, dtype=np.uint8)  # non-negative finite codes
    v = O.e4m3_decode(codes)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    g = np.random.default_rng(1)
    rand = (g.random(20000) * 448).astype(np.float32)
    tiny = (g.random(2000) * 2.0 ** -6).astype(np.float32)
    x = np.concatenate([mids, -mids, rand, -rand, tiny, -tiny, np.float32([0.0, -0.0, 448.0, -448.0])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)
    even = O.e4m3_encode(mids) & 1
    assert np.all(even == 0)


def test_scale_exponent_is_the_smallest_that_fits():
    g = np.random.default_rng(2)
    k = bits(g.standard_normal((500, 128)) * np.exp(g.uniform(-20, 20, (500, 1))))
    e = O.key_scale_exponent(k)
    amax = np.abs(O.bf16_to_f64(k)).max(axis=1)
    assert np.all(amax <= 448.0 * np.ldexp(1.0, e))
    assert np.all(amax > 448.0 * np.ldexp(1.0, e - 1))
    assert O.key_scale_exponent(np.zeros((1, 128), np.uint16))[0] == 0


def test_quantised_keys_are_within_half_a_code_step():
    """Each decoded key differs from the bf16 key by at most half the spacing of E4M3 at that
    magnitude (relative 2^-4 for normal codes, absolute 2^-10 * scale below them), and the
    largest element of each row uses a code in [224, 448]."""
    lay = synth.decode_layout("q8", 3, [600])
    k = O.layernorm_keys_bf16(synth.inputs_np(lay, parts=("index",))["raw_keys"],
                              np.ones(128, np.float32), np.zeros(128, np.float32), 1e-6)
    codes, scales = O.quantize_keys_fp8(k)
    kd = O.dequantize_keys_fp8(codes, scales)
    kf = O.bf16_to_f64(k)
    s = scales.astype(np.float64)[:, None]
    a = np.abs(kf) / s
    step = np.where(a >= 2.0 ** -6, np.ldexp(1.0, np.floor(np.log2(np.maximum(a, 1e-300))).astype(int) - 3), 2.0 ** -9)
    assert np.all(np.abs(kd - kf) <= step / 2 * s + 1e-300)
    top = np.abs(O.e4m3_decode(codes)).max(axis=1)
    assert np.all((top >= 224) & (top <= 448))


def test_fp8_scores_are_scores_of_the_decoded_keys_and_scale_out():
    """Scores over the FP8 cache equal indexer_scores of the decoded keys; scaling a row's
    keys by 2^j leaves its codes unchanged and scales its scores by 2^j (ReLU commutes with a
    positive scale)."""
    lay = synth.decode_layout("s8", 4, [300, 50])
    d = synth.inputs_np(lay, parts=("index",))
    k = synth.bf16_bits_from_f32(d["raw_keys"])
    codes, scales = O.quantize_keys_fp8(k)
    s8 = O.indexer_scores_fp8(d["q_idx"], d["w"], codes, scales, lay.kv_off, lay.q_req, lay.q_pos)
    sd = O.indexer_scores(d["q_idx"], d["w"], O.dequantize_keys_fp8(codes, scales), lay.kv_off,
                          lay.q_req, lay.q_pos)
    for a, b in zip(s8, sd):
        assert np.array_equal(a, b)
    k4 = bits(O.bf16_to_f64(k) * 16.0)
    codes4, scales4 = O.quantize_keys_fp8(k4)
    assert np.array_equal(codes4, codes) and np.array_equal(scales4, scales * 16)
    s4 = O.indexer_scores_fp8(d["q_idx"], d["w"], codes4, scales4, lay.kv_off, lay.q_req, lay.q_pos)
    for a, b in zip(s4, s8):
        assert np.allclose(a, 16.0 * b, rtol=1e-12, atol=0)
