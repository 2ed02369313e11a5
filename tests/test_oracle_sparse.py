"""Pins for the oracle's restricted-softmax sparse read, its dense reference and the
dropped-mass bound, plus the page's printed byte arithmetic (CPU only)."""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import synth
from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")


def _small(seed, s_len, pos=None, k=2048):
    lay = synth.decode_layout("t", seed, s_len)
    if pos is not None:
        lay.q_pos[:] = pos
    d = synth.inputs_np(lay, parts=("mla",))
    return lay, d


def test_short_prefix_equals_dense_causal_sdpa():
    # with n_t <= 2048 every admissible position is selected: the read is dense attention
    lay, d = _small(31, [300, 1000, 2048])
    ids = O.topk_rows([np.zeros(min(p + 1, s)) for p, s in zip(lay.q_pos, lay.s_len)])
    out, lse = O.sparse_mla(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, ids,
                            synth.ATTN_SCALE)
    for t in range(lay.T):
        b, n = lay.q_req[t], lay.s_len[t]
        rows = O.gather_rows(d["latent"], d["kpe"], lay.kv_off[b] + np.arange(n))
        q = torch.from_numpy(O.bf16_to_f64(d["q"][t]))[:, None, :]        # [96,1,576]
        k = torch.from_numpy(rows)[None].expand(96, n, 576)
        v = torch.from_numpy(rows[:, :512])[None].expand(96, n, 512)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=synth.ATTN_SCALE)
        assert np.allclose(out[t], ref[:, 0].numpy(), rtol=0, atol=1e-12)
        a = synth.ATTN_SCALE * (O.bf16_to_f64(d["q"][t]) @ rows.T)
        assert np.allclose(lse[t], scipy.special.logsumexp(a, axis=1), atol=1e-12)


def test_weights_sum_to_one_via_ones_column():
    lay, d = _small(32, [5000, 3000])
    lat = O.bf16_to_f64(d["latent"])
    lat[:, 0] = 1.0
    latent = O.f64_to_bf16(lat)
    ids = synth.random_ids_np(32, lay)
    out, _ = O.sparse_mla(d["q"], latent, d["kpe"], lay.kv_off, lay.q_req, ids,
                          synth.ATTN_SCALE)
    assert np.allclose(out[:, :, 0], 1.0, rtol=0, atol=1e-14)


def test_single_valid_id_reads_that_row_and_empty_row_reads_zero():
    lay, d = _small(33, [100, 100])
    ids = np.full((2, 2048), -1, np.int32)
    ids[0, 0] = 42
    ids[1, 5] = 1000  # beyond S_b: padding, so row 1 has no valid id
    out, lse = O.sparse_mla(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, ids,
                            synth.ATTN_SCALE)
    expect = O.bf16_to_f64(d["latent"][lay.kv_off[0] + 42])
    assert np.array_equal(out[0], np.broadcast_to(expect, (96, 512)))
    rows = O.gather_rows(d["latent"], d["kpe"], [lay.kv_off[0] + 42])
    assert np.allclose(lse[0], synth.ATTN_SCALE * (O.bf16_to_f64(d["q"][0]) @ rows[0]))
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_id_order_and_padding_do_not_matter():
    lay, d = _small(34, [6000])
    ids = synth.random_ids_np(34, lay)
    g = np.random.default_rng(0)
    shuffled = ids.copy()
    shuffled[0] = g.permutation(shuffled[0])
    shuffled = np.concatenate([shuffled, np.full((1, 10), -1, np.int32)], axis=1)
    a = O.sparse_mla(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, ids, 0.07)
    b = O.sparse_mla(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, shuffled, 0.07)
    assert np.allclose(a[0], b[0], atol=1e-13) and np.allclose(a[1], b[1], atol=1e-12)


def test_dropped_mass_identity_and_bounds():
    lay, d = _small(35, [9000, 4096, 2500])
    ids = synth.random_ids_np(35, lay)
    out, _ = O.sparse_mla(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, ids,
                          synth.ATTN_SCALE)
    dr = O.dense_read(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, lay.q_pos, ids,
                      synth.ATTN_SCALE)
    eps = dr["eps"][:, :, None]
    assert np.all((dr["eps"] > 0) & (dr["eps"] < 1))
    # exact identity: the full read is the eps-mixture of the retained and dropped reads
    assert np.allclose(dr["o_full"], (1 - eps) * out + eps * dr["o_drop"], rtol=0, atol=1e-12)
    diff = np.abs(out - dr["o_full"])
    assert np.all(diff <= eps * dr["v_range"][:, None, :] + 1e-12)
    norms = np.sqrt((( out - dr["o_full"]) ** 2).sum(-1))
    assert np.all(norms <= 2 * dr["eps"] * dr["v_maxnorm"][:, None] + 1e-12)


def test_all_selected_means_no_dropped_mass():
    lay, d = _small(36, [1500])
    ids = synth.random_ids_np(36, lay)
    dr = O.dense_read(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, lay.q_pos, ids,
                      synth.ATTN_SCALE)
    out, _ = O.sparse_mla(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, ids,
                          synth.ATTN_SCALE)
    assert np.all(dr["eps"] == 0)
    assert np.allclose(out, dr["o_full"], atol=1e-12)


def test_page_printed_byte_arithmetic():
    g = json.load(open(GOLDEN))
    per_token = O.payload_bytes_per_token()
    assert per_token == g["payload_per_token_KiB"] * 1024
    assert O.payload_bytes_at(g["context_limit_tokens"]) == g["payload_at_limit_GiB"] * 2 ** 30
    assert O.selection_fraction(g["topk"], g["context_limit_tokens"]) == \
        1 / g["selected_fraction_denominator"]
    assert 100 * O.selection_fraction() == g["selected_fraction_percent"]
    assert O.payload_bytes_per_position_per_layer() == \
        (g["latent_elems"] + g["companion_elems"] + g["index_key_elems"]) * g["elem_bytes_bf16"]
    assert O.GLOBAL_LAYERS == g["global_layers"] and O.TOPK == g["topk"]
