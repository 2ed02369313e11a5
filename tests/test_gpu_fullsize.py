"""Parity at the full workload sizes, in the launch configuration the benchmark times.

Inputs are drawn on the GPU (seeded); the oracle receives host copies of the same bits and
recomputes sampled queries from scratch (its own LayerNorm, scores, top-k and sparse read).
"""
import numpy as np
import pytest

import synth
from oracle import dsa_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_indexer_top_key_amd as dsa
    dsa.library()
    yield
    torch.cuda.empty_cache()


def dsa_mod():
    import dsa_indexer_top_key_amd as dsa
    return dsa


def hb(x):
    return synth.to_bits_np(x)


def check_query(lay, t, keys_ref_req, q_idx, w, ids_gpu_row, band_rel=1e-3):
    """Oracle scores + top-k for query t over its request's keys; returns oracle IDs."""
    n = O.admissible_count(lay.q_pos[t], lay.s_len[lay.q_req[t]])
    s = O.indexer_scores_one(O.bf16_to_f64(q_idx), O.bf16_to_f64(w),
                             O.bf16_to_f64(keys_ref_req[:n]))
    ref = O.topk_ids(s)
    m = min(n, 2048)
    got = ids_gpu_row
    assert np.all(got[m:] == -1) and np.all(np.diff(got[:m]) > 0)
    diff = set(got[:m].tolist()) ^ set(ref[:m].tolist())
    assert diff <= set(O.selection_band(s, 2048, band_rel).tolist()), f"query {t}"
    return ref


def sparse_check(lay, t, ids_ref_row, ids_gpu_row, q_t, latent_req, kpe_req, out_t, lse_t):
    if not np.array_equal(ids_ref_row, ids_gpu_row):
        return False
    j = ids_ref_row[ids_ref_row >= 0]
    rows = np.concatenate([O.bf16_to_f64(latent_req[j, :512]), O.bf16_to_f64(kpe_req[j, :64])], 1)
    o, l = O.restricted_softmax_read(O.bf16_to_f64(q_t), rows, synth.ATTN_SCALE)
    half_ulp = np.where(o != 0, np.ldexp(1.0, np.frexp(np.abs(o))[1] - 9), 0.0)
    assert np.all(np.abs(out_t - o) <= 1e-2 + half_ulp)  # bf16 output: + its own rounding
    assert np.all(np.abs(lse_t - l) <= 1e-3 * np.maximum(1, np.abs(l)))
    return True


def run_path(lay, d):
    dsa = dsa_mod()
    if lay.raw_keys:
        keys = dsa.index_keys_layernorm(d["raw_keys"], d["gamma"], d["beta"], synth.LN_EPS)
    else:
        keys = d["keys"]
    ids = dsa.indexer_topk(d["q_idx"], d["w"], keys, d["kv_off"], d["q_req"], d["q_pos"],
                           lay.max_s)
    out, lse = dsa.sparse_mla_attn(d["q"], d["latent"], d["kpe"], d["kv_off"], d["q_req"], ids,
                                   synth.ATTN_SCALE)
    torch.cuda.synchronize()
    return keys, ids, out, lse


@pytest.mark.parametrize("name,sample", [("decode_b64_s32768", [0, 31, 63]),
                                         ("prefill_t4096_s65536", [0, 2047, 4095]),
                                         ("long_decode_b4_s1m", [0, 3]),
                                         ("long_prefill_t8192_s1m", [0, 8191])])
def test_full_size_sampled(name, sample):
    print(f"[full] {name} sample={sample}", flush=True)
    lay = synth.workload(name)
    d = synth.inputs_torch(lay, torch.device(DEV))
    keys, ids, out, lse = run_path(lay, d)
    ids_h = ids.cpu().numpy()
    # whole-array invariants: causality, -1 only as a suffix, ascending
    n_t = np.minimum(lay.q_pos.astype(np.int64) + 1, lay.s_len[lay.q_req])
    m = np.minimum(n_t, 2048)
    col = np.arange(2048)[None, :]
    assert np.all((ids_h >= 0) == (col < m[:, None]))
    assert np.all(ids_h < n_t[:, None])
    v = np.where(col < m[:, None], ids_h, np.iinfo(np.int32).max)
    assert np.all(np.diff(v, axis=1)[:, :] >= 0)
    assert torch.isfinite(out.float()).all()
    matched = 0
    for t in sample:
        b = int(lay.q_req[t])
        lo, hi = int(lay.kv_off[b]), int(lay.kv_off[b + 1])
        if lay.raw_keys:
            raw = hb(d["raw_keys"][lo:hi])
            keys_ref = O.layernorm_keys_bf16(raw, hb(d["gamma"]), hb(d["beta"]), synth.LN_EPS)
        else:
            keys_ref = hb(d["keys"][lo:hi])
        ref_ids = check_query(lay, t, keys_ref, hb(d["q_idx"][t]), hb(d["w"][t]), ids_h[t])
        lat = hb(d["latent"][lo:hi])
        kpe = hb(d["kpe"][lo:hi])
        matched += sparse_check(lay, t, ref_ids, ids_h[t], hb(d["q"][t]), lat, kpe,
                                out[t].float().cpu().numpy(), lse[t].cpu().numpy())
    assert matched >= 1, "no sampled query had an identical ID set to compare the read on"
    del d, keys, ids, out, lse
    torch.cuda.empty_cache()
