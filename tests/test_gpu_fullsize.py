"""Parity at the full workload sizes, in the launch configuration the benchmark times.

Inputs are drawn on the GPU (seeded); the oracle receives host copies of the same bits and
recomputes 16 evenly spaced queries (the first and the last included; all of them when there
are fewer) from scratch: its own LayerNorm, scores and top-k (the GPU's selected set must
equal the oracle's up to the 1e-3 band of the k-th score), and its read of the GPU's own ID
set (1e-2 on the output, 1e-3 relative on lse).  The whole ID array is checked for the
invariants that hold at any size.
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


def check_query(lay, t, keys_f64_req, q_idx, w, ids_gpu_row, band_rel=1e-3):
    """Oracle scores + top-k for query t over its request's keys (decoded by the oracle's
    codec); returns oracle IDs."""
    n = O.admissible_count(lay.q_pos[t], lay.s_len[lay.q_req[t]])
    s = O.indexer_scores_one(O.bf16_to_f64(q_idx), O.bf16_to_f64(w), keys_f64_req[:n])
    ref = O.topk_ids(s)
    m = min(n, 2048)
    got = ids_gpu_row
    assert np.all(got[m:] == -1) and np.all(np.diff(got[:m]) > 0)
    diff = set(got[:m].tolist()) ^ set(ref[:m].tolist())
    assert diff <= set(O.selection_band(s, 2048, band_rel).tolist()), f"query {t}"
    return ref


def sparse_check(ids_gpu_row, q_t, latent_req, kpe_req, out_t, lse_t):
    """The GPU read against the oracle's read of the GPU's own (valid, checked) ID set:
    attention on the same selected set within 1e-2 (+ half a bf16 ulp for the output)."""
    j = ids_gpu_row[ids_gpu_row >= 0]
    rows = np.concatenate([O.bf16_to_f64(latent_req[j, :512]), O.bf16_to_f64(kpe_req[j, :64])], 1)
    o, l = O.restricted_softmax_read(O.bf16_to_f64(q_t), rows, synth.ATTN_SCALE)
    half_ulp = np.where(o != 0, np.ldexp(1.0, np.frexp(np.abs(o))[1] - 9), 0.0)
    assert np.all(np.abs(out_t - o) <= 1e-2 + half_ulp)  # bf16 output: + its own rounding
    assert np.all(np.abs(lse_t - l) <= 1e-3 * np.maximum(1, np.abs(l)))


def sample_queries(t_count, n=16):
    """n evenly spaced queries, the first and the last included (all of them if fewer)."""
    return sorted(set(np.linspace(0, t_count - 1, min(n, t_count)).round().astype(int).tolist()))


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


@pytest.mark.parametrize("name", ["decode_b64_s32768", "prefill_t4096_s65536",
                                  "long_decode_b4_s1m", "long_prefill_t8192_s1m"])
def test_full_size_sampled(name):
    lay = synth.workload(name)
    sample = sample_queries(lay.T)
    print(f"[full] {name} sample={sample}", flush=True)
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
    cache = {}  # per request: the oracle's keys, latent and companion rows
    for t in sample:
        b = int(lay.q_req[t])
        if b not in cache:
            cache.clear()
            lo, hi = int(lay.kv_off[b]), int(lay.kv_off[b + 1])
            if lay.raw_keys:
                raw = hb(d["raw_keys"][lo:hi])
                keys_ref = O.layernorm_keys_bf16(raw, hb(d["gamma"]), hb(d["beta"]), synth.LN_EPS)
            else:
                keys_ref = hb(d["keys"][lo:hi])
            cache[b] = (O.bf16_to_f64(keys_ref), hb(d["latent"][lo:hi]), hb(d["kpe"][lo:hi]))
        keys_ref, lat, kpe = cache[b]
        check_query(lay, t, keys_ref, hb(d["q_idx"][t]), hb(d["w"][t]), ids_h[t])
        sparse_check(ids_h[t], hb(d["q"][t]), lat, kpe, out[t].float().cpu().numpy(),
                     lse[t].cpu().numpy())
        print(f"  query {t} ok", flush=True)
    del d, keys, ids, out, lse, cache
    torch.cuda.empty_cache()
