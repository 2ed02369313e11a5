"""GPU parity of the indexer-side projections (dsa_indexer_project) against the oracle.

Tolerances, derived from the arithmetic (bf16 operands, exact products, fp32 sums):
each output is a chain of at most K/16 MFMA accumulations (16 products per step) plus the
split-K partial sums, each an fp32 rounding, so
    |x_gpu - x_exact| <= delta = 2 (K/16 + 64) 2^-24 sum_k |a_k b_k|
before the output rounding.  q_idx and w then add one bf16 ulp.  The key adds the key
LayerNorm's own bound (one bf16 ulp, or 2^-16 (|x_hat gamma| + |beta|) where its terms
cancel) and the projection error carried through the normalisation,
|gamma| (2 + |x_hat|) delta_row / sigma.  Integer inputs make every sum exact in fp32: there
q_idx and w must equal the oracle bit for bit.
"""
import numpy as np
import pytest

import synth
from oracle import dsa_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = 0x7FC1  # a NaN pattern the kernel never writes


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_indexer_top_key_amd as dsa
    dsa.library()
    return dsa


def dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).to(DEV)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_ulp(v):
    a = np.abs(v)
    return np.where(a > 0, np.ldexp(1.0, np.maximum(np.frexp(a)[1] - 8, -133)), np.ldexp(1.0, -133))


def sum_bound(mag, k):
    return 2.0 * (k / 16 + 64) * 2.0 ** -24 * mag


def run_project(d, key_rows, cache_rows):
    import dsa_indexer_top_key_amd as dsa
    cache = torch.full((cache_rows, 128), SENTINEL, dtype=torch.int16, device=DEV)
    q, w = dsa.indexer_project(dev(d["c_q"]), dev(d["h"]), dev(d["w_qi"]), dev(d["w_k"]),
                               dev(d["w_w"]), dev(d["gamma"]), dev(d["beta"]), synth.LN_EPS,
                               cache, dev(key_rows.astype(np.int64)))
    torch.cuda.synchronize()
    return host_bits(q), host_bits(w), host_bits(cache)


def check_untouched(cache, key_rows):
    other = np.ones(cache.shape[0], bool)
    other[key_rows] = False
    assert np.all(cache[other] == SENTINEL)


def check_keys(got_bits, d, rows=None):
    """Key parity for the given token rows (all by default)."""
    h = d["h"] if rows is None else d["h"][rows]
    ref = O.indexer_projections(d["c_q"][:1], h, d["w_qi"], d["w_k"], d["w_w"], d["gamma"],
                                d["beta"], synth.LN_EPS)
    k_raw = ref["k_raw"]
    delta = sum_bound(O.linear_magnitude(h, d["w_k"]), 7168).max(axis=1, keepdims=True)
    mu = k_raw.mean(axis=1, keepdims=True)
    sigma = np.sqrt(((k_raw - mu) ** 2).mean(axis=1, keepdims=True) + np.float32(synth.LN_EPS))
    xhat = (k_raw - mu) / sigma
    g = d["gamma"].astype(np.float64)
    b = d["beta"].astype(np.float64)
    tol = (bf16_ulp(ref["key"]) + 2.0 ** -16 * (np.abs(xhat * g) + np.abs(b))
           + np.abs(g) * (2 + np.abs(xhat)) * delta / sigma)
    err = np.abs(O.bf16_to_f64(got_bits) - ref["key"])
    assert np.all(err <= tol), f"key max err {err.max()}"


def check_linear_out(got_bits, x, weight, k, ref_bits):
    ref = O.linear(x, weight)
    tol = bf16_ulp(ref) + sum_bound(O.linear_magnitude(x, weight), k)
    err = np.abs(O.bf16_to_f64(got_bits).reshape(ref.shape) - ref)
    assert np.all(err <= tol), f"max err {err.max()}"
    # the common case: the fp32 sum rounds to the oracle's bf16 value
    assert np.mean(got_bits.reshape(ref_bits.shape) == ref_bits) > 0.98


@pytest.mark.parametrize("t_count", [1, 64, 300, 512, 700])
def test_indexer_project_parity(t_count):
    """1 to 700 tokens: one partial 128-row tile up to five full tiles and a ragged one, with
    split counts from 32 down to a few."""
    print(f"[project] T={t_count}", flush=True)
    lay = synth.decode_layout("pj", 80 + t_count, [10] * t_count)
    d = synth.inputs_np(lay, parts=("proj",))
    g = np.random.default_rng(t_count)
    cache_rows = 2 * t_count + 5
    key_rows = g.permutation(cache_rows)[:t_count]  # distinct rows, scattered
    q, w, cache = run_project(d, key_rows, cache_rows)
    ref = O.indexer_projections(d["c_q"], d["h"], d["w_qi"], d["w_k"], d["w_w"], d["gamma"],
                                d["beta"], synth.LN_EPS)
    check_linear_out(q, d["c_q"], d["w_qi"], 1536, ref["q_idx"])
    check_linear_out(w, d["h"], d["w_w"], 7168, ref["w"])
    check_keys(cache[key_rows], d)
    check_untouched(cache, key_rows)


@pytest.mark.parametrize("t", [33, 64, 70, 600, 1000])
def test_indexer_project_exact_on_integer_inputs(t):
    """Small integers: every fp32 sum is exact, so q_idx and w equal the oracle bit for bit;
    the keys are the key LayerNorm of the exact integer projection.  33, 64 and 70 tokens: one
    ragged 128-row tile and many K splits; 600: four full tiles and a ragged one; 1000: an
    unsplit query product (its product kernel writes bf16 q_idx itself), ragged last tile."""
    print(f"[project] exact integers T={t}", flush=True)
    g = np.random.default_rng(90 + t)
    bits = synth.bf16_bits_from_f32
    d = {"c_q": bits(g.integers(-3, 4, size=(t, 1536))),
         "h": bits(g.integers(-3, 4, size=(t, 7168))),
         "w_qi": bits(g.integers(-1, 2, size=(4096, 1536)) * (g.random((4096, 1536)) < 0.3)),
         "w_k": bits(g.integers(-1, 2, size=(128, 7168)) * (g.random((128, 7168)) < 0.3)),
         "w_w": bits(g.integers(-1, 2, size=(32, 7168)) * (g.random((32, 7168)) < 0.3)),
         "gamma": (1 + 0.3 * g.standard_normal(128)).astype(np.float32),
         "beta": (0.3 * g.standard_normal(128)).astype(np.float32)}
    key_rows = np.arange(t)[::-1] * 3 + 1
    q, w, cache = run_project(d, key_rows, 3 * t + 2)
    ref = O.indexer_projections(d["c_q"], d["h"], d["w_qi"], d["w_k"], d["w_w"], d["gamma"],
                                d["beta"], synth.LN_EPS)
    assert np.abs(ref["k_raw"]).max() < 2 ** 24 and np.array_equal(ref["k_raw"], np.round(ref["k_raw"]))
    assert np.array_equal(q.reshape(ref["q_idx"].shape), ref["q_idx"])
    assert np.array_equal(w, ref["w"])
    # keys: the LayerNorm of an exactly computed fp32 raw key (key LayerNorm parity rule)
    got = cache[key_rows]
    ref_bits = O.layernorm_keys_bf16(ref["k_raw"].astype(np.float32), d["gamma"], d["beta"], synth.LN_EPS)
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    ulp1 = np.abs(ordered(got) - ordered(ref_bits)) <= 1
    close = np.abs(O.bf16_to_f64(got) - ref["key"]) <= 2.0 ** -20 * O.layernorm_error_scale(
        ref["k_raw"].astype(np.float32), d["gamma"], d["beta"], synth.LN_EPS)
    assert np.all(ulp1 | close)
    check_untouched(cache, key_rows)


def test_indexer_project_prefill_chunk_sampled():
    """A 4096-token prefill chunk (no K split for the query product): sampled tokens against
    the oracle, every output finite, every key row written."""
    print("[project] T=4096 sampled", flush=True)
    import dsa_indexer_top_key_amd as dsa
    lay = synth.prefill_layout("pjp", 95, 65536, 61440, 4096)
    dg = synth.inputs_torch(lay, torch.device(DEV), parts=("proj",))
    cache = torch.full((65536, 128), SENTINEL, dtype=torch.int16, device=DEV)
    key_rows = torch.arange(61440, 65536, dtype=torch.int64, device=DEV)
    q, w = dsa.indexer_project(dg["c_q"], dg["h"], dg["w_qi"], dg["w_k"], dg["w_w"], dg["gamma"],
                               dg["beta"], synth.LN_EPS, cache, key_rows)
    torch.cuda.synchronize()
    assert torch.isfinite(q.float()).all() and torch.isfinite(w.float()).all()
    cb = host_bits(cache)
    assert np.all(cb[:61440] == SENTINEL) and not np.any(cb[61440:] == SENTINEL)
    sample = np.array([0, 1, 2047, 4095])
    d = {k: synth.to_bits_np(v) for k, v in dg.items() if k in ("c_q", "h", "w_qi", "w_k", "w_w", "gamma", "beta")}
    sub = dict(d, c_q=d["c_q"][sample], h=d["h"][sample])
    ref = O.indexer_projections(sub["c_q"], sub["h"], d["w_qi"], d["w_k"], d["w_w"], d["gamma"],
                                d["beta"], synth.LN_EPS)
    check_linear_out(host_bits(q)[sample], sub["c_q"], d["w_qi"], 1536, ref["q_idx"])
    check_linear_out(host_bits(w)[sample], sub["h"], d["w_w"], 7168, ref["w"])
    check_keys(cb[61440 + sample], sub)


def test_projected_inputs_drive_the_indexer():
    """Layer front end to end: 8 decode tokens are projected, their keys appended at the end
    of their requests' caches, and the projected q_idx / w / keys drive dsa_indexer_topk; the
    selection equals the oracle's on the same bf16 tensors (up to the 1e-3 band)."""
    print("[project] feeds the indexer", flush=True)
    import dsa_indexer_top_key_amd as dsa
    s_len = [3000, 2049, 500, 4096, 2048, 7000, 100, 2500]
    lay = synth.decode_layout("pje", 97, s_len)
    d = synth.inputs_np(lay, parts=("proj",))
    g = np.random.default_rng(97)
    keys_np = synth.bf16_bits_from_f32(g.standard_normal((lay.N, 128)))  # earlier keys
    cache = dev(keys_np)
    key_rows = lay.kv_off[1:] - 1  # each token's own position, the last row of its request
    q, w = dsa.indexer_project(dev(d["c_q"]), dev(d["h"]), dev(d["w_qi"]), dev(d["w_k"]),
                               dev(d["w_w"]), dev(d["gamma"]), dev(d["beta"]), synth.LN_EPS,
                               cache, dev(key_rows.astype(np.int64)))
    ids = dsa.indexer_topk(q, w, cache, dev(lay.kv_off), dev(lay.q_req), dev(lay.q_pos), lay.max_s)
    torch.cuda.synchronize()
    kb = host_bits(cache)
    other = np.ones(lay.N, bool)
    other[key_rows] = False
    assert np.array_equal(kb[other], keys_np[other])
    s_ref = O.indexer_scores(host_bits(q), host_bits(w), kb, lay.kv_off, lay.q_req, lay.q_pos)
    got = ids.cpu().numpy()
    for t in range(lay.T):
        a = set(got[t][got[t] >= 0].tolist())
        ref_ids = O.topk_ids(s_ref[t])
        b = set(ref_ids[ref_ids >= 0].tolist())
        assert len(a) == len(b) and (a ^ b) <= set(O.selection_band(s_ref[t]).tolist()), t
