"""GPU parity of the paged page-pool layout (dsa_indexer_topk_paged, dsa_sparse_mla_attn_paged).

The paged entry points run the same arithmetic as the contiguous ones on the same logical
cache, so their results must be identical bit for bit (decode layouts: both use the streaming
scoring kernel).  A prefill-shaped call, which the contiguous path scores with the prefill
kernel (another summation order), is checked against the oracle over the unpaged cache:
selected sets up to the 1e-3 band of the k-th score.
"""
import numpy as np
import pytest

import synth
from oracle import dsa_oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_indexer_top_key_amd as dsa
    dsa.library()
    return dsa


def dsa_mod():
    import dsa_indexer_top_key_amd as dsa
    return dsa


def dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).to(DEV)


def page_layout(s_len, page_size, seed, spare=5):
    """A random page table: the requests' pages are a permutation of a pool that also holds
    `spare` unused pages.  Returns (page_table [B, max_pages] int32, pool_rows, row_of), where
    row_of[i] is the pool row of logical row i of the request-contiguous cache."""
    g = np.random.default_rng(seed)
    s_len = np.asarray(s_len, np.int64)
    pages = -(-s_len // page_size)
    perm = g.permutation(int(pages.sum()) + spare)
    pt = np.zeros((len(s_len), int(pages.max())), np.int32)
    row_of = []
    k = 0
    for b, n in enumerate(s_len):
        pt[b, :pages[b]] = perm[k:k + pages[b]]
        k += pages[b]
        p = np.arange(n, dtype=np.int64)
        row_of.append(pt[b, p // page_size].astype(np.int64) * page_size + p % page_size)
    return pt, len(perm) * page_size, np.concatenate(row_of)


def to_pool(contig, pool_rows, row_of):
    pool = torch.zeros((pool_rows,) + tuple(contig.shape[1:]), dtype=contig.dtype, device=DEV)
    pool[torch.as_tensor(row_of, device=DEV)] = contig
    return pool


DECODE = [[1, 63, 64, 65, 2047, 2049, 4096, 5000], [70000, 3, 33000]]


@pytest.mark.parametrize("page_size", [64, 256])
@pytest.mark.parametrize("s_len", DECODE)
def test_indexer_topk_paged_equals_contiguous(page_size, s_len):
    print(f"[paged] indexer_topk P={page_size} S={s_len}", flush=True)
    dsa = dsa_mod()
    lay = synth.decode_layout("pg", 21, s_len)
    d = synth.inputs_np(lay, parts=("index",))
    keys = dev(synth.bf16_bits_from_f32(np.random.default_rng(21).standard_normal((lay.N, 128))))
    pt, pool_rows, row_of = page_layout(s_len, page_size, 22)
    pool = to_pool(keys, pool_rows, row_of)
    args = (dev(d["q_idx"]), dev(d["w"]))
    lay_args = (dev(lay.kv_off), dev(lay.q_req), dev(lay.q_pos))
    ids = dsa.indexer_topk(*args, keys, *lay_args, lay.max_s)
    ids_p = dsa.indexer_topk_paged(*args, pool, dev(pt), page_size, *lay_args, lay.max_s)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_p)


@pytest.mark.parametrize("page_size,packed,f32", [(64, False, False), (128, True, True),
                                                  (64, True, False)])
def test_sparse_mla_paged_equals_contiguous(page_size, packed, f32):
    print(f"[paged] sparse read P={page_size} packed={packed} f32={f32}", flush=True)
    dsa = dsa_mod()
    s_len = [3000, 2049, 40, 6000]
    lay = synth.decode_layout("pgs", 23, s_len, packed_latent=packed)
    d = synth.inputs_np(lay, parts=("mla",))
    ids = dev(synth.random_ids_np(23, lay))
    pt, pool_rows, row_of = page_layout(s_len, page_size, 24)
    if packed:
        lat = dev(d["latent"])  # [N,576]
        pool = to_pool(lat, pool_rows, row_of)
        latent, kpe, lat_p, kpe_p = lat, lat[:, 512:], pool, pool[:, 512:]
    else:
        latent, kpe = dev(d["latent"]), dev(d["kpe"])
        lat_p, kpe_p = to_pool(latent, pool_rows, row_of), to_pool(kpe, pool_rows, row_of)
    od = torch.float32 if f32 else None
    o, l = dsa.sparse_mla_attn(dev(d["q"]), latent, kpe, dev(lay.kv_off), dev(lay.q_req), ids,
                               synth.ATTN_SCALE, out_dtype=od)
    op, lp = dsa.sparse_mla_attn_paged(dev(d["q"]), lat_p, kpe_p, dev(pt), page_size,
                                       dev(lay.kv_off), dev(lay.q_req), ids, synth.ATTN_SCALE,
                                       out_dtype=od)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16) if not f32 else o, op.view(torch.int16) if not f32 else op)
    assert torch.equal(l, lp)


def test_paged_prefill_chunk_against_oracle():
    print("[paged] prefill-shaped chunk", flush=True)
    dsa = dsa_mod()
    lay = synth.prefill_layout("pgp", 25, 9000, 8900, 100)
    d = synth.inputs_np(lay, parts=("index",))
    keys_np = synth.bf16_bits_from_f32(np.random.default_rng(25).standard_normal((lay.N, 128)))
    pt, pool_rows, row_of = page_layout([9000], 64, 26)
    pool = to_pool(dev(keys_np), pool_rows, row_of)
    ids = dsa.indexer_topk_paged(dev(d["q_idx"]), dev(d["w"]), pool, dev(pt), 64, dev(lay.kv_off),
                                 dev(lay.q_req), dev(lay.q_pos), lay.max_s)
    torch.cuda.synchronize()
    pool_np = pool.view(torch.int16).cpu().numpy().view(np.uint16)
    unpaged = O.unpage_rows(pool_np, pt, 64, lay.kv_off)
    assert np.array_equal(unpaged, keys_np)
    ref = O.indexer_scores(d["q_idx"], d["w"], unpaged, lay.kv_off, lay.q_req, lay.q_pos)
    got = ids.cpu().numpy()
    for t in range(lay.T):
        m = min(len(ref[t]), 2048)
        valid = got[t][got[t] >= 0]
        assert len(valid) == m
        diff = set(valid.tolist()) ^ set(O.topk_ids(ref[t])[:m].tolist())
        assert diff <= set(O.selection_band(ref[t]).tolist()), t


def test_paged_decode_full_size_equals_contiguous():
    """The 64 x 32768 decode batch, keys and latent in 64-position pages of a permuted pool:
    the paged selection and read equal the contiguous ones bit for bit."""
    print("[paged] full-size decode", flush=True)
    dsa = dsa_mod()
    lay = synth.workload("decode_b64_s32768")
    dg = synth.inputs_torch(lay, torch.device(DEV))
    keys = dsa.index_keys_layernorm(dg["raw_keys"], dg["gamma"], dg["beta"], synth.LN_EPS)
    del dg["raw_keys"]
    pt, pool_rows, row_of = page_layout(lay.s_len, 64, 27)
    key_pool = to_pool(keys, pool_rows, row_of)
    lay_args = (dg["kv_off"], dg["q_req"], dg["q_pos"])
    ids = dsa.indexer_topk(dg["q_idx"], dg["w"], keys, *lay_args, lay.max_s)
    ids_p = dsa.indexer_topk_paged(dg["q_idx"], dg["w"], key_pool, dev(pt), 64, *lay_args, lay.max_s)
    del key_pool
    lat_pool = to_pool(dg["latent"], pool_rows, row_of)
    kpe_pool = to_pool(dg["kpe"], pool_rows, row_of)
    o, l = dsa.sparse_mla_attn(dg["q"], dg["latent"], dg["kpe"], dg["kv_off"], dg["q_req"], ids,
                               synth.ATTN_SCALE)
    op, lp = dsa.sparse_mla_attn_paged(dg["q"], lat_pool, kpe_pool, dev(pt), 64, dg["kv_off"],
                                       dg["q_req"], ids_p, synth.ATTN_SCALE)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_p)
    assert torch.equal(o.view(torch.int16), op.view(torch.int16)) and torch.equal(l, lp)
