"""GPU parity of the paged page-pool layout (dsa_indexer_topk_paged, dsa_sparse_mla_attn_paged).

The paged entry points run the same arithmetic as the contiguous ones on the same logical
cache, so their results must be identical bit for bit (decode layouts: both use the streaming
scoring kernel).  Every paged result is also checked against the oracle over the cache
unpaged from the pool (the pool read back from the GPU and gathered through the page table
by the oracle's own routine): selected sets up to the 1e-3 band of the k-th score, and the
read within 1e-2 (+ half a bf16 ulp for a bf16 output) of the oracle's read of the same IDs.
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


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_selection_vs_oracle(got, ref):
    """got [T,2048] GPU IDs, ref: oracle score rows."""
    for t in range(len(ref)):
        m = min(len(ref[t]), 2048)
        valid = got[t][got[t] >= 0]
        assert len(valid) == m and np.all(got[t][m:] == -1) and np.all(np.diff(valid) > 0), t
        diff = set(valid.tolist()) ^ set(O.topk_ids(ref[t])[:m].tolist())
        assert diff <= set(O.selection_band(ref[t]).tolist()), f"query {t}"


def check_read_vs_oracle(q_bits, lat_c, kpe_c, kv_off, q_req, ids, got_o, got_l, f32):
    """The paged read against the oracle's read of the same IDs over the unpaged rows."""
    ref_o, ref_l = O.sparse_mla(q_bits, lat_c, kpe_c, kv_off, q_req, ids, synth.ATTN_SCALE)
    half_ulp = 0.0 if f32 else np.where(ref_o != 0, np.ldexp(1.0, np.frexp(np.abs(ref_o))[1] - 9), 0.0)
    assert np.all(np.abs(got_o - ref_o) <= 1e-2 + half_ulp), f"max err {np.abs(got_o - ref_o).max()}"
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(got_l))
    assert np.all(np.abs(got_l[fin] - ref_l[fin]) <= 1e-3 * np.maximum(1, np.abs(ref_l[fin])))


def to_pool(contig, pool_rows, row_of):
    pool = torch.zeros((pool_rows,) + tuple(contig.shape[1:]), dtype=contig.dtype, device=DEV)
    pool[torch.as_tensor(row_of, device=DEV)] = contig
    return pool


DECODE = [[1, 63, 64, 65, 2047, 2049, 4096, 5000], [70000, 3, 33000]]


# pages smaller than a scoring block's chunk of keys, and one (4096) at least as large
@pytest.mark.parametrize("page_size", [64, 256, 4096])
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
    unpaged = O.unpage_rows(host_bits(pool), pt, page_size, lay.kv_off)
    ref = O.indexer_scores(d["q_idx"], d["w"], unpaged, lay.kv_off, lay.q_req, lay.q_pos)
    check_selection_vs_oracle(ids_p.cpu().numpy(), ref)


@pytest.mark.parametrize("page_size,packed,f32", [(64, False, False), (128, True, True),
                                                  (64, True, False), (4096, False, True)])
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
    lat_c = O.unpage_rows(host_bits(lat_p), pt, page_size, lay.kv_off)
    kpe_c = O.unpage_rows(host_bits(kpe_p), pt, page_size, lay.kv_off)
    check_read_vs_oracle(d["q"], lat_c, kpe_c, lay.kv_off, lay.q_req, ids.cpu().numpy(),
                         op.float().cpu().numpy(), lp.cpu().numpy(), f32)


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
    the paged selection and read equal the contiguous ones bit for bit, and four sampled
    queries match the oracle over the rows gathered from the pools."""
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
    lat_pool = to_pool(dg["latent"], pool_rows, row_of)
    kpe_pool = to_pool(dg["kpe"], pool_rows, row_of)
    o, l = dsa.sparse_mla_attn(dg["q"], dg["latent"], dg["kpe"], dg["kv_off"], dg["q_req"], ids,
                               synth.ATTN_SCALE)
    op, lp = dsa.sparse_mla_attn_paged(dg["q"], lat_pool, kpe_pool, dev(pt), 64, dg["kv_off"],
                                       dg["q_req"], ids_p, synth.ATTN_SCALE)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_p)
    assert torch.equal(o.view(torch.int16), op.view(torch.int16)) and torch.equal(l, lp)
    # sampled queries against the oracle over rows gathered from the pools by the oracle
    got = ids_p.cpu().numpy()
    for t in (0, 21, 42, 63):
        s_b = int(lay.s_len[t])
        one_off = np.array([0, s_b], np.int64)
        n_pages = -(-s_b // 64)
        # the request's pages, copied out of each pool in page-table order, form a small pool
        # whose page table is 0 .. n_pages - 1; the oracle unpages that
        phys = torch.as_tensor(pt[t, :n_pages].astype(np.int64) * 64, device=DEV)
        idx = (phys[:, None] + torch.arange(64, device=DEV)[None, :]).reshape(-1)
        pt_local = np.arange(n_pages, dtype=np.int32)[None, :]

        def unpaged(pool):
            return O.unpage_rows(host_bits(pool[idx]), pt_local, 64, one_off)

        ref = O.indexer_scores(synth.to_bits_np(dg["q_idx"][t:t + 1]),
                               synth.to_bits_np(dg["w"][t:t + 1]), unpaged(key_pool), one_off,
                               np.zeros(1, np.int32), np.array([s_b - 1], np.int32))
        check_selection_vs_oracle(got[t:t + 1], ref)
        check_read_vs_oracle(synth.to_bits_np(dg["q"][t:t + 1]), unpaged(lat_pool),
                             unpaged(kpe_pool), one_off, np.zeros(1, np.int32), got[t:t + 1],
                             op[t:t + 1].float().cpu().numpy(), lp[t:t + 1].cpu().numpy(), False)
