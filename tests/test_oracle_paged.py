"""Pins of the oracle's paged page-pool layout helper (page "Kimi K3.1 Pro: Sparse-Zugriffe,
keine kleinere Historie", section "Warum Top-2048 keinen 2048-Token-Cache bedeutet": page
allocation changes the physical cache, not the logical positions)."""
import numpy as np

from oracle import dsa_oracle as O


def test_identity_table_is_the_contiguous_cache():
    pool = np.arange(3 * 64 * 2).reshape(3 * 64, 2)
    kv_off = np.array([0, 64, 150], np.int64)  # lengths 64 and 86: pages 0 | 1, 2
    pt = np.array([[0, 0], [1, 2]], np.int32)
    assert np.array_equal(O.unpage_rows(pool, pt, 64, kv_off), pool[:150])


def test_permuted_pages_gather_by_hand():
    g = np.random.default_rng(1)
    P = 64
    lens = [130, 1, 64, 300]
    pages = [-(-n // P) for n in lens]
    perm = g.permutation(sum(pages) + 3)  # spare pages in the pool
    pt = np.zeros((4, max(pages)), np.int32)
    k = 0
    for b, n in enumerate(pages):
        pt[b, :n] = perm[k:k + n]
        k += n
    pool = g.standard_normal((len(perm) * P, 5))
    kv_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    got = O.unpage_rows(pool, pt, P, kv_off)
    for b, n in enumerate(lens):
        for p in (0, n // 2, n - 1):
            assert np.array_equal(got[kv_off[b] + p], pool[pt[b, p // P] * P + p % P])


def test_page_then_unpage_round_trips():
    """Scattering a contiguous cache into permuted pages and gathering it back is the
    identity (the GPU tests build their pools this way)."""
    g = np.random.default_rng(2)
    P = 128
    lens = [1000, 5, 129]
    kv_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    contig = g.integers(0, 1 << 16, size=(sum(lens), 3))
    pages = [-(-n // P) for n in lens]
    perm = g.permutation(sum(pages))
    pt = np.zeros((3, max(pages)), np.int32)
    pool = np.zeros((len(perm) * P, 3), contig.dtype)
    k = 0
    for b, n in enumerate(lens):
        pt[b, :pages[b]] = perm[k:k + pages[b]]
        k += pages[b]
        p = np.arange(n)
        pool[pt[b, p // P] * P + p % P] = contig[kv_off[b]:kv_off[b] + n]
    assert np.array_equal(O.unpage_rows(pool, pt, P, kv_off), contig)
