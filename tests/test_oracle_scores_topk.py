"""Pins for the oracle's indexer scores and top-k selection (CPU only)."""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import dsa_oracle as O


def test_scores_hand_worked_example():
    # two heads of width 2 against four keys, worked by hand:
    # head 0 logits: 1, 2, -3, 0 -> ReLU 1, 2, 0, 0 ; head 1 logits: -1, 1, 0, -3 -> 0, 1, 0, 0
    # s = 0.5 * [1, 2, 0, 0] - 2 * [0, 1, 0, 0] = [0.5, -1, 0, 0]
    q = np.array([[1.0, 2.0], [-1.0, 1.0]])
    w = np.array([0.5, -2.0])
    k = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, -1.0], [2.0, -1.0]])
    assert np.array_equal(O.indexer_scores_one(q, w, k), np.array([0.5, -1.0, 0.0, 0.0]))


def _bits(x):
    return synth.bf16_bits_from_f32(np.asarray(x, np.float32))


def test_scores_integer_inputs_brute_force_exact():
    # small integers and powers of two are exact in bf16; pure-Python exact arithmetic
    g = np.random.default_rng(11)
    s_len = [5, 9]
    lay = synth.Layout("t", 0, s_len, [0, 1, 1], [4, 3, 100])
    h, d = 3, 4
    q = g.integers(-2, 3, size=(lay.T, h, d))
    w = 2.0 ** g.integers(-3, 3, size=(lay.T, h)) * g.choice([-1, 1], size=(lay.T, h))
    keys = g.integers(-2, 3, size=(lay.N, d))
    got = O.indexer_scores(_bits(q), _bits(w), _bits(keys), lay.kv_off, lay.q_req, lay.q_pos)
    for t in range(lay.T):
        b = lay.q_req[t]
        n = min(lay.q_pos[t] + 1, s_len[b])
        assert len(got[t]) == n
        for j in range(n):
            row = keys[lay.kv_off[b] + j]
            exact = sum(Fraction(float(w[t, hh])) * max(0, sum(int(q[t, hh, dd]) * int(row[dd])
                        for dd in range(d))) for hh in range(h))
            assert Fraction(got[t][j]) == exact


def test_scores_one_hot_weights_reduce_to_relu_matmul():
    g = np.random.default_rng(12)
    lay = synth.decode_layout("t", 0, [40])
    q = _bits(g.standard_normal((1, 32, 128)))
    keys = _bits(g.standard_normal((40, 128)))
    for hh in (0, 17, 31):
        w = np.zeros((1, 32), np.float32)
        w[0, hh] = 1.0
        got = O.indexer_scores(q, _bits(w), keys, lay.kv_off, lay.q_req, lay.q_pos)[0]
        ref = torch.relu(torch.from_numpy(O.bf16_to_f64(keys)) @
                         torch.from_numpy(O.bf16_to_f64(q[0, hh]))).numpy()
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-12)


def test_scores_zero_query_and_linearity_in_weights():
    g = np.random.default_rng(13)
    lay = synth.decode_layout("t", 0, [33])
    keys = _bits(g.standard_normal((33, 128)))
    q = _bits(g.standard_normal((1, 32, 128)))
    w1 = _bits(g.standard_normal((1, 32)))
    w2 = _bits(g.standard_normal((1, 32)))
    z = O.indexer_scores(np.zeros_like(q), w1, keys, lay.kv_off, lay.q_req, lay.q_pos)[0]
    assert np.all(z == 0)
    s1 = O.indexer_scores(q, w1, keys, lay.kv_off, lay.q_req, lay.q_pos)[0]
    s2 = O.indexer_scores(q, w2, keys, lay.kv_off, lay.q_req, lay.q_pos)[0]
    w12 = O.bf16_to_f64(w1) + O.bf16_to_f64(w2)
    s12 = O.indexer_scores_one(O.bf16_to_f64(q[0]), w12[0], O.bf16_to_f64(keys))
    assert np.allclose(s1 + s2, s12, rtol=1e-12, atol=1e-10)


@pytest.mark.parametrize("pos,s_b,n", [(0, 10, 1), (4, 10, 5), (9, 10, 10), (50, 10, 10),
                                       (-1, 10, 0), (3, 0, 0)])
def test_admissible_count_is_causal_with_diagonal(pos, s_b, n):
    assert O.admissible_count(pos, s_b) == n


# ---------------------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------------------
def _beats(v, i, j):
    """i ranks above j: numbers above NaN, larger value first, -0 == +0, lower id on ties."""
    a, b = v[i], v[j]
    if np.isnan(a) != np.isnan(b):
        return np.isnan(b)
    if np.isnan(a) or a == b:
        return i < j
    return a > b


def _check_topk_properties(v, ids, k):
    n = len(v)
    valid = ids[ids >= 0]
    assert len(valid) == min(n, k)
    assert np.all(ids[len(valid):] == -1)
    assert np.all(np.diff(valid) > 0) and np.all(valid < n)
    if n > k:
        sel = np.zeros(n, bool)
        sel[valid] = True
        # canonical set: the weakest selected beats the strongest unselected
        ws = min(np.nonzero(sel)[0], key=lambda i: (not np.isnan(v[i]), 0 if np.isnan(v[i])
                                                      else v[i] + 0.0, -i))
        su = max(np.nonzero(~sel)[0], key=lambda i: (not np.isnan(v[i]), 0 if np.isnan(v[i])
                                                       else v[i] + 0.0, -i))
        assert _beats(v, ws, su)


def test_topk_brute_force_tiny():
    g = np.random.default_rng(21)
    for trial in range(300):
        n = int(g.integers(1, 9))
        k = int(g.integers(1, 5))
        v = g.integers(-2, 3, size=n).astype(np.float64)
        v[g.random(n) < 0.1] = np.nan
        v[g.random(n) < 0.1] = -0.0
        got = O.topk_ids(v, k)
        if n <= k:
            assert got[:n].tolist() == list(range(n))
            continue
        winners = [s for s in itertools.combinations(range(n), k)
                   if all(_beats(v, i, j) for i in s for j in range(n) if j not in s)]
        assert len(winners) == 1
        assert got.tolist() == list(winners[0])


@pytest.mark.parametrize("kind", ["gauss", "ints", "two_valued", "all_equal", "zeros_signed",
                                  "special", "sorted_up", "sorted_down", "heavy_tail"])
def test_topk_properties_adversarial(kind):
    rows = synth.score_rows_np(5, kind, 3, 5000)
    for r in rows:
        _check_topk_properties(r, O.topk_ids(r, 2048), 2048)
        assert np.array_equal(O.topk_ids(r, 2048), O.topk_ids(r.astype(np.float64), 2048))


def test_topk_ties_go_to_lowest_positions_and_short_rows():
    assert O.topk_ids(np.full(5000, 1.5), 2048).tolist() == list(range(2048))
    z = np.where(np.arange(3000) % 2 == 0, 0.0, -0.0)
    assert O.topk_ids(z, 2048).tolist() == list(range(2048))
    short = O.topk_ids(np.random.default_rng(0).standard_normal(700), 2048)
    assert short[:700].tolist() == list(range(700)) and np.all(short[700:] == -1)
    assert np.all(O.topk_ids(np.zeros(0), 2048) == -1)


def test_topk_matches_torch_topk_on_distinct_values():
    g = np.random.default_rng(22)
    for n in (2049, 4096, 32768):
        v = g.permutation(n).astype(np.float64) * 0.5 - 1000
        ref = np.sort(torch.topk(torch.from_numpy(v), 2048).indices.numpy())
        assert np.array_equal(O.topk_ids(v, 2048), ref)


def test_selection_band_contains_kth():
    g = np.random.default_rng(23)
    v = g.standard_normal(10000)
    band = O.selection_band(v, 2048, 1e-3)
    theta = O.kth_score(v, 2048)
    assert theta == np.sort(v)[::-1][2047]
    assert np.any(v[band] == theta)
