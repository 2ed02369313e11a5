"""Pins of the oracle's tolerance helpers: the row scale, the selection band and the three
error-magnitude helpers that size the parity bars of the GPU tests.

The set tolerance follows the reading of "positions within 1e-3 relative of the k-th score"
for the index I_t of the page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere Historie",
section "Die Mathematik der Sparse Attention und ihrer fehlenden Masse" (I_t holds the up to
2048 highest-scoring positions): a GPU selection may differ from the oracle's only at
positions j with |s_j - theta| <= rel * max(|theta|, r_t), theta the k-th score, r_t the
row's root-mean-square score.  Every expected value below is worked out by hand in the
comments; a helper that is off by a factor of two, drops a term, or reduces over the wrong
axis fails at least one check.
"""
import math

import numpy as np

from oracle import dsa_oracle as O


def bits(x):
    """Exact bf16 patterns of values that bf16 represents exactly."""
    x = np.asarray(x, dtype=np.float32)
    b = x.view(np.uint32) >> np.uint32(16)
    assert np.array_equal((b.astype(np.uint32) << np.uint32(16)).view(np.float32), x)
    return b.astype(np.uint16)


def bf16_round(x):
    """Values truncated to bf16 (exactly representable inputs for bits())."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


# ---------------------------------------------------------------------------------------
# row scale: root mean square of the row
# ---------------------------------------------------------------------------------------
def test_row_scale_closed_forms():
    assert O.row_scale([3.0, 4.0]) == math.sqrt(12.5)          # (9 + 16) / 2
    assert O.row_scale([-2.5] * 7) == 2.5                       # constant row: |c|
    assert O.row_scale([1.0, -1.0] * 50) == 1.0                 # signs cancel in a mean, not here
    assert O.row_scale([2.0] * 4 + [0.0] * 12) == 1.0           # 16 / 16
    assert O.row_scale([6.0] + [0.0] * 8) == 2.0                # 36 / 9
    assert O.row_scale([]) == 0.0
    # mean over the row's length (not a sum, not a fixed length): appending zeros shrinks it
    assert O.row_scale([2.0] * 4) == 2.0 and O.row_scale([2.0] * 4 + [0.0] * 4) == math.sqrt(2.0)


# ---------------------------------------------------------------------------------------
# selection band
# ---------------------------------------------------------------------------------------
def test_selection_band_relative_to_theta():
    """k = 4, theta = 8.0 (the fourth largest of 10, 9, 8.006, 8.0, ...), and with 100 zeros
    the row scale is about 2.03 < 8, so the half-width is 1e-3 * 8 = 0.008:
    8.006 (0.006 above) and 7.993 (0.007 below) are inside, 7.991 (0.009) and 8.0085 are not
    (8.0085 would be the third score; it is absent here).  A band twice as wide would take
    7.991, one half as wide would lose 7.993 and 8.006."""
    row = np.array([10.0, 9.0, 8.006, 8.0, 7.993, 7.991] + [0.0] * 100)
    assert O.kth_score(row, 4) == 8.0
    assert 2.0 < O.row_scale(row) < 2.1
    assert O.selection_band(row, 4, 1e-3).tolist() == [2, 3, 4]
    assert O.selection_band(row, 4, 2e-3).tolist() == [2, 3, 4, 5]  # 0.016 half-width
    assert O.selection_band(row, 4, 0.5e-3).tolist() == [3]          # 0.004 half-width


def test_selection_band_floor_is_the_row_scale():
    """theta near zero (signed head weights cancel): the half-width is 1e-3 * r_t.  Row of
    +-4 (four each) and six small values; r_t = sqrt((8 * 16 + small) / 14) ~ 3.0237, so the
    half-width is ~0.0030237.  k = 6 picks 4, 4, 4, 4, 0.0065, 0.005: theta = 0.005.
    Inside: 0.0065 (0.0015 above), 0.005, 0.0025 (0.0025 below), 0.0021 (0.0029 below).
    Outside: 0.0019 (0.0031 below), 0.0 (0.005 below) and -4.  With |theta| as the only scale
    the band would be {theta} alone; with twice the floor (0.00605) 0.0019 and 0.0 would join;
    with half of it 0.0025 and 0.0021 would drop out."""
    small = [0.0065, 0.005, 0.0025, 0.0021, 0.0019, 0.0]
    row = np.array([4.0, -4.0] * 4 + small)
    r = O.row_scale(row)
    assert abs(r - 3.0237) < 1e-4
    assert O.kth_score(row, 6) == 0.005
    assert O.selection_band(row, 6, 1e-3).tolist() == [8, 9, 10, 11]
    assert O.selection_band(row, 6, 2e-3).tolist() == [8, 9, 10, 11, 12, 13]
    assert O.selection_band(row, 6, 0.5e-3).tolist() == [8, 9]


def test_selection_band_ties_and_short_rows():
    # every position equal to theta is in the band, whichever of them the top-k kept
    row = np.array([5.0, 1.0, 1.0, 1.0, 1.0, -3.0])
    assert O.kth_score(row, 2) == 1.0
    assert O.selection_band(row, 2, 1e-3).tolist() == [1, 2, 3, 4]
    # a row with no more than k positions selects all of them: nothing is uncertain
    assert O.selection_band(np.arange(5.0), 5).size == 0
    assert O.selection_band(np.arange(2048.0)).size == 0
    # 0..2048: theta = 1, r_t = sqrt(2048 * 4097 / 6) ~ 1182.6, half-width ~ 1.18
    assert O.selection_band(np.arange(2049.0)).tolist() == [0, 1, 2]


# ---------------------------------------------------------------------------------------
# error scales and magnitudes: hand-worked rows; equal to the value when every term is
# non-negative (the magnitudes)
# ---------------------------------------------------------------------------------------
def test_layernorm_error_scale():
    """The fp32 error scale |gamma| A/sigma + |x_hat gamma| (1 + A/sigma) + |beta| (A: the
    row's mean absolute value), on rows worked by hand, eps = 0 unless stated:
    - a = +-1 alternating: mean 0, sigma 1, A 1, x_hat = a.  gamma 2, beta -3:
      2 * 1 + 2 * 2 + 3 = 9 everywhere;
    - 10 a + 7 (values 17, -3): mean 7, sigma 10, A 10, so A/sigma = 1 again and x_hat = a: 9
      (a reduction over the wrong axis would not give it);
    - a + 9 (values 10, 8): mean 9, sigma 1, A 9: 2 * 9 + 2 * 10 + 3 = 41, and -(a + 9) the
      same (the signed mean, -9, in place of A would not give it; |mean| in place of A fails
      on row a, whose mean is 0);
    - a with eps = 3: sigma 2, A/sigma 1/2, x_hat = a/2: 2 * 0.5 + 1 * 1.5 + 3 = 5.5;
    - per-element gamma_d, beta_d on a: |gamma_d| + 2 |gamma_d| + |beta_d|."""
    a = np.tile([1.0, -1.0], 64).astype(np.float32)
    raw = np.stack([a, 10 * a + 7, a + 9, -(a + 9)]).astype(np.float32)
    gamma = np.full(128, 2.0, np.float32)
    beta = np.full(128, -3.0, np.float32)
    want = np.stack([np.full(128, 9.0), np.full(128, 9.0), np.full(128, 41.0), np.full(128, 41.0)])
    assert np.array_equal(O.layernorm_error_scale(raw, gamma, beta, 0.0), want)
    assert np.array_equal(O.layernorm_error_scale(raw[:1], gamma, beta, 3.0), np.full((1, 128), 5.5))
    gd = np.arange(128, dtype=np.float32) - 64
    bd = np.linspace(-1, 1, 128).astype(np.float32)
    want_d = 3 * np.abs(gd.astype(np.float64)) + np.abs(bd.astype(np.float64))
    assert np.array_equal(O.layernorm_error_scale(raw[:1], gd, bd, 0.0)[0], want_d)
    # float64 rows (an exact projection) are taken unrounded: 1 + 2^-30 is not an fp32 value
    x64 = np.stack([a.astype(np.float64) + 2.0 ** -30 * np.arange(128)])
    assert O.layernorm_error_scale(x64, gamma, beta, 0.0).dtype == np.float64
    assert not np.array_equal(O.layernorm_error_scale(x64, gamma, beta, 0.0),
                              O.layernorm_error_scale(x64.astype(np.float32), gamma, beta, 0.0))


def test_value_gate_magnitude():
    """Head h's W_UV has (h + 1) at latent dims 0 and 1 of every value coordinate, zero
    elsewhere; o[t, h] = (2, -3, 0, ...); gate logits 0 (sigmoid 1/2).  The value is
    (h + 1)(2 - 3) / 2 = -(h + 1) / 2, the magnitude (h + 1)(2 + 3) / 2 = 5 (h + 1) / 2.
    A head index taken from the wrong operand, a missing sigmoid or |sum| instead of the sum
    of |terms| all change these numbers."""
    t_count, h_count = 2, 96
    w = np.zeros((h_count, 128, 512), np.float32)
    w[:, :, :2] = (np.arange(h_count, dtype=np.float32) + 1)[:, None, None]
    o = np.zeros((t_count, h_count, 512), np.float32)
    o[:, :, 0], o[:, :, 1] = 2.0, -3.0
    gate = np.zeros((t_count, h_count, 128), np.float32)
    hp1 = (np.arange(h_count) + 1.0)[None, :, None]
    val = O.value_gate(bits(o), bits(w), bits(gate))
    mag = O.value_gate_magnitude(bits(o), bits(w), bits(gate))
    assert np.array_equal(val, np.broadcast_to(-hp1 / 2, val.shape))
    assert np.array_equal(mag, np.broadcast_to(5 * hp1 / 2, mag.shape))
    # closed gate (logit -2^100): value and magnitude both vanish; open gate: sigmoid 1
    gate[1] = -(2.0 ** 100)
    gate[0, :, 0] = 2.0 ** 100
    mag = O.value_gate_magnitude(bits(o), bits(w), bits(gate))
    assert np.all(mag[1] == 0) and np.array_equal(mag[0, :, 0], 5 * hp1[0, :, 0])
    # non-negative terms: the magnitude is the value itself
    g = np.random.default_rng(5)
    ob = bits(bf16_round(np.abs(g.standard_normal((3, 96, 512)))))
    wb = bits(bf16_round(np.abs(g.standard_normal((96, 128, 512)))))
    gb = bits(bf16_round(g.standard_normal((3, 96, 128))))
    assert np.allclose(O.value_gate_magnitude(ob, wb, gb), O.value_gate(ob, wb, gb),
                       rtol=1e-14, atol=0)


def test_linear_magnitude():
    """x = [[2, -3], [-1, 4]], weight rows [1, 1], [1, -1], [-2, 0] ([out, in]):
    x W^T = [[-1, 5, -4], [3, -5, 2]]; sum |x w| = [[5, 5, 4], [5, 5, 2]]."""
    x = bits([[2.0, -3.0], [-1.0, 4.0]])
    w = bits([[1.0, 1.0], [1.0, -1.0], [-2.0, 0.0]])
    assert np.array_equal(O.linear(x, w), [[-1.0, 5.0, -4.0], [3.0, -5.0, 2.0]])
    assert np.array_equal(O.linear_magnitude(x, w), [[5.0, 5.0, 4.0], [5.0, 5.0, 2.0]])
    # float64 activations are used as given (no bf16 rounding of an exact projection)
    assert np.array_equal(O.linear_magnitude(np.array([[0.1, -0.2]]), w),
                          [[0.1 + 0.2, 0.1 + 0.2, 0.2]])
    # non-negative terms: the magnitude is the value itself
    g = np.random.default_rng(6)
    xb = bits(bf16_round(np.abs(g.standard_normal((4, 300)))))
    wb = bits(bf16_round(np.abs(g.standard_normal((7, 300)))))
    assert np.allclose(O.linear_magnitude(xb, wb), O.linear(xb, wb), rtol=1e-14, atol=0)
