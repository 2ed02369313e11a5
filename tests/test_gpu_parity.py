"""GPU parity of every stage against the CPU oracle (same seeded inputs on both sides).

Tolerances: LayerNorm <= 1 bf16 ulp (or, where its two terms cancel, 2^-16 of their size);
indexer scores |s - s_ref| <= 1e-3 * max(|s_ref|, r_t)
(r_t: the row's RMS score); top-k bit-exact on identical fp32 arrays; selected sets equal
up to positions within the 1e-3 band of the k-th score; sparse read max-abs 1e-2 on out (fp32
output; a bf16 output adds half a bf16 ulp of the reference for its own rounding) and
1e-3 * max(1, |lse|) on lse, given the same ID set.
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


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ln_tolerance_ok(got_bits, raw, gamma, beta, eps):
    """LayerNorm parity: within 1 bf16 ulp of the oracle, or -- where the rounding of a result
    near a bf16 boundary, or cancellation in x_hat*gamma + beta, makes the fp32 evaluation's
    error more than an ulp -- within 16 fp32 unit roundoffs (2^-20) of the exact value's
    error scale |gamma| A/sigma + |x_hat gamma| (1 + A/sigma) + |beta|: a first-order bound of
    an fp32 evaluation with a mean summed in a tree of depth 7 needs about 7 + a few units
    per term.  Returns the fraction of elements that needed the second clause."""
    ref_bits = O.layernorm_keys_bf16(raw, gamma, beta, eps)
    one_ulp = bf16_ulp_dist(got_bits, ref_bits) <= 1
    exact = O.layernorm_keys(raw, gamma, beta, eps)
    scale = O.layernorm_error_scale(raw, gamma, beta, eps)
    close = np.abs(O.bf16_to_f64(got_bits) - exact) <= 2.0 ** -20 * scale
    assert np.all(one_ulp | close)
    return float((~one_ulp).mean())


def bf16_ulp_dist(a, b):
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x)
    return np.abs(ordered(a) - ordered(b))


# ---------------------------------------------------------------------------------------
# stage 1
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 3, 1000, 16391])
def test_layernorm_parity(n):
    print(f"[ln] n={n}", flush=True)
    g = np.random.default_rng(100 + n)
    raw = (g.standard_normal((n, 128)) * 2 + 0.5).astype(np.float32)
    raw[0] = 5.5  # constant row -> exactly beta
    if n > 2:
        raw[1] = np.tile([3.0, -3.0], 64)
    if n > 100:  # rows whose mean dwarfs their spread (the mean's rounding shows in x - mu)
        raw[10:40] += 10.0
        raw[40:70] += 1000.0
        raw[70:100] -= 300.0
    gamma = (1 + 0.3 * g.standard_normal(128)).astype(np.float32)
    beta = (0.3 * g.standard_normal(128)).astype(np.float32)
    keys = dsa_mod().index_keys_layernorm(dev(raw), dev(gamma), dev(beta), 1e-6)
    torch.cuda.synchronize()
    got = host_bits(keys)
    ref = O.layernorm_keys_bf16(raw, gamma, beta, 1e-6)
    assert ln_tolerance_ok(got, raw, gamma, beta, 1e-6) < 1e-3
    assert (bf16_ulp_dist(got, ref) > 0).mean() < 0.01
    assert np.array_equal(got[0], O.f64_to_bf16(beta.astype(np.float64)))


# ---------------------------------------------------------------------------------------
# stage 2
# ---------------------------------------------------------------------------------------
def run_scores(lay, d, keys_bits):
    dsa = dsa_mod()
    s = dsa.indexer_scores(dev(d["q_idx"]), dev(d["w"]), dev(keys_bits), dev(lay.kv_off),
                           dev(lay.q_req), dev(lay.q_pos), lay.max_s)
    torch.cuda.synchronize()
    return s.cpu().numpy()


def check_scores(lay, d, keys_bits, got):
    ref = O.indexer_scores(d["q_idx"], d["w"], keys_bits, lay.kv_off, lay.q_req, lay.q_pos)
    for t in range(lay.T):
        n = len(ref[t])
        r = O.row_scale(ref[t])
        err = np.abs(got[t, :n] - ref[t])
        assert np.all(err <= 1e-3 * np.maximum(np.abs(ref[t]), r) + 1e-30), \
            f"query {t}: max rel err {(err / np.maximum(np.abs(ref[t]), r)).max()}"
        assert np.all(np.isnan(got[t, n:])), f"query {t}: wrote past n_t"
    return ref


def idx_inputs(lay, seed):
    d = synth.inputs_np(lay, parts=("index",))
    g = np.random.default_rng(seed)
    keys = synth.bf16_bits_from_f32(g.standard_normal((lay.N, 128)))
    return d, keys


DECODE_LAYOUTS = [
    ("decode_ragged", [1, 5, 2047, 2048, 2049, 4096, 5000]),
    ("decode_long", [70000, 3]),
]


@pytest.mark.parametrize("name,s_len", DECODE_LAYOUTS)
def test_scores_decode_kernel(name, s_len):
    print(f"[scores decode] {name}", flush=True)
    lay = synth.decode_layout(name, 11, s_len)
    lay.q_pos[-1] = max(0, s_len[-1] // 2)  # one query cut by causality inside its cache
    d, keys = idx_inputs(lay, 11)
    check_scores(lay, d, keys, run_scores(lay, d, keys))


def test_scores_decode_kernel_unaligned_rows():
    """Score rows that do not start on 16-byte boundaries (an odd row stride, one float into
    the buffer) are stored element by element: every admissible score is right, and nothing
    is written past n_t, before the row or after it."""
    print("[scores decode] unaligned rows", flush=True)
    dsa = dsa_mod()
    lay = synth.decode_layout("unal", 12, [3, 2049, 5001, 4096])
    lay.q_pos[-1] = 3001
    d, keys = idx_inputs(lay, 12)
    buf = torch.full((lay.T, lay.max_s + 2), float("nan"), dtype=torch.float32, device=DEV)
    view = buf[:, 1:1 + lay.max_s]
    assert view.data_ptr() % 16 != 0 and view.stride(0) % 4 != 0
    dsa.indexer_scores(dev(d["q_idx"]), dev(d["w"]), dev(keys), dev(lay.kv_off),
                       dev(lay.q_req), dev(lay.q_pos), lay.max_s, scores=view)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    check_scores(lay, d, keys, b[:, 1:1 + lay.max_s])
    assert np.all(np.isnan(b[:, 0])) and np.all(np.isnan(b[:, -1]))


def test_scores_prefill_kernel_one_request():
    print("[scores prefill] one request", flush=True)
    s = 3000
    pos = np.concatenate([np.arange(2800, 3000), [0, 1, 31, 32, 33, 2047]]).astype(np.int32)
    lay = synth.Layout("prefill", 12, [s], np.zeros(len(pos), np.int32), pos)
    d, keys = idx_inputs(lay, 12)
    check_scores(lay, d, keys, run_scores(lay, d, keys))


def test_scores_prefill_kernel_mixed_requests():
    print("[scores prefill] mixed requests", flush=True)
    req = np.array([0] * 10 + [1] * 30 + [0] * 25, np.int32)
    pos = np.concatenate([np.arange(10) + 500, np.arange(30) * 40, np.arange(25) + 990]).astype(np.int32)
    lay = synth.Layout("mixed", 13, [1000, 1300], req, pos)
    assert lay.T >= 8 * lay.B
    d, keys = idx_inputs(lay, 13)
    check_scores(lay, d, keys, run_scores(lay, d, keys))


@pytest.mark.parametrize("prefill", [False, True])
def test_scores_integer_inputs_bit_exact(prefill):
    print(f"[scores exact] prefill={prefill}", flush=True)
    g = np.random.default_rng(14)
    if prefill:
        lay = synth.prefill_layout("p", 14, 700, 600, 40)
    else:
        lay = synth.decode_layout("d", 14, [300, 4100])
    q = synth.bf16_bits_from_f32(g.integers(-2, 3, size=(lay.T, 32, 128)))
    w = synth.bf16_bits_from_f32(2.0 ** g.integers(-4, 2, size=(lay.T, 32)) *
                                 g.choice([-1, 1], size=(lay.T, 32)))
    keys = synth.bf16_bits_from_f32(g.integers(-2, 3, size=(lay.N, 128)))
    d = {"q_idx": q, "w": w}
    got = run_scores(lay, d, keys)
    ref = O.indexer_scores(q, w, keys, lay.kv_off, lay.q_req, lay.q_pos)
    for t in range(lay.T):
        assert np.array_equal(got[t, :len(ref[t])], ref[t].astype(np.float32))


# ---------------------------------------------------------------------------------------
# stage 3
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["gauss", "ints", "two_valued", "all_equal", "zeros_signed",
                                  "special", "sorted_up", "sorted_down", "heavy_tail"])
def test_topk_bit_exact_on_identical_scores(kind):
    print(f"[topk] {kind}", flush=True)
    dsa = dsa_mod()
    ld = 9000
    rows = synth.score_rows_np(20, kind, 6, ld)
    n_valid = np.array([1, 2048, 2049, 4097, 8192, 9000], np.int32)
    ids = dsa.topk(dev(rows), dev(n_valid), max_n=ld)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for t in range(len(rows)):
        ref = O.topk_ids(rows[t, :n_valid[t]])
        assert np.array_equal(got[t], ref), f"row {t} (n={n_valid[t]})"


@pytest.mark.parametrize("n,kind", [(32768, "gauss"), (32768, "special"), (65536, "gauss"),
                                    (65536, "ints"), (65536, "special"), (65536, "coarse"),
                                    (40000, "coarse"), (40001, "gauss"), (33000, "coarse"),
                                    (50000, "heavy_tail"), (70001, "gauss"),
                                    (70001, "two_valued"), (200000, "special"),
                                    (1_000_001, "coarse"), (1_100_000, "gauss")])
def test_topk_bit_exact_long_rows(n, kind):
    print(f"[topk long] n={n} {kind}", flush=True)
    dsa = dsa_mod()
    rows = synth.score_rows_np(21, kind, 2, n)
    n_valid = np.array([n, n - 17], np.int32)
    ids = dsa.topk(dev(rows), dev(n_valid), max_n=n)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for t in range(2):
        assert np.array_equal(got[t], O.topk_ids(rows[t, :n_valid[t]])), f"row {t}"


# Row lengths around every switch of the selection of rows of up to 2^20 elements: segments of
# 64, 32, 16 and 8 positions, rows of at most 65536 (register path), short and empty rows.
SEGMENT_ROW_LENGTHS = [1 << 20, (1 << 20) - 5, 262_145, 262_144, 200_001, 131_073, 131_072,
                       65_537, 65_536, 2_049, 0]


@pytest.mark.parametrize("kind", ["gauss", "coarse", "special", "heavy_tail", "ints",
                                  "sorted_up", "sorted_down", "zeros_signed"])
def test_topk_segment_maxima_rows_bit_exact(kind):
    """Rows of 65537 .. 2^20 elements select from the elements at or above a threshold taken
    from segment maxima.  Gaussian, coarse and heavy-tailed rows take that path at every
    length (coarse ones with ties at the k-th key); sorted rows gather too many candidates and
    fall back to the streamed selection, and integer, special and signed-zero rows take either
    path depending on their length (flat maxima fall back).  Every row must equal the oracle."""
    print(f"[topk segments] {kind}", flush=True)
    dsa = dsa_mod()
    ld = 1 << 20
    n_valid = np.array(SEGMENT_ROW_LENGTHS, np.int32)
    rows = synth.score_rows_np(41, kind, len(n_valid), ld)
    ids = dsa.topk(dev(rows), dev(n_valid), max_n=ld)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for t in range(len(rows)):
        assert np.array_equal(got[t], O.topk_ids(rows[t, :n_valid[t]])), f"row {t} (n={n_valid[t]})"


@pytest.mark.parametrize("max_n,kind", [(3000, "gauss"), (6000, "coarse"), (12000, "special"),
                                        (30000, "gauss"), (30000, "two_valued"),
                                        (50000, "heavy_tail"), (1_100_001, "gauss")])
def test_topk_unaligned_rows_bit_exact(max_n, kind):
    """Score rows that do not start on 16-byte boundaries (a view one float into its buffer)
    take the element-wise load path of every row class: 4 .. 64 elements per thread and rows
    streamed per pass beyond 2^20.  Ragged lengths end inside a group of four."""
    print(f"[topk unaligned] max_n={max_n} {kind}", flush=True)
    dsa = dsa_mod()
    rows = synth.score_rows_np(43, kind, 3, max_n + 1)
    n_valid = np.array([max_n, max_n - 3, 2049 + max_n % 7], np.int32)
    full = dev(rows)
    view = full[:, 1:]
    assert view.data_ptr() % 16 != 0
    ids = dsa.topk(view, dev(n_valid), max_n=max_n)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for t in range(3):
        ref = O.topk_ids(rows[t, 1:1 + n_valid[t]])
        assert np.array_equal(got[t], ref), f"row {t} (n={n_valid[t]})"


def test_topk_persistent_rows_bit_exact():
    """More rows than CUs, each of up to 40000 elements: the selection runs one persistent
    block per CU that prefetches its next row into LDS while selecting the current one.  Row
    lengths of every class (empty, short, ragged, full) follow one another inside a block."""
    print("[topk persistent] 600 rows", flush=True)
    dsa = dsa_mod()
    t_count, ld = 600, 40000
    g = np.random.default_rng(31)
    rows = np.concatenate([synth.score_rows_np(31, "gauss", t_count // 2, ld),
                           synth.score_rows_np(32, "coarse", t_count - t_count // 2, ld)])
    rows = rows[g.permutation(t_count)]
    n_valid = g.integers(32769, ld + 1, size=t_count).astype(np.int32)
    n_valid[::7] = g.integers(0, 2049, size=len(n_valid[::7]))
    n_valid[3::11] = ld
    n_valid[5::13] = g.integers(2049, 32769, size=len(n_valid[5::13]))
    ids = dsa.topk(dev(rows), dev(n_valid), max_n=ld)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for t in range(t_count):
        assert np.array_equal(got[t], O.topk_ids(rows[t, :n_valid[t]])), f"row {t} (n={n_valid[t]})"


# Row lengths that end exactly on, or one position around, the span of one wave of a block
# (64 E positions: 2048 for rows of up to 32768, 4096 for rows of up to 65536).  A wave whose
# span lies wholly below the row length counts its level-0 bins without the per-element check
# for absent positions; the wave holding the row's end keeps it.
WAVE_EDGE_LENGTHS = {32768: [2049, 4095, 4096, 4097, 30719, 30720, 30721, 32767, 32768],
                     65536: [32769, 36863, 36864, 36865, 61439, 61440, 61441, 65535, 65536]}


@pytest.mark.parametrize("max_n", [32768, 65536])
@pytest.mark.parametrize("kind", ["gauss", "coarse", "special"])
def test_topk_rows_ending_at_wave_spans_bit_exact(max_n, kind):
    """Every row equals the oracle.  At 65536 the 300 rows run the persistent grid (more rows
    than CUs), so each length also follows other lengths inside a block."""
    print(f"[topk wave edges] max_n={max_n} {kind}", flush=True)
    dsa = dsa_mod()
    lengths = WAVE_EDGE_LENGTHS[max_n]
    t_count = len(lengths) if max_n == 32768 else 300
    rows = synth.score_rows_np(47, kind, t_count, max_n)
    n_valid = np.array([lengths[t % len(lengths)] for t in range(t_count)], np.int32)
    ids = dsa.topk(dev(rows), dev(n_valid), max_n=max_n)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for t in range(t_count):
        assert np.array_equal(got[t], O.topk_ids(rows[t, :n_valid[t]])), f"row {t} (n={n_valid[t]})"


def check_selection(lay, ids, ref_scores):
    for t in range(lay.T):
        row = ids[t]
        n = len(ref_scores[t])
        m = min(n, 2048)
        valid = row[:m]
        assert np.all(row[m:] == -1), f"query {t}: -1 only as suffix"
        assert np.all(np.diff(valid) > 0) and np.all((valid >= 0) & (valid < n))
        refset = set(O.topk_ids(ref_scores[t])[:m].tolist())
        band = set(O.selection_band(ref_scores[t]).tolist())
        diff = set(valid.tolist()) ^ refset
        assert diff <= band, f"query {t}: {len(diff)} positions differ outside the band"


@pytest.mark.parametrize("name,s_len", DECODE_LAYOUTS)
def test_indexer_topk_matches_oracle_and_standalone_topk(name, s_len):
    print(f"[indexer_topk] {name}", flush=True)
    dsa = dsa_mod()
    lay = synth.decode_layout(name, 15, s_len)
    d, keys = idx_inputs(lay, 15)
    args = (dev(d["q_idx"]), dev(d["w"]), dev(keys), dev(lay.kv_off), dev(lay.q_req),
            dev(lay.q_pos))
    ids = dsa.indexer_topk(*args, lay.max_s)
    scores = dsa.indexer_scores(*args, lay.max_s)
    n_valid = np.minimum(lay.q_pos + 1, lay.s_len[lay.q_req]).astype(np.int32)
    ids2 = dsa.topk(scores, dev(n_valid), max_n=lay.max_s)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    ref = O.indexer_scores(d["q_idx"], d["w"], keys, lay.kv_off, lay.q_req, lay.q_pos)
    check_selection(lay, ids.cpu().numpy(), ref)


def test_decode_several_queries_per_request():
    """A decode batch with three queries per request at its last three positions (fewer than
    eight per request on average, so the per-query scoring kernel runs; the queries of one
    request see prefixes one position apart).  Scores, the fused selection (equal to the
    standalone one, and to the oracle's set up to the band) and the read of the selected rows
    all match the oracle; one request is shorter than 2048 positions."""
    print("[decode] three queries per request", flush=True)
    dsa = dsa_mod()
    s_len = np.array([3000, 2100, 5000, 40, 2049])
    q_req = np.repeat(np.arange(5), 3).astype(np.int32)
    q_pos = (s_len[q_req] - 3 + np.tile(np.arange(3), 5)).astype(np.int32)
    lay = synth.Layout("multi", 21, s_len, q_req, q_pos)
    assert lay.T < 8 * lay.B
    d, keys = idx_inputs(lay, 21)
    check_scores(lay, d, keys, run_scores(lay, d, keys))
    args = (dev(d["q_idx"]), dev(d["w"]), dev(keys), dev(lay.kv_off), dev(lay.q_req),
            dev(lay.q_pos), lay.max_s)
    ids = dsa.indexer_topk(*args)
    n_valid = np.minimum(lay.q_pos + 1, lay.s_len[lay.q_req]).astype(np.int32)
    ids2 = dsa.topk(dsa.indexer_scores(*args), dev(n_valid), max_n=lay.max_s)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    got = ids.cpu().numpy()
    check_selection(lay, got, O.indexer_scores(d["q_idx"], d["w"], keys, lay.kv_off, lay.q_req,
                                                lay.q_pos))
    dm = synth.inputs_np(lay, parts=("mla",))
    got_o, got_l = run_mla(lay, dm, got)
    check_mla(lay, dm, got, got_o, got_l)


def test_indexer_topk_two_stage_long_rows_bit_exact():
    """Few long rows take the two-stage selection (parts of >= 65536 positions, then a merge
    of the part lists).  Integer inputs make every score exact in fp32 and produce many ties,
    so the IDs must equal the oracle's top-2048 (ties to the lower position) exactly; the
    second request leaves parts partly and wholly empty."""
    print("[indexer_topk] two-stage long rows", flush=True)
    dsa = dsa_mod()
    g = np.random.default_rng(17)
    lay = synth.decode_layout("long2", 17, [300000, 140000])
    q = synth.bf16_bits_from_f32(g.integers(-2, 3, size=(lay.T, 32, 128)))
    w = synth.bf16_bits_from_f32(2.0 ** g.integers(-4, 2, size=(lay.T, 32)) *
                                 g.choice([-1, 1], size=(lay.T, 32)))
    keys = synth.bf16_bits_from_f32(g.integers(-2, 3, size=(lay.N, 128)))
    args = (dev(q), dev(w), dev(keys), dev(lay.kv_off), dev(lay.q_req), dev(lay.q_pos))
    assert dsa.indexer_topk_workspace_size(lay.T, lay.max_s) > lay.T * lay.max_s * 4  # split
    ids = dsa.indexer_topk(*args, lay.max_s)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    ref = O.indexer_scores(q, w, keys, lay.kv_off, lay.q_req, lay.q_pos)
    for t in range(lay.T):
        assert np.array_equal(got[t], O.topk_ids(ref[t])), f"row {t}"


def _int_index_inputs(g, t, n_keys):
    """Integer index queries and keys in {-2..2} and signed power-of-two head weights: every
    score is exact in fp32 (and in the oracle's fp64), and the scores take few distinct
    values, so the k-th score is shared by many positions."""
    q = synth.bf16_bits_from_f32(g.integers(-2, 3, size=(t, 32, 128)))
    w = synth.bf16_bits_from_f32(2.0 ** g.integers(-4, 2, size=(t, 32)) *
                                 g.choice([-1, 1], size=(t, 32)))
    keys = synth.bf16_bits_from_f32(g.integers(-2, 3, size=(n_keys, 128)))
    return q, w, keys


@pytest.mark.parametrize("s_total,q_pos,parts", [
    (1_048_576, [1_048_575, 1_048_574, 1_000_000, 70_000], 16),
    (600_000, [599_999, 450_000], 8)])
def test_indexer_topk_multi_part_merge_bit_exact(s_total, q_pos, parts):
    """Few rows of up to 1,048,576 positions run the two-stage selection in 8 or 16 parts of
    >= 65,536 positions, then the merge of the part lists.  All queries read one request, so
    the rows share their keys; with exact integer scores and many ties across part borders the
    IDs must equal the oracle's top-2048 (ties to the lower position) bit for bit.  Shorter
    rows leave trailing parts partly or wholly empty."""
    print(f"[indexer_topk] {parts}-part merge S={s_total}", flush=True)
    dsa = dsa_mod()
    g = np.random.default_rng(18 + parts)
    lay = synth.Layout(f"merge{parts}", 18, [s_total], np.zeros(len(q_pos), np.int32),
                       np.array(q_pos, np.int32))
    assert lay.T < 8 * lay.B  # the streaming scoring kernel, as decode uses
    q, w, keys = _int_index_inputs(g, lay.T, lay.N)
    ws = dsa.indexer_topk_workspace_size(lay.T, lay.max_s)
    assert ws - (lay.T * lay.max_s * 4) >= lay.T * parts * 2048 * 4  # candidate lists of `parts`
    args = (dev(q), dev(w), dev(keys), dev(lay.kv_off), dev(lay.q_req), dev(lay.q_pos))
    ids = dsa.indexer_topk(*args, lay.max_s)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    ref = O.indexer_scores(q, w, keys, lay.kv_off, lay.q_req, lay.q_pos)
    for t in range(lay.T):
        want = O.topk_ids(ref[t])
        kth = ref[t][want[-1]] if len(ref[t]) > 2048 else None
        ties = int(np.sum(ref[t] == np.min(ref[t][want]))) if kth is not None else 0
        print(f"  row {t}: n={len(ref[t])} ties at the k-th score: {ties}", flush=True)
        assert np.array_equal(got[t], want), f"row {t}"


def test_queries_outside_the_batch_select_and_read_nothing():
    """q_req values outside [0, B) (B itself and -1): such a query has no admissible position.
    Its scores are not written, its ID row is all -1 and its read is zero with lse -inf; the
    other queries' results equal those of a call without the stray queries.  Both scoring
    kernels (streaming decode and the prefill kernel) and the FP8 variant are covered."""
    print("[contract] q_req outside [0, B)", flush=True)
    dsa = dsa_mod()
    # streaming decode kernel: 3 requests, 5 queries, two of them outside the batch
    lay = synth.Layout("stray", 19, [3000, 2500, 5000], np.array([0, 3, 1, -1, 2], np.int32),
                       np.array([2999, 100, 2499, 7, 4999], np.int32))
    d, keys = idx_inputs(lay, 19)
    good = [0, 2, 4]
    base = synth.Layout("stray_ok", 19, [3000, 2500, 5000], lay.q_req[good], lay.q_pos[good])
    args = (dev(d["q_idx"]), dev(d["w"]), dev(keys), dev(lay.kv_off), dev(lay.q_req), dev(lay.q_pos))
    s = dsa.indexer_scores(*args, lay.max_s)
    ids = dsa.indexer_topk(*args, lay.max_s)
    codes, scales = dsa.quantize_index_keys_fp8(dev(keys))
    s8 = dsa.indexer_scores_fp8(dev(d["q_idx"]), dev(d["w"]), codes, scales, dev(lay.kv_off),
                                dev(lay.q_req), dev(lay.q_pos), lay.max_s)
    ids_ok = dsa.indexer_topk(dev(d["q_idx"][good]), dev(d["w"][good]), dev(keys),
                              dev(base.kv_off), dev(base.q_req), dev(base.q_pos), base.max_s)
    dm = synth.inputs_np(lay, parts=("mla",))
    out, lse = dsa.sparse_mla_attn(dev(dm["q"]), dev(dm["latent"]), dev(dm["kpe"]),
                                   dev(lay.kv_off), dev(lay.q_req), ids, synth.ATTN_SCALE)
    out_ok, lse_ok = dsa.sparse_mla_attn(dev(dm["q"][good]), dev(dm["latent"]), dev(dm["kpe"]),
                                         dev(base.kv_off), dev(base.q_req), ids_ok,
                                         synth.ATTN_SCALE)
    torch.cuda.synchronize()
    for t in (1, 3):
        assert torch.isnan(s[t]).all() and torch.isnan(s8[t]).all()
        assert (ids[t] == -1).all()
        assert (out[t].float() == 0).all() and torch.isneginf(lse[t]).all()
    assert torch.equal(ids[good], ids_ok)
    assert torch.equal(out[good].view(torch.int16), out_ok.view(torch.int16))
    assert torch.equal(lse[good], lse_ok)
    # prefill kernel (T >= 8 B): one request, 24 queries, four of them outside the batch
    req = np.zeros(24, np.int32)
    req[[0, 5, 17, 23]] = [1, -1, 7, 1]
    pl = synth.Layout("stray_pf", 20, [2000], req, (1900 + np.arange(24)).astype(np.int32))
    pd, pkeys = idx_inputs(pl, 20)
    pargs = (dev(pd["q_idx"]), dev(pd["w"]), dev(pkeys), dev(pl.kv_off), dev(pl.q_req),
             dev(pl.q_pos))
    ps = dsa.indexer_scores(*pargs, pl.max_s)
    pids = dsa.indexer_topk(*pargs, pl.max_s)
    torch.cuda.synchronize()
    ps_h = ps.cpu().numpy()
    ok_rows = [t for t in range(pl.T) if pl.q_req[t] == 0]
    ref = O.indexer_scores(pd["q_idx"], pd["w"], pkeys, pl.kv_off, pl.q_req, pl.q_pos,
                           rows=ok_rows)
    for i, t in enumerate(ok_rows):
        n = len(ref[i])
        assert np.all(np.abs(ps_h[t, :n] - ref[i]) <= 1e-3 * np.maximum(np.abs(ref[i]), O.row_scale(ref[i])))
    for t in (0, 5, 17, 23):
        assert np.all(np.isnan(ps_h[t])) and (pids[t] == -1).all()


def test_indexer_topk_prefill():
    print("[indexer_topk] prefill", flush=True)
    dsa = dsa_mod()
    lay = synth.prefill_layout("pf", 16, 9000, 8900, 100)
    d, keys = idx_inputs(lay, 16)
    ids = dsa.indexer_topk(dev(d["q_idx"]), dev(d["w"]), dev(keys), dev(lay.kv_off),
                           dev(lay.q_req), dev(lay.q_pos), lay.max_s)
    torch.cuda.synchronize()
    ref = O.indexer_scores(d["q_idx"], d["w"], keys, lay.kv_off, lay.q_req, lay.q_pos)
    check_selection(lay, ids.cpu().numpy(), ref)


def test_indexer_topk_persistent_prefill_chunk():
    """600 chunk queries in two requests, rows of 35,701..40,000 admissible positions: more
    rows than CUs, so the selection runs the persistent blocks with row lengths taken from
    kv_off / q_req / q_pos.  The fused selection equals the standalone one over the same
    scores (explicit lengths) bit for bit, and sampled queries match the oracle."""
    print("[indexer_topk] persistent prefill chunk", flush=True)
    dsa = dsa_mod()
    q_req = np.repeat(np.arange(2, dtype=np.int32), 300)
    q_pos = np.concatenate([39700 + np.arange(300), 35700 + np.arange(300)]).astype(np.int32)
    lay = synth.Layout("ppc", 33, [40000, 36000], q_req, q_pos)
    d, keys = idx_inputs(lay, 33)
    args = (dev(d["q_idx"]), dev(d["w"]), dev(keys), dev(lay.kv_off), dev(lay.q_req),
            dev(lay.q_pos), lay.max_s)
    ids = dsa.indexer_topk(*args)
    scores = dsa.indexer_scores(*args)
    n_valid = np.minimum(lay.q_pos + 1, lay.s_len[lay.q_req]).astype(np.int32)
    ids2 = dsa.topk(scores, dev(n_valid), max_n=lay.max_s)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    got = ids.cpu().numpy()
    for t in (0, 299, 300, 599):
        b = int(lay.q_req[t])
        lo, hi = int(lay.kv_off[b]), int(lay.kv_off[b + 1])
        one = synth.Layout("ppc1", 33, [hi - lo], np.zeros(1, np.int32), lay.q_pos[t:t + 1])
        ref = O.indexer_scores(d["q_idx"][t:t + 1], d["w"][t:t + 1], keys[lo:hi], one.kv_off,
                               one.q_req, one.q_pos)
        check_selection(one, got[t:t + 1], ref)


# ---------------------------------------------------------------------------------------
# stage 4
# ---------------------------------------------------------------------------------------
def run_mla(lay, d, ids, scale=synth.ATTN_SCALE, packed=False, f32=False):
    dsa = dsa_mod()
    if packed:
        base = dev(np.concatenate([d["latent"], d["kpe"]], axis=1))
        lat, kpe = base, base[:, 512:]
    else:
        lat, kpe = dev(d["latent"]), dev(d["kpe"])
    out, lse = dsa.sparse_mla_attn(dev(d["q"]), lat, kpe, dev(lay.kv_off), dev(lay.q_req),
                                   dev(ids), scale,
                                   out_dtype=torch.float32 if f32 else torch.bfloat16)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def bf16_half_ulp(v):
    """Half the spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.abs(v)
    return np.where(a > 0, np.ldexp(1.0, np.frexp(a)[1] - 9), 0.0)


def out_tolerance(ref_o, f32):
    """1e-2 on the read itself; a bf16 output adds its own rounding (half an ulp)."""
    return 1e-2 + (0.0 if f32 else bf16_half_ulp(ref_o))


def check_mla(lay, d, ids, got_o, got_l, scale=synth.ATTN_SCALE, f32=False):
    ref_o, ref_l = O.sparse_mla(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, ids, scale)
    err = np.abs(got_o - ref_o)
    assert np.all(err <= out_tolerance(ref_o, f32)), f"max abs err {err.max()}"
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(got_l))
    assert np.all(np.abs(got_l[fin] - ref_l[fin]) <= 1e-3 * np.maximum(1, np.abs(ref_l[fin])))
    assert np.all(got_l[~fin] == -np.inf) and np.all(got_o[~np.isfinite(ref_l)] == 0)


# Query counts that give every split count of the read: 16 (1 and 4 queries), 8 (40), 4 (64),
# 2 (130) and 1 (300), each merged by its own combine.
@pytest.mark.parametrize("t_count,packed,f32", [(1, False, False), (4, True, True),
                                                (40, False, False), (40, True, True),
                                                (64, False, False), (64, False, True),
                                                (130, False, True), (130, True, False),
                                                (300, False, False), (300, True, True)])
def test_sparse_mla_parity(t_count, packed, f32):
    print(f"[mla] T={t_count} packed={packed} f32={f32}", flush=True)
    g = np.random.default_rng(30 + t_count)
    s_len = g.integers(1, 6000, size=t_count)
    s_len[0] = 5000
    lay = synth.decode_layout("mla", 30 + t_count, s_len)
    d = synth.inputs_np(lay, parts=("mla",))
    ids = synth.random_ids_np(30 + t_count, lay)
    got_o, got_l = run_mla(lay, d, ids, packed=packed, f32=f32)
    check_mla(lay, d, ids, got_o, got_l, f32=f32)


@pytest.mark.parametrize("f32", [False, True])
def test_sparse_mla_split_workspace_reuse(f32):
    """Small T splits each ID row over several blocks and merges their partials (bf16 partials
    for a bf16 output); one caller-owned workspace, filled with garbage first, serves several
    calls in a row, and every result matches the oracle."""
    print(f"[mla] split workspace reuse f32={f32}", flush=True)
    dsa = dsa_mod()
    lay = synth.decode_layout("reuse", 77, [5000, 4000, 2500])
    d = synth.inputs_np(lay, parts=("mla",))
    need = dsa.sparse_mla_workspace_size(lay.T)
    assert need > 0  # three queries: split path
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for call in range(3):
        ids = synth.random_ids_np(100 + call, lay)
        out, lse = dsa.sparse_mla_attn(dev(d["q"]), dev(d["latent"]), dev(d["kpe"]),
                                       dev(lay.kv_off), dev(lay.q_req), dev(ids),
                                       synth.ATTN_SCALE, workspace=ws,
                                       out_dtype=torch.float32 if f32 else torch.bfloat16)
        torch.cuda.synchronize()
        check_mla(lay, d, ids, out.float().cpu().numpy(), lse.cpu().numpy(), f32=f32)


def test_sparse_mla_special_rows():
    print("[mla] special rows", flush=True)
    lay = synth.decode_layout("sp", 40, [3000, 3000, 3000, 2000, 50])
    d = synth.inputs_np(lay, parts=("mla",))
    lat = O.bf16_to_f64(d["latent"])
    lat[:, 0] = 1.0
    d["latent"] = O.f64_to_bf16(lat)
    ids = synth.random_ids_np(40, lay)
    ids[1] = -1
    ids[1, 7] = 123                       # a single valid ID in the middle of padding
    ids[2] = -1                           # no valid ID
    ids[2, :5] = [3000, 4000, -5, 99999, -1]  # out-of-range entries are padding
    ids[3] = np.random.default_rng(1).permutation(ids[3])  # order must not matter
    got_o, got_l = run_mla(lay, d, ids)
    check_mla(lay, d, ids, got_o, got_l)
    assert np.all(got_o[[0, 1, 3, 4], :, 0] == 1.0)  # weights sum to one, exactly in bf16
    row = O.bf16_to_f64(d["latent"][lay.kv_off[1] + 123])
    assert np.array_equal(got_o[1], np.broadcast_to(row, (96, 512)))
    assert np.all(got_o[2] == 0) and np.all(got_l[2] == -np.inf)


def test_sparse_mla_short_prefix_equals_dense():
    print("[mla] short prefix == dense", flush=True)
    lay = synth.decode_layout("dense", 41, [1, 100, 2047, 2048])
    d = synth.inputs_np(lay, parts=("mla",))
    ids = O.topk_rows([np.zeros(n) for n in lay.s_len])
    got_o, _ = run_mla(lay, d, ids, f32=True)
    dr = O.dense_read(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, lay.q_pos, ids,
                      synth.ATTN_SCALE)
    assert np.all(dr["eps"] == 0)
    assert np.abs(got_o - dr["o_full"]).max() <= 1e-2


def test_sparse_mla_large_logits_take_the_exact_max_pass():
    print("[mla] large logit spread", flush=True)
    # scale 4: logit spread far beyond 2^32 between the first tile and later ones; the
    # softmax is then nearly one-hot, so outputs reach |o| ~ 4 -- read in fp32
    for t_count in (1, 300):
        lay = synth.decode_layout("big", 42, [4096] * t_count)
        d = synth.inputs_np(lay, parts=("mla",))
        ids = synth.random_ids_np(42, lay)
        got_o, got_l = run_mla(lay, d, ids, scale=4.0, f32=True)
        check_mla(lay, d, ids, got_o, got_l, scale=4.0, f32=True)


# ---------------------------------------------------------------------------------------
# the whole path, and determinism
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["decode_b4_s4096", "decode_b256_mixed"])
def test_end_to_end_small_workloads(name):
    print(f"[e2e] {name}", flush=True)
    dsa = dsa_mod()
    lay = synth.workload(name)
    d = synth.inputs_np(lay)
    keys = dsa.index_keys_layernorm(dev(d["raw_keys"]), dev(d["gamma"]), dev(d["beta"]),
                                    synth.LN_EPS)
    ids = dsa.indexer_topk(dev(d["q_idx"]), dev(d["w"]), keys, dev(lay.kv_off), dev(lay.q_req),
                           dev(lay.q_pos), lay.max_s)
    out, lse = dsa.sparse_mla_attn(dev(d["q"]), dev(d["latent"]), dev(d["kpe"]),
                                   dev(lay.kv_off), dev(lay.q_req), ids, synth.ATTN_SCALE)
    ids2 = dsa.indexer_topk(dev(d["q_idx"]), dev(d["w"]), keys, dev(lay.kv_off), dev(lay.q_req),
                            dev(lay.q_pos), lay.max_s)
    out2, _ = dsa.sparse_mla_attn(dev(d["q"]), dev(d["latent"]), dev(d["kpe"]),
                                  dev(lay.kv_off), dev(lay.q_req), ids2, synth.ATTN_SCALE)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(out, out2), "not deterministic"
    keys_ref = O.layernorm_keys_bf16(d["raw_keys"], d["gamma"], d["beta"], synth.LN_EPS)
    assert ln_tolerance_ok(host_bits(keys), d["raw_keys"], d["gamma"], d["beta"], synth.LN_EPS) < 1e-3
    s_ref = O.indexer_scores(d["q_idx"], d["w"], keys_ref, lay.kv_off, lay.q_req, lay.q_pos)
    got_ids = ids.cpu().numpy()
    check_selection(lay, got_ids, s_ref)
    ids_ref = O.topk_rows(s_ref)
    same = [t for t in range(lay.T) if np.array_equal(got_ids[t], ids_ref[t])]
    assert len(same) >= 0.9 * lay.T
    o_ref, l_ref = O.sparse_mla(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, ids_ref,
                                synth.ATTN_SCALE, rows=same)
    o = out.float().cpu().numpy()[same]
    assert np.all(np.abs(o - o_ref) <= out_tolerance(o_ref, False))
    # the dropped-mass bound against the oracle's full causal read
    dr = O.dense_read(d["q"], d["latent"], d["kpe"], lay.kv_off, lay.q_req, lay.q_pos, ids_ref,
                      synth.ATTN_SCALE, rows=same)
    assert np.all(np.abs(o - dr["o_full"]) <= dr["eps"][:, :, None] * dr["v_range"][:, None, :]
                  + out_tolerance(dr["o_full"], False))


# ---------------------------------------------------------------------------------------
# after stage 4: value up-projection and sigmoid output gate
# ---------------------------------------------------------------------------------------
def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (8 significant bits; subnormal floor 2^-133)."""
    a = np.abs(v)
    return np.where(a > 0, np.ldexp(1.0, np.maximum(np.frexp(a)[1] - 8, -133)), np.ldexp(1.0, -133))


def vg_tolerance(ref, mag):
    """One bf16 ulp of the result (its rounding, with room for the fp32 value to sit across a
    binade boundary) plus the fp32 error of a 512-term dot product and the fp32 sigmoid:
    <= 512 * 2^-24 of the sum of |terms| (2^-15), doubled."""
    return bf16_ulp(ref) + 2.0 ** -14 * mag


def run_vg(o, w_uv, gate):
    dsa = dsa_mod()
    out = dsa.value_gate(dev(o), dev(w_uv), dev(gate))
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


@pytest.mark.parametrize("t_count", [1, 33, 64, 300])
def test_value_gate_parity(t_count):
    print(f"[value_gate] T={t_count}", flush=True)
    lay = synth.decode_layout("vg", 50 + t_count, [100] * t_count)
    d = synth.inputs_np(lay, parts=("gate",))
    got = run_vg(d["o"], d["w_uv"], d["gate"])
    ref = O.value_gate(d["o"], d["w_uv"], d["gate"])
    mag = O.value_gate_magnitude(d["o"], d["w_uv"], d["gate"])
    err = np.abs(got - ref)
    assert np.all(err <= vg_tolerance(ref, mag)), f"max err {err.max()}"


def test_value_gate_exact_on_integer_inputs_and_gate_extremes():
    """Small integers make the fp32 contraction exact; logits of +-2^100 and +-inf give gates
    of exactly 1 and 0, NaN logits give NaN: the output must equal the oracle bit for bit."""
    print("[value_gate] exact", flush=True)
    g = np.random.default_rng(61)
    t = 40
    o = synth.bf16_bits_from_f32(g.integers(-2, 3, size=(t, 96, 512)))
    w = synth.bf16_bits_from_f32(g.integers(-1, 2, size=(96, 128, 512)) * (g.random((96, 128, 512)) < 0.1))
    lg = np.where(g.random((t, 96, 128)) < 0.5, 2.0 ** 100, -(2.0 ** 100)).astype(np.float32)
    lg[0, 0, :4] = [np.inf, -np.inf, np.nan, 0.0]
    gate = synth.bf16_bits_from_f32(lg)
    got = run_vg(o, w, gate)
    ref = O.value_gate(o, w, gate)
    assert np.all(np.abs(ref[np.isfinite(ref)]) < 256)  # every result is a bf16 integer
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.isnan(got[0, 0, 2])


def test_value_gate_on_the_sparse_read():
    """End to end after stage 4: the epilogue applied to the GPU read equals the oracle's
    epilogue of the same (bf16) read."""
    print("[value_gate] after the read", flush=True)
    lay = synth.decode_layout("vgr", 62, [3000, 2500, 40])
    d = synth.inputs_np(lay, parts=("mla", "gate"))
    ids = synth.random_ids_np(62, lay)
    dsa = dsa_mod()
    o, _ = dsa.sparse_mla_attn(dev(d["q"]), dev(d["latent"]), dev(d["kpe"]), dev(lay.kv_off),
                               dev(lay.q_req), dev(ids), synth.ATTN_SCALE)
    u = dsa.value_gate(o, dev(d["w_uv"]), dev(d["gate"]))
    torch.cuda.synchronize()
    o_bits = host_bits(o)
    ref = O.value_gate(o_bits, d["w_uv"], d["gate"])
    mag = O.value_gate_magnitude(o_bits, d["w_uv"], d["gate"])
    assert np.all(np.abs(u.float().cpu().numpy() - ref) <= vg_tolerance(ref, mag))
