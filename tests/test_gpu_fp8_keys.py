"""GPU parity of the FP8 index-key cache variant (dsa_quantize_index_keys_fp8,
dsa_indexer_scores_fp8, dsa_indexer_topk_fp8) against the oracle.

Bars: the codes and scales are integer/byte work and must equal the oracle's bit for bit;
scores over the decoded keys |s - s_ref| <= 1e-3 * max(|s_ref|, r_t) (r_t the row's RMS
score), exactly as for the bf16 cache (the decoded keys are exact in bf16, so only the fp32
sums and the final scale multiply round); integer inputs make the scores exact; the
selection equals the standalone top-k of the same scores bit for bit and the oracle's up to
the 1e-3 band of the k-th score.
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


def quantize(keys_bits):
    codes, scales = dsa_mod().quantize_index_keys_fp8(dev(keys_bits))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def adversarial_keys(seed):
    """Rows that exercise every branch of the rounding: zeros and -0, bf16 subnormals, huge
    and tiny magnitudes, exact E4M3 midpoints, a row whose maximum sits just above 1.75 *
    2^k (the scale-exponent boundary), and LayerNorm-like rows."""
    g = np.random.default_rng(seed)
    rows = [np.zeros(128), -np.zeros(128), np.full(128, 1e-39), g.standard_normal(128) * 1e30,
            g.standard_normal(128) * 1e-30]
    v = O.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))  # 0 .. 448, all finite
    mids = (v[:-1] + v[1:]) / 2                              # 126 midpoints
    rows.append(np.concatenate([mids, [448.0, 0.0]]))        # scale 1: ties to even
    rows.append(np.concatenate([-mids, [448.0, -0.0]]))
    rows.append(np.concatenate([[1.75 * 2 ** 3 * (1 + 2 ** -7)], g.standard_normal(127)]))
    rows.append(np.concatenate([[1.75 * 2 ** 3], g.standard_normal(127)]))
    x = np.stack(rows + [g.standard_normal(128) * np.exp(g.uniform(-8, 8)) for _ in range(300)])
    return synth.bf16_bits_from_f32(x.astype(np.float32))


def test_quantization_bit_exact():
    print("[fp8] quantization", flush=True)
    keys = adversarial_keys(1)
    lay = synth.decode_layout("q8", 2, [777])
    ln = O.layernorm_keys_bf16(synth.inputs_np(lay, parts=("index",))["raw_keys"],
                               np.ones(128, np.float32), np.zeros(128, np.float32), 1e-6)
    keys = np.concatenate([keys, ln])
    codes, scales = quantize(keys)
    rc, rs = O.quantize_keys_fp8(keys)
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(codes, rc)


def test_quantization_every_bf16_value_bit_exact():
    """Every finite bf16 value of magnitude <= 448 (both signs, zeros and bf16 subnormals
    included), in rows whose maximum is 448 (scale 1), and the same values times 2^20 in rows
    whose maximum is 448 * 2^20 (scale 2^20, the scaled values become fp32 subnormals at the
    bottom): the codes must equal the oracle's correctly rounded E4M3 codes, every one."""
    print("[fp8] every bf16 value", flush=True)
    pos = np.arange(0, 0x43E1, dtype=np.uint32)            # +0 .. 448 (0x43E0 = 1.75 * 2^8)
    bits = np.concatenate([pos, pos | 0x8000])
    vals = (bits << 16).view(np.float32)
    per_row = 127
    n_rows = -(-vals.size // per_row)
    body = np.zeros(n_rows * per_row, np.float32)
    body[:vals.size] = vals
    rows = []
    for mult in (1.0, 2.0 ** 20):
        x = np.concatenate([body.reshape(n_rows, per_row) * np.float32(mult),
                            np.full((n_rows, 1), 448.0 * mult, np.float32)], axis=1)
        rows.append(synth.bf16_bits_from_f32(x))
    keys = np.concatenate(rows)
    assert np.array_equal((keys[:n_rows, :per_row].astype(np.uint32) << 16).view(np.float32).ravel()[:vals.size].view(np.uint32),
                          vals.view(np.uint32))                  # the bf16 rows hold the values exactly
    codes, scales = quantize(keys)
    rc, rs = O.quantize_keys_fp8(keys)
    assert np.array_equal(rs[:n_rows], np.ones(n_rows)) and np.array_equal(rs[n_rows:], np.full(n_rows, 2.0 ** 20))
    assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
    bad = np.nonzero(codes != rc)
    assert bad[0].size == 0, (f"{bad[0].size} codes differ, first at row {bad[0][0]} col {bad[1][0]}: "
                              f"got {codes[bad][0]:#04x}, oracle {rc[bad][0]:#04x}")


def check_scores(lay, d, codes, scales, got):
    ref = O.indexer_scores_fp8(d["q_idx"], d["w"], codes, scales, lay.kv_off, lay.q_req, lay.q_pos)
    for t in range(lay.T):
        n = len(ref[t])
        r = O.row_scale(ref[t])
        err = np.abs(got[t, :n] - ref[t])
        assert np.all(err <= 1e-3 * np.maximum(np.abs(ref[t]), r) + 1e-30), \
            f"query {t}: max rel err {(err / np.maximum(np.abs(ref[t]), r)).max()}"
        assert np.all(np.isnan(got[t, n:])), f"query {t}: wrote past n_t"
    return ref


LAYOUTS = [
    ("decode_ragged", lambda: synth.decode_layout("f8r", 11, [1, 5, 2047, 2048, 2049, 4096, 5000])),
    ("decode_long", lambda: synth.decode_layout("f8l", 12, [70000, 3])),
    ("prefill", lambda: synth.prefill_layout("f8p", 13, 3000, 2900, 100)),
]


@pytest.mark.parametrize("name,make", LAYOUTS)
def test_scores_fp8_parity(name, make):
    print(f"[fp8] scores {name}", flush=True)
    lay = make()
    d = synth.inputs_np(lay, parts=("index",))
    keys = synth.bf16_bits_from_f32(np.random.default_rng(14).standard_normal((lay.N, 128)))
    codes, scales = quantize(keys)
    s = dsa_mod().indexer_scores_fp8(dev(d["q_idx"]), dev(d["w"]), dev(codes), dev(scales),
                                     dev(lay.kv_off), dev(lay.q_req), dev(lay.q_pos), lay.max_s)
    torch.cuda.synchronize()
    check_scores(lay, d, codes, scales, s.cpu().numpy())


def test_scores_fp8_unaligned_rows():
    """FP8-key scores into rows that do not start on 16-byte boundaries (an odd row stride,
    one float into the buffer) are stored element by element, and only at positions < n_t."""
    print("[fp8] scores unaligned rows", flush=True)
    lay = synth.decode_layout("f8u", 16, [3, 2049, 5001, 4096])
    lay.q_pos[-1] = 3001
    d = synth.inputs_np(lay, parts=("index",))
    keys = synth.bf16_bits_from_f32(np.random.default_rng(16).standard_normal((lay.N, 128)))
    codes, scales = quantize(keys)
    buf = torch.full((lay.T, lay.max_s + 2), float("nan"), dtype=torch.float32, device=DEV)
    view = buf[:, 1:1 + lay.max_s]
    assert view.data_ptr() % 16 != 0 and view.stride(0) % 4 != 0
    dsa_mod().indexer_scores_fp8(dev(d["q_idx"]), dev(d["w"]), dev(codes), dev(scales),
                                 dev(lay.kv_off), dev(lay.q_req), dev(lay.q_pos), lay.max_s,
                                 scores=view)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    check_scores(lay, d, codes, scales, b[:, 1:1 + lay.max_s])
    assert np.all(np.isnan(b[:, 0])) and np.all(np.isnan(b[:, -1]))


def test_scores_fp8_exact_on_integer_inputs():
    """Integer keys up to 8 quantise exactly (scale 2^-5, codes up to 256) and integer queries
    with power-of-two weights keep every fp32 sum exact: bit-exact scores."""
    print("[fp8] exact integers", flush=True)
    g = np.random.default_rng(15)
    lay = synth.decode_layout("f8x", 15, [300, 4100])
    keys_f = g.integers(-8, 9, size=(lay.N, 128)).astype(np.float32)
    keys_f[:, 0] = 8.0
    keys = synth.bf16_bits_from_f32(keys_f)
    q = synth.bf16_bits_from_f32(g.integers(-2, 3, size=(lay.T, 32, 128)))
    w = synth.bf16_bits_from_f32(2.0 ** g.integers(-4, 2, size=(lay.T, 32)) * g.choice([-1, 1], size=(lay.T, 32)))
    codes, scales = quantize(keys)
    assert np.array_equal(O.dequantize_keys_fp8(codes, scales), keys_f.astype(np.float64))
    s = dsa_mod().indexer_scores_fp8(dev(q), dev(w), dev(codes), dev(scales), dev(lay.kv_off),
                                     dev(lay.q_req), dev(lay.q_pos), lay.max_s)
    torch.cuda.synchronize()
    got = s.cpu().numpy()
    ref = O.indexer_scores_fp8(q, w, codes, scales, lay.kv_off, lay.q_req, lay.q_pos)
    for t in range(lay.T):
        assert np.array_equal(got[t, :len(ref[t])], ref[t].astype(np.float32))


def test_indexer_topk_fp8_matches_standalone_topk_and_oracle():
    print("[fp8] indexer_topk", flush=True)
    dsa = dsa_mod()
    lay = synth.decode_layout("f8k", 16, [1, 2047, 2049, 4096, 9000, 33000])
    d = synth.inputs_np(lay, parts=("index",))
    keys = synth.bf16_bits_from_f32(np.random.default_rng(16).standard_normal((lay.N, 128)))
    codes, scales = quantize(keys)
    args = (dev(d["q_idx"]), dev(d["w"]), dev(codes), dev(scales), dev(lay.kv_off),
            dev(lay.q_req), dev(lay.q_pos))
    ids = dsa.indexer_topk_fp8(*args, lay.max_s)
    scores = dsa.indexer_scores_fp8(*args, lay.max_s)
    n_valid = np.minimum(lay.q_pos + 1, lay.s_len[lay.q_req]).astype(np.int32)
    ids2 = dsa.topk(scores, dev(n_valid), max_n=lay.max_s)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    ref = O.indexer_scores_fp8(d["q_idx"], d["w"], codes, scales, lay.kv_off, lay.q_req, lay.q_pos)
    got = ids.cpu().numpy()
    for t in range(lay.T):
        n = len(ref[t])
        m = min(n, 2048)
        valid = got[t][got[t] >= 0]
        assert len(valid) == m and np.all(got[t][m:] == -1)
        diff = set(valid.tolist()) ^ set(O.topk_ids(ref[t])[:m].tolist())
        assert diff <= set(O.selection_band(ref[t]).tolist()), f"query {t}"


def test_indexer_topk_fp8_long_rows_many_queries():
    """300 chunk queries with 33,001..33,300 admissible positions (more rows than CUs, so the
    persistent selection): every row's FP8 selection equals the oracle's top-k of the GPU's
    own FP8 scores bit for bit, and sampled queries match the oracle over the same codes."""
    print("[fp8] indexer_topk long rows", flush=True)
    dsa = dsa_mod()
    lay = synth.prefill_layout("f8p2", 17, 33300, 33000, 300)
    d = synth.inputs_np(lay, parts=("index",))
    keys = synth.bf16_bits_from_f32(np.random.default_rng(17).standard_normal((lay.N, 128)))
    codes, scales = quantize(keys)
    args = (dev(d["q_idx"]), dev(d["w"]), dev(codes), dev(scales), dev(lay.kv_off),
            dev(lay.q_req), dev(lay.q_pos))
    ids = dsa.indexer_topk_fp8(*args, lay.max_s)
    scores = dsa.indexer_scores_fp8(*args, lay.max_s)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    s_gpu = scores.cpu().numpy()
    n_valid = np.minimum(lay.q_pos + 1, lay.s_len[lay.q_req])
    # every row: the fused selection equals the oracle's top-k of the GPU's own fp32 FP8
    # scores, bit for bit (identical score arrays)
    for t in range(lay.T):
        assert np.array_equal(got[t], O.topk_ids(s_gpu[t, :n_valid[t]])), f"row {t}"
    # sampled rows: the scores themselves against the oracle over the same codes
    for t in (0, 150, 299):
        one = synth.Layout("f8p2one", 17, [lay.N], np.zeros(1, np.int32), lay.q_pos[t:t + 1])
        ref = O.indexer_scores_fp8(d["q_idx"][t:t + 1], d["w"][t:t + 1], codes, scales,
                                   one.kv_off, one.q_req, one.q_pos)[0]
        valid = got[t][got[t] >= 0]
        assert len(valid) == 2048
        diff = set(valid.tolist()) ^ set(O.topk_ids(ref)[:2048].tolist())
        assert diff <= set(O.selection_band(ref).tolist()), f"query {t}"


def test_fp8_full_size_decode_sampled():
    """The 64 x 32768 decode batch: LayerNorm keys quantised on the GPU, the FP8 selection of
    sampled queries against the oracle over the same codes."""
    print("[fp8] full size decode", flush=True)
    dsa = dsa_mod()
    lay = synth.workload("decode_b64_s32768")
    dg = synth.inputs_torch(lay, torch.device(DEV), parts=("index", "ln"))
    keys = dsa.index_keys_layernorm(dg["raw_keys"], dg["gamma"], dg["beta"], synth.LN_EPS)
    codes, scales = dsa.quantize_index_keys_fp8(keys)
    ids = dsa.indexer_topk_fp8(dg["q_idx"], dg["w"], codes, scales, dg["kv_off"], dg["q_req"],
                               dg["q_pos"], lay.max_s)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    for t in (0, 37, 63):
        lo, hi = int(lay.kv_off[t]), int(lay.kv_off[t + 1])
        kb = keys[lo:hi].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        rc, rs = O.quantize_keys_fp8(kb)
        assert np.array_equal(codes[lo:hi].cpu().numpy(), rc)
        assert np.array_equal(scales[lo:hi].cpu().numpy(), rs)
        q = synth.to_bits_np(dg["q_idx"][t:t + 1])
        w = synth.to_bits_np(dg["w"][t:t + 1])
        ref = O.indexer_scores_fp8(q, w, rc, rs, np.array([0, hi - lo]), np.zeros(1, np.int32),
                                   np.array([hi - lo - 1], np.int32))[0]
        valid = got[t][got[t] >= 0]
        assert len(valid) == 2048
        diff = set(valid.tolist()) ^ set(O.topk_ids(ref)[:2048].tolist())
        assert diff <= set(O.selection_band(ref).tolist()), f"query {t}"
