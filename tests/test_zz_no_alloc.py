"""The allocation-free stages 2+3 (dsa_indexer_topk_noalloc, through the C ABI binding) against
dsa_indexer_topk with a caller workspace: identical IDs, bit for bit, on consecutive calls that
share the library's per-GPU scratch array, each call smaller than the one before (so every
call also runs over the stale contents the previous one left)."""
import numpy as np
import pytest

import synth

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


def dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).to(DEV)


CALLS = [
    # two long rows: the two-stage selection (8 parts + merge), candidate lists in the scratch
    ("two rows of 600,000", [600_000, 599_000]),
    # the decode batch shape at a smaller length
    ("64 rows of 20,000", [20_000] * 64),
    # ragged short rows, -1 padding included
    ("ragged", [5, 2048, 2049, 9000]),
]


def test_noalloc_equals_workspace_entry_point_on_shrinking_calls():
    import dsa_indexer_top_key_amd as dsa
    for i, (name, s_len) in enumerate(CALLS):
        print(f"[noalloc] call {i}: {name}", flush=True)
        lay = synth.decode_layout(f"noalloc{i}", 90 + i, s_len)
        assert dsa.indexer_topk_workspace_size(lay.T, lay.max_s) <= dsa.NOALLOC_SCRATCH_BYTES
        d = synth.inputs_np(lay, parts=("index",))
        keys = synth.bf16_bits_from_f32(np.random.default_rng(90 + i).standard_normal((lay.N, 128)))
        args = (dev(d["q_idx"]), dev(d["w"]), dev(keys), dev(lay.kv_off), dev(lay.q_req),
                dev(lay.q_pos), lay.max_s)
        ids_ws = dsa.indexer_topk(*args)
        ids_na = torch.full((lay.T, 2048), 7, dtype=torch.int32, device=DEV)
        dsa.indexer_topk_noalloc(*args, ids=ids_na)
        torch.cuda.synchronize()
        assert torch.equal(ids_na, ids_ws), f"call {i} ({name})"
        n = np.minimum(lay.q_pos.astype(np.int64) + 1, lay.s_len[lay.q_req])
        got = ids_na.cpu().numpy()
        assert np.all((got >= 0).sum(axis=1) == np.minimum(n, 2048))


def test_noalloc_refuses_sizes_beyond_the_scratch():
    import dsa_indexer_top_key_amd as dsa
    lay = synth.decode_layout("noalloc_big", 95, [40_000] * 256)
    assert dsa.indexer_topk_workspace_size(lay.T, lay.max_s) > dsa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((lay.T, 32, 128), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((lay.T, 32), dtype=torch.bfloat16, device=DEV)
    keys = torch.zeros((8, 128), dtype=torch.bfloat16, device=DEV)  # never read: refused first
    with pytest.raises(dsa.DsaError, match="scratch"):
        dsa.indexer_topk_noalloc(q, w, keys, dev(lay.kv_off), dev(lay.q_req), dev(lay.q_pos),
                                 lay.max_s)
