"""The decode step (dsa_indexer_topk + dsa_sparse_mla_attn with caller-provided outputs and
workspaces) captured into a HIP graph: every replay equals the eager result bit for bit.

The entry points allocate nothing when the caller passes outputs and workspaces, and their
kernels record no memset, so the step can be captured as it is; replays run with eager work
(overwriting the outputs) and synchronisations in between.
"""
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dsa_indexer_top_key_amd as dsa
    dsa.library()
    return dsa


@pytest.mark.parametrize("name", ["decode_b256_mixed", "decode_b4_s4096"])
def test_decode_step_graph_replays_equal_eager(name):
    print(f"[graph] {name}", flush=True)
    import dsa_indexer_top_key_amd as dsa
    dev = torch.device("cuda:0")
    lay = synth.workload(name)
    d = synth.inputs_torch(lay, dev)
    keys = dsa.index_keys_layernorm(d["raw_keys"], d["gamma"], d["beta"], synth.LN_EPS)
    ids = torch.empty((lay.T, 2048), dtype=torch.int32, device=dev)
    ws_idx = torch.empty(max(dsa.indexer_topk_workspace_size(lay.T, lay.max_s), 256),
                         dtype=torch.uint8, device=dev)
    out = torch.empty((lay.T, 96, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((lay.T, 96), dtype=torch.float32, device=dev)
    ws_mla = torch.empty(max(dsa.sparse_mla_workspace_size(lay.T), 256), dtype=torch.uint8,
                         device=dev)

    def step():
        dsa.indexer_topk(d["q_idx"], d["w"], keys, d["kv_off"], d["q_req"], d["q_pos"],
                         lay.max_s, ids=ids, workspace=ws_idx)
        dsa.sparse_mla_attn(d["q"], d["latent"], d["kpe"], d["kv_off"], d["q_req"], ids,
                            synth.ATTN_SCALE, out=out, lse=lse, workspace=ws_mla)

    step()
    torch.cuda.synchronize()
    ref = (ids.clone(), out.view(torch.int16).clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for replay in range(3):
        ids.fill_(-7)
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ids, ref[0]), f"replay {replay}: ids"
        assert torch.equal(out.view(torch.int16), ref[1]), f"replay {replay}: out"
        assert torch.equal(lse, ref[2]), f"replay {replay}: lse"
