"""The algorithmic work the benchmark divides its measured times by, against counts worked out
by hand from the tensor shapes of the page's indexer and read (page "Kimi K3.1 Pro:
Sparse-Zugriffe, keine kleinere Historie", sections "Eine Query durch den Indexer verfolgen"
and "Die Mathematik der Sparse Attention und ihrer fehlenden Masse").

Unit sizes: an index key is 128 bf16 values (256 bytes); a query's indexer input is 32 heads x
128 bf16 plus 32 bf16 head weights (8,256 bytes); the selection writes 2048 int32 IDs (8,192
bytes); a selected position gathers its 512-wide latent and 64-wide companion key (1,152
bytes); the read takes 96 x 576 bf16 queries (110,592 bytes) and writes 96 x 512 bf16
(98,304 bytes).  A query at position p of a request with S cached positions scores
min(p + 1, S) positions and reads min(p + 1, S, 2048) of them.
"""
import bench
import synth


def test_headline_decode_step_bytes_and_flops():
    alg = bench.decode_alg(synth.workload("decode_b64_s32768"))
    assert alg["bytes_indexer"] == 537_399_296      # 64 x (32,768 x 256 + 8,256)
    assert alg["bytes_topk"] == 524_288             # 64 x 8,192
    assert alg["bytes_mla"] == 164_364_288          # 64 x (2,048 x 1,152 + 110,592 + 98,304)
    assert alg["bytes"] == 702_287_872
    assert alg["flops_indexer"] == 17_179_869_184   # 64 x 32,768 pairs x 8,192 flop (2^34)
    assert alg["flops_mla"] == 27_380_416_512       # 64 x 2,048 rows x 2 x 96 x 1,088


def test_fp8_key_cache_bytes():
    # 128 one-byte codes and a 4-byte scale per position instead of 256 bytes
    alg = bench.decode_alg(synth.workload("decode_b64_s32768"), key_bytes=132)
    assert alg["bytes_indexer"] == 277_352_448      # 64 x (32,768 x 132 + 8,256)
    assert alg["bytes"] == 442_241_024


def test_short_prefixes_and_positions_inside_a_request():
    # request 0: 100 positions (fewer than 2048 to select); request 1: 5,000 positions, read
    # at its last position and at position 10; the third query's prefix is 11 positions
    lay = synth.Layout("hand", 0, [100, 5000], [0, 1, 1], [99, 4999, 10])
    assert bench.n_admissible(lay).tolist() == [100, 5000, 11]
    alg = bench.decode_alg(lay)
    assert alg["bytes_indexer"] == 1_333_184        # 256 x 5,111 + 3 x 8,256
    assert alg["bytes_mla"] == 3_113_856            # 1,152 x (100 + 2,048 + 11) + 3 x 208,896
    assert alg["flops_indexer"] == 5111 * 8192
    assert alg["flops_mla"] == 2159 * 208_896


def test_position_beyond_the_request_is_clamped_to_its_length():
    lay = synth.Layout("hand", 0, [300], [0], [1000])
    assert bench.n_admissible(lay).tolist() == [300]


def test_prefill_chunk_causal_pairs():
    # queries at positions 61,440 .. 65,535 of one 65,536-position request: query t scores
    # 61,441 + t positions, 4,096 x 61,441 + 4,095 x 4,096 / 2 pairs in all (2.13 TFLOP)
    lay = synth.workload("prefill_t4096_s65536")
    pairs = int(bench.n_admissible(lay).sum())
    assert pairs == 260_048_896
    assert pairs * 2 * 32 * 128 == 2_130_320_556_032
    # the long chunk: positions 2^20 - 8,192 .. 2^20 - 1 of 2^20
    lay = synth.workload("long_prefill_t8192_s1m")
    assert int(bench.n_admissible(lay).sum()) == 8192 * 1_040_385 + 8191 * 8192 // 2


def test_projection_and_value_gate_bytes():
    # weights 4,096 x 1,536 + 128 x 7,168 + 32 x 7,168 bf16 once; per token 1,536 + 7,168 bf16
    # read and 4,096 + 32 + 128 bf16 written
    assert bench.proj_alg_bytes(64) == 14_876_672 + 1_114_112 + 544_768
    assert bench.proj_flops(4096) == 60_934_848_512
    # W_UV 96 x 128 x 512 bf16 once; per query 96 x 512 bf16 read and 96 x 128 bf16 gate logits
    # read and gated values written
    assert bench.value_gate_bytes(64) == 12_582_912 + 9_437_184


def test_per_position_bytes_match_the_pages_cache_budget():
    # The pages' budget: 33 KiB per token over the 24 global layers, i.e. 1,408 bytes per token
    # and layer = the 128-wide index key (scored at every admissible position) + the 512-wide
    # latent and 64-wide companion key (gathered at each selected position); at 2^20 tokens
    # the selection of 2048 is 1/512 of the history.
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")))
    per_layer = g["payload_per_token_KiB"] * 1024 // g["global_layers"]
    one = synth.Layout("one", 0, [1 << 20], [0], [(1 << 20) - 1])
    alg = bench.decode_alg(one)
    key_bytes = (alg["bytes_indexer"] - (32 * 128 + 32) * 2) // (1 << 20)
    row_bytes = (alg["bytes_mla"] - (96 * 576 + 96 * 512) * 2) // g["topk"]
    assert key_bytes + row_bytes == per_layer == 1408
    assert (1 << 20) // g["topk"] == g["selected_fraction_denominator"]
