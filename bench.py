"""Benchmark of the MI355X DSA read path (one GPU).

Headline: decode step = indexer scores + top-2048 (dsa_indexer_topk) followed by the
restricted-softmax absorbed-MLA read (dsa_sparse_mla_attn), on a batch of 64 requests with
32768 cached positions each (one query per request), inputs resident in HBM.  Also reported:
the prefill indexer (indexer + top-k) on a 4096-query chunk at positions 61440..65535 of a
65536-position request, in TFLOP/s of causal scoring work, the index-key LayerNorm
cache fill, and beside the step the two neighbouring steps of the layer: the indexer-side
projections (query latent / residual -> q_idx, LayerNorm key into its cache row, head
weights) for the decode batch (GB/s) and the prefill chunk (TFLOP/s), the post-read value
up-projection with its sigmoid gate, the decode step over the FP8 index-key cache variant
(E4M3 codes + one scale per key: 132 instead of 256 key bytes per position), and the decode
step over a paged page-pool cache (64-position pages in random pool order).  All timings use HIP events on the stream the kernels
run on.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill]
    python bench.py --profile-kernels   # a few launches of each kernel, for rocprofv3

Prints one JSON line (plus nothing else on stdout).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode queries/s + HBM GB/s at S=32K top-2048; prefill indexer TFLOP/s"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
DECODE_WORKLOAD = "decode_b64_s32768"
PREFILL_WORKLOAD = "prefill_t4096_s65536"
PROFILES = os.path.join(ROOT, "profiles")


# ---------------------------------------------------------------------------------------
# algorithmic work (what the method must move / compute; no intermediates)
# ---------------------------------------------------------------------------------------
def n_admissible(lay):
    return np.maximum(0, np.minimum(lay.q_pos.astype(np.int64) + 1, lay.s_len[lay.q_req]))


def decode_alg(lay, key_bytes=256):
    """Algorithmic bytes and flops of a decode step; key_bytes per cached index key (256 for
    the bf16 cache, 132 for 128 FP8 codes + a 4-byte scale)."""
    n = n_admissible(lay)
    sel = np.minimum(n, 2048)
    b_idx = key_bytes * n + 32 * 128 * 2 + 32 * 2    # keys, q_idx, w
    b_topk = 2048 * 4                               # IDs written
    b_mla = 1152 * sel + 96 * 576 * 2 + 96 * 512 * 2  # gathered rows, q, out
    f_idx = 2 * 32 * 128 * n
    f_mla = (2 * 96 * 576 + 2 * 96 * 512) * sel
    return {"bytes_indexer": int(b_idx.sum()), "bytes_topk": int(b_topk * lay.T),
            "bytes_mla": int(b_mla.sum()),
            "bytes": int((b_idx + b_topk + b_mla).sum()),
            "flops_indexer": int(f_idx.sum()), "flops_mla": int(f_mla.sum())}


def proj_alg_bytes(t):
    """Indexer-side projections of t tokens: the three weights once, the query latents and
    residual states read, q_idx, w and the cache rows written."""
    weights = (4096 * 1536 + 128 * 7168 + 32 * 7168) * 2
    return weights + t * (1536 + 7168) * 2 + t * (4096 + 32 + 128) * 2


def proj_flops(t):
    return 2 * t * (1536 * 4096 + 7168 * (128 + 32))


def source_digest(name):
    with open(os.path.join(ROOT, "dsa_indexer_top_key_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_file, summary_name):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken on
    the current source of the kernel (else None)."""
    path = os.path.join(PROFILES, summary_name)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != source_digest(kernel_file):
        return None
    return float(m_b.group(1))


# ---------------------------------------------------------------------------------------
def timed(fn, steps, warmup, stream, torch):
    """Run fn warmup times, then `steps` times bracketed by events; returns ms per call."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_call_events(fn, steps, stream, torch):
    """Average duration of each call, each bracketed by its own pair of events.  A short GPU
    spin queued first keeps the GPU behind the host while all calls are enqueued, so a call
    shorter than its host-side launch cost is still timed by the GPU alone."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    try:
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(2e6) * max(1, steps // 10))  # about 1 ms per 10 calls
    except (AttributeError, RuntimeError):
        pass
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def cpu_baseline(lay, host, n_total, budget_s=12.0):
    """The oracle (as it stands) on the first queries of the decode batch, cycled until about
    budget_s seconds of host work; queries/s of indexer scores + top-2048 + sparse read."""
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s or done < 2:
        t = done % lay.T
        s = O.indexer_scores(host["q_idx"], host["w"], host["keys"], lay.kv_off, lay.q_req,
                             lay.q_pos, rows=[t])
        ids = np.full((lay.T, 2048), -1, np.int32)
        ids[t] = O.topk_ids(s[0])
        O.sparse_mla(host["q"], host["latent"], host["kpe"], lay.kv_off, lay.q_req, ids,
                     1.0 / 192 ** 0.5, rows=[t])
        done += 1
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 2), "unit": "queries/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"the first {lay.T} of the {n_total} queries of {lay.name} (S=32768 each), "
                      f"cycled: {done} query evaluations (indexer scores + top-2048 + sparse "
                      f"read, fp64 numpy) in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="launch each kernel a few times (for rocprofv3), print nothing")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the DSA read path shards over requests with no "
              "exchange (see the design notes); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import dsa_indexer_top_key_amd as dsa
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------- decode workload
    lay = synth.workload(DECODE_WORKLOAD)
    d = synth.inputs_torch(lay, dev)
    keys = dsa.index_keys_layernorm(d["raw_keys"], d["gamma"], d["beta"], synth.LN_EPS)
    ids = torch.empty((lay.T, 2048), dtype=torch.int32, device=dev)
    ws_idx = torch.empty(dsa.indexer_topk_workspace_size(lay.T, lay.max_s), dtype=torch.uint8,
                         device=dev)
    out = torch.empty((lay.T, 96, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((lay.T, 96), dtype=torch.float32, device=dev)
    ws_mla_n = dsa.sparse_mla_workspace_size(lay.T)
    ws_mla = torch.empty(max(ws_mla_n, 256), dtype=torch.uint8, device=dev)
    idx_args = (d["q_idx"], d["w"], keys, d["kv_off"], d["q_req"], d["q_pos"], lay.max_s)
    scores = ws_idx.view(torch.float32)[: lay.T * lay.max_s].view(lay.T, lay.max_s)
    n_valid = torch.as_tensor(n_admissible(lay).astype(np.int32), device=dev)

    def step_indexer():
        dsa.indexer_topk(*idx_args, ids=ids, workspace=ws_idx)

    def step_mla():
        dsa.sparse_mla_attn(d["q"], d["latent"], d["kpe"], d["kv_off"], d["q_req"], ids,
                            synth.ATTN_SCALE, out=out, lse=lse, workspace=ws_mla)

    def step():
        step_indexer()
        step_mla()

    def scores_only():
        dsa.indexer_scores(*idx_args, scores=scores)

    def topk_only():
        dsa.topk(scores, n_valid, ids=ids)

    def ln_fill():
        dsa.index_keys_layernorm(d["raw_keys"], d["gamma"], d["beta"], synth.LN_EPS, keys=keys)

    # post-read epilogue (value up-projection + sigmoid gate) on the read of this batch;
    # measured beside the step, which covers the four stages of the read path
    dg = synth.inputs_torch(lay, dev, parts=("gate",))
    u_out = torch.empty((lay.T, 96, 128), dtype=torch.bfloat16, device=dev)

    def value_gate():
        dsa.value_gate(out, dg["w_uv"], dg["gate"], out=u_out)

    # indexer-side projections of the batch's new tokens (query latent -> q_idx, residual ->
    # key -> LayerNorm -> cache row, residual -> head weights); also measured beside the step
    dp = synth.inputs_torch(lay, dev, parts=("proj",))
    p_keys = torch.empty_like(keys)
    p_rows = d["kv_off"][1:] - 1  # each token's own position: the last row of its request
    p_q = torch.empty_like(d["q_idx"])
    p_w = torch.empty_like(d["w"])
    p_ws = torch.empty(dsa.indexer_project_workspace_size(lay.T), dtype=torch.uint8, device=dev)

    def project():
        dsa.indexer_project(dp["c_q"], dp["h"], dp["w_qi"], dp["w_k"], dp["w_w"], dp["gamma"],
                            dp["beta"], synth.LN_EPS, p_keys, p_rows, q_idx=p_q, w=p_w,
                            workspace=p_ws)

    # FP8 index-key cache variant (a reduced-precision cache option; no quality is claimed):
    # the same decode step with the keys read as E4M3 codes + one scale per key
    f8_codes, f8_scales = dsa.quantize_index_keys_fp8(keys)

    def quantize_fill():
        dsa.quantize_index_keys_fp8(keys, codes=f8_codes, scales=f8_scales)

    def step_fp8():
        dsa.indexer_topk_fp8(d["q_idx"], d["w"], f8_codes, f8_scales, d["kv_off"], d["q_req"],
                             d["q_pos"], lay.max_s, ids=ids, workspace=ws_idx)
        step_mla()

    def scores_fp8():
        dsa.indexer_scores_fp8(d["q_idx"], d["w"], f8_codes, f8_scales, d["kv_off"], d["q_req"],
                               d["q_pos"], lay.max_s, scores=scores)

    # paged page-pool layout: the same decode step with the keys, latent and companion rows in
    # 64-position pages of a pool in seeded random page order
    page = 64
    n_pages = -(-lay.s_len // page)
    perm = np.random.default_rng(7).permutation(int(n_pages.sum()))
    pt_np = np.zeros((lay.B, int(n_pages.max())), np.int32)
    row_of, k = [], 0
    for bq in range(lay.B):
        pt_np[bq, :n_pages[bq]] = perm[k:k + n_pages[bq]]
        k += n_pages[bq]
        pp = np.arange(lay.s_len[bq], dtype=np.int64)
        row_of.append(pt_np[bq, pp // page].astype(np.int64) * page + pp % page)
    rows_t = torch.as_tensor(np.concatenate(row_of), device=dev)
    pg_table = torch.as_tensor(pt_np, device=dev)
    pg_keys = torch.empty((len(perm) * page, 128), dtype=keys.dtype, device=dev)
    pg_keys[rows_t] = keys
    pg_lat = torch.empty((len(perm) * page, 512), dtype=d["latent"].dtype, device=dev)
    pg_lat[rows_t] = d["latent"]
    pg_kpe = torch.empty((len(perm) * page, 64), dtype=d["kpe"].dtype, device=dev)
    pg_kpe[rows_t] = d["kpe"]
    del rows_t

    def step_paged():
        dsa.indexer_topk_paged(d["q_idx"], d["w"], pg_keys, pg_table, page, d["kv_off"],
                               d["q_req"], d["q_pos"], lay.max_s, ids=ids, workspace=ws_idx)
        dsa.sparse_mla_attn_paged(d["q"], pg_lat, pg_kpe, pg_table, page, d["kv_off"], d["q_req"],
                                  ids, synth.ATTN_SCALE, out=out, lse=lse, workspace=ws_mla)

    if args.profile_kernels:
        for _ in range(10):
            step()
            scores_only()
            topk_only()
            ln_fill()
            value_gate()
            project()
            quantize_fill()
            step_fp8()
            step_paged()
        torch.cuda.synchronize()
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)  # copy kernel of known size (256 MiB read + 256 MiB written)
        if not args.no_prefill:
            play = synth.workload(PREFILL_WORKLOAD)
            pd = synth.inputs_torch(play, dev, parts=("index", "ln"))
            pkeys = dsa.index_keys_layernorm(pd["raw_keys"], pd["gamma"], pd["beta"], synth.LN_EPS)
            for _ in range(2):
                dsa.indexer_topk(pd["q_idx"], pd["w"], pkeys, pd["kv_off"], pd["q_req"],
                                 pd["q_pos"], play.max_s)
            pp = synth.inputs_torch(play, dev, parts=("proj",))
            for _ in range(2):
                dsa.indexer_project(pp["c_q"], pp["h"], pp["w_qi"], pp["w_k"], pp["w_w"],
                                    pp["gamma"], pp["beta"], synth.LN_EPS, pkeys,
                                    pd["q_pos"].to(torch.int64))
        torch.cuda.synchronize()
        return

    alg = decode_alg(lay)
    ms_step = timed(step, args.steps, args.warmup, stream, torch)
    ms_idx = per_call_events(step_indexer, args.steps, stream, torch)
    ms_mla = per_call_events(step_mla, args.steps, stream, torch)
    ms_scores = per_call_events(scores_only, args.steps, stream, torch)
    ms_topk = per_call_events(topk_only, args.steps, stream, torch)
    ms_ln = per_call_events(ln_fill, max(3, args.steps // 4), stream, torch)
    ms_vg = per_call_events(value_gate, args.steps, stream, torch)
    ms_pj = per_call_events(project, args.steps, stream, torch)
    pj_bytes = proj_alg_bytes(lay.T)
    ms_f8 = timed(step_fp8, args.steps, args.warmup, stream, torch)
    ms_f8_scores = per_call_events(scores_fp8, args.steps, stream, torch)
    ms_f8_fill = per_call_events(quantize_fill, max(3, args.steps // 4), stream, torch)
    alg8 = decode_alg(lay, key_bytes=132)
    ms_pg = timed(step_paged, args.steps, args.warmup, stream, torch)
    vg_bytes = 96 * 128 * 512 * 2 + lay.T * 96 * (512 + 2 * 128) * 2  # W_UV, o, gate, out
    vg_flops = 2 * lay.T * 96 * 128 * 512
    qps = lay.T / (ms_step * 1e-3)
    gbps = alg["bytes"] / (ms_step * 1e-3) / 1e9
    scores_gbps = alg["bytes_indexer"] / (ms_scores * 1e-3) / 1e9
    ln_bytes = lay.N * (512 + 256)
    traffic = measured_traffic("indexer.hip", "indexer_decode_b64_s32768_counters.txt")

    res = {
        "metric": METRIC, "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs of the stated shapes, generated on the GPU)",
        "config": {"workload": DECODE_WORKLOAD, "requests": lay.T, "cached_positions": 32768,
                   "topk": 2048, "index_heads": 32, "mla_heads": 96, "latent": 512,
                   "companion": 64},
        "hbm_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "alg_bytes_per_step": alg["bytes"],
        "stages_ms": {"indexer_topk": round(ms_idx, 5), "sparse_mla": round(ms_mla, 5),
                      "scores_kernel": round(ms_scores, 5), "topk_kernel": round(ms_topk, 5),
                      "ln_cache_fill": round(ms_ln, 5)},
        "ln_cache_fill_GBps": round(ln_bytes / (ms_ln * 1e-3) / 1e9, 1),
        "post_read_value_gate": {"ms": round(ms_vg, 5), "bytes": vg_bytes,
                                 "GBps": round(vg_bytes / (ms_vg * 1e-3) / 1e9, 1),
                                 "tflops": round(vg_flops / (ms_vg * 1e-3) / 1e12, 1)},
        "indexer_projections": {"ms": round(ms_pj, 5), "bytes": pj_bytes,
                                "GBps": round(pj_bytes / (ms_pj * 1e-3) / 1e9, 1),
                                "hbm_frac": round(pj_bytes / (ms_pj * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "fp8_index_key_cache": {
            "ms_per_step": round(ms_f8, 5), "queries_per_s": round(lay.T / (ms_f8 * 1e-3), 1),
            "alg_bytes_per_step": alg8["bytes"],
            "hbm_GBps": round(alg8["bytes"] / (ms_f8 * 1e-3) / 1e9, 1),
            "hbm_frac": round(alg8["bytes"] / (ms_f8 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "scores_kernel_ms": round(ms_f8_scores, 5),
            "scores_kernel_GBps": round(alg8["bytes_indexer"] / (ms_f8_scores * 1e-3) / 1e9, 1),
            "quantize_fill_ms": round(ms_f8_fill, 5),
            "quantize_fill_GBps": round(lay.N * (256 + 132) / (ms_f8_fill * 1e-3) / 1e9, 1)},
        "paged_cache": {
            "page_size": page, "ms_per_step": round(ms_pg, 5),
            "queries_per_s": round(lay.T / (ms_pg * 1e-3), 1),
            "hbm_GBps": round(alg["bytes"] / (ms_pg * 1e-3) / 1e9, 1),
            "hbm_frac": round(alg["bytes"] / (ms_pg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "sparse_mla_tflops": round(alg["flops_mla"] / (ms_mla * 1e-3) / 1e12, 1),
        "roofline": {"kernel": "indexer_decode_kernel", "bound": "hbm",
                     "achieved": round(scores_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(scores_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
    }

    # ------------------------------------------------------------- prefill indexer
    if not args.no_prefill:
        del scores
        play = synth.workload(PREFILL_WORKLOAD)
        pd = synth.inputs_torch(play, dev, parts=("index", "ln"))
        pkeys = dsa.index_keys_layernorm(pd["raw_keys"], pd["gamma"], pd["beta"], synth.LN_EPS)
        pids = torch.empty((play.T, 2048), dtype=torch.int32, device=dev)
        pws = torch.empty(dsa.indexer_topk_workspace_size(play.T, play.max_s),
                          dtype=torch.uint8, device=dev)
        pargs = (pd["q_idx"], pd["w"], pkeys, pd["kv_off"], pd["q_req"], pd["q_pos"], play.max_s)
        pscores = pws.view(torch.float32)[: play.T * play.max_s].view(play.T, play.max_s)

        def prefill():
            dsa.indexer_topk(*pargs, ids=pids, workspace=pws)

        def prefill_scores():
            dsa.indexer_scores(*pargs, scores=pscores)

        psteps = max(3, args.steps // 4)
        ms_pf = timed(prefill, psteps, 2, stream, torch)
        ms_pf_scores = per_call_events(prefill_scores, psteps, stream, torch)
        pflops = float((n_admissible(play) * 2 * 32 * 128).sum())
        res["prefill_indexer_tflops"] = round(pflops / (ms_pf * 1e-3) / 1e12, 1)
        res["prefill_indexer"] = {
            "workload": PREFILL_WORKLOAD, "ms": round(ms_pf, 4),
            "tflops_indexer_plus_topk": res["prefill_indexer_tflops"],
            "tflops_scores_kernel": round(pflops / (ms_pf_scores * 1e-3) / 1e12, 1),
            "mfma_frac": round(pflops / (ms_pf * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del pws, pscores
        # the chunk's indexer-side projections (4096 tokens: 60.9 GFLOP of bf16 products)
        pp = synth.inputs_torch(play, dev, parts=("proj",))
        pp_keys = torch.empty_like(pkeys)
        pp_rows = pd["q_pos"].to(torch.int64)

        def prefill_project():
            dsa.indexer_project(pp["c_q"], pp["h"], pp["w_qi"], pp["w_k"], pp["w_w"],
                                pp["gamma"], pp["beta"], synth.LN_EPS, pp_keys, pp_rows)

        ms_ppj = per_call_events(prefill_project, psteps, stream, torch)
        res["prefill_indexer_projections"] = {
            "ms": round(ms_ppj, 4),
            "tflops": round(proj_flops(play.T) / (ms_ppj * 1e-3) / 1e12, 1),
            "mfma_frac": round(proj_flops(play.T) / (ms_ppj * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    # ------------------------------------------------------------- oracle on the host
    if not args.no_cpu_baseline:
        from synth import to_bits_np
        sample_req = list(range(16))
        lo, hi = int(lay.kv_off[0]), int(lay.kv_off[len(sample_req)])
        host = {"q_idx": to_bits_np(d["q_idx"][: len(sample_req)]),
                "w": to_bits_np(d["w"][: len(sample_req)]),
                "q": to_bits_np(d["q"][: len(sample_req)]),
                "keys": to_bits_np(keys[lo:hi]),
                "latent": to_bits_np(d["latent"][lo:hi]), "kpe": to_bits_np(d["kpe"][lo:hi])}
        sub = synth.decode_layout(lay.name, lay.seed, lay.s_len[: len(sample_req)])
        res["cpu_baseline"] = cpu_baseline(sub, host, lay.T)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
