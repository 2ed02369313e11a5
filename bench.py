"""Benchmark of the MI355X DSA read path (one GPU).

Headline: the decode step = indexer scores + top-2048 (dsa_indexer_topk) followed by the
restricted-softmax absorbed-MLA read (dsa_sparse_mla_attn) on 64 requests with 32768 cached
positions each (one query per request), inputs resident in HBM, caches cold: before every
timed step, outside its events, a 1 GiB buffer is overwritten, which evicts the 256 MB
Infinity Cache and the L2s.  Each step is timed on its own (HIP events on the stream the
kernels run on); medians are reported with p10 and p90, and the same steps run back to back
without the flush are reported beside them as "warm".

Every synthetic workload is measured the same way (configs):
  decode_b4_s4096, decode_b64_s32768, decode_b256_mixed   decode steps: queries/s, GB/s of
                                                           algorithmic bytes, fraction of HBM
  prefill_t4096_s65536, long_prefill_t8192_s1m            prefill indexer (scores + top-k):
                                                           TFLOP/s of causal scoring work and
                                                           fraction of the BF16 MFMA peak; the
                                                           chunk's sparse read; the whole chunk
  long_decode_b4_s1m                                      decode step at 1,048,576 positions
with the index-key LayerNorm cache fill where keys arrive raw, and each workload's peak device
memory (its inputs, outputs and workspaces; the score workspace is stated on its own).

Beside the headline step, on the same batch: the decode step over the FP8 index-key cache and
over a paged page pool, the post-read value up-projection with its sigmoid gate, and the
indexer-side projections (decode batch and prefill chunk).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]
    python bench.py --profile-kernels [--workloads a,b]   # a few launches each, for rocprofv3

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
HEADLINE = "decode_b64_s32768"
DECODE_WORKLOADS = ("decode_b4_s4096", "decode_b64_s32768", "decode_b256_mixed",
                    "long_decode_b4_s1m")
PREFILL_WORKLOADS = ("prefill_t4096_s65536", "long_prefill_t8192_s1m")
PROFILES = os.path.join(ROOT, "profiles")
FLUSH_BYTES = 1 << 30
MIN_CONFIG_STEPS = 50


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


def value_gate_bytes(t):
    """Value up-projection + gate of t queries: W_UV once, o and the gate logits read, the gated
    values written."""
    return 96 * 128 * 512 * 2 + t * 96 * (512 + 2 * 128) * 2


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
# timing
# ---------------------------------------------------------------------------------------
class Clock:
    """Per-step HIP-event timing on the launch stream, cold (a 1 GiB overwrite before each
    step, outside its events) or warm (steps back to back); either way a GPU spin queued
    first keeps the GPU behind the host, so only GPU time falls between a step's events."""

    def __init__(self, torch, stream, dev):
        self.torch = torch
        self.stream = stream
        self.flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def _events(self, n):
        ev = self.torch.cuda.Event
        return [(ev(enable_timing=True), ev(enable_timing=True)) for _ in range(n)]

    def _spin(self, n):
        """A GPU spin queued ahead of n steps keeps the GPU behind the host while they are
        enqueued, so host launch cost never falls between a step's events."""
        try:
            with self.torch.cuda.stream(self.stream):
                self.torch.cuda._sleep(int(2e6) * max(1, n // 10))
        except (AttributeError, RuntimeError):
            pass

    def cold(self, fn, n, warmup=2):
        """Warmup steps are cold steps too (the overwrite, then the step), untimed."""
        torch = self.torch
        for i in range(warmup):
            self.flush_buf.fill_(i & 0x7F)
            fn()
        evs = self._events(n)
        torch.cuda.synchronize()
        self._spin(n)
        for i, (a, b) in enumerate(evs):
            self.flush_buf.fill_(i & 0x7F)  # 1 GiB written: the next step starts cold
            a.record(self.stream)
            fn()
            b.record(self.stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    def warm(self, fn, n, warmup=2):
        """Back to back, each step between its own events."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        evs = self._events(n)
        torch.cuda.synchronize()
        self._spin(n)
        for a, b in evs:
            a.record(self.stream)
            fn()
            b.record(self.stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])


def stats(ms):
    return {"ms_median": round(float(np.median(ms)), 5), "ms_p10": round(float(np.percentile(ms, 10)), 5),
            "ms_p90": round(float(np.percentile(ms, 90)), 5), "steps": int(len(ms))}


def rate(x, ms, scale=1e9):
    return round(x / (ms * 1e-3) / scale, 1)


# ---------------------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------------------
class DecodeStep:
    """Inputs, outputs and workspaces of one decode workload, and its step."""

    def __init__(self, dsa, synth, torch, name, dev):
        self.lay = lay = synth.workload(name)
        self.d = d = synth.inputs_torch(lay, dev)
        self.dsa, self.synth, self.torch = dsa, synth, torch
        if lay.raw_keys:
            self.keys = dsa.index_keys_layernorm(d["raw_keys"], d["gamma"], d["beta"], synth.LN_EPS)
        else:
            self.keys = d["keys"]
        self.ids = torch.empty((lay.T, 2048), dtype=torch.int32, device=dev)
        self.ws_bytes = dsa.indexer_topk_workspace_size(lay.T, lay.max_s)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty((lay.T, 96, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((lay.T, 96), dtype=torch.float32, device=dev)
        self.mla_ws_bytes = dsa.sparse_mla_workspace_size(lay.T)
        self.mla_ws = torch.empty(max(self.mla_ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.idx_args = (d["q_idx"], d["w"], self.keys, d["kv_off"], d["q_req"], d["q_pos"],
                         lay.max_s)

    def indexer(self):
        self.dsa.indexer_topk(*self.idx_args, ids=self.ids, workspace=self.ws)

    def read(self):
        d = self.d
        self.dsa.sparse_mla_attn(d["q"], d["latent"], d["kpe"], d["kv_off"], d["q_req"], self.ids,
                                 self.synth.ATTN_SCALE, out=self.out, lse=self.lse,
                                 workspace=self.mla_ws)

    def step(self):
        self.indexer()
        self.read()

    def ln_fill(self):
        d = self.d
        self.dsa.index_keys_layernorm(d["raw_keys"], d["gamma"], d["beta"], self.synth.LN_EPS,
                                      keys=self.keys)


def measure_decode(clock, ds, n, warm_too=True):
    lay = ds.lay
    alg = decode_alg(lay)
    cold = clock.cold(ds.step, n)
    res = {"workload": lay.name, "kind": "decode", "queries": lay.T,
           "cached_positions": int(lay.max_s) if len(set(lay.s_len.tolist())) == 1 else
           f"{int(lay.s_len.min())}..{int(lay.s_len.max())} (sum {int(lay.s_len.sum())})",
           "cold": stats(cold)}
    if warm_too:
        res["warm"] = stats(clock.warm(ds.step, n))
    med = res["cold"]["ms_median"]
    res.update({"queries_per_s": round(lay.T / (med * 1e-3), 1), "alg_bytes": alg["bytes"],
                "hbm_GBps": rate(alg["bytes"], med), "hbm_frac": round(alg["bytes"] / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "alg_flops": alg["flops_indexer"] + alg["flops_mla"],
                "tflops": rate(alg["flops_indexer"] + alg["flops_mla"], med, 1e12)})
    st_idx = np.median(clock.cold(ds.indexer, n))
    st_mla = np.median(clock.cold(ds.read, n))
    res["stages_cold_ms"] = {"indexer_topk": round(float(st_idx), 5), "sparse_mla": round(float(st_mla), 5)}
    res["stages_GBps"] = {"indexer_topk": rate(alg["bytes_indexer"] + alg["bytes_topk"], st_idx),
                          "sparse_mla": rate(alg["bytes_mla"], st_mla)}
    if lay.raw_keys:
        ms_ln = float(np.median(clock.cold(ds.ln_fill, max(5, n // 5))))
        res["ln_cache_fill"] = {"ms": round(ms_ln, 5), "rows": lay.N,
                                "GBps": rate(lay.N * (512 + 256), ms_ln)}
    res["score_workspace_bytes"] = int(ds.ws_bytes)
    res["split_workspace_bytes"] = int(ds.mla_ws_bytes)
    return res


class PrefillChunk:
    def __init__(self, dsa, synth, torch, name, dev):
        self.lay = lay = synth.workload(name)
        self.d = d = synth.inputs_torch(lay, dev)
        self.dsa, self.synth = dsa, synth
        if lay.raw_keys:
            self.keys = dsa.index_keys_layernorm(d["raw_keys"], d["gamma"], d["beta"], synth.LN_EPS)
        else:
            self.keys = d["keys"]
        self.ids = torch.empty((lay.T, 2048), dtype=torch.int32, device=dev)
        self.ws_bytes = dsa.indexer_topk_workspace_size(lay.T, lay.max_s)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty((lay.T, 96, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((lay.T, 96), dtype=torch.float32, device=dev)
        self.mla_ws_bytes = dsa.sparse_mla_workspace_size(lay.T)
        self.mla_ws = torch.empty(max(self.mla_ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.args = (d["q_idx"], d["w"], self.keys, d["kv_off"], d["q_req"], d["q_pos"], lay.max_s)
        self.scores = self.ws.view(torch.float32)[: lay.T * lay.max_s].view(lay.T, lay.max_s)

    def indexer(self):
        self.dsa.indexer_topk(*self.args, ids=self.ids, workspace=self.ws)

    def scores_only(self):
        self.dsa.indexer_scores(*self.args, scores=self.scores)

    def read(self):
        d = self.d
        self.dsa.sparse_mla_attn(d["q"], d["latent"], d["kpe"], d["kv_off"], d["q_req"], self.ids,
                                 self.synth.ATTN_SCALE, out=self.out, lse=self.lse,
                                 workspace=self.mla_ws)

    def step(self):
        self.indexer()
        self.read()

    def ln_fill(self):
        d = self.d
        self.dsa.index_keys_layernorm(d["raw_keys"], d["gamma"], d["beta"], self.synth.LN_EPS,
                                      keys=self.keys)


def measure_prefill(clock, pc, n):
    lay = pc.lay
    pairs = int(n_admissible(lay).sum())
    f_idx = pairs * 2 * 32 * 128
    sel = np.minimum(n_admissible(lay), 2048)
    f_mla = int(((2 * 96 * 576 + 2 * 96 * 512) * sel).sum())
    idx = clock.cold(pc.indexer, n)
    idx_warm = clock.warm(pc.indexer, n)
    sc = float(np.median(clock.cold(pc.scores_only, max(5, n // 5))))
    pc.indexer()  # the read below uses this chunk's own selection
    rd = clock.cold(pc.read, n)
    stp = clock.cold(pc.step, max(5, n // 5))
    m_idx, m_rd, m_stp = float(np.median(idx)), float(np.median(rd)), float(np.median(stp))
    res = {"workload": lay.name, "kind": "prefill", "queries": lay.T,
           "positions": f"{int(lay.q_pos[0])}..{int(lay.q_pos[-1])} of {int(lay.max_s)}",
           "causal_pairs": pairs,
           "indexer_topk": {"cold": stats(idx), "warm": stats(idx_warm),
                            "alg_flops": f_idx, "tflops": rate(f_idx, m_idx, 1e12),
                            "mfma_frac": round(f_idx / (m_idx * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
           "scores_kernel": {"ms_median": round(sc, 5), "tflops": rate(f_idx, sc, 1e12),
                             "mfma_frac": round(f_idx / (sc * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
           "sparse_read": {"cold": stats(rd), "alg_flops": f_mla, "tflops": rate(f_mla, m_rd, 1e12),
                           "mfma_frac": round(f_mla / (m_rd * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                           "gathered_bytes": int((1152 * sel).sum())},
           "chunk": {"cold": stats(stp), "queries_per_s": round(lay.T / (m_stp * 1e-3), 1)}}
    if lay.raw_keys:
        ms_ln = float(np.median(clock.cold(pc.ln_fill, 5)))
        res["ln_cache_fill"] = {"ms": round(ms_ln, 5), "rows": lay.N,
                                "GBps": rate(lay.N * (512 + 256), ms_ln)}
    res["score_workspace_bytes"] = int(pc.ws_bytes)
    return res


def with_peak_memory(torch, fn):
    """Run fn() and add the device memory the workload itself held at its peak (bytes above
    what was allocated before it started: its inputs, outputs and workspaces)."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    res = fn()
    torch.cuda.synchronize()
    res["peak_device_bytes"] = int(torch.cuda.max_memory_allocated() - base)
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------------------
# beside the headline step: cache variants and the neighbouring steps of the layer
# ---------------------------------------------------------------------------------------
def measure_variants(clock, ds, dsa, synth, torch, dev, n, quick):
    lay, d = ds.lay, ds.d
    out = {}
    # FP8 index-key cache (a reduced-precision option; no quality is claimed)
    codes, scales = dsa.quantize_index_keys_fp8(ds.keys)

    def step_fp8():
        dsa.indexer_topk_fp8(d["q_idx"], d["w"], codes, scales, d["kv_off"], d["q_req"],
                             d["q_pos"], lay.max_s, ids=ds.ids, workspace=ds.ws)
        ds.read()

    def fill_fp8():
        dsa.quantize_index_keys_fp8(ds.keys, codes=codes, scales=scales)

    alg8 = decode_alg(lay, key_bytes=132)
    m8 = float(np.median(clock.cold(step_fp8, n)))
    mq = float(np.median(clock.cold(fill_fp8, max(5, n // 5))))
    out["fp8_index_key_cache"] = {
        "step_cold_ms": round(m8, 5), "queries_per_s": round(lay.T / (m8 * 1e-3), 1),
        "alg_bytes": alg8["bytes"], "hbm_GBps": rate(alg8["bytes"], m8),
        "hbm_frac": round(alg8["bytes"] / (m8 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "quantize_fill_ms": round(mq, 5), "quantize_fill_GBps": rate(lay.N * (256 + 132), mq)}
    del codes, scales
    # paged page pool: 64-position pages in seeded random pool order
    if not quick:
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
        pools = {}
        for key, src in (("keys", ds.keys), ("latent", d["latent"]), ("kpe", d["kpe"])):
            pools[key] = torch.empty((len(perm) * page, src.shape[1]), dtype=src.dtype, device=dev)
            pools[key][rows_t] = src
        del rows_t

        def step_paged():
            dsa.indexer_topk_paged(d["q_idx"], d["w"], pools["keys"], pg_table, page, d["kv_off"],
                                   d["q_req"], d["q_pos"], lay.max_s, ids=ds.ids, workspace=ds.ws)
            dsa.sparse_mla_attn_paged(d["q"], pools["latent"], pools["kpe"], pg_table, page,
                                      d["kv_off"], d["q_req"], ds.ids, synth.ATTN_SCALE,
                                      out=ds.out, lse=ds.lse, workspace=ds.mla_ws)

        alg = decode_alg(lay)
        mp = float(np.median(clock.cold(step_paged, n)))
        out["paged_cache"] = {"page_size": page, "step_cold_ms": round(mp, 5),
                              "queries_per_s": round(lay.T / (mp * 1e-3), 1),
                              "hbm_GBps": rate(alg["bytes"], mp),
                              "hbm_frac": round(alg["bytes"] / (mp * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del pools, pg_table
    # post-read value up-projection + sigmoid gate on this batch's read
    dg = synth.inputs_torch(lay, dev, parts=("gate",))
    u_out = torch.empty((lay.T, 96, 128), dtype=torch.bfloat16, device=dev)

    def value_gate():
        dsa.value_gate(ds.out, dg["w_uv"], dg["gate"], out=u_out)

    vg_bytes = value_gate_bytes(lay.T)
    mv = float(np.median(clock.cold(value_gate, n)))
    out["post_read_value_gate"] = {"ms": round(mv, 5), "bytes": vg_bytes, "GBps": rate(vg_bytes, mv),
                                   "hbm_frac": round(vg_bytes / (mv * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    # indexer-side projections of the batch's new tokens
    dp = synth.inputs_torch(lay, dev, parts=("proj",))
    p_keys = torch.empty_like(ds.keys)
    p_rows = d["kv_off"][1:] - 1
    p_q, p_w = torch.empty_like(d["q_idx"]), torch.empty_like(d["w"])
    p_ws = torch.empty(dsa.indexer_project_workspace_size(lay.T), dtype=torch.uint8, device=dev)

    def project():
        dsa.indexer_project(dp["c_q"], dp["h"], dp["w_qi"], dp["w_k"], dp["w_w"], dp["gamma"],
                            dp["beta"], synth.LN_EPS, p_keys, p_rows, q_idx=p_q, w=p_w,
                            workspace=p_ws)

    pj_bytes = proj_alg_bytes(lay.T)
    mj = float(np.median(clock.cold(project, n)))
    out["indexer_projections"] = {"tokens": lay.T, "ms": round(mj, 5), "bytes": pj_bytes,
                                  "GBps": rate(pj_bytes, mj),
                                  "hbm_frac": round(pj_bytes / (mj * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    return out


def measure_prefill_projections(clock, dsa, synth, torch, dev, n):
    lay = synth.workload("prefill_t4096_s65536")
    pp = synth.inputs_torch(lay, dev, parts=("proj",))
    keys = torch.empty((lay.N, 128), dtype=torch.bfloat16, device=dev)
    rows = torch.as_tensor(lay.q_pos.astype(np.int64), device=dev)
    ws = torch.empty(dsa.indexer_project_workspace_size(lay.T), dtype=torch.uint8, device=dev)

    def project():
        dsa.indexer_project(pp["c_q"], pp["h"], pp["w_qi"], pp["w_k"], pp["w_w"], pp["gamma"],
                            pp["beta"], synth.LN_EPS, keys, rows, workspace=ws)

    m = float(np.median(clock.cold(project, n)))
    f = proj_flops(lay.T)
    return {"tokens": lay.T, "ms": round(m, 4), "tflops": rate(f, m, 1e12),
            "mfma_frac": round(f / (m * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}


# ---------------------------------------------------------------------------------------
# the oracle on the host
# ---------------------------------------------------------------------------------------
def host_cpu():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return model, n


def cpu_baseline(lay, host, n_total, budget_s=12.0):
    """The oracle (as it stands) on the first queries of the decode batch, cycled until about
    budget_s seconds of host work; queries/s of indexer scores + top-2048 + sparse read."""
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    model, n_cpu = host_cpu()
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
    return {"value": round(done / dt, 2), "unit": "queries/s", "cores": int(blas),
            "kind": "oracle", "host_cpus": n_cpu, "cpu_model": model,
            "sample": f"the first {lay.T} of the {n_total} queries of {lay.name} (S=32768 each), "
                      f"cycled: {done} query evaluations (indexer scores + top-2048 + sparse "
                      f"read, fp64 numpy; the products run on {blas} BLAS threads, the rest on "
                      f"one) in {dt:.1f} s"}


# ---------------------------------------------------------------------------------------
def profile_f_rows(dsa, synth, torch, dev, ds, cold):
    """Cold launches of the post-read value gate and the 64-token projections on the decode
    batch (the inputs of measure_variants)."""
    lay = ds.lay
    dg = synth.inputs_torch(lay, dev, parts=("gate",))
    u_out = torch.empty((lay.T, 96, 128), dtype=torch.bfloat16, device=dev)
    cold(lambda: dsa.value_gate(ds.out, dg["w_uv"], dg["gate"], out=u_out), 5)
    dp = synth.inputs_torch(lay, dev, parts=("proj",))
    p_keys = torch.empty_like(ds.keys)
    p_rows = torch.as_tensor((lay.kv_off[1:] - 1).astype(np.int64), device=dev)
    p_ws = torch.empty(dsa.indexer_project_workspace_size(lay.T), dtype=torch.uint8, device=dev)
    cold(lambda: dsa.indexer_project(dp["c_q"], dp["h"], dp["w_qi"], dp["w_k"], dp["w_w"],
                                     dp["gamma"], dp["beta"], synth.LN_EPS, p_keys, p_rows,
                                     workspace=p_ws), 5)


def profile_prefill_projections(dsa, synth, torch, dev, cold):
    """Cold launches of the projections of the 4096-token chunk."""
    lay = synth.workload("prefill_t4096_s65536")
    pp = synth.inputs_torch(lay, dev, parts=("proj",))
    keys = torch.empty((lay.N, 128), dtype=torch.bfloat16, device=dev)
    rows = torch.as_tensor(lay.q_pos.astype(np.int64), device=dev)
    ws = torch.empty(dsa.indexer_project_workspace_size(lay.T), dtype=torch.uint8, device=dev)
    cold(lambda: dsa.indexer_project(pp["c_q"], pp["h"], pp["w_qi"], pp["w_k"], pp["w_w"],
                                     pp["gamma"], pp["beta"], synth.LN_EPS, keys, rows,
                                     workspace=ws), 3)


def profile_kernels(dsa, synth, torch, dev, names):
    """A few cold launches of every kernel of the named workloads (for rocprofv3): each launch
    follows the 1 GiB overwrite the timed steps use, so traced durations are comparable with
    the cold medians.  Ends with a device copy of known size (the counter calibration)."""
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    def cold(fn, reps):
        for i in range(reps):
            flush.fill_(i & 0x7F)
            fn()

    for name in names:
        if name in DECODE_WORKLOADS:
            ds = DecodeStep(dsa, synth, torch, name, dev)
            scores = ds.ws.view(torch.float32)[: ds.lay.T * ds.lay.max_s].view(ds.lay.T, ds.lay.max_s)
            n_valid = torch.as_tensor(n_admissible(ds.lay).astype(np.int32), device=dev)
            cold(ds.step, 5)
            cold(lambda: dsa.indexer_scores(*ds.idx_args, scores=scores), 5)
            cold(lambda: dsa.topk(scores, n_valid, ids=ds.ids), 5)
            if ds.lay.raw_keys:
                cold(ds.ln_fill, 3)
            if name == "decode_b64_s32768":
                profile_f_rows(dsa, synth, torch, dev, ds, cold)
            del ds, scores, n_valid
        else:
            pc = PrefillChunk(dsa, synth, torch, name, dev)
            cold(pc.step, 2)
            cold(pc.scores_only, 2)
            del pc
            if name == "prefill_t4096_s65536":
                profile_prefill_projections(dsa, synth, torch, dev, cold)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    del flush
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)  # copy kernel of known size (256 MiB read + 256 MiB written)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first 40 or so cold steps of a fresh process run about 3% slower than the steady
    # state (medians of steps 1-20, 21-40 and 41-80 after 5 warmup steps: 167, 164 and 162 us
    # on the decode batch), so the untimed warmup covers them
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="headline and the decode batch only (no other workloads or variants)")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="launch each kernel a few times (for rocprofv3), print nothing")
    ap.add_argument("--workloads", default=",".join(DECODE_WORKLOADS[:3] + PREFILL_WORKLOADS[:1]
                                                   + ("long_decode_b4_s1m", "long_prefill_t8192_s1m")))
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
    names = [w for w in args.workloads.split(",") if w]

    if args.profile_kernels:
        profile_kernels(dsa, synth, torch, dev, names)
        return

    clock = Clock(torch, stream, dev)
    n_cfg = max(args.steps, MIN_CONFIG_STEPS)

    # ------------------------------------------------------------- headline: exactly K steps
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ds = DecodeStep(dsa, synth, torch, HEADLINE, dev)
    lay = ds.lay
    alg = decode_alg(lay)
    head = clock.cold(ds.step, args.steps, warmup=args.warmup)
    ms_step = float(np.median(head))
    # dominant kernel: the scoring stream, average launch duration (cold)
    scores = ds.ws.view(torch.float32)[: lay.T * lay.max_s].view(lay.T, lay.max_s)

    def scores_only():
        dsa.indexer_scores(*ds.idx_args, scores=scores)

    ms_scores = float(np.mean(clock.cold(scores_only, n_cfg)))
    scores_gbps = alg["bytes_indexer"] / (ms_scores * 1e-3) / 1e9
    n_valid = torch.as_tensor(n_admissible(lay).astype(np.int32), device=dev)

    def topk_only():
        dsa.topk(scores, n_valid, ids=ds.ids)

    ms_topk = float(np.median(clock.cold(topk_only, n_cfg)))
    res = {
        "metric": METRIC, "value": round(lay.T / (ms_step * 1e-3), 1), "unit": "queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs of the stated shapes, generated on the GPU)",
        "config": {"workload": HEADLINE, "requests": lay.T, "cached_positions": 32768,
                   "topk": 2048, "index_heads": 32, "mla_heads": 96, "latent": 512,
                   "companion": 64},
        "timing": ("each step timed alone (HIP events on the launch stream), caches cold: a 1 GiB "
                   "overwrite before every step, outside its events; value and ms_per_step are "
                   "the median of the K timed steps"),
        "ms_p10": round(float(np.percentile(head, 10)), 5),
        "ms_p90": round(float(np.percentile(head, 90)), 5),
        "hbm_GBps": rate(alg["bytes"], ms_step),
        "hbm_frac": round(alg["bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "alg_bytes_per_step": alg["bytes"],
        "roofline": {"kernel": "indexer_decode_kernel", "bound": "hbm",
                     "achieved": round(scores_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(scores_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("indexer.hip", "indexer_decode_b64_s32768_counters.txt"),
                     "alg_bytes_per_launch": alg["bytes_indexer"],
                     "avg_launch_ms": round(ms_scores, 5)},
        "kernels_cold_ms": {"indexer_decode_kernel_avg": round(ms_scores, 5),
                            "topk_kernel_median": round(ms_topk, 5)},
    }

    # ------------------------------------------------------------- every workload
    configs = {}
    configs[HEADLINE] = measure_decode(clock, ds, n_cfg)
    torch.cuda.synchronize()
    configs[HEADLINE]["peak_device_bytes"] = int(torch.cuda.max_memory_allocated() - base)
    res.update(measure_variants(clock, ds, dsa, synth, torch, dev, n_cfg, args.quick))
    del ds, scores, n_valid
    torch.cuda.empty_cache()
    if not args.quick:
        for name in names:
            if name == HEADLINE:
                continue
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            if name in DECODE_WORKLOADS:
                configs[name] = with_peak_memory(
                    torch, lambda: measure_decode(clock, DecodeStep(dsa, synth, torch, name, dev), n_cfg))
            else:
                configs[name] = with_peak_memory(
                    torch, lambda: measure_prefill(clock, PrefillChunk(dsa, synth, torch, name, dev), n_cfg))
        res["prefill_indexer_projections"] = measure_prefill_projections(clock, dsa, synth, torch, dev, n_cfg)
    res["configs"] = configs
    if "prefill_t4096_s65536" in configs:
        p = configs["prefill_t4096_s65536"]["indexer_topk"]
        res["prefill_indexer_tflops"] = p["tflops"]
        res["prefill_indexer_mfma_frac"] = p["mfma_frac"]

    # ------------------------------------------------------------- oracle on the host
    if not args.no_cpu_baseline:
        from synth import to_bits_np
        lay = synth.workload(HEADLINE)
        d = synth.inputs_torch(lay, dev, parts=("index", "ln", "mla"))
        keys = dsa.index_keys_layernorm(d["raw_keys"][: 16 * 32768], d["gamma"], d["beta"], synth.LN_EPS)
        sample_req = list(range(16))
        lo, hi = int(lay.kv_off[0]), int(lay.kv_off[len(sample_req)])
        host = {"q_idx": to_bits_np(d["q_idx"][: len(sample_req)]),
                "w": to_bits_np(d["w"][: len(sample_req)]),
                "q": to_bits_np(d["q"][: len(sample_req)]),
                "keys": to_bits_np(keys[lo:hi]),
                "latent": to_bits_np(d["latent"][lo:hi]), "kpe": to_bits_np(d["kpe"][lo:hi])}
        del d, keys
        sub = synth.decode_layout(lay.name, lay.seed, lay.s_len[: len(sample_req)])
        res["cpu_baseline"] = cpu_baseline(sub, host, lay.T)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
