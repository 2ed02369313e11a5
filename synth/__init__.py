"""Seeded synthetic inputs for the DSA read path.

This module only draws random numbers and lays them out; it contains none of the method's
arithmetic, so both the CPU oracle and the GPU library can be fed from it without
sharing code with each other.  Every array is seeded separately with
``seed = 1000 * workload_seed + tensor_id``:

    0 request lengths   1 index queries [T,32,128] bf16   2 head weights [T,32] bf16
    3 raw index keys [N,128] fp32 (bf16 for the long-context workload)
    4 LayerNorm gamma [128]   5 LayerNorm beta [128]   6 latent [N,512] (or [N,576])
    7 companion keys [N,64]   8 absorbed main queries [T,96,576] bf16
    10 value up-projection W_UV [96,128,512] bf16   11 output-gate logits [T,96,128] bf16
    12 a stand-in read o [T,96,512] bf16 (for the epilogue alone)
    13 query latent c_q [T,1536] bf16   14 residual states h [T,7168] bf16
    15 W_qi [4096,1536] bf16   16 W_k [128,7168] bf16   17 W_w [32,7168] bf16 (weights [out, in])

Distributions: index queries, raw keys, latents and main queries N(0,1); head weights
N(0, 1/32); gamma 1 + N(0, 0.1); beta N(0, 0.1); W_UV N(0, 1/512) (unit gain); gate logits
N(0, 1); stand-in reads N(0, 0.1) (a read is a convex combination of N(0,1) rows); query
latents and residual states N(0,1); W_qi N(0, 1/1536) and W_k N(0, 1/7168) (unit gain, so
projected queries are N(0,1) like the given ones); W_w N(0, 1/(32*7168)) (projected head
weights N(0, 1/32) like the given ones).  The second argument of N is read as
the variance.  BF16 values are rounded from float32 with round-to-nearest-even.

CPU generation uses numpy's PCG64; large workloads are generated on the GPU with torch's
seeded Philox generator (different numbers, same distributions); whichever side generated
an array, the other side receives a copy of the very same bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

INDEX_HEADS, INDEX_DIM = 32, 128
MLA_HEADS, QK_DIM, LATENT_DIM, COMPANION_DIM = 96, 576, 512, 64
TOPK = 2048
W_STD = (1.0 / 32.0) ** 0.5
AFFINE_STD = 0.1 ** 0.5
LN_EPS = 1e-6
ATTN_SCALE = 1.0 / 192.0 ** 0.5
VALUE_DIM = 128
WUV_STD = (1.0 / 512.0) ** 0.5
READ_STD = 0.1 ** 0.5
Q_LATENT, RESIDUAL = 1536, 7168
WQI_STD = (1.0 / Q_LATENT) ** 0.5
WK_STD = (1.0 / RESIDUAL) ** 0.5
WW_STD = (1.0 / (INDEX_HEADS * RESIDUAL)) ** 0.5


def bf16_bits_from_f32(x) -> np.ndarray:
    """Input preparation: float32 -> bf16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


@dataclass
class Layout:
    """Who is who: requests, their cache segments, and each query's request and position."""
    name: str
    seed: int
    s_len: np.ndarray            # [B] int64
    q_req: np.ndarray            # [T] int32
    q_pos: np.ndarray            # [T] int32
    raw_keys: bool = True        # fp32 raw keys + LayerNorm (else bf16 keys given)
    packed_latent: bool = False  # latent stored as [N,576] (companion in columns 512..575)
    note: str = ""
    kv_off: np.ndarray = field(init=False)

    def __post_init__(self):
        self.s_len = np.asarray(self.s_len, dtype=np.int64)
        self.q_req = np.asarray(self.q_req, dtype=np.int32)
        self.q_pos = np.asarray(self.q_pos, dtype=np.int32)
        self.kv_off = np.concatenate([[0], np.cumsum(self.s_len)]).astype(np.int64)

    @property
    def B(self) -> int:
        return int(self.s_len.shape[0])

    @property
    def T(self) -> int:
        return int(self.q_req.shape[0])

    @property
    def N(self) -> int:
        return int(self.kv_off[-1])

    @property
    def max_s(self) -> int:
        return int(self.s_len.max()) if self.B else 0


def decode_layout(name, seed, s_len, **kw) -> Layout:
    s = np.asarray(s_len, dtype=np.int64)
    return Layout(name, seed, s, np.arange(s.shape[0], dtype=np.int32),
                  (s - 1).astype(np.int32), **kw)


def prefill_layout(name, seed, s_total, first_pos, t, **kw) -> Layout:
    return Layout(name, seed, [s_total], np.zeros(t, np.int32),
                  first_pos + np.arange(t, dtype=np.int32), **kw)


def mixed_lengths(seed: int, b: int, lo: int, hi: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(1000 * seed + 0))
    return g.integers(lo, hi + 1, size=b).astype(np.int64)


def workload(name: str) -> Layout:
    """The five synthetic workloads (sizes as used by the tests and the benchmark)."""
    if name == "decode_b4_s4096":
        return decode_layout(name, 0, [4096] * 4)
    if name == "decode_b64_s32768":
        return decode_layout(name, 1, [32768] * 64)
    if name == "decode_b256_mixed":
        return decode_layout(name, 2, mixed_lengths(2, 256, 1, 8192))
    if name == "prefill_t4096_s65536":
        return prefill_layout(name, 3, 65536, 61440, 4096)
    if name == "long_decode_b4_s1m":
        return decode_layout(name, 4, [1 << 20] * 4, raw_keys=False, packed_latent=True)
    if name == "long_prefill_t8192_s1m":
        # the prefill chunk reads the same cache as request 0 of the long decode batch
        return prefill_layout(name, 4, 1 << 20, (1 << 20) - 8192, 8192,
                              raw_keys=False, packed_latent=True)
    raise KeyError(name)


WORKLOADS = ("decode_b4_s4096", "decode_b64_s32768", "decode_b256_mixed",
             "prefill_t4096_s65536", "long_decode_b4_s1m", "long_prefill_t8192_s1m")


# ---------------------------------------------------------------------------------------
# numpy (CPU) generation
# ---------------------------------------------------------------------------------------
def _normal(seed: int, tid: int, shape, std=1.0, mean=0.0) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(1000 * seed + tid))
    return mean + std * g.standard_normal(shape)


def inputs_np(lay: Layout, parts=("index", "ln", "mla")) -> dict:
    """All input tensors of a layout as numpy arrays (bf16 as uint16 bit patterns)."""
    t, n, s = lay.T, lay.N, lay.seed
    d = {"kv_off": lay.kv_off, "q_req": lay.q_req, "q_pos": lay.q_pos}
    if "index" in parts:
        d["q_idx"] = bf16_bits_from_f32(_normal(s, 1, (t, INDEX_HEADS, INDEX_DIM)))
        d["w"] = bf16_bits_from_f32(_normal(s, 2, (t, INDEX_HEADS), std=W_STD))
        if lay.raw_keys:
            d["raw_keys"] = _normal(s, 3, (n, INDEX_DIM)).astype(np.float32)
        else:
            d["keys"] = bf16_bits_from_f32(_normal(s, 3, (n, INDEX_DIM)))
    if "ln" in parts and lay.raw_keys:
        d["gamma"] = _normal(s, 4, (INDEX_DIM,), std=AFFINE_STD, mean=1.0).astype(np.float32)
        d["beta"] = _normal(s, 5, (INDEX_DIM,), std=AFFINE_STD).astype(np.float32)
    if "mla" in parts:
        if lay.packed_latent:
            packed = bf16_bits_from_f32(_normal(s, 6, (n, QK_DIM)))
            d["latent"] = packed
            d["kpe"] = packed[:, LATENT_DIM:]
        else:
            d["latent"] = bf16_bits_from_f32(_normal(s, 6, (n, LATENT_DIM)))
            d["kpe"] = bf16_bits_from_f32(_normal(s, 7, (n, COMPANION_DIM)))
        d["q"] = bf16_bits_from_f32(_normal(s, 8, (t, MLA_HEADS, QK_DIM)))
    if "gate" in parts:
        d["w_uv"] = bf16_bits_from_f32(_normal(s, 10, (MLA_HEADS, VALUE_DIM, LATENT_DIM), std=WUV_STD))
        d["gate"] = bf16_bits_from_f32(_normal(s, 11, (t, MLA_HEADS, VALUE_DIM)))
        d["o"] = bf16_bits_from_f32(_normal(s, 12, (t, MLA_HEADS, LATENT_DIM), std=READ_STD))
    if "proj" in parts:
        d["c_q"] = bf16_bits_from_f32(_normal(s, 13, (t, Q_LATENT)))
        d["h"] = bf16_bits_from_f32(_normal(s, 14, (t, RESIDUAL)))
        d["w_qi"] = bf16_bits_from_f32(_normal(s, 15, (INDEX_HEADS * INDEX_DIM, Q_LATENT), std=WQI_STD))
        d["w_k"] = bf16_bits_from_f32(_normal(s, 16, (INDEX_DIM, RESIDUAL), std=WK_STD))
        d["w_w"] = bf16_bits_from_f32(_normal(s, 17, (INDEX_HEADS, RESIDUAL), std=WW_STD))
        d["gamma"] = _normal(s, 4, (INDEX_DIM,), std=AFFINE_STD, mean=1.0).astype(np.float32)
        d["beta"] = _normal(s, 5, (INDEX_DIM,), std=AFFINE_STD).astype(np.float32)
    return d


def random_ids_np(seed: int, lay: Layout, k: int = TOPK) -> np.ndarray:
    """Seeded ID rows for stage-4 tests: a random causal subset per query, ascending,
    -1 padded (the shape of a top-k result without needing scores)."""
    g = np.random.Generator(np.random.PCG64(1000 * seed + 9))
    ids = np.full((lay.T, k), -1, np.int32)
    for t in range(lay.T):
        n = int(max(0, min(int(lay.q_pos[t]) + 1, int(lay.s_len[lay.q_req[t]]))))
        m = min(n, k)
        ids[t, :m] = np.sort(g.choice(n, size=m, replace=False)) if m else []
    return ids


# ---------------------------------------------------------------------------------------
# Score-array patterns for the stand-alone top-k (identical fp32 arrays on both sides)
# ---------------------------------------------------------------------------------------
def score_rows_np(seed: int, kind: str, rows: int, n: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(1000 * seed + 10))
    if kind == "gauss":
        x = g.standard_normal((rows, n)) * 8.0
    elif kind == "ints":          # many exact ties
        x = g.integers(-20, 21, size=(rows, n)).astype(np.float64)
    elif kind == "two_valued":
        x = np.where(g.random((rows, n)) < 0.5, 1.0, -1.0)
    elif kind == "all_equal":
        x = np.full((rows, n), 3.25)
    elif kind == "zeros_signed":  # +0 and -0 mixed with a few positives
        x = np.where(g.random((rows, n)) < 0.5, 0.0, -0.0)
        x[g.random((rows, n)) < 0.01] = 1.0
    elif kind == "special":       # +-inf, NaN, denormals, huge values
        x = g.standard_normal((rows, n))
        r = g.random((rows, n))
        x[r < 0.02] = np.inf
        x[(r >= 0.02) & (r < 0.04)] = -np.inf
        x[(r >= 0.04) & (r < 0.06)] = np.nan
        x[(r >= 0.06) & (r < 0.10)] = 1e-42
        x[(r >= 0.10) & (r < 0.12)] = -1e-42
        x[(r >= 0.12) & (r < 0.13)] = 3e38
    elif kind == "sorted_up":
        x = np.tile(np.arange(n, dtype=np.float64), (rows, 1))
    elif kind == "sorted_down":
        x = np.tile(np.arange(n, 0, -1, dtype=np.float64), (rows, 1))
    elif kind == "heavy_tail":
        x = g.standard_cauchy((rows, n))
    elif kind == "coarse":        # gaussian on a 1/64 grid: a handful of equal keys per value
        x = np.round(g.standard_normal((rows, n)) * 512.0) / 64.0
    else:
        raise KeyError(kind)
    return x.astype(np.float32)


# ---------------------------------------------------------------------------------------
# torch (GPU) generation for the large workloads
# ---------------------------------------------------------------------------------------
def inputs_torch(lay: Layout, device, parts=("index", "ln", "mla")) -> dict:
    """Same tensors as inputs_np, drawn on `device` with torch's seeded generator."""
    import torch

    def normal(tid, shape, std=1.0, mean=0.0, dtype=torch.bfloat16):
        g = torch.Generator(device=device)
        g.manual_seed(1000 * lay.seed + tid)
        x = torch.empty(shape, dtype=torch.float32, device=device)
        x.normal_(mean=mean, std=std, generator=g)
        return x if dtype == torch.float32 else x.to(dtype)

    t, n = lay.T, lay.N
    d = {"kv_off": torch.as_tensor(lay.kv_off, device=device),
         "q_req": torch.as_tensor(lay.q_req, device=device),
         "q_pos": torch.as_tensor(lay.q_pos, device=device)}
    if "index" in parts:
        d["q_idx"] = normal(1, (t, INDEX_HEADS, INDEX_DIM))
        d["w"] = normal(2, (t, INDEX_HEADS), std=W_STD)
        if lay.raw_keys:
            d["raw_keys"] = normal(3, (n, INDEX_DIM), dtype=torch.float32)
        else:
            d["keys"] = normal(3, (n, INDEX_DIM))
    if "ln" in parts and lay.raw_keys:
        d["gamma"] = normal(4, (INDEX_DIM,), std=AFFINE_STD, mean=1.0, dtype=torch.float32)
        d["beta"] = normal(5, (INDEX_DIM,), std=AFFINE_STD, dtype=torch.float32)
    if "mla" in parts:
        if lay.packed_latent:
            packed = normal(6, (n, QK_DIM))
            d["latent"] = packed
            d["kpe"] = packed[:, LATENT_DIM:]
        else:
            d["latent"] = normal(6, (n, LATENT_DIM))
            d["kpe"] = normal(7, (n, COMPANION_DIM))
        d["q"] = normal(8, (t, MLA_HEADS, QK_DIM))
    if "gate" in parts:
        d["w_uv"] = normal(10, (MLA_HEADS, VALUE_DIM, LATENT_DIM), std=WUV_STD)
        d["gate"] = normal(11, (t, MLA_HEADS, VALUE_DIM))
        d["o"] = normal(12, (t, MLA_HEADS, LATENT_DIM), std=READ_STD)
    if "proj" in parts:
        d["c_q"] = normal(13, (t, Q_LATENT))
        d["h"] = normal(14, (t, RESIDUAL))
        d["w_qi"] = normal(15, (INDEX_HEADS * INDEX_DIM, Q_LATENT), std=WQI_STD)
        d["w_k"] = normal(16, (INDEX_DIM, RESIDUAL), std=WK_STD)
        d["w_w"] = normal(17, (INDEX_HEADS, RESIDUAL), std=WW_STD)
        d["gamma"] = normal(4, (INDEX_DIM,), std=AFFINE_STD, mean=1.0, dtype=torch.float32)
        d["beta"] = normal(5, (INDEX_DIM,), std=AFFINE_STD, dtype=torch.float32)
    return d


def to_bits_np(x):
    """Host copy of a torch tensor; bf16 tensors become uint16 bit patterns."""
    import torch
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()
