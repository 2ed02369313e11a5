"""CPU oracle for the DeepSeek-Sparse-Attention read path of Kimi K3.1's global layers.

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, fp64 restatement of what the
path computes, written from the page "Kimi K3.1 Pro: Sparse-Zugriffe, keine kleinere
Historie" (flozi.net guide on the K3.1 DSA indexer and cache).  Only the test suite, the
package smoke check and the CPU-baseline leg of the benchmark may import it; the product
path (the HIP library and its Python binding) never does, and shares no code with it.

Every function works on numpy arrays in float64.  BF16 tensors arrive as their raw 16-bit
patterns (uint16) and are decoded here by this module's own codec.  A library primitive
(matmul, sort, exp) is used as a single step; nothing is blocked, fused or reordered.

Readings of the page where it is silent or garbled (its three display equations were lost
in extraction) are stated at each function; all of them are listed in the design notes.
Every function below is pinned by the CPU tests in tests/test_oracle_*.py against
closed forms, library routines, brute force or the page's printed arithmetic.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------
# Shapes fixed by the page (section "Was ändert sich – und was nicht?" and section
# "Der neue Indexer ..." paragraph): 32 indexer query heads of width 128, one shared
# 128-wide index key per stored position, a selection budget of 2048 positions, 96 main
# attention heads, KV latent rank 512 plus a 64-wide companion key component.
# ----------------------------------------------------------------------------------------
INDEX_HEADS = 32
INDEX_DIM = 128
TOPK = 2048
MLA_HEADS = 96
LATENT_DIM = 512
COMPANION_DIM = 64
QK_DIM = LATENT_DIM + COMPANION_DIM  # 576


# ----------------------------------------------------------------------------------------
# BF16 codec (the oracle's own; no code is shared with the input generators or the GPU).
# ----------------------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    """Decode raw bf16 bit patterns: a bf16 is the upper half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round float64 values to bf16 with round-to-nearest-even, in ONE rounding step.

    bf16 keeps 8 significant bits and binary32's exponent range.  For |x| with leading bit
    2^(e-1) the spacing of bf16 numbers is 2^(e-8), never below the subnormal spacing
    2^-133.  Scaling by a power of two is exact in float64, and numpy's round() breaks
    ties to even, so round(x / q) * q is the correctly rounded value.  Results at or
    above 2^128 overflow to infinity; NaN becomes the canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)
    q_exp = np.maximum(e - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.ldexp(np.round(np.ldexp(a, -q_exp)), q_exp)
        r = np.where(r >= 2.0 ** 128, np.inf, r)
        r = np.where(np.isinf(a), np.inf, r)
        bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)
    return bits


# ----------------------------------------------------------------------------------------
# Stage 1: index-key LayerNorm.
# Page section "Eine Query durch den Indexer verfolgen": a projection maps residual states
# to keys [S,128], followed by LayerNorm; the adapter paragraph after it fixes LayerNorm
# (not RMSNorm), FP32 key normalisation, no Hadamard transform and index_rope_dim = 0
# (no rotation of the keys).  Reading: biased variance, affine gamma/beta in fp32, an eps
# passed by the caller, result stored as bf16 (round to nearest even).
# ----------------------------------------------------------------------------------------
def layernorm64(x, gamma, beta, eps) -> np.ndarray:
    """LayerNorm of each 128-wide row of float64 x, evaluated in fp64 (gamma, beta and eps are
    taken at their fp32 values)."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float32).astype(np.float64)
    b = np.asarray(beta, dtype=np.float32).astype(np.float64)
    eps = float(np.float32(eps))
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def layernorm_keys(raw, gamma, beta, eps) -> np.ndarray:
    """Exact-as-fp64 LayerNorm of each 128-wide row of fp32 raw keys; returns float64 [N,128]."""
    return layernorm64(np.asarray(raw, dtype=np.float32).astype(np.float64), gamma, beta, eps)


def layernorm_error_scale(raw, gamma, beta, eps) -> np.ndarray:
    """Per element, the quantity whose multiple bounds the error of an fp32 evaluation of the
    key LayerNorm (page section "Eine Query durch den Indexer verfolgen", adapter paragraph:
    FP32 key normalisation):  |gamma| * A / sigma + |x_hat * gamma| * (1 + A / sigma) + |beta|,
    with A the row's mean absolute value and sigma = sqrt(var + eps).  To first order in the
    unit roundoff u: the rounded mean is off by a few u * A, which every x - mu carries and
    the division by sigma scales (first term); the variance, and so 1/sigma, inherits a
    relative error of a few u * (1 + A / sigma) from the same shift and its own sum (second
    term); the products and the final add cost a few u of the terms (all three).  Rows whose
    mean is large against their spread (A >> sigma) are where the first two terms matter."""
    x = np.asarray(raw)
    x = x.astype(np.float64) if x.dtype == np.float64 else x.astype(np.float32).astype(np.float64)
    g = np.asarray(gamma, dtype=np.float32).astype(np.float64)
    b = np.asarray(beta, dtype=np.float32).astype(np.float64)
    eps = float(np.float32(eps))
    mu = x.mean(axis=-1, keepdims=True)
    sigma = np.sqrt(((x - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    a_over_s = np.abs(x).mean(axis=-1, keepdims=True) / sigma
    return np.abs(g) * a_over_s + np.abs((x - mu) / sigma * g) * (1.0 + a_over_s) + np.abs(b)


def layernorm_keys_bf16(raw, gamma, beta, eps) -> np.ndarray:
    """Stage-1 output as stored in the index-key cache: bf16 bit patterns [N,128]."""
    return f64_to_bf16(layernorm_keys(raw, gamma, beta, eps))


# ----------------------------------------------------------------------------------------
# Admissible set.
# Page section "Eine Query durch den Indexer verfolgen": the scoring path picks up to 2048
# *causal* candidates per query.  Reading: a query at absolute position p in request b
# may see positions j <= p that exist in b's cache, i.e. j in [0, n_t) with
# n_t = min(p + 1, S_b).  The diagonal is admissible.
# ----------------------------------------------------------------------------------------
def admissible_count(q_pos: int, s_b: int) -> int:
    return int(max(0, min(int(q_pos) + 1, int(s_b))))


def request_lengths(kv_off) -> np.ndarray:
    off = np.asarray(kv_off, dtype=np.int64)
    return off[1:] - off[:-1]


# ----------------------------------------------------------------------------------------
# Stage 2: indexer scores.
# The page names the ingredients (32 heads x 128 queries [T,32,128], one shared key [S,128]
# per position, 32 head weights per query from the BF16 head-gate path); the combination
# is the weighted-ReLU sum  s_tj = sum_h w_th * max(0, q_th . k_j)  over admissible j.
# No further scale, softmax or rounding is applied: weights are used as given.
# ----------------------------------------------------------------------------------------
def indexer_scores_one(q_t, w_t, keys_rows) -> np.ndarray:
    """Scores of one query against a block of key rows (all float64 inputs).

    q_t: [H, D], w_t: [H], keys_rows: [n, D]  ->  [n]
    """
    logits = q_t @ keys_rows.T  # [H, n]
    return w_t @ np.maximum(logits, 0.0)


def indexer_scores(q_idx, w, keys, kv_off, q_req, q_pos, rows=None):
    """Scores of every query over its admissible positions.

    q_idx [T,H,D] bf16 bits, w [T,H] bf16 bits, keys [N,D] bf16 bits, kv_off [B+1] int64
    row offsets of each request's segment, q_req [T] request of each query, q_pos [T]
    absolute position of each query.  Returns a list of float64 arrays, one per query
    (or per query listed in `rows`), each of length n_t.
    """
    q_idx = np.asarray(q_idx)
    w = np.asarray(w)
    keys = np.asarray(keys)
    kv_off = np.asarray(kv_off, dtype=np.int64)
    s_len = request_lengths(kv_off)
    out = []
    for t in (range(q_idx.shape[0]) if rows is None else rows):
        b = int(q_req[t])
        n = admissible_count(q_pos[t], s_len[b])
        k_seg = keys[kv_off[b]: kv_off[b] + n]
        k_rows = bf16_to_f64(k_seg) if k_seg.dtype == np.uint16 else k_seg.astype(np.float64)
        out.append(indexer_scores_one(bf16_to_f64(q_idx[t]), bf16_to_f64(w[t]), k_rows))
    return out


def row_scale(scores_row) -> float:
    """Root-mean-square of a query's admissible scores (0 for an empty row)."""
    s = np.asarray(scores_row, dtype=np.float64)
    return float(np.sqrt(np.mean(s * s))) if s.size else 0.0


# ----------------------------------------------------------------------------------------
# Stage 3: top-k selection.
# Page section "Eine Query durch den Indexer verfolgen": up to 2048 causal candidates per
# query, a logical position-ID array [T,2048], invalid entries and short prefixes handled
# by the backend.  Section "Die Mathematik ...": I_t holds the up-to-2048 positions with
# the highest scores.  Readings (the page is silent): when n_t <= k every admissible
# position is selected; a tie at the k-th score goes to the lower position; -0 equals +0;
# NaN ranks below every number; a row lists its selected IDs in ascending position order
# followed by -1 entries up to k.
# ----------------------------------------------------------------------------------------
def topk_ids(scores_row, k: int = TOPK) -> np.ndarray:
    """Canonical top-k position IDs of one row of scores (float32 or float64)."""
    s = np.asarray(scores_row)
    n = int(s.shape[0])
    ids = np.full(k, -1, dtype=np.int32)
    if n <= k:
        ids[:n] = np.arange(n, dtype=np.int32)
        return ids
    nan = np.isnan(s)
    v = np.where(nan, 0.0, s.astype(np.float64)) + 0.0  # -0 + 0 = +0: one zero
    # np.lexsort sorts by the LAST key first: non-NaN first, then larger score, then
    # lower position.  The sort is a full sort of the row: the textbook definition.
    order = np.lexsort((np.arange(n), -v, nan))
    ids[:] = np.sort(order[:k]).astype(np.int32)
    return ids


def topk_rows(score_rows, k: int = TOPK) -> np.ndarray:
    return np.stack([topk_ids(r, k) for r in score_rows]) if len(score_rows) else \
        np.zeros((0, k), np.int32)


def kth_score(scores_row, k: int = TOPK):
    """The score of the k-th selected position (None when n_t <= k)."""
    s = np.asarray(scores_row, dtype=np.float64)
    if s.shape[0] <= k:
        return None
    ids = topk_ids(s, k)
    return float(np.min(s[ids]))


def selection_band(scores_row, k: int = TOPK, rel: float = 1e-3) -> np.ndarray:
    """Positions whose reference score lies within `rel` of the k-th score.

    Reading of the stated set tolerance: a GPU selection may differ from the oracle's only
    at positions j with |s_j - theta| <= rel * max(|theta|, r_t), where theta is the k-th
    score and r_t the row's RMS score (a floor for rows whose weighted heads cancel).
    """
    s = np.asarray(scores_row, dtype=np.float64)
    theta = kth_score(s, k)
    if theta is None:
        return np.zeros(0, dtype=np.int64)
    tol = rel * max(abs(theta), row_scale(s))
    return np.nonzero(np.abs(s - theta) <= tol)[0]


# ----------------------------------------------------------------------------------------
# Stage 4: absorbed-MLA read restricted to I_t.
# Section "Die Mathematik ...": the sparse read is a softmax restricted to I_t over the
# main-attention logits a_tj of each head (the display equation itself was lost).  The
# notation abstracts absorbed MLA projections: per-head K/V are not materialised; all 96
# heads read the one shared latent (section "Warum Top-2048 ..." last paragraphs, and the
# Gated-MLA paragraph: a 64-wide companion key component beside the 512-wide latent,
# skip_rope, no rotation).  Readings: a_tj = scale * q_th . [c_j ; kpe_j] over 576 dims,
# values are the 512-wide latent rows only, scale = 1/sqrt(192) is passed by the caller,
# lse = log sum exp a over I_t.  IDs < 0 or >= S_b are padding and are skipped; a row with
# no valid ID reads zero with lse = -inf.
# ----------------------------------------------------------------------------------------
def gather_rows(latent, kpe, row_index):
    """[n,576] float64 rows: latent[:, :512] next to kpe[:, :64] for absolute rows."""
    lat = bf16_to_f64(np.asarray(latent)[row_index, :LATENT_DIM])
    kp = bf16_to_f64(np.asarray(kpe)[row_index, :COMPANION_DIM])
    return np.concatenate([lat, kp], axis=1)


def restricted_softmax_read(q_t, rows576, scale):
    """One query, all heads: softmax over the given rows only, then read their latents.

    q_t [H,576] float64, rows576 [n,576] float64 -> (o [H,512], lse [H]).
    """
    h = q_t.shape[0]
    if rows576.shape[0] == 0:
        return np.zeros((h, LATENT_DIM)), np.full(h, -np.inf)
    a = scale * (q_t @ rows576.T)  # [H, n]
    m = a.max(axis=1, keepdims=True)
    p = np.exp(a - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ rows576[:, :LATENT_DIM]) / l
    return o, (m + np.log(l))[:, 0]


def valid_ids(ids_row, s_b):
    r = np.asarray(ids_row, dtype=np.int64)
    return r[(r >= 0) & (r < s_b)]


def sparse_mla(q, latent, kpe, kv_off, q_req, ids, scale, rows=None):
    """Stage 4 for every query (or the listed ones): returns (out [T,H,512], lse [T,H])."""
    q = np.asarray(q)
    kv_off = np.asarray(kv_off, dtype=np.int64)
    s_len = request_lengths(kv_off)
    sel = list(range(q.shape[0]) if rows is None else rows)
    out = np.zeros((len(sel), q.shape[1], LATENT_DIM))
    lse = np.zeros((len(sel), q.shape[1]))
    for i, t in enumerate(sel):
        b = int(q_req[t])
        j = valid_ids(ids[t], s_len[b])
        c = gather_rows(latent, kpe, kv_off[b] + j)
        out[i], lse[i] = restricted_softmax_read(bf16_to_f64(q[t]), c, scale)
    return out, lse


# ----------------------------------------------------------------------------------------
# Post-read epilogue (the row after stage 4).  Section "Was ändert sich – und was nicht?":
# 96 main-attention heads with 128-wide value heads; the read above stays in the shared
# 512-wide latent (absorbed MLA), so each head's value comes from its own up-projection of
# that read.  The paragraph after the Gated-MLA one: after the sparse attention and before
# the output projection a learned, coordinatewise sigmoid output gate is applied; the K3
# guide's MLA section adds that the gate is input-dependent and acts on the attention
# output.  Reading (the pages give no formula): per query t and head h
#   v_th = W_UV[h] o_th            (128 x 512 times 512)
#   u_th = v_th * sigmoid(g_th)    (elementwise over the 128 coordinates)
# with W_UV [96,128,512] the learned up-projection and g [T,96,128] the gate logits that an
# upstream projection of the token's hidden state produces (both inputs here).
# ----------------------------------------------------------------------------------------
def sigmoid(x) -> np.ndarray:
    """1 / (1 + exp(-x)) in float64, written in the form that does not overflow."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def value_gate(o, w_uv, gate) -> np.ndarray:
    """u [T,96,128] = (W_UV[h] o_th) * sigmoid(g_th); o is the read (bf16 bits or float),
    w_uv [96,128,512] and gate [T,96,128] are bf16 bits."""
    o = np.asarray(o)
    o64 = bf16_to_f64(o) if o.dtype == np.uint16 else o.astype(np.float64)
    w = bf16_to_f64(w_uv)
    g = bf16_to_f64(gate)
    v = np.einsum("hck,thk->thc", w, o64)  # one contraction per (t, h): W_UV[h] @ o_th
    return v * sigmoid(g)


def value_gate_magnitude(o, w_uv, gate) -> np.ndarray:
    """sum_k |W_UV[h,c,k] o_thk| * sigmoid(g_thc): the scale of the rounding error of any
    finite-precision evaluation of value_gate."""
    o = np.asarray(o)
    o64 = bf16_to_f64(o) if o.dtype == np.uint16 else o.astype(np.float64)
    return np.einsum("hck,thk->thc", np.abs(bf16_to_f64(w_uv)), np.abs(o64)) * sigmoid(bf16_to_f64(gate))


# ----------------------------------------------------------------------------------------
# Indexer-side projections (the steps before the key LayerNorm and the scoring).
# Section "Eine Query durch den Indexer verfolgen": the indexer projects the query latent to
# [T,32,128]; another projection maps residual states to [S,128] keys, followed by the key
# LayerNorm; a further one makes 32 head weights from each query's residual state.  Section
# "Was ändert sich – und was nicht?": query latent rank 1536, residual width 7168.  The
# adapter paragraph: FP32 key normalisation, BF16 head-gate path.
# Reading (the page gives no formula): plain linear maps, weights stored [out, in]; no bias,
# scale or activation; q_idx and w are rounded to bf16 once, the key is normalised from the
# exact projection and then rounded (as layernorm_keys_bf16 does for a given raw key).
# ----------------------------------------------------------------------------------------
def linear(x, weight) -> np.ndarray:
    """x [T, K] (bf16 bits or float) times weight [N, K] (bf16 bits) transposed -> [T, N] fp64."""
    x = np.asarray(x)
    x64 = bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    return x64 @ bf16_to_f64(weight).T


def linear_magnitude(x, weight) -> np.ndarray:
    """sum_k |x_tk w_nk|: the scale of the rounding error of any finite-precision evaluation."""
    x = np.asarray(x)
    x64 = bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    return np.abs(x64) @ np.abs(bf16_to_f64(weight)).T


def indexer_projections(c_q, h, w_qi, w_k, w_w, gamma, beta, eps) -> dict:
    """The indexer's inputs for T new tokens.

    c_q [T,1536] query latent and h [T,7168] residual states (bf16 bits); w_qi [4096,1536],
    w_k [128,7168], w_w [32,7168] (bf16 bits, [out, in]); gamma, beta [128] fp32.
    Returns q_idx [T,32,128] and w [T,32] as bf16 bits, the exact raw key k_raw [T,128]
    (fp64), its LayerNorm key [T,128] (fp64) and that key as bf16 bits (the cache rows)."""
    t = np.asarray(c_q).shape[0]
    q = linear(c_q, w_qi).reshape(t, INDEX_HEADS, INDEX_DIM)  # output j = 128 head + dim
    k_raw = linear(h, w_k)
    key = layernorm64(k_raw, gamma, beta, eps)
    return {"q_idx": f64_to_bf16(q), "w": f64_to_bf16(linear(h, w_w)), "k_raw": k_raw,
            "key": key, "key_bf16": f64_to_bf16(key)}


# ----------------------------------------------------------------------------------------
# Reduced-precision index-key cache.  Section "Warum Top-2048 keinen 2048-Token-Cache
# bedeutet": index quantisation and scale metadata change the physical cache; section "Was
# ein Deployment validieren muss": cache precision is an optional configuration and must not
# be presented as quality-preserving (no quality is claimed here).
# Reading: each key row is stored as 128 OCP FP8 E4M3 codes (1 sign, 4 exponent bits with bias
# 7, 3 mantissa bits, subnormals, no infinities, 448 the largest finite value) times one
# power-of-two scale 2^e per row, e the smallest exponent with max_d |k_d| <= 448 * 2^e (e = 0
# for an all-zero row).  Codes round k * 2^-e to nearest, ties to even.  Scores use the
# decoded keys code * 2^e in the same formula as indexer_scores.
# ----------------------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> float64 values (0x7F and 0xFF are NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def e4m3_encode(x) -> np.ndarray:
    """float32 values with |x| <= 448 -> OCP E4M3 codes, round to nearest, ties to even; the
    sign bit is kept (-0 -> 0x80).  Values below 2^-6 round to multiples of 2^-9 (subnormal
    codes; 8 * 2^-9 is the smallest normal, code 0x08)."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    sign = ((u >> 31) << 7).astype(np.uint8)
    a = np.abs(x)
    assert np.all(a <= E4M3_MAX)
    sub = np.rint(a.astype(np.float64) * 512.0).astype(np.int64)  # a < 2^-6: exact, then RNE
    ua = a.view(np.uint32).astype(np.int64)
    r = ua + 0x7FFFF + ((ua >> 20) & 1)  # round the fp32 mantissa to 3 bits, ties to even
    norm = ((((r >> 23) - 127 + 7) << 3) | ((r >> 20) & 7))
    mag = np.where(a < np.float32(2.0 ** -6), sub, norm)
    return (sign | mag.astype(np.uint8)).astype(np.uint8)


def key_scale_exponent(keys) -> np.ndarray:
    """Per row: the smallest e with max|k| <= 448 * 2^e (keys as bf16 bits or float)."""
    k = np.asarray(keys)
    k64 = bf16_to_f64(k) if k.dtype == np.uint16 else k.astype(np.float64)
    amax = np.abs(k64).max(axis=-1)
    f, x = np.frexp(amax)  # amax = f * 2^x, f in [0.5, 1)
    e = (x - 1) - 8 + (f > 0.875)
    return np.where(amax > 0, e, 0).astype(np.int32)


def quantize_keys_fp8(keys_bf16):
    """bf16 keys [N,128] -> (codes [N,128] uint8, scales [N] float32 = 2^e)."""
    k32 = bf16_to_f64(keys_bf16).astype(np.float32)
    e = key_scale_exponent(keys_bf16)
    scaled = np.ldexp(k32, -e[:, None]).astype(np.float32)  # exact: a power-of-two scaling
    return e4m3_encode(scaled), np.ldexp(np.float32(1.0), e).astype(np.float32)


def dequantize_keys_fp8(codes, scales) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def indexer_scores_fp8(q_idx, w, codes, scales, kv_off, q_req, q_pos, rows=None):
    """indexer_scores with the keys decoded from the FP8 cache."""
    return indexer_scores(q_idx, w, dequantize_keys_fp8(codes, scales), kv_off, q_req, q_pos,
                          rows=rows)


# ----------------------------------------------------------------------------------------
# Paged page-pool layout.  Section "Warum Top-2048 keinen 2048-Token-Cache bedeutet": page
# allocation changes the physical cache, not the logical positions the method works on.
# Reading: position p of request b lives in pool row page_table[b][p // P] * P + p % P; every
# stage computes on the logical (request-contiguous) rows, so the oracle unpages first.
# ----------------------------------------------------------------------------------------
def unpage_rows(pool, page_table, page_size, kv_off) -> np.ndarray:
    """Request-contiguous rows [sum S_b, ...] gathered from a page pool."""
    pool = np.asarray(pool)
    pt = np.asarray(page_table, dtype=np.int64)
    lens = request_lengths(kv_off)
    parts = []
    for b, n in enumerate(lens):
        p = np.arange(n, dtype=np.int64)
        parts.append(pool[pt[b, p // page_size] * page_size + p % page_size])
    return np.concatenate(parts) if parts else pool[:0]


# ----------------------------------------------------------------------------------------
# Dense reference and dropped mass (oracle only, never timed).
# Section "Die Mathematik ...": compared with a hypothetical full read at fixed logits and
# values, with eps the full softmax mass outside I_t, the retained and dropped reads are
# convex combinations of bounded values (the bound's display was lost).  Reading:
#   o_full = (1 - eps) o_sparse + eps o_drop   (exact identity)
#   |o_sparse - o_full|_c <= eps * (max_j v_jc - min_j v_jc)   per coordinate c
#   ||o_sparse - o_full|| <= eps * max_{i,j} ||v_i - v_j|| <= 2 eps max_j ||v_j||.
# ----------------------------------------------------------------------------------------
def dense_read(q, latent, kpe, kv_off, q_req, q_pos, ids, scale, rows=None):
    """Full causal read and the split into retained/dropped parts.

    Returns dict with o_full [T,H,512], eps [T,H], o_drop [T,H,512] (zeros where eps=0),
    v_range [T,512] (max - min of each latent coordinate over the admissible rows) and
    v_diam [T] (max pairwise distance of admissible latent rows, bounded by 2 max norm).
    """
    q = np.asarray(q)
    kv_off = np.asarray(kv_off, dtype=np.int64)
    s_len = request_lengths(kv_off)
    sel = list(range(q.shape[0]) if rows is None else rows)
    h = q.shape[1]
    res = {k: [] for k in ("o_full", "eps", "o_drop", "v_range", "v_maxnorm")}
    for t in sel:
        b = int(q_req[t])
        n = admissible_count(q_pos[t], s_len[b])
        c = gather_rows(latent, kpe, kv_off[b] + np.arange(n))
        if n == 0:
            res["o_full"].append(np.zeros((h, LATENT_DIM)))
            res["eps"].append(np.zeros(h))
            res["o_drop"].append(np.zeros((h, LATENT_DIM)))
            res["v_range"].append(np.zeros(LATENT_DIM))
            res["v_maxnorm"].append(0.0)
            continue
        a = scale * (bf16_to_f64(q[t]) @ c.T)
        pi = np.exp(a - a.max(axis=1, keepdims=True))
        pi /= pi.sum(axis=1, keepdims=True)
        v = c[:, :LATENT_DIM]
        in_i = np.zeros(n, dtype=bool)
        in_i[valid_ids(ids[t], n)] = True
        eps = pi[:, ~in_i].sum(axis=1)
        drop = pi[:, ~in_i] @ v[~in_i]
        o_drop = np.where(eps[:, None] > 0, drop / np.where(eps > 0, eps, 1.0)[:, None], 0.0)
        res["o_full"].append(pi @ v)
        res["eps"].append(eps)
        res["o_drop"].append(o_drop)
        res["v_range"].append(v.max(axis=0) - v.min(axis=0))
        res["v_maxnorm"].append(float(np.sqrt((v * v).sum(axis=1)).max()))
    return {k: np.asarray(x) for k, x in res.items()}


# ----------------------------------------------------------------------------------------
# Byte budget, section "Warum Top-2048 keinen 2048-Token-Cache bedeutet": per global layer
# and position a 512+64 element MLA representation plus a 128-element index key, all BF16,
# summed over the 24 global layers; and the selected fraction at the 1,048,576-token limit.
# ----------------------------------------------------------------------------------------
GLOBAL_LAYERS = 24
CONTEXT_LIMIT = 1_048_576


def payload_bytes_per_position_per_layer(elem_bytes: int = 2) -> int:
    return (LATENT_DIM + COMPANION_DIM + INDEX_DIM) * elem_bytes


def payload_bytes_per_token(layers: int = GLOBAL_LAYERS, elem_bytes: int = 2) -> int:
    return layers * payload_bytes_per_position_per_layer(elem_bytes)


def payload_bytes_at(tokens: int, layers: int = GLOBAL_LAYERS) -> int:
    return tokens * payload_bytes_per_token(layers)


def selection_fraction(k: int = TOPK, context: int = CONTEXT_LIMIT) -> float:
    return k / context

