"""MI355X (gfx950) DeepSeek-Sparse-Attention read path of Kimi K3.1's global layers.

Thin Python binding over the C ABI in include/dsa.h (libdsa_amd.so, built in-tree by
dsa_indexer_top_key_amd.build).  This module only marshals arguments: every step of the
path runs in the HIP kernels.  Tensors are torch tensors on the GPU (torch provides device
memory and streams); bf16 tensors may be torch.bfloat16 or int16/uint16 bit patterns.
There is no CPU or PyTorch fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["DsaError", "library", "index_keys_layernorm", "indexer_scores", "topk", "value_gate",
           "indexer_project", "indexer_project_workspace_size", "Q_LATENT", "RESIDUAL",
           "quantize_index_keys_fp8", "indexer_scores_fp8", "indexer_topk_fp8",
           "indexer_topk_paged", "sparse_mla_attn_paged",
           "indexer_topk", "indexer_topk_workspace_size", "sparse_mla_attn",
           "sparse_mla_workspace_size", "INDEX_HEADS", "INDEX_DIM", "TOPK", "MLA_HEADS",
           "LATENT_DIM", "COMPANION_DIM", "VALUE_DIM"]

INDEX_HEADS, INDEX_DIM, TOPK = 32, 128, 2048
MLA_HEADS, LATENT_DIM, COMPANION_DIM, VALUE_DIM = 96, 512, 64, 128
QK_DIM = LATENT_DIM + COMPANION_DIM
Q_LATENT, RESIDUAL = 1536, 7168

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa_amd.so")

_STATUS = {0: "DSA_OK", 1: "DSA_ERR_INVALID_ARG", 2: "DSA_ERR_UNSUPPORTED",
           3: "DSA_ERR_WORKSPACE", 4: "DSA_ERR_HIP"}


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_f32 = ctypes.c_float

_SIGNATURES = {
    "dsa_abi_version": ([], ctypes.c_int),
    "dsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "dsa_last_error": ([], ctypes.c_char_p),
    "dsa_index_keys_layernorm": ([_p, _p, _p, _f32, _p, _i64, _p], ctypes.c_int),
    "dsa_indexer_scores": ([_p, _p, _p, _p, _p, _p, _i32, _i32, _i64, _i32, _i32, _p, _i64, _p],
                           ctypes.c_int),
    "dsa_topk": ([_p, _i64, _p, _i32, _i64, _i32, _p, _p], ctypes.c_int),
    "dsa_indexer_topk_workspace_size": ([_i32, _i64], _sz),
    "dsa_indexer_topk": ([_p, _p, _p, _p, _p, _p, _i32, _i32, _i64, _i32, _i32, _i32, _p, _p, _sz,
                          _p], ctypes.c_int),
    "dsa_sparse_mla_workspace_size": ([_i32, _i32, _i32], _sz),
    "dsa_sparse_mla_attn": ([_p, _p, _i64, _p, _i64, _p, _p, _p, _i32, _i32, _i32, _i32, _f32, _p,
                             _i32, _p, _p, _sz, _p], ctypes.c_int),
    "dsa_value_gate": ([_p, _p, _p, _i32, _i32, _p, _p], ctypes.c_int),
    "dsa_indexer_project_workspace_size": ([_i32], _sz),
    "dsa_quantize_index_keys_fp8": ([_p, _i64, _p, _p, _p], ctypes.c_int),
    "dsa_indexer_topk_paged": ([_p, _p, _p, _p, _i32, _i32, _p, _p, _p, _i32, _i32, _i64, _i32, _i32,
                                _i32, _p, _p, _sz, _p], ctypes.c_int),
    "dsa_sparse_mla_attn_paged": ([_p, _p, _i64, _p, _i64, _p, _i32, _i32, _p, _p, _p, _i32, _i32,
                                   _i32, _i32, _f32, _p, _i32, _p, _p, _sz, _p], ctypes.c_int),
    "dsa_indexer_scores_fp8": ([_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i64, _i32, _i32, _p, _i64,
                                _p], ctypes.c_int),
    "dsa_indexer_topk_fp8": ([_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i64, _i32, _i32, _i32, _p,
                              _p, _sz, _p], ctypes.c_int),
    "dsa_indexer_project": ([_p, _p, _p, _p, _p, _p, _p, _f32, _i32, _p, _p, _p, _p, _p, _sz, _p],
                            ctypes.c_int),
}


def library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa_amd.so (once); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"DSA HIP library not found at {path}; build it with "
                "`python -m dsa_indexer_top_key_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        raise DsaError(fn, status, library().dsa_last_error().decode())


def _torch():
    import torch
    return torch


def _dev(x, name):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise TypeError(f"{name} must be a torch tensor on the GPU")
    return x


def _ptr(x):
    return ctypes.c_void_p(x.data_ptr()) if x is not None else ctypes.c_void_p(0)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _bits16(x, name):
    torch = _torch()
    _dev(x, name)
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 values (bfloat16 or 16-bit bit patterns)")
    return x


def _contig(x, name):
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return x


def _rows_ld(x, name, width):
    """Row stride (elements) of a 2-D view whose rows hold at least `width` elements."""
    if x.dim() != 2 or x.stride(1) != 1 or x.shape[1] < width:
        raise ValueError(f"{name} must be a 2-D row-major view with >= {width} columns")
    return x.stride(0)


def index_keys_layernorm(raw, gamma, beta, eps: float = 1e-6, keys=None, stream=None):
    """Stage 1: raw [N,128] float32 -> LayerNormed bf16 keys [N,128]."""
    torch = _torch()
    _contig(_dev(raw, "raw"), "raw")
    n = raw.shape[0]
    if keys is None:
        keys = torch.empty((n, INDEX_DIM), dtype=torch.bfloat16, device=raw.device)
    _check("dsa_index_keys_layernorm", library().dsa_index_keys_layernorm(
        _ptr(raw), _ptr(_contig(_dev(gamma, "gamma"), "gamma")),
        _ptr(_contig(_dev(beta, "beta"), "beta")), float(eps), _ptr(_contig(keys, "keys")), n,
        _stream(stream)))
    return keys


def _layout(kv_off, q_req, q_pos):
    for x, n in ((kv_off, "kv_off"), (q_req, "q_req"), (q_pos, "q_pos")):
        _contig(_dev(x, n), n)
    torch = _torch()
    if kv_off.dtype != torch.int64 or q_req.dtype != torch.int32 or q_pos.dtype != torch.int32:
        raise TypeError("kv_off must be int64, q_req and q_pos int32")
    return kv_off.shape[0] - 1


def indexer_scores(q_idx, w, keys, kv_off, q_req, q_pos, max_s: int, scores=None, stream=None):
    """Stage 2 alone: fp32 scores [T, max_s]; entries j >= n_t are left untouched."""
    torch = _torch()
    b = _layout(kv_off, q_req, q_pos)
    t = q_idx.shape[0]
    if scores is None:
        scores = torch.full((t, max_s), float("nan"), dtype=torch.float32, device=q_idx.device)
    _check("dsa_indexer_scores", library().dsa_indexer_scores(
        _ptr(_contig(_bits16(q_idx, "q_idx"), "q_idx")), _ptr(_contig(_bits16(w, "w"), "w")),
        _ptr(_contig(_bits16(keys, "keys"), "keys")), _ptr(kv_off), _ptr(q_req), _ptr(q_pos), t,
        b, int(max_s), q_idx.shape[1], q_idx.shape[2], _ptr(scores), scores.stride(0),
        _stream(stream)))
    return scores


def topk(scores, n_valid, k: int = TOPK, max_n=None, ids=None, stream=None):
    """Stage 3 alone: canonical top-k column IDs of fp32 score rows."""
    torch = _torch()
    _dev(scores, "scores")
    if scores.dim() != 2 or scores.stride(1) != 1 or scores.dtype != torch.float32:
        raise ValueError("scores must be a row-major float32 [T, ld] tensor")
    _contig(_dev(n_valid, "n_valid"), "n_valid")
    t = scores.shape[0]
    max_n = scores.shape[1] if max_n is None else int(max_n)
    if ids is None:
        ids = torch.empty((t, k), dtype=torch.int32, device=scores.device)
    _check("dsa_topk", library().dsa_topk(_ptr(scores), scores.stride(0), _ptr(n_valid), t, max_n,
                                          k, _ptr(_contig(ids, "ids")), _stream(stream)))
    return ids


def indexer_topk_workspace_size(t: int, max_s: int) -> int:
    return int(library().dsa_indexer_topk_workspace_size(t, max_s))


def indexer_topk(q_idx, w, keys, kv_off, q_req, q_pos, max_s: int, k: int = TOPK, ids=None,
                 workspace=None, stream=None):
    """Stages 2+3: [T,2048] request-local position IDs (ascending, -1 padded)."""
    torch = _torch()
    b = _layout(kv_off, q_req, q_pos)
    t = q_idx.shape[0]
    if ids is None:
        ids = torch.empty((t, k), dtype=torch.int32, device=q_idx.device)
    need = indexer_topk_workspace_size(t, max_s)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_idx.device)
    _check("dsa_indexer_topk", library().dsa_indexer_topk(
        _ptr(_contig(_bits16(q_idx, "q_idx"), "q_idx")), _ptr(_contig(_bits16(w, "w"), "w")),
        _ptr(_contig(_bits16(keys, "keys"), "keys")), _ptr(kv_off), _ptr(q_req), _ptr(q_pos), t,
        b, int(max_s), q_idx.shape[1], q_idx.shape[2], k, _ptr(_contig(ids, "ids")),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return ids


def sparse_mla_workspace_size(t: int, n_heads: int = MLA_HEADS, k: int = TOPK) -> int:
    return int(library().dsa_sparse_mla_workspace_size(t, n_heads, k))


def sparse_mla_attn(q, latent, kpe, kv_off, q_req, ids, scale: float, out=None, lse=None,
                    workspace=None, stream=None, out_dtype=None):
    """Stage 4: restricted-softmax absorbed-MLA read -> (out [T,96,512], lse [T,96]).

    out is bfloat16 unless out_dtype=torch.float32 (or a float32 `out` is passed)."""
    torch = _torch()
    _contig(_bits16(q, "q"), "q")
    _bits16(latent, "latent")
    _bits16(kpe, "kpe")
    ld_lat = _rows_ld(latent, "latent", LATENT_DIM)
    ld_kpe = _rows_ld(kpe, "kpe", COMPANION_DIM)
    b = kv_off.shape[0] - 1
    for x, n in ((kv_off, "kv_off"), (q_req, "q_req"), (ids, "ids")):
        _contig(_dev(x, n), n)
    t, h = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((t, h, LATENT_DIM), dtype=out_dtype or torch.bfloat16, device=q.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    out_code = 1 if out.dtype == torch.float32 else 0
    if lse is None:
        lse = torch.empty((t, h), dtype=torch.float32, device=q.device)
    need = sparse_mla_workspace_size(t, h, ids.shape[1] if ids.dim() == 2 else TOPK)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_sparse_mla_attn", library().dsa_sparse_mla_attn(
        _ptr(q), _ptr(latent), ld_lat, _ptr(kpe), ld_kpe, _ptr(kv_off), _ptr(q_req), _ptr(ids), t,
        b, h, ids.shape[1], float(scale), _ptr(_contig(out, "out")), out_code, _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse


def value_gate(o, w_uv, gate, out=None, stream=None):
    """Value up-projection and sigmoid output gate of the read: o [T,96,512] bf16,
    w_uv [96,128,512] bf16, gate [T,96,128] bf16 logits -> out [T,96,128] bf16 with
    out[t,h] = (w_uv[h] @ o[t,h]) * sigmoid(gate[t,h])."""
    torch = _torch()
    for x, n in ((o, "o"), (w_uv, "w_uv"), (gate, "gate")):
        _contig(_bits16(_dev(x, n), n), n)
    t, h = o.shape[0], o.shape[1]
    if tuple(o.shape[1:]) != (h, LATENT_DIM) or tuple(w_uv.shape) != (h, VALUE_DIM, LATENT_DIM) \
            or tuple(gate.shape) != (t, h, VALUE_DIM):
        raise ValueError("value_gate expects o [T,H,512], w_uv [H,128,512], gate [T,H,128]")
    if out is None:
        out = torch.empty((t, h, VALUE_DIM), dtype=torch.bfloat16, device=o.device)
    _check("dsa_value_gate", library().dsa_value_gate(
        _ptr(o), _ptr(w_uv), _ptr(gate), t, h, _ptr(_contig(out, "out")), _stream(stream)))
    return out


def indexer_project_workspace_size(t: int) -> int:
    return int(library().dsa_indexer_project_workspace_size(t))


def indexer_project(c_q, h, w_qi, w_k, w_w, gamma, beta, eps: float, keys, key_rows, q_idx=None,
                    w=None, workspace=None, stream=None):
    """Indexer-side projections of T new tokens: c_q [T,1536] and h [T,7168] bf16, weights
    w_qi [4096,1536], w_k [128,7168], w_w [32,7168] bf16 ([out, in]), gamma/beta [128] fp32.
    Returns (q_idx [T,32,128], w [T,32]) bf16 and writes LayerNorm(w_k h[t]) as bf16 into row
    key_rows[t] (int64, absolute) of the index-key cache `keys` [rows,128]."""
    torch = _torch()
    for x, n in ((c_q, "c_q"), (h, "h"), (w_qi, "w_qi"), (w_k, "w_k"), (w_w, "w_w"),
                 (keys, "keys")):
        _contig(_bits16(_dev(x, n), n), n)
    for x, n in ((gamma, "gamma"), (beta, "beta"), (key_rows, "key_rows")):
        _contig(_dev(x, n), n)
    t = c_q.shape[0]
    if tuple(c_q.shape) != (t, Q_LATENT) or tuple(h.shape) != (t, RESIDUAL) \
            or tuple(w_qi.shape) != (INDEX_HEADS * INDEX_DIM, Q_LATENT) \
            or tuple(w_k.shape) != (INDEX_DIM, RESIDUAL) or tuple(w_w.shape) != (INDEX_HEADS, RESIDUAL) \
            or keys.dim() != 2 or keys.shape[1] != INDEX_DIM or tuple(key_rows.shape) != (t,):
        raise ValueError("indexer_project expects c_q [T,1536], h [T,7168], w_qi [4096,1536], "
                         "w_k [128,7168], w_w [32,7168], keys [rows,128], key_rows [T]")
    if key_rows.dtype != torch.int64 or gamma.dtype != torch.float32 or beta.dtype != torch.float32:
        raise TypeError("key_rows must be int64, gamma and beta float32")
    if q_idx is None:
        q_idx = torch.empty((t, INDEX_HEADS, INDEX_DIM), dtype=torch.bfloat16, device=c_q.device)
    if w is None:
        w = torch.empty((t, INDEX_HEADS), dtype=torch.bfloat16, device=c_q.device)
    need = indexer_project_workspace_size(t)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=c_q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_indexer_project", library().dsa_indexer_project(
        _ptr(c_q), _ptr(h), _ptr(w_qi), _ptr(w_k), _ptr(w_w), _ptr(gamma), _ptr(beta), float(eps), t,
        _ptr(_contig(q_idx, "q_idx")), _ptr(_contig(w, "w")), _ptr(keys), _ptr(key_rows),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return q_idx, w


def _codes(codes, scales):
    torch = _torch()
    _contig(_dev(codes, "codes"), "codes")
    _contig(_dev(scales, "scales"), "scales")
    if codes.dtype != torch.uint8 or scales.dtype != torch.float32:
        raise TypeError("codes must be uint8 and scales float32")
    if codes.dim() != 2 or codes.shape[1] != INDEX_DIM or tuple(scales.shape) != (codes.shape[0],):
        raise ValueError("codes must be [rows,128] and scales [rows]")


def quantize_index_keys_fp8(keys, codes=None, scales=None, stream=None):
    """FP8 index-key cache: bf16 keys [N,128] -> (codes [N,128] uint8 OCP E4M3, scales [N]
    float32 powers of two); key = E4M3(code) * scale."""
    torch = _torch()
    _contig(_bits16(_dev(keys, "keys"), "keys"), "keys")
    n = keys.shape[0]
    if codes is None:
        codes = torch.empty((n, INDEX_DIM), dtype=torch.uint8, device=keys.device)
    if scales is None:
        scales = torch.empty((n,), dtype=torch.float32, device=keys.device)
    _codes(codes, scales)
    _check("dsa_quantize_index_keys_fp8", library().dsa_quantize_index_keys_fp8(
        _ptr(keys), n, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def indexer_scores_fp8(q_idx, w, codes, scales, kv_off, q_req, q_pos, max_s: int, scores=None,
                       stream=None):
    """Stage 2 over the FP8 key cache: fp32 scores [T, max_s]; entries j >= n_t untouched."""
    torch = _torch()
    b = _layout(kv_off, q_req, q_pos)
    _codes(codes, scales)
    t = q_idx.shape[0]
    if scores is None:
        scores = torch.full((t, max_s), float("nan"), dtype=torch.float32, device=q_idx.device)
    _check("dsa_indexer_scores_fp8", library().dsa_indexer_scores_fp8(
        _ptr(_contig(_bits16(q_idx, "q_idx"), "q_idx")), _ptr(_contig(_bits16(w, "w"), "w")),
        _ptr(codes), _ptr(scales), _ptr(kv_off), _ptr(q_req), _ptr(q_pos), t, b, int(max_s),
        q_idx.shape[1], q_idx.shape[2], _ptr(scores), scores.stride(0), _stream(stream)))
    return scores


def indexer_topk_fp8(q_idx, w, codes, scales, kv_off, q_req, q_pos, max_s: int, k: int = TOPK,
                     ids=None, workspace=None, stream=None):
    """Stages 2+3 over the FP8 key cache: [T,2048] request-local position IDs."""
    torch = _torch()
    b = _layout(kv_off, q_req, q_pos)
    _codes(codes, scales)
    t = q_idx.shape[0]
    if ids is None:
        ids = torch.empty((t, k), dtype=torch.int32, device=q_idx.device)
    need = indexer_topk_workspace_size(t, max_s)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_idx.device)
    _check("dsa_indexer_topk_fp8", library().dsa_indexer_topk_fp8(
        _ptr(_contig(_bits16(q_idx, "q_idx"), "q_idx")), _ptr(_contig(_bits16(w, "w"), "w")),
        _ptr(codes), _ptr(scales), _ptr(kv_off), _ptr(q_req), _ptr(q_pos), t, b, int(max_s),
        q_idx.shape[1], q_idx.shape[2], k, _ptr(_contig(ids, "ids")), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return ids


def _pages(page_table):
    torch = _torch()
    _contig(_dev(page_table, "page_table"), "page_table")
    if page_table.dtype != torch.int32 or page_table.dim() != 2:
        raise TypeError("page_table must be an int32 [B, max_pages] tensor")
    return page_table.shape[1]


def indexer_topk_paged(q_idx, w, key_pool, page_table, page_size: int, kv_off, q_req, q_pos,
                       max_s: int, k: int = TOPK, ids=None, workspace=None, stream=None):
    """Stages 2+3 over a paged key pool: position p of request b is row
    page_table[b, p // page_size] * page_size + p % page_size of key_pool [rows,128];
    kv_off gives only the request lengths.  Same IDs as indexer_topk on the same logical cache."""
    torch = _torch()
    b = _layout(kv_off, q_req, q_pos)
    max_pages = _pages(page_table)
    t = q_idx.shape[0]
    if ids is None:
        ids = torch.empty((t, k), dtype=torch.int32, device=q_idx.device)
    need = indexer_topk_workspace_size(t, max_s)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_idx.device)
    _check("dsa_indexer_topk_paged", library().dsa_indexer_topk_paged(
        _ptr(_contig(_bits16(q_idx, "q_idx"), "q_idx")), _ptr(_contig(_bits16(w, "w"), "w")),
        _ptr(_contig(_bits16(key_pool, "key_pool"), "key_pool")), _ptr(page_table), int(page_size),
        max_pages, _ptr(kv_off), _ptr(q_req), _ptr(q_pos), t, b, int(max_s), q_idx.shape[1],
        q_idx.shape[2], k, _ptr(_contig(ids, "ids")), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return ids


def sparse_mla_attn_paged(q, latent_pool, kpe_pool, page_table, page_size: int, kv_off, q_req, ids,
                          scale: float, out=None, lse=None, workspace=None, stream=None,
                          out_dtype=None):
    """Stage 4 over paged latent/companion pools (rows addressed as in indexer_topk_paged);
    same results as sparse_mla_attn on the same logical cache."""
    torch = _torch()
    _contig(_bits16(q, "q"), "q")
    _bits16(latent_pool, "latent_pool")
    _bits16(kpe_pool, "kpe_pool")
    ld_lat = _rows_ld(latent_pool, "latent_pool", LATENT_DIM)
    ld_kpe = _rows_ld(kpe_pool, "kpe_pool", COMPANION_DIM)
    max_pages = _pages(page_table)
    b = kv_off.shape[0] - 1
    for x, n in ((kv_off, "kv_off"), (q_req, "q_req"), (ids, "ids")):
        _contig(_dev(x, n), n)
    t, h = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty((t, h, LATENT_DIM), dtype=out_dtype or torch.bfloat16, device=q.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("out must be bfloat16 or float32")
    if lse is None:
        lse = torch.empty((t, h), dtype=torch.float32, device=q.device)
    need = sparse_mla_workspace_size(t, h, ids.shape[1] if ids.dim() == 2 else TOPK)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_sparse_mla_attn_paged", library().dsa_sparse_mla_attn_paged(
        _ptr(q), _ptr(latent_pool), ld_lat, _ptr(kpe_pool), ld_kpe, _ptr(page_table),
        int(page_size), max_pages, _ptr(kv_off), _ptr(q_req), _ptr(ids), t, b, h, ids.shape[1],
        float(scale), _ptr(_contig(out, "out")), 1 if out.dtype == torch.float32 else 0, _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return out, lse
