"""The C ABI on a machine without a GPU: the library loads, exports every entry point the
header declares, and rejects every malformed call on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import dsa_indexer_top_key_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH),
                                reason="libdsa_amd.so not built (run __graft_entry__.build())")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
P = ctypes.c_void_p


def fake(addr=0x10000):
    """A non-null, 256-byte aligned pointer value that is never dereferenced."""
    return ctypes.c_void_p(addr)


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dsa_status_t|size_t|int|const char\*)\s+(dsa_\w+)\(",
                                 src, re.M)))


def test_exports_every_declared_symbol():
    lib = dsa.library()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dsa._SIGNATURES)


def test_status_strings_and_version():
    lib = dsa.library()
    assert lib.dsa_abi_version() == 1
    for code in range(5):
        assert lib.dsa_status_string(code)
    assert b"unknown" in lib.dsa_status_string(99)


def last_error():
    return dsa.library().dsa_last_error().decode()


def test_layernorm_validation():
    lib = dsa.library()
    f = lib.dsa_index_keys_layernorm
    assert f(P(0), P(0), P(0), 1e-6, P(0), 0, P(0)) == OK  # empty: no pointer touched
    assert f(fake(), fake(), fake(), 1e-6, fake(), -1, P(0)) == INVALID
    assert "negative" in last_error()
    assert f(fake(), fake(), fake(), -1.0, fake(), 4, P(0)) == INVALID
    assert f(fake(), fake(), fake(), float("nan"), fake(), 4, P(0)) == INVALID
    assert f(P(0), fake(), fake(), 1e-6, fake(), 4, P(0)) == INVALID
    assert f(fake(0x10004), fake(), fake(), 1e-6, fake(), 4, P(0)) == INVALID
    assert "aligned" in last_error()


def idx_args(**kw):
    a = dict(q=fake(), w=fake(), k=fake(), off=fake(), req=fake(), pos=fake(), T=4, B=4,
             max_s=4096, H=32, D=128)
    a.update(kw)
    return a


def call_scores(a, scores=fake(), ld=4096):
    return dsa.library().dsa_indexer_scores(a["q"], a["w"], a["k"], a["off"], a["req"], a["pos"],
                                            a["T"], a["B"], a["max_s"], a["H"], a["D"], scores, ld,
                                            P(0))


def test_indexer_scores_validation():
    assert call_scores(idx_args(T=0, q=P(0))) == OK
    assert call_scores(idx_args(T=-1)) == INVALID
    assert call_scores(idx_args(B=0)) == INVALID
    assert call_scores(idx_args(max_s=0)) == INVALID
    assert call_scores(idx_args(H=16)) == UNSUPPORTED
    assert call_scores(idx_args(D=64)) == UNSUPPORTED
    assert call_scores(idx_args(k=P(0))) == INVALID
    assert call_scores(idx_args(q=fake(0x10008))) == INVALID
    assert call_scores(idx_args(), scores=P(0)) == INVALID
    assert call_scores(idx_args(), ld=100) == INVALID
    assert "ld_scores" in last_error()


def call_itk(a, k=2048, ids=fake(), ws=fake(), ws_bytes=1 << 40):
    return dsa.library().dsa_indexer_topk(a["q"], a["w"], a["k"], a["off"], a["req"], a["pos"],
                                          a["T"], a["B"], a["max_s"], a["H"], a["D"], k, ids, ws,
                                          ws_bytes, P(0))


def test_indexer_topk_validation_and_workspace():
    lib = dsa.library()
    need = lib.dsa_indexer_topk_workspace_size(4, 4096)
    assert need >= 4 * 4096 * 4 and need % 256 == 0
    assert lib.dsa_indexer_topk_workspace_size(0, 4096) == 0
    assert call_itk(idx_args(T=0)) == OK
    assert call_itk(idx_args(), k=1024) == UNSUPPORTED
    assert call_itk(idx_args(), ids=P(0)) == INVALID
    assert call_itk(idx_args(), ws=P(0)) == WORKSPACE
    assert call_itk(idx_args(), ws=fake(0x10010)) == WORKSPACE
    assert call_itk(idx_args(), ws_bytes=need - 1) == WORKSPACE
    assert "required" in last_error()


def test_indexer_topk_noalloc_validation():
    """Every argument check runs before the scratch lookup (the first HIP call), so each
    malformed call is refused here without a GPU; sizes beyond the scratch array are refused
    with a message naming the limit."""
    lib = dsa.library()

    def call(a, k=2048, ids=fake()):
        return lib.dsa_indexer_topk_noalloc(a["q"], a["w"], a["k"], a["off"], a["req"], a["pos"],
                                            a["T"], a["B"], a["max_s"], a["H"], a["D"], k, ids, P(0))
    assert call(idx_args(T=0, q=P(0))) == OK
    assert call(idx_args(T=-1)) == INVALID
    assert call(idx_args(), k=1024) == UNSUPPORTED
    assert call(idx_args(H=16)) == UNSUPPORTED
    assert call(idx_args(q=P(0))) == INVALID
    assert call(idx_args(), ids=P(0)) == INVALID
    assert call(idx_args(max_s=0)) == INVALID
    # 256 x 32768 fits the 32 MiB array exactly; one more position per row does not
    assert lib.dsa_indexer_topk_workspace_size(256, 32768) == dsa.NOALLOC_SCRATCH_BYTES
    assert call(idx_args(T=256, B=256, max_s=32769)) == UNSUPPORTED
    assert "scratch" in last_error() and str(dsa.NOALLOC_SCRATCH_BYTES) in last_error()
    assert call(idx_args(T=4, B=4, max_s=1 << 22)) == UNSUPPORTED


def test_topk_validation():
    f = dsa.library().dsa_topk
    assert f(P(0), 10, P(0), 0, 10, 2048, P(0), P(0)) == OK
    assert f(fake(), 10, fake(), 3, 10, 100, fake(), P(0)) == UNSUPPORTED
    assert f(fake(), 10, fake(), -2, 10, 2048, fake(), P(0)) == INVALID
    assert f(fake(), 5, fake(), 3, 10, 2048, fake(), P(0)) == INVALID
    assert f(P(0), 10, fake(), 3, 10, 2048, fake(), P(0)) == INVALID
    assert f(fake(), 10, fake(), 3, -1, 2048, fake(), P(0)) == INVALID


def call_mla(**kw):
    a = dict(q=fake(), lat=fake(), ld_lat=576, kpe=fake(0x10400), ld_kpe=576, off=fake(),
             req=fake(), ids=fake(), T=64, B=64, H=96, k=2048, scale=0.07, out=fake(), dt=0,
             lse=fake(), ws=fake(), ws_bytes=1 << 40)
    a.update(kw)
    return dsa.library().dsa_sparse_mla_attn(
        a["q"], a["lat"], a["ld_lat"], a["kpe"], a["ld_kpe"], a["off"], a["req"], a["ids"], a["T"],
        a["B"], a["H"], a["k"], a["scale"], a["out"], a["dt"], a["lse"], a["ws"], a["ws_bytes"],
        P(0))


def test_sparse_mla_validation_and_workspace():
    lib = dsa.library()
    assert lib.dsa_sparse_mla_workspace_size(4096, 96, 2048) == 0  # large T: no split
    small = lib.dsa_sparse_mla_workspace_size(4, 96, 2048)
    assert small > 0 and small % 256 == 0
    assert call_mla(T=0, q=P(0)) == OK
    assert call_mla(H=128) == UNSUPPORTED
    assert call_mla(k=1024) == UNSUPPORTED
    assert call_mla(T=-1) == INVALID
    assert call_mla(scale=float("inf")) == INVALID
    assert call_mla(ld_lat=500) == INVALID
    assert call_mla(ld_lat=580) == INVALID
    assert call_mla(ld_kpe=60) == INVALID
    assert call_mla(kpe=fake(0x10008)) == INVALID
    assert call_mla(out=P(0)) == INVALID
    assert call_mla(dt=2) == UNSUPPORTED
    assert call_mla(ws=P(0)) == WORKSPACE
    assert call_mla(ws_bytes=16) == WORKSPACE


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(TypeError):
        dsa.index_keys_layernorm(torch.zeros(4, 128), torch.ones(128), torch.zeros(128))


def _binding_calls(torch):
    """Well-formed arguments for every binding entry point, as CPU tensors (the GPU check
    comes last, so each call below reaches every shape and dtype check and then stops)."""
    bf, i32, i64, f32, u8 = torch.bfloat16, torch.int32, torch.int64, torch.float32, torch.uint8
    z = torch.zeros
    T, B, S = 4, 2, 100
    lay = dict(kv_off=z(B + 1, dtype=i64), q_req=z(T, dtype=i32), q_pos=z(T, dtype=i32))
    iq = dict(q_idx=z(T, 32, 128, dtype=bf), w=z(T, 32, dtype=bf))
    mla = dict(q=z(T, 96, 576, dtype=bf), latent=z(S, 512, dtype=bf), kpe=z(S, 64, dtype=bf),
               kv_off=lay["kv_off"], q_req=lay["q_req"], ids=z(T, 2048, dtype=i32))
    f8 = dict(codes=z(S, 128, dtype=u8), scales=z(S, dtype=f32))
    return {
        "index_keys_layernorm": (dsa.index_keys_layernorm, dict(
            raw=z(S, 128, dtype=f32), gamma=z(128, dtype=f32), beta=z(128, dtype=f32),
            keys=z(S, 128, dtype=bf))),
        "indexer_scores": (dsa.indexer_scores, dict(
            **iq, keys=z(S, 128, dtype=bf), **lay, max_s=S, scores=z(T, S, dtype=f32))),
        "topk": (dsa.topk, dict(scores=z(T, S, dtype=f32), n_valid=z(T, dtype=i32),
                                ids=z(T, 2048, dtype=i32))),
        "indexer_topk_noalloc": (dsa.indexer_topk_noalloc, dict(
            **iq, keys=z(S, 128, dtype=bf), **lay, max_s=S, ids=z(T, 2048, dtype=i32))),
        "indexer_topk": (dsa.indexer_topk, dict(
            **iq, keys=z(S, 128, dtype=bf), **lay, max_s=S, ids=z(T, 2048, dtype=i32),
            workspace=z(1 << 20, dtype=u8))),
        "sparse_mla_attn": (dsa.sparse_mla_attn, dict(
            **mla, scale=0.07, out=z(T, 96, 512, dtype=bf), lse=z(T, 96, dtype=f32))),
        "value_gate": (dsa.value_gate, dict(o=z(T, 96, 512, dtype=bf), w_uv=z(96, 128, 512, dtype=bf),
                                            gate=z(T, 96, 128, dtype=bf), out=z(T, 96, 128, dtype=bf))),
        "indexer_project": (dsa.indexer_project, dict(
            c_q=z(T, 1536, dtype=bf), h=z(T, 7168, dtype=bf), w_qi=z(4096, 1536, dtype=bf),
            w_k=z(128, 7168, dtype=bf), w_w=z(32, 7168, dtype=bf), gamma=z(128, dtype=f32),
            beta=z(128, dtype=f32), eps=1e-6, keys=z(S, 128, dtype=bf), key_rows=z(T, dtype=i64),
            q_idx=z(T, 32, 128, dtype=bf), w=z(T, 32, dtype=bf))),
        "quantize_index_keys_fp8": (dsa.quantize_index_keys_fp8, dict(keys=z(S, 128, dtype=bf), **f8)),
        "indexer_scores_fp8": (dsa.indexer_scores_fp8, dict(
            **iq, **f8, **lay, max_s=S, scores=z(T, S, dtype=f32))),
        "indexer_topk_fp8": (dsa.indexer_topk_fp8, dict(
            **iq, **f8, **lay, max_s=S, ids=z(T, 2048, dtype=i32))),
        "indexer_topk_paged": (dsa.indexer_topk_paged, dict(
            **iq, key_pool=z(128, 128, dtype=bf), page_table=z(B, 2, dtype=i32), page_size=64,
            **lay, max_s=S, ids=z(T, 2048, dtype=i32))),
        "sparse_mla_attn_paged": (dsa.sparse_mla_attn_paged, dict(
            q=mla["q"], latent_pool=z(128, 512, dtype=bf), kpe_pool=z(128, 64, dtype=bf),
            page_table=z(B, 2, dtype=i32), page_size=64, kv_off=lay["kv_off"],
            q_req=lay["q_req"], ids=mla["ids"], scale=0.07)),
    }


# (entry point, argument, replacement builder, exception): one bad argument per case; each
# must be refused by the binding with a message naming the argument, before any launch.
_BAD_ARGS = [
    ("index_keys_layernorm", "raw", lambda t: t.zeros(100, 64), ValueError),
    ("index_keys_layernorm", "raw", lambda t: t.zeros(100, 128, dtype=t.float64), TypeError),
    ("index_keys_layernorm", "gamma", lambda t: t.zeros(64), ValueError),
    ("index_keys_layernorm", "keys", lambda t: t.zeros(99, 128, dtype=t.bfloat16), ValueError),
    ("indexer_scores", "q_idx", lambda t: t.zeros(4, 32, 64, dtype=t.bfloat16), ValueError),
    ("indexer_scores", "w", lambda t: t.zeros(3, 32, dtype=t.bfloat16), ValueError),
    ("indexer_scores", "q_req", lambda t: t.zeros(4, dtype=t.int64), TypeError),
    ("indexer_scores", "q_pos", lambda t: t.zeros(5, dtype=t.int32), ValueError),
    ("indexer_scores", "kv_off", lambda t: t.zeros(3, dtype=t.int32), TypeError),
    ("indexer_scores", "keys", lambda t: t.zeros(100, 64, dtype=t.bfloat16), ValueError),
    ("indexer_scores", "scores", lambda t: t.zeros(4, 50), ValueError),
    ("indexer_scores", "scores", lambda t: t.zeros(100, 4).t(), ValueError),
    ("topk", "n_valid", lambda t: t.zeros(4, dtype=t.int64), TypeError),
    ("topk", "n_valid", lambda t: t.zeros(3, dtype=t.int32), ValueError),
    ("topk", "ids", lambda t: t.zeros(4, 1024, dtype=t.int32), ValueError),
    ("topk", "ids", lambda t: t.zeros(4, 2048, dtype=t.int64), TypeError),
    ("indexer_topk", "ids", lambda t: t.zeros(3, 2048, dtype=t.int32), ValueError),
    ("indexer_topk", "workspace", lambda t: t.zeros(16, dtype=t.uint8), ValueError),
    ("sparse_mla_attn", "q", lambda t: t.zeros(4, 96, 512, dtype=t.bfloat16), ValueError),
    ("sparse_mla_attn", "latent", lambda t: t.zeros(100, 256, dtype=t.bfloat16), ValueError),
    ("sparse_mla_attn", "kpe", lambda t: t.zeros(100, 64, dtype=t.float32), TypeError),
    ("sparse_mla_attn", "ids", lambda t: t.zeros(4, 2048, dtype=t.int64), TypeError),
    ("sparse_mla_attn", "ids", lambda t: t.zeros(4, 1024, dtype=t.int32), ValueError),
    ("sparse_mla_attn", "q_req", lambda t: t.zeros(5, dtype=t.int32), ValueError),
    ("sparse_mla_attn", "out", lambda t: t.zeros(4, 96, 512, dtype=t.float16), TypeError),
    ("sparse_mla_attn", "out", lambda t: t.zeros(4, 96, 128, dtype=t.bfloat16), ValueError),
    ("sparse_mla_attn", "lse", lambda t: t.zeros(4, 96, dtype=t.bfloat16), TypeError),
    ("sparse_mla_attn", "lse", lambda t: t.zeros(96, 4).t(), ValueError),
    ("value_gate", "gate", lambda t: t.zeros(4, 96, 64, dtype=t.bfloat16), ValueError),
    ("value_gate", "out", lambda t: t.zeros(4, 96, 128, dtype=t.float32), TypeError),
    ("indexer_project", "h", lambda t: t.zeros(4, 4096, dtype=t.bfloat16), ValueError),
    ("indexer_project", "key_rows", lambda t: t.zeros(4, dtype=t.int32), TypeError),
    ("indexer_project", "w", lambda t: t.zeros(4, 16, dtype=t.bfloat16), ValueError),
    ("quantize_index_keys_fp8", "codes", lambda t: t.zeros(99, 128, dtype=t.uint8), ValueError),
    ("quantize_index_keys_fp8", "scales", lambda t: t.zeros(100, dtype=t.float64), TypeError),
    ("indexer_scores_fp8", "scales", lambda t: t.zeros(99), ValueError),
    ("indexer_topk_fp8", "codes", lambda t: t.zeros(100, 128, dtype=t.int8), TypeError),
    ("indexer_topk_paged", "page_table", lambda t: t.zeros(3, 2, dtype=t.int32), ValueError),
    ("indexer_topk_paged", "page_table", lambda t: t.zeros(2, 2, dtype=t.int64), TypeError),
    ("sparse_mla_attn_paged", "latent_pool", lambda t: t.zeros(128, 500, dtype=t.bfloat16), ValueError),
    ("sparse_mla_attn_paged", "page_table", lambda t: t.zeros(2, dtype=t.int32), ValueError),
]


def test_binding_checks_every_entry_point_before_any_launch():
    torch = pytest.importorskip("torch")
    for name, (fn, kw) in _binding_calls(torch).items():
        with pytest.raises(TypeError, match="on the GPU"):
            fn(**kw)  # well-formed: stops at the device check, nothing launched


@pytest.mark.parametrize("name,arg,bad,exc", _BAD_ARGS, ids=[f"{c[0]}-{c[1]}-{i}" for i, c in enumerate(_BAD_ARGS)])
def test_binding_refuses_a_malformed_argument(name, arg, bad, exc):
    torch = pytest.importorskip("torch")
    fn, kw = _binding_calls(torch)[name]
    kw = dict(kw)
    kw[arg] = bad(torch)
    with pytest.raises(exc, match=arg):
        fn(**kw)


def test_value_gate_clears_an_earlier_error():
    lib = dsa.library()
    assert lib.dsa_value_gate(P(0), P(0), P(0), -1, 96, P(0), P(0)) == INVALID
    assert last_error()
    assert lib.dsa_value_gate(P(0), P(0), P(0), 0, 96, P(0), P(0)) == OK
    assert last_error() == ""


def test_value_gate_validation():
    lib = dsa.library()
    vg = lambda o=fake(), w=fake(), g=fake(), T=2, H=96, out=fake(): lib.dsa_value_gate(o, w, g, T, H, out, P(0))
    assert vg(T=0, o=P(0), w=P(0), g=P(0), out=P(0)) == OK  # nothing to do, no pointer touched
    assert vg(T=-1) == INVALID
    assert vg(H=128) == UNSUPPORTED
    assert vg(o=P(0)) == INVALID
    assert vg(out=P(0)) == INVALID
    assert vg(o=fake(0x10008)) == INVALID   # o must be 16-byte aligned
    assert vg(w=fake(0x10004)) == INVALID   # w_uv must be 16-byte aligned
    assert vg(out=fake(0x10002)) == INVALID  # out must be 4-byte aligned
    assert vg(g=fake(0x10001)) == INVALID   # gate must be 2-byte aligned


def test_indexer_project_validation_and_workspace():
    lib = dsa.library()
    need = lib.dsa_indexer_project_workspace_size(64)
    assert need > 0 and need % 256 == 0
    assert lib.dsa_indexer_project_workspace_size(0) == 0
    # 4096 tokens: the query product is not split (its blocks write bf16 q_idx directly), so
    # only the residual product's fp32 partials remain: at least one [T, 160] set
    big = lib.dsa_indexer_project_workspace_size(4096)
    assert 4096 * 160 * 4 <= big < 4096 * 4096 * 4

    def pj(T=64, eps=1e-6, ws=fake(), ws_bytes=need, **kw):
        a = dict(c_q=fake(), h=fake(), w_qi=fake(), w_k=fake(), w_w=fake(), gamma=fake(),
                 beta=fake(), q_idx=fake(), w=fake(), keys=fake(), key_rows=fake())
        a.update(kw)
        return lib.dsa_indexer_project(a["c_q"], a["h"], a["w_qi"], a["w_k"], a["w_w"],
                                       a["gamma"], a["beta"], eps, T, a["q_idx"], a["w"],
                                       a["keys"], a["key_rows"], ws, ws_bytes, P(0))

    zeros = {n: P(0) for n in ("c_q", "h", "w_qi", "w_k", "w_w", "gamma", "beta", "q_idx", "w",
                               "keys", "key_rows")}
    assert pj(T=0, ws=P(0), ws_bytes=0, **zeros) == OK  # nothing to do, no pointer touched
    assert pj(T=-1) == INVALID
    assert pj(eps=float("nan")) == INVALID
    assert pj(eps=-1.0) == INVALID
    for n in zeros:
        assert pj(**{n: P(0)}) == INVALID, n
        assert n in last_error() or "null" in last_error()
    for n in ("c_q", "h", "w_qi", "w_k", "w_w", "q_idx", "keys"):
        assert pj(**{n: fake(0x10008)}) == INVALID, n  # 16-byte alignment
    assert pj(key_rows=fake(0x10004)) == INVALID
    assert pj(gamma=fake(0x10002)) == INVALID
    assert pj(w=fake(0x10001)) == INVALID
    assert pj(ws=P(0)) == WORKSPACE
    assert pj(ws_bytes=need - 1) == WORKSPACE
    assert pj(ws=fake(0x10010)) == WORKSPACE  # 256-byte alignment


def test_fp8_key_cache_validation():
    lib = dsa.library()
    qz = lambda k=fake(), n=4, c=fake(), s=fake(): lib.dsa_quantize_index_keys_fp8(k, n, c, s, P(0))
    assert qz(n=0, k=P(0), c=P(0), s=P(0)) == OK
    assert qz(n=-1) == INVALID
    assert qz(k=P(0)) == INVALID and qz(c=P(0)) == INVALID and qz(s=P(0)) == INVALID
    assert qz(k=fake(0x10008)) == INVALID and qz(c=fake(0x10004)) == INVALID
    assert qz(s=fake(0x10002)) == INVALID

    def sc(T=2, B=2, S=100, H=32, D=128, c=fake(), s=fake(), out=fake(), ld=100):
        return lib.dsa_indexer_scores_fp8(fake(), fake(), c, s, fake(), fake(), fake(), T, B, S, H,
                                          D, out, ld, P(0))
    assert sc(T=0) == OK
    assert sc(T=-1) == INVALID
    assert sc(H=16) == UNSUPPORTED
    assert sc(c=P(0)) == INVALID and sc(s=P(0)) == INVALID and sc(out=P(0)) == INVALID
    assert sc(c=fake(0x10008)) == INVALID and sc(s=fake(0x10002)) == INVALID
    assert sc(ld=99) == INVALID
    need = lib.dsa_indexer_topk_workspace_size(2, 100)

    def tk(T=2, k=2048, ids=fake(), ws=fake(), wsb=need, s=fake()):
        return lib.dsa_indexer_topk_fp8(fake(), fake(), fake(), s, fake(), fake(), fake(), T, 2,
                                        100, 32, 128, k, ids, ws, wsb, P(0))
    assert tk(T=0) == OK
    assert tk(k=1024) == UNSUPPORTED
    assert tk(ids=P(0)) == INVALID and tk(s=P(0)) == INVALID
    assert tk(ws=P(0)) == WORKSPACE and tk(wsb=need - 1) == WORKSPACE


def test_paged_validation():
    lib = dsa.library()
    need = lib.dsa_indexer_topk_workspace_size(2, 100)

    def tk(T=2, ps=64, mp=2, pt=fake(), ids=fake()):
        return lib.dsa_indexer_topk_paged(fake(), fake(), fake(), pt, ps, mp, fake(), fake(),
                                          fake(), T, 2, 100, 32, 128, 2048, ids, fake(), need, P(0))
    assert tk(T=0, pt=P(0), ps=0, mp=0) == OK  # nothing to do
    for ps in (0, 32, 63, 96, 1 << 21):
        assert tk(ps=ps) == UNSUPPORTED, ps
    assert tk(mp=0) == INVALID
    assert tk(pt=P(0)) == INVALID and tk(pt=fake(0x10002)) == INVALID
    assert tk(ids=P(0)) == INVALID
    need_s = lib.dsa_sparse_mla_workspace_size(2, 96, 2048)

    def sp(T=2, ps=64, mp=2, pt=fake(), ld=576):
        return lib.dsa_sparse_mla_attn_paged(fake(), fake(), ld, fake(), ld, pt, ps, mp, fake(),
                                             fake(), fake(), T, 2, 96, 2048, 0.07, fake(), 0,
                                             fake(), fake(), need_s, P(0))
    assert sp(T=0, pt=P(0), ps=0, mp=0) == OK
    assert sp(ps=100) == UNSUPPORTED and sp(mp=-1) == INVALID and sp(pt=P(0)) == INVALID
    assert sp(ld=500) == INVALID
