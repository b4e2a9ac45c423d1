"""Host-side checks of the C ABI (no GPU needed): exports, pure helpers, argument validation.

Every invalid call must return its status before any HIP call is made, so these run on a CPU-only
machine: a call that reached a kernel launch would come back as CSA_ERR_HIP instead.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import long_context_compressed_compress_amd as csa
from oracle import paging

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 20  # aligned non-null pointer value that is never dereferenced on these paths
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(csa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return csa.lib()


def test_exports_every_declared_symbol(L):
    with open(os.path.join(ROOT, "include", "csa.h")) as f:
        text = f.read()
    names = set(re.findall(r"^\s*(?:[A-Za-z_][A-Za-z0-9_ ]*[\s*])?(csa_[a-z0-9_]+)\(", text, flags=re.M))
    names |= set(re.findall(r"\b(csa_[a-z0-9_]+)\s*\(", text))
    names = {n for n in names if not n.endswith("_t")}
    assert {"csa_compress_insert", "csa_index_topk", "csa_attend", "csa_inv_rope", "csa_rope_table",
            "csa_inv_rope_quant_fp8"} <= names
    for n in sorted(names):
        assert hasattr(L, n), n


def test_host_helpers_match_oracle(L):
    for m, w in ((4, 8), (128, 128)):
        for n in (0, 1, 7, 8, 9, 127, 128, 129, 255, 256, 131073, 1048577):
            assert L.csa_num_entries(n, m, w) == paging.num_entries(n, m, w)
            assert L.csa_num_eligible(n, m, w) == paging.num_eligible(n, m, w)
    assert L.csa_num_entries(100, 4, 4) == -1
    bt = np.array([7, 3, 11, 0], dtype=np.int32)
    p = bt.ctypes.data_as(ctypes.c_void_p)
    for m in (4, 128):
        for i in range(4 * 256 // m):
            assert L.csa_entry_slot(p, i, m) == paging.entry_slot(bt, i, m)
    for j in (0, 1, 255, 256, 700, 1023):
        assert L.csa_raw_slot(p, j) == paging.raw_slot(bt, j)
    assert L.csa_entry_slot(None, 0, 4) == -1
    assert L.csa_status_string(3) == b"workspace missing or too small"
    assert L.csa_version() >= 1


def _cache(**kw):
    d = dict(ratio=4, window=8, dim=128, rope_dims=64, dtype=csa.BF16, pages=FAKE, scales=None, block_table=FAKE,
             batch=2, bt_stride=4, n_phys=8)
    d.update(kw)
    return csa.CacheDesc(**d)


def _raw(**kw):
    d = dict(dtype=csa.BF16, dim=128, roles=2, kv_pages=FAKE, logit_pages=FAKE, scales=None, block_table=FAKE,
             batch=2, bt_stride=4, n_phys=8)
    d.update(kw)
    return csa.RawDesc(**d)


def _compress(L, cache=None, state=None, **kw):
    a = dict(batch=2, start_pos=FAKE, cu_new=FAKE, total_new=2, max_new=1, kv=FAKE, lg=FAKE, gamma=FAKE, eps=1e-6,
             cs=FAKE, rows=10, slots=FAKE, max_out=1, counts=FAKE)
    a.update(kw)
    c = cache if cache is not None else _cache()
    s = state if state is not None else _raw()
    return L.csa_compress_insert(ctypes.byref(c), ctypes.byref(s), a["batch"], a["start_pos"], a["cu_new"],
                                 a["total_new"], a["max_new"], a["kv"], a["lg"], a["gamma"], a["eps"], a["cs"],
                                 a["rows"], a["slots"], a["max_out"], a["counts"], None)


@pytest.mark.parametrize("bad", [
    dict(cache=_cache(ratio=4, window=4)), dict(cache=_cache(ratio=128, window=8)), dict(cache=_cache(dim=96)),
    dict(cache=_cache(rope_dims=3)), dict(cache=_cache(rope_dims=256)), dict(cache=_cache(dtype=7)),
    dict(cache=_cache(pages=None)), dict(cache=_cache(pages=FAKE + 4)), dict(cache=_cache(dtype=csa.FP8, scales=None)),
    dict(cache=_cache(block_table=None)), dict(cache=_cache(n_phys=0)), dict(cache=_cache(batch=1)),
    dict(state=_raw(dim=64)), dict(state=_raw(roles=1)), dict(state=_raw(dtype=csa.FP8)),
    dict(state=_raw(logit_pages=None)), dict(batch=-1), dict(total_new=-1), dict(start_pos=None), dict(kv=None),
    dict(kv=FAKE + 2), dict(gamma=None), dict(eps=-1.0), dict(eps=float("nan")), dict(cs=None), dict(rows=0),
    dict(max_new=5, max_out=1),
])
def test_compress_validation(L, bad):
    assert _compress(L, **bad) == INVALID


def test_compress_empty_batch_is_ok_without_launch(L):
    assert _compress(L, batch=0, start_pos=None, cu_new=None, total_new=0) == OK


def _index(L, cache=None, **kw):
    a = dict(n_q=2, q_seq=FAKE, q_pos=FAKE, max_elig=1000, q=FAKE, q_dtype=csa.BF16, heads=64, w=FAKE,
             mode=csa.SCORE_WRELU, k=512, out=FAKE, cnt=None, sc=None, ws=FAKE, ws_bytes=None)
    a.update(kw)
    c = cache if cache is not None else _cache()
    if a["ws_bytes"] is None:
        a["ws_bytes"] = L.csa_index_topk_workspace(a["n_q"], a["max_elig"], a["k"], a["heads"])
    return L.csa_index_topk(ctypes.byref(c), a["n_q"], a["q_seq"], a["q_pos"], a["max_elig"], a["q"], a["q_dtype"],
                            a["heads"], a["w"], a["mode"], a["k"], a["out"], a["cnt"], a["sc"], a["ws"],
                            a["ws_bytes"], None)


@pytest.mark.parametrize("bad,code", [
    (dict(k=0), INVALID), (dict(k=2049), INVALID), (dict(heads=0), INVALID), (dict(heads=129), INVALID),
    (dict(mode=5), INVALID), (dict(mode=csa.SCORE_DOT, heads=2), INVALID), (dict(w=None), INVALID),
    (dict(q_dtype=csa.FP8), INVALID), (dict(out=None), INVALID), (dict(max_elig=-1), INVALID),
    (dict(q=FAKE + 8), INVALID), (dict(q_dtype=csa.F32), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE), (dict(ws=FAKE + 16), WORKSPACE),
])
def test_index_validation(L, bad, code):
    assert _index(L, **bad) == code


def test_index_unsupported_shape(L):
    # fp32 cache with a bf16 query, and a too-wide VALU head block
    assert _index(L, cache=_cache(dtype=csa.F32), q_dtype=csa.BF16) == UNSUPPORTED
    assert _index(L, cache=_cache(dim=512), heads=64) == UNSUPPORTED


def test_index_workspace_grows_with_inputs(L):
    a = L.csa_index_topk_workspace(4, 262143, 512, 64)
    b = L.csa_index_topk_workspace(4, 262143 * 2, 512, 64)
    assert 0 < a < b
    assert a >= 4 * 262143 * 12  # keys + candidate pairs


def _attend(L, cache=None, swa=None, **kw):
    a = dict(win=128, n_q=2, q_seq=FAKE, q_pos=FAKE, q=FAKE, q_dtype=csa.BF16, heads=64, topk=FAKE, k=512,
             max_elig=1000, scale=0.05, fuse=1, cs=FAKE, rows=10, out=FAKE, lse=None)
    a.update(kw)
    c = cache if cache is not None else _cache(dim=512)
    s = swa if swa is not None else _raw(dim=512, roles=0, logit_pages=None)
    return L.csa_attend(ctypes.byref(c), ctypes.byref(s), a["win"], a["n_q"], a["q_seq"], a["q_pos"], a["q"],
                        a["q_dtype"], a["heads"], a["topk"], a["k"], a["max_elig"], a["scale"], a["fuse"], a["cs"],
                        a["rows"], a["out"], a["lse"], None, 0, None)


@pytest.mark.parametrize("bad", [
    dict(win=-1), dict(win=1025), dict(heads=0), dict(k=0), dict(k=4096), dict(max_elig=-1),
    dict(scale=float("inf")), dict(fuse=2), dict(cs=None), dict(out=None), dict(q=None), dict(q_dtype=csa.FP8),
    dict(swa=_raw(dim=512, roles=0, logit_pages=None, dtype=csa.F32)), dict(swa=_raw(dim=128, roles=0)),
    dict(swa=_raw(dim=512, roles=2)), dict(cache=_cache(dim=512, dtype=csa.FP8, scales=FAKE),
                                             swa=_raw(dim=512, roles=0, dtype=csa.FP8, scales=None)),
])
def test_attend_validation(L, bad):
    assert _attend(L, **bad) == INVALID


def test_attend_unsupported(L):
    assert _attend(L, cache=_cache(dim=512, dtype=csa.F32), swa=_raw(dim=512, roles=0, dtype=csa.F32),
                   q_dtype=csa.BF16) == UNSUPPORTED


def test_inv_rope_and_table_validation(L):
    assert L.csa_inv_rope(2, 4, 128, 3, FAKE, FAKE, 10, FAKE, None) == INVALID
    assert L.csa_inv_rope(2, 4, 128, 256, FAKE, FAKE, 10, FAKE, None) == INVALID
    assert L.csa_inv_rope(2, 4, 128, 64, None, FAKE, 10, FAKE, None) == INVALID
    assert L.csa_inv_rope(0, 4, 128, 64, None, None, 0, None, None) == OK
    assert L.csa_rope_table(10, 3, 10000.0, FAKE, None) == INVALID
    assert L.csa_rope_table(10, 64, -1.0, FAKE, None) == INVALID
    assert L.csa_rope_table(10, 64, 10000.0, None, None) == INVALID
    assert L.csa_rope_table(0, 64, 10000.0, None, None) == OK


def test_inv_rope_quant_fp8_validation(L):
    f = L.csa_inv_rope_quant_fp8
    good = dict(n_q=2, h=4, dim=512, r=64, pos=FAKE, cs=FAKE, rows=10, x=FAKE, g=128, codes=FAKE, sc=FAKE)

    def call(**kw):
        a = {**good, **kw}
        return f(a["n_q"], a["h"], a["dim"], a["r"], a["pos"], a["cs"], a["rows"], a["x"], a["g"], a["codes"],
                 a["sc"], None)
    for bad in (dict(dim=100), dict(dim=1024), dict(r=3), dict(r=1024), dict(g=4), dict(g=96), dict(g=1024),
                dict(h=0), dict(h=129), dict(n_q=-1), dict(pos=None), dict(x=None), dict(codes=None), dict(sc=None),
                dict(x=FAKE + 8), dict(codes=FAKE + 4), dict(rows=0), dict(cs=None)):
        assert call(**bad) == INVALID, bad
    assert call(dim=64, g=128) == INVALID          # group larger than the row
    assert call(n_q=0, pos=None, x=None, codes=None, sc=None) == OK


def test_prepare_qk_validation(L):
    raw = _raw(dim=512, roles=0, dtype=csa.BF16)
    f = L.csa_prepare_qk

    def call(n=2, h=8, seq=FAKE, pos=FAKE, q=FAKE, qd=csa.BF16, g=FAKE, eps=1e-6, kv=FAKE, swa=raw, r=64, cs=FAKE,
             rows=10, out=FAKE):
        return f(n, h, seq, pos, q, qd, g, eps, kv, ctypes.byref(swa) if swa is not None else None, r, cs, rows, out,
                 None)
    for bad in (dict(h=0), dict(h=129), dict(n=-1), dict(seq=None), dict(q=None), dict(g=None), dict(kv=None),
                dict(out=None), dict(swa=None), dict(qd=csa.F32), dict(r=3), dict(r=1024), dict(cs=None),
                dict(rows=0), dict(eps=-1.0), dict(eps=float("nan")), dict(out=FAKE + 8)):
        assert call(**bad) == INVALID, bad
    assert call(swa=_raw(dim=512, roles=2, dtype=csa.BF16)) == INVALID       # a state descriptor, not a window
    assert call(swa=_raw(dim=100, roles=0, dtype=csa.BF16)) == INVALID
    assert call(qd=csa.BF16, swa=_raw(dim=512, roles=0, dtype=csa.F32)) == INVALID
    assert call(n=0, seq=None, pos=None, q=None, g=None, kv=None, out=None) == OK


def test_compress_pair_validation(L):
    f = L.csa_compress_insert_pair
    good_c, good_s = _cache(dim=512), _raw(dim=512)
    idx_c, idx_s = _cache(dim=128), _raw(dim=128)

    def call(ca=good_c, sa=good_s, cb=idx_c, sb=idx_s, ga=FAKE, gb=FAKE, kva=FAKE, kvb=FAKE, batch=2, eps=1e-6):
        return f(ctypes.byref(ca), ctypes.byref(sa), kva, FAKE, ga, FAKE, 10, ctypes.byref(cb), ctypes.byref(sb), kvb,
                 FAKE, gb, FAKE, 10, batch, FAKE, FAKE, 2, 1, eps, None)
    assert call(cb=_cache(dim=100)) == INVALID
    assert call(sb=_raw(dim=512)) == INVALID          # state of the wrong dim for cache b
    assert call(ga=None) == INVALID and call(gb=None) == INVALID
    assert call(kvb=None) == INVALID and call(kvb=FAKE + 4) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call(batch=0) == OK


def test_compress_index_score_validation(L):
    """Both argument sets checked as for the two calls, plus the decode form: one new token per sequence and
    one query per sequence."""
    f = L.csa_compress_index_score
    good_c, good_s = _cache(dim=512), _raw(dim=512)
    idx_c, idx_s = _cache(dim=128), _raw(dim=128)

    def call(ca=good_c, sa=good_s, cb=idx_c, sb=idx_s, batch=2, total=2, max_new=1, n_q=2, q=FAKE, heads=64,
             w=FAKE, mode=csa.SCORE_WRELU, k=512, ws=FAKE, ws_bytes=1 << 30, gb=FAKE):
        return f(ctypes.byref(ca), ctypes.byref(sa), FAKE, FAKE, FAKE, FAKE, 10, ctypes.byref(cb), ctypes.byref(sb),
                 FAKE, FAKE, gb, FAKE, 10, batch, FAKE, FAKE, total, max_new, 1e-6, n_q, FAKE, FAKE, 1000, q,
                 csa.BF16, heads, w, mode, k, ws, ws_bytes, None)
    assert call(cb=_cache(dim=100)) == INVALID
    assert call(sb=_raw(dim=512)) == INVALID
    assert call(gb=None) == INVALID
    assert call(q=None) == INVALID
    assert call(w=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(ws_bytes=16) == WORKSPACE
    assert call(mode=csa.SCORE_DOT, heads=64) == INVALID
    assert call(n_q=3) == INVALID                     # one query per sequence
    assert call(total=3, max_new=2) == INVALID        # one new token per sequence
    assert call(max_new=2) == INVALID
    assert call(batch=0, total=0, n_q=0) == OK


def test_fp4_cache_validation(L):
    """MXFP4 caches: E8M0 exponents required and 4-byte aligned; scored only by the dim-128 WRELU MFMA path with
    a multiple of 16 heads; never an attention cache or a state/window dtype."""
    fp4 = lambda **kw: _cache(dtype=csa.FP4, scales=FAKE, **kw)
    assert _compress(L, cache=_cache(dtype=csa.FP4, scales=None)) == INVALID
    assert _compress(L, cache=_cache(dtype=csa.FP4, scales=FAKE + 2)) == INVALID
    assert _compress(L, cache=fp4(), state=_raw(dtype=csa.FP4)) == INVALID
    assert _index(L, cache=fp4(), mode=csa.SCORE_DOT, heads=1, w=None) == UNSUPPORTED
    assert _index(L, cache=fp4(), heads=8) == UNSUPPORTED
    assert _index(L, cache=fp4(dim=64)) == UNSUPPORTED
    assert _index(L, cache=fp4(ratio=128, window=128)) == UNSUPPORTED
    assert _attend(L, cache=_cache(dim=512, dtype=csa.FP4, scales=FAKE)) == UNSUPPORTED


def _index_noalloc(L, cache=None, **kw):
    a = dict(n_q=2, q_seq=FAKE, q_pos=FAKE, max_elig=1000, q=FAKE, q_dtype=csa.BF16, heads=64, w=FAKE,
             mode=csa.SCORE_WRELU, k=512, out=FAKE, cnt=None, sc=None)
    a.update(kw)
    c = cache if cache is not None else _cache()
    return L.csa_index_topk_noalloc(ctypes.byref(c), a["n_q"], a["q_seq"], a["q_pos"], a["max_elig"], a["q"],
                                    a["q_dtype"], a["heads"], a["w"], a["mode"], a["k"], a["out"], a["cnt"], a["sc"],
                                    None)


TOO_LARGE = 5


@pytest.mark.parametrize("bad,code", [
    (dict(k=0), INVALID), (dict(heads=129), INVALID), (dict(w=None), INVALID), (dict(out=None), INVALID),
    (dict(max_elig=-1), INVALID), (dict(q_dtype=csa.F32), UNSUPPORTED),
    # beyond the fixed scratch: a 4096-query prefill chunk of 66047 entries, and 4 queries of 2^31-1 entries
    (dict(n_q=4096, max_elig=66047), TOO_LARGE), (dict(n_q=4, max_elig=0x7FFFFFFF), TOO_LARGE),
])
def test_index_noalloc_validation(L, bad, code):
    """Rejected before any HIP call (no scratch lookup, no launch)."""
    assert _index_noalloc(L, **bad) == code


def test_index_noalloc_scratch_holds_decode_sizes(L):
    """The fixed scratch takes the decode workloads: 32 queries of 32767 entries, 4 of 262143."""
    assert L.csa_index_topk_workspace(32, 32767, 512, 64) <= csa.NOALLOC_SCRATCH_BYTES
    assert L.csa_index_topk_workspace(4, 262143, 512, 64) <= csa.NOALLOC_SCRATCH_BYTES
    assert L.csa_index_topk_workspace(4096, 66047, 512, 64) > csa.NOALLOC_SCRATCH_BYTES
    assert L.csa_status_string(TOO_LARGE).startswith(b"request exceeds")


def _attend_q(L, cache=None, swa=None, **kw):
    a = dict(win=128, n_q=2, q_seq=FAKE, q_pos=FAKE, q=FAKE, q_dtype=csa.BF16, heads=64, topk=FAKE, k=512,
             max_elig=1000, scale=0.05, cs=FAKE, rows=10, group=128, codes=FAKE, scales=FAKE, lse=None)
    a.update(kw)
    c = cache if cache is not None else _cache(dim=512)
    s = swa if swa is not None else _raw(dim=512, roles=0, logit_pages=None)
    return L.csa_attend_quant_fp8(ctypes.byref(c), ctypes.byref(s), a["win"], a["n_q"], a["q_seq"], a["q_pos"], a["q"],
                                  a["q_dtype"], a["heads"], a["topk"], a["k"], a["max_elig"], a["scale"], a["cs"],
                                  a["rows"], a["group"], a["codes"], a["scales"], a["lse"], FAKE, 1 << 40, None)


@pytest.mark.parametrize("bad,code", [
    (dict(group=8), INVALID), (dict(group=256), INVALID), (dict(group=48), INVALID), (dict(codes=None), INVALID),
    (dict(scales=None), INVALID), (dict(codes=FAKE + 4), INVALID), (dict(cs=None), INVALID), (dict(heads=0), INVALID),
    (dict(heads=8), UNSUPPORTED),                                  # not a multiple of 16 heads: no fused epilogue
    (dict(cache=_cache(dim=256), swa=_raw(dim=256, roles=0, logit_pages=None)), UNSUPPORTED),
    (dict(cache=_cache(dim=512, dtype=csa.F32), swa=_raw(dim=512, roles=0, logit_pages=None, dtype=csa.F32),
          q_dtype=csa.F32), UNSUPPORTED),
])
def test_attend_quant_fp8_validation(L, bad, code):
    """Rejected before any HIP call."""
    assert _attend_q(L, **bad) == code
