"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, sizes workspaces, computes keep counts, and rejects bad arguments
before launching anything (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

from attention_score_reduction_amd import kvz

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "kvz.h")).read()
    return sorted(set(re.findall(r"KVZ_API\s+[\w\s\*]*?\b(kvz_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = kvz.lib()
    names = _declared()
    assert len(names) == len(set(kvz.SYMBOLS))
    assert sorted(kvz.SYMBOLS) == names
    for n in names:
        assert hasattr(L, n), n


def test_nm_shows_exports():
    out = os.popen(f"nm -D --defined-only {kvz.LIB_PATH}").read()
    for n in _declared():
        assert re.search(rf"\bT {n}\b", out), n


@pytest.mark.parametrize("N,r,K", [(512, 0.3, 154), (2097152, 0.3, 629146), (33554432, 0.3, 10066330),
                                   (46080000, 0.25, 11520000), (65280000, 0.4, 26112000),
                                   (10, 0.0, 0), (10, 1.0, 10), (7, 0.5, 4), (0, 0.5, 0), (9, -1, 0)])
def test_keep_count(N, r, K):
    assert kvz.kvz_keep_count(N, r) == K


def test_status_strings():
    for s in range(5):
        assert kvz.kvz_status_string(s)
    assert kvz.kvz_status_string(99) == "unknown status"


def test_workspace_queries():
    assert kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 8, 4, 2064, 128, 131072) > 0
    assert kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 0, 4, 2064, 128, 131072) == 0
    assert kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 8, 4, 2064, 128, 0) == 0
    assert kvz.kvz_select_workspace(256, 131072) > 0
    assert kvz.kvz_select_workspace(0, 10) == 0
    assert kvz.kvz_select_workspace(1 << 20, 1 << 12) == 0  # N >= 2^31
    assert kvz.kvz_compact_workspace(8, 131072) > 0
    assert kvz.kvz_compact_workspace(0, 1) == 0


P = ctypes.c_void_p
FAKE = P(4096)      # aligned, never dereferenced: validation fails first
MIS = P(4098)       # misaligned


def _score(**kw):
    a = dict(dt=0, H=2, G=4, d=128, n_c=100, n_prompt=4, n_in=20, q=FAKE, kc=FAKE, ki=FAKE,
             scale=0.1, S=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return kvz.lib().kvz_score_chunk(a["dt"], a["H"], a["G"], a["d"], a["n_c"], a["n_prompt"],
                                     a["n_in"], a["q"], a["kc"], a["ki"], a["scale"], a["S"],
                                     a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), kvz.KVZ_ERR_UNSUPPORTED), (dict(dt=7), kvz.KVZ_ERR_UNSUPPORTED),
    (dict(H=0), kvz.KVZ_ERR_INVALID_ARG), (dict(n_in=0), kvz.KVZ_ERR_INVALID_ARG),
    (dict(n_c=0), kvz.KVZ_ERR_INVALID_ARG), (dict(n_prompt=21), kvz.KVZ_ERR_INVALID_ARG),
    (dict(n_prompt=-1), kvz.KVZ_ERR_INVALID_ARG), (dict(q=None), kvz.KVZ_ERR_INVALID_ARG),
    (dict(S=None), kvz.KVZ_ERR_INVALID_ARG), (dict(kc=MIS), kvz.KVZ_ERR_INVALID_ARG),
    (dict(ws=P(4096 + 64)), kvz.KVZ_ERR_INVALID_ARG), (dict(scale=0.0), kvz.KVZ_ERR_INVALID_ARG),
    (dict(scale=float("nan")), kvz.KVZ_ERR_INVALID_ARG), (dict(scale=-1.0), kvz.KVZ_ERR_INVALID_ARG),
    (dict(wsb=16), kvz.KVZ_ERR_WORKSPACE), (dict(G=1 << 11, n_in=1 << 10), kvz.KVZ_ERR_INVALID_ARG),
    # one head's keys past 2 GiB (the 32-bit range of the buffer loads)
    (dict(d=256, n_c=4194304), kvz.KVZ_ERR_INVALID_ARG),
    (dict(d=128, n_c=8388608), kvz.KVZ_ERR_INVALID_ARG),
])
def test_score_validation(kw, status):
    assert _score(**kw) == status


def _attn(**kw):
    a = dict(dt=0, H=2, G=4, d=128, n_c=100, n_prompt=4, n_in=20, q=FAKE, kc=FAKE, ki=FAKE,
             vc=FAKE, vi=FAKE, scale=0.1, S=FAKE, O=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return kvz.lib().kvz_score_chunk_attn(a["dt"], a["H"], a["G"], a["d"], a["n_c"], a["n_prompt"],
                                          a["n_in"], a["q"], a["kc"], a["ki"], a["vc"], a["vi"],
                                          a["scale"], a["S"], a["O"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), kvz.KVZ_ERR_UNSUPPORTED), (dict(dt=7), kvz.KVZ_ERR_UNSUPPORTED),
    (dict(H=0), kvz.KVZ_ERR_INVALID_ARG), (dict(n_prompt=21), kvz.KVZ_ERR_INVALID_ARG),
    (dict(vc=None), kvz.KVZ_ERR_INVALID_ARG), (dict(vi=None), kvz.KVZ_ERR_INVALID_ARG),
    (dict(O=None), kvz.KVZ_ERR_INVALID_ARG), (dict(vi=MIS), kvz.KVZ_ERR_INVALID_ARG),
    (dict(O=MIS), kvz.KVZ_ERR_INVALID_ARG), (dict(scale=0.0), kvz.KVZ_ERR_INVALID_ARG),
    (dict(wsb=16), kvz.KVZ_ERR_WORKSPACE), (dict(d=256, n_c=4194304), kvz.KVZ_ERR_INVALID_ARG),
])
def test_score_attn_validation(kw, status):
    assert _attn(**kw) == status


def test_score_attn_workspace_covers_score_workspace():
    for dt, d in ((kvz.KVZ_BF16, 128), (kvz.KVZ_BF16, 256), (kvz.KVZ_F32, 64)):
        a = kvz.kvz_score_chunk_attn_workspace(dt, 8, 4, 2064, d, 131072)
        s = kvz.kvz_score_chunk_workspace(dt, 8, 4, 2064, d, 131072)
        assert a >= s > 0
    assert kvz.kvz_score_chunk_attn_workspace(kvz.KVZ_BF16, 8, 4, 2064, 96, 131072) == 0
    assert kvz.kvz_score_chunk_attn_workspace(kvz.KVZ_BF16, 8, 4, 2064, 256, 4194304) == 0
    assert kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 8, 4, 2064, 256, 4194304) == 0
    assert kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 8, 4, 2064, 256, 4194303) > 0
    # exactly the required size passes validation, one byte less does not
    need = kvz.kvz_score_chunk_attn_workspace(kvz.KVZ_BF16, 2, 4, 20, 128, 100)
    assert _attn(wsb=need - 1) == kvz.KVZ_ERR_WORKSPACE


def test_score_ex_rejects_unknown_aggregation():
    L = kvz.lib()
    r = L.kvz_score_chunk_ex(0, 7, 2, 4, 128, 100, 4, 20, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE,
                             1 << 30, None)
    assert r == kvz.KVZ_ERR_UNSUPPORTED


def test_head_token_validation():
    L = kvz.lib()
    assert L.kvz_head_scores(None, 4, 10, FAKE, None) == kvz.KVZ_ERR_INVALID_ARG
    assert L.kvz_head_scores(FAKE, 0, 10, FAKE, None) == kvz.KVZ_ERR_INVALID_ARG
    assert L.kvz_head_scores(MIS, 4, 10, FAKE, None) == kvz.KVZ_ERR_INVALID_ARG
    assert L.kvz_token_scores(FAKE, 4, 0, FAKE, None) == kvz.KVZ_ERR_INVALID_ARG
    assert L.kvz_token_scores(FAKE, 4, 10, None, None) == kvz.KVZ_ERR_INVALID_ARG


def test_decode_validation():
    L = kvz.lib()
    f = lambda dt=0, nh=4, G=4, d=128, ml=100, q=FAKE, off=FAKE, out=FAKE, sc=0.1, ws=FAKE, wsb=1 << 30: \
        L.kvz_decode_packed(dt, nh, G, d, ml, q, FAKE, FAKE, off, sc, out, ws, wsb, None)
    assert f(G=9) == kvz.KVZ_ERR_UNSUPPORTED
    assert f(G=0) == kvz.KVZ_ERR_UNSUPPORTED
    assert f(d=96) == kvz.KVZ_ERR_UNSUPPORTED
    assert f(nh=0) == kvz.KVZ_ERR_INVALID_ARG
    assert f(ml=0) == kvz.KVZ_ERR_INVALID_ARG
    assert f(q=None) == kvz.KVZ_ERR_INVALID_ARG
    assert f(q=MIS) == kvz.KVZ_ERR_INVALID_ARG
    assert f(off=P(4100)) == kvz.KVZ_ERR_INVALID_ARG
    assert f(sc=-1.0) == kvz.KVZ_ERR_INVALID_ARG
    assert f(wsb=8) == kvz.KVZ_ERR_WORKSPACE
    assert kvz.kvz_decode_workspace(256, 4, 128, 131072) > 0
    assert kvz.kvz_decode_workspace(256, 9, 128, 131072) == 0


def test_select_validation():
    L = kvz.lib()
    f = lambda S=FAKE, nh=4, nc=10, K=5, m=FAKE, o=FAKE, t=FAKE, ws=FAKE, wsb=1 << 30: \
        L.kvz_select_threshold(S, nh, nc, K, m, o, t, ws, wsb, None)
    assert f(K=41) == kvz.KVZ_ERR_INVALID_ARG
    assert f(K=-1) == kvz.KVZ_ERR_INVALID_ARG
    assert f(nh=0) == kvz.KVZ_ERR_INVALID_ARG
    assert f(S=None) == kvz.KVZ_ERR_INVALID_ARG
    assert f(S=MIS) == kvz.KVZ_ERR_INVALID_ARG
    assert f(o=P(4100)) == kvz.KVZ_ERR_INVALID_ARG
    assert f(wsb=8) == kvz.KVZ_ERR_WORKSPACE
    assert f(nh=1 << 20, nc=1 << 12) == kvz.KVZ_ERR_INVALID_ARG


def test_compact_validation():
    L = kvz.lib()
    f = lambda dt=0, d=128, nc=10, hb=0, hc=2, kc=FAKE, vc=FAKE, ws=FAKE, wsb=1 << 30, idx=FAKE: \
        L.kvz_compact(dt, d, nc, hb, hc, kc, vc, FAKE, FAKE, FAKE, FAKE, idx, ws, wsb, None)
    assert f(d=100) == kvz.KVZ_ERR_UNSUPPORTED
    assert f(dt=3) == kvz.KVZ_ERR_UNSUPPORTED
    assert f(hb=-1) == kvz.KVZ_ERR_INVALID_ARG
    assert f(hc=0) == kvz.KVZ_ERR_INVALID_ARG
    assert f(kc=None) == kvz.KVZ_ERR_INVALID_ARG
    assert f(vc=MIS) == kvz.KVZ_ERR_INVALID_ARG
    assert f(idx=P(4098)) == kvz.KVZ_ERR_INVALID_ARG
    assert f(wsb=8) == kvz.KVZ_ERR_WORKSPACE


def test_prof_read_rejects_unknown_name():
    n, ms = ctypes.c_int64(), ctypes.c_double()
    assert kvz.lib().kvz_prof_read(b"nope", ctypes.byref(n), ctypes.byref(ms)) == kvz.KVZ_ERR_INVALID_ARG
    assert kvz.lib().kvz_prof_read(b"score_pass1", ctypes.byref(n), ctypes.byref(ms)) == kvz.KVZ_OK
    assert n.value == 0


def test_package_exports_every_binding():
    """Every C entry point with a Python wrapper is reachable from the package."""
    import attention_score_reduction_amd as pkg
    for n in kvz.SYMBOLS:
        if hasattr(kvz, n):
            assert hasattr(pkg, n), n
