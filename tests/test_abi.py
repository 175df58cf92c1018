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


@pytest.mark.parametrize("path", [kvz.LIB_PATH, kvz.DEBUG_LIB_PATH])
def test_nm_shows_exports(path):
    out = os.popen(f"nm -D --defined-only {path}").read()
    for n in _declared():
        assert re.search(rf"\bT {n}\b", out), n


def test_debug_library_loads_and_validates_like_release():
    """libkvz_debug.so carries its own build id (the sources plus its debug
    flag) and rejects bad arguments exactly as libkvz.so does."""
    R = kvz.lib()
    try:
        kvz.use_debug_library(True)
        D = kvz.lib()
        for n in _declared():
            assert hasattr(D, n), n
        assert D.kvz_build_id() != R.kvz_build_id()
        assert D.kvz_score_chunk(0, 0, 4, 128, 100, 4, 20, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE,
                                 1 << 30, None) == kvz.KVZ_ERR_INVALID_ARG
        assert D.kvz_decode_packed(0, 4, 9, 128, 100, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE,
                                   1 << 30, None) == kvz.KVZ_ERR_UNSUPPORTED
    finally:
        kvz.use_debug_library(False)


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
    # 2^24 mask tiles (one 256-thread workgroup each): past the 32-bit launch
    assert kvz.kvz_select_workspace((1 << 24) - 1, 1) > 0
    assert kvz.kvz_select_workspace(1 << 24, 1) == 0
    assert kvz.kvz_select_workspace(1 << 24, 64) == 0     # N = 2^30, 2^24 tiles
    r = kvz.lib().kvz_select_threshold(FAKE, 1 << 24, 64, 1, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert r == kvz.KVZ_ERR_INVALID_ARG
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
    (dict(H=4097), kvz.KVZ_ERR_INVALID_ARG),          # more KV heads than one call takes
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
    assert kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 4096, 4, 2064, 128, 8192) > 0
    assert kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 4097, 4, 2064, 128, 8192) == 0
    assert kvz.kvz_score_chunk_attn_workspace(kvz.KVZ_BF16, 4097, 4, 2064, 128, 8192) == 0
    # exactly the required size passes validation, one byte less does not
    need = kvz.kvz_score_chunk_attn_workspace(kvz.KVZ_BF16, 2, 4, 20, 128, 100)
    assert _attn(wsb=need - 1) == kvz.KVZ_ERR_WORKSPACE


def test_launch_size_limits():
    """Problems past the launches' 32-bit work-item counts are refused before
    any launch; the header's sufficient conditions (H*G*n_in <= 2^29,
    H*n_c <= 2^31, and for the output H*G*n_in*d <= 2^33) always fit."""
    ws = kvz.kvz_score_chunk_workspace
    aws = kvz.kvz_score_chunk_attn_workspace
    BF, F32 = kvz.KVZ_BF16, kvz.KVZ_F32
    # rows: H * R_pad reaches 2^31 (4096 heads of 2^20 rows, 256-row tiles)
    assert ws(BF, 4096, 1, 1 << 20, 128, 64) == 0
    assert ws(F32, 4096, 1, 1 << 20, 128, 64) == 0
    assert _score(H=4096, G=1, n_in=1 << 20, n_prompt=0, n_c=64) == kvz.KVZ_ERR_INVALID_ARG
    assert _attn(H=4096, G=1, n_in=1 << 20, n_prompt=0, n_c=64) == kvz.KVZ_ERR_INVALID_ARG
    # pass-2 grid: 4096 heads x 2^24 keys at d=64 (2^15 workgroups per head)
    assert ws(BF, 4096, 1, 16, 64, 1 << 24) == 0
    assert _score(H=4096, G=1, n_in=16, n_c=1 << 24, d=64) == kvz.KVZ_ERR_INVALID_ARG
    # the sufficient conditions, at their edges and in every dtype and d
    for dt in (BF, F32):
        for d in (64, 128, 256):
            assert ws(dt, 512, 1, 1 << 20, d, 64) > 0              # H*G*n_in = 2^29
            assert ws(dt, 4096, 2, 1 << 16, d, 64) > 0             # H*G*n_in = 2^29
            assert ws(dt, 128, 1, 16, d, min(1 << 24, ((1 << 31) - 1) // (2 * d))) > 0
            assert ws(dt, 4096, 1, 16, d, 1 << 19) > 0             # H*n_c = 2^31
            assert aws(dt, 4096, 1, (1 << 33) // (4096 * d), d, 64) > 0
    # the output merge: H*G*n_in*d/4 float4 lanes past 2^32 (d=256)
    assert ws(BF, 4096, 1, 1 << 17, 256, 64) > 0
    assert aws(BF, 4096, 1, 1 << 17, 256, 64) == 0
    assert _attn(H=4096, G=1, n_in=1 << 17, n_prompt=0, d=256, n_c=64) == kvz.KVZ_ERR_INVALID_ARG


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


def test_head_maxima_head_count_limit():
    # one 1024-thread workgroup per head: n_heads < 2^22 keeps the launch 32-bit
    L = kvz.lib()
    assert L.kvz_head_scores(FAKE, 1 << 22, 1, FAKE, None) == kvz.KVZ_ERR_INVALID_ARG
    assert kvz.kvz_select_heads_workspace((1 << 22) - 1, 1) > 0
    assert kvz.kvz_select_heads_workspace(1 << 22, 1) == 0
    r = L.kvz_select_heads(FAKE, 1 << 22, 1, 1, 0, 0, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert r == kvz.KVZ_ERR_INVALID_ARG


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
    # max_len near INT_MAX: 2^20 segments of 2048 rows, no int overflow
    big = 2**31 - 1
    assert kvz.kvz_decode_workspace(1, 1, 64, big) == 2**20 * 66 * 4
    assert f(nh=15, G=1, d=64, ml=big, wsb=8) == kvz.KVZ_ERR_WORKSPACE
    # grid bounds: (head, segment) workgroups < 2^24, query-head threads < 2^32
    assert f(nh=16, G=1, d=64, ml=big) == kvz.KVZ_ERR_INVALID_ARG
    assert kvz.kvz_decode_workspace(16, 1, 64, big) == 0
    assert f(nh=2**21, G=8, d=256, ml=1) == kvz.KVZ_ERR_INVALID_ARG
    assert kvz.kvz_decode_workspace(2**21, 8, 256, 1) == 0
    assert kvz.kvz_decode_workspace(2**21 - 1, 8, 256, 1) > 0


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
    # positions beyond the int32 range, then a launch of 2^24 scatter
    # workgroups (2^32 work-items) while the positions still fit
    assert f(nc=1 << 22, hc=1 << 9) == kvz.KVZ_ERR_INVALID_ARG
    assert f(nc=1 << 21, hc=1 << 9) == kvz.KVZ_ERR_INVALID_ARG


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


# The Python bindings check dtypes, sizes and devices before any launch.  These
# run on CPU tensors: each bad argument is caught by a check that comes before
# the device-memory check.
torch = pytest.importorskip("torch")


def _t(n, dtype):
    return torch.zeros(n, dtype=dtype)


@pytest.mark.parametrize("case", ["S_bf16", "S_1d", "mask_short", "mask_i8", "offs_short",
                                  "offs_i32", "tau_f64"])
def test_select_binding_rejects(case):
    S = torch.zeros(4, 10, dtype=torch.float32)
    kw = {}
    if case == "S_bf16":
        S = S.to(torch.bfloat16)
    elif case == "S_1d":
        S = torch.zeros(40, dtype=torch.float32)
    elif case == "mask_short":
        kw["mask"] = _t(39, torch.uint8)
    elif case == "mask_i8":
        kw["mask"] = _t(40, torch.int8)
    elif case == "offs_short":
        kw["head_offsets"] = _t(4, torch.int64)
    elif case == "offs_i32":
        kw["head_offsets"] = _t(5, torch.int32)
    elif case == "tau_f64":
        kw["tau"] = _t(1, torch.float64)
    full = dict(mask=_t(40, torch.uint8), head_offsets=_t(5, torch.int64), tau=_t(1, torch.float32))
    full.update(kw)
    name = {"S_bf16": "S", "S_1d": "S", "mask_short": "mask", "mask_i8": "mask",
            "offs_short": "head_offsets", "offs_i32": "head_offsets", "tau_f64": "tau"}[case]
    with pytest.raises((TypeError, ValueError), match=name) as e:
        kvz.kvz_select_threshold(S, 5, **full)
    assert "device tensor" not in str(e.value)


def test_select_binding_reaches_device_check_when_valid():
    """Control for the cases above: valid CPU arguments fail only at the
    device-memory check."""
    with pytest.raises(ValueError, match="device tensor"):
        kvz.kvz_select_threshold(torch.zeros(4, 10), 5, _t(40, torch.uint8), _t(5, torch.int64),
                                 _t(1, torch.float32), ws=_t(256, torch.uint8))


@pytest.mark.parametrize("case", ["v_shape", "v_dtype", "mask_short", "mask_f32", "offs_short",
                                  "offs_i32", "kout_dtype", "kout_width", "vout_rows", "idx_i64",
                                  "idx_rows", "begin_neg", "mask_short_for_begin"])
def test_compact_binding_rejects(case):
    H, n_c, d, K = 2, 10, 64, 6
    kc = torch.zeros(H, n_c, d, dtype=torch.bfloat16)
    a = dict(k_ctx=kc, v_ctx=kc.clone(), mask=_t(H * n_c, torch.uint8),
             head_offsets=_t(H + 1, torch.int64), k_out=torch.zeros(K, d, dtype=torch.bfloat16),
             v_out=torch.zeros(K, d, dtype=torch.bfloat16), idx_out=_t(K, torch.int32),
             head_begin=0)
    if case == "v_shape":
        a["v_ctx"] = torch.zeros(H, n_c, d + 64, dtype=torch.bfloat16)
    elif case == "v_dtype":
        a["v_ctx"] = kc.float()
    elif case == "mask_short":
        a["mask"] = _t(H * n_c - 1, torch.uint8)
    elif case == "mask_f32":
        a["mask"] = _t(H * n_c, torch.float32)
    elif case == "offs_short":
        a["head_offsets"] = _t(H, torch.int64)
    elif case == "offs_i32":
        a["head_offsets"] = _t(H + 1, torch.int32)
    elif case == "kout_dtype":
        a["k_out"] = torch.zeros(K, d, dtype=torch.float32)
    elif case == "kout_width":
        a["k_out"] = torch.zeros(K, d // 2, dtype=torch.bfloat16)
    elif case == "vout_rows":
        a["v_out"] = torch.zeros(K - 1, d, dtype=torch.bfloat16)
    elif case == "idx_i64":
        a["idx_out"] = _t(K, torch.int64)
    elif case == "idx_rows":
        a["idx_out"] = _t(K + 1, torch.int32)
    elif case == "begin_neg":
        a["head_begin"] = -1
    elif case == "mask_short_for_begin":
        a["head_begin"] = 3       # heads 3..4 need a mask of 5 * n_c entries
    name = {"v_shape": "v_ctx", "v_dtype": "v_ctx", "mask_short": "mask", "mask_f32": "mask",
            "offs_short": "head_offsets", "offs_i32": "head_offsets", "kout_dtype": "k_out",
            "kout_width": "k_out", "vout_rows": "rows", "idx_i64": "idx_out", "idx_rows": "rows",
            "begin_neg": "head_begin", "mask_short_for_begin": "mask"}[case]
    with pytest.raises((TypeError, ValueError), match=name) as e:
        kvz.kvz_compact(**a, ws=_t(256, torch.uint8))
    assert "device tensor" not in str(e.value)


def test_compact_binding_reaches_device_check_when_valid():
    kc = torch.zeros(2, 10, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        kvz.kvz_compact(kc, kc.clone(), _t(20, torch.uint8), _t(3, torch.int64),
                        torch.zeros(6, 64, dtype=torch.bfloat16),
                        torch.zeros(6, 64, dtype=torch.bfloat16), _t(6, torch.int32),
                        ws=_t(256, torch.uint8))


@pytest.mark.parametrize("fn", ["head", "token"])
@pytest.mark.parametrize("case", ["S_bf16", "S_1d", "out_short", "out_f64"])
def test_head_token_binding_rejects(fn, case):
    S = torch.zeros(4, 10, dtype=torch.float32)
    out = None
    if case == "S_bf16":
        S = S.to(torch.bfloat16)
    elif case == "S_1d":
        S = torch.zeros(40, dtype=torch.float32)
    elif case == "out_short":
        out = _t(3 if fn == "head" else 9, torch.float32)
    elif case == "out_f64":
        out = _t(4 if fn == "head" else 10, torch.float64)
    f = kvz.kvz_head_scores if fn == "head" else kvz.kvz_token_scores
    name = "out" if case.startswith("out") else "S"
    with pytest.raises((TypeError, ValueError), match=name) as e:
        f(S, out=out)
    assert "device tensor" not in str(e.value)
    if out is not None or case != "S_bf16":
        return
    with pytest.raises(ValueError, match="device tensor"):   # control: valid arguments
        f(torch.zeros(4, 10))


def _noalloc(**kw):
    a = dict(dt=0, H=2, G=4, d=128, n_c=100, n_prompt=4, n_in=20, q=FAKE, kc=FAKE, ki=FAKE,
             scale=0.1, S=FAKE, stream=None)
    a.update(kw)
    return kvz.lib().kvz_score_chunk_noalloc(a["dt"], a["H"], a["G"], a["d"], a["n_c"],
                                             a["n_prompt"], a["n_in"], a["q"], a["kc"], a["ki"],
                                             a["scale"], a["S"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), kvz.KVZ_ERR_UNSUPPORTED), (dict(dt=7), kvz.KVZ_ERR_UNSUPPORTED),
    (dict(H=0), kvz.KVZ_ERR_INVALID_ARG), (dict(n_prompt=21), kvz.KVZ_ERR_INVALID_ARG),
    (dict(q=None), kvz.KVZ_ERR_INVALID_ARG), (dict(S=MIS), kvz.KVZ_ERR_INVALID_ARG),
    (dict(scale=0.0), kvz.KVZ_ERR_INVALID_ARG), (dict(d=256, n_c=4194304), kvz.KVZ_ERR_INVALID_ARG),
    # 4 KV heads x 64 query heads x 8192 rows need ~38 MB of scratch: more
    # than the fixed array holds, rejected before any launch
    (dict(H=4, G=64, n_in=8192, n_prompt=16, n_c=1000), kvz.KVZ_ERR_WORKSPACE),
])
def test_noalloc_validation(kw, status):
    assert _noalloc(**kw) == status


def test_noalloc_scratch_covers_the_workloads():
    """The fixed scratch array holds the workspace of every workload's chunk
    (8 KV heads; G = 4 / 5 / 2; 2K / 2K / 1K-token chunks of 128K / 120K /
    170K contexts), and the rejection above is for a larger problem."""
    cap = kvz.NOALLOC_SCRATCH_BYTES
    for (G, n_in, d, n_c) in ((4, 2064, 128, 131072), (5, 2064, 128, 120000),
                              (2, 1040, 256, 170000), (4, 2064, 128, 8192), (2, 136, 64, 512)):
        need = kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 8, G, n_in, d, n_c)
        assert 0 < need <= cap, (G, n_in, d, n_c, need)
    assert kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 32, 4, 2064, 128, 131072) <= cap
    assert kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16, 4, 64, 8192, 128, 1000) > cap
    hdr = open(os.path.join(ROOT, "include", "kvz.h")).read()
    assert re.search(r"#define KVZ_NOALLOC_SCRATCH_BYTES \(16u << 20\)", hdr)


def test_structured_select_validation():
    L = kvz.lib()
    fh = lambda S=FAKE, nh=4, nc=10, K=2, s=1, r=1, m=FAKE, o=FAKE, k=FAKE, ws=FAKE, wsb=1 << 30: \
        L.kvz_select_heads(S, nh, nc, K, s, r, m, o, k, ws, wsb, None)
    assert fh(K=5) == kvz.KVZ_ERR_INVALID_ARG
    assert fh(K=-1) == kvz.KVZ_ERR_INVALID_ARG
    assert fh(s=-1) == kvz.KVZ_ERR_INVALID_ARG
    assert fh(r=-2) == kvz.KVZ_ERR_INVALID_ARG
    assert fh(nh=0) == kvz.KVZ_ERR_INVALID_ARG
    assert fh(S=None) == kvz.KVZ_ERR_INVALID_ARG
    assert fh(k=None) == kvz.KVZ_ERR_INVALID_ARG
    assert fh(m=P(4097)) == kvz.KVZ_ERR_INVALID_ARG      # mask must be 16-byte aligned
    assert fh(o=P(4100)) == kvz.KVZ_ERR_INVALID_ARG
    assert fh(wsb=8) == kvz.KVZ_ERR_WORKSPACE
    assert fh(nh=1 << 20, nc=1 << 12) == kvz.KVZ_ERR_INVALID_ARG
    ft = lambda S=FAKE, nh=4, nc=10, K=3, m=FAKE, o=FAKE, k=FAKE, ws=FAKE, wsb=1 << 30: \
        L.kvz_select_tokens(S, nh, nc, K, m, o, k, ws, wsb, None)
    assert ft(K=11) == kvz.KVZ_ERR_INVALID_ARG
    assert ft(K=-1) == kvz.KVZ_ERR_INVALID_ARG
    assert ft(S=MIS) == kvz.KVZ_ERR_INVALID_ARG
    assert ft(k=None) == kvz.KVZ_ERR_INVALID_ARG
    assert ft(ws=P(4096 + 128)) == kvz.KVZ_ERR_INVALID_ARG
    assert ft(wsb=8) == kvz.KVZ_ERR_WORKSPACE
    assert kvz.kvz_select_heads_workspace(256, 131072) > 0
    assert kvz.kvz_select_tokens_workspace(256, 131072) > 0
    assert kvz.kvz_select_heads_workspace(0, 10) == 0
    assert kvz.kvz_select_tokens_workspace(1 << 20, 1 << 12) == 0


@pytest.mark.parametrize("fn", ["heads", "tokens"])
def test_structured_select_binding_rejects(fn):
    S = torch.zeros(4, 10)
    f = (lambda **kw: kvz.kvz_select_heads(S, 2, 1, 1, **kw)) if fn == "heads" else \
        (lambda **kw: kvz.kvz_select_tokens(S, 3, **kw))
    keep_n = 4 if fn == "heads" else 10
    keep_name = "head_keep" if fn == "heads" else "token_keep"
    for kw, name in ((dict(mask=_t(39, torch.uint8)), "mask"),
                     (dict(head_offsets=_t(5, torch.int32)), "head_offsets"),
                     ({keep_name: _t(keep_n - 1, torch.uint8)}, keep_name),
                     ({keep_name: _t(keep_n, torch.int8)}, keep_name)):
        with pytest.raises((TypeError, ValueError), match=name) as e:
            f(**kw)
        assert "device tensor" not in str(e.value)


@pytest.mark.parametrize("case", ["q_2d", "k_1d", "v_shape", "kv_dtype", "offs_short", "offs_i32",
                                  "out_bf16", "out_shape"])
def test_decode_binding_rejects(case):
    n_heads, G, d, rows = 3, 2, 64, 50
    a = dict(q=torch.zeros(n_heads, G, d, dtype=torch.bfloat16),
             k_rows=torch.zeros(rows, d, dtype=torch.bfloat16),
             v_rows=torch.zeros(rows, d, dtype=torch.bfloat16),
             head_offsets=_t(n_heads + 1, torch.int64), max_len=rows,
             out=torch.zeros(n_heads, G, d, dtype=torch.float32))
    if case == "q_2d":
        a["q"] = torch.zeros(n_heads * G, d, dtype=torch.bfloat16)
    elif case == "k_1d":
        a["k_rows"] = torch.zeros(rows * d, dtype=torch.bfloat16)
    elif case == "v_shape":
        a["v_rows"] = torch.zeros(rows - 1, d, dtype=torch.bfloat16)
    elif case == "kv_dtype":
        a["k_rows"] = a["k_rows"].float()
    elif case == "offs_short":
        a["head_offsets"] = _t(n_heads, torch.int64)
    elif case == "offs_i32":
        a["head_offsets"] = _t(n_heads + 1, torch.int32)
    elif case == "out_bf16":
        a["out"] = torch.zeros(n_heads, G, d, dtype=torch.bfloat16)
    elif case == "out_shape":
        a["out"] = torch.zeros(n_heads, G, d - 1, dtype=torch.float32)
    name = {"q_2d": "q", "k_1d": "k_rows", "v_shape": "v_rows", "kv_dtype": "share a dtype",
            "offs_short": "head_offsets", "offs_i32": "head_offsets", "out_bf16": "out",
            "out_shape": "out"}[case]
    with pytest.raises((TypeError, ValueError), match=name) as e:
        kvz.kvz_decode_packed(**a, ws=_t(256, torch.uint8))
    assert "device tensor" not in str(e.value)


def test_decode_binding_reaches_device_check_when_valid():
    with pytest.raises(ValueError, match="device tensor"):
        kvz.kvz_decode_packed(torch.zeros(3, 2, 64, dtype=torch.bfloat16),
                              torch.zeros(50, 64, dtype=torch.bfloat16),
                              torch.zeros(50, 64, dtype=torch.bfloat16), _t(4, torch.int64), 50,
                              out=torch.zeros(3, 2, 64, dtype=torch.float32),
                              ws=_t(256, torch.uint8))
