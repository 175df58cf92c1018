"""Python binding of libkvz (ctypes): argument marshalling only.

Every function here has the name of the C entry point it calls (include/kvz.h)
and forwards torch tensors as raw device pointers together with the current
HIP stream.  No arithmetic of the method happens in Python.  If libkvz.so has
not been built, loading fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvz.so")
DEBUG_LIB_PATH = os.path.join(HERE, "libkvz_debug.so")

KVZ_OK, KVZ_ERR_INVALID_ARG, KVZ_ERR_UNSUPPORTED, KVZ_ERR_WORKSPACE, KVZ_ERR_HIP = range(5)
KVZ_BF16, KVZ_F32 = 0, 1
KVZ_AGG_MAX, KVZ_AGG_SUM, KVZ_AGG_RAW_MAX = 0, 1, 2
AGG = {"max": KVZ_AGG_MAX, "sum": KVZ_AGG_SUM, "raw": KVZ_AGG_RAW_MAX}

# every symbol declared in include/kvz.h
SYMBOLS = (
    "kvz_build_id", "kvz_status_string", "kvz_score_chunk_workspace", "kvz_score_chunk", "kvz_score_chunk_ex",
    "kvz_score_chunk_attn_workspace", "kvz_score_chunk_attn", "kvz_score_chunk_noalloc",
    "kvz_keep_count", "kvz_select_workspace", "kvz_select_threshold",
    "kvz_select_heads_workspace", "kvz_select_heads", "kvz_select_tokens_workspace",
    "kvz_select_tokens", "kvz_compact_workspace",
    "kvz_compact", "kvz_head_scores", "kvz_token_scores", "kvz_decode_workspace",
    "kvz_decode_packed", "kvz_prof_enable", "kvz_prof_read",
)

_libs = {}
_use_debug = False


class KvzError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {kvz_status_string(status)} (status {status})")


def use_debug_library(on: bool = True):
    """Route every binding of this module to libkvz_debug.so (the checked
    build: a failed kernel-side check returns KVZ_ERR_INVALID_ARG) or, with
    on=False, back to libkvz.so."""
    global _use_debug
    _use_debug = bool(on)


def lib():
    """The library the bindings call (libkvz.so, or libkvz_debug.so after
    use_debug_library()), loaded once, its signatures declared."""
    key = "debug" if _use_debug else "release"
    if key not in _libs:
        _libs[key] = _open(DEBUG_LIB_PATH if _use_debug else LIB_PATH, _use_debug)
    return _libs[key]


def _open(path, debug):
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7);
    # loading torch first makes libkvz bind to that runtime, so the streams
    # and device pointers torch hands over belong to the runtime that
    # launches the kernels.  Opened the other way round, the process would
    # hold two HIP runtimes and every launch on a torch stream would fail.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
            " (the HIP library is required; there is no CPU fallback)")
    L = ctypes.CDLL(path)
    L.kvz_build_id.argtypes = []
    L.kvz_build_id.restype = ctypes.c_char_p
    from .build import source_digest
    built, want = L.kvz_build_id().decode(), source_digest(debug)
    if built != want:
        raise RuntimeError(
            f"{path} was built from other sources (build id {built[:16]}) than the ones in "
            f"this checkout (digest {want[:16]}): rebuild it with "
            "`python -c 'import __graft_entry__ as g; g.build()'`")
    c_int, c_i64, c_sz, c_f, c_d, c_p = (ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                                         ctypes.c_float, ctypes.c_double, ctypes.c_void_p)
    L.kvz_status_string.argtypes = [c_int]
    L.kvz_status_string.restype = ctypes.c_char_p
    L.kvz_score_chunk_workspace.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
    L.kvz_score_chunk_workspace.restype = c_sz
    L.kvz_score_chunk.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_p, c_p, c_p,
                                  c_f, c_p, c_p, c_sz, c_p]
    L.kvz_score_chunk.restype = c_int
    L.kvz_score_chunk_ex.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_p,
                                     c_p, c_p, c_f, c_p, c_p, c_sz, c_p]
    L.kvz_score_chunk_ex.restype = c_int
    L.kvz_score_chunk_noalloc.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_p, c_p,
                                          c_p, c_f, c_p, c_p]
    L.kvz_score_chunk_noalloc.restype = c_int
    L.kvz_score_chunk_attn_workspace.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
    L.kvz_score_chunk_attn_workspace.restype = c_sz
    L.kvz_score_chunk_attn.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_p, c_p,
                                       c_p, c_p, c_p, c_f, c_p, c_p, c_p, c_sz, c_p]
    L.kvz_score_chunk_attn.restype = c_int
    L.kvz_head_scores.argtypes = [c_p, c_i64, c_int, c_p, c_p]
    L.kvz_head_scores.restype = c_int
    L.kvz_token_scores.argtypes = [c_p, c_i64, c_int, c_p, c_p]
    L.kvz_token_scores.restype = c_int
    L.kvz_decode_workspace.argtypes = [c_i64, c_int, c_int, c_int]
    L.kvz_decode_workspace.restype = c_sz
    L.kvz_decode_packed.argtypes = [c_int, c_i64, c_int, c_int, c_int, c_p, c_p, c_p, c_p, c_f,
                                    c_p, c_p, c_sz, c_p]
    L.kvz_decode_packed.restype = c_int
    L.kvz_keep_count.argtypes = [c_i64, c_d]
    L.kvz_keep_count.restype = c_i64
    L.kvz_select_workspace.argtypes = [c_i64, c_int]
    L.kvz_select_workspace.restype = c_sz
    L.kvz_select_threshold.argtypes = [c_p, c_i64, c_int, c_i64, c_p, c_p, c_p, c_p, c_sz, c_p]
    L.kvz_select_threshold.restype = c_int
    L.kvz_select_heads_workspace.argtypes = [c_i64, c_int]
    L.kvz_select_heads_workspace.restype = c_sz
    L.kvz_select_heads.argtypes = [c_p, c_i64, c_int, c_i64, c_int, c_int, c_p, c_p, c_p, c_p,
                                   c_sz, c_p]
    L.kvz_select_heads.restype = c_int
    L.kvz_select_tokens_workspace.argtypes = [c_i64, c_int]
    L.kvz_select_tokens_workspace.restype = c_sz
    L.kvz_select_tokens.argtypes = [c_p, c_i64, c_int, c_i64, c_p, c_p, c_p, c_p, c_sz, c_p]
    L.kvz_select_tokens.restype = c_int
    L.kvz_compact_workspace.argtypes = [c_i64, c_int]
    L.kvz_compact_workspace.restype = c_sz
    L.kvz_compact.argtypes = [c_int, c_int, c_int, c_i64, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_p,
                              c_p, c_sz, c_p]
    L.kvz_compact.restype = c_int
    L.kvz_prof_enable.argtypes = [c_int, c_int]
    L.kvz_prof_enable.restype = c_int
    L.kvz_prof_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(c_i64), ctypes.POINTER(c_d)]
    L.kvz_prof_read.restype = c_int
    return L


def _check(status, where):
    if status != KVZ_OK:
        raise KvzError(status, where)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KVZ_BF16
    if t.dtype == torch.float32:
        return KVZ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, numel=None, shape=None, device=None):
    """Reject a tensor of the wrong dtype, size or device before any launch:
    the kernels index raw pointers and would run past a short allocation."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {numel}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ws(nbytes, device):
    import torch
    # uint8 storage; the caching allocator returns >= 256-byte aligned blocks
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def kvz_build_id() -> str:
    """sha256 of the sources the loaded library was built from (it equals the
    checkout's digest, or lib() refuses to load)."""
    return lib().kvz_build_id().decode()


def kvz_status_string(status: int) -> str:
    return lib().kvz_status_string(int(status)).decode()


def kvz_keep_count(n_total: int, ratio: float) -> int:
    return int(lib().kvz_keep_count(int(n_total), float(ratio)))


def kvz_score_chunk_workspace(dtype_code, H, G, n_in, d, n_c) -> int:
    return int(lib().kvz_score_chunk_workspace(dtype_code, H, G, n_in, d, n_c))


def kvz_select_workspace(n_heads, n_c) -> int:
    return int(lib().kvz_select_workspace(int(n_heads), int(n_c)))


def kvz_compact_workspace(head_count, n_c) -> int:
    return int(lib().kvz_compact_workspace(int(head_count), int(n_c)))


def kvz_score_chunk(q, k_ctx, k_in, S, n_prompt, scale=None, ws=None, stream=None):
    """One reconstruction chunk of one layer.  q [H][G][n_in][d], k_ctx
    [H][n_c][d], k_in [H][n_in][d] (bf16 or fp32), S [H][n_c] fp32 in/out."""
    return kvz_score_chunk_ex(q, k_ctx, k_in, S, n_prompt, "max", scale, ws, stream)


def kvz_score_chunk_ex(q, k_ctx, k_in, S, n_prompt, agg="max", scale=None, ws=None, stream=None):
    """kvz_score_chunk with aggregation agg in {"max", "sum", "raw"}."""
    import torch
    H, G, n_in, d = q.shape
    n_c = k_ctx.shape[1]
    if tuple(k_ctx.shape) != (H, n_c, d) or tuple(k_in.shape) != (H, n_in, d):
        raise ValueError("shape mismatch between q, k_ctx and k_in")
    if tuple(S.shape) != (H, n_c) or S.dtype != torch.float32:
        raise ValueError("S must be fp32 [H][n_c]")
    if k_ctx.dtype != q.dtype or k_in.dtype != q.dtype:
        raise TypeError("q, k_ctx and k_in must share a dtype")
    dt = _dtype_code(q)
    if scale is None:
        scale = d ** -0.5
    need = kvz_score_chunk_workspace(dt, H, G, n_in, d, n_c)
    if ws is None:
        ws = _ws(need, q.device)
    st = lib().kvz_score_chunk_ex(dt, AGG[agg], H, G, d, n_c, int(n_prompt), n_in, _ptr(q, "q"),
                                  _ptr(k_ctx, "k_ctx"), _ptr(k_in, "k_in"), float(scale),
                                  _ptr(S, "S"), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
                                  _stream(stream))
    _check(st, "kvz_score_chunk_ex")
    return S


NOALLOC_SCRATCH_BYTES = 16 << 20   # KVZ_NOALLOC_SCRATCH_BYTES


def kvz_score_chunk_noalloc(q, k_ctx, k_in, S, n_prompt, scale=None, stream=None):
    """kvz_score_chunk without a workspace: the library's fixed device scratch
    array holds it, and nothing is allocated (for code under graph capture
    or loops that must not allocate).  Calls overlapping on one device race."""
    import torch
    H, G, n_in, d = q.shape
    n_c = k_ctx.shape[1]
    if tuple(k_ctx.shape) != (H, n_c, d) or tuple(k_in.shape) != (H, n_in, d):
        raise ValueError("shape mismatch between q, k_ctx and k_in")
    if tuple(S.shape) != (H, n_c) or S.dtype != torch.float32:
        raise ValueError("S must be fp32 [H][n_c]")
    if k_ctx.dtype != q.dtype or k_in.dtype != q.dtype:
        raise TypeError("q, k_ctx and k_in must share a dtype")
    dt = _dtype_code(q)
    if scale is None:
        scale = d ** -0.5
    st = lib().kvz_score_chunk_noalloc(dt, H, G, d, n_c, int(n_prompt), n_in, _ptr(q, "q"),
                                       _ptr(k_ctx, "k_ctx"), _ptr(k_in, "k_in"), float(scale),
                                       _ptr(S, "S"), _stream(stream))
    _check(st, "kvz_score_chunk_noalloc")
    return S


def kvz_score_chunk_attn_workspace(dtype_code, H, G, n_in, d, n_c) -> int:
    return int(lib().kvz_score_chunk_attn_workspace(dtype_code, H, G, n_in, d, n_c))


def kvz_score_chunk_attn(q, k_ctx, k_in, v_ctx, v_in, S, n_prompt, O=None, scale=None, ws=None,
                         stream=None):
    """kvz_score_chunk plus the chunk's attention output O [H][G][n_in][d]
    fp32 over the values v_ctx [H][n_c][d] and v_in [H][n_in][d].  Returns O."""
    import torch
    H, G, n_in, d = q.shape
    n_c = k_ctx.shape[1]
    if tuple(k_ctx.shape) != (H, n_c, d) or tuple(k_in.shape) != (H, n_in, d):
        raise ValueError("shape mismatch between q, k_ctx and k_in")
    if tuple(v_ctx.shape) != (H, n_c, d) or tuple(v_in.shape) != (H, n_in, d):
        raise ValueError("shape mismatch between k and v")
    if tuple(S.shape) != (H, n_c) or S.dtype != torch.float32:
        raise ValueError("S must be fp32 [H][n_c]")
    if any(t.dtype != q.dtype for t in (k_ctx, k_in, v_ctx, v_in)):
        raise TypeError("q, k and v tensors must share a dtype")
    dt = _dtype_code(q)
    if O is None:
        O = torch.empty(H, G, n_in, d, dtype=torch.float32, device=q.device)
    if tuple(O.shape) != (H, G, n_in, d) or O.dtype != torch.float32:
        raise ValueError("O must be fp32 [H][G][n_in][d]")
    if scale is None:
        scale = d ** -0.5
    need = kvz_score_chunk_attn_workspace(dt, H, G, n_in, d, n_c)
    if ws is None:
        ws = _ws(need, q.device)
    st = lib().kvz_score_chunk_attn(dt, H, G, d, n_c, int(n_prompt), n_in, _ptr(q, "q"),
                                    _ptr(k_ctx, "k_ctx"), _ptr(k_in, "k_in"),
                                    _ptr(v_ctx, "v_ctx"), _ptr(v_in, "v_in"), float(scale),
                                    _ptr(S, "S"), _ptr(O, "O"), _ptr(ws, "ws"),
                                    ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "kvz_score_chunk_attn")
    return O


def kvz_head_scores(S, out=None, stream=None):
    """[n_heads][n_c] fp32 -> [n_heads]: max over each head's tokens."""
    import torch
    _need(S, "S", torch.float32)
    if S.dim() != 2:
        raise ValueError("S must be [n_heads][n_c]")
    n_heads, n_c = S.shape
    if out is None:
        out = torch.empty(n_heads, dtype=torch.float32, device=S.device)
    _need(out, "out", torch.float32, numel=n_heads, device=S.device)
    _check(lib().kvz_head_scores(_ptr(S, "S"), n_heads, n_c, _ptr(out, "out"), _stream(stream)),
           "kvz_head_scores")
    return out


def kvz_token_scores(S, out=None, stream=None):
    """[n_heads][n_c] fp32 -> [n_c]: max over all heads per token."""
    import torch
    _need(S, "S", torch.float32)
    if S.dim() != 2:
        raise ValueError("S must be [n_heads][n_c]")
    n_heads, n_c = S.shape
    if out is None:
        out = torch.empty(n_c, dtype=torch.float32, device=S.device)
    _need(out, "out", torch.float32, numel=n_c, device=S.device)
    _check(lib().kvz_token_scores(_ptr(S, "S"), n_heads, n_c, _ptr(out, "out"), _stream(stream)),
           "kvz_token_scores")
    return out


def kvz_select_threshold(S, K, mask=None, head_offsets=None, tau=None, ws=None, stream=None):
    """Exact top-K over S [n_heads][n_c] (fp32).  Returns (mask uint8 [N],
    head_offsets int64 [n_heads + 1], tau fp32 [1]), all on the device."""
    import torch
    _need(S, "S", torch.float32)
    if S.dim() != 2:
        raise ValueError("S must be [n_heads][n_c]")
    n_heads, n_c = S.shape
    dev = S.device
    if mask is None:
        mask = torch.empty(n_heads * n_c, dtype=torch.uint8, device=dev)
    if head_offsets is None:
        head_offsets = torch.empty(n_heads + 1, dtype=torch.int64, device=dev)
    if tau is None:
        tau = torch.empty(1, dtype=torch.float32, device=dev)
    _need(mask, "mask", torch.uint8, numel=n_heads * n_c, device=dev)
    _need(head_offsets, "head_offsets", torch.int64, numel=n_heads + 1, device=dev)
    _need(tau, "tau", torch.float32, numel=1, device=dev)
    if ws is None:
        ws = _ws(kvz_select_workspace(n_heads, n_c), dev)
    _need(ws, "ws", torch.uint8, device=dev)
    st = lib().kvz_select_threshold(_ptr(S, "S"), n_heads, n_c, int(K), _ptr(mask, "mask"),
                                    _ptr(head_offsets, "head_offsets"), _ptr(tau, "tau"),
                                    _ptr(ws, "ws"), ws.numel() * ws.element_size(),
                                    _stream(stream))
    _check(st, "kvz_select_threshold")
    return mask, head_offsets, tau


def kvz_select_heads_workspace(n_heads, n_c) -> int:
    return int(lib().kvz_select_heads_workspace(int(n_heads), int(n_c)))


def kvz_select_tokens_workspace(n_heads, n_c) -> int:
    return int(lib().kvz_select_tokens_workspace(int(n_heads), int(n_c)))


def _agg_outputs(S, n_keep, mask, head_offsets, keep):
    import torch
    n_heads, n_c = S.shape
    dev = S.device
    if mask is None:
        mask = torch.empty(n_heads * n_c, dtype=torch.uint8, device=dev)
    if head_offsets is None:
        head_offsets = torch.empty(n_heads + 1, dtype=torch.int64, device=dev)
    if keep is None:
        keep = torch.empty(n_keep, dtype=torch.uint8, device=dev)
    _need(mask, "mask", torch.uint8, numel=n_heads * n_c, device=dev)
    _need(head_offsets, "head_offsets", torch.int64, numel=n_heads + 1, device=dev)
    return mask, head_offsets, keep


def kvz_select_heads(S, K_heads, n_sink, n_recent, mask=None, head_offsets=None, head_keep=None,
                     ws=None, stream=None):
    """Head-level eviction over S [n_heads][n_c] (fp32): the K_heads heads
    with the highest max score keep every token, the others their first
    n_sink and last n_recent tokens.  Returns (mask uint8 [N], head_offsets
    int64 [n_heads + 1], head_keep uint8 [n_heads]), all on the device."""
    import torch
    _need(S, "S", torch.float32)
    if S.dim() != 2:
        raise ValueError("S must be [n_heads][n_c]")
    n_heads, n_c = S.shape
    mask, head_offsets, head_keep = _agg_outputs(S, n_heads, mask, head_offsets, head_keep)
    _need(head_keep, "head_keep", torch.uint8, numel=n_heads, device=S.device)
    if ws is None:
        ws = _ws(kvz_select_heads_workspace(n_heads, n_c), S.device)
    _need(ws, "ws", torch.uint8, device=S.device)
    st = lib().kvz_select_heads(_ptr(S, "S"), n_heads, n_c, int(K_heads), int(n_sink),
                                int(n_recent), _ptr(mask, "mask"),
                                _ptr(head_offsets, "head_offsets"), _ptr(head_keep, "head_keep"),
                                _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "kvz_select_heads")
    return mask, head_offsets, head_keep


def kvz_select_tokens(S, K_tokens, mask=None, head_offsets=None, token_keep=None, ws=None,
                      stream=None):
    """Token-level eviction over S [n_heads][n_c] (fp32): the K_tokens
    positions with the highest max score over all heads are kept in every
    head.  Returns (mask uint8 [N], head_offsets int64 [n_heads + 1],
    token_keep uint8 [n_c]), all on the device."""
    import torch
    _need(S, "S", torch.float32)
    if S.dim() != 2:
        raise ValueError("S must be [n_heads][n_c]")
    n_heads, n_c = S.shape
    mask, head_offsets, token_keep = _agg_outputs(S, n_c, mask, head_offsets, token_keep)
    _need(token_keep, "token_keep", torch.uint8, numel=n_c, device=S.device)
    if ws is None:
        ws = _ws(kvz_select_tokens_workspace(n_heads, n_c), S.device)
    _need(ws, "ws", torch.uint8, device=S.device)
    st = lib().kvz_select_tokens(_ptr(S, "S"), n_heads, n_c, int(K_tokens), _ptr(mask, "mask"),
                                 _ptr(head_offsets, "head_offsets"),
                                 _ptr(token_keep, "token_keep"), _ptr(ws, "ws"),
                                 ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "kvz_select_tokens")
    return mask, head_offsets, token_keep


def kvz_compact(k_ctx, v_ctx, mask, head_offsets, k_out, v_out, idx_out, head_begin=0,
                ws=None, stream=None):
    """Pack heads [head_begin, head_begin + k_ctx.shape[0]) of the kept rows.
    k_ctx, v_ctx [head_count][n_c][d]; k_out, v_out [K][d]; idx_out int32 [K]."""
    import torch
    if k_ctx.dim() != 3:
        raise ValueError("k_ctx must be [head_count][n_c][d]")
    head_count, n_c, d = k_ctx.shape
    dt = _dtype_code(k_ctx)
    dev = k_ctx.device
    _need(v_ctx, "v_ctx", k_ctx.dtype, shape=k_ctx.shape, device=dev)
    end = int(head_begin) + head_count
    if int(head_begin) < 0:
        raise ValueError("head_begin must be >= 0")
    _need(mask, "mask", torch.uint8, numel=end * n_c, device=dev)
    _need(head_offsets, "head_offsets", torch.int64, numel=end + 1, device=dev)
    # the packed outputs must hold every row up to the last head's offset;
    # that offset lives on the device, so the check is on the row width and
    # the caller sizes the row count from head_offsets
    for t, nm in ((k_out, "k_out"), (v_out, "v_out")):
        _need(t, nm, k_ctx.dtype, device=dev)
        if t.dim() != 2 or t.shape[1] != d:
            raise ValueError(f"{nm} must be [rows][{d}]")
    _need(idx_out, "idx_out", torch.int32, device=dev)
    if idx_out.dim() != 1 or idx_out.shape[0] != k_out.shape[0] or v_out.shape[0] != k_out.shape[0]:
        raise ValueError("k_out, v_out and idx_out must hold the same number of rows")
    if ws is None:
        ws = _ws(kvz_compact_workspace(head_count, n_c), dev)
    _need(ws, "ws", torch.uint8, device=dev)
    st = lib().kvz_compact(dt, d, n_c, int(head_begin), head_count, _ptr(k_ctx, "k_ctx"),
                           _ptr(v_ctx, "v_ctx"), _ptr(mask, "mask"),
                           _ptr(head_offsets, "head_offsets"), _ptr(k_out, "k_out"),
                           _ptr(v_out, "v_out"), _ptr(idx_out, "idx_out"), _ptr(ws, "ws"),
                           ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "kvz_compact")
    return k_out, v_out, idx_out


def kvz_decode_workspace(n_heads, G, d, max_len) -> int:
    return int(lib().kvz_decode_workspace(int(n_heads), int(G), int(d), int(max_len)))


def kvz_decode_packed(q, k_rows, v_rows, head_offsets, max_len, scale=None, out=None, ws=None,
                      stream=None):
    """Decode attention: q [n_heads][G][d] over each head's rows of the packed
    k_rows/v_rows [rows][d] (head h owns head_offsets[h]..head_offsets[h+1]).
    Returns out [n_heads][G][d] fp32."""
    import torch
    if q.dim() != 3:
        raise ValueError("q must be [n_heads][G][d]")
    n_heads, G, d = q.shape
    if k_rows.dtype != q.dtype or v_rows.dtype != q.dtype:
        raise TypeError("q, k_rows and v_rows must share a dtype")
    if k_rows.dim() != 2 or k_rows.shape[-1] != d or v_rows.shape != k_rows.shape:
        raise ValueError("k_rows/v_rows must be [rows][d] with matching shapes")
    if head_offsets.dtype != torch.int64 or head_offsets.numel() != n_heads + 1:
        raise ValueError("head_offsets must be int64 [n_heads + 1]")
    dt = _dtype_code(q)
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty(n_heads, G, d, dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, shape=(n_heads, G, d), device=q.device)
    if ws is None:
        ws = _ws(kvz_decode_workspace(n_heads, G, d, max_len), q.device)
    st = lib().kvz_decode_packed(dt, n_heads, G, d, int(max_len), _ptr(q, "q"),
                                 _ptr(k_rows, "k_rows"), _ptr(v_rows, "v_rows"),
                                 _ptr(head_offsets, "head_offsets"), float(scale),
                                 _ptr(out, "out"), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
                                 _stream(stream))
    _check(st, "kvz_decode_packed")
    return out


def kvz_prof_enable(on: bool, max_launches: int = 1 << 16):
    _check(lib().kvz_prof_enable(1 if on else 0, int(max_launches)), "kvz_prof_enable")


def kvz_prof_read(name: str):
    """(launches, total_ms) of one kernel name since kvz_prof_enable."""
    n = ctypes.c_int64()
    ms = ctypes.c_double()
    _check(lib().kvz_prof_read(name.encode(), ctypes.byref(n), ctypes.byref(ms)), "kvz_prof_read")
    return int(n.value), float(ms.value)
