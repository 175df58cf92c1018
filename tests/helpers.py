"""Shared helpers of the test-suite (device transfer, tolerance checks)."""
import math

import numpy as np

from oracle import ras

# score tolerance for bf16 inputs with fp32 accumulation (allclose form)
ATOL, RTOL = 2e-3, 1e-2


def to_dev(x, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def bits_of(t):
    """Device bf16 tensor -> uint16 numpy bit patterns."""
    import torch
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_scores_close(gpu, ref, atol=ATOL, rtol=RTOL, what="S"):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    msg = (f"{what}: {int(bad.sum())} of {bad.size} outside |d| <= {atol} + {rtol}|ref|; "
           f"max abs {err.max():.3e}, max rel (ref>1e-3) "
           f"{(rel[np.abs(ref) > 1e-3].max() if np.any(np.abs(ref) > 1e-3) else 0):.3e}")
    print(msg, flush=True)
    assert not bad.any(), msg
    return err.max()


def oracle_layer_scores(gen, layer, heads, chunk_ids=None):
    """fp64 oracle scores [len(heads)][n_c] of one layer over the given chunks."""
    wl = gen.wl
    kc, _ = gen.context(layer, heads)
    kc64 = ras.to_f64(kc, wl.dtype)
    S = np.zeros((len(heads), wl.n_ctx))
    ids = range(len(wl.chunks())) if chunk_ids is None else chunk_ids
    scale = 1.0 / math.sqrt(wl.head_dim)
    for k in ids:
        q, kin = gen.chunk_inputs(layer, k, heads)
        ras.score_chunk(ras.to_f64(q, wl.dtype), kc64, ras.to_f64(kin, wl.dtype), scale, S)
    return S
