"""kvz_score_chunk_noalloc (fixed device scratch, no allocation) against
kvz_score_chunk (caller workspace) through the C ABI: calls in a row, each
with a smaller problem than the one before (the first fills 89% of the
16 MiB scratch), each bit-identical to the workspace call (the same kernels
and launch plan run on the same inputs)."""
import math

import numpy as np
import pytest

from attention_score_reduction_amd import kvz
from attention_score_reduction_amd.inputs import HostGen, Workload
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(wl, chunk_ids):
    gen = HostGen(wl)
    kc, _ = gen.context(0)
    kc_d = to_dev(kc, wl.dtype)
    S_ws = torch.zeros(wl.heads, wl.n_ctx, dtype=torch.float32, device="cuda")
    S_na = torch.full((wl.heads, wl.n_ctx), 0.0, dtype=torch.float32, device="cuda")
    scale = 1 / math.sqrt(wl.head_dim)
    for k in chunk_ids:
        q, kin = gen.chunk_inputs(0, k)
        qd, kd = to_dev(q, wl.dtype), to_dev(kin, wl.dtype)
        kvz.kvz_score_chunk(qd, kc_d, kd, S_ws, wl.n_prompt, scale)
        kvz.kvz_score_chunk_noalloc(qd, kc_d, kd, S_na, wl.n_prompt, scale)
    torch.cuda.synchronize()
    return S_ws.cpu().numpy(), S_na.cpu().numpy()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_call_twice_shrinking(dtype):
    # 32 KV heads x 8 query heads x 2064 rows: the bf16 plan needs 14.9 MB
    fill = Workload("na_fill", 53, 1, 32, 8, 128, 2048, 2048, 16, 0.3, dtype=dtype)
    need = kvz.kvz_score_chunk_workspace(kvz.KVZ_BF16 if dtype == "bf16" else kvz.KVZ_F32,
                                         32, 8, 2064, 128, 2048)
    assert need <= kvz.NOALLOC_SCRATCH_BYTES
    big = Workload("na_big", 51, 1, 4, 4, 128, 6000, 1500, 16, 0.3, dtype=dtype,
                   key_lognormal_sigma=0.5, sink=True)
    small = Workload("na_small", 52, 1, 2, 2, 64, 900, 300, 8, 0.3, dtype=dtype, sink=True)
    for wl, ids in ((fill, [0]), (big, [0, 3]), (small, [0, 2])):
        a, b = _case(wl, ids)
        assert np.array_equal(a, b), f"{wl.name}: noalloc scores differ from the workspace call"
        assert np.all(a > 0) and np.all(a <= 1)


def test_noalloc_calls_captured_in_a_graph():
    """The callers this entry point is for include code under HIP graph
    capture: three chunk calls captured into one graph (after a first,
    uncaptured call has set up the scratch address), then replayed three
    times with eager work between the replays; every replay gives the eager
    result bit for bit (the scoring path records no memset node)."""
    wl = Workload("na_graph", 54, 1, 4, 4, 128, 3000, 1000, 16, 0.3, key_lognormal_sigma=0.5)
    gen = HostGen(wl)
    kc, _ = gen.context(0)
    kc_d = to_dev(kc, wl.dtype)
    scale = 1 / math.sqrt(wl.head_dim)
    chunks = []
    for k in range(len(wl.chunks())):
        q, kin = gen.chunk_inputs(0, k)
        chunks.append((to_dev(q, wl.dtype), to_dev(kin, wl.dtype)))
    S_eager = torch.zeros(wl.heads, wl.n_ctx, dtype=torch.float32, device="cuda")
    for qd, kd in chunks:
        kvz.kvz_score_chunk_noalloc(qd, kc_d, kd, S_eager, wl.n_prompt, scale)
    torch.cuda.synchronize()
    want = S_eager.cpu().numpy()

    S = torch.zeros_like(S_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for qd, kd in chunks:
                kvz.kvz_score_chunk_noalloc(qd, kc_d, kd, S, wl.n_prompt, scale, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        S.zero_()                                   # eager work between replays
        noise = torch.randn(1 << 20, device="cuda")  # unrelated eager kernels
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(S.cpu().numpy(), want), f"replay {rep}"
        del noise
