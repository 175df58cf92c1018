"""The optional kernel timer with scoring calls launched from two host threads.

ctypes releases the GIL around each library call, so the two threads' calls
overlap on the host; each thread has its own stream, workspace and S.  Every
launch must be timed exactly once, and the scores must be those of a
single-thread run with the timer off (the same kernels on the same inputs).
"""
import math
import threading

import pytest

from attention_score_reduction_amd import kvz
from attention_score_reduction_amd.inputs import HostGen, Workload
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_timer_counts_launches_from_two_threads():
    wl = Workload("timer_threads", 5, 1, 2, 4, 128, 2048, 256, 16, 0.3)
    gen = HostGen(wl)
    kc, _ = gen.context(0)
    kc_d = to_dev(kc, wl.dtype)
    dev = []
    for k in range(len(wl.chunks())):
        q, kin = gen.chunk_inputs(0, k)
        dev.append((to_dev(q, wl.dtype), to_dev(kin, wl.dtype)))
    H, n_c, d = kc.shape
    scale = 1.0 / math.sqrt(d)
    n_rep = 6
    q0 = dev[0][0]
    need = kvz.kvz_score_chunk_workspace(kvz._dtype_code(q0), H, q0.shape[1], q0.shape[2], d, n_c)

    def run(S, stream, ws):
        for _ in range(n_rep):
            for q, kin in dev:
                kvz.kvz_score_chunk(q, kc_d, kin, S, wl.n_prompt, scale, ws=ws, stream=stream)

    s_ref = torch.zeros(H, n_c, dtype=torch.float32, device="cuda")
    run(s_ref, torch.cuda.current_stream(), torch.empty(need, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.zeros(H, n_c, dtype=torch.float32, device="cuda") for _ in streams]
    wss = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in streams]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            run(outs[i], streams[i], wss[i])
        except Exception as e:  # re-raised in the main thread below
            errors.append(e)

    kvz.kvz_prof_enable(True, 4096)
    try:
        threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(streams))]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        counts = {nm: kvz.kvz_prof_read(nm) for nm in ("score_pass1", "score_combine", "score_pass2")}
    finally:
        kvz.kvz_prof_enable(False)
    assert not errors, errors
    per_kernel = len(streams) * n_rep * len(dev)
    for nm, (n, ms) in counts.items():
        assert n == per_kernel, (nm, n, per_kernel)
        assert ms > 0.0, nm
    for S in outs:
        assert torch.equal(S, s_ref)
