"""Host-side logic without a GPU: the seeded input generator and the
benchmark's cost model."""
import importlib.util
import os

import numpy as np

from attention_score_reduction_amd.inputs import WORKLOADS, HostGen, Workload, bf16_bits, bf16_to_f32

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, -2.5, 3.0e38, 1e-40], np.float32)
    back = bf16_to_f32(bf16_bits(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to the even mantissa (1.0)
    np.testing.assert_array_equal(back[:4], np.array([1.0, 1.0, 1.0 + 2**-7, -2.5], np.float32))
    # half a unit in the last place: 2^-8 relative for normal numbers, 2^-134
    # absolute below the smallest normal
    assert np.all(np.abs(back.astype(np.float64) - x) <= np.maximum(np.abs(x) * 2.0**-8, 2.0**-134))


def test_generator_is_deterministic_and_head_subsets_are_slices():
    wl = Workload("g", 5, 2, 3, 2, 64, 300, 100, 8, 0.3, key_lognormal_sigma=0.5, sink=True,
                  peaked_frac=0.05)
    a, b = HostGen(wl), HostGen(wl)
    kc, vc = a.context(1)
    kc2, vc2 = b.context(1)
    assert np.array_equal(kc, kc2) and np.array_equal(vc, vc2)
    ks, vs = a.context(1, [2])
    assert np.array_equal(ks[0], kc[2]) and np.array_equal(vs[0], vc[2])
    q, kin = a.chunk_inputs(1, 2)
    qs, kins = a.chunk_inputs(1, 2, [0, 2])
    assert np.array_equal(qs, q[[0, 2]]) and np.array_equal(kins, kin[[0, 2]])
    vin = a.chunk_values(1, 2)
    assert vin.shape == kin.shape and np.array_equal(a.chunk_values(1, 2, [1]), vin[[1]])
    assert not np.array_equal(vin, kin)
    # the last chunk is ragged: 300 = 100 + 100 + 100, n_in = 8 + 100
    assert wl.chunks() == [(0, 100), (100, 100), (200, 100)] and q.shape[2] == 108


def test_workload_shapes_and_keep_counts():
    assert [len(WORKLOADS[n].chunks()) for n in
            ("tiny_fp32", "llama8b_8k", "llama8b_128k", "qwen14b_120k", "gemma12b_170k")] == \
        [4, 4, 64, 59, 167]
    assert WORKLOADS["qwen14b_120k"].chunks()[-1] == (118784, 1216)
    assert WORKLOADS["gemma12b_170k"].chunks()[-1] == (169984, 16)
    assert WORKLOADS["llama8b_128k"].n_total == 33554432


def test_cost_model_matches_the_two_times_prefill_statement():
    """The scoring forward's attention work: every chunk's n_in rows attend to
    all n_c context keys plus their causal chunk keys.  Against the causal
    prefill over the context (n_c (n_c + 1) / 2 logits per query head), the
    128K workload does about 2x the logits, as the authors state for their
    scoring stage (twice the prefill's attention FLOPs)."""
    bench = _bench()
    wl = WORKLOADS["llama8b_128k"]
    H, G, d, n_c = wl.heads, wl.group, wl.head_dim, wl.n_ctx
    p1 = sum(bench.score_flops(wl, wl.n_prompt + m)[0] for _, m in wl.chunks())
    prefill = 2 * d * H * G * n_c * (n_c + 1) // 2
    ratio = p1 / prefill
    assert 2.0 <= ratio <= 2.05, ratio
    # pass 2 covers exactly the context part of pass 1's logits
    a, b = bench.score_flops(wl, 2064)
    assert b == 2 * d * H * G * 2064 * n_c and a - b == 2 * d * H * G * 2064 * 2065 // 2


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU: any other --gpus exits with status 2 and a
    message, before it imports torch or touches a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
