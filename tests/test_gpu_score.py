"""Parity of the HIP score kernels with the fp64 oracle, plus exact invariants.

Tolerance for bf16 inputs with fp32 accumulation: |gpu - ref| <= 2e-3 +
1e-2 |ref| elementwise.  The fp32 path is held to 1e-6 + 1e-4 |ref|.
"""
import math

import numpy as np
import pytest

from attention_score_reduction_amd import kvz
from attention_score_reduction_amd.inputs import WORKLOADS, HostGen, Workload
from oracle import ras
from tests.helpers import assert_scores_close, oracle_layer_scores, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def gpu_layer_scores(gen, layer, chunk_ids=None, heads=None, order=None):
    wl = gen.wl
    kc, _ = gen.context(layer, heads)
    kc_d = to_dev(kc, wl.dtype)
    S = torch.zeros(kc.shape[0], wl.n_ctx, dtype=torch.float32, device="cuda")
    ids = list(range(len(wl.chunks()))) if chunk_ids is None else list(chunk_ids)
    if order is not None:
        ids = [ids[i] for i in order]
    for k in ids:
        q, kin = gen.chunk_inputs(layer, k, heads)
        kvz.kvz_score_chunk(to_dev(q, wl.dtype), kc_d, to_dev(kin, wl.dtype), S, wl.n_prompt,
                            1.0 / math.sqrt(wl.head_dim))
    torch.cuda.synchronize()
    return S.cpu().numpy()


def test_tiny_fp32_workload_full():
    """512-token fp32 workload: one chunk of 8 prompt + 128 copy tokens."""
    gen = HostGen(WORKLOADS["tiny_fp32"])
    ref = oracle_layer_scores(gen, 0, [0])
    got = gpu_layer_scores(gen, 0)
    assert_scores_close(got, ref, atol=1e-6, rtol=1e-4, what="tiny fp32")


SMALL = [
    # (name, H, G, d, n_c, chunk, n_prompt, sigma, sink)
    ("d128_g4_ragged", 2, 4, 128, 1000, 300, 16, 0.5, True),
    ("d64_g5", 2, 5, 64, 777, 250, 16, 0.0, False),
    ("d256_g2", 1, 2, 256, 1500, 640, 16, 1.0, False),
    ("d128_g1_one_row_tail", 1, 1, 128, 513, 512, 7, 0.3, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_bf16_shapes(case):
    name, H, G, d, n_c, chunk, n_p, sig, sink = case
    wl = Workload(name, 11, 1, H, G, d, n_c, chunk, n_p, 0.3, key_lognormal_sigma=sig, sink=sink)
    gen = HostGen(wl)
    ref = oracle_layer_scores(gen, 0, list(range(H)))
    got = gpu_layer_scores(gen, 0)
    assert_scores_close(got, ref, what=name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_queries_closed_form(dtype):
    """Q = 0 gives S = 1/(n_c + 1) exactly in real arithmetic (row 0 sees the
    n_c context keys and in-chunk key 0)."""
    H, G, d, n_c, n_in = 2, 3, 128, 3000, 200
    rng = np.random.default_rng(5)
    kc = rng.standard_normal((H, n_c, d)).astype(np.float32)
    ki = rng.standard_normal((H, n_in, d)).astype(np.float32)
    q = np.zeros((H, G, n_in, d), np.float32)
    if dtype == "bf16":
        from attention_score_reduction_amd.inputs import bf16_bits
        kc, ki, q = bf16_bits(kc), bf16_bits(ki), bf16_bits(q)
    S = torch.zeros(H, n_c, dtype=torch.float32, device="cuda")
    kvz.kvz_score_chunk(to_dev(q, dtype), to_dev(kc, dtype), to_dev(ki, dtype), S, 8, 1 / math.sqrt(d))
    got = S.cpu().numpy()
    np.testing.assert_allclose(got, 1.0 / (n_c + 1), rtol=1e-5)


def test_chunk_order_and_repeat_are_bitwise_invariant():
    wl = Workload("inv", 12, 1, 2, 4, 128, 1200, 400, 16, 0.3, key_lognormal_sigma=0.5, sink=True)
    gen = HostGen(wl)
    a = gpu_layer_scores(gen, 0)
    b = gpu_layer_scores(gen, 0, order=[2, 0, 1])
    c = gpu_layer_scores(gen, 0, chunk_ids=[0, 1, 2, 1, 0])
    d = gpu_layer_scores(gen, 0)
    assert np.array_equal(a, b) and np.array_equal(a, c) and np.array_equal(a, d)


def test_group_split_equals_max_of_single_query_heads():
    H, G, d, n_c, n_in = 2, 4, 128, 900, 260
    rng = np.random.default_rng(6)
    from attention_score_reduction_amd.inputs import bf16_bits
    kc = bf16_bits(rng.standard_normal((H, n_c, d)).astype(np.float32))
    ki = bf16_bits(rng.standard_normal((H, n_in, d)).astype(np.float32))
    q = bf16_bits(rng.standard_normal((H, G, n_in, d)).astype(np.float32))
    kc_d, ki_d = to_dev(kc, "bf16"), to_dev(ki, "bf16")
    S = torch.zeros(H, n_c, dtype=torch.float32, device="cuda")
    kvz.kvz_score_chunk(to_dev(q, "bf16"), kc_d, ki_d, S, 16)
    parts = []
    for g in range(G):
        Sg = torch.zeros(H, n_c, dtype=torch.float32, device="cuda")
        kvz.kvz_score_chunk(to_dev(np.ascontiguousarray(q[:, g:g + 1]), "bf16"), kc_d, ki_d, Sg, 16)
        parts.append(Sg.cpu().numpy())
    # the row log-sum-exp of a row does not depend on G, and the column max of
    # a union of rows is the max of the column maxima; the two launches split
    # the key axis differently, so the lse may differ in its last bits
    np.testing.assert_allclose(S.cpu().numpy(), np.maximum.reduce(parts), rtol=2e-6, atol=0)


def test_running_max_respects_existing_scores():
    """S enters as a running max: a preset larger value survives, a preset
    smaller one is overwritten."""
    wl = Workload("rm", 13, 1, 1, 2, 128, 600, 200, 8, 0.3)
    gen = HostGen(wl)
    base = gpu_layer_scores(gen, 0, chunk_ids=[0])
    kc, _ = gen.context(0)
    q, kin = gen.chunk_inputs(0, 0)
    S0 = np.zeros_like(base)
    S0[0, ::2] = 0.75
    S = torch.from_numpy(S0.astype(np.float32)).cuda()
    kvz.kvz_score_chunk(to_dev(q, "bf16"), to_dev(kc, "bf16"), to_dev(kin, "bf16"), S, 8)
    np.testing.assert_array_equal(S.cpu().numpy(), np.maximum(base, S0.astype(np.float32)))


def test_llama8b_8k_layer_sampled_heads():
    """8192-token LLaMA3.1-8B-shaped layer (8 KV heads, G = 4, 4 chunks of
    16 + 2048 rows), the full layer on the GPU, two heads in the oracle."""
    wl = WORKLOADS["llama8b_8k"]
    gen = HostGen(wl)
    got = gpu_layer_scores(gen, 3)
    heads = [0, 5]
    ref = oracle_layer_scores(gen, 3, heads)
    assert_scores_close(got[heads], ref, what="llama8b_8k layer 3")


F32_CASES = [
    # (name, H, G, d, n_c, chunk, n_prompt, sigma, sink): random fp32 inputs,
    # several key tiles, ragged context tail, several chunks (the last ragged)
    ("f32_d128_g2", 2, 2, 128, 700, 300, 16, 0.5, True),
    ("f32_d256_g2", 2, 2, 256, 701, 250, 16, 1.0, False),
    ("f32_d64_g3", 1, 3, 64, 650, 400, 8, 0.0, True),
]


@pytest.mark.parametrize("case", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_small_f32_shapes(case):
    """The fp32 (VALU) score path against the oracle on random inputs, at
    every head size: 1e-6 + 1e-4 |ref|."""
    name, H, G, d, n_c, chunk, n_p, sig, sink = case
    wl = Workload(name, 14, 1, H, G, d, n_c, chunk, n_p, 0.3, dtype="f32",
                  key_lognormal_sigma=sig, sink=sink)
    gen = HostGen(wl)
    ref = oracle_layer_scores(gen, 0, list(range(H)))
    got = gpu_layer_scores(gen, 0)
    assert_scores_close(got, ref, atol=1e-6, rtol=1e-4, what=name)


DEGENERATE = [
    # (name, H, G, d, n_c, chunk, n_prompt, dtype): shapes at the edges of
    # the tiling: one context key and one query row, contexts shorter than
    # one 32-key tile, no prompt rows, wide query groups (rows i-major, so a
    # 32-row tile spans few tokens)
    ("one_key_one_row", 1, 1, 128, 1, 1, 0, "bf16"),
    ("ctx5_no_prompt", 2, 2, 64, 5, 3, 0, "bf16"),
    ("ctx31_g8", 1, 8, 128, 31, 33, 4, "bf16"),
    ("g16_d256", 1, 16, 256, 200, 70, 5, "bf16"),
    ("f32_one_key_one_row", 1, 1, 64, 1, 1, 0, "f32"),
    ("f32_g16", 2, 16, 64, 90, 40, 3, "f32"),
]


@pytest.mark.parametrize("case", DEGENERATE, ids=[c[0] for c in DEGENERATE])
def test_degenerate_shapes(case):
    name, H, G, d, n_c, chunk, n_p, dtype = case
    wl = Workload(name, 16, 1, H, G, d, n_c, chunk, n_p, 0.3, dtype=dtype)
    gen = HostGen(wl)
    ref = oracle_layer_scores(gen, 0, list(range(H)))
    got = gpu_layer_scores(gen, 0)
    if dtype == "f32":
        assert_scores_close(got, ref, atol=1e-6, rtol=1e-4, what=name)
    else:
        assert_scores_close(got, ref, what=name)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_most_heads_in_one_call(dtype):
    """4096 KV heads in one call (the most it takes), checked on sampled
    heads spread over the grid (first, last, and around the XCD boundaries
    of the head-major workgroup order)."""
    wl = Workload("heads4096", 17, 1, 4096, 2, 64, 100, 40, 8, 0.3, dtype=dtype)
    gen = HostGen(wl)
    got = gpu_layer_scores(gen, 0)
    heads = [0, 1, 511, 512, 2047, 2048, 3583, 4095]
    ref = oracle_layer_scores(gen, 0, heads)
    tol = dict(atol=1e-6, rtol=1e-4) if dtype == "f32" else {}
    assert_scores_close(got[heads], ref, what=f"4096 heads {dtype}", **tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_resume_from_saved_scores_is_bitwise_identical(dtype):
    """Scoring can stop after any chunk and resume from a host copy of S: the
    result equals the uninterrupted run bit for bit (S is the whole state)."""
    wl = Workload("resume", 15, 1, 2, 4, 128, 1500, 400, 16, 0.3, dtype=dtype,
                  key_lognormal_sigma=0.5, sink=True)
    gen = HostGen(wl)
    whole = gpu_layer_scores(gen, 0)
    kc, _ = gen.context(0)
    kc_d = to_dev(kc, dtype)
    S = torch.zeros(wl.heads, wl.n_ctx, dtype=torch.float32, device="cuda")
    n = len(wl.chunks())
    for k in range(n):
        q, kin = gen.chunk_inputs(0, k)
        kvz.kvz_score_chunk(to_dev(q, dtype), kc_d, to_dev(kin, dtype), S, wl.n_prompt,
                            1.0 / math.sqrt(wl.head_dim))
        if k == 1:
            saved = S.cpu().numpy().copy()       # checkpoint after chunk 1
            del S
            torch.cuda.synchronize()
            S = torch.from_numpy(saved).cuda()   # resume in a new buffer
    torch.cuda.synchronize()
    assert np.array_equal(S.cpu().numpy(), whole)
