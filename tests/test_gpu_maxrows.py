"""The largest query-row count one scoring call takes (G * n_in = 2^20 rows),
checked exactly against the oracle from a few rows.

Construction: every query row is zero except a few planted rows.  A zero row
has logit 0 on every key it sees, so its softmax is uniform: on a context
key, 1 / (n_c + i + 1) for the row at chunk position i, largest at i = 0.  A
planted row (g, i) is a multiple of one key and puts a large share of its
softmax on that key.  So the score of context key j is the larger of
1 / (n_c + 1) and the planted rows' probabilities on j.  The oracle gives a
planted row's softmax from a one-row problem: the row's visible chunk keys
(positions 0 .. i-1) join the context and its own key stays the one chunk
key, which leaves the set of keys it sees unchanged.  Output rows of the
fused call are checked the same way, zero rows included (the mean of the
values the row sees).

Tolerances: scores 1e-6 + 1e-4 |ref| (fp32 softmax sums over up to 65,632
keys); bf16 outputs |dO| <= 2^-8 sum_j p_j |v_j| + 1e-6 (p rounded to bf16,
relative 2^-9, with a factor 2 of slack); fp32 outputs 1e-5 + 1e-4 |O|.
"""
import math

import numpy as np
import pytest

from attention_score_reduction_amd import kvz
from attention_score_reduction_amd.inputs import bf16_bits
from oracle import ras
from tests.helpers import assert_scores_close, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

H, G, N_IN, D, N_C, N_PROMPT = 1, 16, 65536, 64, 96, 16
ALPHA = 1.5
# (g, i, target): the planted row q[g][i] = ALPHA * target key; targets are
# context keys ("c", j) or chunk keys ("in", m) with m <= i
PLANTED = [(15, N_IN - 1, ("c", 0)), (0, N_IN - 1, ("c", 1)), (7, 32767, ("c", 2)),
           (8, 32768, ("c", 3)), (3, 1, ("c", 4)), (12, 40000, ("c", 5)), (1, 255, ("c", 0)),
           (9, 256, ("in", 100)), (2, 65000, ("in", 64999))]
ZERO_ROWS = [(0, 0), (5, N_IN - 1), (14, 12345)]


def _inputs(dtype):
    """Storage arrays (bf16 bit patterns or fp32) of the planted problem."""
    rng = np.random.default_rng(20261204)
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    kc, kin, vc, vin = f32(H, N_C, D), f32(H, N_IN, D), f32(H, N_C, D), f32(H, N_IN, D)
    store = bf16_bits if dtype == "bf16" else (lambda x: x.astype(np.float32))
    kc, kin, vc, vin = (store(x) for x in (kc, kin, vc, vin))
    as32 = lambda x: ras.to_f64(x, dtype).astype(np.float32)
    q = np.zeros((H, G, N_IN, D), np.float32)
    for g, i, (kind, t) in PLANTED:
        q[0, g, i] = ALPHA * (as32(kc)[0, t] if kind == "c" else as32(kin)[0, t])
    return store(q), kc, kin, vc, vin


def _row_problem(q, kc, kin, vc, vin, dtype, g, i):
    """fp64 one-row problem equivalent to query row (g, i)."""
    f = lambda x: ras.to_f64(x, dtype)
    q1 = f(q[:, g:g + 1, i:i + 1])
    kc1 = np.concatenate([f(kc), f(kin[:, :i])], axis=1)
    vc1 = np.concatenate([f(vc), f(vin[:, :i])], axis=1)
    return q1, kc1, f(kin[:, i:i + 1]), vc1, f(vin[:, i:i + 1])


def _oracle_scores(arrs, dtype, scale):
    S = np.full((H, N_C), 1.0 / (N_C + 1))  # zero rows at i = 0
    for g, i, _ in PLANTED:
        q1, kc1, kin1, _, _ = _row_problem(*arrs, dtype, g, i)
        S1 = np.zeros((H, kc1.shape[1]))
        ras.score_chunk(q1, kc1, kin1, scale, S1)
        S = np.maximum(S, S1[:, :N_C])
    return S


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scores_at_the_row_limit(dtype):
    arrs = _inputs(dtype)
    scale = 1.0 / math.sqrt(D)
    ref = _oracle_scores(arrs, dtype, scale)
    assert ref.max() > 0.2  # the planted rows dominate their target keys
    q, kc, kin = (to_dev(x, dtype) for x in arrs[:3])
    assert q.shape[1] * q.shape[2] == 1 << 20
    S = torch.zeros(H, N_C, dtype=torch.float32, device="cuda")
    kvz.kvz_score_chunk(q, kc, kin, S, N_PROMPT, scale)
    torch.cuda.synchronize()
    assert_scores_close(S.cpu().numpy(), ref, atol=1e-6, rtol=1e-4, what=f"S {dtype} 2^20 rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sum_aggregation_at_the_row_limit(dtype):
    """Sum over all 2^20 rows: the zero rows give every context key
    sum over g, i of 1 / (n_c + i + 1) (a harmonic sum, about 104 here), each
    planted row replaces its zero-row term by its probability on the key."""
    arrs = _inputs(dtype)
    scale = 1.0 / math.sqrt(D)
    harmonic = G * sum(1.0 / (N_C + i + 1) for i in range(N_IN))
    ref = np.full((H, N_C), harmonic)
    for g, i, _ in PLANTED:
        q1, kc1, kin1, _, _ = _row_problem(*arrs, dtype, g, i)
        S1 = np.zeros((H, kc1.shape[1]))
        ras.score_chunk(q1, kc1, kin1, scale, S1, mode="sum")
        ref += S1[:, :N_C] - 1.0 / (N_C + i + 1)
    q, kc, kin = (to_dev(x, dtype) for x in arrs[:3])
    S = torch.zeros(H, N_C, dtype=torch.float32, device="cuda")
    kvz.kvz_score_chunk_ex(q, kc, kin, S, N_PROMPT, "sum", scale)
    torch.cuda.synchronize()
    assert_scores_close(S.cpu().numpy(), ref, atol=1e-6, rtol=1e-5,
                        what=f"sum S {dtype} 2^20 rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attention_output_at_the_row_limit(dtype):
    arrs = _inputs(dtype)
    scale = 1.0 / math.sqrt(D)
    q, kc, kin, vc, vin = (to_dev(x, dtype) for x in arrs)
    S = torch.zeros(H, N_C, dtype=torch.float32, device="cuda")
    O = kvz.kvz_score_chunk_attn(q, kc, kin, vc, vin, S, N_PROMPT, scale=scale)
    torch.cuda.synchronize()
    assert_scores_close(S.cpu().numpy(), _oracle_scores(arrs, dtype, scale), atol=1e-6,
                        rtol=1e-4, what=f"fused S {dtype} 2^20 rows")
    O = O.cpu().numpy()
    for g, i in [(g, i) for g, i, _ in PLANTED] + ZERO_ROWS:
        q1, kc1, kin1, vc1, vin1 = _row_problem(*arrs, dtype, g, i)
        ref = ras.chunk_attention_output(q1, kc1, kin1, vc1, vin1, scale)[0, 0, 0]
        got = O[0, g, i].astype(np.float64)
        if dtype == "bf16":
            mag = ras.chunk_attention_output(q1, kc1, kin1, np.abs(vc1), np.abs(vin1), scale)
            tol = 2.0 ** -8 * mag[0, 0, 0] + 1e-6
        else:
            tol = 1e-5 + 1e-4 * np.abs(ref)
        err = np.abs(got - ref)
        print(f"O {dtype} row (g={g}, i={i}): max err {err.max():.3e}, "
              f"max err / tol {(err / tol).max():.3f}", flush=True)
        assert np.all(err <= tol), (g, i)
