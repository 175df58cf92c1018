"""Pins of the CPU oracle against facts other than the oracle itself.

Each test ties one part of oracle/ras.py to a closed form, a hand-derived
worked example, a library routine in a special case, a brute force on tiny
inputs, or an invariant the definition forces.  A plausible slip in the oracle
(a dropped causal mask, a transposed operand, mean instead of max, a wrong
scale, a wrong tie rule, an off-by-one in the key set) fails at least one.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ras

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# exact conversion of the storage types
# ---------------------------------------------------------------------------

def test_bf16_conversion_exact_values():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x0000, 0x8000], np.uint16)
    got = ras.bf16_to_f64(bits)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133,
            (2.0 - 2.0 ** -7) * 2.0 ** 127, 0.0, -0.0]
    assert got.tolist() == want


def test_f32_conversion_exact():
    x = np.array([1.0 / 3.0, 1e-40, -7.25], np.float32)
    assert ras.to_f64(x, "f32").tolist() == [float(v) for v in x]


# ---------------------------------------------------------------------------
# scoring
# ---------------------------------------------------------------------------

def test_hand_derived_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "rational_chunk.json")))
    q = np.array(g["q_rows"], np.float64)[None, None]          # [1][1][2][2]
    kc = np.log(np.array(g["k_ctx_log"], np.float64))[None]   # [1][3][2]
    ki = np.log(np.array(g["k_in_log"], np.float64))[None]    # [1][2][2]
    P = ras.chunk_probabilities(q[0, 0], kc[0], ki[0], g["scale"])
    want_p = np.array(g["row_probs_num"], np.float64) / np.array(g["row_probs_den"], np.float64)[:, None]
    np.testing.assert_allclose(P, want_p, rtol=1e-14, atol=1e-15)
    S = ras.score_layer([(q, ki)], kc, g["scale"])
    want = np.array(g["S_num"], np.float64) / np.array(g["S_den"], np.float64)
    np.testing.assert_allclose(S[0], want, rtol=1e-14)


@pytest.mark.parametrize("n_c,n_in,G,H", [(37, 9, 2, 2), (5, 1, 1, 1), (64, 20, 3, 1)])
def test_zero_queries_closed_form(n_c, n_in, G, H):
    """Q = 0: every visible key gets 1/(#visible).  Row i sees n_c + i + 1 keys,
    so every context key's max is 1/(n_c + 1), taken at row 0.  This fixes the
    key set (the whole context, not only the chunk) and the causal mask over
    the in-chunk keys (all in-chunk keys visible would give 1/(n_c + n_in))."""
    d = 8
    q = np.zeros((H, G, n_in, d))
    kc = _rand((H, n_c, d), 1)
    ki = _rand((H, n_in, d), 2)
    S = ras.score_layer([(q, ki)], kc, 1 / math.sqrt(d))
    np.testing.assert_allclose(S, 1.0 / (n_c + 1), rtol=1e-14)


def test_single_query_row_is_library_softmax():
    """n_in = 1: S[h] = max_g softmax(scale * q_g . [K_c; k_in_0])[:n_c]."""
    torch = pytest.importorskip("torch")
    H, G, n_c, d = 2, 3, 50, 16
    q = _rand((H, G, 1, d), 3)
    kc = _rand((H, n_c, d), 4)
    ki = _rand((H, 1, d), 5)
    scale = 1 / math.sqrt(d)
    S = ras.score_layer([(q, ki)], kc, scale)
    for h in range(H):
        keys = torch.from_numpy(np.concatenate([kc[h], ki[h]]))
        lg = torch.from_numpy(q[h, :, 0]) @ keys.T * scale
        p = torch.softmax(lg, dim=-1)[:, :n_c].max(dim=0).values.numpy()
        np.testing.assert_allclose(S[h], p, rtol=1e-13, atol=1e-16)


def test_rows_are_scipy_softmax_over_visible_prefix():
    """Each row is the library softmax of the logits of its visible keys: all
    context keys and in-chunk keys 0..i."""
    from scipy.special import softmax

    n_c, n_in, d = 23, 7, 8
    q = _rand((n_in, d), 6)
    kc = _rand((n_c, d), 7, 2.0)
    ki = _rand((n_in, d), 8)
    scale = 0.37
    P = ras.chunk_probabilities(q, kc, ki, scale)
    for i in range(n_in):
        vis = np.concatenate([kc, ki[: i + 1]])
        want = softmax(vis @ q[i] * scale)
        np.testing.assert_allclose(P[i, : n_c + i + 1], want, rtol=1e-13, atol=1e-17)
        assert np.all(P[i, n_c + i + 1:] == 0.0)


@pytest.mark.parametrize("row_block", [256, 2, 1])
def test_brute_force_pure_python(row_block):
    """Tiny case by pure-Python loops with math.exp and math.fsum; the
    oracle's rows taken in blocks of row_block (2: a second, ragged block)."""
    H, G, n_c, n_in, d = 2, 2, 5, 3, 4
    q = _rand((H, G, n_in, d), 9)
    kc = _rand((H, n_c, d), 10)
    ki = _rand((H, n_in, d), 11)
    scale = 0.5
    S = ras.score_chunk(q, kc, ki, scale, np.zeros((H, n_c)), row_block=row_block)
    for h in range(H):
        best = [0.0] * n_c
        for g in range(G):
            for i in range(n_in):
                keys = [kc[h, j] for j in range(n_c)] + [ki[h, t] for t in range(i + 1)]
                lg = [scale * math.fsum(float(a) * float(b) for a, b in zip(q[h, g, i], k))
                      for k in keys]
                m = max(lg)
                z = math.fsum(math.exp(x - m) for x in lg)
                for j in range(n_c):
                    best[j] = max(best[j], math.exp(lg[j] - m) / z)
        np.testing.assert_allclose(S[h], best, rtol=1e-12)


def test_probability_invariants():
    n_c, n_in, d = 40, 12, 16
    q = _rand((n_in, d), 12, 3.0)
    kc = _rand((n_c, d), 13)
    ki = _rand((n_in, d), 14)
    P = ras.chunk_probabilities(q, kc, ki, 1 / 4)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(P >= 0) and np.all(P <= 1)
    S = ras.score_layer([(q[None, None], ki[None])], kc[None], 1 / 4)
    assert np.all(S >= 0) and np.all(S <= 1)
    # S is the column max over rows of the context block, nothing else
    np.testing.assert_array_equal(S[0], P[:, :n_c].max(axis=0))


def test_max_not_mean():
    """A case where the max and the mean over query rows rank two context keys
    the other way round; the score must follow the max (blog section 4.3.2;
    paperhub rebuttal, answer on average aggregation)."""
    # key A = e0, key B = e1, in-chunk keys = e2; logits are the q entries.
    kc = np.array([[1.0, 0, 0], [0, 1.0, 0]])
    n_in = 4
    ki = np.tile([0, 0, 1.0], (n_in, 1))
    q = np.array([[5.0, 0, 0]] + [[-5.0, 0.5, 0]] * (n_in - 1))
    P = ras.chunk_probabilities(q, kc, ki, 1.0)
    mean = P[:, :2].mean(axis=0)
    assert mean[1] > mean[0]                         # the mean prefers B
    S = ras.score_layer([(q[None, None], ki[None])], kc[None], 1.0)[0]
    assert S[0] > S[1]                               # the max prefers A
    assert S[0] == pytest.approx(math.exp(5) / (math.exp(5) + 2), rel=1e-14)


def test_chunk_merge_is_order_free_and_idempotent():
    H, G, n_c, d = 2, 2, 30, 8
    kc = _rand((H, n_c, d), 20)
    chunks = [(_rand((H, G, n, d), 21 + n), _rand((H, n, d), 40 + n)) for n in (5, 9, 3)]
    scale = 1 / math.sqrt(d)
    S = ras.score_layer(chunks, kc, scale)
    for perm in itertools.permutations(range(3)):
        S2 = ras.score_layer([chunks[p] for p in perm], kc, scale)
        np.testing.assert_array_equal(S, S2)
    S3 = ras.score_layer(chunks + [chunks[1]], kc, scale)
    np.testing.assert_array_equal(S, S3)


def test_group_split_is_max_of_single_heads():
    H, G, n_c, n_in, d = 1, 3, 25, 6, 8
    q = _rand((H, G, n_in, d), 30)
    kc = _rand((H, n_c, d), 31)
    ki = _rand((H, n_in, d), 32)
    S = ras.score_layer([(q, ki)], kc, 0.3)
    parts = [ras.score_layer([(q[:, g:g + 1], ki)], kc, 0.3) for g in range(G)]
    np.testing.assert_array_equal(S, np.maximum.reduce(parts))


def test_scale_enters_as_temperature():
    """Doubling the scale equals doubling the queries (exactly for powers of 2)."""
    H, G, n_c, n_in, d = 1, 2, 20, 5, 8
    q = _rand((H, G, n_in, d), 33)
    kc = _rand((H, n_c, d), 34)
    ki = _rand((H, n_in, d), 35)
    a = ras.score_layer([(q, ki)], kc, 0.5)
    b = ras.score_layer([(q * 2.0, ki)], kc, 0.25)
    np.testing.assert_array_equal(a, b)
    c = ras.score_layer([(q, ki)], kc, 0.25)
    assert not np.allclose(a, c)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,r,K", [(512, 0.3, 154), (2097152, 0.3, 629146),
                                   (33554432, 0.3, 10066330), (46080000, 0.25, 11520000),
                                   (65280000, 0.4, 26112000), (10, 0.0, 0), (10, 1.0, 10),
                                   (7, 0.5, 4)])
def test_keep_count_values(N, r, K):
    """K = r * N rounded half up: 0.3 * 512 = 153.6 -> 154, 0.5 * 7 = 3.5 -> 4."""
    assert ras.keep_count(N, r) == K


def _brute_select(S, n_heads, n_c, K):
    items = sorted(range(len(S)), key=lambda i: (-float(S[i]), i))
    keep = set(items[:K])
    mask = [1 if i in keep else 0 for i in range(len(S))]
    budgets = [sum(mask[h * n_c:(h + 1) * n_c]) for h in range(n_heads)]
    offs = [0]
    for b in budgets:
        offs.append(offs[-1] + b)
    return mask, offs


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n_heads, n_c = 4, 9
    S = rng.integers(0, 5, n_heads * n_c).astype(np.float32) / 8  # many ties
    for K in (0, 1, 7, 18, 35, 36):
        mask, offs, tau = ras.select(S, n_heads, n_c, K)
        bm, bo = _brute_select(S, n_heads, n_c, K)
        assert mask.tolist() == bm
        assert offs.tolist() == bo
        assert int(mask.sum()) == K
        if 0 < K:
            assert S[mask == 1].min() >= tau
            assert tau == sorted(S.tolist(), reverse=True)[K - 1]
            if K < len(S):
                assert S[mask == 0].max() <= tau
        else:
            assert tau == math.inf


@pytest.mark.parametrize("n_heads,n_c,ratio", [(7, 1000, 0.3), (3, 4099, 0.5), (1, 2018, 0.001),
                                                (5, 1009, 1.0)])
def test_select_periodic_scores_closed_form(n_heads, n_c, ratio):
    """Scores (f mod P) / P of the flat index: each value's count is known,
    so the kept set, tau and the head offsets have a closed form."""
    from tests.helpers import (PERIOD, periodic_kept_before, periodic_mask, periodic_scores,
                               periodic_select_params)
    N = n_heads * n_c
    K = ras.keep_count(N, ratio)
    mask, offs, tau = ras.select(periodic_scores(np.arange(N)), n_heads, n_c, K)
    r_star, need = periodic_select_params(N, K)
    assert np.array_equal(mask, periodic_mask(0, N, r_star, need))
    assert np.array_equal(offs, periodic_kept_before(np.arange(n_heads + 1) * n_c, r_star, need))
    assert tau == float(np.float32(r_star) / np.float32(PERIOD))


def test_select_nonuniform_budgets():
    """One global threshold gives per-head budgets that follow each head's
    scores (atlas summary, Measured effects: non-uniform head budgets)."""
    n_heads, n_c = 3, 10
    S = np.concatenate([np.full(n_c, 0.9), np.full(n_c, 0.1), np.linspace(0, 1, n_c)])
    mask, offs, tau = ras.select(S.astype(np.float32), n_heads, n_c, 15)
    assert np.diff(offs).tolist() == [10, 0, 5]


# ---------------------------------------------------------------------------
# compaction
# ---------------------------------------------------------------------------

def test_compact_rows_and_index():
    rng = np.random.default_rng(50)
    n_heads, n_c, d = 3, 11, 4
    kc = rng.integers(0, 2 ** 16, (n_heads, n_c, d)).astype(np.uint16)
    vc = rng.integers(0, 2 ** 16, (n_heads, n_c, d)).astype(np.uint16)
    S = rng.random(n_heads * n_c).astype(np.float32)
    mask, offs, _ = ras.select(S, n_heads, n_c, 13)
    ko, vo, idx = ras.compact(kc, vc, mask, offs)
    assert ko.shape == (13, d) and idx.shape == (13,)
    m = mask.reshape(n_heads, n_c)
    for h in range(n_heads):
        seg = slice(offs[h], offs[h + 1])
        js = idx[seg]
        assert np.all(np.diff(js) > 0)
        assert set(js.tolist()) == set(np.nonzero(m[h])[0].tolist())
        assert np.array_equal(ko[seg], kc[h, js]) and np.array_equal(vo[seg], vc[h, js])


def test_exact_fractions_for_three_token_case():
    """Pin with exact rational arithmetic: logits ln(1), ln(2), ln(3) on three
    context keys and one in-chunk key ln(2), a single query row."""
    kc = np.log(np.array([[1.0], [2.0], [3.0]]))
    ki = np.log(np.array([[2.0]]))
    q = np.array([[[[1.0]]]])
    S = ras.score_layer([(q, ki[None])], kc[None], 1.0)[0]
    want = [Fraction(1, 8), Fraction(2, 8), Fraction(3, 8)]
    np.testing.assert_allclose(S, [float(w) for w in want], rtol=1e-14)


# ---------------------------------------------------------------------------
# aggregation variants (sum / raw logits), head and token aggregates, decode
# ---------------------------------------------------------------------------

def test_sum_mode_zero_queries_closed_form():
    """Q = 0: row i puts 1/(n_c + i + 1) on every context key, so the sum over
    the G heads and n_in rows is G * sum_i 1/(n_c + i + 1) for every key."""
    H, G, n_c, n_in, d = 2, 3, 40, 7, 8
    q = np.zeros((H, G, n_in, d))
    S = ras.score_layer([(q, _rand((H, n_in, d), 60))], _rand((H, n_c, d), 61), 0.3, mode="sum")
    want = G * sum(1.0 / (n_c + i + 1) for i in range(n_in))
    np.testing.assert_allclose(S, want, rtol=1e-14)


@pytest.mark.parametrize("row_block", [256, 3, 1])
def test_sum_mode_brute_force_and_mass(row_block):
    H, G, n_c, n_in, d = 1, 2, 6, 4, 5
    q = _rand((H, G, n_in, d), 62)
    kc = _rand((H, n_c, d), 63)
    ki = _rand((H, n_in, d), 64)
    S = ras.score_chunk(q, kc, ki, 0.4, np.zeros((H, n_c)), row_block=row_block, mode="sum")[0]
    want = [0.0] * n_c
    chunk_mass = 0.0
    for g in range(G):
        for i in range(n_in):
            keys = [kc[0, j] for j in range(n_c)] + [ki[0, t] for t in range(i + 1)]
            lg = [0.4 * math.fsum(float(a) * float(b) for a, b in zip(q[0, g, i], k)) for k in keys]
            z = math.fsum(math.exp(x) for x in lg)
            for j in range(n_c):
                want[j] += math.exp(lg[j]) / z
            chunk_mass += math.fsum(math.exp(x) for x in lg[n_c:]) / z
    np.testing.assert_allclose(S, want, rtol=1e-12)
    # every row sums to one: context mass + chunk mass = G * n_in
    assert math.isclose(S.sum() + chunk_mass, G * n_in, rel_tol=1e-12)


def test_sum_and_mean_give_identical_priorities():
    """The paperhub rebuttal's answer on average aggregation: sum and mean
    rank keys identically (mean = sum / number of query rows)."""
    H, G, n_c, d = 2, 2, 50, 8
    chunks = [(_rand((H, G, n, d), 65 + n), _rand((H, n, d), 75 + n)) for n in (9, 6)]
    kc = _rand((H, n_c, d), 66)
    S_sum = ras.score_layer(chunks, kc, 0.35, mode="sum")
    S_mean = S_sum / (G * (9 + 6))
    K = 37
    a = ras.select(S_sum.reshape(-1), H, n_c, K)[0]
    b = ras.select(S_mean.reshape(-1), H, n_c, K)[0]
    assert np.array_equal(a, b)


def test_raw_mode_is_max_logit():
    H, G, n_c, n_in, d = 2, 2, 30, 5, 8
    q = _rand((H, G, n_in, d), 67)
    kc = _rand((H, n_c, d), 68)
    ki = _rand((H, n_in, d), 69)
    S = ras.score_layer([(q, ki)], kc, 0.25, mode="raw")
    for h in range(H):
        for j in range(n_c):
            want = max(0.25 * math.fsum(float(a) * float(b) for a, b in zip(q[h, g, i], kc[h, j]))
                       for g in range(G) for i in range(n_in))
            assert math.isclose(S[h, j], want, rel_tol=1e-12, abs_tol=1e-15)
    S0 = ras.score_layer([(np.zeros_like(q), ki)], kc, 0.25, mode="raw")
    assert np.all(S0 == 0.0)


def test_raw_and_softmax_rank_differently():
    """A key with a large logit in a row that also has a larger competitor
    scores high raw but low after normalisation (what the ablation removes)."""
    kc = np.array([[1.0, 0, 0], [0, 1.0, 0], [0, 0, 1.0]])   # A, B, C
    ki = np.array([[0, 0, 0.0]])
    q = np.array([[4.0, 6.0, 0.0]])                            # row sees A=4, B=6
    raw = ras.score_layer([(q[None, None], ki[None])], kc[None], 1.0, mode="raw")[0]
    mx = ras.score_layer([(q[None, None], ki[None])], kc[None], 1.0)[0]
    q2 = np.array([[0.0, 0.0, 3.0]])                           # row sees C=3 alone
    raw2 = ras.score_layer([(q2[None, None], ki[None])], kc[None], 1.0, mode="raw")[0]
    mx2 = ras.score_layer([(q2[None, None], ki[None])], kc[None], 1.0)[0]
    r = np.maximum(raw, raw2)
    m = np.maximum(mx, mx2)
    assert r[0] > r[2] and m[0] < m[2]


def test_head_and_token_scores_brute_force():
    rng = np.random.default_rng(70)
    S = rng.random((6, 33))
    hs = ras.head_scores(S)
    ts = ras.token_scores(S)
    assert hs.tolist() == [max(S[h].tolist()) for h in range(6)]
    assert ts.tolist() == [max(S[:, j].tolist()) for j in range(33)]
    assert np.all(S <= hs[:, None]) and np.all(S <= ts[None, :])


def test_decode_attention_library_and_closed_forms():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(71)
    n_heads, G, d, L = 3, 4, 16, 9
    q = rng.standard_normal((n_heads, G, d))
    k = rng.standard_normal((n_heads * L, d))
    v = rng.standard_normal((n_heads * L, d))
    offs = np.arange(n_heads + 1) * L
    out = ras.decode_attention(q, k, v, offs, 0.25)
    for h in range(n_heads):
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h])[None], torch.from_numpy(k[h * L:(h + 1) * L])[None],
            torch.from_numpy(v[h * L:(h + 1) * L])[None], scale=0.25)[0].numpy()
        np.testing.assert_allclose(out[h], want, rtol=1e-12, atol=1e-14)
    # one kept row: softmax of one logit is 1, the output is that V row;
    # no kept row: zeros
    offs2 = np.array([0, 1, 1, 3])
    out2 = ras.decode_attention(q, k[:3], v[:3], offs2, 0.5)
    np.testing.assert_allclose(out2[0], np.broadcast_to(v[0], (G, d)), rtol=0, atol=0)
    assert np.all(out2[1] == 0.0)


# ---------------------------------------------------------------------------
# reconstruction attention output O = P [V_c; V_in]
# ---------------------------------------------------------------------------

def test_attention_output_closed_forms():
    """V = ones gives O = 1 (rows of P sum to 1); Q = 0 gives O_i = the mean
    of the visible value rows (all context rows and chunk rows 0..i)."""
    H, G, n_c, n_in, d = 2, 3, 11, 6, 5
    q = _rand((H, G, n_in, d), 81)
    kc = _rand((H, n_c, d), 82)
    ki = _rand((H, n_in, d), 83)
    O = ras.chunk_attention_output(q, kc, ki, np.ones((H, n_c, 4)), np.ones((H, n_in, 4)), 0.6)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-14)
    vc = _rand((H, n_c, d), 84)
    vi = _rand((H, n_in, d), 85)
    O0 = ras.chunk_attention_output(np.zeros_like(q), kc, ki, vc, vi, 0.6)
    for h in range(H):
        for i in range(n_in):
            vis = np.concatenate([vc[h], vi[h, : i + 1]])
            for g in range(G):
                np.testing.assert_allclose(O0[h, g, i], vis.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_attention_output_single_row_is_library_attention():
    """n_in = 1 (no prompt, one copied token): O is torch's scaled dot-product
    attention of that query over [K_c; k_0] and [V_c; v_0] in fp64."""
    torch = pytest.importorskip("torch")
    H, G, n_c, d = 2, 2, 23, 8
    q = _rand((H, G, 1, d), 86)
    kc = _rand((H, n_c, d), 87)
    ki = _rand((H, 1, d), 88)
    vc = _rand((H, n_c, d), 89)
    vi = _rand((H, 1, d), 90)
    O = ras.chunk_attention_output(q, kc, ki, vc, vi, 0.3)
    for h in range(H):
        keys = torch.from_numpy(np.concatenate([kc[h], ki[h]]))[None]
        vals = torch.from_numpy(np.concatenate([vc[h], vi[h]]))[None]
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h, :, 0])[None], keys, vals, scale=0.3)[0].numpy()
        np.testing.assert_allclose(O[h, :, 0], want, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("row_block", [256, 2, 1])
def test_attention_output_brute_force_pure_python(row_block):
    """Tiny case by pure-Python loops (math.exp, math.fsum), causal key set;
    value rows differ from key rows, so a P.K or transposed contraction fails.
    The oracle takes the rows in blocks of row_block."""
    H, G, n_c, n_in, d, dv = 1, 2, 4, 3, 3, 2
    q = _rand((H, G, n_in, d), 91)
    kc = _rand((H, n_c, d), 92)
    ki = _rand((H, n_in, d), 93)
    vc = _rand((H, n_c, dv), 94)
    vi = _rand((H, n_in, dv), 95)
    scale = 0.8
    O = ras.chunk_attention_output(q, kc, ki, vc, vi, scale, row_block=row_block)
    for g in range(G):
        for i in range(n_in):
            keys = [kc[0, j] for j in range(n_c)] + [ki[0, t] for t in range(i + 1)]
            vals = [vc[0, j] for j in range(n_c)] + [vi[0, t] for t in range(i + 1)]
            lg = [scale * math.fsum(float(a) * float(b) for a, b in zip(q[0, g, i], k))
                  for k in keys]
            m = max(lg)
            w = [math.exp(x - m) for x in lg]
            z = math.fsum(w)
            for c in range(dv):
                want = math.fsum(wk * float(v[c]) for wk, v in zip(w, vals)) / z
                assert abs(O[0, g, i, c] - want) <= 1e-13 * max(1.0, abs(want))


def test_attention_output_one_hot_values_give_probabilities():
    """Value row j = unit vector e_j: O equals the probability matrix, so the
    output and the scores come from the same softmax rows."""
    H, G, n_c, n_in, d = 1, 2, 7, 5, 6
    q = _rand((H, G, n_in, d), 96, 2.0)
    kc = _rand((H, n_c, d), 97)
    ki = _rand((H, n_in, d), 98)
    eye = np.eye(n_c + n_in)
    O = ras.chunk_attention_output(q, kc, ki, eye[None, :n_c], eye[None, n_c:], 0.5)
    for g in range(G):
        P = ras.chunk_probabilities(q[0, g], kc[0], ki[0], 0.5)
        np.testing.assert_allclose(O[0, g], P, rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# head-level and token-level eviction
# ---------------------------------------------------------------------------

def _brute_head_evict(S, K_heads, n_sink, n_recent):
    """Pure-Python reference: rank heads by (max score desc, index asc)."""
    n_heads, n_c = len(S), len(S[0])
    score = [max(row) for row in S]
    order = sorted(range(n_heads), key=lambda h: (-score[h], h))
    kept = set(order[:K_heads])
    mask = []
    for h in range(n_heads):
        for j in range(n_c):
            mask.append(1 if (h in kept or j < n_sink or j >= n_c - n_recent) else 0)
    offs = [0]
    for h in range(n_heads):
        offs.append(offs[-1] + sum(mask[h * n_c:(h + 1) * n_c]))
    return mask, offs, [1 if h in kept else 0 for h in range(n_heads)]


@pytest.mark.parametrize("K_heads,n_sink,n_recent", [(3, 2, 4), (0, 1, 1), (7, 0, 0), (2, 0, 5),
                                                      (4, 6, 9), (1, 20, 0), (5, 11, 11)])
def test_head_evict_brute_force(K_heads, n_sink, n_recent):
    rng = np.random.default_rng(80 + K_heads)
    S = (rng.integers(0, 5, (7, 13)) / 8.0)          # equal head maxima happen: ties
    m, o, keep = ras.head_evict(S, K_heads, n_sink, n_recent)
    bm, bo, bk = _brute_head_evict(S.tolist(), K_heads, n_sink, n_recent)
    assert m.tolist() == bm and o.tolist() == bo and keep.tolist() == bk
    # closed form of the kept count: whole heads plus two windows per evicted head
    n_c = S.shape[1]
    w = min(n_c, min(n_sink, n_c) + min(n_recent, n_c))
    assert int(o[-1]) == K_heads * n_c + (S.shape[0] - K_heads) * w


def test_head_evict_ties_go_to_lower_index():
    S = np.zeros((4, 5))
    S[1, 2] = S[3, 0] = S[2, 4] = 0.5                 # heads 1, 2, 3 tie at 0.5
    _, _, keep = ras.head_evict(S, 2, 0, 0)
    assert keep.tolist() == [0, 1, 1, 0]


def _brute_token_evict(S, K_tokens):
    n_heads, n_c = len(S), len(S[0])
    score = [max(S[h][j] for h in range(n_heads)) for j in range(n_c)]
    kept = set(sorted(range(n_c), key=lambda j: (-score[j], j))[:K_tokens])
    mask = [1 if j in kept else 0 for h in range(n_heads) for j in range(n_c)]
    return mask, [h * K_tokens for h in range(n_heads + 1)], [1 if j in kept else 0
                                                              for j in range(n_c)]


@pytest.mark.parametrize("K_tokens", [0, 1, 6, 17, 19])
def test_token_evict_brute_force(K_tokens):
    rng = np.random.default_rng(90 + K_tokens)
    S = rng.integers(0, 6, (5, 19)) / 16.0
    m, o, keep = ras.token_evict(S, K_tokens)
    bm, bo, bk = _brute_token_evict(S.tolist(), K_tokens)
    assert m.tolist() == bm and o.tolist() == bo and keep.tolist() == bk
    # every head keeps the same positions, K_tokens of them
    assert np.all(m.reshape(5, 19) == keep[None, :]) and int(keep.sum()) == K_tokens


def test_evictions_compose_with_compaction():
    """The packed cache of either eviction holds, per head, exactly the rows
    its mask keeps, in ascending position."""
    rng = np.random.default_rng(95)
    S = rng.random((6, 40))
    kc = rng.integers(0, 1 << 16, (6, 40, 8), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, (6, 40, 8), dtype=np.uint16)
    for m, o, _ in (ras.head_evict(S, 2, 3, 5), ras.token_evict(S, 9)):
        ko, vo, idx = ras.compact(kc, vc, m, o)
        for h in range(6):
            js = [j for j in range(40) if m[h * 40 + j]]
            assert idx[o[h]:o[h + 1]].tolist() == js
            assert np.array_equal(ko[o[h]:o[h + 1]], kc[h, js])
