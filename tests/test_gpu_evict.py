"""Head-level and token-level eviction on the GPU (kvz_select_heads,
kvz_select_tokens), bit-exact against the oracle's head_evict / token_evict
fed the same fp32 scores, composed with kvz_compact, and on a scored layer."""
import math

import numpy as np
import pytest

from attention_score_reduction_amd import kvz
from attention_score_reduction_amd.inputs import HostGen, Workload
from oracle import ras
from tests.helpers import ATOL, RTOL, bits_of, oracle_layer_scores, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _scores(shape, seed, ties):
    rng = np.random.default_rng(seed)
    if ties:
        return (rng.integers(0, 9, shape) / 64).astype(np.float32)
    return rng.random(shape).astype(np.float32)


def check_heads(S_np, K, n_sink, n_recent):
    S = torch.from_numpy(np.ascontiguousarray(S_np)).cuda()
    m, o, keep = kvz.kvz_select_heads(S, K, n_sink, n_recent)
    torch.cuda.synchronize()
    rm, ro, rk = ras.head_evict(S_np.astype(np.float32), K, n_sink, n_recent)
    assert np.array_equal(keep.cpu().numpy(), rk), "kept heads differ"
    assert np.array_equal(o.cpu().numpy(), ro), "head offsets differ"
    got = m.cpu().numpy()
    assert np.array_equal(got, rm), f"mask differs at {np.nonzero(got != rm)[0][:10]}"


def check_tokens(S_np, K):
    S = torch.from_numpy(np.ascontiguousarray(S_np)).cuda()
    m, o, keep = kvz.kvz_select_tokens(S, K)
    torch.cuda.synchronize()
    rm, ro, rk = ras.token_evict(S_np.astype(np.float32), K)
    assert np.array_equal(keep.cpu().numpy(), rk), "kept tokens differ"
    assert np.array_equal(o.cpu().numpy(), ro), "head offsets differ"
    got = m.cpu().numpy()
    assert np.array_equal(got, rm), f"mask differs at {np.nonzero(got != rm)[0][:10]}"


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (8, 1000), (37, 4099), (256, 2048),
                                   (2000, 33), (5, 48)])
def test_select_heads_matches_oracle(shape, ties):
    n_heads, n_c = shape
    S = _scores(shape, n_heads * 7 + n_c, ties)
    for K in sorted({0, 1, n_heads // 3, n_heads // 2, n_heads - 1, n_heads}):
        for (s, r) in ((0, 0), (4, 64), (1, n_c), (n_c + 5, 3), (n_c // 2, n_c // 2 + 1)):
            check_heads(S, K, s, r)


@pytest.mark.parametrize("ties", [False, True])
@pytest.mark.parametrize("shape", [(1, 1), (3, 7), (8, 1000), (37, 4099), (2, 20000),
                                   (300, 97), (5, 48)])
def test_select_tokens_matches_oracle(shape, ties):
    n_heads, n_c = shape
    S = _scores(shape, n_heads * 11 + n_c, ties)
    for K in sorted({0, 1, n_c // 4, n_c // 2 + 1, n_c - 1, n_c}):
        check_tokens(S, K)


@pytest.mark.parametrize("mode", ["heads", "tokens"])
def test_eviction_then_compaction_bit_exact(mode):
    rng = np.random.default_rng(61)
    n_heads, n_c, d = 12, 3000, 128
    S = rng.random((n_heads, n_c)).astype(np.float32)
    S[3] *= 0.01                                       # a weak head
    kc = rng.integers(0, 1 << 16, (n_heads, n_c, d), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, (n_heads, n_c, d), dtype=np.uint16)
    Sd = torch.from_numpy(S).cuda()
    if mode == "heads":
        m, o, _ = kvz.kvz_select_heads(Sd, 5, 16, 256)
        rm, ro, _ = ras.head_evict(S, 5, 16, 256)
    else:
        m, o, _ = kvz.kvz_select_tokens(Sd, 700)
        rm, ro, _ = ras.token_evict(S, 700)
    total = int(ro[-1])
    ko = torch.empty(total, d, dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    idx = torch.empty(total, dtype=torch.int32, device="cuda")
    kvz.kvz_compact(to_dev(kc, "bf16"), to_dev(vc, "bf16"), m, o, ko, vo, idx)
    torch.cuda.synchronize()
    rko, rvo, ridx = ras.compact(kc, vc, rm, ro)
    assert np.array_equal(bits_of(ko), rko) and np.array_equal(bits_of(vo), rvo)
    assert np.array_equal(idx.cpu().numpy(), ridx)


def test_evictions_on_a_scored_cache():
    """Scores of a 2-layer, 4-KV-head cache from the GPU's score kernel: both
    evictions bit-exact against the oracle fed the GPU's scores; against the
    oracle's own fp64 scores the kept heads and tokens agree except where two
    aggregate scores lie within the score tolerance of each other."""
    wl = Workload("evict_e2e", 62, 2, 4, 4, 128, 2500, 1024, 16, 0.3, key_lognormal_sigma=1.0,
                  sink=True)
    gen = HostGen(wl)
    H = wl.heads
    S = torch.zeros(wl.n_heads, wl.n_ctx, dtype=torch.float32, device="cuda")
    refs = []
    for l in range(wl.layers):
        kc, _ = gen.context(l)
        kc_d = to_dev(kc, "bf16")
        for k in range(len(wl.chunks())):
            q, kin = gen.chunk_inputs(l, k)
            kvz.kvz_score_chunk(to_dev(q, "bf16"), kc_d, to_dev(kin, "bf16"),
                                S[l * H:(l + 1) * H], wl.n_prompt, 1 / math.sqrt(wl.head_dim))
        refs.append(oracle_layer_scores(gen, l, list(range(H))))
    torch.cuda.synchronize()
    s_gpu = S.cpu().numpy()
    s_ref = np.concatenate(refs)
    K_h, K_t = 3, kvz.kvz_keep_count(wl.n_ctx, 0.3)
    check_heads(s_gpu, K_h, 4, 128)
    check_tokens(s_gpu, K_t)
    # against the oracle's own scores
    _, _, kh = ras.head_evict(s_gpu, K_h, 4, 128)
    _, _, kh_ref = ras.head_evict(s_ref, K_h, 4, 128)
    hs = ras.head_scores(s_ref)
    tau_h = np.sort(hs)[::-1][K_h - 1]
    flip = np.nonzero(kh != kh_ref)[0]
    assert np.all(np.abs(hs[flip] - tau_h) <= ATOL + RTOL * tau_h)
    _, _, kt = ras.token_evict(s_gpu, K_t)
    _, _, kt_ref = ras.token_evict(s_ref, K_t)
    ts = ras.token_scores(s_ref)
    tau_t = np.sort(ts)[::-1][K_t - 1]
    flip = np.nonzero(kt != kt_ref)[0]
    assert flip.size <= 0.001 * wl.n_ctx + 2
    assert np.all(np.abs(ts[flip] - tau_t) <= ATOL + RTOL * tau_t)


@pytest.mark.parametrize("ties", [False, True])
def test_evictions_at_full_cache_size(ties):
    """The 128K LLaMA cache's score array (256 (layer, head) rows x 131072
    tokens, the launch shapes the benchmark times): head eviction keeping 77
    heads whole with 64 + 1024-token windows, token eviction keeping 39322
    positions, both bit-exact against the oracle on the same scores."""
    S = _scores((256, 131072), 4242 + int(ties), ties)
    check_heads(S, 77, 64, 1024)
    check_tokens(S, 39322)
