"""The longest context one scoring call takes: one head's keys just under
2 GiB in bf16 (the range of the buffer loads that stage them), n_c =
16,777,215 / 8,388,607 / 4,194,303 keys at d = 64 / 128 / 256, ragged in
the last 32-key tile, against the oracle on the whole problem (bf16 at each
d, fp32 at d = 128).

Query rows are zero except a few planted ones (a multiple of one key), so
the scores span the uniform floor 1/(n_c + i + 1) of the zero rows and the
large probabilities the planted rows put on their target keys, the first and
the last context key among them.  Inputs come from torch's seeded device
generator and are copied to the host for the oracle (fp64, rows in blocks of
64: about 30 GB of host memory at the peak).

Tolerances: scores 1e-9 + 1e-4 |ref| (the floor is 1.2e-7); bf16 outputs
|dO| <= 2^-8 sum_j p_j |v_j| + 1e-6 (p rounded to bf16, relative 2^-9, with
a factor 2 of slack); fp32 outputs 1e-5 + 1e-4 |O|.
"""
import math

import numpy as np
import pytest

from attention_score_reduction_amd import kvz
from oracle import ras
from tests.helpers import assert_scores_close, bits_of

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_IN, N_PROMPT = 64, 16
ALPHA = 2.5
N_C_MAX = {64: 16_777_215, 128: 8_388_607, 256: 4_194_303}  # n_c * d * 2 < 2^31


def _planted(n_c):
    """(row i, target) with one query head: targets are context keys
    ("c", j) or chunk keys ("in", m), m <= i."""
    return [(63, ("c", n_c - 1)), (1, ("c", 0)), (32, ("c", n_c // 2)), (40, ("in", 20)),
            (50, ("c", n_c - 33))]


def _device_inputs(dtype, N_C, D):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261205)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    r = lambda *s: torch.randn(*s, generator=gen, device="cuda", dtype=torch.float32).to(tdt)
    kc, vc, kin, vin = r(1, N_C, D), r(1, N_C, D), r(1, N_IN, D), r(1, N_IN, D)
    q = torch.zeros(1, 1, N_IN, D, dtype=tdt, device="cuda")
    for i, (kind, t) in _planted(N_C):
        q[0, 0, i] = (ALPHA * (kc[0, t] if kind == "c" else kin[0, t]).float()).to(tdt)
    torch.cuda.synchronize()
    return q, kc, kin, vc, vin


def _f64(x, dtype):
    return ras.to_f64(bits_of(x) if dtype == "bf16" else x.cpu().numpy(), dtype)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("bf16", 256), ("f32", 128)])
def test_scores_and_output_at_the_context_limit(dtype, D):
    N_C = N_C_MAX[D]
    q, kc, kin, vc, vin = _device_inputs(dtype, N_C, D)
    scale = 1.0 / math.sqrt(D)
    S1 = torch.zeros(1, N_C, dtype=torch.float32, device="cuda")
    kvz.kvz_score_chunk(q, kc, kin, S1, N_PROMPT, scale)
    S2 = torch.zeros(1, N_C, dtype=torch.float32, device="cuda")
    O = kvz.kvz_score_chunk_attn(q, kc, kin, vc, vin, S2, N_PROMPT, scale=scale)
    torch.cuda.synchronize()
    S1, S2, O = S1.cpu().numpy(), S2.cpu().numpy(), O.cpu().numpy()

    q64, kin64 = _f64(q, dtype), _f64(kin, dtype)
    kc64 = _f64(kc, dtype)
    del kc
    ref = np.zeros((1, N_C))
    ras.score_chunk(q64, kc64, kin64, scale, ref, row_block=64)
    assert ref[0, 0] > 0.2 and ref[0, N_C - 1] > 0.2  # planted on the first and last key
    assert_scores_close(S1, ref, atol=1e-9, rtol=1e-4, what=f"S {dtype} n_c={N_C}")
    assert_scores_close(S2, ref, atol=1e-9, rtol=1e-4, what=f"fused S {dtype} n_c={N_C}")
    del ref

    vc64, vin64 = _f64(vc, dtype), _f64(vin, dtype)
    del vc
    ref_o = ras.chunk_attention_output(q64, kc64, kin64, vc64, vin64, scale, row_block=64)
    if dtype == "bf16":
        np.abs(vc64, out=vc64)
        np.abs(vin64, out=vin64)
        mag = ras.chunk_attention_output(q64, kc64, kin64, vc64, vin64, scale, row_block=64)
        tol = 2.0 ** -8 * mag + 1e-6
    else:
        tol = 1e-5 + 1e-4 * np.abs(ref_o)
    err = np.abs(O.astype(np.float64) - ref_o)
    print(f"O {dtype} n_c={N_C}: max err {err.max():.3e}, max err / tol {(err / tol).max():.3f}",
          flush=True)
    assert np.all(err <= tol)
