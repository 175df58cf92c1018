"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a scratch copy of oracle/ras.py (CPU only) and runs
tests/test_oracle_pins.py against it, which must fail."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    # (name, text in oracle/ras.py, replacement)
    ("causal mask shifted by one key",
     "invisible = t[None, :] > rows[:, None]",
     "invisible = t[None, :] > rows[:, None] + 1"),
    ("causal limits counted from the row block",
     "invisible = t[None, :] > rows[:, None]",
     "invisible = t[None, :] > (rows - rows[0])[:, None]"),
    ("select breaks ties to the higher index",
     "order = np.lexsort((np.arange(N), -S_flat.astype(np.float64)))",
     "order = np.lexsort((-np.arange(N), -S_flat.astype(np.float64)))"),
    ("select keeps K + 1",
     "mask[order[:K]] = 1",
     "mask[order[:K + 1]] = 1"),
    ("tau is the (K+1)-th score",
     "tau = float(S_flat[order[K - 1]]) if K > 0 else math.inf",
     "tau = float(S_flat[order[min(K, N - 1)]]) if K > 0 else math.inf"),
    ("sink window one token too long",
     "window = (j < n_sink) | (j >= n_c - n_recent)",
     "window = (j <= n_sink) | (j >= n_c - n_recent)"),
    ("recent window one token too short",
     "window = (j < n_sink) | (j >= n_c - n_recent)",
     "window = (j < n_sink) | (j > n_c - n_recent)"),
    ("decode without the scale",
     "x = (q[h] @ K.T) * scale",
     "x = (q[h] @ K.T)"),
    ("decode weights the keys instead of the values",
     "out[h] = p @ V",
     "out[h] = p @ K"),
    ("attention output over the keys",
     "vals = np.concatenate([v_ctx[h], v_in[h]], axis=0)",
     "vals = np.concatenate([k_ctx[h], k_in[h]], axis=0)"),
    ("token score is the mean over heads",
     "return np.asarray(S2d).max(axis=0)",
     "return np.asarray(S2d).mean(axis=0)"),
    ("head score is the sum over tokens",
     "return np.asarray(S2d).max(axis=1)",
     "return np.asarray(S2d).sum(axis=1)"),
    ("only the first query head of a group",
     "        for g in range(G):\n            for r0 in range(0, n_in, row_block):\n                rows = np.arange(r0, min(n_in, r0 + row_block))\n                if mode",
     "        for g in range(1):\n            for r0 in range(0, n_in, row_block):\n                rows = np.arange(r0, min(n_in, r0 + row_block))\n                if mode"),
    ("score overwritten instead of a running max",
     "np.maximum(S[h], P[:, :n_c].max(axis=0), out=S[h])",
     "S[h] = P[:, :n_c].max(axis=0)"),
    ("softmax over the context keys only",
     "keys = np.concatenate([k_ctx_h, k_in_h], axis=0)",
     "keys = np.concatenate([k_ctx_h, 0 * k_in_h - 1e300], axis=0)"),
    ("sum aggregation takes the max",
     "S[h] += P[:, :n_c].sum(axis=0)",
     "S[h] += P[:, :n_c].max(axis=0)"),
    ("compaction stores positions from 1",
     "idx[o:o + len(js)] = js",
     "idx[o:o + len(js)] = js + 1"),
    ("compaction takes V rows for K",
     "k_out[o:o + len(js)] = k_ctx[h, js]",
     "k_out[o:o + len(js)] = v_ctx[h, js]"),
]


def _run_pins(tmp_path, old=None, new=None):
    """Run the pin suite on a scratch copy of the oracle, with `old`
    replaced by `new` in oracle/ras.py when given."""
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    (tmp_path / "tests").mkdir()
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    for f in ("test_oracle_pins.py", "helpers.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests")
    if old is not None:
        src = tmp_path / "oracle" / "ras.py"
        text = src.read_text()
        assert text.count(old) == 1, f"mutation site not unique: {old}"
        src.write_text(text.replace(old, new))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True,
                          text=True, timeout=300)


def test_pins_pass_on_the_unchanged_copy(tmp_path):
    # the control: the scratch setup itself passes, so each failure below
    # comes from its planted mistake
    r = _run_pins(tmp_path)
    assert r.returncode == 0, r.stdout[-800:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_fail_on_planted_mistake(tmp_path, name, old, new):
    r = _run_pins(tmp_path, old, new)
    assert r.returncode != 0, f"the pins pass with the planted mistake: {name}\n{r.stdout[-500:]}"
    assert "ImportError" not in r.stdout and "ModuleNotFoundError" not in r.stdout, r.stdout[-800:]
