"""The oracle's pins catch plausible slips (CPU only).

Each case plants one plausible mistake in a temporary copy of
oracle/proxyattn.py -- a wrong causal comparison, a dropped mask or scale, a
wrong head map, a reversed tie-break, an off-by-one budget, a wrong probe
average, a wrong query offset of the strided scoring, a wrong rounding of the
ratio budget, a wrong skip rule -- and runs the oracle pin tests against that
copy in a separate process.  Every planted slip must make some pin fail (pytest
exit status 1: a test failed, not a crash while collecting); the unchanged copy
must pass.  The repository's oracle itself is never modified.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle_pins.py", "tests/test_golden.py"]

# name -> (exact text in oracle/proxyattn.py, its replacement)
MUTATIONS = {
    "score_causal_strict": ("np.where(np.arange(nkeys)[None, :] <= rows[:, None], L, NEG_INF)",
                            "np.where(np.arange(nkeys)[None, :] < rows[:, None], L, NEG_INF)"),
    "score_no_causal_mask": ("np.where(np.arange(nkeys)[None, :] <= rows[:, None], L, NEG_INF)", "L"),
    "score_no_scale": ("L = scale * (qbar_g[rows] @ kbar_g[:nkeys].T)",
                       "L = (qbar_g[rows] @ kbar_g[:nkeys].T)"),
    "stride_first_query": ("rows = toks[query_stride - 1::query_stride]",
                           "rows = toks[0::query_stride]"),
    "stride_drops_last_query": ("if toks.size % query_stride:", "if False:"),
    "kv_head_modulo": ("return h // (H // Hkv)", "return h % Hkv"),
    "group_modulo": ("return h // (H // G)", "return h % G"),
    "kbar_sum": ("kbar[g] = np.mean(np.asarray(k[kh], dtype=np.float64), axis=0)",
                 "kbar[g] = np.sum(np.asarray(k[kh], dtype=np.float64), axis=0)"),
    "tie_break_reversed": ("return np.lexsort((J, -s))", "return np.lexsort((-J, -s))"),
    "ranking_ascending": ("return np.lexsort((J, -s))", "return np.lexsort((J, s))"),
    "ranking_in_float32": ("s = np.asarray(S_row[: I + 1], dtype=np.float64)",
                           "s = np.asarray(S_row[: I + 1], dtype=np.float32).astype(np.float64)"),
    "pool_rounded_bf16": ("        kbar[g] = np.mean(np.asarray(k[kh], dtype=np.float64), axis=0)\n    return",
                          "        kbar[g] = np.mean(np.asarray(k[kh], dtype=np.float64), axis=0)\n"
                          "    qbar = qbar.astype(np.float32).astype(np.float64)\n    return"),
    "budget_strict": ("if cum >= gamma:", "if cum > gamma:"),
    "budget_off_by_one": ("order[: min(int(k), I + 1)]", "order[: min(int(k) + 1, I + 1)]"),
    "no_diagonal": ("    kept.add(I)\n", ""),
    "masses_no_causal_mask": ("L = np.where(np.arange(N)[None, :] <= rows[:, None], L, NEG_INF)",
                              "pass"),
    "masses_wrong_ranking_row": ("order = rank_blocks(S[g, nb - 1], nb - 1)",
                                 "order = rank_blocks(S[g, 0], nb - 1)"),
    "probe_average_full_blocks": ("count += rows.size", "count += block"),
    "ratio_floor": ("int(np.ceil(prod))", "int(np.floor(prod))"),
    "attn_no_causal_mask": ("L = np.where(cols[None, :] <= qrows[:, None], L, NEG_INF)", "pass"),
    "attn_no_scale": ("L = scale * (qi @ np.asarray(k_kv[cols], dtype=np.float64).T)",
                      "L = (qi @ np.asarray(k_kv[cols], dtype=np.float64).T)"),
    "skip_descending_order": ("        for J in sorted(int(b) for b in blocks if 0 <= b <= I):\n            cols",
                              "        for J in sorted((int(b) for b in blocks if 0 <= b <= I), reverse=True):\n            cols"),
    "skip_updates_running_state": ("                skipped.append((J, r))\n                continue\n",
                                   "                skipped.append((J, r))\n"),
    "skip_bound_undercounts_mass": ("if math.exp(x.max() - M) < threshold)", "if math.exp(x.max() - M) < threshold / 4)"),
    "density_diagonal_whole": ("keep.sum() - 0.5 * diag", "keep.sum()"),
    "blocks_floor": ("return -(-N // block)", "return max(1, N // block)"),
    "partial_block_past_the_end": ("np.arange(I * block, min((I + 1) * block, N))",
                                   "np.arange(I * block, (I + 1) * block)"),
    "group_kv_first_only": ("return sorted({kv_head_of(h, H, Hkv) for h in group_query_heads(g, H, G)})",
                            "return [kv_head_of(g * (H // G), H, Hkv)]"),
}

# The pin tests run against the copy: it is imported before pytest starts, so
# `from oracle import proxyattn` in the tests finds it in sys.modules.
DRIVER = r"""
import sys
sys.path.insert(0, sys.argv[1])
import oracle
assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__
sys.path.insert(1, sys.argv[2])
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + sys.argv[3:]))
"""


def _run_pins(tmp_path, name, source):
    pkg = tmp_path / name / "oracle"
    pkg.mkdir(parents=True)
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), pkg / "__init__.py")
    (pkg / "proxyattn.py").write_text(source)
    env = dict(os.environ, OMP_NUM_THREADS="2", PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-c", DRIVER, str(tmp_path / name), ROOT] + PIN_TESTS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


def test_every_planted_slip_fails_a_pin(tmp_path):
    src = open(os.path.join(ROOT, "oracle", "proxyattn.py")).read()
    for name, (old, _) in MUTATIONS.items():
        assert src.count(old) == 1, f"{name}: the text to mutate must occur exactly once"
    jobs = {"unchanged": src}
    jobs.update({n: src.replace(old, new, 1) for n, (old, new) in MUTATIONS.items()})
    with ThreadPoolExecutor(max_workers=4) as pool:
        results = dict(zip(jobs, pool.map(lambda kv: _run_pins(tmp_path, *kv), jobs.items())))
    rc, out = results.pop("unchanged")
    assert rc == 0, "the unchanged oracle copy must pass its pins:\n" + out
    missed = {n: rc for n, (rc, _) in results.items() if rc != 1}
    assert not missed, "slips not caught by a failing pin (exit status): " + repr(missed)
