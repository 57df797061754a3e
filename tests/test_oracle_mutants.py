"""Planted mistakes in the oracle, on the CPU: each mutant below is a copy of
the oracle with one plausible error (a dropped term, a wrong sign, index or
bound, a transposed or swapped operand).  The pin suites (test_oracle.py,
test_oracle_rope.py, test_oracle_threshold.py) must fail on every one of them, and pass on an
unmodified copy, which shows the pins constrain each part of the oracle and
that the copy is the module the suites import."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_SUITES = [os.path.join(ROOT, "tests", "test_oracle.py"),
              os.path.join(ROOT, "tests", "test_oracle_rope.py"),
              os.path.join(ROOT, "tests", "test_oracle_threshold.py")]

# (name, original text, planted text) in oracle/lcsa_oracle.py
MUTANTS = [
    ("kv_frames_max", "min(qf + cf, _snap_ceil(ratio * qf))", "max(qf + cf, _snap_ceil(ratio * qf))"),
    ("budget_floor", "return int(math.floor(x + 0.5))", "return int(math.floor(x))"),
    ("window_half_open", "(np.abs(kx - bx) <= g.half)", "(np.abs(kx - bx) < g.half)"),
    ("window_full_range", 'half=desc["local_range"] // 2', 'half=desc["local_range"]'),
    ("block_tokens_transposed", "((t * g.grid_h + ys[:, None]) * g.grid_w + xs[None, :])",
     "((t * g.grid_h + xs[None, :]) * g.grid_w + ys[:, None])"),
    ("pool_sum_not_mean", ".sum(axis=1) / len(tok)", ".sum(axis=1)"),
    ("score_channels_misaligned", 'kbar[:, :, e, :])', 'kbar[:, :, e, ::-1])'),
    ("select_lowest_scores", "np.lexsort((e, -s[b, h, qb, e]))", "np.lexsort((e, s[b, h, qb, e]))"),
    ("select_ties_to_higher", "np.lexsort((e, -s[b, h, qb, e]))", "np.lexsort((-e, -s[b, h, qb, e]))"),
    ("select_unsorted_row", "rows.append(np.sort(order[:keep]))", "rows.append(order[:keep])"),
    ("attend_scale_dropped", "z = (qi @ kj.T) * g.scale", "z = (qi @ kj.T)"),
    ("attend_not_normalised", "o = (p @ vj) / den", "o = (p @ vj)"),
    ("attend_values_are_keys", "vj = v[b, ktok, h, :]", "vj = k[b, ktok, h, :]"),
    ("attend_lse_without_log", "lse = m[:, 0] + np.log(den[:, 0])", "lse = m[:, 0] + den[:, 0]"),
    ("attend_row_head_swap", "r = (b * g.heads + h) * g.nqb + qb", "r = (h * g.batch + b) * g.nqb + qb"),
    ("flops_half", "return 4.0 * g.head_dim", "return 2.0 * g.head_dim"),
    ("attend_rows_head_block_swapped", "        h, qb = divmod(rem, g.nqb)\n        blocks",
     "        qb, h = divmod(rem, g.heads)\n        blocks"),
    ("attend_rows_batch_stride", "b, rem = divmod(int(r), g.heads * g.nqb)",
     "b, rem = divmod(int(r), g.batch * g.nqb)"),
]

# the same in oracle/rope_oracle.py
ROPE_MUTANTS = [
    ("rope_sine_sign", "out[..., 0::2] = x0 * c - x1 * s", "out[..., 0::2] = x0 * c + x1 * s"),
    ("rope_rows_and_columns_swapped", "tab.h[pos_h], tab.w[pos_w]", "tab.h[pos_w % tab.h.shape[0]], tab.w[pos_h]"),
    ("rope_query_frame_offset", "g.kv_frames - g.q_frames, round_out", "0, round_out"),
    ("rope_rounds_through_float32", "b = np.ascontiguousarray(x, dtype=np.float64)",
     "b = np.ascontiguousarray(np.asarray(x, dtype=np.float32), dtype=np.float64)"),
    ("rope_ties_away_from_zero", "(b + half_minus_one + lsb)", "(b + half_minus_one + np.uint64(1))"),
    ("rope_token_row_from_columns", "(s // grid_w) % grid_h, s % grid_w", "s % grid_h, s % grid_w"),
]


# the same in oracle/threshold_oracle.py
THRESHOLD_MUTANTS = [
    ("threshold_strict", "out.append(e[s[b, h, qb, e] >= tau[r]])", "out.append(e[s[b, h, qb, e] > tau[r]])"),
    ("threshold_one_past_keep", "np.sort(s[b, h, qb, e])[::-1][keep - 1]",
     "np.sort(s[b, h, qb, e])[::-1][min(keep, len(e) - 1)]"),
    ("threshold_smallest_instead", "np.sort(s[b, h, qb, e])[::-1][keep - 1]", "np.sort(s[b, h, qb, e])[keep - 1]"),
    ("threshold_whole_row", "out.append(e[s[b, h, qb, e] >= tau[r]])",
     "out.append(np.flatnonzero(s[b, h, qb] >= tau[r]))"),
    ("threshold_padding_zero", "col_idx = np.full(len(rows) * w, -1, dtype=np.int64)",
     "col_idx = np.full(len(rows) * w, 0, dtype=np.int64)"),
    ("threshold_row_order_swapped", "yield (b * g.heads + h) * g.nqb + qb, b, h, qb",
     "yield (h * g.batch + b) * g.nqb + qb, b, h, qb"),
]


def _run_suite(tmp, name, fname, old, new):
    d = os.path.join(tmp, name)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    if old is not None:
        src = open(os.path.join(ROOT, "oracle", fname)).read()
        assert src.count(old) == 1, f"{name}: mutation site not unique or missing"
        open(os.path.join(d, "oracle", fname), "w").write(src.replace(old, new))
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([d, ROOT]), OMP_NUM_THREADS="2")
    # run from the copy's directory: `python -m` puts the working directory
    # first on sys.path, so the copy shadows the repository's oracle
    # the suite of the mutated module first: with -x a caught mutant stops
    # at its first failing pin instead of after the other suites pass
    own = {"rope_oracle.py": 1, "threshold_oracle.py": 2}.get(fname, 0)
    suites = [PIN_SUITES[own]] + [x for i, x in enumerate(PIN_SUITES) if i != own]
    r = subprocess.run([sys.executable, "-m", "pytest", *suites,
                        "-x", "-q", "-p", "no:cacheprovider", "--rootdir", ROOT], cwd=d, env=env,
                       capture_output=True, text=True, timeout=900)
    return name, r.returncode, (r.stdout + r.stderr)[-600:]


def test_pins_fail_on_every_planted_mistake(tmp_path):
    jobs = ([("control", None, None, None)]
            + [(n, "lcsa_oracle.py", a, b) for n, a, b in MUTANTS]
            + [(n, "rope_oracle.py", a, b) for n, a, b in ROPE_MUTANTS]
            + [(n, "threshold_oracle.py", a, b) for n, a, b in THRESHOLD_MUTANTS])
    with ThreadPoolExecutor(max_workers=6) as pool:
        results = list(pool.map(lambda j: _run_suite(str(tmp_path), *j), jobs))
    control = results[0]
    assert control[1] == 0, "unmodified oracle copy fails its pins:\n" + control[2]
    survivors = [(n, tail) for n, rc, tail in results[1:] if rc != 1]
    # exit status 1 = tests ran and some failed (not a collection or usage error)
    assert not survivors, "mutants not caught by the pins: " + ", ".join(n for n, _ in survivors) \
        + "\n" + "\n".join(t for _, t in survivors)
