"""The oracle's pins catch plausible mistakes in it. Each mutant below plants one mistake (a
dropped term, a wrong sign, index or operand, a missing step of the method) in a temporary copy
of oracle/lite_attn_oracle.py; the pin suite (tests/test_oracle_pins.py) then runs against that
copy in a subprocess and must fail. An unchanged copy must pass (the harness itself works).
Nothing here touches the oracle in the repository or anything the GPU path uses."""
import concurrent.futures
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "lite_attn_oracle.py")

# (name, [(old, new), ...]): every `old` must occur exactly once in the oracle's source
MUTANTS = [
    ("softmax scale dropped",
     [("s = scale * (qi @ kh.T)", "s = (qi @ kh.T)")]),
    ("V in place of K in the scores",
     [("s = scale * (qi @ kh.T)", "s = scale * (qi @ vh.T)")]),
    ("budget added instead of subtracted",
     [("margin = np.max(mt - running) - log_eps", "margin = np.max(mt - running) + log_eps")]),
    ("minimum over the tile's rows instead of the maximum",
     [("margin = np.max(mt - running) - log_eps", "margin = np.min(mt - running) - log_eps")]),
    ("running maximum updated before the test",
     [("        mt = tile_max[:, j]\n", "        mt = tile_max[:, j]\n        running = np.maximum(running, mt)\n")]),
    ("descending steps traversed ascending",
     [("order = range(tk - 1, -1, -1) if descending else range(tk)", "order = range(tk)")]),
    ("dense-prefix columns not exempt",
     [("col_exempt = j * tile_k < dense_prefix", "col_exempt = False")]),
    ("dense-prefix rows not exempt",
     [("row_exempt = i * tile_q < dense_prefix", "row_exempt = False")]),
    ("softmax not normalised",
     [("out = (p @ vh) / p.sum(axis=1, keepdims=True)", "out = p @ vh")]),
    ("earlier flags not carried forward",
     [("mask_next[b, h, i] = mask[b, h, i] | bits_to_mask(flags)",
       "mask_next[b, h, i] = bits_to_mask(flags)")]),
    ("the mask ignored by the output",
     [("allowed_cols = np.repeat(~out_skipped, tile_k)[:n]", "allowed_cols = np.ones(n, dtype=bool)")]),
    ("skipped tiles still tested",
     [("        if skipped[j]:\n            continue\n", "")]),
    ("bit order reversed inside the mask words",
     [("return ((mask[..., j // 32] >> (j % 32).astype(np.uint32)) & 1).astype(bool)",
       "return ((mask[..., j // 32] >> (31 - j % 32).astype(np.uint32)) & 1).astype(bool)"),
      ("out[..., j // 32] |= bits[..., j].astype(np.uint32) << np.uint32(j % 32)",
       "out[..., j // 32] |= bits[..., j].astype(np.uint32) << np.uint32(31 - j % 32)")]),
    ("non-strict test (a zero margin flags)",
     [("if margin < 0 and not (row_exempt or col_exempt):",
       "if margin <= 0 and not (row_exempt or col_exempt):")]),
    ("a NaN margin flags",
     [("if margin < 0 and not (row_exempt or col_exempt):",
       "if not (margin >= 0) and not (row_exempt or col_exempt):")]),
    ("in-step skip ignored",
     [("out_skipped = (skipped | flags) if in_step_skip else skipped", "out_skipped = skipped")]),
    ("ragged key tile padded with 0 instead of -inf",
     [("padded = np.full((nr, tk * tile_k), -np.inf)", "padded = np.zeros((nr, tk * tile_k))")]),
    ("refresh decision inverted",
     [("elif not (abs(stat - ref) <= refresh_delta):", "elif abs(stat - ref) <= refresh_delta:")]),
    ("refresh statistic: maximum of the rows instead of the mean",
     [("stat = float(np.mean(running))", "stat = float(np.max(running))")]),
    ("refresh keeps the row's bits",
     [("mask_next[b, h, i] = 0          # valid bits cleared, reserved bits stay 0", "pass")]),
    ("chain yields the mask after the step as its start mask",
     [("yield t, mask, res", "yield t, res.mask_next, res")]),
]


def _tree(dst, source):
    """A minimal copy of the repository: the (mutated) oracle package and the pin suite."""
    os.makedirs(os.path.join(dst, "oracle"))
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(dst, "oracle"))
    with open(os.path.join(dst, "oracle", "lite_attn_oracle.py"), "w") as f:
        f.write(source)
    tests = os.path.join(dst, "tests")
    os.makedirs(tests)
    for name in ("conftest.py", "test_oracle_pins.py", "pyref.py"):
        shutil.copy(os.path.join(ROOT, "tests", name), tests)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tests, "golden"))
    return os.path.join(tests, "test_oracle_pins.py")


def _run_pins(dst, source):
    pins = _tree(dst, source)
    env = dict(os.environ)
    env.pop("PYTHONPATH", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        pins], cwd=dst, capture_output=True, text=True, timeout=600, env=env)
    return r.returncode, r.stdout[-1500:]


def _mutate(source, edits):
    for old, new in edits:
        assert source.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
        source = source.replace(old, new)
    return source


def test_pins_catch_every_planted_mistake(tmp_path):
    source = open(ORACLE).read()
    jobs = [("unchanged", source)] + [(name, _mutate(source, edits)) for name, edits in MUTANTS]
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(lambda kv: (kv[0], _run_pins(str(tmp_path / f"m{jobs.index(kv)}"),
                                                              kv[1])), jobs))
    code, out = results[0][1]
    assert code == 0, f"the unchanged oracle copy fails its pins:\n{out}"
    survivors = []
    for name, (code, out) in results[1:]:
        # 1: a pin failed (pytest's "tests failed"); anything else is a harness problem
        assert code in (0, 1), f"{name}: pytest exit {code}\n{out}"
        if code == 0:
            survivors.append(name)
    assert not survivors, f"mutants no pin catches: {survivors}"
