"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that the pin suite catches every one: a dropped term, a wrong sign or index,
a transposed operand, an off-by-one in the mask or a slice.  Each mutant runs
the pins in a fresh process against a scratch copy of the Python packages."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what is planted, exact text in the oracle file, replacement, occurrence);
# the file is oracle/ks_oracle.py unless the name says "toy:"
MUTANTS = [
    ("mask admits i == e_j", "return (j <= rows) & (rows < ej)",
     "return (j <= rows) & (rows <= ej)", 1),
    ("mask drops the causal bound", "return (j <= rows) & (rows < ej)",
     "return rows < ej", 1),
    ("RoPE rotates the wrong way", "x1 * c - x2 * s, x2 * c + x1 * s",
     "x1 * c + x2 * s, x2 * c - x1 * s", 1),
    ("RoPE frequency exponent", "-2.0 * kk / D", "-1.0 * kk / D", 1),
    ("dS drops the D_i term", "dS = P * (dP - Di)", "dS = P * dP", 1),
    ("dK uses P instead of dS", "dk[b, cols, kv] += sc * (dS.T @ qq)",
     "dk[b, cols, kv] += sc * (P.T @ qq)", 1),
    ("GQA maps heads round robin", "kv = h // (Hq // Hkv)", "kv = h % Hkv", 2),
    ("compaction keeps block 0 always", "if keep[b][x]]", "if keep[b][x] or x == 0]", 1),
    ("decode reads one token too many", "[:L]", "[:L + 1]", 2),
    ("softmax scale squared", "return 1.0 / math.sqrt(D) if scale is None else float(scale)",
     "return 1.0 / D if scale is None else float(scale)", 1),
    ("toy: generation keeps evicted spans", "                gone[a:b] = True",
     "                gone[a:a] = True", 1),
    ("toy: MLP activation without the gate", "return x / (1.0 + np.exp(-x))", "return x", 1),
]


def _copy_tree(dst):
    for d in ("oracle", "workloads", "tests"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d),
                        ignore=shutil.ignore_patterns("__pycache__"))


def _run_pins(root, pins="test_oracle_pins.py"):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           str(root / "tests" / pins)],
                          cwd=root, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes(tmp_path):
    """control: the copied packages pass the pins, so a failure below comes
    from the planted mistake"""
    _copy_tree(tmp_path)
    for pins in ("test_oracle_pins.py", "test_toy_oracle.py"):
        r = _run_pins(tmp_path, pins)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, count):
    _copy_tree(tmp_path)
    toy = name.startswith("toy:")
    src = tmp_path / "oracle" / ("toy_stack.py" if toy else "ks_oracle.py")
    text = src.read_text()
    assert text.count(old) == count, f"mutation target moved: {old!r}"
    src.write_text(text.replace(old, new))
    r = _run_pins(tmp_path, "test_toy_oracle.py" if toy else "test_oracle_pins.py")
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout or "error" in r.stdout.lower(), r.stdout[-2000:]
