"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/ep_oracle.py (a text
substitution: a dropped weight, a wrong tie rule, another claim order, a
reciprocal-multiply scale, swapped byte order, a missing rebase, an
off-by-one bound, a changed summation order, a bias added at the end, a
wrong segment rounding, a wrong expert's weights) and runs the CPU pin tests
against the copy in a child process: they must fail.  An unmutated copy
must pass, so a failure is the mistake's doing.  Only the oracle is
changed; the kernels are not involved.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FORMATS = "test_oracle_formats.py"
LAYOUT = "test_oracle_layout.py"
DC = "test_oracle_dispatch_combine.py"
NEXT = "test_oracle_next.py"
PROPS = "test_oracle_properties.py"

# name -> ([(old, new), ...], pin files expected to catch it)
MUTATIONS = {
    "combine drops the weight": (
        [("        p = (w[sel, k][:, None] * rows).astype(np.float32)\n        acc[sel]",
          "        p = rows.astype(np.float32)\n        acc[sel]")],
        [DC],
    ),
    "bf16 ties away from zero": (
        [("up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint32(1)) == 1))", "up = lo >= 0x8000")],
        [FORMATS],
    ),
    "e4m3 ties to the odd code": (
        [("((m == mid) & ((hi & 1) == 0))", "((m == mid) & ((hi & 1) == 1))")],
        [FORMATS],
    ),
    "slots claimed in (k, t) order": (
        [("    for t in range(T):\n        for k in range(K):\n            if vl[t][k]:\n                e = idl[t][k]\n"
          "                slot[t][k] = offsets[e] + claimed[e]",
          "    for k in range(K):\n        for t in range(T):\n            if vl[t][k]:\n                e = idl[t][k]\n"
          "                slot[t][k] = offsets[e] + claimed[e]")],
        [LAYOUT],
    ),
    "fp8 quotient by reciprocal multiply": (
        [("v = (xf[nz] / s[nz][:, None]).astype(np.float32)",
          "v = (xf[nz] * (np.float32(1.0) / s[nz])[:, None]).astype(np.float32)")],
        [DC],
    ),
    "fp8 scales big-endian": (
        [('s.astype("<f4")', 's.astype(">f4")')],
        [FORMATS, DC],
    ),
    "grouped list ids not rebased": (
        [("ridx[r, k] = idl[t][k] - g * epg", "ridx[r, k] = idl[t][k]")],
        [LAYOUT],
    ),
    "expert id E treated as valid": (
        [("valid = (idx >= 0) & (idx < E)", "valid = (idx >= 0) & (idx <= E)")],
        [LAYOUT],
    ),
    "grouped combine without group partials": (
        [("            P[sel] = (P[sel] + p).astype(np.float32)", "            tot[sel] = (tot[sel] + p).astype(np.float32)")],
        [DC],
    ),
    "groups summed in reverse order": (
        [("    for g in range(num_groups):\n        P = np.zeros_like(tot)",
          "    for g in reversed(range(num_groups)):\n        P = np.zeros_like(tot)")],
        [DC],
    ),
    "bias added after the reduction": (
        [("    acc = _bias_seed(bias0, bias1, (T, y.shape[1]))\n    for k in range(K):",
          "    acc = np.zeros((T, y.shape[1]), dtype=np.float32)\n    for k in range(K):"),
         ("        acc[sel] = (acc[sel] + p).astype(np.float32)\n    return bf16_rne(acc)",
          "        acc[sel] = (acc[sel] + p).astype(np.float32)\n"
          "    return bf16_rne((acc + _bias_seed(bias0, bias1, acc.shape)).astype(np.float32))")],
        [NEXT],
    ),
    "aligned segment rounded wrongly": (
        [("seg = (counts[e] + A - 1) // A * A", "seg = counts[e] // A * A + (A if A > 1 else 0)")],
        [NEXT, PROPS],
    ),
    "gemm uses the next expert's weights": (
        [("y[rs] = x[rs] @ w[e].T", "y[rs] = x[rs] @ w[(e + 1) % E].T")],
        [NEXT],
    ),
    "gemm bound without the accumulation term": (
        [("return np.abs(y64) * 2.0**-8 + absdot * H * 2.0**-24", "return np.abs(y64) * 2.0**-8")],
        [NEXT],
    ),
}


def _copy_tree(dst):
    for d in ("oracle", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d),
                        ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    for f in ("conftest.py", FORMATS, LAYOUT, DC, NEXT, PROPS):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))


def _run_pins(dst, files):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join("tests", f) for f in files]]
    return subprocess.run(cmd, cwd=dst, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes(tmp_path):
    _copy_tree(str(tmp_path))
    res = _run_pins(str(tmp_path), [FORMATS, LAYOUT, DC, NEXT, PROPS])
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch(name, tmp_path):
    subs, files = MUTATIONS[name]
    _copy_tree(str(tmp_path))
    path = os.path.join(str(tmp_path), "oracle", "ep_oracle.py")
    src = open(path).read()
    for old, new in subs:
        assert src.count(old) >= 1, f"mutation text not found: {old[:60]!r}"
        src = src.replace(old, new, 1)
    open(path, "w").write(src)
    res = _run_pins(str(tmp_path), files)
    assert res.returncode != 0, f"the pins in {files} did not catch: {name}\n" + res.stdout[-1500:]
