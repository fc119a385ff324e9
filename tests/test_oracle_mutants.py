"""The oracle's pins catch plausible mistakes.

Each case plants one mistake -- a dropped term, a wrong sign, index or operand, an
off-by-one, a broken special-value rule -- in a copy of the oracle in a temporary
directory (the C oracle is rebuilt there with the same compiler flags; the fp64
backward module is loaded from the edited text), points the ``oracle`` package at
the copy in a fresh interpreter, and runs the pin files against it: at least one pin
must fail.  A control run of the unedited copy through the same path must pass.
The committed oracle is never modified.  CPU only.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C_SRC = os.path.join(ROOT, "oracle", "bsa_oracle.c")
PY_SRC = os.path.join(ROOT, "oracle", "bsa_bwd.py")
C_PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_coarse_pins.py"]
PY_PINS = ["tests/test_oracle_bwd_pins.py"]

# name: (text in the source, replacement, occurrences replaced)
C_MUTANTS = {
    "scale dropped": ("scores[nkeys++] = p->scale * dot;", "scores[nkeys++] = dot;", 1),
    "scale 1/D": ("return (float)(1.0 / sqrt((double)D));", "return (float)(1.0 / (double)D);", 1),
    "max subtracted with the wrong sign": ("expf(scores[key] - m)", "expf(m - scores[key])", 1),
    "max of the first key only": ("for (key = 0; key < nkeys; ++key)\n    if (scores[key] > m) m = scores[key];",
                                  "m = scores[0];", 1),
    "keys from the query tile": ("p->k + (bh * S + j * T + c) * D", "p->k + (bh * S + i * T + c) * D", 1),
    "values from K": ("p->v + (bh * S + j * T + c) * D", "p->k + (bh * S + j * T + c) * D", 1),
    "query head offset dropped": ("p->q + (bh * S + i * T + r) * D", "p->q + (i * T + r) * D", 1),
    "padding query rows computed": ("if (r >= p->vbs[i]) return; /* padding query row */", "", 1),
    "last valid key dropped": ("const int64_t vk = p->vbs[j];",
                               "const int64_t vk = p->vbs[j] > 1 ? p->vbs[j] - 1 : p->vbs[j];", 2),
    "last listed tile dropped": ("* p->MS;\n  const int64_t count = p->q2k_num[bh * p->NT + i];",
                                 "* p->MS;\n  const int64_t count = p->q2k_num[bh * p->NT + i] > 1 ? "
                                 "p->q2k_num[bh * p->NT + i] - 1 : p->q2k_num[bh * p->NT + i];", 1),
    "no normalisation": ("for (d = 0; d < D; ++d) dst[d] = acc[d] / l;", "for (d = 0; d < D; ++d) dst[d] = acc[d];", 1),
    "NaN sum tested with l > 0": ("if (l != 0.0f)\n    for (d = 0; d < D; ++d) dst[d]",
                                  "if (l > 0.0f)\n    for (d = 0; d < D; ++d) dst[d]", 1),
    "pool divided by the tile size": ("acc / (float)n : 0.0f", "acc / (float)T : 0.0f", 1),
    "ties to the higher index": ("return a->j < b->j ? -1 : (a->j > b->j ? 1 : 0);",
                                 "return a->j > b->j ? -1 : (a->j < b->j ? 1 : 0);", 1),
    "NaN logit ranked first": ("if (g != g) return -INFINITY;", "if (g != g) return INFINITY;", 1),
    "one tile too few kept": ("const int64_t k = topk < cand ? topk : cand;",
                              "const int64_t k = topk < cand ? (topk > 1 ? topk - 1 : topk) : cand;", 1),
    "logits against the pooled queries": ("km[(bh * NT + j) * D + d], dot)", "qm[(bh * NT + j) * D + d], dot)", 1),
    "coarse output without the scale": ("scale * g[j]", "g[j]", 3),
    "empty key tiles as candidates": ("keep[j] = 0;\n        if (vbs[j] <= 0) continue;", "keep[j] = 0;", 1),
    "kept tiles listed by rank": ("for (j = 0; j < NT; ++j)\n        if (vbs[j] > 0 && keep[j]) list[w++] = (int32_t)j;",
                                  "for (n = 0; n < k; ++n) list[w++] = (int32_t)order[n].j;", 1),
}

PY_MUTANTS = {
    "D_r dropped": ("ds = p * (dp - d_row)", "ds = p * dp", 1),
    "dq without the scale": ("dq[b, h, rows] = sc * (ds @ kk)", "dq[b, h, rows] = ds @ kk", 1),
    "dk from dO instead of q": ("sc * (ds.T @ qi)", "sc * (ds.T @ do)", 1),
    "dv from dS instead of P": ("np.add.at(dv[b, h], keys, p.T @ do)", "np.add.at(dv[b, h], keys, ds.T @ do)", 1),
    "dk overwritten, not accumulated": ("np.add.at(dk[b, h], keys, sc * (ds.T @ qi))",
                                        "dk[b, h][keys] = sc * (ds.T @ qi)", 1),
    "D_r over the wrong axis": ("d_row = (do * o).sum(axis=1, keepdims=True)",
                                "d_row = (do * o).sum(axis=0, keepdims=True)", 1),
    "lse in base 2": ("m + np.log(l)", "m + np.log2(l)", 1),
    "lse with the wrong sign": ("m + np.log(l)", "m - np.log(l)", 1),
}

C_BOOT = """
import os, sys
sys.path.insert(0, {root!r})
import oracle
oracle._SRC, oracle._LIB, oracle._lib = {src!r}, {lib!r}, None
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "--rootdir", {root!r}] + {pins!r}))
"""

PY_BOOT = """
import importlib.util, os, sys
sys.path.insert(0, {root!r})
import oracle
spec = importlib.util.spec_from_file_location("oracle_bwd_copy", {src!r})
mod = importlib.util.module_from_spec(spec)
spec.loader.exec_module(mod)
oracle.bsa_bwd, oracle.bwd, oracle.fwd64 = mod, mod.bwd, mod.fwd64
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "--rootdir", {root!r}] + {pins!r}))
"""


def _edit(text, old, new, count):
    assert text.count(old) == count, f"the oracle no longer holds {old!r} {count} time(s)"
    return text.replace(old, new)


def _run(boot, tmp_path):
    env = dict(os.environ)
    env.pop("PYTEST_ADDOPTS", None)
    return subprocess.run([sys.executable, "-c", boot], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=600)


def _c_copy(tmp_path, text):
    src = tmp_path / "bsa_oracle.c"
    src.write_text(text)
    lib = tmp_path / "liboracle.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                    "-pthread", str(src), "-o", str(lib), "-lm"], check=True)
    return C_BOOT.format(root=ROOT, src=str(src), lib=str(lib), pins=C_PINS)


def _py_copy(tmp_path, text):
    src = tmp_path / "bsa_bwd_copy.py"
    src.write_text(text)
    return PY_BOOT.format(root=ROOT, src=str(src), pins=PY_PINS)


def test_unedited_copies_pass_the_pins(tmp_path):
    (tmp_path / "c").mkdir()
    (tmp_path / "py").mkdir()
    for boot in (_c_copy(tmp_path / "c", open(C_SRC).read()), _py_copy(tmp_path / "py", open(PY_SRC).read())):
        res = _run(boot, tmp_path)
        assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_oracle_mistake_fails_a_pin(tmp_path, name):
    old, new, count = C_MUTANTS[name]
    res = _run(_c_copy(tmp_path, _edit(open(C_SRC).read(), old, new, count)), tmp_path)
    assert res.returncode == 1, f"no pin caught '{name}':\n{res.stdout[-2000:]}{res.stderr[-2000:]}"


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_backward_oracle_mistake_fails_a_pin(tmp_path, name):
    old, new, count = PY_MUTANTS[name]
    res = _run(_py_copy(tmp_path, _edit(open(PY_SRC).read(), old, new, count)), tmp_path)
    assert res.returncode == 1, f"no pin caught '{name}':\n{res.stdout[-2000:]}{res.stderr[-2000:]}"
