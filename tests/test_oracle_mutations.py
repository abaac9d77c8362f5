"""The oracle's pins catch plausible mistakes. Each case copies oracle/oracle.c, plants one
mistake in the copy (a dropped term, a wrong index, a missing normalisation, a reversed tie
order, a wrong rounding), builds it with the oracle's own flags and runs the pin tests
(tests/test_oracle_pins.py) against that build in a separate process: at least one pin must
fail. An unchanged copy must pass. CPU only; nothing here touches the GPU library."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (what the mistake is, text in oracle.c, replacement); the first occurrence is replaced.
MUTATIONS = [
    ("compress: bias dropped",
     "a[i] = (double)Z[(t0 + g * m + i) * d + c] + (double)B[(int64_t)i * d + c];",
     "a[i] = (double)Z[(t0 + g * m + i) * d + c];"),
    ("compress: token rows of a group reversed",
     "acc += w[i] * (double)X[(t0 + g * m + i) * d + c];",
     "acc += w[i] * (double)X[(t0 + g * m + (m - 1 - i)) * d + c];"),
    ("compress: weights not normalised",
     "w[i] = exp(a[i] - mx) / den;",
     "w[i] = exp(a[i] - mx);"),
    ("index score: ReLU dropped",
     "acc += (double)w[h] * (dot > 0.0 ? dot : 0.0);",
     "acc += (double)w[h] * dot;"),
    ("index score: head 0's weight for every head",
     "acc += (double)w[h] * (dot > 0.0 ? dot : 0.0);",
     "acc += (double)w[0] * (dot > 0.0 ? dot : 0.0);"),
    ("top-k: ties to the higher index",
     "return (a->j < b->j) ? -1 : (a->j > b->j);",
     "return (a->j > b->j) ? -1 : (a->j < b->j);"),
    ("top-k: indices left in score order",
     "qsort(out, (size_t)cnt, sizeof(int32_t), cmp_i32);",
     ";"),
    ("attention: logit scale dropped",
     "l[i] = scale * dot;",
     "l[i] = dot;"),
    ("attention: lse without the maximum",
     "double ls = (nkeys > 0) ? mx + log(sum) : -INFINITY;",
     "double ls = (nkeys > 0) ? log(sum) : -INFINITY;"),
    ("bf16 storage: truncation instead of round to nearest even",
     "double r = nearbyint(ldexp(mant, 8));",
     "double r = trunc(ldexp(mant, 8));"),
    ("E4M3 decode: exponent bias off by one",
     "else v = ldexp(1.0 + m / 8.0, e - 7);",
     "else v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("E4M3 encode: ties to the odd code",
     "if (err < best_err || (err == best_err && (c & 1) == 0)) { best = c; best_err = err; }",
     "if (err < best_err || (err == best_err && (c & 1) == 1)) { best = c; best_err = err; }"),
    ("E4M3 encode: no saturation above 448",
     "if (a > 448.0) best = 0x7E;",
     "if (a > 464.0) best = 0x7F;"),
    ("E4M3 quantisation: stored scale for a row maximum of 240 instead of 448",
     "const float s = (float)((double)amax / 448.0);",
     "const float s = (float)((double)amax / 240.0);"),
    ("E4M3 quantisation: row maximum mapped to 240 instead of 448",
     "float inv = (float)(448.0 / (double)amax);",
     "float inv = (float)(240.0 / (double)amax);"),
]


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.c"
    lib = tmp_path / f"lib{name}.so"
    src.write_text(text, encoding="utf-8")
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", str(src),
                    "-o", str(lib), "-lm"], check=True)
    return lib


def _pins(lib):
    env = dict(os.environ, CHS_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                           "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=300)


def test_unchanged_copy_passes_the_pins(tmp_path):
    r = _pins(_build(tmp_path, "same", open(SRC, encoding="utf-8").read()))
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("what,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, what, old, new):
    text = open(SRC, encoding="utf-8").read()
    assert old in text, f"the oracle no longer contains the line this case mutates: {old}"
    lib = _build(tmp_path, "mutant", text.replace(old, new, 1))
    r = _pins(lib)
    assert r.returncode != 0, f"no pin caught: {what}"
