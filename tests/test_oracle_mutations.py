"""The oracle's pins catch plausible slips: each case below plants one slip
in a private copy of oracle/dsa_oracle.c (a dropped ReLU, a dropped head
weight, a slot off by one, ties broken the wrong way, wrong padding, an
unshifted softmax, an lse without its maximum, a swapped value column, a
missing softmax scale, the smallest scores kept), builds it, and runs the pin
suite (tests/test_oracle_pins.py) against that build, which must fail.
Runs on the CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dsa_oracle.c")

# (name, text in dsa_oracle.c, its replacement)
MUTATIONS = [
    ("dropped_relu", "if (relu && dot < 0.0) dot = 0.0;", ""),
    ("dropped_head_weight", "total += (double)w[(int64_t)i * H_idx + h] * dot;", "total += dot;"),
    ("slot_off_by_one", "return (int64_t)block * block_size + pos % block_size;",
     "return (int64_t)block * block_size + (pos + 1) % block_size;"),
    ("ties_to_higher_position", "return (x->pos > y->pos) - (x->pos < y->pos);",
     "return (x->pos < y->pos) - (x->pos > y->pos);"),
    ("padding_zero", "for (int64_t r = kept; r < K; ++r) row[r] = -1;",
     "for (int64_t r = kept; r < K; ++r) row[r] = 0;"),
    ("unshifted_softmax", "const double p = exp(logit[j] - m);", "const double p = exp(logit[j]);"),
    ("lse_without_max", "(float)(m + log(z))", "(float)(log(z))"),
    ("swapped_value_column", "acc[d] += p * bf16_value(vr[d]);",
     "acc[d] += p * bf16_value(vr[d ^ 1]);"),
    ("missing_scale", "logit[j] = sm_scale * dot;", "logit[j] = dot;"),
    ("smallest_kept", "if (x->score > y->score) return -1;\n  if (x->score < y->score) return 1;",
     "if (x->score > y->score) return 1;\n  if (x->score < y->score) return -1;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_slip(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site of {name} not found exactly once"
    mutant = tmp_path / "dsa_oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libdsa_oracle_mutant.so"
    r = subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutant),
                        "-o", str(lib), "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, DSA_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    assert r.returncode == 1, f"{name}: the pins did not catch the slip\n{r.stdout[-2000:]}"
