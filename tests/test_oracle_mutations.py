"""The oracle's pins catch plausible slips: each case below plants one slip
in a private copy of the oracle's sources -- in the DSA part (a dropped ReLU,
a dropped head weight, a slot off by one, ties broken the wrong way, wrong
padding, an unshifted softmax, an lse without its maximum, a swapped value
column, a missing softmax scale, the smallest scores kept) or the MoE expert
part (a wrong FP4 exponent bias or subnormal, a wrong E8M0 bias, E4M3 ties
rounded down, overflow to NaN, swapped nibbles, a swapped scale block, a
reversed reduction, the expert id ignored) -- builds it, and runs the matching
pin suite against that build, which must fail.  Runs on the CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dsa_oracle.c")

# (name, oracle source file, text in it, its replacement)
DSA = "dsa_oracle.c"
MOE = "moe_oracle.c"
MUTATIONS = [
    ("dropped_relu", DSA, "if (relu && dot < 0.0) dot = 0.0;", ""),
    ("dropped_head_weight", DSA, "total += (double)w[(int64_t)i * H_idx + h] * dot;",
     "total += dot;"),
    ("slot_off_by_one", DSA, "return (int64_t)block * block_size + pos % block_size;",
     "return (int64_t)block * block_size + (pos + 1) % block_size;"),
    ("ties_to_higher_position", DSA, "return (x->pos > y->pos) - (x->pos < y->pos);",
     "return (x->pos < y->pos) - (x->pos > y->pos);"),
    ("padding_zero", DSA, "for (int64_t r = kept; r < K; ++r) row[r] = -1;",
     "for (int64_t r = kept; r < K; ++r) row[r] = 0;"),
    ("unshifted_softmax", DSA, "const double p = exp(logit[j] - m);",
     "const double p = exp(logit[j]);"),
    ("lse_without_max", DSA, "(float)(m + log(z))", "(float)(log(z))"),
    ("swapped_value_column", DSA, "acc[d] += p * bf16_value(vr[d]);",
     "acc[d] += p * bf16_value(vr[d ^ 1]);"),
    ("missing_scale", DSA, "logit[j] = sm_scale * dot;", "logit[j] = dot;"),
    ("smallest_kept", DSA,
     "if (x->score > y->score) return -1;\n  if (x->score < y->score) return 1;",
     "if (x->score > y->score) return 1;\n  if (x->score < y->score) return -1;"),
    ("fp4_exponent_bias", MOE, "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    ("fp4_subnormal", MOE, "e == 0 ? 0.5 * m :", "e == 0 ? 1.0 * m :"),
    ("e8m0_bias", MOE, "ldexp(1.0, (int)code - 127)", "ldexp(1.0, (int)code - 128)"),
    ("e4m3_ties_down", MOE, "else pick = (best & 1) ? (uint8_t)(best + 1) : best;",
     "else pick = best;"),
    ("e4m3_overflow_nan", MOE, "if (a >= 448.0) return sign | 0x7e;",
     "if (a >= 448.0) return sign | 0x7f;"),
    ("nibble_order", MOE, "(k & 1) ? (byte >> 4) : (byte & 15)",
     "(k & 1) ? (byte & 15) : (byte >> 4)"),
    ("scale_block_swapped", MOE, "table[s[n * (K / 32) + k / 32]][code]",
     "table[s[n * (K / 32) + ((k / 32) ^ 1)]][code]"),
    ("gemm_k_reversed", MOE, "e4m3[w8[n * K + k]]", "e4m3[w8[n * K + (K - 1 - k)]]"),
    ("expert_id_ignored", MOE, "oracle_mxfp4_to_fp8(codes, scales, expert_ids + i, 1, N, K, w8);",
     "{ const int32_t first = expert_ids[0]; oracle_mxfp4_to_fp8(codes, scales, &first, 1, N, K, w8); }"),
]
PINS = {DSA: "test_oracle_pins.py", MOE: "test_moe_oracle_pins.py"}


@pytest.mark.parametrize("name,src_file,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_slip(tmp_path, name, src_file, old, new):
    sources = {f: open(os.path.join(ROOT, "oracle", f)).read() for f in (DSA, MOE)}
    assert sources[src_file].count(old) == 1, f"mutation site of {name} not found exactly once"
    sources[src_file] = sources[src_file].replace(old, new)
    paths = []
    for f, text in sources.items():
        pth = tmp_path / f
        pth.write_text(text)
        paths.append(str(pth))
    lib = tmp_path / "libdsa_oracle_mutant.so"
    r = subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *paths,
                        "-o", str(lib), "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, DSA_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", PINS[src_file])],
                       capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    assert r.returncode == 1, f"{name}: the pins did not catch the slip\n{r.stdout[-2000:]}"
