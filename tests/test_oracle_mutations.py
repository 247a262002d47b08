"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/oracle.c (a wrong bias or
exponent, a dropped term, a flipped tie rule, a transposed index, an off-by-one
window), builds that copy with gcc, and runs the pin suites against it in a fresh
process (CSA2_ORACLE_LIB points the oracle at the copy).  The pin suite must fail.
Runs on the CPU only; the mistakes never reach the committed oracle.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (label, text in oracle.c, replacement)
MUTATIONS = [
    ("e2m1 exponent bias", "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    ("e4m3 subnormal step", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("e4m3 exponent bias", "ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    ("e8m0 bias", "ldexp(1.0, (int)u - 127)", "ldexp(1.0, (int)u - 126)"),
    ("nv16 scale divides by 4, not 6", "fabs(6.0 * oracle_e4m3_value((uint8_t)b) - a)",
     "fabs(4.0 * oracle_e4m3_value((uint8_t)b) - a)"),
    ("nv16 scale ties to the odd byte", "(d == bestd && (b & 1) == 0 && (best & 1) == 1)", "(d == bestd)"),
    ("e2m1 ties to the higher magnitude", "(d == bestd && (i & 1) == 0 && (best & 1) == 1)", "(d == bestd)"),
    ("e2m1 drops the sign of small values", "return (uint8_t)((signbit(x) ? 8 : 0) | best);",
     "return (uint8_t)((best && signbit(x) ? 8 : 0) | best);"),
    ("mx32 exponent offset", "u = (e - 1) - 2 + 127;", "u = (e - 1) - 1 + 127;"),
    ("nibble order swapped", "codes[2 * k] | (codes[2 * k + 1] << 4)", "codes[2 * k + 1] | (codes[2 * k] << 4)"),
    ("score without ReLU", "float r = d > 0.0f ? d : 0.0f;", "float r = d;"),
    ("score heads reversed against weights", "acc = fmaf(wq[h], r, acc);", "acc = fmaf(wq[Hi - 1 - h], r, acc);"),
    ("score block scale off by 2", "- 254 - 2);", "- 254 - 1);"),
    ("score ignores the block table row", "block_table[(int64_t)row * max_pages + j / page_size]",
     "block_table[j / page_size]"),
    ("top-k ties to the higher index", "return (a->j < b->j) ? -1 : (a->j > b->j);",
     "return (a->j > b->j) ? -1 : (a->j < b->j);"),
    ("top-k pads with 0", "for (int64_t i = m; i < k; ++i) out[i] = -1;", "for (int64_t i = m; i < k; ++i) out[i] = 0;"),
    ("top-k output left in score order", "qsort(out, (size_t)m, sizeof(int32_t), by_index);", ";"),
    ("main-cache scale of the wrong block", "main_scales[s * 32 + c / NV_BLOCK]", "main_scales[s * 32 + c / MX_BLOCK]"),
    ("softmax scale dropped", "z[r] = scale * dot;", "z[r] = dot;"),
    ("lse without the max", "lse[h] = (float)(m + log(l));", "lse[h] = (float)log(l);"),
    ("decode window drops its first row", "for (int64_t r = win_first; r < win_end; ++r, ++nrows)",
     "for (int64_t r = win_first + 1; r < win_end; ++r, ++nrows)"),
    ("prefill window not causal", "int64_t first = i > swa_first_valid ? i : swa_first_valid;",
     "int64_t first = swa_first_valid;"),
    ("footprint ignores m", "if (mode[l] == 1) total += per_entry / (double)m[l];",
     "if (mode[l] == 1) total += per_entry;"),
    ("footprint counts reindex layers", "if (mode[l] == 1) total", "if (mode[l] == 1 || mode[l] == 2) total"),
    ("pool ranks blocks by their smallest member", "if (scores[(int64_t)q * ld + j] > m) m",
     "if (scores[(int64_t)q * ld + j] < m) m"),
    ("pool scores one entry past the visible end", "j >= n_visible[q]) continue;\n      int64_t s = slot_of",
     "j > n_visible[q]) continue;\n      int64_t s = slot_of"),
    ("pool top-k reports pool positions", "all[m].j = j;", "all[m].j = p;"),
    ("fp8 window scale twice too large", "while (ldexp(448.0, e) < amax) ++e;", "while (ldexp(224.0, e) < amax) ++e;"),
    ("fp8 window ties to the odd byte", "(d == bestd && !(b & 1) && (best & 1))", "(d == bestd)"),
    ("visibility from t // m", "out[i] = (int32_t)((t + 1) / m);", "out[i] = (int32_t)(t / m);"),
    ("visibility one entry early", "out[i] = (int32_t)((t + 1) / m);", "out[i] = (int32_t)((t + m) / m);"),
    ("fp8 window drops the sign", "(uint8_t)((signbit(v) ? 0x80 : 0) | e4m3_nearest(", "(uint8_t)((0) | e4m3_nearest("),
]


def _build_mutant(tmp, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found exactly once: {old!r}"
    path = os.path.join(tmp, "oracle.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmp, "liboracle_mutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared",
                    "-o", so, path, "-lm"], check=True)
    return so


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the mutants")
@pytest.mark.parametrize("label,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, label, old, new):
    so = _build_mutant(str(tmp_path), old, new)
    env = dict(os.environ, CSA2_ORACLE_LIB=so, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"),
                        os.path.join(HERE, "test_oracle_pool.py"), os.path.join(HERE, "test_oracle_fp8win.py"),
                        "-x", "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 1, f"mistake '{label}' was not caught by any pin:\n{r.stdout[-1500:]}"
