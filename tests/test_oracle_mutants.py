"""Planted mistakes in the oracle, on the CPU. Each mutant is rope_oracle.c
with one plausible slip: a sign, a partner index, the lane of a table read,
the backward's sign, the broadcast index, the slice start, the row order, a
rounding rule, the fp16 range, the precision of the products, in the tables
built from positions the angle's precision, the rounding and the layout,
and in the rotary coefficient the part width, the sign, the table layout and
the check of the coefficient. Every mutant must fail at least one pin of the oracle's own test
files (closed forms, brute force, library conversions, the golden cases); a
mutant that passed them all would be a mistake the pins cannot see.

The pins run in a subprocess against the mutant's library (ROPE_ORACLE_LIB);
a mutant that crashes its process counts as caught."""
import concurrent.futures
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_golden.py", "test_oracle_pins.py", "test_oracle_pos.py", "test_oracle_coeff.py",
              "test_oracle_converters.py")]

# (name, text in rope_oracle.c, replacement)
MUTANTS = [
    ("interleave sign on the odd lane", "return (j % 2 == 0) ? -1 : 1;", "return (j % 2 == 0) ? 1 : -1;"),
    ("rotate_half sign on the second half", "return j < L / 2 ? -1 : 1;", "return j < L / 2 ? 1 : -1;"),
    ("interleave partner is the next lane", "return j ^ 1;", "return (j + 1) % L;"),
    ("rotate_half partner mirrored", "return j < L / 2 ? j + L / 2 : j - L / 2;", "return L - 1 - j;"),
    ("forward sine at the partner's lane", "direction == ORACLE_FWD ? j : pj);", "direction == ORACLE_FWD ? pj : pj);"),
    ("backward sine at the lane itself", "direction == ORACLE_FWD ? j : pj);", "direction == ORACLE_FWD ? j : j);"),
    ("backward sign not flipped", "const int sign = direction == ORACLE_FWD ? sg : -sg;", "const int sign = sg;"),
    ("cosine at the partner's lane", "table_index(r1_shape, r1_strides, b, s, n, j);",
     "table_index(r1_shape, r1_strides, b, s, n, partner(mode, j, L));"),
    ("b and s swapped in the table index", "int64_t idx[4] = { b, s, n, j };", "int64_t idx[4] = { s, b, n, j };"),
    ("head index ignored by the table", "int64_t idx[4] = { b, s, n, j };", "int64_t idx[4] = { b, s, 0, j };"),
    ("slice start dropped", "const int64_t rowbase = r * D + start;", "const int64_t rowbase = r * D;"),
    ("heads and positions swapped in the row order", "const int64_t n = flat % N;\n        const int64_t s = (flat / N) % S;",
     "const int64_t s = flat % S;\n        const int64_t n = (flat / S) % N;"),
    ("bf16 narrowing truncates", "q = round_nearest_even(q, u & 0xffffu, 16);", "(void)0;"),
    ("ties rounded away from zero", "if (rem > half || (rem == half && (q & 1u)))", "if (rem >= half)"),
    ("fp16 subnormals flushed", "if (shift > 25)", "if (shift > 13)"),
    ("fp16 overflow saturates", "return (uint16_t)(sign | 0x7c00u);                  /* >= 2^16: overflow */",
     "return (uint16_t)(sign | 0x7bffu);"),
    ("16-bit products kept exact (fused)", "float a = xs[j] * c;                 /* fp32 product */",
     "double a = (double)xs[j] * (double)c;"),
    ("fp32 data computed in fp32", "double a = (double)xs[j] * (double)c;\n                double t = (double)sign * (double)xs[pj] * (double)sn;",
     "float a = xs[j] * c;\n                float t = (float)sign * xs[pj] * sn;"),
    ("bf16 NaN not kept quiet", "return (uint16_t)((u >> 16) | 0x40u);", "return (uint16_t)(u >> 16);"),
    ("position tables rounded through fp32", "if (dtype == ORACLE_F32) return (float)v;", "if (1) return (float)v;"),
    ("position angle in single precision", "const double theta = p * inv_freq[i];",
     "const double theta = (double)((float)p * (float)inv_freq[i]);"),
    ("rotate_half position table laid out as interleave", "int64_t j0 = mode == ORACLE_INTERLEAVE ? 2 * i : i;",
     "int64_t j0 = 2 * i;"),
    ("one-step rounding ties away from zero", "const double r = ldexp(rint(ldexp(v, -q)), q);",
     "const double r = ldexp(round(ldexp(v, -q)), q);"),
    ("coefficient parts half as wide in the partner", "const int64_t H = L / mode;\n        return (j / H) % 2 == 0 ? j + H : j - H;",
     "const int64_t H = L / (2 * mode);\n        return (j / H) % 2 == 0 ? j + H : j - H;"),
    ("coefficient sign on the odd part", "return (j / H) % 2 == 0 ? -1 : 1;", "return (j / H) % 2 == 0 ? 1 : -1;"),
    ("coefficient pair as rotate_half in the position table", "j0 = (i / H) * 2 * H + i % H;", "j0 = i;"),
    ("odd coefficient accepted", "return mode >= 2 && mode % 2 == 0 && (L == 0 || L % mode == 0);",
     "return mode >= 2 && (L == 0 || L % mode == 0);"),
]


def build_mutant(name, old, new, workdir):
    src = open(os.path.join(ROOT, "oracle", "rope_oracle.c"), encoding="utf-8").read()
    assert src.count(old) == 1, f"mutant '{name}': the text to replace must occur once"
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    c_path = os.path.join(workdir, f"{tag}.c")
    so_path = os.path.join(workdir, f"{tag}.so")
    with open(c_path, "w", encoding="utf-8") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc"] + oracle.GCC_FLAGS + [c_path, "-o", so_path, "-lm"], check=True, capture_output=True)
    return so_path


def run_pins(lib_path):
    env = dict(os.environ, ROPE_ORACLE_LIB=lib_path)
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_FILES],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return res.returncode, res.stdout[-2000:]


def test_the_unmutated_oracle_passes_the_pins_through_the_override(tmp_path):
    """The same subprocess route with the real oracle source passes, so a
    failing mutant fails for its mutation and not for the route."""
    so = build_mutant("unmutated", "#include <math.h>", "#include <math.h>", str(tmp_path))
    code, out = run_pins(so)
    assert code == 0, out


def test_every_planted_mistake_fails_a_pin(tmp_path):
    libs = {name: build_mutant(name, old, new, str(tmp_path)) for name, old, new in MUTANTS}
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        results = dict(zip(libs, pool.map(run_pins, libs.values())))
    # 1: a pin failed; a negative code: the mutant crashed the run (also caught).
    # 2-5 would be pytest itself going wrong (interrupted, internal, usage, nothing collected).
    broken = {n: r for n, r in results.items() if r[0] in (2, 3, 4, 5)}
    assert not broken, {n: r[1] for n, r in broken.items()}
    missed = [n for n, r in results.items() if r[0] == 0]
    assert not missed, f"mistakes no pin catches: {missed}"
