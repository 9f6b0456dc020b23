"""The pins have teeth: copies of oracle/attn_ref.c with one plausible
mistake planted each (a dropped term, a wrong sign, index or operand, an
off-by-one mask, a wrong decode constant, a wrong head grouping) are built
on the CPU, and the oracle pin suite (tests/test_oracle_pins.py) must fail
against every one of them while passing against the unaltered copy built
the same way. The mistakes are planted in the oracle only; nothing here
touches the GPU path."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attn_ref.c")

# (name, exact source text, replacement); every replacement keeps all
# accesses in bounds.
MUTANTS = [
    ("forward: scale dropped",
     "s_row[j] = jb->scale * dot;", "s_row[j] = dot;"),
    ("forward: causal mask admits the next key",
     "const int64_t n_vis = jb->causal ? i + 1 : N;",
     "const int64_t n_vis = jb->causal ? (i + 1 < N ? i + 2 : N) : N;"),
    ("forward: K row of the query, not of the key",
     "dot += qrow[c] * decode_one(jb->k, kv_slice + j * d + c, jb->dtype);",
     "dot += qrow[c] * decode_one(jb->k, kv_slice + i * d + c, jb->dtype);"),
    ("forward: V row of the query, not of the key",
     "o[c] += p * decode_one(jb->v, kv_slice + j * d + c, jb->dtype);",
     "o[c] += p * decode_one(jb->v, kv_slice + i * d + c, jb->dtype);"),
    ("forward: softmax without the max shift (overflows for large scores)",
     "s_row[j] = exp(s_row[j] - m);   /* e_ij, overwrites s_ij */",
     "s_row[j] = exp(s_row[j]); m = 0.0;"),
    ("forward: lse in base 2",
     "jb->lse[t] = m + log(l);", "jb->lse[t] = m + log2(l);"),
    ("forward: probabilities not normalised",
     "s_row[j] = s_row[j] / l;        /* p_ij */", "s_row[j] = s_row[j];"),
    ("GQA: query head h reads K/V head h mod H_kv",
     "h / (jb->H / jb->H_kv)", "h % jb->H_kv"),
    ("decode: bfloat16 shifted by 15",
     "uint32_t bits = (uint32_t)h << 16;", "uint32_t bits = (uint32_t)h << 15;"),
    ("decode: binary16 exponent bias off by one",
     "v = ldexp((double)(1024 + m), e - 25);", "v = ldexp((double)(1024 + m), e - 24);"),
    ("backward: sign of D in dS",
     "ds[j] = p[j] * (dp - D);", "ds[j] = p[j] * (dp + D);"),
    ("backward: dK without the scale",
     "const double a = w->scale * ds[j], pj = p[j];", "const double a = ds[j], pj = p[j];"),
    ("backward: dV from q instead of dO",
     "dv[c] += pj * grow[c];", "dv[c] += pj * qrow[c];"),
    ("backward: dQ without the scale",
     "        dq[c] *= w->scale;\n    if (w->eq) {", "        dq[c] *= 1.0;\n    if (w->eq) {"),
    # The backward error scales set the backward parity tolerance; an
    # inflated one would loosen it silently.
    ("backward error scale: eq doubled",
     "eq[c] *= w->scale;", "eq[c] *= 2.0 * w->scale;"),
    ("backward error scale: ek doubled",
     "const double b = w->scale * wt[j];", "const double b = 2.0 * w->scale * wt[j];"),
    ("backward error scale: ev doubled",
     "ev[c] += pj * ga[c];", "ev[c] += 2.0 * pj * ga[c];"),
    ("backward error scale: zq doubled",
     "zq[c] *= w->scale;", "zq[c] *= 2.0 * w->scale;"),
    ("backward error scale: zk with a doubled rounding term",
     "const double z = w->scale * (1.0 + pj * gs);", "const double z = w->scale * (2.0 + pj * gs);"),
    ("backward error scale: o's rounding counted twice in w",
     "wt[j] = fabs(ds[j]) + p[j] * A;", "wt[j] = fabs(ds[j]) + 2.0 * p[j] * A;"),
    ("backward error scale: eq over signed k",
     "eq[c] += wt[j] * w->ka[j * d + c];", "eq[c] += wt[j] * kd[j * d + c];"),
    ("backward error scale: o's rounding dropped from w",
     "A += fabs(grow[c] * orow[c]);", "A += 0.0;"),
]


def _build(src_text, out_dir, name):
    c_path = os.path.join(out_dir, name + ".c")
    so_path = os.path.join(out_dir, name + ".so")
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                    "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"), c_path, "-o",
                    so_path, "-lm"], check=True)
    return so_path


def _pins_pass(so_path):
    env = dict(os.environ, ATTN_ORACLE_LIB=so_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests",
                        "test_oracle_pins.py"), "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode == 0, r.stdout[-400:]


def test_pins_catch_every_planted_mistake(tmp_path):
    src = open(SRC).read().replace('#include "../include/attn_ref.h"',
                                   '#include "' + os.path.join(ROOT, "include", "attn_ref.h") + '"')
    builds = [("control", _build(src, str(tmp_path), "control"))]
    for k, (name, old, new) in enumerate(MUTANTS):
        assert src.count(old) == 1, f"mutant '{name}': source text not found exactly once"
        builds.append((name, _build(src.replace(old, new), str(tmp_path), f"mutant{k}")))
    with ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(lambda b: (b[0],) + _pins_pass(b[1]), builds))
    control = results[0]
    assert control[1], "the unaltered oracle must pass its pins: " + control[2]
    survivors = [name for name, ok, _ in results[1:] if ok]
    assert not survivors, f"planted mistakes the pins did not catch: {survivors}"
