"""Planted mistakes: each mutant is a copy of the oracle's C source with one
plausible slip (a dropped term, a wrong sign or index, a swapped operand, an
off-by-one).  The pin suite must fail on every one of them; a mutant that passes
would mean the pins leave that part of the oracle unchecked.  CPU only."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from oracle import ckv_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "score-drops-last-term": (
        "for (int i = 0; i < d; ++i)\n                dot = dot + widen(q",
        "for (int i = 0; i < d - 1; ++i)\n                dot = dot + widen(q"),
    "score-no-scale": ("out[c] = (float)(best * (double)scale);", "out[c] = (float)best;"),
    "score-last-head-not-max": ("if (dot > best)\n                best = dot;",
                                "best = dot;"),
    "score-transposed-centroid": ("q_dtype) * (double)cent[(long)c * d + i]",
                                  "q_dtype) * (double)cent[(long)i * C + c]"),
    "select-strict-budget": ("total + size[it[k].c] <= (long)budget",
                             "total + size[it[k].c] < (long)budget"),
    "select-tie-high-id-first": ("return (x->c < y->c) ? -1 : (x->c > y->c);",
                                 "return (x->c > y->c) ? -1 : (x->c < y->c);"),
    "select-ascending-score": ("if (x->s > y->s) return -1;\n    if (x->s < y->s) return 1;",
                               "if (x->s < y->s) return -1;\n    if (x->s > y->s) return 1;"),
    "select-skips-misfits": ("while (k < m && total + size[it[k].c] <= (long)budget) {\n"
                             "        total += size[it[k].c];\n"
                             "        sel[it[k].c] = 1;\n        ++k;\n    }",
                             "for (int t = 0; t < m; ++t) {\n"
                             "        if (total + size[it[t].c] > (long)budget) continue;\n"
                             "        total += size[it[t].c];\n"
                             "        sel[it[t].c] = 1;\n        ++k;\n    }"),
    "list-drops-a-sink": ("for (int j = 0; j < ns; ++j)\n        idx[len++] = j;",
                          "for (int j = 1; j < ns; ++j)\n        idx[len++] = j;"),
    "list-drops-last-member": ("for (int j = 0; j < size[c]; ++j)\n            idx[len++]",
                               "for (int j = 0; j < size[c] - 1; ++j)\n            idx[len++]"),
    "attend-no-scale": ("z[t] = dot * (double)scale;", "z[t] = dot;"),
    "attend-no-normalise": ("out[i] = out[i] / denom;", "out[i] = out[i];"),
    "attend-values-from-keys": ("widen(V, row + i, kv_dtype)", "widen(K, row + i, kv_dtype)"),
    "update-farthest": ("if (dist < best_d || (dist == best_d && c < best))",
                        "if (best < 0 || dist > best_d || (dist == best_d && c < best))"),
    "update-tie-high-id": ("(dist == best_d && c < best)", "(dist == best_d && c > best)"),
    "update-wrong-count": ("double cnt = (double)size[best];",
                           "double cnt = (double)size[best] + 1.0;"),
    "update-wrong-position": ("members[start[best] + size[best]] = n;",
                              "members[start[best] + size[best]] = n - 1;"),
    "update-no-square": ("dist = dist + diff * diff;", "dist = dist + diff;"),
    "rebuild-skips-first-member": ("for (int m = 0; m < size[c]; ++m)\n                s = s + widen(K",
                                   "for (int m = 1; m < size[c]; ++m)\n                s = s + widen(K"),
    "rebuild-wrong-count": ("(float)(s / (double)size[c])", "(float)(s / (double)(size[c] + 1))"),
    "edges-self-link": ("int cnt = i - lo > 0 ? i - lo : 0;\n        if (cnt == 0)\n"
                        "            continue;\n"
                        "        double *z = (double *)malloc(sizeof(double) * (size_t)cnt);\n"
                        "        for (int j = lo; j < i; ++j) {",
                        "int cnt = i + 1 - lo > 0 ? i + 1 - lo : 0;\n        if (cnt == 0)\n"
                        "            continue;\n"
                        "        double *z = (double *)malloc(sizeof(double) * (size_t)cnt);\n"
                        "        for (int j = lo; j <= i; ++j) {"),
    "edge-scores-min-of-heads": ("best = dot > best ? dot : best;",
                                 "best = (h == 0 || dot < best) ? dot : best;"),
    "layer-update-first-slice-only": (
        "for (long e = 0; e < row; ++e) {\n            const double gap",
        "for (long e = 0; e < d; ++e) {\n            const double gap"),
    "layer-update-centroid-stride": (
        "const double gap = widen(k_new, e, dtype) - (double)cent[(long)c * row + e];",
        "const double gap = widen(k_new, e, dtype) - (double)cent[(long)c * d + e];"),
    "pairs-higher-first": ("out[2 * slot] = y < cnt ? keys[x] : -1;\n"
                           "                out[2 * slot + 1] = y < cnt ? keys[y] : -1;",
                           "out[2 * slot] = y < cnt ? keys[y] : -1;\n"
                           "                out[2 * slot + 1] = y < cnt ? keys[x] : -1;"),
    "pairs-unsorted": ("while (at > 0 && keys[at - 1] > j) {",
                       "while (at > 0 && keys[at - 1] > j && 0) {"),
    "pairs-padding-on-lower-key": ("out[2 * slot] = y < cnt ? keys[x] : -1;\n"
                                   "                out[2 * slot + 1] = y < cnt ? keys[y] : -1;",
                                   "out[2 * slot] = x < cnt ? keys[x] : -1;\n"
                                   "                out[2 * slot + 1] = x < cnt ? keys[y] : -1;"),
    "pairs-skip-first-key": ("for (int t = 0; t < topk; ++t) {\n            int32_t j = idx",
                             "for (int t = 1; t < topk; ++t) {\n            int32_t j = idx"),
    "edges-include-sinks": ("int lo = S;\n        int cnt", "int lo = 0;\n        int cnt"),
    "edges-tie-high-position": ("(arg < 0 || z[j] > z[arg])", "(arg < 0 || z[j] >= z[arg])"),
    "drift-not-relative": ("double r = den > 0.0 ? sqrt(num) / sqrt(den) : sqrt(num);",
                           "double r = sqrt(num);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(O.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.check_call(["gcc", *O.CFLAGS, str(mut), "-o", str(so), "-lm"])
    env = dict(os.environ, CKV_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
