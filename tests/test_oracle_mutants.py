"""Plant plausible slips in a copy of the oracle and check that the pins catch each.

Every mutant is a one-place textual change of ``oracle/hla2_oracle.c`` built into
a temporary library (on the CPU); the condensed pin set below must flag it.  The
unmodified source must pass the same set, so the pins are not trivially failing.
"""
import os
import subprocess

import numpy as np
import pytest

from oracle import oracle as O
from tests.test_oracle_pins import matrix_form, rel

SRC = os.path.join(os.path.dirname(O.__file__), "hla2_oracle.c")

MUTANTS = {
    "cross-term sign in G update": (
        "G[(long)a * dv + c] = g2 * G[(long)a * dv + c] + gamma * k[a] * kC[c];",
        "G[(long)a * dv + c] = g2 * G[(long)a * dv + c] - gamma * k[a] * kC[c];"),
    "G decays by gamma instead of gamma^2": ("double g2 = gamma * gamma;", "double g2 = gamma;"),
    "readout adds G": ("s += p[a] * C[(long)a * dv + c] - q[a] * G[(long)a * dv + c];",
                       "s += p[a] * C[(long)a * dv + c] + q[a] * G[(long)a * dv + c];"),
    "cross term built from q instead of k": ("kC[c] += k[a] * C[(long)a * dv + c];",
                                             "kC[c] += q[a] * C[(long)a * dv + c];"),
    "h cross term from q": ("km += k[a] * m[a];", "km += q[a] * m[a];"),
    "key moment k q^T": ("S[(long)a * d + b] = gamma * S[(long)a * d + b] + k[a] * k[b];",
                         "S[(long)a * d + b] = gamma * S[(long)a * d + b] + k[a] * q[b];"),
    "accumulator k v^T": ("C[(long)a * dv + c] = gamma * C[(long)a * dv + c] + q[a] * v[c];",
                          "C[(long)a * dv + c] = gamma * C[(long)a * dv + c] + k[a] * v[c];"),
    "h lacks the gamma factor": ("h[a] = g2 * h[a] + gamma * k[a] * km;", "h[a] = g2 * h[a] + k[a] * km;"),
    "den ignores h": ("sd += p[a] * m[a] - q[a] * h[a];", "sd += p[a] * m[a];"),
    "combine cross term S_A C_B": ("for (b = 0; b < d; ++b) s += SB[(long)a * d + b] * CA[(long)b * dv + c];",
                                   "for (b = 0; b < d; ++b) s += SA[(long)a * d + b] * CB[(long)b * dv + c];"),
    "combine G_A decays once": ("Go[(long)a * dv + c] = GB * GB * GgA[(long)a * dv + c]",
                                "Go[(long)a * dv + c] = GB * GgA[(long)a * dv + c]"),
    "combine h cross term sign": ("ho[a] = GB * GB * hA[a] + hB[a] + GB * s;",
                                  "ho[a] = GB * GB * hA[a] + hB[a] - GB * s;"),
    "segment G includes the diagonal": ("for (j = 0; j < i; ++j) {", "for (j = 0; j <= i; ++j) {"),
    "chunk carry decays once": ("double carry = pow(gamma, 2.0 * (tau + 1));",
                                "double carry = pow(gamma, (double)(tau + 1));"),
    "brute force unmasked inner sum": ("for (i = 0; i <= j; ++i)\n        w +=", "for (i = 0; i <= t; ++i)\n        w +="),
    "down-sweep combines in the wrong order": ("hla2_oracle_combine(d, dv, xr, left, tmp);",
                                               "hla2_oracle_combine(d, dv, left, xr, tmp);"),
    "chunk outputs skip the S0 term": ("double w = pow(gamma, (double)(tau - j)) * (pow(gamma, (double)(tau + 1)) * qsq + inner);",
                                       "double w = pow(gamma, (double)(tau - j)) * inner;"),
}


def pin_failures(lib):
    """Condensed pins; returns the names of the ones that fail."""
    bad = []
    r = np.random.default_rng(101)
    n, d, dv = 37, 5, 3
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))
    for g in (1.0, 0.9):
        rn, rd = matrix_form(q, k, v, g)
        num, den, st = O.serial(q, k, v, g, lib=lib)
        if rel(num, rn) > 1e-12 or rel(den, rd) > 1e-12:
            bad.append("serial vs matrix form, gamma=%g" % g)
        bn, bd = O.bruteforce(q, k, v, g, lib=lib)
        if rel(bn, rn) > 1e-12 or rel(bd, rd) > 1e-12:
            bad.append("bruteforce vs matrix form, gamma=%g" % g)
        for chunk in (4, 16):
            cn, cd, cst = O.chunked(q, k, v, g, chunk=chunk, lib=lib)
            if rel(cn, num) > 1e-12 or rel(cd, den) > 1e-12 or rel(cst, st) > 1e-12:
                bad.append("chunked vs serial, gamma=%g chunk=%d" % (g, chunk))
        whole = O.segment_summary(q, k, v, g, lib=lib)
        a = O.segment_summary(q[:15], k[:15], v[:15], g, lib=lib)
        b = O.segment_summary(q[15:], k[15:], v[15:], g, lib=lib)
        if rel(O.combine(a, b, d, dv, lib=lib), whole) > 1e-12:
            bad.append("concatenation, gamma=%g" % g)
    one = np.ones((4, 1))
    num, den, _ = O.serial(one, one, one, 0.5, lib=lib)
    if not (np.array_equal(num[:, 0], [1.0, 1.75, 2.1875, 2.421875]) and np.array_equal(den, num[:, 0])):
        bad.append("closed form gamma=1/2")
    return bad


def _build(tmp_path, text, name):
    src = tmp_path / (name + ".c")
    lib = tmp_path / ("lib" + name + ".so")
    src.write_text(text)
    subprocess.run(["gcc", "-std=c99", "-O1", "-ffp-contract=off", "-fPIC", "-shared", str(src), "-o", str(lib),
                    "-lm"], check=True)
    return O._load(str(lib))


def test_unmodified_oracle_passes_condensed_pins(tmp_path):
    lib = _build(tmp_path, open(SRC).read(), "clean")
    assert pin_failures(lib) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site moved: %r" % old
    lib = _build(tmp_path, text.replace(old, new), "mut")
    assert pin_failures(lib), "planted slip not caught: " + name
