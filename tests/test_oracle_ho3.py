"""Pins of the oracle's third-order path against things other than itself, and
planted slips that the pins must catch.

Pins:
  * the masked matrix form (L o D_{g^2} o (A_g A^T)) (A_g V) with A = L o (Q K^T),
    A_g = D_g o A (numpy matmuls);
  * closed forms for all-ones inputs: sum_{l<=t} (l+1)^2 without decay, exact
    binary fractions with decay 1/2 (summed with Python fractions);
  * exact integer arithmetic for entries in {-1, 0, 1};
  * strict causality;
  * folding a segment's summary into the incoming state equals running the
    recurrence over the segment (the chunk-parallel form).
"""
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "hla2_oracle.c")


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def matrix_form(q, k, v, gamma):
    n = q.shape[0]
    t = np.arange(n)
    low = t[:, None] >= t[None, :]

    def D(p):
        return np.where(low, p ** np.where(low, t[:, None] - t[None, :], 0), 0.0)

    A = np.where(low, q @ k.T, 0.0)
    Ag = D(gamma) * A
    M = D(gamma * gamma) * np.where(low, Ag @ A.T, 0.0)
    return M @ (Ag @ v), M @ (Ag @ np.ones(n))


def den_column_norms(q, k, gamma):
    """|w_t| from the matrix form: w_t = sum_{l<=t} g^{3(t-l)} (q_l . m_l) z_l with z_l = S_l q_l, i.e. the
    rows of (L o D_{g^3}) diag(A_g 1) (A_g K) (so den = Q w row by row)."""
    n = q.shape[0]
    t = np.arange(n)
    low = t[:, None] >= t[None, :]

    def D(p):
        return np.where(low, p ** np.where(low, t[:, None] - t[None, :], 0), 0.0)

    Ag = D(gamma) * (q @ k.T)
    Wd = D(gamma ** 3) @ ((Ag @ np.ones(n))[:, None] * (Ag @ k))
    return np.linalg.norm(Wd, axis=1)


def closed_form(n, gamma):
    g = Fraction(gamma)
    return [float(sum(g ** (3 * t - j - l - i) for l in range(t + 1) for j in range(l + 1) for i in range(l + 1)))
            for t in range(n)]


def draw(seed, n, d, dv, scale=0.5):
    r = np.random.default_rng(seed)
    return (scale * r.standard_normal((n, d)), scale * r.standard_normal((n, d)),
            scale * r.standard_normal((n, dv)))


def pin_failures(lib):
    bad = []
    d, dv = 5, 3
    for gamma in (1.0, 0.9, 0.5):
        q, k, v = draw(5, 27, d, dv)
        rn, rd = matrix_form(q, k, v, gamma)
        num, den, st = O.ho3_serial(q, k, v, gamma, lib=lib)
        if rel(num, rn) > 1e-11 or rel(den, rd) > 1e-11:
            bad.append("serial vs matrix form gamma=%g" % gamma)
        un_num, un_den, un, _ = O.ho3_serial_unorm(q, k, v, gamma, lib=lib)
        if rel(un, den_column_norms(q, k, gamma)) > 1e-11 or not np.array_equal(un_num, num) or \
                not np.array_equal(un_den, den):
            bad.append("den-column norms vs matrix form gamma=%g" % gamma)
        bn, bd = O.ho3_bruteforce(q[:12], k[:12], v[:12], gamma, lib=lib)
        if rel(bn, rn[:12]) > 1e-11 or rel(bd, rd[:12]) > 1e-11:
            bad.append("bruteforce vs matrix form gamma=%g" % gamma)
        _, _, st1 = O.ho3_serial(q[:10], k[:10], v[:10], gamma, lib=lib)
        folded = O.ho3_apply(O.ho3_summary(q[10:], k[10:], v[10:], gamma, lib=lib), st1, d, dv, lib=lib)
        if rel(folded, st) > 1e-12:
            bad.append("fold vs serial gamma=%g" % gamma)
        zero = np.zeros_like(st)
        if rel(O.ho3_apply(O.ho3_summary(q, k, v, gamma, lib=lib), zero, d, dv, lib=lib), st) > 1e-12:
            bad.append("summary state vs serial gamma=%g" % gamma)
    one = np.ones((4, 1))
    num, den, _ = O.ho3_serial(one, one, one, 0.5, lib=lib)
    if not (np.array_equal(num[:, 0], closed_form(4, 0.5)) and np.array_equal(den, num[:, 0])):
        bad.append("closed form gamma=1/2")
    return bad


@pytest.mark.parametrize("n,d,dv,gamma", [(1, 3, 2, 1.0), (2, 1, 1, 0.5), (40, 8, 5, 1.0), (65, 4, 7, 0.95),
                                          (100, 16, 16, 0.99)])
def test_serial_equals_matrix_form(n, d, dv, gamma):
    q, k, v = draw(n + d, n, d, dv)
    rn, rd = matrix_form(q, k, v, gamma)
    num, den, _ = O.ho3_serial(q, k, v, gamma)
    assert rel(num, rn) < 1e-11 and rel(den, rd) < 1e-11


@pytest.mark.parametrize("gamma", [1.0, 0.8])
def test_bruteforce_equals_matrix_form(gamma):
    q, k, v = draw(3, 15, 4, 3)
    rn, rd = matrix_form(q, k, v, gamma)
    bn, bd = O.ho3_bruteforce(q, k, v, gamma)
    assert rel(bn, rn) < 1e-12 and rel(bd, rd) < 1e-12


def test_closed_forms_all_ones():
    n = 10
    one = np.ones((n, 1))
    num, den, _ = O.ho3_serial(one, one, one, 1.0)
    t = np.arange(n, dtype=np.float64)
    assert np.array_equal(num[:, 0], (t + 1) * (t + 2) * (2 * t + 3) / 6) and np.array_equal(den, num[:, 0])
    num, _, _ = O.ho3_serial(one[:6], one[:6], one[:6], 0.5)
    assert np.array_equal(num[:, 0], closed_form(6, 0.5))


def test_differs_from_second_order_and_ahla():
    q, k, v = draw(8, 30, 4, 3)
    a, _, _ = O.ho3_serial(q, k, v, 1.0)
    assert rel(a, O.serial(q, k, v, 1.0)[0]) > 0.1 and rel(a, O.ahla_serial(q, k, v, 1.0)[0]) > 0.1


def test_integer_inputs_exact():
    r = np.random.default_rng(12)
    q, k, v = (r.integers(-1, 2, size=(40, 6)).astype(np.float64) for _ in range(3))
    rn, rd = matrix_form(q, k, v, 1.0)
    num, den, _ = O.ho3_serial(q, k, v, 1.0)
    assert np.array_equal(num, rn) and np.array_equal(den, rd)


@pytest.mark.parametrize("tstar", [0, 17, 39])
def test_causality(tstar):
    q, k, v = draw(21, 40, 4, 3)
    a, ad, _ = O.ho3_serial(q, k, v, 0.9)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[tstar:] += 1.0
    k2[tstar:] -= 2.0
    v2[tstar:] *= 3.0
    b, bd, _ = O.ho3_serial(q2, k2, v2, 0.9)
    assert np.array_equal(a[:tstar], b[:tstar]) and np.array_equal(ad[:tstar], bd[:tstar])
    if tstar < 39:
        assert not np.array_equal(a[tstar:], b[tstar:])


def test_fold_of_segments_equals_serial():
    q, k, v = draw(30, 50, 4, 3)
    d, dv = 4, 3
    _, _, st = O.ho3_serial(q, k, v, 0.97)
    s = np.zeros(O.ho3_state_len(d, dv))
    for a, b in ((0, 9), (9, 32), (32, 50)):
        s = O.ho3_apply(O.ho3_summary(q[a:b], k[a:b], v[a:b], 0.97), s, d, dv)
    assert rel(s, st) < 1e-12


def test_clean_source_passes_condensed_pins():
    assert pin_failures(O._load()) == []


MUTANTS = {
    "W decays by gamma^2": ("const double g3 = gamma * gamma * gamma;", "const double g3 = gamma * gamma;"),
    "P absorbs q v^T": ("for (c = 0; c < dv; ++c) P[(long)a * dvp + c] = gamma * P[(long)a * dvp + c] + k[a] * v[c];",
                        "for (c = 0; c < dv; ++c) P[(long)a * dvp + c] = gamma * P[(long)a * dvp + c] + q[a] * v[c];"),
    "z from S^T k": ("for (b = 0; b < d; ++b) z[a] += S[(long)a * d + b] * q[b];\n    for (c = 0; c < dvp; ++c) y[c] += q[a]",
                     "for (b = 0; b < d; ++b) z[a] += S[(long)a * d + b] * k[b];\n    for (c = 0; c < dvp; ++c) y[c] += q[a]"),
    "key mass absorbs q": ("P[(long)a * dvp + dv] = gamma * P[(long)a * dvp + dv] + k[a];",
                           "P[(long)a * dvp + dv] = gamma * P[(long)a * dvp + dv] + q[a];"),
    "Q2 weight off by one": ("const double wq = pow(gamma, (double)(3 * len - 1 - u)),",
                             "const double wq = pow(gamma, (double)(3 * len - u)),"),
    "X2 from q z^T": ("X2[(long)a * d + b] += wx * z[a] * qu[b];", "X2[(long)a * d + b] += wx * qu[a] * z[b];"),
    "fold drops S_A X1": ("s += SQ[(long)a * d + b] * P[(long)b * dvp + c] + S[(long)a * d + b] * X1[(long)b * dvp + c] +",
                          "s += SQ[(long)a * d + b] * P[(long)b * dvp + c] + 0.0 * X1[(long)b * dvp + c] +"),
    "fold W decays once": ("const double G = sum[0], G3 = G * G * G;", "const double G = sum[0], G3 = G;"),
    "den-column norm of P instead of W": ("const double *W = st + (long)d * d + (long)d * dvp;",
                                          "const double *W = st + (long)d * d;"),
    "brute force decays the middle index once": (
        "double w = pow(gamma, (double)((t - j) + (t - l) + (t - i))) * f1",
        "double w = pow(gamma, (double)((t - j) + (t - i))) * f1"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site moved: %r" % old
    src = tmp_path / "mut.c"
    lib = tmp_path / "libmut.so"
    src.write_text(text.replace(old, new))
    subprocess.run(["gcc", "-std=c99", "-O1", "-ffp-contract=off", "-fPIC", "-shared", str(src), "-o", str(lib),
                    "-lm"], check=True)
    assert pin_failures(O._load(str(lib))), "planted slip not caught: " + name


@pytest.mark.parametrize("gamma", [1.0, 0.8])
def test_den_column_norms_equal_matrix_form(gamma):
    # |w_t| (the conditioning scale of the ratio) against its matrix form, and num, den unchanged from
    # ho3_serial; multi-head and threaded
    r = np.random.default_rng(11)
    q, k, v = (0.5 * r.standard_normal((2, 3, 36, 4)), 0.5 * r.standard_normal((2, 3, 36, 4)),
               r.standard_normal((2, 3, 36, 3)))
    num, den, un, st = O.ho3_serial_unorm(q, k, v, gamma, threads=3)
    num2, den2, st2 = O.ho3_serial(q, k, v, gamma)
    np.testing.assert_array_equal(num, num2)
    np.testing.assert_array_equal(den, den2)
    np.testing.assert_array_equal(st, st2)
    for a in range(2):
        for b in range(3):
            assert rel(un[a, b], den_column_norms(q[a, b], k[a, b], gamma)) < 1e-11
    assert np.all(np.abs(den) <= np.linalg.norm(q, axis=-1) * un * (1 + 1e-12))
