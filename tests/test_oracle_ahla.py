"""Pins of the oracle's AHLA path (the asymmetric variant, Q (K^T Q)(K^T V)) against
things other than itself, and planted slips that the pins must catch.

Pins:
  * the masked matrix form A_g A_g V with A_g = D o L o (Q K^T) (numpy matmuls;
    for gamma = 1 the textbook product of two masked score matrices);
  * closed forms for all-ones inputs, which differ from the second-order ones;
  * exact integer arithmetic for entries in {-1, 0, 1};
  * strict causality;
  * the segment summary of a concatenation equals the combine of the summaries
    (the chunk-parallel form), the combine is associative with an identity, and
    a summary's state part equals the serial state.
"""
import os
import subprocess

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
    Ag = np.where(low, gamma ** np.where(low, t[:, None] - t[None, :], 0) * (q @ k.T), 0.0)
    M = Ag @ Ag
    return M @ v, M.sum(axis=1)


def den_column_norms(q, k, gamma):
    """|n_t| from the matrix form: n_t = sum_{j<=t} g^{t-j} (q_j . m_j) k_j with q_j . m_j = (A_g 1)_j,
    i.e. the rows of (L o D_g) diag(A_g 1) K (so den = Q n = A_g A_g 1 row by row)."""
    n = q.shape[0]
    t = np.arange(n)
    low = t[:, None] >= t[None, :]
    Dg = np.where(low, gamma ** np.where(low, t[:, None] - t[None, :], 0), 0.0)
    Ag = Dg * (q @ k.T)
    N = Dg @ ((Ag @ np.ones(n))[:, None] * k)
    return np.linalg.norm(N, axis=1)


def draw(seed, n, d, dv):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))


def pin_failures(lib):
    bad = []
    for gamma in (1.0, 0.9, 0.5):
        q, k, v = draw(5, 31, 5, 3)
        rn, rd = matrix_form(q, k, v, gamma)
        num, den, st = O.ahla_serial(q, k, v, gamma, lib=lib)
        if rel(num, rn) > 1e-12 or rel(den, rd) > 1e-12:
            bad.append("serial vs matrix form gamma=%g" % gamma)
        un_num, un_den, un, _ = O.ahla_serial_unorm(q, k, v, gamma, lib=lib)
        if rel(un, den_column_norms(q, k, gamma)) > 1e-12 or not np.array_equal(un_num, num) or \
                not np.array_equal(un_den, den):
            bad.append("den-column norms vs matrix form gamma=%g" % gamma)
        bn, bd = O.ahla_bruteforce(q, k, v, gamma, lib=lib)
        if rel(bn, rn) > 1e-12 or rel(bd, rd) > 1e-12:
            bad.append("bruteforce vs matrix form gamma=%g" % gamma)
        d, dv = 5, 3
        s1 = O.ahla_summary(q[:12], k[:12], v[:12], gamma, lib=lib)
        s2 = O.ahla_summary(q[12:], k[12:], v[12:], gamma, lib=lib)
        whole = O.ahla_summary(q, k, v, gamma, lib=lib)
        if rel(O.ahla_combine(s1, s2, d, dv, lib=lib), whole) > 1e-12:
            bad.append("concatenation gamma=%g" % gamma)
        if rel(whole[1:1 + st.shape[-1]], st) > 1e-13:
            bad.append("summary state vs serial state gamma=%g" % gamma)
        # continuing the serial recurrence from the summary of a prefix gives the rest
        _, _, st1 = O.ahla_serial(q[:12], k[:12], v[:12], gamma, lib=lib)
        n2, d2, _ = O.ahla_serial(q[12:], k[12:], v[12:], gamma, state=st1, lib=lib)
        if rel(n2, rn[12:]) > 1e-12 or rel(d2, rd[12:]) > 1e-12:
            bad.append("continuation gamma=%g" % gamma)
    one = np.ones((4, 1))
    num, den, _ = O.ahla_serial(one, one, one, 0.5, lib=lib)
    if not (np.array_equal(num[:, 0], [1.0, 2.0, 2.75, 3.25]) and np.array_equal(den, num[:, 0])):
        bad.append("closed form gamma=1/2")
    return bad


@pytest.mark.parametrize("n,d,dv,gamma", [(1, 3, 2, 1.0), (2, 1, 1, 0.5), (40, 8, 5, 1.0), (65, 4, 7, 0.95),
                                          (100, 16, 16, 0.99)])
def test_serial_equals_matrix_form(n, d, dv, gamma):
    q, k, v = draw(n + d, n, d, dv)
    rn, rd = matrix_form(q, k, v, gamma)
    num, den, _ = O.ahla_serial(q, k, v, gamma)
    assert rel(num, rn) < 1e-12 and rel(den, rd) < 1e-12


@pytest.mark.parametrize("gamma", [1.0, 0.8])
def test_bruteforce_equals_matrix_form(gamma):
    q, k, v = draw(3, 25, 4, 3)
    rn, rd = matrix_form(q, k, v, gamma)
    bn, bd = O.ahla_bruteforce(q, k, v, gamma)
    assert rel(bn, rn) < 1e-12 and rel(bd, rd) < 1e-12


def test_closed_forms_all_ones():
    n = 12
    one = np.ones((n, 1))
    num, den, _ = O.ahla_serial(one, one, one, 1.0)
    t = np.arange(n, dtype=np.float64)
    assert np.array_equal(num[:, 0], (t + 1) * (t + 2) / 2) and np.array_equal(den, num[:, 0])
    # with decay the term (j, i) carries gamma^(t-i): sum_i gamma^(t-i) (t - i + 1)
    num, _, _ = O.ahla_serial(one[:4], one[:4], one[:4], 0.5)
    assert np.array_equal(num[:, 0], [1.0, 2.0, 2.75, 3.25])


def test_differs_from_second_order():
    """The asymmetric operator is not the symmetric one (random inputs)."""
    q, k, v = draw(8, 30, 4, 3)
    a, _, _ = O.ahla_serial(q, k, v, 1.0)
    b, _, _ = O.serial(q, k, v, 1.0)
    assert rel(a, b) > 0.1


def test_integer_inputs_exact():
    r = np.random.default_rng(12)
    q, k, v = (r.integers(-1, 2, size=(48, 8)).astype(np.float64) for _ in range(3))
    rn, rd = matrix_form(q, k, v, 1.0)
    num, den, _ = O.ahla_serial(q, k, v, 1.0)
    assert np.array_equal(num, rn) and np.array_equal(den, rd)


@pytest.mark.parametrize("tstar", [0, 17, 39])
def test_causality(tstar):
    q, k, v = draw(21, 40, 4, 3)
    a, ad, _ = O.ahla_serial(q, k, v, 0.9)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[tstar:] += 1.0
    k2[tstar:] -= 2.0
    v2[tstar:] *= 3.0
    b, bd, _ = O.ahla_serial(q2, k2, v2, 0.9)
    assert np.array_equal(a[:tstar], b[:tstar]) and np.array_equal(ad[:tstar], bd[:tstar])
    if tstar < 39:
        assert not np.array_equal(a[tstar:], b[tstar:])


def test_combine_associative_with_identity():
    q, k, v = draw(30, 30, 4, 3)
    d, dv = 4, 3
    s = [O.ahla_summary(q[a:b], k[a:b], v[a:b], 0.9) for a, b in ((0, 7), (7, 19), (19, 30))]
    left = O.ahla_combine(O.ahla_combine(s[0], s[1], d, dv), s[2], d, dv)
    right = O.ahla_combine(s[0], O.ahla_combine(s[1], s[2], d, dv), d, dv)
    assert rel(left, right) < 1e-13
    ident = np.zeros_like(s[0])
    ident[0] = 1.0
    assert np.array_equal(O.ahla_combine(ident, s[1], d, dv), s[1])
    assert rel(O.ahla_combine(s[1], ident, d, dv), s[1]) < 1e-15


def test_clean_source_passes_condensed_pins():
    assert pin_failures(O._load()) == []


MUTANTS = {
    "P absorbs q v^T": ("for (c = 0; c < dv; ++c) P[(long)a * dv + c] = gamma * P[(long)a * dv + c] + k[a] * v[c];",
                        "for (c = 0; c < dv; ++c) P[(long)a * dv + c] = gamma * P[(long)a * dv + c] + q[a] * v[c];"),
    "key mass absorbs q": ("    m[a] = gamma * m[a] + k[a];\n  }\n  for (a = 0; a < d; ++a) {\n    for (c = 0; c < dv; ++c) qP",
                           "    m[a] = gamma * m[a] + q[a];\n  }\n  for (a = 0; a < d; ++a) {\n    for (c = 0; c < dv; ++c) qP"),
    "E absorbs q (q^T P)": ("E[(long)a * dv + c] = gamma * E[(long)a * dv + c] + k[a] * qP[c];",
                            "E[(long)a * dv + c] = gamma * E[(long)a * dv + c] + q[a] * qP[c];"),
    "n decays twice": ("nn[a] = gamma * nn[a] + k[a] * qm;", "nn[a] = gamma * gamma * nn[a] + k[a] * qm;"),
    "readout from P": ("for (a = 0; a < d; ++a) s += q[a] * E[(long)a * dv + c];",
                       "for (a = 0; a < d; ++a) s += q[a] * P[(long)a * dv + c];"),
    "combine cross term from M_A": ("for (b = 0; b < d; ++b) s += MB[(long)a * d + b] * PA[(long)b * dv + c];",
                                    "for (b = 0; b < d; ++b) s += MA[(long)a * d + b] * PA[(long)b * dv + c];"),
    "combine E cross term without Gamma_B": (
        "Eo[(long)a * dv + c] = GB * EA[(long)a * dv + c] + EB[(long)a * dv + c] + GB * s;",
        "Eo[(long)a * dv + c] = GB * EA[(long)a * dv + c] + EB[(long)a * dv + c] + s;"),
    "summary M transposed": ("M[(long)a * d + b] += k[(long)t * d + a] * q[(long)t * d + b];",
                             "M[(long)a * d + b] += q[(long)t * d + a] * k[(long)t * d + b];"),
    "den-column norm of m instead of n": ("const double *nn = st + 2L * d * dv + d;",
                                          "const double *nn = st + (long)d * dv;"),
    "brute force decays by the middle index": ("double w = pow(gamma, (double)(t - i)) * qk_tj * qk_ji;",
                                               "double w = pow(gamma, (double)(t - j)) * qk_tj * qk_ji;"),
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
    # |n_t| (the conditioning scale of the ratio) against its matrix form, and num, den unchanged from
    # ahla_serial; multi-head and threaded
    r = np.random.default_rng(9)
    q, k, v = r.standard_normal((2, 3, 40, 4)), r.standard_normal((2, 3, 40, 4)), r.standard_normal((2, 3, 40, 3))
    num, den, un, st = O.ahla_serial_unorm(q, k, v, gamma, threads=3)
    num2, den2, st2 = O.ahla_serial(q, k, v, gamma)
    np.testing.assert_array_equal(num, num2)
    np.testing.assert_array_equal(den, den2)
    np.testing.assert_array_equal(st, st2)
    for a in range(2):
        for b in range(3):
            assert rel(un[a, b], den_column_norms(q[a, b], k[a, b], gamma)) < 1e-12
    assert np.all(np.abs(den) <= np.linalg.norm(q, axis=-1) * un * (1 + 1e-12))
