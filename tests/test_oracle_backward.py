"""Pins of the oracle's gradients (``oracle.backward``, the chain rule through the
definition in matrix form, and ``oracle.backward_serial``, the adjoint of the
serial recurrence in ``hla2_oracle.c``) against things other than themselves.

The pages print no backward formulas, so the pins come from calculus:
  * central finite differences of the loss sum(dout * o), with o from the
    oracle's brute-force triple sum (a separate C routine; neither gradient
    path calls it);
  * Euler's theorem: num is homogeneous of degree 2 in q, 2 in k and 1 in v, and
    the ratio o = num / den of degree 0 in q and in k, which fixes sum(q * dq),
    sum(k * dk) and sum(v * dv) in closed form;
  * closed forms for all-ones inputs (d = dv = 1, no decay);
  * one token under the ratio: o_0 = v_0 whatever q_0, k_0 are, so dq = dk = 0
    and dv = dout;
  * the two gradient paths (different algorithms) agree to rounding.
Planted slips in either path must fail one of these (``test_mutant_*``).
"""
import os
import subprocess
import types

import numpy as np
import pytest

from oracle import oracle as O

SRC_C = os.path.join(os.path.dirname(O.__file__), "hla2_oracle.c")
SRC_PY = os.path.join(os.path.dirname(O.__file__), "oracle.py")


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def draw(seed, n, d, dv, positive=False):
    r = np.random.default_rng(seed)
    q, k, v, do = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv)), \
        r.standard_normal((n, dv))
    if positive:  # keeps den well away from zero for the ratio
        q, k, v = np.abs(q) + 0.2, np.abs(k) + 0.2, np.abs(v)
    return q, k, v, do


def loss_bruteforce(q, k, v, do, gamma, normalize):
    num, den = O.bruteforce(q, k, v, gamma)
    o = O.ratio(num, den) if normalize else num
    return float(np.sum(do * o))


def fd_grads(q, k, v, do, gamma, normalize, h=1e-5):
    out = []
    for which in range(3):
        x = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(x[which])
        for idx in np.ndindex(g.shape):
            xp = [a.copy() for a in x]
            xm = [a.copy() for a in x]
            xp[which][idx] += h
            xm[which][idx] -= h
            g[idx] = (loss_bruteforce(*xp, do, gamma, normalize) - loss_bruteforce(*xm, do, gamma, normalize)) / (2 * h)
        out.append(g)
    return out


def pin_failures(backward_fn):
    """Condensed pins for one gradient path ``backward_fn(q, k, v, do, gamma, normalize)``;
    returns the names of the pins that fail."""
    bad = []
    for (n, d, dv, gamma, normalize, seed) in [(7, 3, 2, 1.0, False, 1), (7, 3, 2, 0.8, False, 2),
                                               (6, 2, 3, 0.9, True, 3), (6, 3, 2, 1.0, True, 4)]:
        q, k, v, do = draw(seed, n, d, dv, positive=normalize)
        got = backward_fn(q, k, v, do, gamma, normalize)
        ref = fd_grads(q, k, v, do, gamma, normalize)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            if rel(a, b) > 1e-7:
                bad.append("finite differences %s n=%d gamma=%g normalize=%d" % (name, n, gamma, normalize))
    # Euler's theorem on a longer sequence
    for gamma in (1.0, 0.9):
        q, k, v, do = draw(11, 40, 5, 4)
        dq, dk, dv = backward_fn(q, k, v, do, gamma, False)
        num, _ = O.bruteforce(q, k, v, gamma)
        L = float(np.sum(do * num))
        if abs(np.sum(q * dq) - 2 * L) > 1e-10 * abs(L) or abs(np.sum(k * dk) - 2 * L) > 1e-10 * abs(L) \
                or abs(np.sum(v * dv) - L) > 1e-10 * abs(L):
            bad.append("Euler unnormalised gamma=%g" % gamma)
        q, k, v, do = draw(12, 40, 5, 4, positive=True)
        dq, dk, dv = backward_fn(q, k, v, do, gamma, True)
        num, den = O.bruteforce(q, k, v, gamma)
        L = float(np.sum(do * O.ratio(num, den)))
        scale = np.linalg.norm(q) * np.linalg.norm(dq) + np.linalg.norm(k) * np.linalg.norm(dk)
        if abs(np.sum(q * dq)) > 1e-12 * scale or abs(np.sum(k * dk)) > 1e-12 * scale \
                or abs(np.sum(v * dv) - L) > 1e-10 * abs(L):
            bad.append("Euler ratio gamma=%g" % gamma)
    # all-ones closed forms (d = dv = 1, gamma = 1, dout = 1)
    n = 9
    one = np.ones((n, 1))
    dq, dk, dv = backward_fn(one, one, one, one, 1.0, False)
    t = np.arange(n, dtype=np.float64)
    if not (np.array_equal(dv[:, 0], (n - t) * (t + 1)) and
            np.array_equal(dq[:, 0], (t + 1) * (t + 2) / 2 + (n - t) * (t + 1)) and
            np.array_equal(dk[:, 0], (n - t) * (n - t + 1))):
        bad.append("all-ones closed form")
    # one token under the ratio
    q, k, v, do = draw(13, 1, 4, 3, positive=True)
    dq, dk, dv = backward_fn(q, k, v, do, 0.7, True)
    if np.abs(dq).max() > 1e-12 or np.abs(dk).max() > 1e-12 or rel(dv, do) > 1e-14:
        bad.append("single token ratio")
    return bad


def _matrix(q, k, v, do, gamma, normalize):
    return O.backward(q, k, v, do, gamma, normalize)


def _serial(lib):
    return lambda q, k, v, do, gamma, normalize: O.backward_serial(q, k, v, do, gamma, normalize, lib=lib)


def test_matrix_form_passes_pins():
    assert pin_failures(_matrix) == []


def test_serial_adjoint_passes_pins():
    assert pin_failures(_serial(O._load())) == []


@pytest.mark.parametrize("n,d,dv,gamma,normalize", [
    (1, 4, 4, 1.0, False), (2, 3, 5, 0.5, False), (33, 8, 6, 0.97, False), (64, 16, 16, 1.0, True),
    (50, 6, 9, 0.9, True), (129, 4, 3, 0.99, False)])
def test_serial_adjoint_equals_matrix_form(n, d, dv, gamma, normalize):
    r = np.random.default_rng(n * 100 + d)
    q, k, v, do = r.standard_normal((2, n, d)), r.standard_normal((2, n, d)), r.standard_normal((2, n, dv)), \
        r.standard_normal((2, n, dv))
    if normalize:
        q, k, v = np.abs(q) + 0.1, np.abs(k) + 0.1, np.abs(v)
    a = O.backward(q, k, v, do, gamma, normalize)
    b = O.backward_serial(q, k, v, do, gamma, normalize)
    for x, y in zip(a, b):
        assert rel(y, x) < 1e-12


def test_given_forward_outputs_are_used():
    """For the ratio, out and den passed in replace the forward's own (both paths)."""
    q, k, v, do = draw(21, 10, 3, 2, positive=True)
    num, den = O.bruteforce(q, k, v, 0.9)
    o = O.ratio(num, den)
    a = O.backward(q, k, v, do, 0.9, True, out=o, den=den)
    b = O.backward(q, k, v, do, 0.9, True)
    c = O.backward_serial(q, k, v, do, 0.9, True, out=o * 1.5, den=den)
    d_ = O.backward(q, k, v, do, 0.9, True, out=o * 1.5, den=den)
    for x, y in zip(a, b):
        assert rel(x, y) < 1e-13
    for x, y in zip(c, d_):
        assert rel(x, y) < 1e-12
    assert rel(d_[0], a[0]) > 1e-3


MUTANTS_C = {
    "Ubar decays by gamma": ("Ub[(long)a * dvp + c] = gsq * Ub[(long)a * dvp + c] + qt[a] * gt[c];",
                             "Ub[(long)a * dvp + c] = gamma * Ub[(long)a * dvp + c] + qt[a] * gt[c];"),
    "zbar drops the ones column": ("double s = Ub[(long)a * dvp + dv];  /* the ones column of v' */",
                                   "double s = 0.0;"),
    "dk without the transpose": ("s += (Sb[(long)a * d + b] + Sb[(long)b * d + a]) * kt[b];",
                                 "s += 2.0 * Sb[(long)a * d + b] * kt[b];"),
    "Sbar decays by gamma^2": ("Sb[(long)a * d + b] = gamma * Sb[(long)a * d + b] + zbt[a] * qt[b];",
                               "Sb[(long)a * d + b] = gsq * Sb[(long)a * d + b] + zbt[a] * qt[b];"),
    "dq drops S zbar": ("for (b = 0; b < d; ++b) s += S[(long)a * d + b] * zbt[b];\n      dq",
                        "for (b = 0; b < 0; ++b) s += S[(long)a * d + b] * zbt[b];\n      dq"),
    "ratio gradient of den squared": ("gt[dv] = -dot / den[t];", "gt[dv] = -dot / (den[t] * den[t]);"),
    "dv from Ubar transposed use": ("for (a = 0; a < d; ++a) s += Ub[(long)a * dvp + c] * z[(long)t * d + a];",
                                    "for (a = 0; a < d; ++a) s += Ub[(long)a * dvp + c] * zb[(long)t * d + a];"),
}

MUTANTS_PY = {
    "dV from M instead of M^T": ("dvv[h] = M.T @ gnum", "dvv[h] = M @ gnum"),
    "P without the decay": ("P = D * dM", "P = dM"),
    "dA misses the D factor": ("dA = P.T @ Ag + D * dAg", "dA = P.T @ Ag + dAg"),
    "dA uses A instead of A_g": ("dA = P.T @ Ag + D * dAg", "dA = P.T @ A + D * dAg"),
    "scores gradient unmasked": ("dX = np.where(lower, dA, 0.0)", "dX = dA"),
    "dK from dX instead of dX^T": ("dk[h] = dX.T @ Q", "dk[h] = dX @ Q"),
    "ratio den gradient sign": ("gden = -np.sum(G * oh[h], axis=-1) / dh[h]",
                                "gden = np.sum(G * oh[h], axis=-1) / dh[h]"),
}


def _build_c(tmp_path, text, name):
    src = tmp_path / (name + ".c")
    lib = tmp_path / ("lib" + name + ".so")
    src.write_text(text)
    subprocess.run(["gcc", "-std=c99", "-O1", "-ffp-contract=off", "-fPIC", "-shared", str(src), "-o", str(lib),
                    "-lm"], check=True)
    return O._load(str(lib))


@pytest.mark.parametrize("name", sorted(MUTANTS_C))
def test_mutant_serial_adjoint_is_caught(tmp_path, name):
    old, new = MUTANTS_C[name]
    text = open(SRC_C).read()
    assert text.count(old) == 1, "mutation site moved: %r" % old
    lib = _build_c(tmp_path, text.replace(old, new), "mut")
    assert pin_failures(_serial(lib)), "planted slip not caught: " + name


@pytest.mark.parametrize("name", sorted(MUTANTS_PY))
def test_mutant_matrix_form_is_caught(name):
    old, new = MUTANTS_PY[name]
    text = open(SRC_PY).read()
    assert text.count(old) == 1, "mutation site moved: %r" % old
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC_PY
    exec(compile(text.replace(old, new), SRC_PY, "exec"), mod.__dict__)
    fn = lambda q, k, v, do, gamma, normalize: mod.backward(q, k, v, do, gamma, normalize)  # noqa: E731
    assert pin_failures(fn), "planted slip not caught: " + name
