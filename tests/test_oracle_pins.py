"""Pins of the fp64 oracle against things other than itself.

Each pin is chosen so that a plausible slip in ``oracle/hla2_oracle.c`` (a dropped
term, a wrong sign or index, the wrong time of a state read, a transposed
operand) fails at least one of them; ``test_oracle_mutants.py`` plants such slips
and checks that they are caught.

Pins used (none of them calls the code it checks twice):
  * the masked matrix form L o D^2 o (A (D o A)^T) with A = L o (Q K^T), written
    with numpy matmuls -- for gamma = 1 this is the textbook two-GEMM form
    L o (A A^T) V;
  * closed forms for constant inputs;
  * exact integer arithmetic (entries in {-1, 0, 1});
  * invariants the pages state: scan output equals serial output
    ("Scan-equivalentie", §4 of the gist.science technical summary), strict
    causality ("Resultaten en claims"), and the concatenation property a
    segment summary must have.
"""
import numpy as np
import pytest

from oracle import oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def matrix_form(q, k, v, gamma):
    """num, den from the masked matrix form (numpy, one head)."""
    n = q.shape[0]
    t = np.arange(n)
    expo = (t[:, None] - t[None, :]).astype(np.float64)
    low = expo >= 0
    Dg = np.where(low, gamma ** np.where(low, expo, 0.0), 0.0)  # gamma^{t-i}, i <= t
    A = np.where(low, q @ k.T, 0.0)
    M = np.where(low, Dg * ((A * Dg) @ A.T), 0.0)
    return M @ v, M.sum(axis=1)


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.mark.parametrize("gamma", [1.0, 0.9, 0.5])
@pytest.mark.parametrize("n,d,dv", [(1, 3, 2), (29, 5, 3), (40, 3, 7)])
def test_serial_equals_matrix_form(n, d, dv, gamma):
    r = _rng(n * 100 + d)
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))
    num, den, _ = O.serial(q, k, v, gamma)
    rn, rd = matrix_form(q, k, v, gamma)
    assert rel(num, rn) < 1e-12
    assert rel(den, rd) < 1e-12


@pytest.mark.parametrize("gamma", [1.0, 0.8])
def test_bruteforce_equals_matrix_form(gamma):
    r = _rng(7)
    q, k, v = r.standard_normal((33, 4)), r.standard_normal((33, 4)), r.standard_normal((33, 6))
    num, den = O.bruteforce(q, k, v, gamma)
    rn, rd = matrix_form(q, k, v, gamma)
    assert rel(num, rn) < 1e-12
    assert rel(den, rd) < 1e-12


def test_single_token():
    # n = 1: the only pair is (0, 0): num = (q.k)^2 v, den = (q.k)^2.
    q, k, v = np.array([[0.5, -2.0]]), np.array([[1.5, 0.25]]), np.array([[3.0, -1.0, 2.0]])
    num, den, _ = O.serial(q, k, v, 0.7)
    s = (0.5 * 1.5 - 2.0 * 0.25) ** 2
    np.testing.assert_array_equal(num[0], s * v[0])
    assert den[0] == s


def test_closed_form_all_ones_no_decay():
    # d = dv = 1, q = k = v = 1: every pair i <= j <= t counts once, so
    # num_t = den_t = (t+1)(t+2)/2 and the ratio is exactly 1.
    n = 50
    one = np.ones((n, 1))
    num, den, _ = O.serial(one, one, one, 1.0)
    t = np.arange(n)
    np.testing.assert_array_equal(num[:, 0], (t + 1) * (t + 2) / 2)
    np.testing.assert_array_equal(den, (t + 1) * (t + 2) / 2)
    np.testing.assert_array_equal(O.ratio(num, den)[:, 0], np.ones(n))


def test_closed_form_all_ones_decay_half():
    # d = dv = 1, all ones, gamma = 1/2.  Summing gamma^{(t-i)+(t-j)} over
    # i <= j <= t gives num_t = sum_j gamma^{2(t-j)} (1 - gamma^{j+1}) / (1 - gamma):
    # 1, 7/4, 35/16, 155/64 for t = 0..3 (exact binary fractions).
    one = np.ones((4, 1))
    num, den, _ = O.serial(one, one, one, 0.5)
    np.testing.assert_array_equal(num[:, 0], [1.0, 1.75, 2.1875, 2.421875])
    np.testing.assert_array_equal(den, [1.0, 1.75, 2.1875, 2.421875])


def test_closed_form_onehot_random_values():
    # q = k = e_1 in d = 4: (q_t.k_i)(q_j.k_i) = 1 for every pair, so with
    # gamma = 1 the weight of v_j at time t is the number of i <= j, i.e. j + 1.
    n, d, dv = 30, 4, 5
    e = np.zeros((n, d))
    e[:, 0] = 1.0
    v = _rng(3).standard_normal((n, dv))
    num, den, _ = O.serial(e, e, v, 1.0)
    w = np.arange(1, n + 1, dtype=np.float64)
    ref = np.cumsum(w[:, None] * v, axis=0)
    assert rel(num, ref) < 1e-14
    np.testing.assert_array_equal(den, np.cumsum(w))


def test_integer_inputs_exact():
    # Entries in {-1, 0, 1} at the tiny-config shape: every intermediate is an
    # integer far below 2^53, so all three oracle paths agree bit for bit with
    # the matrix form.
    r = _rng(11)
    n, d, dv = 64, 16, 16
    q, k, v = (r.integers(-1, 2, size=(n, x)).astype(np.float64) for x in (d, d, dv))
    num, den, st = O.serial(q, k, v, 1.0)
    bn, bd = O.bruteforce(q, k, v, 1.0)
    cn, cd, cst = O.chunked(q, k, v, 1.0, chunk=16)
    rn, rd = matrix_form(q, k, v, 1.0)
    for a in (num, bn, cn):
        np.testing.assert_array_equal(a, rn)
    for a in (den, bd, cd):
        np.testing.assert_array_equal(a, rd)
    np.testing.assert_array_equal(st, cst)
    assert np.all(num == np.round(num)) and np.abs(num).max() < 2 ** 24


@pytest.mark.parametrize("gamma", [1.0, 0.9])
@pytest.mark.parametrize("n,chunk", [(64, 1), (64, 4), (64, 16), (64, 64), (100, 16), (37, 8), (5, 16)])
def test_chunked_scan_equals_serial(n, chunk, gamma):
    r = _rng(n + chunk)
    d, dv = 6, 4
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))
    num, den, st = O.serial(q, k, v, gamma)
    cn, cd, cst = O.chunked(q, k, v, gamma, chunk=chunk)
    assert rel(cn, num) < 1e-12
    assert rel(cd, den) < 1e-12
    assert rel(cst, st) < 1e-12  # the scan total is the serial final state


@pytest.mark.parametrize("gamma", [1.0, 0.95])
def test_summary_concatenation(gamma):
    # The summary of a concatenation (by definition, pairs inside the whole
    # segment) equals the combine of the parts' summaries.
    r = _rng(5)
    d, dv, la, lb = 4, 3, 7, 9
    q, k, v = r.standard_normal((la + lb, d)), r.standard_normal((la + lb, d)), r.standard_normal((la + lb, dv))
    whole = O.segment_summary(q, k, v, gamma)
    a = O.segment_summary(q[:la], k[:la], v[:la], gamma)
    b = O.segment_summary(q[la:], k[la:], v[la:], gamma)
    assert rel(O.combine(a, b, d, dv), whole) < 1e-13
    # and the order matters: the combine is not commutative
    assert rel(O.combine(b, a, d, dv), whole) > 1e-3


def test_summary_equals_serial_state():
    # A summary's (S, C, m, G, h) is the serial state after the segment from zero.
    r = _rng(9)
    d, dv, n = 5, 3, 21
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))
    _, _, st = O.serial(q, k, v, 0.9)
    s = O.segment_summary(q, k, v, 0.9)
    assert s[0] == pytest.approx(0.9 ** n, rel=1e-15)
    assert rel(s[1:], st) < 1e-13


def test_combine_associative_and_identity():
    r = _rng(13)
    d, dv = 4, 5
    segs = []
    for ln in (3, 6, 4):
        q, k, v = r.standard_normal((ln, d)), r.standard_normal((ln, d)), r.standard_normal((ln, dv))
        segs.append(O.segment_summary(q, k, v, 0.9))
    A, B, C = segs
    left = O.combine(O.combine(A, B, d, dv), C, d, dv)
    right = O.combine(A, O.combine(B, C, d, dv), d, dv)
    assert rel(left, right) < 1e-13
    e = O.identity(d, dv)
    np.testing.assert_array_equal(O.combine(e, A, d, dv), A)
    np.testing.assert_array_equal(O.combine(A, e, d, dv), A)


def test_exclusive_scan_matches_left_fold():
    r = _rng(17)
    d, dv, cnt = 3, 2, 6
    sums = []
    for i in range(cnt):
        q, k, v = r.standard_normal((4, d)), r.standard_normal((4, d)), r.standard_normal((4, dv))
        sums.append(O.segment_summary(q, k, v, 0.8))
    sums = np.stack(sums)
    ex = O.exclusive_scan(sums, d, dv)
    acc = O.identity(d, dv)
    for i in range(cnt):
        assert rel(ex[i], acc) < 1e-13 or np.array_equal(ex[i], acc)
        acc = O.combine(acc, sums[i], d, dv)


@pytest.mark.parametrize("tstar", [0, 1, 15, 16, 31, 63])
def test_causality(tstar):
    r = _rng(21)
    n, d, dv = 64, 4, 4
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))
    num, den, _ = O.serial(q, k, v, 0.9)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[tstar:] += 1.0
    k2[tstar:] -= 2.0
    v2[tstar:] *= 3.0
    num2, den2, _ = O.serial(q2, k2, v2, 0.9)
    np.testing.assert_array_equal(num2[:tstar], num[:tstar])
    np.testing.assert_array_equal(den2[:tstar], den[:tstar])
    assert not np.array_equal(num2[tstar:], num[tstar:])


def test_decode_continues_serial():
    # Prefix by the serial run, then one step at a time: same outputs and state
    # as one serial run over the whole sequence.
    r = _rng(23)
    n, m, d, dv = 24, 17, 4, 3
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))
    num, den, st = O.serial(q, k, v, 0.9)
    _, _, s = O.serial(q[:m], k[:m], v[:m], 0.9)
    for t in range(m, n):
        nm, dn, s = O.step(s, q[t], k[t], v[t], 0.9)
        assert rel(nm, num[t]) < 1e-13 and dn == pytest.approx(den[t], rel=1e-13)
    assert rel(s, st) < 1e-13


def test_unnormalised_is_linear_in_v():
    r = _rng(29)
    n, d, dv = 20, 3, 2
    q, k = r.standard_normal((n, d)), r.standard_normal((n, d))
    v1, v2 = r.standard_normal((n, dv)), r.standard_normal((n, dv))
    a, _, _ = O.serial(q, k, v1, 0.9)
    b, _, _ = O.serial(q, k, v2, 0.9)
    c, _, _ = O.serial(q, k, 2.0 * v1 - v2, 0.9)
    assert rel(c, 2.0 * a - b) < 1e-13


def test_multihead_threads_match_single():
    r = _rng(31)
    q, k, v = r.standard_normal((3, 2, 19, 4)), r.standard_normal((3, 2, 19, 4)), r.standard_normal((3, 2, 19, 5))
    a = O.serial(q, k, v, 0.9, threads=4)
    b = O.serial(q, k, v, 0.9, threads=1)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    for h in range(3):
        for g in range(2):
            one = O.serial(q[h, g], k[h, g], v[h, g], 0.9)
            np.testing.assert_array_equal(one[0], a[0][h, g])


def test_unorm_matches_state_and_serial():
    # |S_t m_t - h_t| from the recurrence's own state, and num/den identical to serial()
    r = _rng(37)
    n, d, dv = 15, 4, 3
    q, k, v = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal((n, dv))
    num, den, st = O.serial(q, k, v, 0.9)
    n2, d2, un, st2 = O.serial_unorm(q, k, v, 0.9)
    np.testing.assert_array_equal(num, n2)
    np.testing.assert_array_equal(den, d2)
    np.testing.assert_array_equal(st, st2)
    parts = O.split_state(st, d, dv)
    u = parts["S"] @ parts["m"] - parts["h"]
    assert un[-1] == pytest.approx(np.linalg.norm(u), rel=1e-13)
    # den_t = q_t . u_t, so |den_t| <= |q_t| |u_t|
    assert np.all(np.abs(den) <= np.linalg.norm(q, axis=1) * un * (1 + 1e-12))


def test_state_only_run_equals_serial_state():
    # skipping the readouts (a prefix absorbed into the state) leaves the state bit for bit as the
    # full serial run's, which the matrix form and the decode continuation pin; multi-head, from a
    # given state too
    r = _rng(41)
    q, k, v = r.standard_normal((3, 26, 5)), r.standard_normal((3, 26, 5)), r.standard_normal((3, 26, 4))
    for g in (1.0, 0.9):
        _, _, st = O.serial(q, k, v, g)
        only = O.serial(q, k, v, g, outputs=False)
        np.testing.assert_array_equal(only, st)
        _, _, st_a = O.serial(q[:, :11], k[:, :11], v[:, :11], g)
        _, _, full = O.serial(q[:, 11:], k[:, 11:], v[:, 11:], g, state=st_a)
        np.testing.assert_array_equal(O.serial(q[:, 11:], k[:, 11:], v[:, 11:], g, state=st_a, outputs=False), full)
