"""ctypes front end of the fp64 HLA2 oracle (``hla2_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module; the GPU library and its
Python binding never do, and this module imports nothing from them.

Every function takes numpy arrays (any float dtype; they are converted to
float64 C-contiguous copies) and returns float64 arrays.  Leading dimensions
before (n, d) are independent heads; they are spread over a thread pool (the C
calls release the GIL), one head per task, each head computed serially.

What the C code computes, and the page passages it follows, is written out in
the header of ``hla2_oracle.c``.  ``backward`` (numpy, the chain rule through the
definition in matrix form) and ``backward_serial`` (C, the adjoint of the serial
recurrence) give the gradients; the pages print none, so both are derived here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hla2_oracle.c")
_LIB = os.path.join(_HERE, "libhla2_oracle.so")
_lock = threading.Lock()
_libs: dict = {}

_dp = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (strict IEEE double, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load(path: str | None = None):
    """The oracle library (built on first use), or another build of the same
    source at `path` (the tests load deliberately broken builds this way)."""
    key = path or _LIB
    with _lock:
        lib = _libs.get(key)
        if lib is None:
            if path is None:
                build()
            lib = ctypes.CDLL(key)
            i, d_ = ctypes.c_int, ctypes.c_double
            lib.hla2_oracle_state_len.restype = ctypes.c_long
            lib.hla2_oracle_state_len.argtypes = [i, i]
            lib.hla2_oracle_summary_len.restype = ctypes.c_long
            lib.hla2_oracle_summary_len.argtypes = [i, i]
            lib.hla2_oracle_step.restype = None
            lib.hla2_oracle_step.argtypes = [i, i, d_, _dp, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_serial.restype = i
            lib.hla2_oracle_serial.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_serial_unorm.restype = i
            lib.hla2_oracle_serial_unorm.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_bruteforce.restype = i
            lib.hla2_oracle_bruteforce.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_segment_summary.restype = None
            lib.hla2_oracle_segment_summary.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_identity.restype = None
            lib.hla2_oracle_identity.argtypes = [i, i, _dp]
            lib.hla2_oracle_combine.restype = None
            lib.hla2_oracle_combine.argtypes = [i, i, _dp, _dp, _dp]
            lib.hla2_oracle_exclusive_scan.restype = i
            lib.hla2_oracle_exclusive_scan.argtypes = [i, i, i, _dp]
            lib.hla2_oracle_chunked.restype = i
            lib.hla2_oracle_chunked.argtypes = [i, i, i, d_, i, _dp, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_ahla_state_len.restype = ctypes.c_long
            lib.hla2_oracle_ahla_state_len.argtypes = [i, i]
            lib.hla2_oracle_ahla_summary_len.restype = ctypes.c_long
            lib.hla2_oracle_ahla_summary_len.argtypes = [i, i]
            lib.hla2_oracle_ahla_serial.restype = i
            lib.hla2_oracle_ahla_serial.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_ahla_serial_unorm.restype = i
            lib.hla2_oracle_ahla_serial_unorm.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_ho3_serial_unorm.restype = i
            lib.hla2_oracle_ho3_serial_unorm.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_ahla_bruteforce.restype = i
            lib.hla2_oracle_ahla_bruteforce.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_ahla_summary.restype = None
            lib.hla2_oracle_ahla_summary.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_ahla_combine.restype = None
            lib.hla2_oracle_ahla_combine.argtypes = [i, i, _dp, _dp, _dp]
            lib.hla2_oracle_ho3_state_len.restype = ctypes.c_long
            lib.hla2_oracle_ho3_state_len.argtypes = [i, i]
            lib.hla2_oracle_ho3_summary_len.restype = ctypes.c_long
            lib.hla2_oracle_ho3_summary_len.argtypes = [i, i]
            lib.hla2_oracle_ho3_serial.restype = i
            lib.hla2_oracle_ho3_serial.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_ho3_bruteforce.restype = i
            lib.hla2_oracle_ho3_bruteforce.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_ho3_summary.restype = None
            lib.hla2_oracle_ho3_summary.argtypes = [i, i, i, d_, _dp, _dp, _dp, _dp]
            lib.hla2_oracle_ho3_apply.restype = None
            lib.hla2_oracle_ho3_apply.argtypes = [i, i, _dp, _dp]
            lib.hla2_oracle_backward_serial.restype = i
            lib.hla2_oracle_backward_serial.argtypes = [i, i, i, d_, i, _dp, _dp, _dp, _dp, _dp, _dp, _dp,
                                                        _dp, _dp]
            _libs[key] = lib
    return lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def state_len(d: int, dv: int, lib=None) -> int:
    return int((lib or _load()).hla2_oracle_state_len(d, dv))


def summary_len(d: int, dv: int, lib=None) -> int:
    return int((lib or _load()).hla2_oracle_summary_len(d, dv))


def split_state(state: np.ndarray, d: int, dv: int) -> dict:
    """Views of S, C, m, G, h inside a state block (last axis = state_len)."""
    o = 0
    out = {}
    for name, shape in (("S", (d, d)), ("C", (d, dv)), ("m", (d,)), ("G", (d, dv)), ("h", (d,))):
        size = int(np.prod(shape))
        out[name] = state[..., o:o + size].reshape(state.shape[:-1] + shape)
        o += size
    return out


def default_threads() -> int:
    env = os.environ.get("HLA2_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _run_heads(fn, count: int, threads: int | None):
    threads = default_threads() if threads is None else max(1, threads)
    if threads == 1 or count <= 1:
        for h in range(count):
            fn(h)
        return
    with ThreadPoolExecutor(max_workers=min(threads, count)) as ex:
        list(ex.map(fn, range(count)))


def serial(q, k, v, gamma: float = 1.0, state=None, threads: int | None = None, lib=None, outputs: bool = True):
    """Serial recurrence over every head.

    q, k: [..., n, d]; v: [..., n, dv]; state: optional [..., state_len] initial
    state.  Returns (num [..., n, dv], den [..., n], final_state [..., state_len]).
    With outputs=False the readouts are skipped and only final_state is
    returned (the same state, bit for bit: the readout does not touch it).
    """
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, n, d = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and tuple(v.shape[:-1]) == tuple(q.shape[:-1])
    H = int(np.prod(lead)) if lead else 1
    qh, kh, vh = q.reshape(H, n, d), k.reshape(H, n, d), v.reshape(H, n, dv)
    L = state_len(d, dv, lib)
    st = np.zeros((H, L)) if state is None else _f64(state).reshape(H, L).copy()
    if not outputs:
        def only_state(h):
            rc = lib.hla2_oracle_serial(n, d, dv, float(gamma), _p(qh[h]), _p(kh[h]), _p(vh[h]), None, None,
                                        _p(st[h]))
            assert rc == 0

        _run_heads(only_state, H, threads)
        return st.reshape(*lead, L)
    num = np.empty((H, n, dv))
    den = np.empty((H, n))

    def one(h):
        rc = lib.hla2_oracle_serial(n, d, dv, float(gamma), _p(qh[h]), _p(kh[h]), _p(vh[h]),
                                    _p(num[h]), _p(den[h]), _p(st[h]))
        assert rc == 0

    _run_heads(one, H, threads)
    return (num.reshape(*lead, n, dv), den.reshape(*lead, n), st.reshape(*lead, L))


def serial_unorm(q, k, v, gamma: float = 1.0, state=None, threads: int | None = None, lib=None):
    """Like serial(), plus |S_t m_t - h_t| per token.

    Returns (num, den, unorm [..., n], final_state)."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, n, d = q.shape
    dv = v.shape[-1]
    H = int(np.prod(lead)) if lead else 1
    qh, kh, vh = q.reshape(H, n, d), k.reshape(H, n, d), v.reshape(H, n, dv)
    L = state_len(d, dv, lib)
    st = np.zeros((H, L)) if state is None else _f64(state).reshape(H, L).copy()
    num = np.empty((H, n, dv))
    den = np.empty((H, n))
    un = np.empty((H, n))

    def one(h):
        assert lib.hla2_oracle_serial_unorm(n, d, dv, float(gamma), _p(qh[h]), _p(kh[h]), _p(vh[h]),
                                            _p(num[h]), _p(den[h]), _p(un[h]), _p(st[h])) == 0

    _run_heads(one, H, threads)
    lt = tuple(lead)
    return num.reshape(lt + (n, dv)), den.reshape(lt + (n,)), un.reshape(lt + (n,)), st.reshape(lt + (L,))


def step(state, q, k, v, gamma: float = 1.0, lib=None):
    """One decode step for every head.  state: [..., state_len] (copied);
    q, k: [..., d]; v: [..., dv].  Returns (num, den, new_state)."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, d = q.shape
    dv = v.shape[-1]
    H = int(np.prod(lead)) if lead else 1
    L = state_len(d, dv, lib)
    st = _f64(state).reshape(H, L).copy()
    qh, kh, vh = q.reshape(H, d), k.reshape(H, d), v.reshape(H, dv)
    num = np.empty((H, dv))
    den = np.empty((H,))
    for h in range(H):
        dd = ctypes.c_double(0.0)
        lib.hla2_oracle_step(d, dv, float(gamma), _p(st[h]), _p(qh[h]), _p(kh[h]), _p(vh[h]),
                             _p(num[h]), ctypes.byref(dd))
        den[h] = dd.value
    return num.reshape(tuple(lead) + (dv,)), den.reshape(tuple(lead)), st.reshape(tuple(lead) + (L,))


def bruteforce(q, k, v, gamma: float = 1.0, threads: int | None = None, lib=None):
    """Definition-level triple sum (small n).  Returns (num, den)."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, n, d = q.shape
    dv = v.shape[-1]
    H = int(np.prod(lead)) if lead else 1
    qh, kh, vh = q.reshape(H, n, d), k.reshape(H, n, d), v.reshape(H, n, dv)
    num = np.empty((H, n, dv))
    den = np.empty((H, n))

    def one(h):
        assert lib.hla2_oracle_bruteforce(n, d, dv, float(gamma), _p(qh[h]), _p(kh[h]), _p(vh[h]),
                                          _p(num[h]), _p(den[h])) == 0

    _run_heads(one, H, threads)
    return num.reshape(*lead, n, dv), den.reshape(*lead, n)


def chunked(q, k, v, gamma: float = 1.0, chunk: int = 16, threads: int | None = None, lib=None):
    """Chunk summaries + exclusive Blelloch scan + chunk outputs.
    Returns (num, den, final_state)."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, n, d = q.shape
    dv = v.shape[-1]
    H = int(np.prod(lead)) if lead else 1
    qh, kh, vh = q.reshape(H, n, d), k.reshape(H, n, d), v.reshape(H, n, dv)
    L = state_len(d, dv, lib)
    num = np.empty((H, n, dv))
    den = np.empty((H, n))
    st = np.empty((H, L))

    def one(h):
        assert lib.hla2_oracle_chunked(n, d, dv, float(gamma), int(chunk), _p(qh[h]), _p(kh[h]),
                                       _p(vh[h]), _p(num[h]), _p(den[h]), _p(st[h])) == 0

    _run_heads(one, H, threads)
    return num.reshape(*lead, n, dv), den.reshape(*lead, n), st.reshape(*lead, L)


def segment_summary(q, k, v, gamma: float = 1.0, lib=None):
    """Summary (Gamma, S, C, m, G, h) of one segment; q,k: [len, d], v: [len, dv]."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    dv = v.shape[-1]
    out = np.empty(summary_len(d, dv, lib))
    lib.hla2_oracle_segment_summary(n, d, dv, float(gamma), _p(q), _p(k), _p(v), _p(out))
    return out


def identity(d: int, dv: int, lib=None):
    lib = lib or _load()
    out = np.empty(summary_len(d, dv, lib))
    lib.hla2_oracle_identity(d, dv, _p(out))
    return out


def combine(a, b, d: int, dv: int, lib=None):
    """a then b (a is the earlier segment)."""
    lib = lib or _load()
    a, b = _f64(a), _f64(b)
    out = np.empty(summary_len(d, dv, lib))
    lib.hla2_oracle_combine(d, dv, _p(a), _p(b), _p(out))
    return out


def exclusive_scan(sums, d: int, dv: int, lib=None):
    """Exclusive Blelloch scan of a [count, summary_len] array (copied)."""
    lib = lib or _load()
    s = _f64(sums).copy()
    assert lib.hla2_oracle_exclusive_scan(d, dv, s.shape[0], _p(s)) == 0
    return s


def ratio(num, den):
    """o = num / den with IEEE semantics (no epsilon)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.asarray(num) / np.asarray(den)[..., None]


def _upstream(dout, gamma, normalize, out, den, q, k, v, lib):
    """out and den for the ratio's upstream gradient: the ones given, else the forward's."""
    if not normalize:
        return None, None
    if out is None or den is None:
        num, den_, _ = serial(q, k, v, gamma, lib=lib)
        out = ratio(num, den_) if out is None else out
        den = den_ if den is None else den
    return _f64(out), _f64(den)


def backward(q, k, v, dout, gamma: float = 1.0, normalize: bool = False, out=None, den=None,
             threads: int | None = None):
    """Gradients (dq, dk, dv) of L = sum(dout * o) by the chain rule through the
    definition, in matrix form, per head (memory and time grow as n^2 and n^3:
    for small n only).

    Forward, as defined for the oracle (0-based t, lower triangles include the
    diagonal): A = L o (Q K^T), D[t, i] = gamma^(t - i) for t >= i (else 0),
    A_g = D o A, M = D o L o (A_g A^T), num = M V, den = M 1, o = num or num / den.
    Backward of a loss with upstream g_num, g_den (g_num = dout, g_den = 0
    unnormalised; g_num = dout / den, g_den = -(dout . out) / den for the ratio,
    with out and den the forward's outputs, given or computed here):
        dV = M^T g_num,   dM = L o (g_num V^T + g_den 1^T),   P = D o dM,
        dA_g = P A,       dA = P^T A_g + D o dA_g,            dX = L o dA,
        dQ = dX K,        dK = dX^T Q            (X = Q K^T, the raw scores).
    The pages print no backward formulas; this is the definition's chain rule.
    """
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    out, den = _upstream(dout, gamma, normalize, out, den, q, k, v, lib)
    *lead, n, d = q.shape
    dv = v.shape[-1]
    H = int(np.prod(lead)) if lead else 1
    qh, kh, vh, gh = q.reshape(H, n, d), k.reshape(H, n, d), v.reshape(H, n, dv), dout.reshape(H, n, dv)
    oh = out.reshape(H, n, dv) if normalize else None
    dh = den.reshape(H, n) if normalize else None
    t = np.arange(n)
    lower = t[:, None] >= t[None, :]
    D = np.where(lower, float(gamma) ** np.maximum(t[:, None] - t[None, :], 0), 0.0)
    dq, dk, dvv = np.empty((H, n, d)), np.empty((H, n, d)), np.empty((H, n, dv))

    def one(h):
        Q, K, V, G = qh[h], kh[h], vh[h], gh[h]
        A = np.where(lower, Q @ K.T, 0.0)
        Ag = D * A
        M = D * np.where(lower, Ag @ A.T, 0.0)
        if normalize:
            gnum = G / dh[h][:, None]
            gden = -np.sum(G * oh[h], axis=-1) / dh[h]
        else:
            gnum, gden = G, np.zeros(n)
        dvv[h] = M.T @ gnum
        dM = np.where(lower, gnum @ V.T + gden[:, None], 0.0)
        P = D * dM
        dAg = P @ A
        dA = P.T @ Ag + D * dAg
        dX = np.where(lower, dA, 0.0)
        dq[h] = dX @ K
        dk[h] = dX.T @ Q

    _run_heads(one, H, threads)
    lt = tuple(lead)
    return dq.reshape(lt + (n, d)), dk.reshape(lt + (n, d)), dvv.reshape(lt + (n, dv))


def backward_serial(q, k, v, dout, gamma: float = 1.0, normalize: bool = False, out=None, den=None,
                    threads: int | None = None, lib=None):
    """Gradients (dq, dk, dv) of L = sum(dout * o) by the adjoint of the serial
    recurrence (``hla2_oracle_backward_serial``): O(n (d^2 + d dv)) per head, for
    any n.  out and den as for ``backward``."""
    lib = lib or _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    out, den = _upstream(dout, gamma, normalize, out, den, q, k, v, lib)
    *lead, n, d = q.shape
    dv = v.shape[-1]
    H = int(np.prod(lead)) if lead else 1
    qh, kh, vh, gh = q.reshape(H, n, d), k.reshape(H, n, d), v.reshape(H, n, dv), dout.reshape(H, n, dv)
    oh = np.ascontiguousarray(out.reshape(H, n, dv)) if normalize else None
    dh = np.ascontiguousarray(den.reshape(H, n)) if normalize else None
    dq, dk, dvv = np.empty((H, n, d)), np.empty((H, n, d)), np.empty((H, n, dv))

    def one(h):
        rc = lib.hla2_oracle_backward_serial(n, d, dv, float(gamma), int(bool(normalize)), _p(qh[h]), _p(kh[h]),
                                             _p(vh[h]), _p(gh[h]), _p(oh[h]) if normalize else None,
                                             _p(dh[h]) if normalize else None, _p(dq[h]), _p(dk[h]), _p(dvv[h]))
        assert rc == 0

    _run_heads(one, H, threads)
    lt = tuple(lead)
    return dq.reshape(lt + (n, d)), dk.reshape(lt + (n, d)), dvv.reshape(lt + (n, dv))


# ---------------------------------------------------------------------------
# AHLA, the asymmetric variant (see the AHLA section of hla2_oracle.c).

def ahla_state_len(d: int, dv: int, lib=None) -> int:
    return int((lib or _load()).hla2_oracle_ahla_state_len(d, dv))


def ahla_summary_len(d: int, dv: int, lib=None) -> int:
    return int((lib or _load()).hla2_oracle_ahla_summary_len(d, dv))


def ahla_serial(q, k, v, gamma: float = 1.0, state=None, threads: int | None = None, lib=None):
    """AHLA serial recurrence over every head.  Returns (num, den, final_state);
    state: optional [..., ahla_state_len] initial state (P | m | E | n)."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, n, d = q.shape
    dv = v.shape[-1]
    H = int(np.prod(lead)) if lead else 1
    qh, kh, vh = q.reshape(H, n, d), k.reshape(H, n, d), v.reshape(H, n, dv)
    L = ahla_state_len(d, dv, lib)
    st = np.zeros((H, L)) if state is None else _f64(state).reshape(H, L).copy()
    num = np.empty((H, n, dv))
    den = np.empty((H, n))

    def one(h):
        assert lib.hla2_oracle_ahla_serial(n, d, dv, float(gamma), _p(qh[h]), _p(kh[h]), _p(vh[h]), _p(num[h]),
                                           _p(den[h]), _p(st[h])) == 0

    _run_heads(one, H, threads)
    lt = tuple(lead)
    return num.reshape(lt + (n, dv)), den.reshape(lt + (n,)), st.reshape(lt + (L,))


def ahla_bruteforce(q, k, v, gamma: float = 1.0, lib=None):
    """AHLA definition as a triple sum, one head (small n).  Returns (num, den)."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    dv = v.shape[-1]
    num, den = np.empty((n, dv)), np.empty(n)
    assert lib.hla2_oracle_ahla_bruteforce(n, d, dv, float(gamma), _p(q), _p(k), _p(v), _p(num), _p(den)) == 0
    return num, den


def ahla_summary(q, k, v, gamma: float = 1.0, lib=None):
    """(Gamma, P, m, E, n, M) of one run of tokens; q, k: [len, d], v: [len, dv]."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    dv = v.shape[-1]
    out = np.empty(ahla_summary_len(d, dv, lib))
    lib.hla2_oracle_ahla_summary(n, d, dv, float(gamma), _p(q), _p(k), _p(v), _p(out))
    return out


def ahla_combine(a, b, d: int, dv: int, lib=None):
    """a then b (a is the earlier segment)."""
    lib = lib or _load()
    a, b = _f64(a), _f64(b)
    out = np.empty(ahla_summary_len(d, dv, lib))
    lib.hla2_oracle_ahla_combine(d, dv, _p(a), _p(b), _p(out))
    return out


# ---------------------------------------------------------------------------
# Third-order HLA (see the third-order section of hla2_oracle.c).

def ho3_state_len(d: int, dv: int, lib=None) -> int:
    return int((lib or _load()).hla2_oracle_ho3_state_len(d, dv))


def ho3_summary_len(d: int, dv: int, lib=None) -> int:
    return int((lib or _load()).hla2_oracle_ho3_summary_len(d, dv))


def ho3_serial(q, k, v, gamma: float = 1.0, state=None, threads: int | None = None, lib=None):
    """Third-order serial recurrence over every head.  Returns (num, den, final_state);
    state: optional [..., ho3_state_len] initial state (S | P' | W')."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, n, d = q.shape
    dv = v.shape[-1]
    H = int(np.prod(lead)) if lead else 1
    qh, kh, vh = q.reshape(H, n, d), k.reshape(H, n, d), v.reshape(H, n, dv)
    L = ho3_state_len(d, dv, lib)
    st = np.zeros((H, L)) if state is None else _f64(state).reshape(H, L).copy()
    num = np.empty((H, n, dv))
    den = np.empty((H, n))

    def one(h):
        assert lib.hla2_oracle_ho3_serial(n, d, dv, float(gamma), _p(qh[h]), _p(kh[h]), _p(vh[h]), _p(num[h]),
                                          _p(den[h]), _p(st[h])) == 0

    _run_heads(one, H, threads)
    lt = tuple(lead)
    return num.reshape(lt + (n, dv)), den.reshape(lt + (n,)), st.reshape(lt + (L,))


def ho3_bruteforce(q, k, v, gamma: float = 1.0, lib=None):
    """Third-order definition as a quadruple sum, one head (small n).  Returns (num, den)."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    dv = v.shape[-1]
    num, den = np.empty((n, dv)), np.empty(n)
    assert lib.hla2_oracle_ho3_bruteforce(n, d, dv, float(gamma), _p(q), _p(k), _p(v), _p(num), _p(den)) == 0
    return num, den


def ho3_summary(q, k, v, gamma: float = 1.0, lib=None):
    """(Gamma, S, P', W', Q2, X1, X2) of one run of tokens."""
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    dv = v.shape[-1]
    out = np.empty(ho3_summary_len(d, dv, lib))
    lib.hla2_oracle_ho3_summary(n, d, dv, float(gamma), _p(q), _p(k), _p(v), _p(out))
    return out


def ho3_apply(summary, state, d: int, dv: int, lib=None):
    """The state after a segment, from the state before it and the segment's summary (copied)."""
    lib = lib or _load()
    st = _f64(state).copy()
    lib.hla2_oracle_ho3_apply(d, dv, _p(_f64(summary)), _p(st))
    return st



def _serial_unorm_variant(fn_name, len_fn, q, k, v, gamma, state, threads, lib):
    lib = lib or _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, n, d = q.shape
    dv = v.shape[-1]
    H = int(np.prod(lead)) if lead else 1
    qh, kh, vh = q.reshape(H, n, d), k.reshape(H, n, d), v.reshape(H, n, dv)
    L = len_fn(d, dv, lib)
    st = np.zeros((H, L)) if state is None else _f64(state).reshape(H, L).copy()
    num = np.empty((H, n, dv))
    den = np.empty((H, n))
    un = np.empty((H, n))
    fn = getattr(lib, fn_name)

    def one(h):
        rc = fn(n, d, dv, float(gamma), _p(qh[h]), _p(kh[h]), _p(vh[h]), _p(num[h]), _p(den[h]), _p(un[h]), _p(st[h]))
        assert rc == 0

    _run_heads(one, H, threads)
    return num.reshape(*lead, n, dv), den.reshape(*lead, n), un.reshape(*lead, n), st.reshape(*lead, L)


def ahla_serial_unorm(q, k, v, gamma: float = 1.0, state=None, threads: int | None = None, lib=None):
    """ahla_serial() plus |n_t| per token, the norm of the den column n_t of the state
    (den_t = q_t . n_t).  Returns (num, den, unorm [..., n], final_state)."""
    return _serial_unorm_variant("hla2_oracle_ahla_serial_unorm", ahla_state_len, q, k, v, gamma, state, threads, lib)


def ho3_serial_unorm(q, k, v, gamma: float = 1.0, state=None, threads: int | None = None, lib=None):
    """ho3_serial() plus |w_t| per token, the norm of the den column w_t of the corrected accumulator
    (den_t = q_t . w_t).  Returns (num, den, unorm [..., n], final_state)."""
    return _serial_unorm_variant("hla2_oracle_ho3_serial_unorm", ho3_state_len, q, k, v, gamma, state, threads, lib)
