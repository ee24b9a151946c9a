"""GPU parity of hla2_ho3_forward (third order, through the C ABI) against the
oracle's third-order recurrence.

num and den are compared over all tokens (relative L2 at the forward's bars);
under the ratio, the conditioning-normalised error e_t is bounded as for the
second-order forward (its RMS at half the tolerance), with the conditioning
taken from the den column w_t of the oracle's corrected accumulator
(den_t = q_t . w_t); at the normalised workload's shape o is also compared on
the well-conditioned tokens.
"""
import numpy as np
import pytest
import torch

from causal_prefix_scan_hla2_amd import hla2 as H
from causal_prefix_scan_hla2_amd import inputs as I
from oracle import oracle as O
from tests.parity import (per_row_rel_l2, ratio_ok, ratio_report, ratio_workload_figures, ratio_workload_ok,
                          record, rel_l2, tol_for)

pytestmark = pytest.mark.gpu


def draw(B, H_, n, d, dv, dtype, seed):
    w = I.Workload("ho3", B, H_, n, d, dv, dtype, 1.0, False, 64, seed=seed)
    return I.make_qkv(w)


def gpu_ho3(q, k, v, decay, normalize, segments=0):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(vd)
    den = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    H.hla2_ho3_forward(qd, kd, vd, out, decay=decay, normalize=normalize, den_out=den, segments=segments)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), den.double().cpu().numpy()


def check(q, k, v, decay, normalize, dtype, segments=0, heads=None, subset=False):
    tol = tol_for(dtype)
    o_gpu, den_gpu = gpu_ho3(q, k, v, decay, normalize, segments)
    num_gpu = gpu_ho3(q, k, v, decay, False, segments)[0] if normalize else o_gpu
    if heads is not None:
        idx = tuple(np.array(heads).T)
        tidx = tuple(torch.as_tensor(x) for x in idx)
        q, k, v = q[tidx], k[tidx], v[tidx]
        o_gpu, den_gpu, num_gpu = o_gpu[idx], den_gpu[idx], num_gpu[idx]
    num, den, unorm, _ = O.ho3_serial_unorm(q.double().numpy(), k.double().numpy(), v.double().numpy(), decay)
    r_num, r_den = rel_l2(num_gpu, num), rel_l2(den_gpu, den)
    msg = "num %.3g den %.3g" % (r_num, r_den)
    ok = r_num <= tol and r_den <= tol
    if normalize:
        rep = ratio_report(o_gpu, den_gpu, num, den, unorm, q.double().numpy())
        msg += " | e_rms %.3g ratio(well) %.3g excluded %.3f" % (rep["e_rms"], rep["ratio_well"], rep["excluded"])
        ok = ok and ratio_ok(rep, tol, subset=subset)
    print(msg)
    assert ok, msg


SMALL = [
    # B, H, n, d, dv, dtype, decay, normalize, segments
    (1, 1, 64, 16, 16, "f32", 1.0, False, 0),
    (2, 3, 200, 32, 48, "f32", 0.9, True, 3),
    (1, 2, 333, 64, 64, "f32", 0.97, False, 0),
    (1, 1, 40, 64, 64, "f32", 0.9, True, 1),
    (2, 3, 300, 64, 128, "bf16", 0.99, False, 0),
    (1, 2, 1000, 64, 128, "bf16", 1.0, True, 4),
    (1, 1, 1000, 64, 128, "bf16", 0.99, False, 7),
    (1, 2, 700, 64, 64, "bf16", 0.98, True, 3),
    (1, 1, 100, 16, 16, "bf16", 1.0, False, 1),
    (1, 1, 200, 48, 80, "bf16", 0.9, True, 2),
    (1, 2, 2048, 64, 64, "bf16", 1.0, True, 0),
    (1, 1, 37, 64, 128, "bf16", 0.9, False, 0),
    # three segments at d = 64: segment 2 folds segment 1's summary in its prologue (ragged tail,
    # decay, with and without the ratio)
    (1, 2, 900, 64, 128, "bf16", 0.95, False, 3),
    (2, 1, 1000, 48, 48, "bf16", 0.9, True, 3),
    # the same without decay, or with a weak one: the folded prefix keeps its weight
    (1, 2, 900, 64, 128, "bf16", 1.0, False, 3),
    (1, 2, 900, 64, 64, "bf16", 1.0, True, 3),
    (2, 1, 1000, 48, 48, "bf16", 0.999, False, 3),
]


# Lead plans (bf16, automatic): segment 0's output walk leaves segment 1's prefix and the scan
# starts there; these shapes give a segment 0 shorter than the others and a ragged tail.
LEAD = [
    # B, H, n, d, dv, decay, normalize, oracle heads (None: all)
    (4, 16, 2900, 64, 128, 0.99, False, [(0, 0), (1, 7), (3, 15)]),
    (4, 16, 2900, 64, 64, 0.98, True, [(0, 5), (2, 10), (3, 1)]),
    (4, 16, 2900, 64, 128, 0.99, True, [(1, 2), (2, 13), (3, 9)]),  # ratio at dv = 128: 32-token chunks
]


@pytest.mark.parametrize("case", LEAD, ids=lambda c: "-".join(str(x) for x in c[:7]))
def test_ho3_lead_plan_cases(case):
    B, H_, n, d, dv, decay, normalize, heads = case
    print("case", case, flush=True)
    q, k, v = draw(B, H_, n, d, dv, "bf16", seed=800 + n + d)
    check(q, k, v, decay, normalize, "bf16", heads=heads)


@pytest.mark.parametrize("B,H_,n,d,dv,dtype,decay,normalize,segments", SMALL)
def test_ho3_matches_oracle(B, H_, n, d, dv, dtype, decay, normalize, segments):
    print("case", B, H_, n, d, dv, dtype, decay, normalize, segments, flush=True)
    q, k, v = draw(B, H_, n, d, dv, dtype, seed=500 + n + d)
    check(q, k, v, decay, normalize, dtype, segments)


def test_ho3_causal_bitwise():
    q, k, v = draw(1, 2, 500, 64, 64, "bf16", seed=3)
    a, ad = gpu_ho3(q, k, v, 0.95, False)
    for tstar in (0, 63, 64, 200, 499):
        q2, k2, v2 = q.clone(), k.clone(), v.clone()
        q2[:, :, tstar:] *= -1
        k2[:, :, tstar:] += 0.25
        v2[:, :, tstar:] *= 2
        b, bd = gpu_ho3(q2, k2, v2, 0.95, False)
        assert np.array_equal(a[:, :, :tstar], b[:, :, :tstar]) and np.array_equal(ad[:, :, :tstar], bd[:, :, :tstar])


def test_ho3_segments_change_rounding_only():
    q, k, v = draw(1, 2, 900, 64, 64, "bf16", seed=4)
    a, _ = gpu_ho3(q, k, v, 0.99, False, 1)
    for seg in (2, 5, 14):
        b, _ = gpu_ho3(q, k, v, 0.99, False, seg)
        assert rel_l2(b, a) < 5e-3


def test_ho3_decay_workload_shape_sampled():
    """The decay workload's shape (B=8, H=16, n=8192, d=64, dv=128, decay 0.99), sampled heads."""
    w = I.WORKLOADS["decay_8k"]
    q, k, v = I.make_qkv(w)
    check(q, k, v, w.decay, False, w.dtype, heads=I.sample_heads(w.B, w.H, 3))


def test_ho3_norm_workload_all_heads():
    """The normalised workload's shape (B=4, H=8, n=2048, d=dv=64, ratio), every head against the
    oracle: num and den per head, and the ratio criterion per head with the well-conditioned subset."""
    w = I.WORKLOADS["norm_2k"]
    q, k, v = I.make_qkv(w)
    o_gpu, den_gpu = gpu_ho3(q, k, v, w.decay, True)
    num_gpu = gpu_ho3(q, k, v, w.decay, False)[0]
    qn = q.double().numpy()
    num, den, un, _ = O.ho3_serial_unorm(qn, k.double().numpy(), v.double().numpy(), w.decay,
                                        threads=min(16, O.default_threads()))
    fig, msg = ratio_workload_figures(o_gpu, den_gpu, num_gpu, num, den, un, qn)
    record("third_order_norm_2k", **fig)
    print(msg)
    assert ratio_workload_ok(fig, tol_for(w.dtype)), msg


# Without a den buffer and without the ratio the walkers carry no den column (the instantiations the
# benchmark times): the outputs are compared with the oracle's num.
# At d <= 64 and dv > 64 these run on the register-resident walker: one segment, the plain scan
# (five and seven segments), three-segment lead plans whose segment 2 folds segment 1's summary in its
# prologue (with and without decay), an automatic lead plan, padded head sizes, a sequence of one
# partial chunk, one chunk exactly and one token past it.
NODEN = [
    # B, H, n, d, dv, decay, segments, oracle heads (None: all)
    (2, 3, 300, 64, 128, 0.99, 0, None),
    (1, 2, 777, 64, 64, 0.97, 3, None),
    (1, 1, 1000, 64, 128, 1.0, 2, None),
    (1, 1, 200, 48, 80, 0.9, 0, None),
    (1, 2, 900, 64, 128, 0.95, 3, None),
    (1, 2, 900, 64, 128, 0.999, 3, None),
    (1, 2, 900, 64, 128, 1.0, 3, None),
    (2, 1, 1000, 48, 80, 1.0, 3, None),
    (1, 2, 4100, 64, 128, 1.0, 5, None),
    (1, 1, 1000, 32, 112, 0.99, 7, None),
    (4, 16, 1700, 64, 128, 0.97, 0, [(0, 3), (2, 9), (3, 14)]),
    (1, 1, 37, 64, 128, 0.9, 0, None),
    (2, 1, 64, 64, 128, 1.0, 0, None),
    (2, 1, 65, 16, 96, 0.95, 0, None),
]


def gpu_ho3_noden(q, k, v, decay, segments=0):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(vd)
    H.hla2_ho3_forward(qd, kd, vd, out, decay=decay, normalize=False, den_out=None, segments=segments)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


@pytest.mark.parametrize("case", NODEN, ids=lambda c: "-".join(str(x) for x in c[:7]))
def test_ho3_without_den_matches_oracle(case):
    B, H_, n, d, dv, decay, segments, heads = case
    print("case", case, flush=True)
    q, k, v = draw(B, H_, n, d, dv, "bf16", seed=950 + n + d)
    o = gpu_ho3_noden(q, k, v, decay, segments)
    if heads is not None:
        idx = tuple(np.array(heads).T)
        tidx = tuple(torch.as_tensor(x) for x in idx)
        q, k, v, o = q[tidx], k[tidx], v[tidx], o[idx]
    num, _, _ = O.ho3_serial(q.double().numpy(), k.double().numpy(), v.double().numpy(), decay)
    r = rel_l2(o, num)
    print("num %.3g" % r)
    assert r <= tol_for("bf16"), r


def test_ho3_without_den_decay_workload_all_heads():
    """The benchmark's call on the decay workload's shape (no den buffer, no ratio): every head against
    the oracle, with the aggregate and the worst head's rel-L2 each within the bar."""
    w = I.WORKLOADS["decay_8k"]
    q, k, v = I.make_qkv(w)
    o = gpu_ho3_noden(q, k, v, w.decay)
    num, _, _ = O.ho3_serial(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.decay,
                             threads=min(16, O.default_threads()))
    r = rel_l2(o, num)
    head = per_row_rel_l2(o, num, (-2, -1))
    record("ho3_noden_decay_8k", num_rel_l2=r, num_head_max=float(head.max()))
    print("num %.3g, worst head %.3g" % (r, head.max()))
    assert r <= tol_for(w.dtype) and head.max() <= tol_for(w.dtype), (r, head.max())


def test_ho3_without_den_causal_bitwise():
    """Causality of the no-den walker (d <= 64, dv > 64): outputs before t* are bitwise unchanged by any
    change of the tokens from t* on, with a plain plan and with three segments (prologue fold)."""
    q, k, v = draw(1, 2, 700, 64, 128, "bf16", seed=5)
    for segments in (0, 3):
        a = gpu_ho3_noden(q, k, v, 0.97, segments)
        for tstar in (0, 63, 64, 300, 699):
            q2, k2, v2 = q.clone(), k.clone(), v.clone()
            q2[:, :, tstar:] *= -1
            k2[:, :, tstar:] += 0.25
            v2[:, :, tstar:] *= 2
            b = gpu_ho3_noden(q2, k2, v2, 0.97, segments)
            assert np.array_equal(a[:, :, :tstar], b[:, :, :tstar]), (segments, tstar)
