"""GPU parity of hla2_backward (through the C ABI) against the fp64 oracle.

The gradients of sum(dout * out) with respect to q, k, v are compared, tensor
by tensor (relative L2, the same bar as the forward), with the oracle's chain
rule through the definition (small n) or its adjoint of the serial recurrence
(workload sizes, sampled heads).  Under the ratio both sides take the same
out and den (the oracle's forward outputs, rounded to what the GPU receives),
as an autograd function takes its saved tensors.
"""
import numpy as np
import pytest
import torch

from causal_prefix_scan_hla2_amd import hla2 as H
from causal_prefix_scan_hla2_amd import inputs as I
from oracle import oracle as O
from tests.parity import rel_l2, tol_for

pytestmark = pytest.mark.gpu


def draw(B, H_, n, d, dv, dtype, seed):
    w = I.Workload("bwd", B, H_, n, d, dv, dtype, 1.0, False, 64, seed=seed)
    q, k, v = I.make_qkv(w)
    g = torch.Generator().manual_seed(seed + 7)
    dout = torch.randn(B, H_, n, dv, generator=g).to(q.dtype)
    return q, k, v, dout


def forward_saved(q, k, v, decay, normalize):
    """out (element type) and den (fp32) of the forward, from the oracle."""
    if not normalize:
        return None, None
    num, den, _ = O.serial(q.double().numpy(), k.double().numpy(), v.double().numpy(), decay)
    out = torch.from_numpy(O.ratio(num, den)).to(q.dtype)
    return out, torch.from_numpy(den).float()


def gpu_backward(q, k, v, dout, decay, normalize, out, den, segments=0):
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (x.to(dev) for x in (q, k, v, dout))
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    H.hla2_backward(qd, kd, vd, gd, dq, dk, dv, decay=decay, normalize=normalize,
                    out=None if out is None else out.to(dev), den=None if den is None else den.to(dev),
                    segments=segments)
    torch.cuda.synchronize()
    return [x.double().cpu().numpy() for x in (dq, dk, dv)]


def compare(got, ref, tol):
    errs = {name: rel_l2(a, b) for name, a, b in zip(("dq", "dk", "dv"), got, ref)}
    msg = " ".join("%s %.3g" % kv for kv in errs.items())
    print(msg)
    assert all(e <= tol for e in errs.values()), msg
    return errs


SMALL = [
    # B, H, n, d, dv, dtype, decay, normalize, segments
    (1, 1, 64, 16, 16, "f32", 1.0, False, 0),
    (2, 3, 200, 32, 48, "f32", 0.9, True, 3),
    (1, 2, 333, 64, 64, "f32", 0.97, False, 0),
    (1, 1, 40, 64, 64, "f32", 0.9, True, 0),
    (1, 2, 130, 16, 16, "f32", 0.95, False, 2),
    (2, 3, 300, 64, 128, "bf16", 0.99, False, 0),
    (1, 2, 1000, 128, 128, "bf16", 1.0, True, 4),
    (1, 1, 1000, 64, 128, "bf16", 0.99, False, 7),
    (1, 2, 700, 128, 64, "bf16", 0.98, True, 3),
    (1, 1, 100, 16, 16, "bf16", 1.0, False, 1),
    (1, 2, 1024, 64, 64, "bf16", 0.999, True, 0),
    (1, 1, 200, 48, 80, "bf16", 0.9, True, 2),
    (1, 1, 37, 128, 128, "bf16", 0.9, False, 0),
    (1, 2, 777, 64, 128, "bf16", 0.97, True, 3),  # ratio at dv = 128: 32-token chunks
    # two segments with 64-token chunks: segment 0's forward-state walk runs in two halves, the
    # second starting from the first half's summary (with and without decay, with the den column,
    # ragged tails)
    (1, 2, 900, 64, 64, "bf16", 0.99, False, 2),
    (1, 1, 1000, 64, 128, "bf16", 1.0, False, 2),
    (2, 1, 777, 48, 48, "bf16", 0.95, True, 2),
    (1, 1, 1300, 32, 96, "bf16", 0.999, False, 2),
]


@pytest.mark.parametrize("B,H_,n,d,dv,dtype,decay,normalize,segments", SMALL)
def test_backward_matches_oracle(B, H_, n, d, dv, dtype, decay, normalize, segments):
    print("case", B, H_, n, d, dv, dtype, decay, normalize, segments, flush=True)
    q, k, v, dout = draw(B, H_, n, d, dv, dtype, seed=300 + n + d)
    out, den = forward_saved(q, k, v, decay, normalize)
    got = gpu_backward(q, k, v, dout, decay, normalize, out, den, segments)
    ref = O.backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(), decay,
                     normalize, out=None if out is None else out.double().numpy(),
                     den=None if den is None else den.double().numpy())
    compare(got, ref, tol_for(dtype))


def test_backward_segments_change_rounding_only():
    q, k, v, dout = draw(1, 2, 900, 64, 64, "bf16", seed=9)
    a = gpu_backward(q, k, v, dout, 0.99, False, None, None, 1)
    for seg in (2, 5):
        b = gpu_backward(q, k, v, dout, 0.99, False, None, None, seg)
        for x, y in zip(b, a):
            assert rel_l2(x, y) < 5e-3


def test_backward_is_repeatable_and_heads_independent():
    q, k, v, dout = draw(2, 2, 300, 64, 64, "bf16", seed=10)
    a = gpu_backward(q, k, v, dout, 0.95, False, None, None)
    b = gpu_backward(q, k, v, dout, 0.95, False, None, None)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # changing head (1, 1) leaves every other head's gradients bitwise unchanged
    q2 = q.clone()
    q2[1, 1] = -q2[1, 1]
    c = gpu_backward(q2, k, v, dout, 0.95, False, None, None)
    for x, y in zip(a, c):
        assert np.array_equal(x[0], y[0]) and np.array_equal(x[1, 0], y[1, 0])


@pytest.mark.parametrize("wname", ["decay_8k", "norm_2k"])
def test_backward_workload_sampled(wname):
    """The workload's full shape and launch configuration; the oracle's serial
    adjoint recomputes sampled heads in full."""
    w = I.WORKLOADS[wname]
    print("workload", wname, flush=True)
    q, k, v = I.make_qkv(w)
    g = torch.Generator().manual_seed(w.seed + 7)
    dout = torch.randn(w.B, w.H, w.n, w.dv, generator=g).to(q.dtype)
    heads = I.sample_heads(w.B, w.H, 3)
    idx = tuple(torch.as_tensor(x) for x in np.array(heads).T)
    out, den = forward_saved(q, k, v, w.decay, w.normalize)  # the oracle's forward, every head
    got = gpu_backward(q, k, v, dout, w.decay, w.normalize, out, den)
    got = [x[tuple(np.array(heads).T)] for x in got]
    ref = O.backward_serial(q[idx].double().numpy(), k[idx].double().numpy(), v[idx].double().numpy(),
                            dout[idx].double().numpy(), w.decay, w.normalize,
                            out=None if out is None else out[idx].double().numpy(),
                            den=None if den is None else den[idx].double().numpy())
    compare(got, ref, tol_for(w.dtype))


def test_backward_long_head():
    """Two heads of 65,536 tokens (d = dv = 64, bf16, decay 0.999): many segments and a long
    adjoint scan; every gradient is compared with the oracle's serial adjoint."""
    print("case 1 2 65536 64 64 bf16 0.999", flush=True)
    q, k, v, dout = draw(1, 2, 65536, 64, 64, "bf16", seed=88)
    got = gpu_backward(q, k, v, dout, 0.999, False, None, None)
    ref = O.backward_serial(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                            0.999, False)
    compare(got, ref, tol_for("bf16"))
