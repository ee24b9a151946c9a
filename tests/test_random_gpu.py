"""Seeded random shapes through every forward variant and the backward, against the fp64 oracle.

The fixed cases elsewhere cover each plan and edge on purpose; these draw the head sizes (every
multiple of 16 up to 128; d <= 64 for AHLA and the third order), value widths, lengths (ragged,
single-token, one off a chunk), decays, the ratio and forced segment counts at random from a fixed
seed, so that combinations nobody listed are exercised too.  Criteria as for the small fixed cases:
num and den rel-L2 <= tol; under the ratio, the RMS of e_t <= tol / 2 (the rel-L2 of o over the
well-conditioned tokens is printed: a few tokens of a small random head can sit just above the
conditioning cut-off).  Backward calls under the ratio keep n > 1: with a single token the output
is v exactly, and the gradients with respect to q and k vanish.
"""
import random

import numpy as np
import pytest
import torch

from causal_prefix_scan_hla2_amd import hla2 as H
from causal_prefix_scan_hla2_amd import inputs as I
from oracle import oracle as O
from tests.parity import ratio_ok, ratio_report, rel_l2, tol_for

pytestmark = pytest.mark.gpu


def _cases(seed=20261203, count=48):
    rng = random.Random(seed)
    out = []
    for i in range(count):
        kind = rng.choice(["fwd", "fwd", "fwd", "ahla", "ho3", "bwd", "bwd"])
        d = rng.choice([16, 32, 48, 64, 80, 96, 112, 128]) if kind in ("fwd", "bwd") else rng.choice([16, 32, 48, 64])
        dv = rng.choice([16, 32, 48, 64, 80, 96, 112, 128])
        B, H_ = rng.choice([1, 2]), rng.choice([1, 2, 3])
        norm = rng.choice([False, True])
        lengths = [1, 63, 64, 65, 200, 777, 1000, 1500, 2100] if kind != "bwd" else [63, 65, 200, 777, 1000]
        if kind == "bwd" and not norm:
            lengths = [1] + lengths
        n = rng.choice(lengths)
        decay = rng.choice([1.0, 0.999, 0.99, 0.95, 0.9])
        seg = rng.choice([0, 0, 1, 2, 3, 5])
        out.append((i, kind, B, H_, n, d, dv, decay, norm, seg))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%d-%s-%s" % (c[0], c[1], "-".join(str(x) for x in c[2:])))
def test_random_case(case):
    i, kind, B, H_, n, d, dv, decay, norm, seg = case
    print("case", case, flush=True)
    dev = torch.device("cuda:0")
    w = I.Workload("rand", B, H_, n, d, dv, "bf16", decay, norm, 64, seed=1000 + i)
    q, k, v = I.make_qkv(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    qn, kn, vn = q.double().numpy(), k.double().numpy(), v.double().numpy()
    tol = tol_for("bf16")
    if kind == "bwd":
        g = torch.Generator().manual_seed(2000 + i)
        dout = torch.randn(B, H_, n, dv, generator=g).to(q.dtype)
        out = den = None
        if norm:
            num, dn, _ = O.serial(qn, kn, vn, decay)
            out = torch.from_numpy(O.ratio(num, dn)).to(q.dtype)
            den = torch.from_numpy(dn).float()
        dq, dk, dvv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        H.hla2_backward(qd, kd, vd, dout.to(dev), dq, dk, dvv, decay=decay, normalize=norm,
                        out=None if out is None else out.to(dev), den=None if den is None else den.to(dev),
                        segments=seg)
        torch.cuda.synchronize()
        ref = O.backward(qn, kn, vn, dout.double().numpy(), decay, norm,
                         out=None if out is None else out.double().numpy(),
                         den=None if den is None else den.double().numpy())
        errs = [rel_l2(x.double().cpu().numpy(), r) for x, r in zip((dq, dk, dvv), ref)]
        print("dq %.3g dk %.3g dv %.3g" % tuple(errs))
        assert all(e <= tol for e in errs), errs
        return
    fwd = {"fwd": H.hla2_forward, "ahla": H.hla2_ahla_forward, "ho3": H.hla2_ho3_forward}[kind]
    oracle = {"fwd": O.serial_unorm, "ahla": O.ahla_serial_unorm, "ho3": O.ho3_serial_unorm}[kind]
    out = torch.empty_like(vd)
    num_out = torch.empty_like(vd)
    den = torch.empty(B, H_, n, dtype=torch.float32, device=dev)
    fwd(qd, kd, vd, out, decay=decay, normalize=norm, den_out=den, segments=seg)
    fwd(qd, kd, vd, num_out, decay=decay, normalize=False, segments=seg)
    torch.cuda.synchronize()
    num, dn, un, _ = oracle(qn, kn, vn, decay)
    o, dg, ng = (x.double().cpu().numpy() for x in (out, den, num_out))
    r_num, r_den = rel_l2(ng, num), rel_l2(dg, dn)
    msg = "num %.3g den %.3g" % (r_num, r_den)
    assert np.isfinite(o).all(), msg
    assert r_num <= tol and r_den <= tol, msg
    if norm:
        rep = ratio_report(o, dg, num, dn, un, qn)
        msg += " e_rms %.3g ratio(well) %.3g excluded %.3f" % (rep["e_rms"], rep["ratio_well"], rep["excluded"])
        assert ratio_ok(rep, tol), msg
    else:
        assert rel_l2(o, num) <= tol, msg
    print(msg)
