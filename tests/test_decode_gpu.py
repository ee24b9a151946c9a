"""GPU parity of hla2_decode_step (through the C ABI) against the fp64 oracle.

The oracle builds each head's state from its own prefix in fp64; the state is
rounded once to fp32 and both sides continue from that same fp32 state, so the
comparison isolates the decode step.  Outputs of every step and the final
state are compared.  The decode workload itself (all 256 x 32 heads) is in
test_workloads_gpu.py.
"""
import numpy as np
import pytest
import torch

from causal_prefix_scan_hla2_amd import hla2 as H
from causal_prefix_scan_hla2_amd import inputs as I
from oracle import oracle as O
from tests.parity import ratio_ok, ratio_report, rel_l2, tol_for

pytestmark = pytest.mark.gpu


def oracle_prefix_state(w, heads, length):
    """fp64 states after each listed head's prefix (oracle), rounded to fp32."""
    sts = []
    for (s, h) in heads:
        q, k, v = I.decode_prefix_tokens(w, s, h, length)
        _, _, st = O.serial(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.decay)
        sts.append(st)
    return np.stack(sts).astype(np.float32)


def run_steps(w, N, H_, steps, state_gpu, heads):
    """Run `steps` GPU decode steps; return outputs at the listed heads and the
    step tokens of those heads (CPU)."""
    dev = torch.device("cuda:0")
    outs, toks = [], []
    idx = tuple(torch.as_tensor(x) for x in np.array(heads).T)
    for s in range(steps):
        q, k, v = I.decode_step_tokens(w, s, N, H_)
        out = torch.empty(N, H_, w.dv, dtype=q.dtype, device=dev)
        H.hla2_decode_step(state_gpu, q.to(dev), k.to(dev), v.to(dev), out, decay=w.decay, normalize=w.normalize)
        outs.append(out[idx].double().cpu().numpy())
        toks.append((q[idx], k[idx], v[idx]))
    torch.cuda.synchronize()
    return np.stack(outs, 1), toks


def check(w, N, H_, steps, prefix, heads, fill_others=True):
    dev = torch.device("cuda:0")
    L = H.hla2_state_floats(w.d, w.dv)
    st0 = oracle_prefix_state(w, heads, prefix)
    state = torch.zeros(N, H_, L, dtype=torch.float32)
    if fill_others:  # other heads: any valid state (a short oracle prefix of head 0's tokens)
        state[:] = torch.from_numpy(oracle_prefix_state(w, [(0, 0)], 8)[0])
    for i, (s, h) in enumerate(heads):
        state[s, h] = torch.from_numpy(st0[i])
    sg = state.to(dev)
    o_gpu, toks = run_steps(w, N, H_, steps, sg, heads)
    st_gpu = sg[tuple(torch.as_tensor(x) for x in np.array(heads).T)].double().cpu().numpy()
    # oracle continues from the same fp32 state
    q = torch.stack([t[0] for t in toks], 1).double().numpy()
    k = torch.stack([t[1] for t in toks], 1).double().numpy()
    v = torch.stack([t[2] for t in toks], 1).double().numpy()
    num, den, un, st = O.serial_unorm(q, k, v, w.decay, state=st0.astype(np.float64))
    tol = tol_for(w.dtype)
    r_state = rel_l2(st_gpu, st)
    if w.normalize:
        rep = ratio_report(o_gpu, np.zeros_like(den), num, den, un, q)
        msg = "e_max %.3g e_rms %.3g | ratio(well) %.3g excluded %.3f | state %.3g" % (
            rep["e_max"], rep["e_rms"], rep["ratio_well"], rep["excluded"], r_state)
        ok = ratio_ok(rep, tol, subset=True)
    else:
        r_o = rel_l2(o_gpu, num)
        msg = "out %.3g state %.3g" % (r_o, r_state)
        ok = r_o <= tol
    print(msg)
    assert ok, msg
    assert r_state <= 1e-5, msg  # the state stays fp32 end to end
    return msg


@pytest.mark.parametrize("d,dv", [(16, 16), (32, 64), (64, 64), (64, 128), (128, 128), (128, 16)])
@pytest.mark.parametrize("decay,norm", [(1.0, True), (0.9, False)])
def test_small(d, dv, decay, norm):
    w = I.DecodeWorkload("case", 2, 3, d, dv, 40, 6, decay, norm)
    heads = [(0, 0), (1, 2), (0, 1)]
    check(w, 2, 3, 6, 40, heads)


def test_fp32_tokens():
    w = I.DecodeWorkload("case", 1, 2, 64, 64, 30, 5, 0.95, True, dtype="f32")
    check(w, 1, 2, 5, 30, [(0, 0), (0, 1)])


def test_decode_from_zero_matches_oracle_sequence():
    # starting from the zero state, n decode steps are the serial recurrence
    w = I.DecodeWorkload("case", 1, 2, 64, 64, 0, 40, 1.0, False)
    dev = torch.device("cuda:0")
    L = H.hla2_state_floats(64, 64)
    sg = torch.zeros(1, 2, L, dtype=torch.float32, device=dev)
    heads = [(0, 0), (0, 1)]
    o_gpu, toks = run_steps(w, 1, 2, 40, sg, heads)
    q = torch.stack([t[0] for t in toks], 1).double().numpy()
    k = torch.stack([t[1] for t in toks], 1).double().numpy()
    v = torch.stack([t[2] for t in toks], 1).double().numpy()
    num, _, _ = O.serial(q, k, v, 1.0)
    assert rel_l2(o_gpu, num) <= 2e-2
