"""GPU parity at the full sizes of the benchmark workloads, every head compared with the fp64 oracle.

The forward workloads run the exact calls the benchmark times (automatic segment plan; with and
without the den buffer) and compare every head and every token: rel-L2 of num and den over each head
and over each (head, segment) of the plan, besides the aggregate over the workload.  The
ratio-normalised workloads add the ratio criterion per head (RMS of the conditioning-normalised
error) and on the well-conditioned tokens.  The decode workload compares all 256 x 32 heads over its
128 steps and the final state: the oracle runs every head's 4096-token prefix in fp64, the state is
rounded once to fp32, and both sides continue from it.

The figures are kept (tests/parity.py RECORDS) and written to $HLA2_PARITY_DIR at the end of the
session.  The claim under test is the technical summary's scan equivalence (gist.science, §4: the
chunk-parallel activations equal the serial recurrence's) and its exactness claim ("Resultaten en
claims").
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from causal_prefix_scan_hla2_amd import hla2 as H
from causal_prefix_scan_hla2_amd import inputs as I
from oracle import oracle as O
from tests.parity import (per_row_rel_l2, ratio_per_head, ratio_report, record, rel_l2, segment_bounds,
                          tol_for)

pytestmark = pytest.mark.gpu

THREADS = min(16, O.default_threads())  # the GPU machine's CPU share


def say(*a):
    print(*a, flush=True)


def gpu_call(q, k, v, w, normalize, want_den):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(vd)
    den = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev) if want_den else None
    H.hla2_forward(qd, kd, vd, out, decay=w.decay, normalize=normalize, chunk=w.chunk, den_out=den)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    dn = den.double().cpu().numpy() if want_den else None
    del qd, kd, vd, out, den
    return o, dn


_ORACLE = {}


def oracle_of(w):
    """(q, k, v, num, den, unorm) of a workload, the oracle run once per session."""
    if w.name not in _ORACLE:
        q, k, v = I.make_qkv(w)
        say("oracle %s: %d heads x %d tokens on %d threads" % (w.name, w.B * w.H, w.n, THREADS))
        num, den, un, _ = O.serial_unorm(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.decay,
                                         threads=THREADS)
        _ORACLE.clear()  # one workload's arrays at a time
        _ORACLE[w.name] = (q, k, v, num, den, un)
    return _ORACLE[w.name]


def per_head_and_segment(x_gpu, x_ref, segs, tok_axis_vals):
    """Per-head rel-L2 and the largest per-(head, segment) rel-L2 of x (num: [..., n, dv]; den: [..., n])."""
    axes = (-2, -1) if tok_axis_vals else (-1,)
    head = per_row_rel_l2(x_gpu, x_ref, axes)
    seg = []
    for t0, t1 in segs:
        if tok_axis_vals:
            seg.append(per_row_rel_l2(x_gpu[..., t0:t1, :], x_ref[..., t0:t1, :], axes))
        else:
            seg.append(per_row_rel_l2(x_gpu[..., t0:t1], x_ref[..., t0:t1], axes))
    return head, np.max(np.stack(seg), axis=0)


def check_forward_workload(name, w, o_gpu, den_gpu, num_gpu):
    """Every head of a forward workload: num and den per head and per (head, segment), and the ratio
    criterion per head.  `num_gpu` is the unnormalised output (o_gpu itself when not normalised);
    `den_gpu` may be None (the call without the den buffer)."""
    tol = tol_for(w.dtype)
    q, k, v, num, den, un = oracle_of(w)
    if w.dtype == "f32":  # the fp32 path's plan is not the bf16 lead plan the query reports
        nseg, segs = 1, [(0, w.n)]
    else:
        nseg, c0, cs, _ = H.hla2_forward_plan(w.B, w.H, w.n, w.d, w.dv, w.chunk)
        segs = segment_bounds(w.n, nseg, c0, cs)
    fig = {"heads": w.B * w.H, "tokens": w.n, "segments": nseg}
    num_head, num_seg = per_head_and_segment(num_gpu, num, segs, True)
    fig.update(num=rel_l2(num_gpu, num), num_head_max=float(num_head.max()), num_seg_max=float(num_seg.max()),
               num_worst_head=[int(x) for x in np.unravel_index(np.argmax(num_seg), num_seg.shape)])
    msgs = ["num %.3g (head max %.3g, segment max %.3g)" % (fig["num"], fig["num_head_max"], fig["num_seg_max"])]
    if den_gpu is not None:
        den_head, den_seg = per_head_and_segment(den_gpu, den, segs, False)
        fig.update(den=rel_l2(den_gpu, den), den_head_max=float(den_head.max()), den_seg_max=float(den_seg.max()))
        msgs.append("den %.3g (head max %.3g, segment max %.3g)" % (fig["den"], fig["den_head_max"],
                                                                     fig["den_seg_max"]))
    if w.normalize:
        qn = q.double().numpy()
        rep = ratio_report(o_gpu, den_gpu, num, den, un, qn)
        ph = ratio_per_head(o_gpu, num, den, un, qn)
        fig.update(e_rms=rep["e_rms"], e_max=rep["e_max"], ratio_well=rep["ratio_well"], excluded=rep["excluded"],
                   e_rms_head_max=float(ph["e_rms"].max()), e_rms_well_head_max=float(ph["e_rms_well"].max()),
                   ratio_well_head_max=float(ph["ratio_well"].max()), excluded_head_max=float(ph["excluded"].max()))
        msgs.append("e_rms %.3g (head max %.3g, well-conditioned %.3g) e_max %.3g | ratio(well) %.3g (head max %.3g) "
                    "excluded %.3f" % (rep["e_rms"], fig["e_rms_head_max"], fig["e_rms_well_head_max"], rep["e_max"],
                                       rep["ratio_well"], fig["ratio_well_head_max"], rep["excluded"]))
    record(name, **fig)
    msg = "; ".join(msgs)
    say(name, msg)
    assert fig["num"] <= tol and fig["num_seg_max"] <= tol and fig["num_head_max"] <= tol, msg
    if den_gpu is not None:
        assert fig["den"] <= tol and fig["den_seg_max"] <= tol and fig["den_head_max"] <= tol, msg
    if w.normalize:
        # the ratio: e_t's RMS over all tokens of the workload, per head over its well-conditioned
        # tokens, and the rel-L2 of o over the well-conditioned tokens of the workload
        assert fig["e_rms"] <= tol / 2 and fig["e_rms_well_head_max"] <= tol / 2, msg
        assert fig["ratio_well"] <= tol, msg
    return fig


def test_workload_tiny_f32_all():
    w = I.WORKLOADS["tiny_f32"]
    q, k, v = oracle_of(w)[:3]
    o, dn = gpu_call(q, k, v, w, w.normalize, True)
    check_forward_workload("tiny_f32", w, o, dn, o)


def test_workload_norm_2k_all_heads():
    w = I.WORKLOADS["norm_2k"]
    q, k, v = oracle_of(w)[:3]
    o, dn = gpu_call(q, k, v, w, True, True)
    num, _ = gpu_call(q, k, v, w, False, False)
    check_forward_workload("norm_2k", w, o, dn, num)


def test_workload_decay_8k_all_heads():
    """The decay workload with a den buffer (the walkers carry the den state)."""
    w = I.WORKLOADS["decay_8k"]
    q, k, v = oracle_of(w)[:3]
    o, dn = gpu_call(q, k, v, w, w.normalize, True)
    check_forward_workload("decay_8k (den buffer)", w, o, dn, o)


def test_workload_decay_8k_benchmark_call_all_heads():
    """The exact call the benchmark times: no den buffer (the instantiation without the den state),
    every head against the oracle, and bitwise equal to the same call repeated."""
    w = I.WORKLOADS["decay_8k"]
    q, k, v = oracle_of(w)[:3]
    o, _ = gpu_call(q, k, v, w, w.normalize, False)
    o2, _ = gpu_call(q, k, v, w, w.normalize, False)
    np.testing.assert_array_equal(o, o2)
    check_forward_workload("decay_8k (benchmark call)", w, o, None, o)


def test_workload_long_64k_all_heads():
    w = I.WORKLOADS["long_64k"]
    q, k, v = oracle_of(w)[:3]
    o, dn = gpu_call(q, k, v, w, True, True)
    num, _ = gpu_call(q, k, v, w, False, False)
    check_forward_workload("long_64k", w, o, dn, num)


# ---- decode: all 256 x 32 heads, 128 steps, from the oracle's prefix states ----

def oracle_prefix_states(w):
    """fp32 state of every (sequence, head) after its prefix: the fp64 serial recurrence, rounded once
    to fp32 (round to nearest even)."""
    L = O.state_len(w.d, w.dv)
    st = np.empty((w.N, w.H, L), dtype=np.float32)

    def one(i):
        s, h = divmod(i, w.H)
        q, k, v = I.decode_prefix_tokens(w, s, h)
        fs = O.serial(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.decay, threads=1, outputs=False)
        st[s, h] = fs.astype(np.float32)

    total = w.N * w.H
    say("oracle prefill: %d heads x %d tokens on %d threads" % (total, w.prefix, THREADS))
    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        for j, _ in enumerate(ex.map(one, range(total))):
            if (j + 1) % 1024 == 0:
                say("  prefill %d / %d heads" % (j + 1, total))
    return st


def test_workload_decode_256x32_all_heads():
    w = I.DECODE
    tol = tol_for(w.dtype)
    st0 = oracle_prefix_states(w)
    dev = torch.device("cuda:0")
    sa = torch.from_numpy(st0).to(dev)  # ratio-normalised steps (the workload)
    sb = sa.clone()                     # the same steps unnormalised, for num
    o_n, o_u, toks = [], [], []
    for s in range(w.steps):
        q, k, v = I.decode_step_tokens(w, s)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        out_n = torch.empty(w.N, w.H, w.dv, dtype=q.dtype, device=dev)
        out_u = torch.empty_like(out_n)
        H.hla2_decode_step(sa, qd, kd, vd, out_n, decay=w.decay, normalize=True)
        H.hla2_decode_step(sb, qd, kd, vd, out_u, decay=w.decay, normalize=False)
        o_n.append(out_n.cpu())
        o_u.append(out_u.cpu())
        toks.append((q, k, v))
    torch.cuda.synchronize()
    say("decode: %d GPU steps done" % w.steps)
    st_a, st_b = sa.cpu().numpy(), sb.cpu().numpy()
    np.testing.assert_array_equal(st_a, st_b)  # the ratio does not touch the state
    o_gpu = torch.stack(o_n, 2).double().numpy()   # [N, H, steps, dv]
    num_gpu = torch.stack(o_u, 2).double().numpy()
    q = torch.stack([t[0] for t in toks], 2).double().numpy()
    k = torch.stack([t[1] for t in toks], 2).double().numpy()
    v = torch.stack([t[2] for t in toks], 2).double().numpy()
    num, den, un, st = O.serial_unorm(q, k, v, w.decay, state=st0.astype(np.float64), threads=THREADS)
    num_head = per_row_rel_l2(num_gpu, num, (-2, -1))
    rep = ratio_report(o_gpu, np.zeros_like(den), num, den, un, q)
    ph = ratio_per_head(o_gpu, num, den, un, q)
    st_head = per_row_rel_l2(st_a, st, (-1,))
    pieces = O.split_state(st_a.astype(np.float64), w.d, w.dv)
    pref = O.split_state(st, w.d, w.dv)
    piece_max = {p: float(per_row_rel_l2(pieces[p], pref[p], tuple(range(2, pref[p].ndim))).max())
                 for p in ("S", "C", "m", "G", "h")}
    fig = {"heads": w.N * w.H, "tokens": w.steps, "num": rel_l2(num_gpu, num), "num_head_max": float(num_head.max()),
           "e_rms": rep["e_rms"], "e_max": rep["e_max"], "e_rms_head_max": float(ph["e_rms"].max()),
           "e_rms_well_head_max": float(ph["e_rms_well"].max()),
           "ratio_well": rep["ratio_well"], "ratio_well_head_max": float(ph["ratio_well"].max()),
           "excluded": rep["excluded"], "state": rel_l2(st_a, st), "state_head_max": float(st_head.max()),
           "state_piece_head_max": piece_max}
    record("decode_256x32", **fig)
    msg = ("num %.3g (head max %.3g) | e_rms %.3g (head max %.3g) e_max %.3g | ratio(well) %.3g (head max %.3g) "
           "excluded %.3f | state %.3g (head max %.3g; pieces %s)"
           % (fig["num"], fig["num_head_max"], fig["e_rms"], fig["e_rms_head_max"], fig["e_max"], fig["ratio_well"],
              fig["ratio_well_head_max"], fig["excluded"], fig["state"], fig["state_head_max"],
              ", ".join("%s %.2g" % kv for kv in piece_max.items())))
    say("decode_256x32", msg)
    assert fig["num"] <= tol and fig["num_head_max"] <= tol, msg
    assert fig["e_rms"] <= tol / 2 and fig["e_rms_well_head_max"] <= tol / 2 and fig["ratio_well"] <= tol, msg
    assert fig["state_head_max"] <= 1e-5, msg  # the state stays fp32 end to end
    assert max(piece_max.values()) <= 1e-4, msg
