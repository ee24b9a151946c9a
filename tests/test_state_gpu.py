"""GPU parity of hla2_forward_state (through the C ABI) against the fp64 oracle.

The exported state after the last token is compared with the state the
oracle's serial recurrence holds after the same tokens (S, C, m, G, h each by
relative L2), the activations with the oracle's outputs, and decoding resumed
from the exported state with the oracle's serial pass over prefix + the new
tokens.  Cases cover one and many segments, a last segment with and without
full chunks, a sequence shorter than one chunk, every padded head size and
both element types.
"""
import numpy as np
import pytest
import torch

from causal_prefix_scan_hla2_amd import hla2 as H
from causal_prefix_scan_hla2_amd import inputs as I
from oracle import oracle as O
from tests.parity import ratio_ok, ratio_report, rel_l2, tol_for

pytestmark = pytest.mark.gpu


def draw(B, H_, n, d, dv, dtype, seed):
    w = I.Workload("state", B, H_, n, d, dv, dtype, 1.0, False, 64, seed=seed)
    return I.make_qkv(w)


def gpu_forward_state(q, k, v, decay, normalize, chunk, segments):
    dev = torch.device("cuda:0")
    B, H_, n, d = q.shape
    dv = v.shape[-1]
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(vd)
    st = torch.full((B, H_, H.hla2_state_floats(d, dv)), float("nan"), dtype=torch.float32, device=dev)
    H.hla2_forward_state(qd, kd, vd, out, st, decay=decay, normalize=normalize, chunk=chunk, segments=segments)
    torch.cuda.synchronize()
    return out, st


def state_errors(st_gpu, st_ref, d, dv):
    g, r = O.split_state(st_gpu, d, dv), O.split_state(st_ref, d, dv)
    return {key: rel_l2(g[key], r[key]) for key in ("S", "C", "m", "G", "h")}


CASES = [
    # B, H, n, d, dv, dtype, decay, normalize, chunk, segments
    (1, 2, 64, 16, 16, "f32", 1.0, False, 16, 0),      # one segment, no tail
    (2, 3, 200, 32, 48, "f32", 0.9, True, 16, 3),      # tail of 8 tokens after 3 segments
    (1, 2, 333, 64, 64, "f32", 0.97, False, 32, 0),
    (1, 1, 130, 16, 64, "f32", 0.95, False, 128, 0),
    (1, 1, 40, 64, 64, "f32", 0.9, False, 64, 0),      # shorter than a chunk: all tail
    (2, 3, 300, 64, 128, "bf16", 0.99, False, 64, 0),
    (1, 2, 1000, 128, 128, "bf16", 1.0, True, 64, 16),  # last segment has no full chunk
    (1, 1, 1000, 64, 128, "bf16", 0.99, False, 64, 7),
    (1, 2, 2048, 64, 64, "bf16", 0.999, False, 64, 0),  # several automatic segments, no tail
    (1, 2, 700, 128, 64, "bf16", 0.98, True, 64, 4),
    (1, 1, 40, 64, 64, "bf16", 0.9, False, 64, 0),     # shorter than a chunk: all tail
    (1, 1, 100, 16, 16, "bf16", 1.0, False, 16, 1),
    (1, 2, 3000, 64, 128, "bf16", 0.95, True, 64, 2),  # strong decays over many chunks
    (1, 1, 2000, 64, 64, "bf16", 0.7, False, 64, 1),
]


@pytest.mark.parametrize("B,H_,n,d,dv,dtype,decay,normalize,chunk,segments", CASES)
def test_final_state_matches_oracle(B, H_, n, d, dv, dtype, decay, normalize, chunk, segments):
    print("case", B, H_, n, d, dv, dtype, decay, normalize, chunk, segments, flush=True)
    q, k, v = draw(B, H_, n, d, dv, dtype, seed=1000 + n + d)
    out, st = gpu_forward_state(q, k, v, decay, normalize, chunk, segments)
    num, den, un, st_ref = O.serial_unorm(q.double().numpy(), k.double().numpy(), v.double().numpy(), decay)
    tol = tol_for(dtype)
    errs = state_errors(st.double().cpu().numpy(), st_ref, d, dv)
    msg = " ".join("%s %.3g" % kv for kv in errs.items())
    o = out.double().cpu().numpy()
    if normalize:
        rep = ratio_report(o, np.zeros_like(den), num, den, un, q.double().numpy())
        msg += " | ratio(well) %.3g excluded %.3f" % (rep["ratio_well"], rep["excluded"])
        ok_out = ratio_ok(rep, tol, subset=True)
    else:
        r_o = rel_l2(o, num)
        msg += " | out %.3g" % r_o
        ok_out = r_o <= tol
    print(msg)
    assert all(e <= tol for e in errs.values()), msg
    assert ok_out, msg


@pytest.mark.parametrize("normalize", [False, True])
def test_state_export_leaves_outputs_unchanged(normalize):
    """The activations of hla2_forward_state are those of hla2_forward up to rounding.

    The two calls may use different segment plans (hla2_forward's lead plan walks segment
    0's outputs beside the summaries; the export summarises every segment), so their
    roundings differ.  The quotient num/den amplifies rounding where den is near zero, so
    with normalisation the comparison is made on num = out * den and on den."""
    q, k, v = draw(2, 2, 777, 64, 64, "bf16", seed=5)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out_s, den_s = torch.empty_like(vd), torch.empty(2, 2, 777, dtype=torch.float32, device=dev)
    st = torch.empty(2, 2, H.hla2_state_floats(64, 64), dtype=torch.float32, device=dev)
    H.hla2_forward_state(qd, kd, vd, out_s, st, decay=0.99, normalize=normalize, chunk=64, den_out=den_s)
    out, den = torch.empty_like(vd), torch.empty_like(den_s)
    H.hla2_forward(qd, kd, vd, out, decay=0.99, normalize=normalize, chunk=64, den_out=den)
    torch.cuda.synchronize()
    o_s, o = out_s.double().cpu().numpy(), out.double().cpu().numpy()
    d_s, d_ = den_s.double().cpu().numpy(), den.double().cpu().numpy()
    if normalize:
        o_s, o = o_s * d_s[..., None], o * d_[..., None]
    assert rel_l2(o_s, o) <= 1e-2, rel_l2(o_s, o)
    assert rel_l2(d_s, d_) <= 1e-2, rel_l2(d_s, d_)


@pytest.mark.parametrize("d,dv,dtype,decay,normalize,prefix", [
    (64, 64, "bf16", 0.99, False, 1000),
    (128, 128, "bf16", 1.0, True, 777),
    (64, 128, "bf16", 0.95, False, 64),
    (32, 32, "f32", 0.9, True, 150),
])
def test_decode_resumes_from_exported_state(d, dv, dtype, decay, normalize, prefix):
    """Forward over a prefix, export the state, decode more tokens; compare with the
    oracle's serial pass over prefix + decoded tokens."""
    print("case", d, dv, dtype, decay, normalize, prefix, flush=True)
    B, H_, steps = 2, 3, 6
    q, k, v = draw(B, H_, prefix + steps, d, dv, dtype, seed=77 + prefix)
    _, st = gpu_forward_state(q[:, :, :prefix].contiguous(), k[:, :, :prefix].contiguous(),
                              v[:, :, :prefix].contiguous(), decay, normalize, 64 if dtype == "bf16" else 16, 0)
    dev = torch.device("cuda:0")
    outs = []
    for s in range(steps):
        t = prefix + s
        o = torch.empty(B, H_, dv, dtype=q.dtype, device=dev)
        H.hla2_decode_step(st, q[:, :, t].contiguous().to(dev), k[:, :, t].contiguous().to(dev),
                           v[:, :, t].contiguous().to(dev), o, decay=decay, normalize=normalize)
        outs.append(o)
    torch.cuda.synchronize()
    o_gpu = torch.stack(outs, 2).double().cpu().numpy()
    num, den, un, st_ref = O.serial_unorm(q.double().numpy(), k.double().numpy(), v.double().numpy(), decay)
    tol = tol_for(dtype)
    tail = slice(prefix, prefix + steps)
    if normalize:
        rep = ratio_report(o_gpu, np.zeros_like(den[..., tail]), num[..., tail, :], den[..., tail],
                           un[..., tail], q[:, :, tail].double().numpy())
        msg = "ratio(well) %.3g excluded %.3f" % (rep["ratio_well"], rep["excluded"])
        ok = ratio_ok(rep, tol, subset=True)
    else:
        r = rel_l2(o_gpu, num[..., tail, :])
        msg = "out %.3g" % r
        ok = r <= tol
    errs = state_errors(st.double().cpu().numpy(), st_ref, d, dv)
    msg += " | " + " ".join("%s %.3g" % kv for kv in errs.items())
    print(msg)
    assert ok, msg
    assert all(e <= tol for e in errs.values()), msg


def test_decode_workload_prefix_state_sampled():
    """The state after the decode workload's 4096-token prefix (d = dv = 64, normalised), built by the
    forward pass with its export for two sequences x all 32 heads, matches the oracle's serial state on
    sampled heads; the same per-head shape the benchmark prefills."""
    w = I.DECODE
    N = 2
    toks = [[I.decode_prefix_tokens(w, s, h) for h in range(w.H)] for s in range(N)]
    q = torch.stack([torch.stack([t[0] for t in row]) for row in toks])
    k = torch.stack([torch.stack([t[1] for t in row]) for row in toks])
    v = torch.stack([torch.stack([t[2] for t in row]) for row in toks])
    _, st = gpu_forward_state(q, k, v, w.decay, w.normalize, 64, 0)
    st = st.double().cpu().numpy()
    for (s, h) in I.sample_heads(N, w.H, 4):
        _, _, ref = O.serial(q[s, h].double().numpy(), k[s, h].double().numpy(), v[s, h].double().numpy(), w.decay)
        errs = state_errors(st[s, h], ref, w.d, w.dv)
        msg = "head (%d, %d): " % (s, h) + " ".join("%s %.3g" % kv for kv in errs.items())
        print(msg)
        assert all(e <= tol_for(w.dtype) for e in errs.values()), msg
