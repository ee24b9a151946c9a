"""GPU parity of hla2_forward (through the C ABI) against the fp64 oracle.

Small cases span several chunk tiles, several segments and a ragged tail.  The
benchmark workloads at their full sizes are compared head by head in
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


def gpu_forward(q, k, v, decay, normalize, chunk, segments=0, want_den=True):
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(vd)
    den = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev) if want_den else None
    H.hla2_forward(qd, kd, vd, out, decay=decay, normalize=normalize, chunk=chunk, den_out=den,
                   segments=segments)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), (den.double().cpu().numpy() if want_den else None)


def check_case(q, k, v, decay, normalize, chunk, dtype_name, segments=0, heads=None, subset=False):
    """Compare GPU vs oracle; `heads` restricts the oracle to a list of (b, h)."""
    tol = tol_for(dtype_name)
    o_gpu, den_gpu = gpu_forward(q, k, v, decay, normalize, chunk, segments)
    if normalize:
        num_gpu, _ = gpu_forward(q, k, v, decay, False, chunk, segments, want_den=False)
    else:
        num_gpu = o_gpu
    if heads is not None:
        idx = tuple(np.array(heads).T)
        tidx = tuple(torch.as_tensor(x) for x in idx)
        q, k, v = q[tidx], k[tidx], v[tidx]
        o_gpu, den_gpu, num_gpu = o_gpu[idx], den_gpu[idx], num_gpu[idx]
    num, den, un, _ = O.serial_unorm(q.double().numpy(), k.double().numpy(), v.double().numpy(), decay)
    r_num = rel_l2(num_gpu, num)
    r_den = rel_l2(den_gpu, den)
    msg = "num %.3g den %.3g" % (r_num, r_den)
    assert r_num <= tol, msg
    assert r_den <= tol, msg
    if normalize:
        rep = ratio_report(o_gpu, den_gpu, num, den, un, q.double().numpy())
        msg += " e_max %.3g e_rms %.3g | ratio(well) %.3g excluded %.3f" % (
            rep["e_max"], rep["e_rms"], rep["ratio_well"], rep["excluded"])
        assert ratio_ok(rep, tol, subset), msg
    print(msg)
    return msg


def draw(B, H_, n, d, dv, dtype, seed, unit_rows=False, v_scale=None):
    w = I.Workload("case", B, H_, n, d, dv, dtype, 1.0, False, 64, qk_unit_rows=unit_rows, v_scale=v_scale,
                   seed=seed)
    return I.make_qkv(w)


SMALL = [
    # B, H, n, d, dv, dtype, decay, normalize, chunk, segments
    (1, 1, 64, 16, 16, "f32", 1.0, False, 16, 0),
    (2, 3, 200, 32, 48, "f32", 0.9, True, 16, 0),
    (1, 2, 300, 64, 64, "f32", 1.0, True, 64, 0),
    (1, 1, 130, 16, 64, "f32", 0.95, False, 128, 0),
    (1, 2, 333, 48, 32, "f32", 0.97, False, 32, 3),
    (2, 3, 300, 64, 128, "bf16", 0.99, False, 64, 0),
    (2, 2, 333, 64, 64, "bf16", 1.0, True, 64, 0),
    (1, 2, 260, 128, 128, "bf16", 1.0, True, 128, 0),
    (1, 2, 200, 48, 80, "bf16", 0.9, True, 32, 0),
    (1, 1, 100, 16, 16, "bf16", 1.0, False, 16, 0),
    (1, 2, 700, 128, 64, "bf16", 0.98, False, 64, 4),
    (1, 1, 1000, 64, 128, "bf16", 0.99, False, 64, 1),
    (1, 1, 1000, 64, 128, "bf16", 0.99, False, 64, 2),
    (1, 1, 1000, 64, 128, "bf16", 0.99, False, 64, 7),
    (1, 2, 4100, 64, 64, "bf16", 1.0, True, 32, 0),
    # lead plans at d = 64 with 8 and 9 segments (6 and 7 summaries to fold, a ragged last
    # segment in the first)
    (1, 2, 2304, 64, 64, "bf16", 0.98, True, 64, 8),
    (1, 2, 2304, 64, 128, "bf16", 0.98, True, 64, 9),
    # Strong decays (the state shrinks by 2^-5 to 2^-47 per 64-token chunk), many chunks per
    # segment, one and several segments, ratio on and off.
    (1, 2, 3000, 64, 128, "bf16", 0.95, False, 64, 1),
    (1, 2, 3000, 64, 128, "bf16", 0.95, True, 64, 3),
    (1, 2, 3000, 64, 64, "bf16", 0.95, False, 64, 2),
    (1, 2, 2000, 64, 128, "bf16", 0.7, False, 64, 2),
    (1, 2, 2000, 48, 64, "bf16", 0.7, True, 64, 1),
    (1, 2, 2000, 64, 128, "bf16", 0.6, True, 64, 2),
    (1, 1, 2000, 64, 64, "bf16", 0.6, False, 64, 1),
]


# Automatic lead plans whose segment 0 is shorter than the others (segment 0's output walk
# leaves the incoming state of segment 1; the scan continues from it): decay, ratio, ragged
# tails, both padded head sizes, value widths 64 and 128.
LEAD = [
    # B, H, n, d, dv, decay, normalize, oracle heads (None: all)
    (2, 2, 777, 64, 64, 0.99, True, None),
    (1, 4, 2074, 64, 128, 0.95, False, None),
    (2, 2, 1537, 48, 80, 0.97, True, None),
    (4, 16, 1937, 128, 128, 0.99, True, [(0, 0), (1, 7), (3, 15)]),
    (4, 16, 1700, 128, 64, 1.0, False, [(0, 3), (2, 9), (3, 14)]),
]


@pytest.mark.parametrize("case", LEAD, ids=lambda c: "-".join(str(x) for x in c[:7]))
def test_lead_plan_cases(case):
    B, H_, n, d, dv, decay, norm, heads = case
    nseg, c0, cs, lead = H.hla2_forward_plan(B, H_, n, d, dv, 64)
    assert lead and nseg >= 3 and c0 < cs, (nseg, c0, cs)
    q, k, v = draw(B, H_, n, d, dv, "bf16", seed=n + d + dv + 1)
    check_case(q, k, v, decay, norm, 64, "bf16", heads=heads)


# Three-segment lead plans at d <= 64 launch no scan: segment 2's output walk folds segment 1's
# summary onto segment 1's prefix in its prologue.  Without decay (or with a weak one) the folded
# cross term S0 C_1 keeps its full weight (a strong decay all but removes it over a segment), so
# these cases see a wrong fold; segment 2's tokens are also checked on their own.
FOLD = [
    # B, H, n, d, dv, decay, normalize, segments (0: automatic)
    (2, 2, 777, 64, 64, 1.0, True, 0),
    (1, 3, 1000, 64, 128, 1.0, False, 3),
    (2, 2, 900, 48, 80, 0.999, True, 3),
    (1, 2, 1500, 32, 128, 1.0, True, 3),
]


@pytest.mark.parametrize("case", FOLD, ids=lambda c: "-".join(str(x) for x in c))
def test_prologue_fold_cases(case):
    B, H_, n, d, dv, decay, norm, segs = case
    nseg, c0, cs, lead = H.hla2_forward_plan(B, H_, n, d, dv, 64, segs)
    assert lead and nseg == 3, (nseg, lead)
    q, k, v = draw(B, H_, n, d, dv, "bf16", seed=n + d + 5)
    check_case(q, k, v, decay, norm, 64, "bf16", segments=segs)
    t2 = (c0 + cs) * 64  # first token of segment 2
    num_gpu, _ = gpu_forward(q, k, v, decay, False, 64, segs, want_den=False)
    num, _, _, _ = O.serial_unorm(q.double().numpy(), k.double().numpy(), v.double().numpy(), decay)
    r2 = rel_l2(num_gpu[..., t2:, :], num[..., t2:, :])
    print("segment 2 from token %d: num %.3g" % (t2, r2))
    assert r2 <= tol_for("bf16"), r2


# Degenerate lengths: a single token, one short of a chunk, one past a chunk, exactly one chunk
# (both element types, ratio and decay on).
SHORT = [
    # B, H, n, d, dv, dtype
    (2, 2, 1, 64, 64, "bf16"), (1, 2, 63, 64, 128, "bf16"), (1, 2, 65, 128, 64, "bf16"),
    (1, 1, 64, 64, 64, "bf16"), (2, 1, 1, 16, 16, "f32"), (1, 2, 17, 32, 48, "f32"),
]


@pytest.mark.parametrize("case", SHORT, ids=lambda c: "-".join(str(x) for x in c))
def test_short_sequences(case):
    B, H_, n, d, dv, dt = case
    q, k, v = draw(B, H_, n, d, dv, dt, seed=31 + n + d)
    check_case(q, k, v, 0.97, True, 16 if dt == "f32" else 64, dt)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(str(x) for x in c))
def test_small_cases(case):
    B, H_, n, d, dv, dt, decay, norm, chunk, segs = case
    q, k, v = draw(B, H_, n, d, dv, dt, seed=n + d + dv)
    check_case(q, k, v, decay, norm, chunk, dt, segments=segs)


def test_integer_inputs_exact_fp32():
    # entries in {-1, 0, 1} at the tiny shape: every fp32 intermediate is an
    # exact integer, so the GPU must reproduce the oracle bit for bit
    g = torch.Generator().manual_seed(5)
    q, k, v = (torch.randint(-1, 2, (1, 1, 64, 16), generator=g).float() for _ in range(3))
    for segs in (1, 4):
        o_gpu, den_gpu = gpu_forward(q, k, v, 1.0, False, 16, segments=segs)
        num, den, _ = O.serial(q.double().numpy(), k.double().numpy(), v.double().numpy(), 1.0)
        np.testing.assert_array_equal(o_gpu, num)
        np.testing.assert_array_equal(den_gpu, den)


@pytest.mark.parametrize("dt,chunk,segs", [("bf16", 64, 3), ("f32", 16, 5)])
def test_causality_bitwise(dt, chunk, segs):
    # changing tokens >= t* must leave every output before t* bit-identical,
    # across chunk and segment boundaries
    B, H_, n, d, dv = 1, 2, 640, 64, 64
    q, k, v = draw(B, H_, n, d, dv, dt, seed=77)
    base, bden = gpu_forward(q, k, v, 0.97, True, chunk, segments=segs)
    for ts in (0, chunk - 1, chunk, 200, 333, n - 1):
        q2, k2, v2 = q.clone(), k.clone(), v.clone()
        q2[..., ts:, :] = -q2[..., ts:, :] + 0.5
        k2[..., ts:, :] = k2[..., ts:, :] * 2
        v2[..., ts:, :] = v2[..., ts:, :] - 1
        o2, d2 = gpu_forward(q2, k2, v2, 0.97, True, chunk, segments=segs)
        np.testing.assert_array_equal(o2[..., :ts, :], base[..., :ts, :])
        np.testing.assert_array_equal(d2[..., :ts], bden[..., :ts])
        assert not np.array_equal(o2[..., ts:, :], base[..., ts:, :])


def test_repeatable_bitwise():
    q, k, v = draw(2, 4, 1500, 64, 128, "bf16", seed=3)
    a, da = gpu_forward(q, k, v, 0.99, True, 64)
    b, db = gpu_forward(q, k, v, 0.99, True, 64)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(da, db)


@pytest.mark.parametrize("segs", [3, 2])
def test_timed_entry_point_matches_and_records_phases(segs):
    # the phase events change nothing in the results and bracket every kernel (with two
    # segments under the lead plan no scan runs: events 1 and 2 are back to back)
    q, k, v = draw(2, 4, 1500, 64, 128, "bf16", seed=3)
    assert H.hla2_forward_plan(2, 4, 1500, 64, 128, 64, segments=segs)[0] == segs
    a, da = gpu_forward(q, k, v, 0.99, True, 64, segments=segs)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty_like(vd)
    den = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()
    H.hla2_forward(qd, kd, vd, out, decay=0.99, normalize=True, chunk=64, den_out=den, segments=segs, events=evs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.double().cpu().numpy(), a)
    np.testing.assert_array_equal(den.double().cpu().numpy(), da)
    spans = [evs[i].elapsed_time(evs[i + 1]) for i in range(3)]
    assert all(s >= 0 for s in spans) and spans[0] > 0 and spans[2] > 0


def test_heads_independent():
    # one head computed alone equals the same head inside a batch (same plan)
    q, k, v = draw(2, 3, 500, 64, 64, "bf16", seed=9)
    full, _ = gpu_forward(q, k, v, 1.0, False, 64, segments=2)
    one, _ = gpu_forward(q[1:2, 2:3].contiguous(), k[1:2, 2:3].contiguous(), v[1:2, 2:3].contiguous(), 1.0,
                         False, 64, segments=2)
    np.testing.assert_array_equal(one[0, 0], full[1, 2])


def test_chunk_size_bf16_bitwise_same():
    # the bf16 path walks 64-token chunks whatever `chunk` says: every valid value gives the
    # same bits (the header states this)
    q, k, v = draw(1, 2, 512, 64, 64, "bf16", seed=21)
    outs = [gpu_forward(q, k, v, 0.98, True, c) for c in (16, 32, 64, 128)]
    for o, dn in outs[1:]:
        np.testing.assert_array_equal(o, outs[0][0])
        np.testing.assert_array_equal(dn, outs[0][1])


@pytest.mark.parametrize("segs", [0, 3])
def test_chunk_size_changes_rounding_only_fp32(segs):
    # the fp32 path tiles by the requested chunk: results differ between chunk sizes, but only by
    # rounding, and every one matches the oracle [scan equivalence]
    q, k, v = draw(1, 2, 520, 64, 64, "f32", seed=22)
    outs = [gpu_forward(q, k, v, 0.98, False, c, segments=segs)[0] for c in (16, 32, 64, 128)]
    num, _, _ = O.serial(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.98)
    assert any(not np.array_equal(o, outs[0]) for o in outs[1:])
    for o in outs:
        assert rel_l2(o, num) < tol_for("f32")
        assert rel_l2(o, outs[0]) < 1e-5


def test_long_single_head_max_segments():
    """One head of 262,144 tokens (d = dv = 64, bf16, decay 0.999): the automatic plan cuts it into the
    maximum of 64 segments of 64 chunks; every token is compared with the oracle."""
    print("case 1 1 262144 64 64 bf16 0.999", flush=True)
    assert H.hla2_forward_segments(1, 1, 262144, 64, 64, 64) == 64
    q, k, v = draw(1, 1, 262144, 64, 64, "bf16", seed=77)
    print(check_case(q, k, v, 0.999, False, 64, "bf16"))
