"""GPU check of hla2_forward_noalloc (through the C ABI): the forward pass with the library's fixed
device workspace gives exactly what hla2_forward gives with a caller-allocated workspace.

Both run the same kernels on the same segment plan, so the outputs (and den) must be bitwise equal.
Calls follow each other on one stream, the later ones with smaller inputs, so that a call reading
what an earlier, larger call left in the shared array would show.
"""
import numpy as np
import pytest
import torch

from causal_prefix_scan_hla2_amd import hla2 as H
from causal_prefix_scan_hla2_amd import inputs as I

pytestmark = pytest.mark.gpu


def run_both(w, want_den, B=None, H_=None, n=None, seed=None):
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in I.make_qkv(w, B=B, H=H_, n=n, seed=seed))
    print("case %s B=%d H=%d n=%d den=%s" % (w.name, q.shape[0], q.shape[1], q.shape[2], want_den), flush=True)
    outs = []
    for fn in ("ref", "noalloc"):
        out = torch.empty_like(v)
        den = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev) if want_den else None
        if fn == "ref":
            H.hla2_forward(q, k, v, out, decay=w.decay, normalize=w.normalize, chunk=w.chunk, den_out=den)
        else:
            H.hla2_forward_noalloc(q, k, v, out, decay=w.decay, normalize=w.normalize, chunk=w.chunk, den_out=den)
        torch.cuda.synchronize()
        outs.append((out.cpu(), None if den is None else den.cpu()))
    (o1, d1), (o2, d2) = outs
    assert torch.equal(o1, o2)
    if want_den:
        assert torch.equal(d1, d2)
    return o2


def test_noalloc_matches_forward_large_then_smaller():
    # the largest benchmark workspace first (16 heads x 65536 tokens, d = dv = 128: 82 MiB of the 96),
    # then the decay workload, then smaller and ragged inputs, all on the one shared array
    run_both(I.WORKLOADS["long_64k"], True)
    run_both(I.WORKLOADS["decay_8k"], False)
    run_both(I.WORKLOADS["decay_8k"], True, B=2, H_=3, n=1000, seed=5)
    run_both(I.WORKLOADS["norm_2k"], True)
    run_both(I.WORKLOADS["norm_2k"], False, B=1, H_=2, n=333, seed=6)


def test_noalloc_two_calls_in_a_row_second_smaller():
    w = I.WORKLOADS["decay_8k"]
    run_both(w, True, B=4, H_=16, n=4096, seed=7)
    run_both(w, True, B=1, H_=5, n=700, seed=8)


def test_noalloc_single_segment_needs_no_array():
    # one segment per head: no workspace at all (the array is not touched)
    w = I.WORKLOADS["decay_8k"]
    assert H.hla2_forward_workspace_bytes(32, 16, 512, 64, 128, 64) == 0
    run_both(w, True, B=32, H_=16, n=512, seed=9)


def test_noalloc_rejects_oversized_workspace_before_launch():
    dev = torch.device("cuda:0")
    B, H_, n, d, dv = 1, 255, 65536, 128, 128
    assert H.hla2_forward_workspace_bytes(B, H_, n, d, dv, 128) > H.HLA2_NOALLOC_SCRATCH_BYTES
    q = torch.empty(16, dtype=torch.bfloat16, device=dev)  # never read: the call is refused first
    L = H.lib()
    rc = L.hla2_forward_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), B, H_, n, d, dv, 1.0, 0, 128,
                                H.HLA2_BF16, None, None)
    assert rc == H.HLA2_ERR_UNSUPPORTED
