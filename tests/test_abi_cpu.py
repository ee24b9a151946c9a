"""The C ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects invalid calls on the host before touching a device.

Only error paths are called here (no kernel is launched): every argument check
in the library runs before its first HIP call.
"""
import ctypes
import os
import re

import pytest

from causal_prefix_scan_hla2_amd import build as B
from causal_prefix_scan_hla2_amd import hla2 as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hla2.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(H.LIB_PATH):
        B.build()
    return H.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hla2_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_functions():
    assert header_functions() == sorted(H.EXPORTS)


def test_library_exports_every_header_symbol(L):
    for name in header_functions():
        assert hasattr(L, name), name
    out = os.popen("nm -D --defined-only %s" % H.LIB_PATH).read()
    for name in header_functions():
        assert re.search(r"\bT %s\b" % name, out), name


def test_strerror_and_version(L):
    assert H.strerror(0) == "ok"
    for c in (-1, -2, -3, -4):
        assert H.strerror(c) and H.strerror(c) != "ok"
    assert H.strerror(12345) == "unknown error code"
    assert L.hla2_abi_version() == 1


def test_state_floats(L):
    assert H.hla2_state_floats(64, 64) == 64 * 64 + 2 * 64 * 64 + 2 * 64
    assert H.hla2_state_floats(16, 128) == 16 * 16 + 2 * 16 * 128 + 2 * 16
    assert L.hla2_state_floats(0, 4) == H.HLA2_ERR_INVALID


P = ctypes.c_void_p(4096)  # a non-null, aligned pointer that is never dereferenced


def fwd(L, q=P, k=P, v=P, out=P, B_=1, H_=1, n=64, d=16, dv=16, decay=1.0, norm=0, chunk=16, dtype=0,
        den=None, ws=None, wsb=0, segments=0):
    return L.hla2_forward_ex(q, k, v, out, B_, H_, n, d, dv, decay, norm, chunk, dtype, den, ws, wsb, segments,
                             None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), H.HLA2_ERR_INVALID),
    (dict(out=None), H.HLA2_ERR_INVALID),
    (dict(B_=0), H.HLA2_ERR_INVALID),
    (dict(n=0), H.HLA2_ERR_INVALID),
    (dict(n=-5), H.HLA2_ERR_INVALID),
    (dict(decay=0.0), H.HLA2_ERR_INVALID),
    (dict(decay=1.5), H.HLA2_ERR_INVALID),
    (dict(decay=float("nan")), H.HLA2_ERR_INVALID),
    (dict(norm=2), H.HLA2_ERR_INVALID),
    (dict(dtype=7), H.HLA2_ERR_INVALID),
    (dict(segments=-1), H.HLA2_ERR_INVALID),
    (dict(d=24), H.HLA2_ERR_UNSUPPORTED),
    (dict(dv=144), H.HLA2_ERR_UNSUPPORTED),
    (dict(chunk=48), H.HLA2_ERR_UNSUPPORTED),
    (dict(chunk=256), H.HLA2_ERR_UNSUPPORTED),
    (dict(d=128, dv=16, dtype=0), H.HLA2_ERR_UNSUPPORTED),  # fp32 is limited to d, dv <= 64
    (dict(q=ctypes.c_void_p(4098)), H.HLA2_ERR_INVALID),   # misaligned
    (dict(den=ctypes.c_void_p(4098)), H.HLA2_ERR_INVALID),
])
def test_forward_rejects(L, kw, code):
    assert fwd(L, **kw) == code


def test_forward_workspace_checks(L):
    # 4 x 8 heads x 2048 tokens in chunks of 64 uses several segments -> needs a workspace
    need = H.hla2_forward_workspace_bytes(4, 8, 2048, 64, 64, 64)
    assert need > 0
    assert H.hla2_forward_segments(4, 8, 2048, 64, 64, 64) > 1
    args = dict(B_=4, H_=8, n=2048, d=64, dv=64, chunk=64, dtype=1)
    assert fwd(L, **args) == H.HLA2_ERR_WORKSPACE                         # missing
    assert fwd(L, ws=P, wsb=need - 1, **args) == H.HLA2_ERR_WORKSPACE    # too small
    assert fwd(L, ws=ctypes.c_void_p(4096 + 16), wsb=need, **args) == H.HLA2_ERR_WORKSPACE  # misaligned


def test_workspace_and_segment_plan(L):
    # one segment -> no workspace
    assert H.hla2_forward_segments(1, 1, 64, 16, 16, 16, segments=1) == 1
    assert H.hla2_forward_workspace_bytes(1, 1, 64, 16, 16, 16, segments=1) == 0
    # explicit segment counts are clamped to the number of chunks and to 64
    assert H.hla2_forward_segments(1, 1, 100, 64, 64, 64, segments=10) == 2
    assert H.hla2_forward_segments(1, 1, 1 << 16, 128, 128, 128, segments=1000) == 64
    # the automatic plan fills at least one round of workgroups on 256 CUs when there are enough
    # chunks, keeping at least 4 chunks of 64 tokens (the bf16 walker's step) per segment
    for shape in [(4, 8, 2048, 64, 64, 64), (8, 16, 8192, 64, 128, 64), (1, 16, 65536, 128, 128, 128)]:
        b, h, n, d, dv, c = shape
        r = H.hla2_forward_segments(*shape)
        nc = -(-n // 64)
        assert 1 <= r <= min(max(nc // 4, 1), 64)
        assert b * h * r >= min(256, b * h * min(nc // 4, 64)) - b * h  # within one segment of the target
    assert H.hla2_forward_segments(4, 8, 2048, 64, 64, 64) == 8
    assert H.hla2_forward_segments(8, 16, 8192, 64, 128, 64) == 3
    # invalid shapes report 0 bytes / an error code
    assert H.hla2_forward_workspace_bytes(1, 1, 64, 24, 16, 16) == 0
    assert H.hla2_forward_segments(1, 1, 64, 24, 16, 16) == H.HLA2_ERR_UNSUPPORTED


@pytest.mark.parametrize("shape,segments", [
    ((8, 16, 8192, 64, 128, 64), 0), ((4, 8, 2048, 64, 64, 64), 0), ((1, 16, 65536, 128, 128, 128), 0),
    ((2, 3, 300, 64, 128, 64), 0), ((1, 1, 4000, 64, 64, 64), 0), ((2, 2, 777, 64, 64, 64), 3),
    ((1, 1, 100, 64, 64, 64), 2), ((512, 1, 8192, 64, 64, 64), 0), ((1, 1, 64, 64, 64, 64), 0),
])
def test_lead_plan_covers_every_chunk(L, shape, segments):
    b, h, n, d, dv, c = shape
    nseg, c0, cs, lead = H.hla2_forward_plan(*shape, segments=segments)
    nc = -(-n // 64)
    assert nseg == H.hla2_forward_segments(*shape, segments=segments)
    assert 1 <= c0 <= cs
    # segment 0, then nseg-1 segments of cs chunks, the last one non-empty and at most cs
    assert c0 + (nseg - 1) * cs >= nc > c0 + (nseg - 2) * cs if nseg > 1 else c0 >= nc
    assert lead == (nseg > 1)
    if segments == 0 and nseg > 1:
        # the output walk of segments 1 .. nseg-1 puts at most one workgroup on each of 256 CUs
        assert b * h * (nseg - 1) <= 256
        # segment 0 is the shorter one (it shares its launch with the summary walks) when the
        # chunks allow it; the chunks after it are spread evenly
        assert c0 < cs or nc < 64
    if segments > 0:
        assert c0 == cs  # explicit counts split evenly


def test_lead_plan_sweep(L):
    # every automatic and explicit plan over a spread of shapes covers each 64-token chunk once,
    # keeps segment 0 no longer than the others and stays within 64 segments
    for bh in (1, 2, 3, 7, 16, 32, 100, 128, 255, 256, 300, 1024):
        for n in (1, 63, 64, 65, 257, 1000, 4096, 8191, 8192, 65536):
            for d, dv in ((64, 64), (64, 128), (128, 128), (16, 48)):
                for segments in (0, 1, 2, 3, 17, 1000):
                    nseg, c0, cs, lead = H.hla2_forward_plan(bh, 1, n, d, dv, 64, segments=segments)
                    nc = -(-n // 64)
                    key = (bh, n, d, dv, segments, nseg, c0, cs)
                    assert 1 <= nseg <= min(nc, 64), key
                    assert 1 <= c0 <= cs, key
                    assert lead == (nseg > 1), key
                    if nseg == 1:
                        assert c0 >= nc, key
                    else:
                        assert c0 + (nseg - 2) * cs < nc <= c0 + (nseg - 1) * cs, key
                    if segments == 0 and nseg > 1:
                        assert bh * (nseg - 1) <= 256, key


def test_plan_query_rejects(L):
    x = ctypes.c_int()
    assert L.hla2_forward_ex_plan(1, 1, 64, 64, 64, 64, 0, None, ctypes.byref(x), ctypes.byref(x)) == \
        H.HLA2_ERR_INVALID
    assert L.hla2_forward_ex_plan(1, 1, 64, 64, 64, 64, -1, ctypes.byref(x), ctypes.byref(x), ctypes.byref(x)) == \
        H.HLA2_ERR_INVALID
    assert L.hla2_forward_ex_plan(1, 1, 64, 24, 64, 64, 0, ctypes.byref(x), ctypes.byref(x), ctypes.byref(x)) == \
        H.HLA2_ERR_UNSUPPORTED


def dec(L, state=P, q=P, k=P, v=P, out=P, N=1, H_=1, d=64, dv=64, decay=1.0, norm=1, dtype=1):
    return L.hla2_decode_step(state, q, k, v, out, N, H_, d, dv, decay, norm, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(state=None), H.HLA2_ERR_INVALID),
    (dict(v=None), H.HLA2_ERR_INVALID),
    (dict(N=0), H.HLA2_ERR_INVALID),
    (dict(decay=-1.0), H.HLA2_ERR_INVALID),
    (dict(norm=3), H.HLA2_ERR_INVALID),
    (dict(dtype=2), H.HLA2_ERR_INVALID),
    (dict(d=48), H.HLA2_ERR_UNSUPPORTED),
    (dict(dv=256), H.HLA2_ERR_UNSUPPORTED),
    (dict(state=ctypes.c_void_p(4100)), H.HLA2_ERR_INVALID),  # state must be 16-byte aligned
])
def test_decode_rejects(L, kw, code):
    assert dec(L, **kw) == code


def test_binding_refuses_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(H, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(H, "_lib", None)
    with pytest.raises(RuntimeError):
        H.lib()


def test_forward_timed_validates_like_forward_ex(L):
    ev = (ctypes.c_void_p * 4)()
    args = (P, P, P, P, 1, 1, 64, 16, 16, 1.0, 0, 16, 0, None, None, 0, 0)
    assert L.hla2_forward_timed(None, *args[1:], ev, None) == H.HLA2_ERR_INVALID
    bad = list(args)
    bad[11] = 48  # chunk
    assert L.hla2_forward_timed(*bad, ev, None) == H.HLA2_ERR_UNSUPPORTED
    big = (P, P, P, P, 4, 8, 2048, 64, 64, 1.0, 0, 64, 1, None, None, 0, 0)
    assert L.hla2_forward_timed(*big, ev, None) == H.HLA2_ERR_WORKSPACE


def fst(L, state=P, ws=None, wsb=0, segments=0, B_=1, H_=1, n=64, d=16, dv=16, chunk=16, dtype=0, decay=1.0):
    return L.hla2_forward_state(P, P, P, P, B_, H_, n, d, dv, decay, 0, chunk, dtype, None, state, ws, wsb,
                                segments, None)


def test_forward_state_validates(L):
    # every segment keeps a summary for the export, so even one segment needs a workspace
    # (bf16 at d = dv = 64: the size reported is exactly what that call checks)
    need1 = H.hla2_forward_state_workspace_bytes(1, 1, 64, 64, 64, 64, segments=1)
    assert need1 > 0 and H.hla2_forward_workspace_bytes(1, 1, 64, 64, 64, 64, segments=1) == 0
    bf = dict(d=64, dv=64, chunk=64, dtype=1, segments=1)
    assert fst(L, state=None, ws=P, wsb=1 << 30, **bf) == H.HLA2_ERR_INVALID
    assert fst(L, state=ctypes.c_void_p(4098), ws=P, wsb=1 << 30, **bf) == H.HLA2_ERR_INVALID  # misaligned
    assert fst(L, **bf) == H.HLA2_ERR_WORKSPACE                                         # missing
    assert fst(L, ws=P, wsb=need1 - 1, **bf) == H.HLA2_ERR_WORKSPACE                    # too small
    assert fst(L, ws=ctypes.c_void_p(4096 + 64), wsb=need1, **bf) == H.HLA2_ERR_WORKSPACE  # misaligned
    assert fst(L, ws=P, wsb=1 << 30, chunk=48) == H.HLA2_ERR_UNSUPPORTED
    assert fst(L, ws=P, wsb=1 << 30, decay=0.0) == H.HLA2_ERR_INVALID
    assert fst(L, ws=P, wsb=1 << 30, segments=-2) == H.HLA2_ERR_INVALID
    # the export adds one summary block per (b, h) to the plain forward's workspace
    for shape in [(4, 8, 2048, 64, 64, 64), (1, 2, 1000, 128, 128, 64), (2, 3, 200, 32, 48, 16)]:
        b, h, n, d, dv, c = shape
        for seg in (0, 1, 3):
            plain = H.hla2_forward_workspace_bytes(*shape, segments=seg)
            st = H.hla2_forward_state_workspace_bytes(*shape, segments=seg)
            dk = 16 if max(d, dv) <= 16 and d <= 64 and dv <= 64 else (64 if d <= 64 else 128)
            assert st > plain
            assert st >= b * h * H.hla2_forward_segments(*shape, segments=seg) * dk * dk * 4
    assert H.hla2_forward_state_workspace_bytes(1, 1, 64, 24, 16, 16, 0) == 0


def bwd(L, q=P, k=P, v=P, out=None, den=None, dout=P, gq=P, gk=P, gv=P, B_=1, H_=1, n=64, d=64, dv=64, decay=1.0,
        norm=0, dtype=1, ws=None, wsb=0, segments=0):
    return L.hla2_backward(q, k, v, out, den, dout, gq, gk, gv, B_, H_, n, d, dv, decay, norm, dtype, ws, wsb,
                           segments, None)


def test_backward_validates(L):
    need = H.hla2_backward_workspace_bytes(1, 1, 64, 64, 64, 0, 1)
    assert need > 0
    big = dict(ws=P, wsb=1 << 40)
    assert bwd(L, q=None, **big) == H.HLA2_ERR_INVALID
    assert bwd(L, gv=None, **big) == H.HLA2_ERR_INVALID
    assert bwd(L, norm=1, **big) == H.HLA2_ERR_INVALID               # out and den required
    assert bwd(L, norm=1, out=P, **big) == H.HLA2_ERR_INVALID
    assert bwd(L, norm=2, **big) == H.HLA2_ERR_INVALID
    assert bwd(L, decay=0.0, **big) == H.HLA2_ERR_INVALID
    assert bwd(L, decay=float("nan"), **big) == H.HLA2_ERR_INVALID
    assert bwd(L, segments=-1, **big) == H.HLA2_ERR_INVALID
    assert bwd(L, dtype=3, **big) == H.HLA2_ERR_INVALID
    assert bwd(L, d=24, **big) == H.HLA2_ERR_UNSUPPORTED
    assert bwd(L, d=128, dtype=0, **big) == H.HLA2_ERR_UNSUPPORTED
    assert bwd(L, q=ctypes.c_void_p(4104), **big) == H.HLA2_ERR_INVALID  # misaligned
    assert bwd(L) == H.HLA2_ERR_WORKSPACE
    assert bwd(L, ws=P, wsb=need - 1) == H.HLA2_ERR_WORKSPACE
    assert bwd(L, ws=ctypes.c_void_p(4096 + 128), wsb=need) == H.HLA2_ERR_WORKSPACE
    # the ratio adds a prepared upstream-gradient buffer; more tokens need more
    assert H.hla2_backward_workspace_bytes(1, 1, 64, 64, 64, 1, 1) > need
    assert H.hla2_backward_workspace_bytes(1, 1, 4096, 64, 64, 0, 1) > need
    assert H.hla2_backward_workspace_bytes(1, 1, 64, 24, 64, 0, 1) == 0


def ahla(L, q=P, k=P, v=P, out=P, B_=1, H_=1, n=64, d=64, dv=64, decay=1.0, norm=0, dtype=1, den=None, ws=None,
         wsb=0, segments=0):
    return L.hla2_ahla_forward(q, k, v, out, B_, H_, n, d, dv, decay, norm, dtype, den, ws, wsb, segments, None)


def test_ahla_validates(L):
    big = dict(ws=P, wsb=1 << 40)
    assert ahla(L, q=None, **big) == H.HLA2_ERR_INVALID
    assert ahla(L, norm=3, **big) == H.HLA2_ERR_INVALID
    assert ahla(L, decay=1.5, **big) == H.HLA2_ERR_INVALID
    assert ahla(L, segments=-1, **big) == H.HLA2_ERR_INVALID
    assert ahla(L, dtype=5, **big) == H.HLA2_ERR_INVALID
    assert ahla(L, dv=200, **big) == H.HLA2_ERR_UNSUPPORTED
    assert ahla(L, d=128, dtype=0, **big) == H.HLA2_ERR_UNSUPPORTED
    assert ahla(L, out=ctypes.c_void_p(4100), **big) == H.HLA2_ERR_INVALID
    assert ahla(L, den=ctypes.c_void_p(4098), **big) == H.HLA2_ERR_INVALID
    # several segments need a workspace; one segment needs none
    shape = (4, 8, 2048, 64, 64)
    need = H.hla2_ahla_forward_workspace_bytes(*shape, 1, 0)
    assert need > 0 and H.hla2_ahla_forward_workspace_bytes(*shape, 1, 1) == 0
    args = dict(B_=4, H_=8, n=2048)
    assert ahla(L, **args) == H.HLA2_ERR_WORKSPACE
    assert ahla(L, ws=P, wsb=need - 1, **args) == H.HLA2_ERR_WORKSPACE


def test_ho3_validates(L):
    def ho3(**kw):
        base = dict(q=P, k=P, v=P, out=P, B_=1, H_=1, n=64, d=64, dv=64, decay=1.0, norm=0, dtype=1, den=None,
                    ws=P, wsb=1 << 40, segments=0)
        base.update(kw)
        b = base
        return L.hla2_ho3_forward(b["q"], b["k"], b["v"], b["out"], b["B_"], b["H_"], b["n"], b["d"], b["dv"],
                                  b["decay"], b["norm"], b["dtype"], b["den"], b["ws"], b["wsb"], b["segments"], None)
    assert ho3(q=None) == H.HLA2_ERR_INVALID
    assert ho3(norm=2) == H.HLA2_ERR_INVALID
    assert ho3(decay=0.0) == H.HLA2_ERR_INVALID
    assert ho3(d=128) == H.HLA2_ERR_UNSUPPORTED      # the third-order state is held for d <= 64
    assert ho3(dv=40) == H.HLA2_ERR_UNSUPPORTED
    assert ho3(k=ctypes.c_void_p(4104)) == H.HLA2_ERR_INVALID
    need = H.hla2_ho3_forward_workspace_bytes(4, 8, 2048, 64, 64, 1, 0)
    assert need > 0
    assert ho3(B_=4, H_=8, n=2048, ws=None, wsb=0) == H.HLA2_ERR_WORKSPACE
    assert ho3(B_=4, H_=8, n=2048, wsb=need - 1) == H.HLA2_ERR_WORKSPACE
    assert H.hla2_ho3_forward_workspace_bytes(1, 1, 64, 128, 64, 1, 0) == 0


def test_head_rows_beyond_32bit_offsets_rejected():
    """One head's rows are addressed with 32-bit byte offsets: a length whose padded rows
    pass 2^31 - 256 bytes is refused before anything is launched."""
    n_ok = (0x7FFFFF00 // ((64 + 16) * 4))
    assert H.hla2_forward_segments(1, 1, n_ok, 64, 64, 64) > 0
    assert H.hla2_forward_segments(1, 1, n_ok + 1, 64, 64, 64) == H.HLA2_ERR_UNSUPPORTED


def test_grids_beyond_2_32_work_items_rejected(L):
    """Every launch keeps its work-items along one grid dimension below 2^32: counts of heads (or
    heads times segments) whose grids would not fit are refused on the host, not at launch."""
    # decode: one 256-thread workgroup per (sequence, head)
    assert dec(L, N=1 << 12, H_=1 << 12) == H.HLA2_ERR_UNSUPPORTED   # 2^24 workgroups
    assert dec(L, N=1 << 14, H_=1 << 12) == H.HLA2_ERR_UNSUPPORTED
    # forward: up to 512 threads per workgroup, one per head and segment (here one segment)
    assert fwd(L, B_=1 << 13, H_=1 << 10, n=64, d=16, dv=16, chunk=16, dtype=0) == H.HLA2_ERR_UNSUPPORTED
    assert fwd(L, B_=1 << 13, H_=1 << 10, n=64, d=64, dv=64, chunk=64, dtype=1) == H.HLA2_ERR_UNSUPPORTED
    # an explicit segment count multiplies the grid: 2^18 heads x 64 segments
    assert fwd(L, B_=1 << 9, H_=1 << 9, n=64 * 64, d=64, dv=64, chunk=64, dtype=1, segments=64, ws=P,
               wsb=1 << 62) == H.HLA2_ERR_UNSUPPORTED
    big = dict(ws=P, wsb=1 << 62)
    assert bwd(L, B_=1 << 12, H_=1 << 12, n=64, **big) == H.HLA2_ERR_UNSUPPORTED
    # the ratio's upstream-gradient preparation: one thread per 4 values of dout
    assert bwd(L, B_=1 << 7, H_=1 << 7, n=1 << 14, norm=1, out=P, den=P, **big) == H.HLA2_ERR_UNSUPPORTED
    assert ahla(L, B_=1 << 13, H_=1 << 10, n=64, **big) == H.HLA2_ERR_UNSUPPORTED


def test_noalloc_validates_on_the_host(L):
    """The no-allocation forward rejects bad calls, and workspaces beyond its fixed array, before any
    device call (no kernel runs here)."""
    def na(**kw):
        b = dict(q=P, k=P, v=P, out=P, B_=1, H_=1, n=64, d=64, dv=64, decay=1.0, norm=0, chunk=64, dtype=1, den=None)
        b.update(kw)
        return L.hla2_forward_noalloc(b["q"], b["k"], b["v"], b["out"], b["B_"], b["H_"], b["n"], b["d"], b["dv"],
                                      b["decay"], b["norm"], b["chunk"], b["dtype"], b["den"], None)
    assert na(q=None) == H.HLA2_ERR_INVALID
    assert na(decay=0.0) == H.HLA2_ERR_INVALID
    assert na(norm=2) == H.HLA2_ERR_INVALID
    assert na(d=24) == H.HLA2_ERR_UNSUPPORTED
    assert na(k=ctypes.c_void_p(4098)) == H.HLA2_ERR_INVALID
    assert na(den=ctypes.c_void_p(4098)) == H.HLA2_ERR_INVALID
    # 255 heads of 65536 tokens at d = dv = 128 (two segments each) need more than the fixed array holds
    assert H.hla2_forward_workspace_bytes(1, 255, 65536, 128, 128, 128) > H.HLA2_NOALLOC_SCRATCH_BYTES
    assert na(B_=1, H_=255, n=65536, d=128, dv=128, chunk=128) == H.HLA2_ERR_UNSUPPORTED
    # the benchmark's forward workloads fit
    for shape in [(8, 16, 8192, 64, 128, 64), (4, 8, 2048, 64, 64, 64), (1, 16, 65536, 128, 128, 128)]:
        assert H.hla2_forward_workspace_bytes(*shape) <= H.HLA2_NOALLOC_SCRATCH_BYTES
