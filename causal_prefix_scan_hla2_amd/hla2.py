"""Thin ctypes binding of ``libhla2.so`` (the C ABI in ``include/hla2.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.  The
binding refuses to run without the compiled library (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhla2.so")

HLA2_F32, HLA2_BF16 = 0, 1
HLA2_OK, HLA2_ERR_INVALID, HLA2_ERR_UNSUPPORTED, HLA2_ERR_WORKSPACE, HLA2_ERR_LAUNCH = 0, -1, -2, -3, -4

# every symbol include/hla2.h declares
EXPORTS = ("hla2_strerror", "hla2_abi_version", "hla2_forward_workspace_bytes", "hla2_forward_segments",
           "hla2_forward", "hla2_forward_ex_workspace_bytes", "hla2_forward_ex_segments", "hla2_forward_ex_plan",
           "hla2_forward_ex",
           "hla2_forward_timed", "hla2_decode_step", "hla2_state_floats", "hla2_forward_state_workspace_bytes",
           "hla2_forward_state", "hla2_backward_workspace_bytes", "hla2_backward",
           "hla2_ahla_forward_workspace_bytes", "hla2_ahla_forward", "hla2_ho3_forward_workspace_bytes",
           "hla2_ho3_forward", "hla2_forward_noalloc")
HLA2_NOALLOC_SCRATCH_BYTES = 96 << 20  # the fixed workspace of hla2_forward_noalloc (include/hla2.h)

_lock = threading.Lock()
_lib = None


class HLA2Error(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (what, strerror(code) if _lib else "", code))


def lib():
    """Load libhla2.so (built beforehand by ``build.build()``); raise if absent."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libhla2.so is not built; run causal_prefix_scan_hla2_amd.build.build()")
            L = ctypes.CDLL(LIB_PATH)
            vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
            L.hla2_strerror.restype = ctypes.c_char_p
            L.hla2_strerror.argtypes = [i]
            L.hla2_abi_version.restype = i
            L.hla2_abi_version.argtypes = []
            L.hla2_forward_workspace_bytes.restype = sz
            L.hla2_forward_workspace_bytes.argtypes = [i, i, i, i, i, i]
            L.hla2_forward_segments.restype = i
            L.hla2_forward_segments.argtypes = [i, i, i, i, i, i]
            L.hla2_forward.restype = i
            L.hla2_forward.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, vp, sz, vp]
            L.hla2_forward_ex_workspace_bytes.restype = sz
            L.hla2_forward_ex_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
            L.hla2_forward_ex_segments.restype = i
            L.hla2_forward_ex_segments.argtypes = [i, i, i, i, i, i, i]
            ip = ctypes.POINTER(ctypes.c_int)
            L.hla2_forward_ex_plan.restype = i
            L.hla2_forward_ex_plan.argtypes = [i, i, i, i, i, i, i, ip, ip, ip]
            L.hla2_forward_ex.restype = i
            L.hla2_forward_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, vp, sz, i, vp]
            L.hla2_forward_timed.restype = i
            L.hla2_forward_timed.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, vp, sz, i, vp, vp]
            L.hla2_decode_step.restype = i
            L.hla2_decode_step.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
            L.hla2_state_floats.restype = ctypes.c_long
            L.hla2_state_floats.argtypes = [i, i]
            L.hla2_forward_state_workspace_bytes.restype = sz
            L.hla2_forward_state_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
            L.hla2_forward_state.restype = i
            L.hla2_forward_state.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, vp, vp, sz, i, vp]
            L.hla2_backward_workspace_bytes.restype = sz
            L.hla2_backward_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
            L.hla2_ahla_forward_workspace_bytes.restype = sz
            L.hla2_ahla_forward_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
            L.hla2_ahla_forward.restype = i
            L.hla2_ahla_forward.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, vp, sz, i, vp]
            L.hla2_ho3_forward_workspace_bytes.restype = sz
            L.hla2_ho3_forward_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
            L.hla2_ho3_forward.restype = i
            L.hla2_ho3_forward.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, vp, sz, i, vp]
            L.hla2_forward_noalloc.restype = i
            L.hla2_forward_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, vp]
            L.hla2_backward.restype = i
            L.hla2_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, i, vp]
            _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().hla2_strerror(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return HLA2_F32
    if t.dtype == torch.bfloat16:
        return HLA2_BF16
    raise TypeError("q, k, v must be float32 or bfloat16, got %s" % t.dtype)


def hla2_forward_workspace_bytes(B, H, n, d, dv, chunk, segments=0) -> int:
    return int(lib().hla2_forward_ex_workspace_bytes(B, H, n, d, dv, chunk, segments))


def hla2_forward_segments(B, H, n, d, dv, chunk, segments=0) -> int:
    return int(lib().hla2_forward_ex_segments(B, H, n, d, dv, chunk, segments))


def hla2_forward_plan(B, H, n, d, dv, chunk, segments=0):
    """The bf16 forward's segment plan: (nseg, chunks of segment 0, chunks of each later
    segment, lead) where lead says segment 0's outputs are walked beside the summary walks."""
    nseg, c0, cs = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    rc = lib().hla2_forward_ex_plan(B, H, n, d, dv, chunk, segments, ctypes.byref(nseg), ctypes.byref(c0),
                                    ctypes.byref(cs))
    if rc < 0:
        raise HLA2Error(rc, "hla2_forward_ex_plan")
    return nseg.value, c0.value, cs.value, bool(rc)


def hla2_state_floats(d, dv) -> int:
    return int(lib().hla2_state_floats(d, dv))


def hla2_forward(q, k, v, out, decay=1.0, normalize=False, chunk=64, den_out=None, workspace=None,
                 stream=None, segments=0, check=True, events=None) -> int:
    """Call the C forward pass on torch tensors q, k: [B,H,n,d]; v, out: [B,H,n,dv].

    ``hla2_forward`` when segments == 0, else ``hla2_forward_ex`` with that
    segment count; ``hla2_forward_timed`` when ``events`` (four created
    torch.cuda.Event objects, or None entries) is given.  ``workspace``: a
    uint8 device tensor of at least the required bytes; allocated here (torch
    caching allocator) when None.  Returns the C return code (and raises on
    error when check=True)."""
    import torch
    B, H, n, d = q.shape
    dv = v.shape[-1]
    for t in (q, k, v, out):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    need = hla2_forward_workspace_bytes(B, H, n, d, dv, chunk, segments)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n, d, dv, float(decay), int(bool(normalize)), int(chunk),
            _dtype_code(q), _ptr(den_out), _ptr(workspace), wbytes)
    if events is not None:
        if len(events) != 4:
            raise ValueError("events must hold four entries")
        arr = (ctypes.c_void_p * 4)(*[None if e is None else e.cuda_event for e in events])
        rc = lib().hla2_forward_timed(*args, int(segments), arr, _stream(stream))
    elif segments:
        rc = lib().hla2_forward_ex(*args, int(segments), _stream(stream))
    else:
        rc = lib().hla2_forward(*args, _stream(stream))
    if check and rc != HLA2_OK:
        raise HLA2Error(rc, "hla2_forward")
    return rc


def hla2_forward_noalloc(q, k, v, out, decay=1.0, normalize=False, chunk=64, den_out=None, stream=None,
                         check=True) -> int:
    """Call the C forward pass that uses the library's fixed device workspace (no allocation here
    or in the library).  Same tensors and results as hla2_forward."""
    B, H, n, d = q.shape
    dv = v.shape[-1]
    for t in (q, k, v, out):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    rc = lib().hla2_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n, d, dv, float(decay),
                                    int(bool(normalize)), int(chunk), _dtype_code(q), _ptr(den_out), _stream(stream))
    if check and rc != HLA2_OK:
        raise HLA2Error(rc, "hla2_forward_noalloc")
    return rc


def hla2_forward_state_workspace_bytes(B, H, n, d, dv, chunk, segments=0) -> int:
    return int(lib().hla2_forward_state_workspace_bytes(B, H, n, d, dv, chunk, segments))


def hla2_forward_state(q, k, v, out, state_out, decay=1.0, normalize=False, chunk=64, den_out=None,
                       workspace=None, stream=None, segments=0, check=True) -> int:
    """Call ``hla2_forward_state``: the forward pass of ``hla2_forward`` plus the
    final state, written to ``state_out`` (fp32 [B,H,state_floats], the layout
    ``hla2_decode_step`` reads).  ``workspace`` as for ``hla2_forward``."""
    import torch
    B, H, n, d = q.shape
    dv = v.shape[-1]
    for t in (q, k, v, out, state_out):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if state_out.dtype != torch.float32 or state_out.numel() != B * H * hla2_state_floats(d, dv):
        raise ValueError("state_out must be fp32 [B, H, state_floats]")
    need = hla2_forward_state_workspace_bytes(B, H, n, d, dv, chunk, segments)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().hla2_forward_state(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n, d, dv, float(decay),
                                  int(bool(normalize)), int(chunk), _dtype_code(q), _ptr(den_out),
                                  _ptr(state_out), _ptr(workspace), wbytes, int(segments), _stream(stream))
    if check and rc != HLA2_OK:
        raise HLA2Error(rc, "hla2_forward_state")
    return rc


def hla2_backward_workspace_bytes(B, H, n, d, dv, normalize, dtype_code, segments=0) -> int:
    return int(lib().hla2_backward_workspace_bytes(B, H, n, d, dv, int(bool(normalize)), int(dtype_code), segments))


def hla2_backward(q, k, v, dout, grad_q, grad_k, grad_v, decay=1.0, normalize=False, out=None, den=None,
                  workspace=None, stream=None, segments=0, check=True) -> int:
    """Call ``hla2_backward``: gradients of sum(dout * out) w.r.t. q, k, v written to
    grad_q, grad_k: [B,H,n,d] and grad_v: [B,H,n,dv] (same dtype as q).  Under
    ``normalize`` the forward's ``out`` and fp32 ``den`` are required."""
    import torch
    B, H, n, d = q.shape
    dv = v.shape[-1]
    for t in (q, k, v, dout, grad_q, grad_k, grad_v) + ((out, den) if normalize else ()):
        if t is None or not t.is_contiguous():
            raise ValueError("tensors must be given and contiguous")
    code = _dtype_code(q)
    need = hla2_backward_workspace_bytes(B, H, n, d, dv, normalize, code, segments)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().hla2_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out) if normalize else None,
                             _ptr(den) if normalize else None, _ptr(dout), _ptr(grad_q), _ptr(grad_k), _ptr(grad_v),
                             B, H, n, d, dv, float(decay), int(bool(normalize)), code, _ptr(workspace), wbytes,
                             int(segments), _stream(stream))
    if check and rc != HLA2_OK:
        raise HLA2Error(rc, "hla2_backward")
    return rc


def hla2_ahla_forward_workspace_bytes(B, H, n, d, dv, dtype_code, segments=0) -> int:
    return int(lib().hla2_ahla_forward_workspace_bytes(B, H, n, d, dv, int(dtype_code), segments))


def hla2_ahla_forward(q, k, v, out, decay=1.0, normalize=False, den_out=None, workspace=None, stream=None,
                      segments=0, check=True) -> int:
    """Call ``hla2_ahla_forward`` (the asymmetric variant) on torch tensors q, k: [B,H,n,d];
    v, out: [B,H,n,dv]."""
    import torch
    B, H, n, d = q.shape
    dv = v.shape[-1]
    for t in (q, k, v, out):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    code = _dtype_code(q)
    need = hla2_ahla_forward_workspace_bytes(B, H, n, d, dv, code, segments)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().hla2_ahla_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n, d, dv, float(decay),
                                 int(bool(normalize)), code, _ptr(den_out), _ptr(workspace), wbytes, int(segments),
                                 _stream(stream))
    if check and rc != HLA2_OK:
        raise HLA2Error(rc, "hla2_ahla_forward")
    return rc


def hla2_ho3_forward_workspace_bytes(B, H, n, d, dv, dtype_code, segments=0) -> int:
    return int(lib().hla2_ho3_forward_workspace_bytes(B, H, n, d, dv, int(dtype_code), segments))


def hla2_ho3_forward(q, k, v, out, decay=1.0, normalize=False, den_out=None, workspace=None, stream=None,
                     segments=0, check=True) -> int:
    """Call ``hla2_ho3_forward`` (third order) on torch tensors q, k: [B,H,n,d]; v, out: [B,H,n,dv]."""
    import torch
    B, H, n, d = q.shape
    dv = v.shape[-1]
    for t in (q, k, v, out):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    code = _dtype_code(q)
    need = hla2_ho3_forward_workspace_bytes(B, H, n, d, dv, code, segments)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().hla2_ho3_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, n, d, dv, float(decay),
                                int(bool(normalize)), code, _ptr(den_out), _ptr(workspace), wbytes, int(segments),
                                _stream(stream))
    if check and rc != HLA2_OK:
        raise HLA2Error(rc, "hla2_ho3_forward")
    return rc


def hla2_decode_step(state, q, k, v, out, decay=1.0, normalize=False, stream=None, check=True) -> int:
    """Call ``hla2_decode_step``: state [N,H,state_floats] fp32 (in place);
    q, k: [N,H,d]; v, out: [N,H,dv]."""
    N, H, d = q.shape
    dv = v.shape[-1]
    rc = lib().hla2_decode_step(_ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(out), N, H, d, dv, float(decay),
                                int(bool(normalize)), _dtype_code(q), _stream(stream))
    if check and rc != HLA2_OK:
        raise HLA2Error(rc, "hla2_decode_step")
    return rc
