"""ctypes binding of libhgrn2.so (see include/hgrn2.h).

Argument marshalling only: shapes and dtypes are checked, outputs are
allocated with torch when the caller does not pass them, and every step of the
computation runs in the library's HIP kernels on torch's current stream.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhgrn2.so")

F32, BF16 = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}
# HGRN2_OUT_F32 of include/hgrn2.h: or'ed into a dtype code, float32 token outputs
OUT_F32 = 0x100


def _odt(dt, out_dtype):
    """The token outputs' dtype and the call's dtype code for inputs of dtype
    dt: out_dtype None (or dt) keeps the input dtype; float32 with bfloat16
    inputs writes y and the gradients as float32."""
    if dt not in _DT:
        raise ValueError("dtype must be float32 or bfloat16")
    if out_dtype is None or out_dtype == dt:
        return dt, _DT[dt]
    if out_dtype == torch.float32:
        return torch.float32, _DT[dt] | OUT_F32
    raise ValueError("out_dtype must be None, the input dtype or torch.float32")


class HGRN2Error(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, where: str, msg: str):
        super().__init__("%s: %s (%s)" % (where, _lib().hgrn2_status_string(status).decode(), msg))
        self.status = status


_handle = None


def _lib():
    global _handle
    if _handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libhgrn2.so is not built: run `python -m linear_attention_hgrn2_amd.build` "
                              "(or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        I, P, Z = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        lib.hgrn2_abi_version.restype = I
        lib.hgrn2_status_string.restype = ctypes.c_char_p
        lib.hgrn2_status_string.argtypes = [I]
        lib.hgrn2_last_error.restype = ctypes.c_char_p
        lib.hgrn2_supported.argtypes = [I, I, I]
        lib.hgrn2_supported.restype = I
        lib.hgrn2_num_chunks.argtypes = [I, I]
        lib.hgrn2_num_chunks.restype = I
        lib.hgrn2_states_bytes.argtypes = [I, I, I, I, I, I, I]
        lib.hgrn2_states_bytes.restype = Z
        lib.hgrn2_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
        lib.hgrn2_fwd_workspace_bytes.restype = Z
        lib.hgrn2_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
        lib.hgrn2_bwd_workspace_bytes.restype = Z
        lib.hgrn2_fwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn2_fwd.restype = I
        lib.hgrn2_bwd.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn2_bwd.restype = I
        lib.hgrn2_bwd_noalloc.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.hgrn2_bwd_noalloc.restype = I
        lib.hgrn2_fwd_chunk.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P]
        lib.hgrn2_fwd_chunk.restype = I
        lib.hgrn2_bwd_adjoint.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P]
        lib.hgrn2_bwd_adjoint.restype = I
        lib.hgrn2_bwd_chunk.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.hgrn2_bwd_chunk.restype = I
        lib.hgrn2_fwd_tied.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn2_fwd_tied.restype = I
        lib.hgrn2_bwd_tied.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn2_bwd_tied.restype = I
        lib.hgrn2_fwd_chunk_tied.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P]
        lib.hgrn2_fwd_chunk_tied.restype = I
        lib.hgrn2_bwd_chunk_tied.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P]
        lib.hgrn2_bwd_chunk_tied.restype = I
        lib.hgrn2_decode_step_tied.argtypes = [I, I, I, I, I, P, P, P, P, P, P]
        lib.hgrn2_decode_step_tied.restype = I
        lib.hgrn2_decode_step.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P]
        lib.hgrn2_decode_step.restype = I
        lib.hgrn2_bwd_gate_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
        lib.hgrn2_bwd_gate_workspace_bytes.restype = Z
        lib.hgrn2_fwd_gate.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn2_fwd_gate.restype = I
        lib.hgrn2_bwd_gate.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn2_bwd_gate.restype = I
        lib.hgrn2_decode_step_gate.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P]
        lib.hgrn2_decode_step_gate.restype = I
        for n in ("hgrn1_states_bytes",):
            getattr(lib, n).argtypes = [I, I, I]
            getattr(lib, n).restype = Z
        for n in ("hgrn1_fwd_workspace_bytes", "hgrn1_bwd_workspace_bytes"):
            getattr(lib, n).argtypes = [I, I, I, I]
            getattr(lib, n).restype = Z
        lib.hgrn2_fwd_scalar.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn2_fwd_scalar.restype = I
        lib.hgrn2_bwd_scalar.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn2_bwd_scalar.restype = I
        lib.hgrn2_decode_step_scalar.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P]
        lib.hgrn2_decode_step_scalar.restype = I
        lib.hgrn1_fwd.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn1_fwd.restype = I
        lib.hgrn1_bwd.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P, P, Z, P]
        lib.hgrn1_bwd.restype = I
        _handle = lib
    return _handle


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _lib()


def _check(status: int, where: str):
    if status != 0:
        raise HGRN2Error(status, where, _lib().hgrn2_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _tok(name, t, B, T, H, D, dtype):
    if t.shape != (B, T, H, D):
        raise ValueError("%s: expected shape %s, got %s" % (name, (B, T, H, D), tuple(t.shape)))
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s: expected a contiguous %s CUDA tensor" % (name, dtype))


def _st(name, t, B, H, D):
    if t is None:
        return
    if t.shape != (B, H, D, D) or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s: expected a contiguous float32 CUDA tensor of shape %s" % (name, (B, H, D, D)))


def supported(D: int, chunk: int, dtype: torch.dtype) -> bool:
    return bool(_lib().hgrn2_supported(D, chunk, _DT[dtype]))


def num_chunks(T: int, chunk: int) -> int:
    return int(_lib().hgrn2_num_chunks(T, chunk))


def states_shape(B, T, H, D, chunk):
    return (B, H, num_chunks(T, chunk) + 1, D, D)


def fwd(q, k, v, log_f, h0=None, *, chunk=64, want_ht=True, want_states=False, want_y=True,
        y=None, ht=None, states=None, ws=None, out_dtype=None):
    """Chunked forward.  Returns (y or None, ht or None, states or None).

    Without `states` the chunk-boundary states go to a workspace (`ws`, a
    uint8 CUDA tensor of at least hgrn2_fwd_workspace_bytes, allocated here
    if not given).  want_y=False runs the state scan alone (no y)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("k", k), ("v", v), ("log_f", log_f)):
        _tok(n, t, B, T, H, D, dt)
    _st("h0", h0, B, H, D)
    if want_y and y is None:
        y = torch.empty_like(q, dtype=odt)
    if y is not None:
        _tok("y", y, B, T, H, D, odt)
    if want_ht and ht is None:
        ht = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("ht", ht, B, H, D)
    if want_states and states is None:
        states = torch.empty(states_shape(B, T, H, D, chunk), dtype=dt, device=q.device)
    if states is not None and (tuple(states.shape) != states_shape(B, T, H, D, chunk)
                               or states.dtype != dt or not states.is_contiguous()):
        raise ValueError("states: expected %s %s" % (dt, states_shape(B, T, H, D, chunk)))
    ws_bytes = 0
    if states is None:
        need = int(_lib().hgrn2_fwd_workspace_bytes(B, T, H, D, D, chunk, _DT[dt], 0))
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = ws.numel() * ws.element_size()
    st = _lib().hgrn2_fwd(B, T, H, D, D, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(log_f),
                          _ptr(h0), _ptr(y), _ptr(ht), _ptr(states), _ptr(ws), ws_bytes, _stream())
    _check(st, "hgrn2_fwd")
    return y, ht, states


def bwd(q, k, v, log_f, dy, h0=None, dht=None, states=None, *, chunk=64, want_dh0=True,
        dq=None, dk=None, dv=None, dlog_f=None, dh0=None, ws=None, out_dtype=None):
    """Chunked backward.  Returns (dq, dk, dv, dlog_f, dh0 or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("k", k), ("v", v), ("log_f", log_f), ("dy", dy)):
        _tok(n, t, B, T, H, D, dt)
    _st("h0", h0, B, H, D)
    _st("dht", dht, B, H, D)
    dq = torch.empty_like(q, dtype=odt) if dq is None else dq
    dk = torch.empty_like(k, dtype=odt) if dk is None else dk
    dv = torch.empty_like(v, dtype=odt) if dv is None else dv
    dlog_f = torch.empty_like(log_f, dtype=odt) if dlog_f is None else dlog_f
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dlog_f", dlog_f)):
        _tok(n, t, B, T, H, D, odt)
    if want_dh0 and dh0 is None:
        dh0 = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("dh0", dh0, B, H, D)
    if states is not None and (tuple(states.shape) != states_shape(B, T, H, D, chunk) or states.dtype != dt
                               or not states.is_contiguous()):
        raise ValueError("states: expected %s %s" % (dt, states_shape(B, T, H, D, chunk)))
    need = int(_lib().hgrn2_bwd_workspace_bytes(B, T, H, D, D, chunk, _DT[dt], int(states is not None)))
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = ws.numel() * ws.element_size()
    st = _lib().hgrn2_bwd(B, T, H, D, D, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(log_f),
                          _ptr(h0), _ptr(states), _ptr(dy), _ptr(dht), _ptr(dq), _ptr(dk),
                          _ptr(dv), _ptr(dlog_f), _ptr(dh0), _ptr(ws), ws_bytes, _stream())
    _check(st, "hgrn2_bwd")
    return dq, dk, dv, dlog_f, dh0


# HGRN2_NOALLOC_SCRATCH_BYTES of include/hgrn2.h: the scratch hgrn2_bwd_noalloc uses
NOALLOC_SCRATCH_BYTES = 256 << 20


def bwd_noalloc(q, k, v, log_f, dy, h0=None, dht=None, states=None, *, chunk=64, dq=None, dk=None, dv=None,
                dlog_f=None, dh0=None, want_dh0=True, out_dtype=None):
    """hgrn2_bwd_noalloc: the chunked backward with the library's own scratch
    in place of a workspace (the library allocates nothing; outputs not passed
    are allocated here by torch).  Returns (dq, dk, dv, dlog_f, dh0 or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("k", k), ("v", v), ("log_f", log_f), ("dy", dy)):
        _tok(n, t, B, T, H, D, dt)
    _st("h0", h0, B, H, D)
    _st("dht", dht, B, H, D)
    dq = torch.empty_like(q, dtype=odt) if dq is None else dq
    dk = torch.empty_like(k, dtype=odt) if dk is None else dk
    dv = torch.empty_like(v, dtype=odt) if dv is None else dv
    dlog_f = torch.empty_like(log_f, dtype=odt) if dlog_f is None else dlog_f
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dlog_f", dlog_f)):
        _tok(n, t, B, T, H, D, odt)
    if want_dh0 and dh0 is None:
        dh0 = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("dh0", dh0, B, H, D)
    if states is not None:
        _states_ok(states, B, T, H, D, chunk, dt)
    st = _lib().hgrn2_bwd_noalloc(B, T, H, D, D, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(log_f), _ptr(h0),
                                  _ptr(states), _ptr(dy), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dlog_f),
                                  _ptr(dh0), _stream())
    _check(st, "hgrn2_bwd_noalloc")
    return dq, dk, dv, dlog_f, dh0


def _states_ok(states, B, T, H, D, chunk, dt):
    if (states is None or tuple(states.shape) != states_shape(B, T, H, D, chunk) or states.dtype != dt
            or not states.is_contiguous()):
        raise ValueError("states: expected a contiguous %s tensor of shape %s"
                         % (dt, states_shape(B, T, H, D, chunk)))


def adjoints_shape(B, T, H, D, chunk):
    return (B, H, num_chunks(T, chunk), D, D)


def fwd_chunk(q, k, v, log_f, states, *, chunk=64, y=None, out_dtype=None):
    """The per-chunk output launch of hgrn2_fwd alone (states from
    fwd(..., want_states=True) or fwd with y computed elsewhere).  Returns y."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("k", k), ("v", v), ("log_f", log_f)):
        _tok(n, t, B, T, H, D, dt)
    _states_ok(states, B, T, H, D, chunk, dt)
    y = torch.empty_like(q, dtype=odt) if y is None else y
    _tok("y", y, B, T, H, D, odt)
    st = _lib().hgrn2_fwd_chunk(B, T, H, D, D, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(log_f),
                                _ptr(states), _ptr(y), _stream())
    _check(st, "hgrn2_fwd_chunk")
    return y


def bwd_adjoint(q, log_f, dy, dht=None, *, chunk=64, adjoints=None, dh0=None, want_dh0=False):
    """The reverse adjoint scan of hgrn2_bwd alone.  Returns (adjoints, dh0 or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    for n, t in (("q", q), ("log_f", log_f), ("dy", dy)):
        _tok(n, t, B, T, H, D, dt)
    _st("dht", dht, B, H, D)
    if adjoints is None:
        adjoints = torch.empty(adjoints_shape(B, T, H, D, chunk), dtype=dt, device=q.device)
    if tuple(adjoints.shape) != adjoints_shape(B, T, H, D, chunk) or adjoints.dtype != dt \
            or not adjoints.is_contiguous():
        raise ValueError("adjoints: expected a contiguous %s tensor of shape %s"
                         % (dt, adjoints_shape(B, T, H, D, chunk)))
    if want_dh0 and dh0 is None:
        dh0 = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("dh0", dh0, B, H, D)
    st = _lib().hgrn2_bwd_adjoint(B, T, H, D, D, chunk, _DT[dt], _ptr(q), _ptr(log_f), _ptr(dy), _ptr(dht),
                                  _ptr(adjoints), _ptr(dh0), _stream())
    _check(st, "hgrn2_bwd_adjoint")
    return adjoints, dh0


def bwd_chunk(q, k, v, log_f, dy, states, adjoints, *, chunk=64, dq=None, dk=None, dv=None, dlog_f=None, out_dtype=None):
    """The per-chunk gradient launch of hgrn2_bwd alone.  Returns (dq, dk, dv, dlog_f)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("k", k), ("v", v), ("log_f", log_f), ("dy", dy)):
        _tok(n, t, B, T, H, D, dt)
    _states_ok(states, B, T, H, D, chunk, dt)
    if tuple(adjoints.shape) != adjoints_shape(B, T, H, D, chunk) or adjoints.dtype != dt \
            or not adjoints.is_contiguous():
        raise ValueError("adjoints: expected a contiguous %s tensor of shape %s"
                         % (dt, adjoints_shape(B, T, H, D, chunk)))
    dq = torch.empty_like(q, dtype=odt) if dq is None else dq
    dk = torch.empty_like(k, dtype=odt) if dk is None else dk
    dv = torch.empty_like(v, dtype=odt) if dv is None else dv
    dlog_f = torch.empty_like(log_f, dtype=odt) if dlog_f is None else dlog_f
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dlog_f", dlog_f)):
        _tok(n, t, B, T, H, D, odt)
    st = _lib().hgrn2_bwd_chunk(B, T, H, D, D, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(log_f),
                                _ptr(states), _ptr(adjoints), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv),
                                _ptr(dlog_f), _stream())
    _check(st, "hgrn2_bwd_chunk")
    return dq, dk, dv, dlog_f


def decode_step(q, k, v, log_f, state, *, y=None, out_dtype=None):
    """One recurrent step; `state` [B,H,D,D] float32 is updated in place.  Returns y [B,H,D]."""
    B, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("k", k), ("v", v), ("log_f", log_f)):
        if t.shape != (B, H, D) or t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s: expected a contiguous %s CUDA tensor of shape %s" % (n, dt, (B, H, D)))
    _st("state", state, B, H, D)
    if y is None:
        y = torch.empty_like(q, dtype=odt)
    _vec3("y", y, B, H, D, odt)
    st = _lib().hgrn2_decode_step(B, H, D, D, code, _ptr(q), _ptr(k), _ptr(v), _ptr(log_f),
                                  _ptr(state), _ptr(y), _stream())
    _check(st, "hgrn2_decode_step")
    return y


# ------------------------------------------------------------------ tied gates
# k = 1 - exp(log_f) is formed in the kernels; the backward returns the total
# derivative with respect to log_f and no dk.

def fwd_tied(q, v, log_f, h0=None, *, chunk=64, want_ht=True, want_states=False, want_y=True,
             y=None, ht=None, states=None, ws=None, out_dtype=None):
    """Chunked forward with tied gates.  Returns (y or None, ht or None, states or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("log_f", log_f)):
        _tok(n, t, B, T, H, D, dt)
    _st("h0", h0, B, H, D)
    if want_y and y is None:
        y = torch.empty_like(q, dtype=odt)
    if y is not None:
        _tok("y", y, B, T, H, D, odt)
    if want_ht and ht is None:
        ht = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("ht", ht, B, H, D)
    if want_states and states is None:
        states = torch.empty(states_shape(B, T, H, D, chunk), dtype=dt, device=q.device)
    if states is not None:
        _states_ok(states, B, T, H, D, chunk, dt)
    ws_bytes = 0
    if states is None:
        need = int(_lib().hgrn2_fwd_workspace_bytes(B, T, H, D, D, chunk, _DT[dt], 0))
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = ws.numel() * ws.element_size()
    st = _lib().hgrn2_fwd_tied(B, T, H, D, D, chunk, code, _ptr(q), _ptr(v), _ptr(log_f), _ptr(h0),
                               _ptr(y), _ptr(ht), _ptr(states), _ptr(ws), ws_bytes, _stream())
    _check(st, "hgrn2_fwd_tied")
    return y, ht, states


def bwd_tied(q, v, log_f, dy, h0=None, dht=None, states=None, *, chunk=64, want_dh0=True,
             dq=None, dv=None, dlog_f=None, dh0=None, ws=None, out_dtype=None):
    """Chunked backward with tied gates.  Returns (dq, dv, dlog_f total, dh0 or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("log_f", log_f), ("dy", dy)):
        _tok(n, t, B, T, H, D, dt)
    _st("h0", h0, B, H, D)
    _st("dht", dht, B, H, D)
    dq = torch.empty_like(q, dtype=odt) if dq is None else dq
    dv = torch.empty_like(v, dtype=odt) if dv is None else dv
    dlog_f = torch.empty_like(log_f, dtype=odt) if dlog_f is None else dlog_f
    for n, t in (("dq", dq), ("dv", dv), ("dlog_f", dlog_f)):
        _tok(n, t, B, T, H, D, odt)
    if want_dh0 and dh0 is None:
        dh0 = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("dh0", dh0, B, H, D)
    if states is not None:
        _states_ok(states, B, T, H, D, chunk, dt)
    need = int(_lib().hgrn2_bwd_workspace_bytes(B, T, H, D, D, chunk, _DT[dt], int(states is not None)))
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = ws.numel() * ws.element_size()
    st = _lib().hgrn2_bwd_tied(B, T, H, D, D, chunk, code, _ptr(q), _ptr(v), _ptr(log_f), _ptr(h0),
                               _ptr(states), _ptr(dy), _ptr(dht), _ptr(dq), _ptr(dv), _ptr(dlog_f), _ptr(dh0),
                               _ptr(ws), ws_bytes, _stream())
    _check(st, "hgrn2_bwd_tied")
    return dq, dv, dlog_f, dh0


def fwd_chunk_tied(q, v, log_f, states, *, chunk=64, y=None, out_dtype=None):
    """The per-chunk output launch of hgrn2_fwd_tied alone.  Returns y."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("log_f", log_f)):
        _tok(n, t, B, T, H, D, dt)
    _states_ok(states, B, T, H, D, chunk, dt)
    y = torch.empty_like(q, dtype=odt) if y is None else y
    _tok("y", y, B, T, H, D, odt)
    st = _lib().hgrn2_fwd_chunk_tied(B, T, H, D, D, chunk, code, _ptr(q), _ptr(v), _ptr(log_f),
                                     _ptr(states), _ptr(y), _stream())
    _check(st, "hgrn2_fwd_chunk_tied")
    return y


def bwd_chunk_tied(q, v, log_f, dy, states, adjoints, *, chunk=64, dq=None, dv=None, dlog_f=None, out_dtype=None):
    """The per-chunk gradient launch of hgrn2_bwd_tied alone.  Returns (dq, dv, dlog_f total)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("log_f", log_f), ("dy", dy)):
        _tok(n, t, B, T, H, D, dt)
    _states_ok(states, B, T, H, D, chunk, dt)
    if tuple(adjoints.shape) != adjoints_shape(B, T, H, D, chunk) or adjoints.dtype != dt \
            or not adjoints.is_contiguous():
        raise ValueError("adjoints: expected a contiguous %s tensor of shape %s"
                         % (dt, adjoints_shape(B, T, H, D, chunk)))
    dq = torch.empty_like(q, dtype=odt) if dq is None else dq
    dv = torch.empty_like(v, dtype=odt) if dv is None else dv
    dlog_f = torch.empty_like(log_f, dtype=odt) if dlog_f is None else dlog_f
    for n, t in (("dq", dq), ("dv", dv), ("dlog_f", dlog_f)):
        _tok(n, t, B, T, H, D, odt)
    st = _lib().hgrn2_bwd_chunk_tied(B, T, H, D, D, chunk, code, _ptr(q), _ptr(v), _ptr(log_f), _ptr(states),
                                     _ptr(adjoints), _ptr(dy), _ptr(dq), _ptr(dv), _ptr(dlog_f), _stream())
    _check(st, "hgrn2_bwd_chunk_tied")
    return dq, dv, dlog_f


def decode_step_tied(q, v, log_f, state, *, y=None, out_dtype=None):
    """One recurrent step with k = 1 - exp(log_f); `state` is updated in place.  Returns y."""
    B, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("log_f", log_f)):
        if t.shape != (B, H, D) or t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s: expected a contiguous %s CUDA tensor of shape %s" % (n, dt, (B, H, D)))
    _st("state", state, B, H, D)
    if y is None:
        y = torch.empty_like(q, dtype=odt)
    _vec3("y", y, B, H, D, odt)
    st = _lib().hgrn2_decode_step_tied(B, H, D, D, code, _ptr(q), _ptr(v), _ptr(log_f), _ptr(state), _ptr(y),
                                       _stream())
    _check(st, "hgrn2_decode_step_tied")
    return y


def _lb(lower_bound, H, D, device):
    if lower_bound.shape != (H, D) or lower_bound.dtype != torch.float32 or not lower_bound.is_contiguous() \
            or lower_bound.device != device:
        raise ValueError("lower_bound: expected a contiguous float32 tensor of shape %s on %s" % ((H, D), device))


def fwd_gate(q, v, z, lower_bound, h0=None, *, chunk=64, want_ht=True, want_states=False, want_y=True,
             y=None, ht=None, states=None, ws=None, out_dtype=None):
    """Chunked forward with the gate formed from its pre-activation z and the
    lower bound [H, D] (f = lb + (1 - lb) sigmoid(z), k = 1 - f).
    Returns (y or None, ht or None, states or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("z", z)):
        _tok(n, t, B, T, H, D, dt)
    _lb(lower_bound, H, D, q.device)
    _st("h0", h0, B, H, D)
    if want_y and y is None:
        y = torch.empty_like(q, dtype=odt)
    if y is not None:
        _tok("y", y, B, T, H, D, odt)
    if want_ht and ht is None:
        ht = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("ht", ht, B, H, D)
    if want_states and states is None:
        states = torch.empty(states_shape(B, T, H, D, chunk), dtype=dt, device=q.device)
    if states is not None:
        _states_ok(states, B, T, H, D, chunk, dt)
    ws_bytes = 0
    if states is None:
        need = int(_lib().hgrn2_fwd_workspace_bytes(B, T, H, D, D, chunk, _DT[dt], 0))
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = ws.numel() * ws.element_size()
    st = _lib().hgrn2_fwd_gate(B, T, H, D, D, chunk, code, _ptr(q), _ptr(v), _ptr(z), _ptr(lower_bound),
                               _ptr(h0), _ptr(y), _ptr(ht), _ptr(states), _ptr(ws), ws_bytes, _stream())
    _check(st, "hgrn2_fwd_gate")
    return y, ht, states


def bwd_gate(q, v, z, lower_bound, dy, h0=None, dht=None, states=None, *, chunk=64, want_dh0=True,
             dq=None, dv=None, dz=None, dlower_bound=None, dh0=None, ws=None, out_dtype=None):
    """Chunked backward with the gate formed from its pre-activation.
    Returns (dq, dv, dz, dlower_bound [H, D] float32, dh0 or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("z", z), ("dy", dy)):
        _tok(n, t, B, T, H, D, dt)
    _lb(lower_bound, H, D, q.device)
    _st("h0", h0, B, H, D)
    _st("dht", dht, B, H, D)
    dq = torch.empty_like(q, dtype=odt) if dq is None else dq
    dv = torch.empty_like(v, dtype=odt) if dv is None else dv
    dz = torch.empty_like(z, dtype=odt) if dz is None else dz
    for n, t in (("dq", dq), ("dv", dv), ("dz", dz)):
        _tok(n, t, B, T, H, D, odt)
    if dlower_bound is None:
        dlower_bound = torch.empty((H, D), dtype=torch.float32, device=q.device)
    _lb(dlower_bound, H, D, q.device)
    if want_dh0 and dh0 is None:
        dh0 = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("dh0", dh0, B, H, D)
    if states is not None:
        _states_ok(states, B, T, H, D, chunk, dt)
    need = int(_lib().hgrn2_bwd_gate_workspace_bytes(B, T, H, D, D, chunk, _DT[dt], int(states is not None)))
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = ws.numel() * ws.element_size()
    st = _lib().hgrn2_bwd_gate(B, T, H, D, D, chunk, code, _ptr(q), _ptr(v), _ptr(z), _ptr(lower_bound),
                               _ptr(h0), _ptr(states), _ptr(dy), _ptr(dht), _ptr(dq), _ptr(dv), _ptr(dz),
                               _ptr(dlower_bound), _ptr(dh0), _ptr(ws), ws_bytes, _stream())
    _check(st, "hgrn2_bwd_gate")
    return dq, dv, dz, dlower_bound, dh0


def decode_step_gate(q, v, z, lower_bound, state, *, y=None, out_dtype=None):
    """One recurrent step with the gate formed from z [B, H, D] and the lower
    bound [H, D]; `state` is updated in place.  Returns y."""
    B, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("z", z)):
        if t.shape != (B, H, D) or t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s: expected a contiguous %s CUDA tensor of shape %s" % (n, dt, (B, H, D)))
    _lb(lower_bound, H, D, q.device)
    _st("state", state, B, H, D)
    if y is None:
        y = torch.empty_like(q, dtype=odt)
    _vec3("y", y, B, H, D, odt)
    st = _lib().hgrn2_decode_step_gate(B, H, D, D, code, _ptr(q), _ptr(v), _ptr(z), _ptr(lower_bound),
                                       _ptr(state), _ptr(y), _stream())
    _check(st, "hgrn2_decode_step_gate")
    return y


def fwd_scalar(q, k, v, log_a, h0=None, *, chunk=64, want_ht=True, want_states=False, want_y=True,
               y=None, ht=None, states=None, ws=None, out_dtype=None):
    """Chunked forward with one decay per head, log_a [B, T, H].
    Returns (y or None, ht or None, states or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _tok(n, t, B, T, H, D, dt)
    _tok3("log_a", log_a, B, T, H, dt)
    _st("h0", h0, B, H, D)
    if want_y and y is None:
        y = torch.empty_like(q, dtype=odt)
    if y is not None:
        _tok("y", y, B, T, H, D, odt)
    if want_ht and ht is None:
        ht = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("ht", ht, B, H, D)
    if want_states and states is None:
        states = torch.empty(states_shape(B, T, H, D, chunk), dtype=dt, device=q.device)
    if states is not None:
        _states_ok(states, B, T, H, D, chunk, dt)
    ws_bytes = 0
    if states is None:
        need = int(_lib().hgrn2_fwd_workspace_bytes(B, T, H, D, D, chunk, _DT[dt], 0))
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = ws.numel() * ws.element_size()
    st = _lib().hgrn2_fwd_scalar(B, T, H, D, D, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(h0),
                                 _ptr(y), _ptr(ht), _ptr(states), _ptr(ws), ws_bytes, _stream())
    _check(st, "hgrn2_fwd_scalar")
    return y, ht, states


def bwd_scalar(q, k, v, log_a, dy, h0=None, dht=None, states=None, *, chunk=64, want_dh0=True,
               dq=None, dk=None, dv=None, dlog_a=None, dh0=None, ws=None, out_dtype=None):
    """Chunked backward with one decay per head.  Returns (dq, dk, dv, dlog_a [B, T, H], dh0 or None)."""
    B, T, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("k", k), ("v", v), ("dy", dy)):
        _tok(n, t, B, T, H, D, dt)
    _tok3("log_a", log_a, B, T, H, dt)
    _st("h0", h0, B, H, D)
    _st("dht", dht, B, H, D)
    dq = torch.empty_like(q, dtype=odt) if dq is None else dq
    dk = torch.empty_like(k, dtype=odt) if dk is None else dk
    dv = torch.empty_like(v, dtype=odt) if dv is None else dv
    dlog_a = torch.empty_like(log_a, dtype=odt) if dlog_a is None else dlog_a
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _tok(n, t, B, T, H, D, odt)
    _tok3("dlog_a", dlog_a, B, T, H, odt)
    if want_dh0 and dh0 is None:
        dh0 = torch.empty((B, H, D, D), dtype=torch.float32, device=q.device)
    _st("dh0", dh0, B, H, D)
    if states is not None:
        _states_ok(states, B, T, H, D, chunk, dt)
    need = int(_lib().hgrn2_bwd_workspace_bytes(B, T, H, D, D, chunk, _DT[dt], int(states is not None)))
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = ws.numel() * ws.element_size()
    st = _lib().hgrn2_bwd_scalar(B, T, H, D, D, chunk, code, _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(h0),
                                 _ptr(states), _ptr(dy), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dlog_a),
                                 _ptr(dh0), _ptr(ws), ws_bytes, _stream())
    _check(st, "hgrn2_bwd_scalar")
    return dq, dk, dv, dlog_a, dh0


def decode_step_scalar(q, k, v, log_a, state, *, y=None, out_dtype=None):
    """One recurrent step with one decay per head, log_a [B, H]; `state` is updated in place.  Returns y."""
    B, H, D = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("k", k), ("v", v)):
        if t.shape != (B, H, D) or t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s: expected a contiguous %s CUDA tensor of shape %s" % (n, dt, (B, H, D)))
    if log_a.shape != (B, H) or log_a.dtype != dt or not log_a.is_cuda or not log_a.is_contiguous():
        raise ValueError("log_a: expected a contiguous %s CUDA tensor of shape %s" % (dt, (B, H)))
    _st("state", state, B, H, D)
    if y is None:
        y = torch.empty_like(q, dtype=odt)
    _vec3("y", y, B, H, D, odt)
    st = _lib().hgrn2_decode_step_scalar(B, H, D, D, code, _ptr(q), _ptr(k), _ptr(v), _ptr(log_a), _ptr(state),
                                         _ptr(y), _stream())
    _check(st, "hgrn2_decode_step_scalar")
    return y


def _vec3(name, t, B, H, D, dtype):
    if t.shape != (B, H, D) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s: expected a contiguous %s CUDA tensor of shape %s" % (name, dtype, (B, H, D)))


def _tok3(name, t, B, T, C, dtype):
    if t.shape != (B, T, C) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s: expected a contiguous %s CUDA tensor of shape %s" % (name, dtype, (B, T, C)))


def _vec(name, t, B, C):
    if t is None:
        return
    if t.shape != (B, C) or t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s: expected a contiguous float32 CUDA tensor of shape %s" % (name, (B, C)))


def hgrn1_states_shape(B, T, C):
    return (B, (T + 31) // 32, C)


def hgrn1_fwd(q, k, v, log_f, h0=None, *, tied=False, want_ht=True, want_states=False, y=None, ht=None,
              states=None, ws=None, out_dtype=None):
    """HGRN1 elementwise recurrence over [B, T, C] tensors (k = 1 - exp(log_f)
    when tied; k is then ignored).  Returns (y, hT or None, states or None)."""
    B, T, C = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("log_f", log_f)) + ((("k", k),) if not tied else ()):
        _tok3(n, t, B, T, C, dt)
    _vec("h0", h0, B, C)
    y = torch.empty_like(q, dtype=odt) if y is None else y
    _tok3("y", y, B, T, C, odt)
    if want_ht and ht is None:
        ht = torch.empty((B, C), dtype=torch.float32, device=q.device)
    _vec("hT", ht, B, C)
    if want_states and states is None:
        states = torch.empty(hgrn1_states_shape(B, T, C), dtype=torch.float32, device=q.device)
    if states is not None and (tuple(states.shape) != hgrn1_states_shape(B, T, C) or states.dtype != torch.float32
                               or not states.is_cuda or not states.is_contiguous()):
        raise ValueError("states: expected a contiguous float32 CUDA tensor of shape %s"
                         % (hgrn1_states_shape(B, T, C),))
    need = int(_lib().hgrn1_fwd_workspace_bytes(B, T, C, int(states is not None)))
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = _lib().hgrn1_fwd(B, T, C, code, int(tied), _ptr(q), None if tied else _ptr(k), _ptr(v), _ptr(log_f),
                          _ptr(h0), _ptr(y), _ptr(ht), _ptr(states), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream())
    _check(st, "hgrn1_fwd")
    return y, ht, states


def hgrn1_bwd(q, k, v, log_f, dy, h0=None, dht=None, states=None, *, tied=False, want_dh0=True,
              dq=None, dk=None, dv=None, dlog_f=None, dh0=None, ws=None, out_dtype=None):
    """Backward of hgrn1_fwd.  Returns (dq, dk or None (tied), dv, dlog_f, dh0 or None);
    tied: dlog_f is the total derivative."""
    B, T, C = q.shape
    dt = q.dtype
    odt, code = _odt(dt, out_dtype)
    for n, t in (("q", q), ("v", v), ("log_f", log_f), ("dy", dy)) + ((("k", k),) if not tied else ()):
        _tok3(n, t, B, T, C, dt)
    _vec("h0", h0, B, C)
    _vec("dht", dht, B, C)
    dq = torch.empty_like(q, dtype=odt) if dq is None else dq
    dv = torch.empty_like(q, dtype=odt) if dv is None else dv
    dlog_f = torch.empty_like(q, dtype=odt) if dlog_f is None else dlog_f
    if not tied and dk is None:
        dk = torch.empty_like(q, dtype=odt)
    for n, t in (("dq", dq), ("dv", dv), ("dlog_f", dlog_f)) + ((("dk", dk),) if not tied else ()):
        _tok3(n, t, B, T, C, odt)
    if want_dh0 and dh0 is None:
        dh0 = torch.empty((B, C), dtype=torch.float32, device=q.device)
    _vec("dh0", dh0, B, C)
    if states is not None and (tuple(states.shape) != hgrn1_states_shape(B, T, C) or states.dtype != torch.float32
                               or not states.is_contiguous()):
        raise ValueError("states: expected a contiguous float32 tensor of shape %s" % (hgrn1_states_shape(B, T, C),))
    need = int(_lib().hgrn1_bwd_workspace_bytes(B, T, C, int(states is not None)))
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = _lib().hgrn1_bwd(B, T, C, code, int(tied), _ptr(q), None if tied else _ptr(k), _ptr(v), _ptr(log_f),
                          _ptr(h0), _ptr(states), _ptr(dy), _ptr(dht), _ptr(dq), None if tied else _ptr(dk),
                          _ptr(dv), _ptr(dlog_f), _ptr(dh0), _ptr(ws), ws.numel() * ws.element_size(), _stream())
    _check(st, "hgrn1_bwd")
    return dq, (None if tied else dk), dv, dlog_f, dh0


class HGRN2Chunk(torch.autograd.Function):
    """Autograd wrapper: y, ht = HGRN2Chunk.apply(q, k, v, log_f, h0, chunk, out_dtype).

    k and log_f are independent inputs (a caller tying k = 1 - exp(log_f) in
    torch gets the tied gradient from autograd through that expression).
    out_dtype=torch.float32 with bfloat16 inputs returns y in float32; the
    incoming dy is then taken in the input dtype (the kernels use it as a
    bfloat16 matrix-core operand either way) and the gradients keep the
    inputs' dtype, as autograd requires."""

    @staticmethod
    def forward(ctx, q, k, v, log_f, h0, chunk, out_dtype=None):
        y, ht, states = fwd(q, k, v, log_f, h0, chunk=chunk, want_ht=True, want_states=True, out_dtype=out_dtype)
        ctx.save_for_backward(q, k, v, log_f, h0, states)
        ctx.chunk = chunk
        return y, ht

    @staticmethod
    def backward(ctx, dy, dht):
        q, k, v, log_f, h0, states = ctx.saved_tensors
        dy = dy.to(q.dtype).contiguous() if dy is not None else torch.zeros_like(q)
        dht = dht.contiguous() if dht is not None else None
        dq, dk, dv, dl, dh0 = bwd(q, k, v, log_f, dy, h0, dht, states, chunk=ctx.chunk,
                                  want_dh0=h0 is not None)
        return dq, dk, dv, dl, dh0, None, None


def hgrn2_chunk(q, k, v, log_f, h0=None, chunk=64, out_dtype=None):
    """Differentiable chunked HGRN2 recurrence: returns (y, ht)."""
    return HGRN2Chunk.apply(q, k, v, log_f, h0, chunk, out_dtype)
