"""MI355X (gfx950) Gated DeltaNet token mixer -- Python binding.

A thin ctypes layer over the C ABI in ``include/gdn.h`` (``libgdn.so``, built
in-tree by ``python -m linear_attention_sequence_gdn_amd.build``).  Every step
of the mixer runs in the library's HIP kernels; PyTorch is used only to hold
device memory and to name the current stream.  There is no fallback: if the
library is missing, every call raises.

Functions mirror the ABI names:

* ``gdn_prefill``        -- B sequences of equal length T
* ``gdn_prefill_varlen`` -- packed sequences addressed by ``cu_seqlens``
* ``gdn_decode_step``    -- one new token for each of B sequences
* ``gdn_decode_multi``   -- 1..4 new tokens per sequence, optional state-cache slots
* ``gdn_prefill_workspace_size`` / ``gdn_prefill_varlen_workspace_size``
* ``gdn_status_string``

Tensors are torch tensors on the GPU: q/k/v/conv weights/conv states/o in
``torch.bfloat16``, a/b/states in ``torch.float32``, cu_seqlens in
``torch.int32``, all contiguous.
"""
from __future__ import annotations

import ctypes
import os

from . import inputs  # noqa: F401  (seeded synthetic inputs; no mixer arithmetic)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "gdn.h")

GDN_OK = 0
GDN_ERR_INVALID_ARGUMENT = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_WORKSPACE_TOO_SMALL = 3
GDN_ERR_HIP = 4

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t


class GDNError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {gdn_status_string(status)} ({status})")
        self.status = status


def lib():
    """The loaded ``libgdn.so`` (ctypes), with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} is not built; run "
                "`python -m linear_attention_sequence_gdn_amd.build` (there is no CPU fallback)")
        # The library and torch must share one HIP runtime.  torch ships its
        # own libamdhip64 (soname libamdhip64.so.7, loaded from torch's
        # directory); the library names libamdhip64.so.7.  Importing torch
        # first puts that runtime in the process, and the library then binds
        # to it by soname.  Loaded the other way round, the process would hold
        # two HIP runtimes, and the one the library calls into sees no device.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_status_string.argtypes = [_I]
        L.gdn_prefill_workspace_size.restype = _SZ
        L.gdn_prefill_workspace_size.argtypes = [_I] * 6
        L.gdn_prefill_varlen_workspace_size.restype = _SZ
        L.gdn_prefill_varlen_workspace_size.argtypes = [_I] * 6
        L.gdn_prefill.restype = _I
        L.gdn_prefill.argtypes = [_P] * 11 + [_I] * 6 + [_F, _F, _P, _SZ, _P]
        L.gdn_prefill_varlen.restype = _I
        L.gdn_prefill_varlen.argtypes = [_P] * 12 + [_I] * 6 + [_F, _F, _P, _SZ, _P]
        L.gdn_decode_step.restype = _I
        L.gdn_decode_step.argtypes = [_P] * 10 + [_I] * 5 + [_F, _F, _P]
        L.gdn_prefill_backward_workspace_size.restype = _SZ
        L.gdn_prefill_backward_workspace_size.argtypes = [_I] * 6
        L.gdn_prefill_backward_windows.restype = _I
        L.gdn_prefill_backward_windows.argtypes = [_I] * 6 + [_SZ, ctypes.POINTER(_I)]
        L.gdn_prefill_backward.restype = _I
        L.gdn_prefill_backward.argtypes = [_P] * 18 + [_I] * 6 + [_F, _F, _P, _SZ, _P]
        L.gdn_prefill_backward_varlen_workspace_size.restype = _SZ
        L.gdn_prefill_backward_varlen_workspace_size.argtypes = [_I] * 6
        L.gdn_prefill_backward_varlen.restype = _I
        L.gdn_prefill_backward_varlen.argtypes = [_P] * 19 + [_I] * 6 + [_F, _F, _P, _SZ, _P]
        L.gdn_decode_multi.restype = _I
        L.gdn_decode_multi.argtypes = [_P] * 11 + [_I] * 7 + [_F, _F, _P]
        L.gdn_prefill_with_options.restype = _I
        L.gdn_prefill_with_options.argtypes = [_P] * 11 + [_I] * 6 + [_F, _F, _P, _SZ, _P, _I, _P]
        L.gdn_prefill_varlen_slots.restype = _I
        L.gdn_prefill_varlen_slots.argtypes = [_P] * 13 + [_I] * 7 + [_F, _F, _P, _SZ, _P]
        L.gdn_prefill_noalloc.restype = _I
        L.gdn_prefill_noalloc.argtypes = [_P] * 11 + [_I] * 6 + [_F, _F, _P]
        L.gdn_prefill_noalloc_max_workspace.restype = _SZ
        L.gdn_prefill_noalloc_max_workspace.argtypes = []
        _lib = L
    return _lib


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def gdn_prefill_workspace_size(B, T, Hqk, Hv, dk=128, dv=128) -> int:
    return int(lib().gdn_prefill_workspace_size(B, T, Hqk, Hv, dk, dv))


def gdn_prefill_varlen_workspace_size(N, T_tot, Hqk, Hv, dk=128, dv=128) -> int:
    return int(lib().gdn_prefill_varlen_workspace_size(N, T_tot, Hqk, Hv, dk, dv))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(x):
    return None if x is None else ctypes.c_void_p(x.data_ptr())


def _check(x, name, dtype, shape=None):
    if x is None:
        return
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {x.dtype}")
    if not x.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def gdn_prefill(q, k, v, a, b, conv_w, *, gate_scale, q_scale=1.0, state_in=None,
                conv_state_in=None, state_out=None, o=None, conv_state_out=None,
                workspace=None, stream=None):
    """Chunked prefill of B equal-length sequences.

    q, k: [B][T][Hqk][128] bf16; v: [B][T][Hv][128] bf16; a, b: [B][T][Hv]
    fp32; conv_w: [C_tot][4] bf16; state_in: [B][Hv][128][128] fp32 or None;
    conv_state_in / conv_state_out: [B][3][C_tot] bf16 or None.
    Returns (o, state_out, conv_state_out).
    """
    torch = _torch()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    C_tot = 2 * Hqk * dk + Hv * dv
    bf, f32 = torch.bfloat16, torch.float32
    _check(q, "q", bf, (B, T, Hqk, dk))
    _check(k, "k", bf, (B, T, Hqk, dk))
    _check(v, "v", bf, (B, T, Hv, dv))
    _check(a, "a", f32, (B, T, Hv))
    _check(b, "b", f32, (B, T, Hv))
    _check(conv_w, "conv_w", bf, (C_tot, 4))
    _check(state_in, "state_in", f32, (B, Hv, dk, dv))
    _check(conv_state_in, "conv_state_in", bf, (B, 3, C_tot))
    dev = q.device
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=bf, device=dev)
    if state_out is None:
        state_out = torch.empty((B, Hv, dk, dv), dtype=f32, device=dev)
    _check(o, "o", bf, (B, T, Hv, dv))
    _check(state_out, "state_out", f32, (B, Hv, dk, dv))
    _check(conv_state_out, "conv_state_out", bf, (B, 3, C_tot))
    need = gdn_prefill_workspace_size(B, T, Hqk, Hv, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib().gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                           _ptr(conv_state_in), _ptr(conv_state_out), _ptr(state_in),
                           _ptr(state_out), _ptr(o), B, T, Hqk, Hv, dk, dv,
                           float(gate_scale), float(q_scale), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != GDN_OK:
        raise GDNError("gdn_prefill", rc)
    return o, state_out, conv_state_out


def gdn_prefill_noalloc_max_workspace() -> int:
    return int(lib().gdn_prefill_noalloc_max_workspace())


def gdn_prefill_noalloc(q, k, v, a, b, conv_w, *, gate_scale, q_scale=1.0, state_in=None,
                        conv_state_in=None, state_out=None, o=None, conv_state_out=None, stream=None):
    """``gdn_prefill`` with the library's own device workspace (no workspace
    argument, nothing allocated by the library).  Outputs default to new
    tensors, as in ``gdn_prefill``; pass ``o`` and ``state_out`` to allocate
    nothing at all.  Returns (o, state_out, conv_state_out)."""
    torch = _torch()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    C_tot = 2 * Hqk * dk + Hv * dv
    bf, f32 = torch.bfloat16, torch.float32
    _check(q, "q", bf, (B, T, Hqk, dk))
    _check(k, "k", bf, (B, T, Hqk, dk))
    _check(v, "v", bf, (B, T, Hv, dv))
    _check(a, "a", f32, (B, T, Hv))
    _check(b, "b", f32, (B, T, Hv))
    _check(conv_w, "conv_w", bf, (C_tot, 4))
    _check(state_in, "state_in", f32, (B, Hv, dk, dv))
    _check(conv_state_in, "conv_state_in", bf, (B, 3, C_tot))
    dev = q.device
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=bf, device=dev)
    if state_out is None:
        state_out = torch.empty((B, Hv, dk, dv), dtype=f32, device=dev)
    _check(o, "o", bf, (B, T, Hv, dv))
    _check(state_out, "state_out", f32, (B, Hv, dk, dv))
    _check(conv_state_out, "conv_state_out", bf, (B, 3, C_tot))
    rc = lib().gdn_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                                   _ptr(conv_state_in), _ptr(conv_state_out), _ptr(state_in),
                                   _ptr(state_out), _ptr(o), B, T, Hqk, Hv, dk, dv,
                                   float(gate_scale), float(q_scale), _stream(stream))
    if rc != GDN_OK:
        raise GDNError("gdn_prefill_noalloc", rc)
    return o, state_out, conv_state_out


def gdn_prefill_backward_workspace_size(B, T, Hqk, Hv, dk=128, dv=128) -> int:
    return int(lib().gdn_prefill_backward_workspace_size(B, T, Hqk, Hv, dk, dv))


def gdn_prefill_backward_windows(B, T, Hqk, Hv, workspace_bytes, dk=128, dv=128) -> int:
    """Window length ``gdn_prefill_backward`` takes with ``workspace_bytes`` of
    workspace: T when the batch runs at once, else the window length of its
    sequence-by-sequence run.  Raises GDNError when not even 64-token windows
    fit."""
    out = _I(0)
    rc = lib().gdn_prefill_backward_windows(B, T, Hqk, Hv, dk, dv, int(workspace_bytes), ctypes.byref(out))
    if rc != GDN_OK:
        raise GDNError("gdn_prefill_backward_windows", rc)
    return int(out.value)


def gdn_prefill_backward(q, k, v, a, b, conv_w, grad_o, *, gate_scale, q_scale=1.0,
                         state_in=None, conv_state_in=None, grad_state_out=None,
                         want_conv_state=False, want_state=True, workspace=None, stream=None):
    """Gradients of sum <grad_o, o> + <grad_state_out, state_out> of
    ``gdn_prefill`` with respect to its inputs (fp32 tensors).

    grad_o: [B][T][Hv][128] bf16; grad_state_out: [B][Hv][128][128] fp32 or
    None.  Returns a dict with q, k, v, a, b, conv_w and, when asked for,
    conv_state [B][3][C_tot] and state [B][Hv][128][128].
    """
    torch = _torch()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    C_tot = 2 * Hqk * dk + Hv * dv
    bf, f32 = torch.bfloat16, torch.float32
    _check(q, "q", bf, (B, T, Hqk, dk))
    _check(k, "k", bf, (B, T, Hqk, dk))
    _check(v, "v", bf, (B, T, Hv, dv))
    _check(a, "a", f32, (B, T, Hv))
    _check(b, "b", f32, (B, T, Hv))
    _check(conv_w, "conv_w", bf, (C_tot, 4))
    _check(state_in, "state_in", f32, (B, Hv, dk, dv))
    _check(conv_state_in, "conv_state_in", bf, (B, 3, C_tot))
    _check(grad_o, "grad_o", bf, (B, T, Hv, dv))
    _check(grad_state_out, "grad_state_out", f32, (B, Hv, dk, dv))
    dev = q.device
    g = {"q": torch.empty((B, T, Hqk, dk), dtype=f32, device=dev),
         "k": torch.empty((B, T, Hqk, dk), dtype=f32, device=dev),
         "v": torch.empty((B, T, Hv, dv), dtype=f32, device=dev),
         "a": torch.empty((B, T, Hv), dtype=f32, device=dev),
         "b": torch.empty((B, T, Hv), dtype=f32, device=dev),
         "conv_w": torch.empty((C_tot, 4), dtype=f32, device=dev),
         "conv_state": torch.empty((B, 3, C_tot), dtype=f32, device=dev) if want_conv_state else None,
         "state": torch.empty((B, Hv, dk, dv), dtype=f32, device=dev) if want_state else None}
    need = gdn_prefill_backward_workspace_size(B, T, Hqk, Hv, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib().gdn_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w), _ptr(conv_state_in),
        _ptr(state_in), _ptr(grad_o), _ptr(grad_state_out), _ptr(g["q"]), _ptr(g["k"]),
        _ptr(g["v"]), _ptr(g["a"]), _ptr(g["b"]), _ptr(g["conv_w"]), _ptr(g["conv_state"]),
        _ptr(g["state"]), B, T, Hqk, Hv, dk, dv, float(gate_scale), float(q_scale),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != GDN_OK:
        raise GDNError("gdn_prefill_backward", rc)
    return {n: t for n, t in g.items() if t is not None}


def gdn_prefill_backward_varlen_workspace_size(N, T_tot, Hqk, Hv, dk=128, dv=128) -> int:
    return int(lib().gdn_prefill_backward_varlen_workspace_size(N, T_tot, Hqk, Hv, dk, dv))


def gdn_prefill_backward_varlen(q, k, v, a, b, conv_w, cu_seqlens, grad_o, *, gate_scale, q_scale=1.0,
                                state_in=None, conv_state_in=None, grad_state_out=None,
                                want_conv_state=False, want_state=True, workspace=None, stream=None):
    """Gradients of ``gdn_prefill_varlen`` (packed sequences): q, k:
    [T_tot][Hqk][128] bf16; v, grad_o: [T_tot][Hv][128] bf16; a, b:
    [T_tot][Hv] fp32; cu_seqlens: int32 [N+1] on the GPU.  Returns a dict of
    fp32 gradients as ``gdn_prefill_backward``."""
    torch = _torch()
    T_tot, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    N = cu_seqlens.shape[0] - 1
    C_tot = 2 * Hqk * dk + Hv * dv
    bf, f32 = torch.bfloat16, torch.float32
    _check(q, "q", bf, (T_tot, Hqk, dk))
    _check(k, "k", bf, (T_tot, Hqk, dk))
    _check(v, "v", bf, (T_tot, Hv, dv))
    _check(a, "a", f32, (T_tot, Hv))
    _check(b, "b", f32, (T_tot, Hv))
    _check(conv_w, "conv_w", bf, (C_tot, 4))
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    _check(state_in, "state_in", f32, (N, Hv, dk, dv))
    _check(conv_state_in, "conv_state_in", bf, (N, 3, C_tot))
    _check(grad_o, "grad_o", bf, (T_tot, Hv, dv))
    _check(grad_state_out, "grad_state_out", f32, (N, Hv, dk, dv))
    dev = q.device
    g = {"q": torch.empty((T_tot, Hqk, dk), dtype=f32, device=dev),
         "k": torch.empty((T_tot, Hqk, dk), dtype=f32, device=dev),
         "v": torch.empty((T_tot, Hv, dv), dtype=f32, device=dev),
         "a": torch.empty((T_tot, Hv), dtype=f32, device=dev),
         "b": torch.empty((T_tot, Hv), dtype=f32, device=dev),
         "conv_w": torch.empty((C_tot, 4), dtype=f32, device=dev),
         "conv_state": torch.empty((N, 3, C_tot), dtype=f32, device=dev) if want_conv_state else None,
         "state": torch.empty((N, Hv, dk, dv), dtype=f32, device=dev) if want_state else None}
    need = gdn_prefill_backward_varlen_workspace_size(N, T_tot, Hqk, Hv, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib().gdn_prefill_backward_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w), _ptr(conv_state_in),
        _ptr(state_in), _ptr(grad_o), _ptr(grad_state_out), _ptr(g["q"]), _ptr(g["k"]),
        _ptr(g["v"]), _ptr(g["a"]), _ptr(g["b"]), _ptr(g["conv_w"]), _ptr(g["conv_state"]),
        _ptr(g["state"]), _ptr(cu_seqlens), N, T_tot, Hqk, Hv, dk, dv, float(gate_scale), float(q_scale),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if rc != GDN_OK:
        raise GDNError("gdn_prefill_backward_varlen", rc)
    return {n: t for n, t in g.items() if t is not None}


def gdn_prefill_varlen(q, k, v, a, b, conv_w, cu_seqlens, *, gate_scale, q_scale=1.0,
                       state_in=None, conv_state_in=None, state_out=None, o=None,
                       conv_state_out=None, slots=None, workspace=None, stream=None):
    """Packed variable-length prefill.  q, k: [T_tot][Hqk][128]; v: [T_tot][Hv][128];
    a, b: [T_tot][Hv]; cu_seqlens: int32 [N+1] on the GPU; states [N][...].
    With ``slots`` (int32 [N] on the GPU) the states and conv rows are pools
    of any number of rows and sequence s uses row slots[s]
    (``gdn_prefill_varlen_slots``); state_out then defaults to state_in (the
    pool updated in place).  Returns (o, state_out, conv_state_out)."""
    torch = _torch()
    T_tot, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    N = cu_seqlens.shape[0] - 1
    C_tot = 2 * Hqk * dk + Hv * dv
    bf, f32 = torch.bfloat16, torch.float32
    _check(q, "q", bf, (T_tot, Hqk, dk))
    _check(k, "k", bf, (T_tot, Hqk, dk))
    _check(v, "v", bf, (T_tot, Hv, dv))
    _check(a, "a", f32, (T_tot, Hv))
    _check(b, "b", f32, (T_tot, Hv))
    _check(conv_w, "conv_w", bf, (C_tot, 4))
    _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    rows = N
    if slots is not None:
        _check(slots, "slots", torch.int32, (N,))
        if state_out is None:
            state_out = state_in
        if state_out is None:
            raise ValueError("a slot table needs a state pool (state_in or state_out)")
        rows = state_out.shape[0]
    _check(state_in, "state_in", f32, (rows, Hv, dk, dv))
    _check(conv_state_in, "conv_state_in", bf, (rows, 3, C_tot))
    dev = q.device
    if o is None:
        o = torch.empty((T_tot, Hv, dv), dtype=bf, device=dev)
    if state_out is None:
        state_out = torch.empty((N, Hv, dk, dv), dtype=f32, device=dev)
    _check(o, "o", bf, (T_tot, Hv, dv))
    _check(state_out, "state_out", f32, (rows, Hv, dk, dv))
    _check(conv_state_out, "conv_state_out", bf, (rows, 3, C_tot))
    need = gdn_prefill_varlen_workspace_size(N, T_tot, Hqk, Hv, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if slots is None:
        rc = lib().gdn_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                                      _ptr(conv_state_in), _ptr(conv_state_out), _ptr(state_in),
                                      _ptr(state_out), _ptr(o), _ptr(cu_seqlens), N, T_tot, Hqk, Hv,
                                      dk, dv, float(gate_scale), float(q_scale), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream))
        name = "gdn_prefill_varlen"
    else:
        rc = lib().gdn_prefill_varlen_slots(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                                            _ptr(conv_state_in), _ptr(conv_state_out), _ptr(state_in),
                                            _ptr(state_out), _ptr(o), _ptr(cu_seqlens), _ptr(slots), rows,
                                            N, T_tot, Hqk, Hv, dk, dv, float(gate_scale), float(q_scale),
                                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                                            _stream(stream))
        name = "gdn_prefill_varlen_slots"
    if rc != GDN_OK:
        raise GDNError(name, rc)
    return o, state_out, conv_state_out


def gdn_decode_step(q, k, v, a, b, conv_w, conv_state, state_in, *, gate_scale, q_scale=1.0,
                    state_out=None, o=None, stream=None):
    """One decode step.  q, k: [B][Hqk][128]; v: [B][Hv][128] bf16; a, b: [B][Hv]
    fp32; conv_state: [B][3][C_tot] bf16 (updated in place); state_in:
    [B][Hv][128][128] fp32; state_out defaults to state_in (in place).
    Returns (o, state_out)."""
    torch = _torch()
    B, Hqk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    C_tot = 2 * Hqk * dk + Hv * dv
    bf, f32 = torch.bfloat16, torch.float32
    _check(q, "q", bf, (B, Hqk, dk))
    _check(k, "k", bf, (B, Hqk, dk))
    _check(v, "v", bf, (B, Hv, dv))
    _check(a, "a", f32, (B, Hv))
    _check(b, "b", f32, (B, Hv))
    _check(conv_w, "conv_w", bf, (C_tot, 4))
    _check(conv_state, "conv_state", bf, (B, 3, C_tot))
    _check(state_in, "state_in", f32, (B, Hv, dk, dv))
    if state_out is None:
        state_out = state_in
    if o is None:
        o = torch.empty((B, Hv, dv), dtype=bf, device=q.device)
    _check(state_out, "state_out", f32, (B, Hv, dk, dv))
    _check(o, "o", bf, (B, Hv, dv))
    rc = lib().gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                               _ptr(conv_state), _ptr(state_in), _ptr(state_out), _ptr(o),
                               B, Hqk, Hv, dk, dv, float(gate_scale), float(q_scale),
                               _stream(stream))
    if rc != GDN_OK:
        raise GDNError("gdn_decode_step", rc)
    return o, state_out


def gdn_decode_multi(q, k, v, a, b, conv_w, conv_state, state_in, *, gate_scale, q_scale=1.0,
                     state_out=None, o=None, slots=None, stream=None):
    """T = 1..4 decode tokens per sequence.  q, k: [B][T][Hqk][128]; v:
    [B][T][Hv][128] bf16; a, b: [B][T][Hv] fp32; conv_state: [rows][3][C_tot]
    bf16 (updated in place); state_in: [rows][Hv][128][128] fp32 with rows = B,
    or the pool size when ``slots`` (int32 [B] on the GPU) maps sequence b to
    row slots[b]; state_out defaults to state_in (in place).
    Returns (o [B][T][Hv][128], state_out)."""
    torch = _torch()
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    C_tot = 2 * Hqk * dk + Hv * dv
    bf, f32 = torch.bfloat16, torch.float32
    rows = state_in.shape[0]
    _check(q, "q", bf, (B, T, Hqk, dk))
    _check(k, "k", bf, (B, T, Hqk, dk))
    _check(v, "v", bf, (B, T, Hv, dv))
    _check(a, "a", f32, (B, T, Hv))
    _check(b, "b", f32, (B, T, Hv))
    _check(conv_w, "conv_w", bf, (C_tot, 4))
    _check(conv_state, "conv_state", bf, (rows, 3, C_tot))
    _check(state_in, "state_in", f32, (rows, Hv, dk, dv))
    if slots is None and rows != B:
        raise ValueError(f"state_in has {rows} rows for {B} sequences and no slot table")
    if slots is not None:
        _check(slots, "slots", torch.int32, (B,))
    if state_out is None:
        state_out = state_in
    if o is None:
        o = torch.empty((B, T, Hv, dv), dtype=bf, device=q.device)
    _check(state_out, "state_out", f32, (rows, Hv, dk, dv))
    _check(o, "o", bf, (B, T, Hv, dv))
    rc = lib().gdn_decode_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(conv_w),
                                _ptr(conv_state), _ptr(state_in), _ptr(state_out), _ptr(o),
                                _ptr(slots), rows, B, T, Hqk, Hv, dk, dv, float(gate_scale),
                                float(q_scale), _stream(stream))
    if rc != GDN_OK:
        raise GDNError("gdn_decode_multi", rc)
    return o, state_out


# short aliases
prefill = gdn_prefill
prefill_varlen = gdn_prefill_varlen
decode_step = gdn_decode_step
decode_multi = gdn_decode_multi
