"""fp64 CPU oracle of the Gated DeltaNet token mixer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``linear_attention_sequence_gdn_amd``) never imports, links or loads it,
and the two share no code.

The arithmetic lives in ``gdn_oracle.c`` (plain C, IEEE double, OpenMP only
over independent (sequence, V head) pairs); its header states what each step
follows.  This wrapper only marshals numpy arrays.

Parity pins (see ``tests/test_oracle_pins.py``): every function here is pinned
by a check that does not reuse its own formula -- brute force in exact
rational arithmetic, dense explicit products of the per-token transition
matrices, closed forms and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

_P = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (g++-free plain C, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        d = ctypes.c_double
        i = ctypes.c_int
        lib.gdn_ref_sigmoid.restype = d
        lib.gdn_ref_sigmoid.argtypes = [d]
        lib.gdn_ref_softplus.restype = d
        lib.gdn_ref_softplus.argtypes = [d]
        lib.gdn_ref_silu.restype = d
        lib.gdn_ref_silu.argtypes = [d]
        lib.gdn_ref_num_threads.restype = i
        lib.gdn_ref_conv_silu.argtypes = [_P, ctypes.c_long, i, i, _P, _P, ctypes.c_long, _P]
        lib.gdn_ref_l2norm.argtypes = [_P, i, i, d]
        lib.gdn_ref_gates.argtypes = [_P, _P, ctypes.c_long, i, d, _P, _P]
        lib.gdn_ref_recurrence.argtypes = [_P, _P, _P, _P, _P, i, i, i, d, _P, _P]
        lib.gdn_ref_prefill.restype = i
        lib.gdn_ref_prefill.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, i, i, i, i, i,
                                        d, d, _P, i, _P, _P, _P]
        lib.gdn_ref_prefill_f64.restype = i
        lib.gdn_ref_prefill_f64.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, i, i, i, i, i,
                                            d, d, _P, _P]
        lib.gdn_ref_prefill_backward.restype = i
        lib.gdn_ref_prefill_backward.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, i, i, i, i, i,
                                                 d, d, i, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
        lib.gdn_ref_decode_step.restype = i
        lib.gdn_ref_decode_step.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, i, i, i, i, i,
                                            d, d, _P]
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(_P)


def num_threads() -> int:
    return int(_load().gdn_ref_num_threads())


def sigmoid(x: float) -> float:
    return _load().gdn_ref_sigmoid(float(x))


def softplus(x: float) -> float:
    return _load().gdn_ref_softplus(float(x))


def silu(x: float) -> float:
    return _load().gdn_ref_silu(float(x))


def conv_silu(x_bf16, w_bf16, hist_bf16=None):
    """Causal width-4 depthwise conv + SiLU.  x: uint16 [T][C]; w: [C][4];
    hist: uint16 [3][C] or None.  Returns float64 [T][C]."""
    x, px = _c(x_bf16, np.uint16)
    T, C = x.shape
    w, pw = _c(w_bf16, np.uint16)
    ph = None
    if hist_bf16 is not None:
        hist, ph = _c(hist_bf16, np.uint16)
    out = np.zeros((T, C), np.float64)
    _load().gdn_ref_conv_silu(px, C, T, C, pw, ph, C, out.ctypes.data_as(_P))
    return out


def l2norm(x, eps=1e-6):
    x = np.array(x, dtype=np.float64, copy=True, order="C")
    T, n = x.shape
    _load().gdn_ref_l2norm(x.ctypes.data_as(_P), T, n, float(eps))
    return x


def gates(a, b, gate_scale):
    """alpha, beta (float64 [T]) from raw fp32 pre-activations a, b [T]."""
    a, pa = _c(a, np.float32)
    b, pb = _c(b, np.float32)
    T = a.shape[0]
    al = np.zeros(T, np.float64)
    be = np.zeros(T, np.float64)
    _load().gdn_ref_gates(pa, pb, 1, T, float(gate_scale), al.ctypes.data_as(_P),
                          be.ctypes.data_as(_P))
    return al, be


def recurrence(qh, kh, vh, alpha, beta, S0=None, q_scale=1.0):
    """Token-by-token state update + readout on prepared q^, k^, v^ (float64).
    Returns (o [T][dv], S_T [dk][dv])."""
    qh, pq = _c(qh, np.float64)
    kh, pk = _c(kh, np.float64)
    vh, pv = _c(vh, np.float64)
    al, pal = _c(alpha, np.float64)
    be, pbe = _c(beta, np.float64)
    T, dk = kh.shape
    dv = vh.shape[1]
    S = np.zeros((dk, dv), np.float64) if S0 is None else np.array(S0, np.float64, copy=True, order="C")
    o = np.zeros((T, dv), np.float64)
    _load().gdn_ref_recurrence(pq, pk, pv, pal, pbe, T, dk, dv, float(q_scale),
                               S.ctypes.data_as(_P), o.ctypes.data_as(_P))
    return o, S


def prefill(q, k, v, a, b, conv_w, cu_seqlens, *, Hqk, Hv, gate_scale,
            q_scale=1.0, state_in=None, conv_state_in=None, heads=None):
    """Whole mixer over packed sequences.

    q, k: uint16 [T_tot][Hqk][dk]; v: uint16 [T_tot][Hv][dv]; a, b: fp32
    [T_tot][Hv]; conv_w: uint16 [C_tot][4]; cu_seqlens: int32 [N+1];
    state_in: [N][Hv][dk][dv] (any float dtype) or None; conv_state_in:
    uint16 [N][3][C_tot] or None; heads: iterable of V heads or None (all).

    Returns (o float64 [T_tot][Hv][dv], state_out float64 [N][Hv][dk][dv],
    conv_state_out uint16 [N][3][C_tot]).  Heads not selected stay zero.
    """
    q, pq = _c(q, np.uint16)
    k, pk = _c(k, np.uint16)
    v, pv = _c(v, np.uint16)
    a, pa = _c(a, np.float32)
    b, pb = _c(b, np.float32)
    w, pw = _c(conv_w, np.uint16)
    cu, pcu = _c(cu_seqlens, np.int32)
    T_tot, _, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    C_tot = 2 * Hqk * dk + Hv * dv
    pcs = None
    if conv_state_in is not None:
        cs, pcs = _c(conv_state_in, np.uint16)
    pst = None
    if state_in is not None:
        st, pst = _c(state_in, np.float64)
    ph, nh = None, 0
    if heads is not None:
        hs, ph = _c(list(heads), np.int32)
        nh = hs.shape[0]
    o = np.zeros((T_tot, Hv, dv), np.float64)
    so = np.zeros((N, Hv, dk, dv), np.float64)
    cso = np.zeros((N, 3, C_tot), np.uint16)
    rc = _load().gdn_ref_prefill(pq, pk, pv, pa, pb, pw, pcs, pst, pcu, N, Hqk, Hv, dk, dv,
                                 float(gate_scale), float(q_scale), ph, nh,
                                 o.ctypes.data_as(_P), so.ctypes.data_as(_P),
                                 cso.ctypes.data_as(_P))
    if rc != 0:
        raise ValueError("oracle prefill: bad arguments")
    return o, so, cso


def prefill_f64(q, k, v, a, b, conv_w, cu_seqlens, *, Hqk, Hv, gate_scale,
                q_scale=1.0, state_in=None, conv_state_in=None):
    """The mixer with every input given in float64 (q, k, v [T_tot][H][d], a,
    b [T_tot][Hv], conv_w [C_tot][4], conv_state_in [N][3][C_tot]): the
    forward that finite differences perturb.  Returns (o, state_out)."""
    q, pq = _c(q, np.float64)
    k, pk = _c(k, np.float64)
    v, pv = _c(v, np.float64)
    a, pa = _c(a, np.float64)
    b, pb = _c(b, np.float64)
    w, pw = _c(conv_w, np.float64)
    cu, pcu = _c(cu_seqlens, np.int32)
    T_tot, _, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    pcs = None
    if conv_state_in is not None:
        cs, pcs = _c(conv_state_in, np.float64)
    pst = None
    if state_in is not None:
        st, pst = _c(state_in, np.float64)
    o = np.zeros((T_tot, Hv, dv), np.float64)
    so = np.zeros((N, Hv, dk, dv), np.float64)
    rc = _load().gdn_ref_prefill_f64(pq, pk, pv, pa, pb, pw, pcs, pst, pcu, N, Hqk, Hv, dk, dv,
                                     float(gate_scale), float(q_scale), o.ctypes.data_as(_P),
                                     so.ctypes.data_as(_P))
    if rc != 0:
        raise ValueError("oracle prefill_f64: bad arguments")
    return o, so


def prefill_backward(q, k, v, a, b, conv_w, cu_seqlens, d_o, *, Hqk, Hv, gate_scale,
                     q_scale=1.0, state_in=None, conv_state_in=None, d_state_out=None,
                     f64=None):
    """Gradient of sum <d_o, o> + <d_state_out, state_out> with respect to
    every input of the mixer.  Inputs as ``prefill`` (bf16 as uint16, a/b
    fp32) or all float64 (``f64``; inferred from q's dtype when None).

    Returns a dict of float64 arrays: q, k [T_tot][Hqk][dk]; v
    [T_tot][Hv][dv]; a, b [T_tot][Hv]; conv_w [C_tot][4]; conv_state
    [N][3][C_tot]; state [N][Hv][dk][dv]."""
    if f64 is None:
        f64 = np.asarray(q).dtype == np.float64
    xt = np.float64 if f64 else np.uint16
    gt = np.float64 if f64 else np.float32
    q, pq = _c(q, xt)
    k, pk = _c(k, xt)
    v, pv = _c(v, xt)
    a, pa = _c(a, gt)
    b, pb = _c(b, gt)
    w, pw = _c(conv_w, xt)
    cu, pcu = _c(cu_seqlens, np.int32)
    T_tot, _, dk = q.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    C_tot = 2 * Hqk * dk + Hv * dv
    pcs = None
    if conv_state_in is not None:
        cs, pcs = _c(conv_state_in, xt)
    pst = None
    if state_in is not None:
        st, pst = _c(state_in, np.float64)
    do_, pdo = _c(d_o, np.float64)
    pds = None
    if d_state_out is not None:
        ds, pds = _c(d_state_out, np.float64)
    out = {"q": np.zeros((T_tot, Hqk, dk)), "k": np.zeros((T_tot, Hqk, dk)),
           "v": np.zeros((T_tot, Hv, dv)), "a": np.zeros((T_tot, Hv)), "b": np.zeros((T_tot, Hv)),
           "conv_w": np.zeros((C_tot, 4)), "conv_state": np.zeros((N, 3, C_tot)),
           "state": np.zeros((N, Hv, dk, dv))}
    P = {n: x.ctypes.data_as(_P) for n, x in out.items()}
    rc = _load().gdn_ref_prefill_backward(pq, pk, pv, pa, pb, pw, pcs, pst, pcu, N, Hqk, Hv, dk, dv,
                                          float(gate_scale), float(q_scale), int(bool(f64)), pdo, pds,
                                          P["q"], P["k"], P["v"], P["a"], P["b"], P["conv_w"],
                                          P["conv_state"], P["state"])
    if rc != 0:
        raise ValueError("oracle prefill_backward: bad arguments")
    return out


def decode_step(q, k, v, a, b, conv_w, conv_state, state, *, Hqk, Hv, gate_scale,
                q_scale=1.0):
    """One decode step.  conv_state (uint16 [B][3][C_tot]) and state (float64
    [B][Hv][dk][dv]) are updated IN PLACE (must be C-contiguous of the right
    dtype).  Returns o float64 [B][Hv][dv]."""
    q, pq = _c(q, np.uint16)
    k, pk = _c(k, np.uint16)
    v, pv = _c(v, np.uint16)
    a, pa = _c(a, np.float32)
    b, pb = _c(b, np.float32)
    w, pw = _c(conv_w, np.uint16)
    assert conv_state.dtype == np.uint16 and conv_state.flags.c_contiguous
    assert state.dtype == np.float64 and state.flags.c_contiguous
    B, _, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((B, Hv, dv), np.float64)
    rc = _load().gdn_ref_decode_step(pq, pk, pv, pa, pb, pw,
                                     conv_state.ctypes.data_as(_P), state.ctypes.data_as(_P),
                                     B, Hqk, Hv, dk, dv, float(gate_scale), float(q_scale),
                                     o.ctypes.data_as(_P))
    if rc != 0:
        raise ValueError("oracle decode: bad arguments")
    return o
