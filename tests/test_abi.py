"""The C ABI library loads, exports every entry point the header declares and
rejects bad arguments with the documented status before touching the GPU.

These tests run without a GPU: every call here fails validation (or is a
documented no-op), and validation happens before any HIP call.
"""
import ctypes
import os
import re

import pytest

import linear_attention_sequence_gdn_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gdn.LIB_PATH):
        from linear_attention_sequence_gdn_amd import build
        build.build()
    return gdn.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) >= {"gdn_prefill", "gdn_prefill_varlen", "gdn_decode_step",
                          "gdn_prefill_workspace_size", "gdn_prefill_varlen_workspace_size",
                          "gdn_status_string"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    assert gdn.gdn_status_string(0) == "GDN_OK"
    assert gdn.gdn_status_string(1) == "GDN_ERR_INVALID_ARGUMENT"
    assert gdn.gdn_status_string(2) == "GDN_ERR_UNSUPPORTED"
    assert gdn.gdn_status_string(3) == "GDN_ERR_WORKSPACE_TOO_SMALL"
    assert gdn.gdn_status_string(4) == "GDN_ERR_HIP"
    assert gdn.gdn_status_string(99) == "GDN_ERR_UNKNOWN"


def test_workspace_sizes(L):
    assert gdn.gdn_prefill_workspace_size(1, 8192, 16, 48) > 0
    # (one more chunk can shrink it a little: the segment cut, and with it the
    # parked-state area, is chosen per size)
    assert gdn.gdn_prefill_workspace_size(1, 8192, 16, 48) < gdn.gdn_prefill_workspace_size(1, 16384, 16, 48)
    assert gdn.gdn_prefill_workspace_size(1, 64, 16, 48, 64, 128) == 0  # unsupported dims
    assert gdn.gdn_prefill_workspace_size(1, 64, 16, 47) == 0
    # varlen bound covers any split of T_tot into N sequences
    assert gdn.gdn_prefill_varlen_workspace_size(4, 256, 2, 6) >= gdn.gdn_prefill_workspace_size(4, 64, 2, 6)


FAKE = 0x10000  # 64 KiB-aligned, never dereferenced: validation fails first


def _p(v=FAKE):
    return ctypes.c_void_p(v) if v else None


def call_decode(L, q=FAKE, B=2, Hqk=2, Hv=6, dk=128, dv=128, state=FAKE):
    return L.gdn_decode_step(_p(q), _p(), _p(), _p(), _p(), _p(), _p(), _p(state), _p(state), _p(),
                             B, Hqk, Hv, dk, dv, 0.1, 1.0, None)


def test_decode_validation(L):
    assert call_decode(L, q=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_decode(L, B=-1) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_decode(L, dk=64) == gdn.GDN_ERR_UNSUPPORTED
    assert call_decode(L, dv=96) == gdn.GDN_ERR_UNSUPPORTED
    assert call_decode(L, Hv=7) == gdn.GDN_ERR_UNSUPPORTED
    assert call_decode(L, Hqk=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_decode(L, q=FAKE + 2) == gdn.GDN_ERR_INVALID_ARGUMENT  # q rows are read 4 bytes at a time
    assert call_decode(L, state=FAKE + 4) == gdn.GDN_ERR_INVALID_ARGUMENT  # misaligned state
    assert call_decode(L, B=0) == gdn.GDN_OK  # no-op, nothing launched


def call_prefill(L, B=1, T=64, Hqk=2, Hv=6, dk=128, dv=128, q=FAKE, ws=FAKE, ws_bytes=None,
                 cs_in=0, cs_out=0):
    if ws_bytes is None:
        ws_bytes = gdn.gdn_prefill_workspace_size(B, T, Hqk, Hv, dk, dv)
    return L.gdn_prefill(_p(q), _p(), _p(), _p(), _p(), _p(), _p(cs_in), _p(cs_out), None, _p(), _p(),
                         B, T, Hqk, Hv, dk, dv, 0.1, 1.0, _p(ws), ws_bytes, None)


def test_prefill_validation(L):
    assert call_prefill(L, q=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_prefill(L, T=-1) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_prefill(L, dk=64) == gdn.GDN_ERR_UNSUPPORTED
    assert call_prefill(L, Hv=5) == gdn.GDN_ERR_UNSUPPORTED
    assert call_prefill(L, q=FAKE + 2) == gdn.GDN_ERR_INVALID_ARGUMENT
    need = gdn.gdn_prefill_workspace_size(1, 64, 2, 6)
    assert call_prefill(L, ws_bytes=need - 1) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    assert call_prefill(L, ws=0) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    # the workspace must be 16-byte aligned, as the header states
    assert call_prefill(L, ws=FAKE + 8) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_prefill(L, B=0, T=0, ws=0, ws_bytes=0) == gdn.GDN_OK  # empty batch: nothing to do


def test_varlen_validation(L):
    def call(cu=FAKE, N=2, T_tot=100, Hv=6, ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = gdn.gdn_prefill_varlen_workspace_size(N, T_tot, 2, Hv)
        return L.gdn_prefill_varlen(_p(), _p(), _p(), _p(), _p(), _p(), None, None, None, _p(), _p(),
                                    _p(cu), N, T_tot, 2, Hv, 128, 128, 0.1, 1.0, _p(), ws_bytes, None)
    assert call(cu=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(N=-1) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(Hv=9) == gdn.GDN_ERR_UNSUPPORTED
    assert call(ws_bytes=10) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    assert call(cu=FAKE + 1) == gdn.GDN_ERR_INVALID_ARGUMENT


def test_varlen_slots_validation(L):
    def call(cu=FAKE, slots=FAKE, n_rows=4, N=2, T_tot=100, Hv=6):
        ws_bytes = gdn.gdn_prefill_varlen_workspace_size(N, T_tot, 2, 6)
        return L.gdn_prefill_varlen_slots(_p(), _p(), _p(), _p(), _p(), _p(), None, None, None, _p(), _p(),
                                          _p(cu), _p(slots), n_rows, N, T_tot, 2, Hv, 128, 128, 0.1, 1.0, _p(),
                                          ws_bytes, None)
    assert call(slots=0) == gdn.GDN_ERR_INVALID_ARGUMENT  # the table is required
    assert call(cu=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(n_rows=-1) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(slots=FAKE + 2) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(Hv=9) == gdn.GDN_ERR_UNSUPPORTED
    assert call(N=-1) == gdn.GDN_ERR_INVALID_ARGUMENT


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        gdn.lib()


def call_decode_multi(L, q=FAKE, slots=None, n_rows=0, B=2, T=2, Hqk=2, Hv=6, dk=128, dv=128):
    return L.gdn_decode_multi(_p(q), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(), _p(),
                              None if slots is None else _p(slots), n_rows, B, T, Hqk, Hv, dk, dv, 0.1, 1.0, None)


def test_decode_multi_validation(L):
    L.gdn_decode_multi.restype = ctypes.c_int
    L.gdn_decode_multi.argtypes = [ctypes.c_void_p] * 11 + [ctypes.c_int] * 7 + \
        [ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    assert call_decode_multi(L, T=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_decode_multi(L, T=5) == gdn.GDN_ERR_UNSUPPORTED
    assert call_decode_multi(L, B=-1) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_decode_multi(L, dk=64) == gdn.GDN_ERR_UNSUPPORTED
    assert call_decode_multi(L, slots=FAKE, n_rows=-1) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_decode_multi(L, slots=FAKE + 2, n_rows=8) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_decode_multi(L, q=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_decode_multi(L, B=0) == gdn.GDN_OK



def call_backward(L, B=1, T=64, Hqk=2, Hv=6, dk=128, dv=128, q=FAKE, g_o=FAKE, gw=FAKE, ws=FAKE,
                  ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = gdn.gdn_prefill_backward_workspace_size(B, T, Hqk, Hv, dk, dv)
    return L.gdn_prefill_backward(_p(q), _p(), _p(), _p(), _p(), _p(), None, None, _p(g_o), None,
                                  _p(), _p(), _p(), _p(), _p(), _p(gw), None, None,
                                  B, T, Hqk, Hv, dk, dv, 0.1, 1.0, _p(ws), ws_bytes, None)


def test_backward_validation(L):
    need = gdn.gdn_prefill_backward_workspace_size(1, 64, 2, 6)
    assert need > gdn.gdn_prefill_backward_workspace_size(1, 63, 2, 6) > 0
    assert gdn.gdn_prefill_backward_workspace_size(1, 0, 2, 6) == 0
    assert gdn.gdn_prefill_backward_workspace_size(1, 64, 2, 6, 64, 128) == 0
    assert call_backward(L, q=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_backward(L, g_o=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_backward(L, gw=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_backward(L, T=-1) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_backward(L, dv=64) == gdn.GDN_ERR_UNSUPPORTED
    assert call_backward(L, Hv=7) == gdn.GDN_ERR_UNSUPPORTED
    assert call_backward(L, q=FAKE + 2) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_backward(L, ws=FAKE + 4) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_backward(L, g_o=FAKE + 4) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call_backward(L, ws_bytes=need - 1) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    assert call_backward(L, ws=0) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    assert call_backward(L, B=0, ws=0, ws_bytes=0) == gdn.GDN_OK


def test_backward_window_plan(L):
    # the window a workspace leads to (host-only query)
    need = gdn.gdn_prefill_backward_workspace_size(1, 8192, 16, 48)
    assert gdn.gdn_prefill_backward_windows(1, 8192, 16, 48, need) == 8192
    assert gdn.gdn_prefill_backward_windows(1, 8192, 16, 48, 10 * need) == 8192
    tw = gdn.gdn_prefill_backward_windows(1, 8192, 16, 48, need - 1)
    assert 64 <= tw < 8192 and tw % 64 == 0
    # more workspace never gives shorter windows
    prev = 0
    for frac in (0.1, 0.2, 0.4, 0.6, 0.8, 0.99):
        tw = gdn.gdn_prefill_backward_windows(1, 8192, 16, 48, int(frac * need))
        assert tw >= prev and tw % 64 == 0
        prev = tw
    # the native-context sequence: 262,144 tokens in 3 GiB instead of the one-pass ~78 GiB
    one_pass = gdn.gdn_prefill_backward_workspace_size(1, 262144, 16, 48)
    assert one_pass > 70 * 2**30
    assert gdn.gdn_prefill_backward_windows(1, 262144, 16, 48, 3 * 2**30) >= 4096
    # a batch whose sequences fit one at a time runs them whole
    one = gdn.gdn_prefill_backward_workspace_size(1, 200, 2, 6)
    assert gdn.gdn_prefill_backward_windows(4, 200, 2, 6, 2 * one) == 200
    # too small, bad sizes, nothing to do
    with pytest.raises(gdn.GDNError) as e:
        gdn.gdn_prefill_backward_windows(1, 8192, 16, 48, 2**20)
    assert e.value.status == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    out = ctypes.c_int(-1)
    assert L.gdn_prefill_backward_windows(1, 64, 2, 7, 128, 128, 1 << 30, ctypes.byref(out)) == gdn.GDN_ERR_UNSUPPORTED
    assert L.gdn_prefill_backward_windows(-1, 64, 2, 6, 128, 128, 1 << 30, ctypes.byref(out)) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert L.gdn_prefill_backward_windows(1, 64, 2, 6, 128, 128, 1 << 30, None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert gdn.gdn_prefill_backward_windows(0, 64, 2, 6, 0) == 64
    assert gdn.gdn_prefill_backward_windows(1, 0, 2, 6, 0) == 0
    # a call whose workspace fits no window is refused before anything is launched
    assert call_backward(L, T=8192, Hqk=16, Hv=48, ws_bytes=2**20) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL


def test_backward_varlen_validation(L):
    def call(cu=FAKE, N=3, T_tot=200, Hv=6, ws_bytes=None):
        if ws_bytes is None:
            ws_bytes = gdn.gdn_prefill_backward_varlen_workspace_size(N, T_tot, 2, Hv)
        return L.gdn_prefill_backward_varlen(_p(), _p(), _p(), _p(), _p(), _p(), None, None, _p(), None,
                                             _p(), _p(), _p(), _p(), _p(), _p(), None, None, _p(cu),
                                             N, T_tot, 2, Hv, 128, 128, 0.1, 1.0, _p(), ws_bytes, None)
    # the packed bound covers any split: at least the uniform size
    assert gdn.gdn_prefill_backward_varlen_workspace_size(4, 256, 2, 6) >= gdn.gdn_prefill_backward_workspace_size(4, 64, 2, 6)
    assert call(cu=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(N=-1) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(Hv=9) == gdn.GDN_ERR_UNSUPPORTED
    assert call(ws_bytes=10) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    assert call(cu=FAKE + 2) == gdn.GDN_ERR_INVALID_ARGUMENT


def test_noalloc_validation(L):
    # every failing call returns before any HIP call (no GPU needed)
    def call(q=FAKE, B=1, T=64, Hqk=2, Hv=6, dk=128, cs=0):
        return L.gdn_prefill_noalloc(_p(q), _p(), _p(), _p(), _p(), _p(), _p(cs), _p(cs), None, _p(), _p(),
                                     B, T, Hqk, Hv, dk, 128, 0.1, 1.0, None)
    assert gdn.gdn_prefill_noalloc_max_workspace() >= gdn.gdn_prefill_workspace_size(1, 8192, 16, 48)
    assert call(q=0) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(T=-1) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert call(dk=64) == gdn.GDN_ERR_UNSUPPORTED
    assert call(Hv=5) == gdn.GDN_ERR_UNSUPPORTED
    assert call(q=FAKE + 2) == gdn.GDN_ERR_INVALID_ARGUMENT
    # a longer call runs in windows; only a batch whose 64-token window alone
    # exceeds the array is refused
    assert call(B=64, T=16384, Hqk=16, Hv=48) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
