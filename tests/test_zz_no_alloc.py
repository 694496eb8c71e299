"""gdn_prefill_noalloc -- the prefill with the library's own device workspace
(a file-scope array, for callers that cannot allocate) -- against gdn_prefill
with a caller's workspace.  Both run the same kernels, so the results must be
identical bit for bit.  Two calls in a row, the second smaller, so that the
second runs on the array as the first left it."""
import ctypes

import numpy as np
import pytest

from linear_attention_sequence_gdn_amd import inputs
from gdn_testutil import dev_bf16, dev_f32, host_u16

pytestmark = pytest.mark.gpu


def _run(x, T, noalloc):
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    Hqk, Hv, d = x["Hqk"], x["Hv"], x["d"]
    C_tot = 2 * Hqk * d + Hv * d
    q = dev_bf16(x["q"].reshape(1, T, Hqk, d))
    k = dev_bf16(x["k"].reshape(1, T, Hqk, d))
    v = dev_bf16(x["v"].reshape(1, T, Hv, d))
    a = dev_f32(x["a"].reshape(1, T, Hv))
    b = dev_f32(x["b"].reshape(1, T, Hv))
    w = dev_bf16(x["conv_w"])
    st = dev_f32(x["state_in"])
    cs = dev_bf16(x["conv_state_in"])
    o = torch.empty((1, T, Hv, d), dtype=torch.bfloat16, device="cuda")
    so = torch.empty((1, Hv, d, d), dtype=torch.float32, device="cuda")
    cso = torch.empty((1, 3, C_tot), dtype=torch.bfloat16, device="cuda")
    L = gdn.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        rc = L.gdn_prefill_noalloc(P(q), P(k), P(v), P(a), P(b), P(w), P(cs), P(cso), P(st), P(so), P(o),
                                   1, T, Hqk, Hv, d, d, x["gate_scale"], 1.0, sp)
    else:
        need = gdn.gdn_prefill_workspace_size(1, T, Hqk, Hv)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        rc = L.gdn_prefill(P(q), P(k), P(v), P(a), P(b), P(w), P(cs), P(cso), P(st), P(so), P(o),
                           1, T, Hqk, Hv, d, d, x["gate_scale"], 1.0, P(ws), need, sp)
    assert rc == 0, gdn.gdn_status_string(rc)
    torch.cuda.synchronize()
    return host_u16(o), so.cpu().numpy(), host_u16(cso)


def test_noalloc_equals_workspace_call_twice():
    import linear_attention_sequence_gdn_amd as gdn
    # first call: a sequence cut into segments, two of its V heads without
    # decay (their later segments go through the segment maps, the
    # per-(sequence, head) counters and flags that live in the workspace)
    T1 = 8192 + 37
    x1 = inputs.make_prefill(T_list=[T1], Hqk=2, Hv=6, seed=901, state_std=0.05, conv_state_std=1.0)
    x1["a"][:, :2] = -9.0
    assert gdn.gdn_prefill_workspace_size(1, T1, 2, 6) <= gdn.gdn_prefill_noalloc_max_workspace()
    got1 = _run(x1, T1, noalloc=True)
    ref1 = _run(x1, T1, noalloc=False)
    # second call, smaller, on the array as the first call left it
    T2 = 300
    x2 = inputs.make_prefill(T_list=[T2], Hqk=2, Hv=6, seed=902, state_std=0.05, conv_state_std=1.0)
    got2 = _run(x2, T2, noalloc=True)
    ref2 = _run(x2, T2, noalloc=False)
    for got, ref in ((got1, ref1), (got2, ref2)):
        for g_, r_ in zip(got, ref):
            np.testing.assert_array_equal(g_, r_)


def test_noalloc_rejects_oversize_before_launch():
    """A call longer than the array holds runs in windows; a batch whose
    first 64-token window alone exceeds the array is refused before anything
    is launched (the pointers here are not device memory, so a launch would
    fault)."""
    import linear_attention_sequence_gdn_amd as gdn
    L = gdn.lib()
    B, T = 64, 16384
    assert gdn.gdn_prefill_workspace_size(B, 64, 16, 48) > gdn.gdn_prefill_noalloc_max_workspace()
    fake = ctypes.c_void_p(0x10000)
    rc = L.gdn_prefill_noalloc(fake, fake, fake, fake, fake, fake, None, None, None, fake, fake,
                               B, T, 16, 48, 128, 128, 0.1, 1.0, None)
    assert rc == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
