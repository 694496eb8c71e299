"""GPU parity of gdn_decode_step against the fp64 oracle."""
import numpy as np
import pytest

from linear_attention_sequence_gdn_amd import inputs
from gdn_testutil import (check_output, check_state, dev_bf16, dev_f32, host_bf16, host_u16)

pytestmark = pytest.mark.gpu


def _run_steps(x, steps, B_sub=None, in_place=True):
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    B = x["B"] if B_sub is None else B_sub
    conv = dev_bf16(x["conv_state"][:B])
    st = dev_f32(x["state"][:B])
    w = dev_bf16(x["conv_w"])
    outs = []
    for t in range(steps):
        q, k, v = dev_bf16(x["q"][t, :B]), dev_bf16(x["k"][t, :B]), dev_bf16(x["v"][t, :B])
        a, b = dev_f32(x["a"][t, :B]), dev_f32(x["b"][t, :B])
        so = st if in_place else torch.empty_like(st)
        o, so = gdn.gdn_decode_step(q, k, v, a, b, w, conv, st, state_out=so, gate_scale=x["gate_scale"])
        st = so
        outs.append(host_bf16(o))
    torch.cuda.synchronize()
    return np.stack(outs), st.cpu().numpy(), host_u16(conv)


def _oracle_steps(oracle_lib, x, steps, B_sub):
    conv = np.ascontiguousarray(x["conv_state"][:B_sub])
    st = np.ascontiguousarray(x["state"][:B_sub], dtype=np.float64)
    outs = []
    for t in range(steps):
        outs.append(oracle_lib.decode_step(x["q"][t, :B_sub], x["k"][t, :B_sub], x["v"][t, :B_sub],
                                           x["a"][t, :B_sub], x["b"][t, :B_sub], x["conv_w"], conv, st,
                                           Hqk=x["Hqk"], Hv=x["Hv"], gate_scale=x["gate_scale"]))
    return np.stack(outs), st, conv


@pytest.mark.parametrize("B,Hqk,Hv,steps", [(1, 2, 6, 3), (5, 2, 6, 7), (3, 4, 4, 4), (2, 1, 16, 3), (2, 1, 20, 2)])
def test_decode_small(oracle_lib, B, Hqk, Hv, steps):
    x = inputs.make_decode(B=B, steps=steps, Hqk=Hqk, Hv=Hv, seed=77 + B)
    o, st, conv = _run_steps(x, steps)
    o_ref, st_ref, conv_ref = _oracle_steps(oracle_lib, x, steps, B)
    check_output(o, o_ref)
    check_state(st, st_ref)
    np.testing.assert_array_equal(conv, conv_ref)


def test_decode_out_of_place_equals_in_place(oracle_lib):
    x = inputs.make_decode(B=4, steps=3, Hqk=2, Hv=6, seed=5)
    o1, st1, c1 = _run_steps(x, 3, in_place=True)
    o2, st2, c2 = _run_steps(x, 3, in_place=False)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(st1, st2)
    np.testing.assert_array_equal(c1, c2)


def test_decode_config3_full_size(oracle_lib):
    """B = 256 sequences x 64 steps, 16 QK / 48 V heads.  The GPU runs the full
    batch; the oracle checks a sample of 24 sequences (sequences are
    independent, so the sample is checked exactly), and every sequence is
    checked for finiteness and for the conv-state shift."""
    x = inputs.make_config(3)
    o, st, conv = _run_steps(x, 64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(st))
    sample = 24
    o_ref, st_ref, conv_ref = _oracle_steps(oracle_lib, x, 64, sample)
    check_output(o[:, :sample], o_ref)
    check_state(st[:sample], st_ref)
    for h in (0, 23, 47):
        check_state(st[:sample, h], st_ref[:, h], what=f"state head {h}")
    np.testing.assert_array_equal(conv[:sample], conv_ref)
    # the conv state of every sequence holds its last three raw input rows
    raw = np.concatenate([x["q"].reshape(64, 256, -1), x["k"].reshape(64, 256, -1),
                          x["v"].reshape(64, 256, -1)], axis=2)
    np.testing.assert_array_equal(conv, raw[61:64].transpose(1, 0, 2))
