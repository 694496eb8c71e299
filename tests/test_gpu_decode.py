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


# ---------------------------------------------------------------------------
# multi-token decode and slot tables
# ---------------------------------------------------------------------------
def _multi_inputs(B, T, Hqk, Hv, seed):
    """T tokens per sequence laid out [B][T][...], from the decode generator's
    T consecutive steps."""
    x = inputs.make_decode(B=B, steps=T, Hqk=Hqk, Hv=Hv, seed=seed)
    tr = lambda arr: np.ascontiguousarray(np.swapaxes(arr, 0, 1))
    return x, {key: tr(x[key]) for key in ("q", "k", "v", "a", "b")}


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_decode_multi_equals_single_steps(T):
    """T tokens in one call give bit for bit what T single steps give."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    B, Hqk, Hv = 5, 2, 6
    x, m = _multi_inputs(B, T, Hqk, Hv, seed=700 + T)
    o1, s1, c1 = _run_steps(x, T)
    conv = dev_bf16(x["conv_state"])
    st = dev_f32(x["state"])
    o, so = gdn.gdn_decode_multi(dev_bf16(m["q"]), dev_bf16(m["k"]), dev_bf16(m["v"]), dev_f32(m["a"]),
                                 dev_f32(m["b"]), dev_bf16(x["conv_w"]), conv, st, gate_scale=x["gate_scale"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bf16(o), np.swapaxes(o1, 0, 1))
    np.testing.assert_array_equal(so.cpu().numpy(), s1)
    np.testing.assert_array_equal(host_u16(conv), c1)


def test_decode_multi_against_oracle(oracle_lib):
    """Four tokens per sequence against the fp64 token recurrence (the oracle's
    packed prefill with state and conv carry-in)."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    B, T, Hqk, Hv = 7, 4, 2, 6
    x, m = _multi_inputs(B, T, Hqk, Hv, seed=710)
    d = 128
    cu = np.arange(0, (B + 1) * T, T, dtype=np.int32)
    o_ref, s_ref, cs_ref = oracle_lib.prefill(
        m["q"].reshape(B * T, Hqk, d), m["k"].reshape(B * T, Hqk, d), m["v"].reshape(B * T, Hv, d),
        m["a"].reshape(B * T, Hv), m["b"].reshape(B * T, Hv), x["conv_w"], cu, Hqk=Hqk, Hv=Hv,
        gate_scale=x["gate_scale"], state_in=x["state"], conv_state_in=x["conv_state"])
    conv = dev_bf16(x["conv_state"])
    st = dev_f32(x["state"])
    o, so = gdn.gdn_decode_multi(dev_bf16(m["q"]), dev_bf16(m["k"]), dev_bf16(m["v"]), dev_f32(m["a"]),
                                 dev_f32(m["b"]), dev_bf16(x["conv_w"]), conv, st,
                                 state_out=torch.empty_like(st), gate_scale=x["gate_scale"])
    torch.cuda.synchronize()
    check_output(host_bf16(o).reshape(B * T, Hv, d), o_ref)
    check_state(so.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(host_u16(conv), cs_ref)


def test_decode_multi_slots():
    """Sequences addressing a pool through a slot table: the rows they name get
    what a gathered call computes, the other rows stay as they were, and a
    sequence whose slot lies outside the pool is skipped."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    B, T, Hqk, Hv, rows = 6, 3, 2, 6, 11
    x, m = _multi_inputs(B, T, Hqk, Hv, seed=720)
    rng = np.random.default_rng(721)
    slots = rng.permutation(rows)[:B].astype(np.int32)
    slots[4] = rows + 3  # out of range: skipped
    C_tot = 2 * Hqk * 128 + Hv * 128
    pool_st = (rng.standard_normal((rows, Hv, 128, 128)) * 0.05).astype(np.float32)
    pool_cs = inputs.bf16_bits(rng.standard_normal((rows, 3, C_tot)).astype(np.float32))
    ok = [i for i in range(B) if 0 <= slots[i] < rows]
    pool_st[slots[ok]] = x["state"][ok]
    pool_cs[slots[ok]] = x["conv_state"][ok]
    st = dev_f32(pool_st)
    cs = dev_bf16(pool_cs)
    o = torch.full((B, T, Hv, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_decode_multi(dev_bf16(m["q"]), dev_bf16(m["k"]), dev_bf16(m["v"]), dev_f32(m["a"]), dev_f32(m["b"]),
                         dev_bf16(x["conv_w"]), cs, st, o=o, slots=torch.from_numpy(slots).cuda(),
                         gate_scale=x["gate_scale"])
    # the same sequences without a table
    conv_g = dev_bf16(x["conv_state"])
    st_g = dev_f32(x["state"])
    o_g, _ = gdn.gdn_decode_multi(dev_bf16(m["q"]), dev_bf16(m["k"]), dev_bf16(m["v"]), dev_f32(m["a"]),
                                  dev_f32(m["b"]), dev_bf16(x["conv_w"]), conv_g, st_g, gate_scale=x["gate_scale"])
    torch.cuda.synchronize()
    st_h, cs_h, o_h = st.cpu().numpy(), host_u16(cs), host_u16(o)
    np.testing.assert_array_equal(st_h[slots[ok]], st_g.cpu().numpy()[ok])
    np.testing.assert_array_equal(cs_h[slots[ok]], host_u16(conv_g)[ok])
    np.testing.assert_array_equal(o_h[ok], host_u16(o_g)[ok])
    untouched = sorted(set(range(rows)) - set(slots[ok].tolist()))
    np.testing.assert_array_equal(st_h[untouched], pool_st[untouched])
    np.testing.assert_array_equal(cs_h[untouched], pool_cs[untouched])
    assert (o_h[4] == host_u16(torch.full((1,), 7.0, dtype=torch.bfloat16))[0]).all()
