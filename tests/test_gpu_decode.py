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
    """The oracle's decode steps on sequences B_sub (a count: the first B_sub
    sequences; or an index array: those sequences, in that order)."""
    sel = np.arange(B_sub) if np.isscalar(B_sub) else np.asarray(B_sub)
    conv = np.ascontiguousarray(x["conv_state"][sel])
    st = np.ascontiguousarray(x["state"][sel], dtype=np.float64)
    outs = []
    for t in range(steps):
        outs.append(oracle_lib.decode_step(np.ascontiguousarray(x["q"][t, sel]), np.ascontiguousarray(x["k"][t, sel]),
                                           np.ascontiguousarray(x["v"][t, sel]), np.ascontiguousarray(x["a"][t, sel]),
                                           np.ascontiguousarray(x["b"][t, sel]), x["conv_w"], conv, st,
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
    batch; the oracle checks 24 sequences spread over it (the first, middle and
    last eight: sequences are independent, so the sample is checked exactly),
    and every sequence is checked for finiteness and for the conv-state shift."""
    x = inputs.make_config(3)
    o, st, conv = _run_steps(x, 64)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(st))
    sample = np.r_[0:8, 124:132, 248:256]
    o_ref, st_ref, conv_ref = _oracle_steps(oracle_lib, x, 64, sample)
    r_o, ex = check_output(o[:, sample], o_ref)
    r_s = check_state(st[sample], st_ref)
    for h in (0, 23, 47):
        check_state(st[sample, h], st_ref[:, h], what=f"state head {h}")
    for i, s_ in enumerate(sample):  # every sampled sequence on its own
        check_output(o[:, s_], o_ref[:, i], what=f"o seq {s_}")
        check_state(st[s_], st_ref[i], what=f"state seq {s_}")
    np.testing.assert_array_equal(conv[sample], conv_ref)
    print(f"config 3 margins: o relL2 {r_o:.2e}, max-abs excess {ex:.2e} RMS, state relL2 {r_s:.2e}", flush=True)
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
def test_decode_multi_matches_single_steps(T):
    """T tokens in one call against T single steps.  One call takes all T
    tokens from one pass over the state (the sums over the state's rows run
    once, in another order than T single steps run them), so for T >= 2 the
    two agree to fp32 rounding: the state within 1e-6 relative L2 and 1e-5 of
    (|s| + RMS) per element, the bf16 output within one bf16 rounding step
    (2^-7 relative) of each element.  T = 1 runs the single-step kernel and
    must agree bit for bit; the conv rows are copies and agree bit for bit."""
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
    got_o, ref_o = host_bf16(o).astype(np.float64), np.swapaxes(o1, 0, 1).astype(np.float64)
    got_s, ref_s = so.cpu().numpy().astype(np.float64), s1.astype(np.float64)
    np.testing.assert_array_equal(host_u16(conv), c1)
    if T == 1:
        np.testing.assert_array_equal(got_o, ref_o)
        np.testing.assert_array_equal(got_s, ref_s)
        return
    assert np.linalg.norm(got_s - ref_s) <= 1e-6 * np.linalg.norm(ref_s)
    rms = np.sqrt(np.mean(ref_s ** 2))
    assert np.max(np.abs(got_s - ref_s) / (np.abs(ref_s) + rms)) <= 1e-5
    o_rms = np.sqrt(np.mean(ref_o ** 2))
    assert np.all(np.abs(got_o - ref_o) <= 2.0 ** -7 * np.abs(ref_o) + 1e-6 * o_rms)


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


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_decode_multi_slots(oracle_lib, T):
    """Sequences addressing a pool through a slot table (T = 1 runs the
    one-token slot kernel, the common serving case): the rows they name get
    the oracle's token recurrence with state and conv carry-in from those
    rows, the other rows stay as they were, and a sequence whose slot lies
    outside the pool is skipped (its outputs are not written)."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    B, Hqk, Hv, rows, d = 6, 2, 6, 11, 128
    x, m = _multi_inputs(B, T, Hqk, Hv, seed=720 + T)
    rng = np.random.default_rng(721 + T)
    slots = rng.permutation(rows)[:B].astype(np.int32)
    slots[4] = rows + 3  # out of range: skipped
    C_tot = 2 * Hqk * d + Hv * d
    pool_st = (rng.standard_normal((rows, Hv, d, d)) * 0.05).astype(np.float32)
    pool_cs = inputs.bf16_bits(rng.standard_normal((rows, 3, C_tot)).astype(np.float32))
    ok = [i for i in range(B) if 0 <= slots[i] < rows]
    pool_st[slots[ok]] = x["state"][ok]
    pool_cs[slots[ok]] = x["conv_state"][ok]
    st = dev_f32(pool_st)
    cs = dev_bf16(pool_cs)
    o = torch.full((B, T, Hv, d), 7.0, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_decode_multi(dev_bf16(m["q"]), dev_bf16(m["k"]), dev_bf16(m["v"]), dev_f32(m["a"]), dev_f32(m["b"]),
                         dev_bf16(x["conv_w"]), cs, st, o=o, slots=torch.from_numpy(slots).cuda(),
                         gate_scale=x["gate_scale"])
    torch.cuda.synchronize()
    st_h, cs_h = st.cpu().numpy(), host_u16(cs)
    # the oracle: the sequences that have a slot, T tokens each, carried in
    # from their pool rows
    n = len(ok)
    pick = lambda key: np.ascontiguousarray(m[key][ok])
    cu = np.arange(0, (n + 1) * T, T, dtype=np.int32)
    o_ref, s_ref, cs_ref = oracle_lib.prefill(
        pick("q").reshape(n * T, Hqk, d), pick("k").reshape(n * T, Hqk, d), pick("v").reshape(n * T, Hv, d),
        pick("a").reshape(n * T, Hv), pick("b").reshape(n * T, Hv), x["conv_w"], cu, Hqk=Hqk, Hv=Hv,
        gate_scale=x["gate_scale"], state_in=pool_st[slots[ok]], conv_state_in=pool_cs[slots[ok]])
    check_output(host_bf16(o)[ok].reshape(n * T, Hv, d), o_ref)
    check_state(st_h[slots[ok]], s_ref)
    np.testing.assert_array_equal(cs_h[slots[ok]], cs_ref)
    untouched = sorted(set(range(rows)) - set(slots[ok].tolist()))
    np.testing.assert_array_equal(st_h[untouched], pool_st[untouched])
    np.testing.assert_array_equal(cs_h[untouched], pool_cs[untouched])
    assert (host_u16(o)[4] == host_u16(torch.full((1,), 7.0, dtype=torch.bfloat16))[0]).all()
