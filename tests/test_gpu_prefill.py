"""GPU parity of gdn_prefill / gdn_prefill_varlen against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from linear_attention_sequence_gdn_amd import inputs
from gdn_testutil import (check_output, check_state, dev_bf16, dev_f32, dev_i32, host_bf16,
                          host_u16, rel_l2)

pytestmark = pytest.mark.gpu


def gpu_prefill(x, uniform_T=None, conv_out=True):
    """Run the GPU path on generator output.  uniform_T: use gdn_prefill with
    B = N sequences of that length; else gdn_prefill_varlen."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    N, Hqk, Hv, d = x["N"], x["Hqk"], x["Hv"], x["d"]
    C_tot = 2 * Hqk * d + Hv * d
    w = dev_bf16(x["conv_w"])
    st = None if x["state_in"] is None else dev_f32(x["state_in"])
    cs = None if x["conv_state_in"] is None else dev_bf16(x["conv_state_in"])
    cso = torch.zeros((N, 3, C_tot), dtype=torch.bfloat16, device="cuda") if conv_out else None
    if uniform_T is not None:
        T = uniform_T
        q = dev_bf16(x["q"].reshape(N, T, Hqk, d))
        k = dev_bf16(x["k"].reshape(N, T, Hqk, d))
        v = dev_bf16(x["v"].reshape(N, T, Hv, d))
        a = dev_f32(x["a"].reshape(N, T, Hv))
        b = dev_f32(x["b"].reshape(N, T, Hv))
        o, so, cso = gdn.gdn_prefill(q, k, v, a, b, w, gate_scale=x["gate_scale"], state_in=st,
                                     conv_state_in=cs, conv_state_out=cso)
        o = o.reshape(N * T, Hv, d)
    else:
        q, k, v = dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"])
        a, b = dev_f32(x["a"]), dev_f32(x["b"])
        cu = dev_i32(x["cu_seqlens"])
        o, so, cso = gdn.gdn_prefill_varlen(q, k, v, a, b, w, cu, gate_scale=x["gate_scale"],
                                            state_in=st, conv_state_in=cs, conv_state_out=cso)
    torch.cuda.synchronize()
    return o, so, cso


def oracle_prefill(x, heads=None):
    return oracle.prefill(x["q"], x["k"], x["v"], x["a"], x["b"], x["conv_w"], x["cu_seqlens"],
                          Hqk=x["Hqk"], Hv=x["Hv"], gate_scale=x["gate_scale"],
                          state_in=x["state_in"], conv_state_in=x["conv_state_in"], heads=heads)


def compare(x, o, so, cso, heads=None, seqs=None):
    o_ref, s_ref, cs_ref = oracle_prefill(x, heads)
    hs = list(range(x["Hv"])) if heads is None else list(heads)
    og = host_bf16(o)
    check_output(og[:, hs], o_ref[:, hs])
    sg = so.cpu().numpy()
    check_state(sg[:, hs], s_ref[:, hs])
    if cso is not None:
        np.testing.assert_array_equal(host_u16(cso), cs_ref)
    return og, sg


def test_config0_tiny(oracle_lib):
    x = inputs.make_config(0)
    o, so, cso = gpu_prefill(x, uniform_T=512)
    compare(x, o, so, cso)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 63, 64, 65, 100, 129, 200])
def test_ragged_lengths_with_carries(oracle_lib, T):
    x = inputs.make_prefill(T_list=[T, T], Hqk=2, Hv=6, seed=300 + T, state_std=0.05,
                            conv_state_std=1.0)
    o, so, cso = gpu_prefill(x, uniform_T=T)
    compare(x, o, so, cso)


@pytest.mark.parametrize("Hqk,Hv", [(1, 1), (4, 4), (2, 8), (3, 6), (1, 6), (2, 16)])
def test_head_groupings(oracle_lib, Hqk, Hv):
    x = inputs.make_prefill(T_list=[150], Hqk=Hqk, Hv=Hv, seed=400 + Hv, state_std=0.05)
    o, so, cso = gpu_prefill(x, uniform_T=150)
    compare(x, o, so, cso)


def test_varlen_small_with_empty_sequences(oracle_lib):
    x = inputs.make_prefill(T_list=[0, 70, 1, 0, 128, 2, 33], Hqk=2, Hv=6, seed=500,
                            state_std=0.05, conv_state_std=1.0)
    o, so, cso = gpu_prefill(x)
    compare(x, o, so, cso)
    # empty sequences pass their state through unchanged
    np.testing.assert_array_equal(so.cpu().numpy()[[0, 3]], x["state_in"][[0, 3]])


def test_segmented_pass_weak_and_strong_decay(oracle_lib):
    """A sequence long enough for the sequential pass to be cut into segments.
    V heads 0-2 barely decay (alpha ~ 1), except over tokens 4000-4399 where
    they decay hard: their segments within 64 chunks of the start restart
    from the initial state, those just after the strong stretch start from a
    truncated warm-up, and the rest miss the warm-up bound and are recomputed
    in order from the state handed over.  Heads 3-5 decay as usual."""
    T = 8192 + 37
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=510, state_std=0.05, conv_state_std=1.0)
    x["a"][:, :3] = -9.0
    x["a"][4000:4400, :3] = 5.0
    o, so, cso = gpu_prefill(x, uniform_T=T)
    compare(x, o, so, cso)


def test_segmented_varlen_mixed_decay(oracle_lib):
    """Packed sequences of several lengths cut into segments, two V heads
    without decay (recomputed in order) beside normally decaying ones."""
    x = inputs.make_prefill(T_list=[5000, 300, 9001, 0, 4500], Hqk=2, Hv=6, seed=511, state_std=0.05)
    x["a"][:, 1] = -9.0
    x["a"][:, 4] = -9.0
    o, so, cso = gpu_prefill(x)
    compare(x, o, so, cso)


def test_in_place_state_with_segments():
    """state_out == state_in on a sequence cut into many segments (some of
    them recomputed in order) gives exactly the out-of-place result."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    T = 8192 + 37
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=512, state_std=0.05)
    x["a"][:, :2] = -9.0  # two heads without decay: their later segments are recomputed
    o1, s1, _ = gpu_prefill(x, uniform_T=T, conv_out=False)
    d = x["d"]
    st = dev_f32(x["state_in"])
    o2, s2, _ = gdn.gdn_prefill(dev_bf16(x["q"].reshape(1, T, 2, d)), dev_bf16(x["k"].reshape(1, T, 2, d)),
                                dev_bf16(x["v"].reshape(1, T, 6, d)), dev_f32(x["a"].reshape(1, T, 6)),
                                dev_f32(x["b"].reshape(1, T, 6)), dev_bf16(x["conv_w"]),
                                gate_scale=x["gate_scale"], state_in=st, state_out=st)
    torch.cuda.synchronize()
    assert s2.data_ptr() == st.data_ptr()
    np.testing.assert_array_equal(host_u16(o2.reshape(T, 6, d)), host_u16(o1))
    np.testing.assert_array_equal(st.cpu().numpy(), s1.cpu().numpy())


def test_zero_length_batch_copies_state(oracle_lib):
    x = inputs.make_prefill(T_list=[0, 0], Hqk=2, Hv=6, seed=501, state_std=0.05, conv_state_std=1.0)
    o, so, cso = gpu_prefill(x, uniform_T=0)
    np.testing.assert_array_equal(so.cpu().numpy(), x["state_in"])
    np.testing.assert_array_equal(host_u16(cso), x["conv_state_in"])


def test_varlen_equals_per_sequence_bitwise():
    x = inputs.make_prefill(T_list=[90, 64, 7, 200], Hqk=2, Hv=6, seed=502, state_std=0.05)
    o, so, _ = gpu_prefill(x, conv_out=False)
    og, sg = host_u16(o), so.cpu().numpy()
    cu = x["cu_seqlens"]
    for s in range(4):
        sub = dict(x)
        t0, t1 = cu[s], cu[s + 1]
        for key in ("q", "k", "v", "a", "b"):
            sub[key] = x[key][t0:t1]
        sub["cu_seqlens"] = np.array([0, t1 - t0], np.int32)
        sub["N"], sub["T_tot"] = 1, t1 - t0
        sub["state_in"] = x["state_in"][s:s + 1]
        o1, s1, _ = gpu_prefill(sub, uniform_T=t1 - t0, conv_out=False)
        np.testing.assert_array_equal(host_u16(o1), og[t0:t1])
        np.testing.assert_array_equal(s1.cpu().numpy()[0], sg[s])


def test_deterministic_bitwise():
    x = inputs.make_prefill(T_list=[300], Hqk=2, Hv=6, seed=503, state_std=0.05)
    o1, s1, _ = gpu_prefill(x, uniform_T=300, conv_out=False)
    o2, s2, _ = gpu_prefill(x, uniform_T=300, conv_out=False)
    np.testing.assert_array_equal(host_u16(o1), host_u16(o2))
    np.testing.assert_array_equal(s1.cpu().numpy(), s2.cpu().numpy())


def test_split_with_carries_matches_whole(oracle_lib):
    """prefill(x[:T]) == prefill(x[T1:], carries of prefill(x[:T1])) within tolerance."""
    T, T1 = 200, 77
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=504, state_std=0.05, conv_state_std=1.0)
    o, so, cso = gpu_prefill(x, uniform_T=T)
    a, b = dict(x), dict(x)
    for key in ("q", "k", "v", "a", "b"):
        a[key], b[key] = x[key][:T1], x[key][T1:]
    a["cu_seqlens"], b["cu_seqlens"] = np.array([0, T1], np.int32), np.array([0, T - T1], np.int32)
    oa, sa, csa = gpu_prefill(a, uniform_T=T1)
    b["state_in"] = sa.cpu().numpy()
    b["conv_state_in"] = host_u16(csa)
    ob, sb, csb = gpu_prefill(b, uniform_T=T - T1)
    o_ref, s_ref, cs_ref = oracle_prefill(x)
    check_output(np.concatenate([host_bf16(oa), host_bf16(ob)]), o_ref)
    check_state(sb.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(host_u16(csb), cs_ref)


def test_decode_steps_match_prefill(oracle_lib):
    """64 decode steps carry the same state as a 64-token prefill."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    T = 64
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=505, state_std=0.05, conv_state_std=1.0)
    o, so, cso = gpu_prefill(x, uniform_T=T)
    conv = dev_bf16(x["conv_state_in"])
    st = dev_f32(x["state_in"])
    w = dev_bf16(x["conv_w"])
    outs = []
    for t in range(T):
        od, st = gdn.gdn_decode_step(dev_bf16(x["q"][t:t + 1]), dev_bf16(x["k"][t:t + 1]),
                                     dev_bf16(x["v"][t:t + 1]), dev_f32(x["a"][t:t + 1]),
                                     dev_f32(x["b"][t:t + 1]), w, conv, st, gate_scale=x["gate_scale"])
        outs.append(host_bf16(od)[0])
    torch.cuda.synchronize()
    o_ref, s_ref, cs_ref = oracle_prefill(x)
    check_output(np.stack(outs), o_ref)
    check_state(st.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(host_u16(conv), host_u16(cso))
    # the two GPU paths agree with each other as closely as each agrees with the oracle
    assert rel_l2(np.stack(outs), host_bf16(o)) < 1e-2


def test_config1_layer_prefill(oracle_lib):
    x = inputs.make_config(1)
    o, so, cso = gpu_prefill(x, uniform_T=8192)
    compare(x, o, so, cso)


def test_config4_varlen_sampled(oracle_lib):
    """64 packed sequences, lengths log-uniform in [128, 32768], nonzero
    initial states.  The GPU runs the whole batch; the oracle checks (a) the
    shortest, the longest and four other sequences in full, and (b) the first
    64 outputs of every sequence, where the carried-in state still matters
    (it decays to ~1e-11 of its size within a few hundred tokens)."""
    x = inputs.make_config(4)
    o, so, cso = gpu_prefill(x)
    og, sg, csg = host_bf16(o), so.cpu().numpy(), host_u16(cso)
    cu = x["cu_seqlens"]
    L = np.diff(cu)
    pick = sorted(set([int(np.argmin(L)), int(np.argmax(L)), 3, 17, 40, 63]))
    for s in pick:
        sub = dict(x)
        t0, t1 = cu[s], cu[s + 1]
        for key in ("q", "k", "v", "a", "b"):
            sub[key] = x[key][t0:t1]
        sub["cu_seqlens"] = np.array([0, t1 - t0], np.int32)
        sub["state_in"] = x["state_in"][s:s + 1]
        o_ref, s_ref, cs_ref = oracle_prefill(sub)
        check_output(og[t0:t1], o_ref, what=f"o seq {s}")
        check_state(sg[s:s + 1], s_ref, what=f"state seq {s}")
        np.testing.assert_array_equal(csg[s], cs_ref[0])
    # first 64 tokens of every sequence
    head = dict(x)
    idx = np.concatenate([np.arange(cu[s], cu[s] + 64) for s in range(len(L))])
    for key in ("q", "k", "v", "a", "b"):
        head[key] = x[key][idx]
    head["cu_seqlens"] = np.arange(0, 64 * len(L) + 1, 64, dtype=np.int32)
    o_ref, _, _ = oracle_prefill(head)
    check_output(og[idx], o_ref, what="first 64 tokens of every sequence")


def test_config2_native_context_three_heads(oracle_lib):
    """T = 262,144 with long memory (gate scale 0.02); the oracle evaluates V
    heads 0, 23 and 47 over the whole length."""
    import torch
    x = inputs.make_config(2)
    o, so, _ = gpu_prefill(x, uniform_T=262144, conv_out=False)
    heads = [0, 23, 47]
    og = host_bf16(o[:, heads])
    sg = so[:, heads].cpu().numpy()
    del o
    torch.cuda.empty_cache()
    o_ref, s_ref, _ = oracle_prefill(x, heads=heads)
    check_output(og, o_ref[:, heads])
    check_state(sg, s_ref[:, heads])


def test_stale_workspace_segmented():
    """A workspace full of 0xFF bytes (as a previous call may leave it) gives
    the same results bit for bit, in the case that uses the workspace most: a
    sequence cut into segments, two of whose V heads do not decay, so that
    the segment counters elect a workgroup for the in-order walk."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    T = 8192 + 37
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=513, state_std=0.05, conv_state_std=1.0)
    x["a"][:, :2] = -9.0
    d = x["d"]
    args = (dev_bf16(x["q"].reshape(1, T, 2, d)), dev_bf16(x["k"].reshape(1, T, 2, d)),
            dev_bf16(x["v"].reshape(1, T, 6, d)), dev_f32(x["a"].reshape(1, T, 6)),
            dev_f32(x["b"].reshape(1, T, 6)), dev_bf16(x["conv_w"]))
    need = gdn.gdn_prefill_workspace_size(1, T, 2, 6)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        o, so, _ = gdn.gdn_prefill(*args, gate_scale=x["gate_scale"], state_in=dev_f32(x["state_in"]),
                                   conv_state_in=dev_bf16(x["conv_state_in"]), workspace=ws)
        torch.cuda.synchronize()
        outs.append((host_u16(o), so.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])
