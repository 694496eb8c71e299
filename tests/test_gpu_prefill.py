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


def compare(x, o, so, cso, heads=None, label=None):
    o_ref, s_ref, cs_ref = oracle_prefill(x, heads)
    hs = list(range(x["Hv"])) if heads is None else list(heads)
    og = host_bf16(o)
    r_o, ex = check_output(og[:, hs], o_ref[:, hs])
    sg = so.cpu().numpy()
    r_s = check_state(sg[:, hs], s_ref[:, hs])
    if cso is not None:
        np.testing.assert_array_equal(host_u16(cso), cs_ref)
    if label:
        print(f"{label} margins: o relL2 {r_o:.2e}, max-abs excess {ex:.2e} RMS, state relL2 {r_s:.2e}",
              flush=True)
    return og, sg


def test_config0_tiny(oracle_lib):
    x = inputs.make_config(0)
    o, so, cso = gpu_prefill(x, uniform_T=512)
    compare(x, o, so, cso, label="config 0")


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
    truncated warm-up, and the rest miss the warm-up bound and go through
    their transition matrices and the in-order combine.  Heads 3-5 decay as
    usual."""
    T = 8192 + 37
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=510, state_std=0.05, conv_state_std=1.0)
    x["a"][:, :3] = -9.0
    x["a"][4000:4400, :3] = 5.0
    o, so, cso = gpu_prefill(x, uniform_T=T)
    compare(x, o, so, cso)


def test_long_chain_of_segment_maps(oracle_lib):
    """No V head decays over a 32,787-token sequence, so every segment after
    the first misses its warm-up bound: some forty segment maps S -> M S + S0
    are chained in order (each product while the next M is in flight) before
    the extra workgroups form the segments' outputs.  All heads against the
    oracle, with a carried-in state and conv rows."""
    T = 32768 + 19
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=514, state_std=0.05, conv_state_std=1.0)
    x["a"][:] = -9.0
    o, so, cso = gpu_prefill(x, uniform_T=T)
    compare(x, o, so, cso, label="long chain of segment maps")


def test_segmented_varlen_mixed_decay(oracle_lib):
    """Packed sequences of several lengths cut into segments, two V heads
    without decay (their later segments through transition matrices and the
    in-order combine) beside normally decaying ones."""
    x = inputs.make_prefill(T_list=[5000, 300, 9001, 0, 4500], Hqk=2, Hv=6, seed=511, state_std=0.05)
    x["a"][:, 1] = -9.0
    x["a"][:, 4] = -9.0
    o, so, cso = gpu_prefill(x)
    compare(x, o, so, cso)


def test_in_place_state_with_segments():
    """state_out == state_in on a sequence cut into many segments (some of
    them missing their warm-up bounds) gives exactly the out-of-place result."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    T = 8192 + 37
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=512, state_std=0.05)
    x["a"][:, :2] = -9.0  # two heads without decay: their later segments miss the bound
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
    compare(x, o, so, cso, label="config 1")


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
    worst = [0.0, 0.0, 0.0]
    for s in pick:
        sub = dict(x)
        t0, t1 = cu[s], cu[s + 1]
        for key in ("q", "k", "v", "a", "b"):
            sub[key] = x[key][t0:t1]
        sub["cu_seqlens"] = np.array([0, t1 - t0], np.int32)
        sub["state_in"] = x["state_in"][s:s + 1]
        o_ref, s_ref, cs_ref = oracle_prefill(sub)
        r_o, ex = check_output(og[t0:t1], o_ref, what=f"o seq {s}")
        r_s = check_state(sg[s:s + 1], s_ref, what=f"state seq {s}")
        worst = [max(worst[0], r_o), max(worst[1], ex), max(worst[2], r_s)]
        np.testing.assert_array_equal(csg[s], cs_ref[0])
    # first 64 tokens of every sequence
    head = dict(x)
    idx = np.concatenate([np.arange(cu[s], cu[s] + 64) for s in range(len(L))])
    for key in ("q", "k", "v", "a", "b"):
        head[key] = x[key][idx]
    head["cu_seqlens"] = np.arange(0, 64 * len(L) + 1, 64, dtype=np.int32)
    o_ref, _, _ = oracle_prefill(head)
    r_h, ex_h = check_output(og[idx], o_ref, what="first 64 tokens of every sequence")
    print(f"config 4 margins (worst of the sampled sequences): o relL2 {worst[0]:.2e}, max-abs excess "
          f"{worst[1]:.2e} RMS, state relL2 {worst[2]:.2e}; first 64 tokens of all: o relL2 {r_h:.2e}, "
          f"max-abs excess {ex_h:.2e} RMS", flush=True)


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
    r_o, ex = check_output(og, o_ref[:, heads])
    r_s = check_state(sg, s_ref[:, heads])
    worst_head = max(check_state(sg[:, i], s_ref[:, h], what=f"state head {h}") for i, h in enumerate(heads))
    print(f"config 2 margins (V heads 0, 23, 47): o relL2 {r_o:.2e}, max-abs excess {ex:.2e} RMS, "
          f"state relL2 {r_s:.2e} (worst head {worst_head:.2e})", flush=True)


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


# ---------------------------------------------------------------------------
# slot tables into state / conv-row pools, conv rows in place
# ---------------------------------------------------------------------------
def _pool_case(lens, rows, seed, Hqk=2, Hv=6, bad=None):
    """Packed sequences whose states and conv rows live in pools of `rows`
    rows; sequence s uses row slots[s] (slots[bad] lies outside the pool)."""
    x = inputs.make_prefill(T_list=lens, Hqk=Hqk, Hv=Hv, seed=seed, state_std=0.05, conv_state_std=1.0)
    rng = np.random.default_rng(seed + 1)
    N, d = len(lens), x["d"]
    C_tot = 2 * Hqk * d + Hv * d
    slots = rng.permutation(rows)[:N].astype(np.int32)
    if bad is not None:
        slots[bad] = rows + 5
    ok = [i for i in range(N) if 0 <= slots[i] < rows]
    pool_st = (rng.standard_normal((rows, Hv, d, d)) * 0.05).astype(np.float32)
    pool_cs = inputs.bf16_bits(rng.standard_normal((rows, 3, C_tot)).astype(np.float32))
    pool_st[slots[ok]] = x["state_in"][ok]
    pool_cs[slots[ok]] = x["conv_state_in"][ok]
    return x, slots, ok, pool_st, pool_cs


def test_varlen_slots_in_place_against_oracle(oracle_lib):
    """A slot table into pools updated in place (state and conv rows): the
    named rows get the oracle's results with carry-in from those rows, other
    rows stay untouched, and a sequence whose slot lies outside the pool
    writes nothing (its output rows keep their previous contents)."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    lens = [70, 0, 200, 5, 64, 129, 2]
    rows = 11
    x, slots, ok, pool_st, pool_cs = _pool_case(lens, rows, seed=560, bad=3)
    d, Hv = x["d"], x["Hv"]
    st, cs = dev_f32(pool_st), dev_bf16(pool_cs)
    o = torch.full((x["T_tot"], Hv, d), 7.0, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_prefill_varlen(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), dev_f32(x["a"]), dev_f32(x["b"]),
                           dev_bf16(x["conv_w"]), dev_i32(x["cu_seqlens"]), gate_scale=x["gate_scale"],
                           state_in=st, state_out=st, conv_state_in=cs, conv_state_out=cs, o=o,
                           slots=dev_i32(slots))
    torch.cuda.synchronize()
    og, sg, cg = host_bf16(o), st.cpu().numpy(), host_u16(cs)
    cu = x["cu_seqlens"]
    # the oracle on the sequences that have a slot, carried in from their rows
    sub = dict(x)
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in ok])
    for key in ("q", "k", "v", "a", "b"):
        sub[key] = x[key][idx]
    sub["cu_seqlens"] = np.concatenate([[0], np.cumsum([lens[s] for s in ok])]).astype(np.int32)
    sub["state_in"] = pool_st[slots[ok]]
    sub["conv_state_in"] = pool_cs[slots[ok]]
    o_ref, s_ref, cs_ref = oracle_prefill(sub)
    check_output(og[idx], o_ref)
    check_state(sg[slots[ok]], s_ref)
    np.testing.assert_array_equal(cg[slots[ok]], cs_ref)
    untouched = sorted(set(range(rows)) - set(slots[ok].tolist()))
    np.testing.assert_array_equal(sg[untouched], pool_st[untouched])
    np.testing.assert_array_equal(cg[untouched], pool_cs[untouched])
    assert np.all(og[cu[3]:cu[4]] == 7.0)  # the skipped sequence
    # the empty sequence's row holds its carried state unchanged
    np.testing.assert_array_equal(sg[slots[1]], pool_st[slots[1]])


def test_varlen_slots_in_place_segmented_no_decay(oracle_lib):
    """Long packed sequences through a slot table into pools updated in place,
    cut into segments, with two V heads that do not decay: their later
    segments go through the segment maps, whose in-order pass also moves the
    final states into the pool rows and writes the v conv rows last."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    lens = [9000, 0, 5000, 300]
    rows = 7
    x, slots, ok, pool_st, pool_cs = _pool_case(lens, rows, seed=570, bad=3)
    x["a"][:, 1] = -9.0
    x["a"][:, 4] = -9.0
    d, Hv = x["d"], x["Hv"]
    st, cs = dev_f32(pool_st), dev_bf16(pool_cs)
    o = torch.full((x["T_tot"], Hv, d), 7.0, dtype=torch.bfloat16, device="cuda")
    gdn.gdn_prefill_varlen(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), dev_f32(x["a"]), dev_f32(x["b"]),
                           dev_bf16(x["conv_w"]), dev_i32(x["cu_seqlens"]), gate_scale=x["gate_scale"],
                           state_in=st, state_out=st, conv_state_in=cs, conv_state_out=cs, o=o,
                           slots=dev_i32(slots))
    torch.cuda.synchronize()
    og, sg, cg = host_bf16(o), st.cpu().numpy(), host_u16(cs)
    cu = x["cu_seqlens"]
    sub = dict(x)
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in ok])
    for key in ("q", "k", "v", "a", "b"):
        sub[key] = x[key][idx]
    sub["cu_seqlens"] = np.concatenate([[0], np.cumsum([lens[s] for s in ok])]).astype(np.int32)
    sub["state_in"] = pool_st[slots[ok]]
    sub["conv_state_in"] = pool_cs[slots[ok]]
    o_ref, s_ref, cs_ref = oracle_prefill(sub)
    check_output(og[idx], o_ref)
    check_state(sg[slots[ok]], s_ref)
    np.testing.assert_array_equal(cg[slots[ok]], cs_ref)
    untouched = sorted(set(range(rows)) - set(slots[ok].tolist()))
    np.testing.assert_array_equal(sg[untouched], pool_st[untouched])
    np.testing.assert_array_equal(cg[untouched], pool_cs[untouched])
    assert np.all(og[cu[3]:cu[4]] == 7.0)  # the skipped sequence


def test_varlen_slots_equal_plain_call_bitwise():
    """Through a slot table (out of place, rows permuted) the results are bit
    for bit those of the plain packed call on gathered rows."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    lens = [90, 64, 7, 200]
    rows = 6
    x, slots, ok, pool_st, pool_cs = _pool_case(lens, rows, seed=561)
    o1, s1, c1 = gpu_prefill(x)
    w = dev_bf16(x["conv_w"])
    st_out = dev_f32(np.zeros_like(pool_st))
    cs_out = torch.zeros((rows,) + pool_cs.shape[1:], dtype=torch.bfloat16, device="cuda")
    o2, _, _ = gdn.gdn_prefill_varlen(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), dev_f32(x["a"]),
                                      dev_f32(x["b"]), w, dev_i32(x["cu_seqlens"]), gate_scale=x["gate_scale"],
                                      state_in=dev_f32(pool_st), state_out=st_out,
                                      conv_state_in=dev_bf16(pool_cs), conv_state_out=cs_out, slots=dev_i32(slots))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(o2), host_u16(o1))
    np.testing.assert_array_equal(st_out.cpu().numpy()[slots], s1.cpu().numpy())
    np.testing.assert_array_equal(host_u16(cs_out)[slots], host_u16(c1))


def test_conv_rows_in_place_segmented(oracle_lib):
    """conv_state_out == conv_state_in on a sequence cut into segments, where
    later segments restart from the sequence start (and so read the incoming
    conv rows) and others miss the warm-up bound: bit for bit the
    out-of-place result, which the oracle checks."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    T = 8192 + 37
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=562, state_std=0.05, conv_state_std=1.0)
    x["a"][:, :3] = -9.0
    x["a"][4000:4400, :3] = 5.0
    o1, s1, c1 = gpu_prefill(x, uniform_T=T)
    compare(x, o1, s1, c1)
    d = x["d"]
    cs = dev_bf16(x["conv_state_in"])
    o2, s2, _ = gdn.gdn_prefill(dev_bf16(x["q"].reshape(1, T, 2, d)), dev_bf16(x["k"].reshape(1, T, 2, d)),
                                dev_bf16(x["v"].reshape(1, T, 6, d)), dev_f32(x["a"].reshape(1, T, 6)),
                                dev_f32(x["b"].reshape(1, T, 6)), dev_bf16(x["conv_w"]), gate_scale=x["gate_scale"],
                                state_in=dev_f32(x["state_in"]), conv_state_in=cs, conv_state_out=cs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(o2.reshape(T, 6, d)), host_u16(o1))
    np.testing.assert_array_equal(s2.cpu().numpy(), s1.cpu().numpy())
    np.testing.assert_array_equal(host_u16(cs), host_u16(c1))


def test_conv_rows_in_place_short_sequences(oracle_lib):
    """In place with sequences shorter than the conv window: the new rows
    reach back into the incoming ones, which are read before they are
    overwritten."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    x = inputs.make_prefill(T_list=[1, 2, 0, 3, 40], Hqk=2, Hv=6, seed=563, state_std=0.05, conv_state_std=1.0)
    _, _, cs_ref = oracle_prefill(x)
    cs = dev_bf16(x["conv_state_in"])
    gdn.gdn_prefill_varlen(dev_bf16(x["q"]), dev_bf16(x["k"]), dev_bf16(x["v"]), dev_f32(x["a"]), dev_f32(x["b"]),
                           dev_bf16(x["conv_w"]), dev_i32(x["cu_seqlens"]), gate_scale=x["gate_scale"],
                           state_in=dev_f32(x["state_in"]), conv_state_in=cs, conv_state_out=cs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_u16(cs), cs_ref)


def _prefill_small_workspace(x, T, ws_tokens, in_place=False, carries=True):
    """gdn_prefill of N sequences of T tokens with a workspace sized for
    ws_tokens tokens per sequence, less than the call needs: the library runs
    the call in windows, carrying the state and the conv rows between them."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    N, Hqk, Hv, d = x["N"], x["Hqk"], x["Hv"], x["d"]
    C_tot = 2 * Hqk * d + Hv * d
    need = gdn.gdn_prefill_workspace_size(N, T, Hqk, Hv)
    ws = torch.empty(gdn.gdn_prefill_workspace_size(N, ws_tokens, Hqk, Hv), dtype=torch.uint8, device="cuda")
    assert ws.numel() < need
    st = dev_f32(x["state_in"]) if carries else None
    cs = dev_bf16(x["conv_state_in"]) if carries else None
    so = st if in_place else None
    cso = cs if in_place else torch.zeros((N, 3, C_tot), dtype=torch.bfloat16, device="cuda")
    o, so, cso = gdn.gdn_prefill(dev_bf16(x["q"].reshape(N, T, Hqk, d)), dev_bf16(x["k"].reshape(N, T, Hqk, d)),
                                 dev_bf16(x["v"].reshape(N, T, Hv, d)), dev_f32(x["a"].reshape(N, T, Hv)),
                                 dev_f32(x["b"].reshape(N, T, Hv)), dev_bf16(x["conv_w"]),
                                 gate_scale=x["gate_scale"], state_in=st, conv_state_in=cs, state_out=so,
                                 conv_state_out=cso, workspace=ws)
    torch.cuda.synchronize()
    return o.reshape(N * T, Hv, d), so, cso


@pytest.mark.parametrize("T,ws_tokens", [(700, 192), (194, 64), (130, 64)])
def test_windowed_prefill_against_oracle(oracle_lib, T, ws_tokens):
    """A workspace smaller than the call's: the call runs in windows of whole
    chunks (the last one 2 tokens long in the second and third cases, whose
    carried conv rows reach back into the previous window's rows), and
    matches the oracle and the one-window call."""
    x = inputs.make_prefill(T_list=[T, T], Hqk=2, Hv=6, seed=811 + T, state_std=0.05, conv_state_std=1.0)
    o, so, cso = _prefill_small_workspace(x, T, ws_tokens)
    og, sg = compare(x, o, so, cso, label=f"windowed T={T} (windows of {ws_tokens})")
    o1, s1, cs1 = gpu_prefill(x, uniform_T=T)
    assert rel_l2(og, host_bf16(o1)) < 1e-3
    assert rel_l2(sg, s1.cpu().numpy()) < 1e-4
    np.testing.assert_array_equal(host_u16(cso), host_u16(cs1))


def test_windowed_prefill_in_place(oracle_lib):
    """Windows with the state and the conv rows updated in place."""
    T = 450
    x = inputs.make_prefill(T_list=[T, T, T], Hqk=2, Hv=6, seed=823, state_std=0.05, conv_state_std=1.0)
    o, so, cso = _prefill_small_workspace(x, T, 128, in_place=True)
    compare(x, o, so, cso)


def test_noalloc_beyond_its_array_runs_in_windows(oracle_lib):
    """gdn_prefill_noalloc on a layer longer than its array holds (16 QK / 48
    V heads, T = 16,384): the oracle on V heads 0, 23 and 47, and the plain
    call with a whole workspace on all heads."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    T, Hqk, Hv, d = 16384, 16, 48, 128
    assert gdn.gdn_prefill_workspace_size(1, T, Hqk, Hv) > gdn.gdn_prefill_noalloc_max_workspace()
    x = inputs.make_prefill(T_list=[T], Hqk=Hqk, Hv=Hv, seed=829, state_std=0.05, conv_state_std=1.0)
    args = (dev_bf16(x["q"].reshape(1, T, Hqk, d)), dev_bf16(x["k"].reshape(1, T, Hqk, d)),
            dev_bf16(x["v"].reshape(1, T, Hv, d)), dev_f32(x["a"].reshape(1, T, Hv)),
            dev_f32(x["b"].reshape(1, T, Hv)), dev_bf16(x["conv_w"]))
    kw = dict(gate_scale=x["gate_scale"], state_in=dev_f32(x["state_in"]), conv_state_in=dev_bf16(x["conv_state_in"]))
    C_tot = 2 * Hqk * d + Hv * d
    cso = torch.zeros((1, 3, C_tot), dtype=torch.bfloat16, device="cuda")
    o, so, cso = gdn.gdn_prefill_noalloc(*args, conv_state_out=cso, **kw)
    torch.cuda.synchronize()
    o1, s1, cs1 = gdn.gdn_prefill(*args, conv_state_out=torch.zeros_like(cso), **kw)
    torch.cuda.synchronize()
    og, sg = host_bf16(o.reshape(T, Hv, d)), so.cpu().numpy()
    assert rel_l2(og, host_bf16(o1.reshape(T, Hv, d))) < 1e-3
    assert rel_l2(sg, s1.cpu().numpy()) < 1e-4
    np.testing.assert_array_equal(host_u16(cso), host_u16(cs1))
    del o1
    torch.cuda.empty_cache()
    # the carried rows are checked against the whole call above (the oracle
    # fills only the selected heads)
    compare(x, o.reshape(T, Hv, d), so, None, heads=[0, 23, 47],
            label="noalloc in windows, T=16384 (V heads 0, 23, 47)")


def test_windowed_prefill_without_carries(oracle_lib):
    """Windows of a call with no initial state and no carried conv rows (the
    first window starts from zeros, the later ones from the handed-over
    state)."""
    T = 333
    x = inputs.make_prefill(T_list=[T], Hqk=2, Hv=6, seed=837)
    assert x["state_in"] is None and x["conv_state_in"] is None
    o, so, cso = _prefill_small_workspace(x, T, 64, carries=False)
    compare(x, o, so, cso, label="windowed T=333 (windows of 64), no carries")
