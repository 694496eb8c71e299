"""Pins of the fp64 oracle against what the equations and mathematics fix.

None of these checks re-types the oracle's own formula: they use exact
rational brute force of the state-update equation, dense explicit products of
the per-token transition matrices (the equation's own matrix form, while the
oracle evaluates the equivalent delta form), library routines for special
cases, closed forms and invariants.  Planted-mistake tests at the end show
that a plausible error in the oracle would fail them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from linear_attention_sequence_gdn_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# scalar activations: closed forms / special values
# --------------------------------------------------------------------------
def test_scalar_activations(oracle_lib):
    o = oracle_lib
    assert o.sigmoid(0.0) == 0.5
    assert o.softplus(0.0) == pytest.approx(math.log(2.0), abs=1e-16)
    assert o.silu(0.0) == 0.0
    for x in [-30.0, -5.0, -1.0, -1e-3, 1e-3, 0.7, 3.0, 20.0]:
        assert o.sigmoid(x) == pytest.approx(1.0 / (1.0 + math.exp(-x)), rel=1e-15)
        assert o.softplus(x) == pytest.approx(math.log1p(math.exp(x)), rel=1e-14)
        assert o.silu(x) == pytest.approx(x / (1.0 + math.exp(-x)), rel=1e-15, abs=1e-300)
    # asymptotics: softplus(x) -> x for large x, -> e^x for very negative x
    assert o.softplus(800.0) == 800.0
    assert o.softplus(-800.0) == pytest.approx(math.exp(-800.0), rel=1e-12, abs=0)
    # symmetry identities
    for x in [0.3, 2.5, 11.0]:
        assert o.sigmoid(x) + o.sigmoid(-x) == pytest.approx(1.0, abs=4e-16)
        assert o.softplus(x) - o.softplus(-x) == pytest.approx(x, abs=1e-14)


def test_gates(oracle_lib):
    a = np.array([-3.0, -0.5, 0.0, 0.25, 4.0], np.float32)
    b = np.array([2.0, -1.0, 0.0, 0.5, -6.0], np.float32)
    al, be = oracle_lib.gates(a, b, 0.1)
    for i in range(5):
        # alpha = exp(-c * log(1 + e^a)), beta = 1 / (1 + e^-b)
        assert al[i] == pytest.approx(math.exp(-0.1 * math.log1p(math.exp(float(a[i])))), rel=1e-15)
        assert be[i] == pytest.approx(1.0 / (1.0 + math.exp(-float(b[i]))), rel=1e-15)
        assert 0.0 < al[i] <= 1.0 and 0.0 < be[i] < 1.0
    al0, _ = oracle_lib.gates(a, b, 0.0)
    assert np.all(al0 == 1.0)  # no decay when the gate scale is zero


# --------------------------------------------------------------------------
# conv + SiLU: library convolution, identity and shift kernels
# --------------------------------------------------------------------------
def _bf(x):
    return inputs.bf16_bits(np.asarray(x, np.float32))


def _f(u):
    return inputs.bf16_to_f32(u).astype(np.float64)


def _silu(y):
    return y / (1.0 + np.exp(-y))


def test_conv_matches_numpy_convolve(oracle_lib):
    rng = np.random.default_rng(7)
    T, C = 37, 9
    x = _bf(rng.standard_normal((T, C)))
    w = _bf(rng.standard_normal((C, 4)) * 0.25)
    hist = _bf(rng.standard_normal((3, C)))
    for h in (None, hist):
        got = oracle_lib.conv_silu(x, w, h)
        pre = np.zeros((3, C)) if h is None else _f(h)
        xs = np.concatenate([pre, _f(x)], axis=0)
        for c in range(C):
            # np.convolve flips its kernel: tap 3 (current token) must meet x[t]
            y = np.convolve(xs[:, c], _f(w)[c, ::-1], mode="valid")
            np.testing.assert_allclose(got[:, c], _silu(y), rtol=1e-14, atol=1e-300)


def test_conv_identity_and_shift(oracle_lib):
    rng = np.random.default_rng(8)
    T, C = 11, 5
    x = _bf(rng.standard_normal((T, C)))
    hist = _bf(rng.standard_normal((3, C)))
    for j in range(4):
        w = np.zeros((C, 4), np.float32)
        w[:, j] = 1.0
        got = oracle_lib.conv_silu(x, _bf(w), hist)
        shift = 3 - j  # tap j reads the token `shift` steps back
        full = np.concatenate([_f(hist), _f(x)], axis=0)
        want = _silu(full[3 - shift: 3 - shift + T])
        np.testing.assert_allclose(got, want, rtol=5e-16, atol=0)
        # zero history: the first `shift` rows see zeros -> SiLU(0) = 0
        got0 = oracle_lib.conv_silu(x, _bf(w), None)
        assert np.all(got0[:shift] == 0.0)


def test_l2norm_unit_and_direction(oracle_lib):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((20, 128)) * 3.0
    y = oracle_lib.l2norm(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), 1.0, atol=1e-14)
    # same direction: y is a positive multiple of x
    ratio = y / x
    np.testing.assert_allclose(ratio, ratio[:, :1] * np.ones_like(ratio), rtol=1e-13)
    assert np.all(ratio > 0)
    # eps keeps the zero vector finite
    assert np.all(oracle_lib.l2norm(np.zeros((1, 4))) == 0.0)


# --------------------------------------------------------------------------
# the recurrence
# --------------------------------------------------------------------------
def _parse_golden(path):
    vals = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, rest = line.split(":", 1)
        vals[name.strip()] = [Fraction(t) for t in rest.split()]
    return vals


def test_hand_worked_example(oracle_lib):
    g = _parse_golden(os.path.join(GOLDEN, "hand_example_d2.txt"))
    f = lambda key, shape: np.array([float(x) for x in g[key]]).reshape(shape)
    o, S = oracle_lib.recurrence(f("q", (2, 2)), f("k", (2, 2)), f("v", (2, 2)),
                                 f("alpha", (2,)), f("beta", (2,)), S0=f("S0", (2, 2)))
    np.testing.assert_array_equal(o, f("o", (2, 2)))
    np.testing.assert_array_equal(S, f("S2", (2, 2)))


def _exact_update(S0, qs, ks, vs, al, be):
    """The walkthrough's update S_t = a(I - b k k^T) S + b k v^T in exact
    rational arithmetic, with the readout o_t = S_t^T q_t."""
    dk, dv = len(S0), len(S0[0])
    S = [row[:] for row in S0]
    outs = []
    for q, k, v, a, b in zip(qs, ks, vs, al, be):
        M = [[a * ((1 if i == j else 0) - b * k[i] * k[j]) for j in range(dk)] for i in range(dk)]
        S = [[sum(M[i][m] * S[m][j] for m in range(dk)) + b * k[i] * v[j] for j in range(dv)]
             for i in range(dk)]
        outs.append([sum(S[i][j] * q[i] for i in range(dk)) for j in range(dv)])
    return outs, S


def test_exact_rational_bruteforce(oracle_lib):
    rng = np.random.default_rng(11)
    T, dk, dv = 6, 3, 4
    rnd = lambda *s: [[Fraction(int(x), 8) for x in row] for row in rng.integers(-8, 9, size=s)]
    qs, ks, vs, S0 = rnd(T, dk), rnd(T, dk), rnd(T, dv), rnd(dk, dv)
    al = [Fraction(int(x), 16) for x in rng.integers(8, 17, size=T)]
    be = [Fraction(int(x), 16) for x in rng.integers(0, 17, size=T)]
    outs, S = _exact_update(S0, qs, ks, vs, al, be)
    fl = lambda m: np.array([[float(x) for x in row] for row in m])
    o_or, S_or = oracle_lib.recurrence(fl(qs), fl(ks), fl(vs), [float(x) for x in al],
                                       [float(x) for x in be], S0=fl(S0))
    np.testing.assert_allclose(o_or, fl(outs), rtol=0, atol=1e-13)
    np.testing.assert_allclose(S_or, fl(S), rtol=0, atol=1e-13)


def _dense_unrolled(S0, Q, K, V, al, be):
    """S_T = A_T..A_1 S_0 + sum_s A_T..A_{s+1} b_s k_s v_s^T with explicit
    transition matrices A_t = a_t (I - b_t k_t k_t^T); outputs S_t^T q_t."""
    T, dk = K.shape
    A = [al[t] * (np.eye(dk) - be[t] * np.outer(K[t], K[t])) for t in range(T)]
    outs = []
    for t in range(T):
        P = np.eye(dk)
        St = np.zeros_like(S0)
        for s in range(t, -1, -1):  # accumulate A_t .. A_{s+1} from the right end
            St += P @ (be[s] * np.outer(K[s], V[s]))
            P = P @ A[s]
        St += P @ S0
        outs.append(St.T @ Q[t])
    return np.array(outs), St


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_dense_unrolled_product(oracle_lib, T):
    rng = np.random.default_rng(100 + T)
    dk, dv = 16, 12
    K = rng.standard_normal((T, dk))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q = rng.standard_normal((T, dk))
    V = rng.standard_normal((T, dv))
    S0 = rng.standard_normal((dk, dv)) * 0.3
    al = rng.uniform(0.5, 1.0, T)
    be = rng.uniform(0.0, 1.0, T)
    o_ref, S_ref = _dense_unrolled(S0, Q, K, V, al, be)
    o, S = oracle_lib.recurrence(Q, K, V, al, be, S0=S0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-13)


def test_identity_when_no_write_no_decay(oracle_lib):
    rng = np.random.default_rng(12)
    T, d = 9, 32
    Q, K, V = rng.standard_normal((3, T, d))
    S0 = rng.standard_normal((d, d))
    o, S = oracle_lib.recurrence(Q, K, V, np.ones(T), np.zeros(T), S0=S0)
    np.testing.assert_array_equal(S, S0)
    np.testing.assert_allclose(o, Q @ S0, rtol=1e-14, atol=1e-14)


def test_unit_key_full_write_recalls_value(oracle_lib):
    rng = np.random.default_rng(13)
    T, d = 20, 64
    K = rng.standard_normal((T, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q, V = rng.standard_normal((2, T, d))
    S = rng.standard_normal((d, d))
    for t in range(T):  # after each write, S_t^T k_t == v_t
        _, S = oracle_lib.recurrence(Q[t:t + 1], K[t:t + 1], V[t:t + 1], [1.0], [1.0], S0=S)
        np.testing.assert_allclose(S.T @ K[t], V[t], atol=1e-13)


def test_orthonormal_keys_store_all_pairs(oracle_lib):
    rng = np.random.default_rng(14)
    T, d = 48, 64
    Kq, _ = np.linalg.qr(rng.standard_normal((d, d)))
    K = Kq[:, :T].T  # orthonormal rows
    V = rng.standard_normal((T, d))
    Q = rng.standard_normal((T, d))
    _, S = oracle_lib.recurrence(Q, K, V, np.ones(T), np.ones(T))
    np.testing.assert_allclose(S, K.T @ V, atol=1e-13)
    np.testing.assert_allclose(K @ S, V, atol=1e-13)


def test_pure_decay(oracle_lib):
    rng = np.random.default_rng(15)
    T, d = 30, 16
    Q, K, V = rng.standard_normal((3, T, d))
    S0 = rng.standard_normal((d, d))
    al = rng.uniform(0.8, 1.0, T)
    o, S = oracle_lib.recurrence(Q, K, V, al, np.zeros(T), S0=S0)
    cum = np.cumprod(al)
    np.testing.assert_allclose(S, cum[-1] * S0, rtol=1e-13)
    np.testing.assert_allclose(o, cum[:, None] * (Q @ S0), rtol=1e-12, atol=1e-14)


def test_linearity_in_values_and_state(oracle_lib):
    rng = np.random.default_rng(16)
    T, d = 25, 32
    Q, K, V = rng.standard_normal((3, T, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    S0 = rng.standard_normal((d, d))
    al, be = rng.uniform(0.5, 1, T), rng.uniform(0, 1, T)
    o1, S1 = oracle_lib.recurrence(Q, K, V, al, be, S0=S0)
    o2, S2 = oracle_lib.recurrence(Q, K, 2.5 * V, al, be, S0=2.5 * S0)
    np.testing.assert_allclose(o2, 2.5 * o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, 2.5 * S1, rtol=1e-12, atol=1e-13)
    # superposition: (V, S0) + (V', S0') -> sum of the outputs
    V2, S02 = rng.standard_normal((T, d)), rng.standard_normal((d, d))
    o3, S3 = oracle_lib.recurrence(Q, K, V2, al, be, S0=S02)
    o4, S4 = oracle_lib.recurrence(Q, K, V + V2, al, be, S0=S0 + S02)
    np.testing.assert_allclose(o4, o1 + o3, atol=1e-12)
    np.testing.assert_allclose(S4, S1 + S3, atol=1e-12)


@pytest.mark.parametrize("decay", [True, False])
def test_segment_map_from_identity_run(oracle_lib, decay):
    """The state a stretch of tokens leaves behind is M S + S0 in the state S
    it starts from, where M is the stretch run with zero values from the
    identity and S0 the stretch run from a zero state: what lets a segment
    whose warm-up cannot reach back be chained exactly.  Checked with and
    without decay (alpha = 1)."""
    rng = np.random.default_rng(19)
    T, d = 40, 24
    Q, K, V = rng.standard_normal((3, T, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    al = rng.uniform(0.6, 1.0, T) if decay else np.ones(T)
    be = rng.uniform(0.0, 1.0, T)
    _, M = oracle_lib.recurrence(Q, K, np.zeros_like(V), al, be, S0=np.eye(d))
    _, S0 = oracle_lib.recurrence(Q, K, V, al, be, S0=np.zeros((d, d)))
    for trial in range(3):
        S = rng.standard_normal((d, d))
        _, S_out = oracle_lib.recurrence(Q, K, V, al, be, S0=S)
        np.testing.assert_allclose(S_out, M @ S + S0, rtol=1e-12, atol=1e-12)
    # M is the product of the per-token transitions alpha_t (I - beta_t k_t k_t^T), latest on the left
    P = np.eye(d)
    for t in range(T):
        P = al[t] * (np.eye(d) - be[t] * np.outer(K[t], K[t])) @ P
    np.testing.assert_allclose(M, P, rtol=1e-12, atol=1e-12)


def test_columns_of_state_evolve_independently(oracle_lib):
    rng = np.random.default_rng(17)
    T, d = 15, 16
    Q, K, V = rng.standard_normal((3, T, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    S0 = rng.standard_normal((d, d))
    al, be = rng.uniform(0.5, 1, T), rng.uniform(0, 1, T)
    o, S = oracle_lib.recurrence(Q, K, V, al, be, S0=S0)
    oc, Sc = oracle_lib.recurrence(Q, K, V[:, 3:7], al, be, S0=S0[:, 3:7])
    np.testing.assert_allclose(oc, o[:, 3:7], rtol=0, atol=0)
    np.testing.assert_allclose(Sc, S[:, 3:7], rtol=0, atol=0)


# --------------------------------------------------------------------------
# the whole mixer: wiring of prologue, head sharing, sequences, carries
# --------------------------------------------------------------------------
def _small(seed=3, T_list=(40,), Hqk=2, Hv=6, d=16, state_std=0.0, conv_std=None):
    return inputs.make_prefill(T_list=list(T_list), Hqk=Hqk, Hv=Hv, seed=seed, d=d,
                               state_std=state_std, conv_state_std=conv_std)


def _run(o, x, **kw):
    return o.prefill(x["q"], x["k"], x["v"], x["a"], x["b"], x["conv_w"], x["cu_seqlens"],
                     Hqk=x["Hqk"], Hv=x["Hv"], gate_scale=x["gate_scale"],
                     state_in=kw.get("state_in", x["state_in"]),
                     conv_state_in=kw.get("conv_state_in", x["conv_state_in"]),
                     heads=kw.get("heads"))


def test_prefill_wiring_matches_pieces(oracle_lib):
    x = _small(T_list=(23, 40), state_std=0.1, conv_std=1.0)
    o, S, cs = _run(oracle_lib, x)
    d, Hqk, Hv = x["d"], x["Hqk"], x["Hv"]
    G = Hv // Hqk
    C_tot = 2 * Hqk * d + Hv * d
    w = x["conv_w"]
    for s in range(2):
        t0, t1 = x["cu_seqlens"][s], x["cu_seqlens"][s + 1]
        hist = x["conv_state_in"][s]
        for h in range(Hv):
            g = h // G
            cq, ck, cv = g * d, Hqk * d + g * d, 2 * Hqk * d + h * d
            qh = oracle_lib.l2norm(oracle_lib.conv_silu(x["q"][t0:t1, g], w[cq:cq + d], hist[:, cq:cq + d]))
            kh = oracle_lib.l2norm(oracle_lib.conv_silu(x["k"][t0:t1, g], w[ck:ck + d], hist[:, ck:ck + d]))
            vh = oracle_lib.conv_silu(x["v"][t0:t1, h], w[cv:cv + d], hist[:, cv:cv + d])
            al, be = oracle_lib.gates(x["a"][t0:t1, h], x["b"][t0:t1, h], x["gate_scale"])
            oh, Sh = oracle_lib.recurrence(qh, kh, vh, al, be, S0=x["state_in"][s, h])
            np.testing.assert_array_equal(o[t0:t1, h], oh)
            np.testing.assert_array_equal(S[s, h], Sh)
    assert cs.shape == (2, 3, C_tot)


def test_gqa_duplicate_heads(oracle_lib):
    x = _small(T_list=(30,), Hqk=2, Hv=6)
    # make the three V heads of group 1 identical in every input
    for h in (4, 5):
        x["v"][:, h] = x["v"][:, 3]
        x["a"][:, h] = x["a"][:, 3]
        x["b"][:, h] = x["b"][:, 3]
        d = x["d"]
        base = 2 * x["Hqk"] * d
        x["conv_w"][base + h * d: base + (h + 1) * d] = x["conv_w"][base + 3 * d: base + 4 * d]
    o, S, _ = _run(oracle_lib, x)
    for h in (4, 5):
        np.testing.assert_array_equal(o[:, h], o[:, 3])
        np.testing.assert_array_equal(S[:, h], S[:, 3])
    assert not np.array_equal(o[:, 0], o[:, 3])


def test_varlen_equals_per_sequence(oracle_lib):
    x = _small(T_list=(5, 1, 37, 64, 2), state_std=0.05)
    o, S, cs = _run(oracle_lib, x)
    cu = x["cu_seqlens"]
    for s in range(5):
        t0, t1 = cu[s], cu[s + 1]
        sub = dict(x)
        for key in ("q", "k", "v", "a", "b"):
            sub[key] = x[key][t0:t1]
        sub["cu_seqlens"] = np.array([0, t1 - t0], np.int32)
        sub["state_in"] = x["state_in"][s:s + 1]
        o1, S1, cs1 = _run(oracle_lib, sub)
        np.testing.assert_array_equal(o[t0:t1], o1)
        np.testing.assert_array_equal(S[s], S1[0])
        np.testing.assert_array_equal(cs[s], cs1[0])


def test_split_equals_whole(oracle_lib):
    x = _small(T_list=(50,), state_std=0.05, conv_std=1.0)
    o, S, cs = _run(oracle_lib, x)
    for T1 in (1, 2, 3, 17, 49):
        a = dict(x)
        b = dict(x)
        for key in ("q", "k", "v", "a", "b"):
            a[key] = x[key][:T1]
            b[key] = x[key][T1:]
        a["cu_seqlens"] = np.array([0, T1], np.int32)
        b["cu_seqlens"] = np.array([0, 50 - T1], np.int32)
        oa, Sa, csa = _run(oracle_lib, a)
        ob, Sb, csb = _run(oracle_lib, b, state_in=Sa, conv_state_in=csa)
        np.testing.assert_array_equal(np.concatenate([oa, ob]), o)
        np.testing.assert_array_equal(Sb, S)
        np.testing.assert_array_equal(csb, cs)


def test_conv_state_out_is_last_three_raw_rows(oracle_lib):
    x = _small(T_list=(2, 9), conv_std=1.0)
    _, _, cs = _run(oracle_lib, x)
    Hqk, d = x["Hqk"], x["d"]
    raw = np.concatenate([x["q"].reshape(x["T_tot"], -1), x["k"].reshape(x["T_tot"], -1),
                          x["v"].reshape(x["T_tot"], -1)], axis=1)
    np.testing.assert_array_equal(cs[1], raw[8:11])
    # the 2-token sequence reaches one row back into its incoming history
    np.testing.assert_array_equal(cs[0][0], x["conv_state_in"][0][2])
    np.testing.assert_array_equal(cs[0][1:], raw[0:2])
    assert raw.shape[1] == 2 * Hqk * d + x["Hv"] * d


def test_decode_steps_equal_prefill(oracle_lib):
    x = _small(T_list=(12,), state_std=0.05, conv_std=1.0)
    o, S, cs = _run(oracle_lib, x)
    conv = np.ascontiguousarray(x["conv_state_in"])
    st = np.ascontiguousarray(x["state_in"], dtype=np.float64)
    for t in range(12):
        ot = oracle_lib.decode_step(x["q"][t:t + 1], x["k"][t:t + 1], x["v"][t:t + 1],
                                    x["a"][t:t + 1], x["b"][t:t + 1], x["conv_w"], conv, st,
                                    Hqk=x["Hqk"], Hv=x["Hv"], gate_scale=x["gate_scale"])
        np.testing.assert_array_equal(ot[0], o[t])
    np.testing.assert_array_equal(st, S)
    np.testing.assert_array_equal(conv, cs)


def test_empty_sequence_passes_state_through(oracle_lib):
    x = _small(T_list=(0, 7, 0), state_std=0.05, conv_std=1.0)
    _, S, cs = _run(oracle_lib, x)
    np.testing.assert_array_equal(S[0], x["state_in"][0].astype(np.float64))
    np.testing.assert_array_equal(S[2], x["state_in"][2].astype(np.float64))
    np.testing.assert_array_equal(cs[0], x["conv_state_in"][0])


def test_head_subset_matches_full(oracle_lib):
    x = _small(T_list=(33,))
    o, S, _ = _run(oracle_lib, x)
    os_, Ss, _ = _run(oracle_lib, x, heads=[1, 5])
    for h in (1, 5):
        np.testing.assert_array_equal(os_[:, h], o[:, h])
        np.testing.assert_array_equal(Ss[:, h], S[:, h])
    assert np.all(os_[:, 0] == 0)


# --------------------------------------------------------------------------
# the chunk-parallel (WY) form the GPU kernels use reaches the same result
# --------------------------------------------------------------------------
def chunked_form(Q, K, V, g, beta, S0, C):
    """fp64 chunked evaluation of the same recurrence (the WY / UT form):
    per chunk of n tokens with in-chunk log decays gam = cumsum(g),
      A    = strict_lower(diag(beta) (K K^T) * exp(gam_i - gam_j))
      Tm   = (I + A)^-1 diag(beta)
      W    = Tm diag(e^gam) K,  U' = Tm V
      Vnew = U' - W S
      O    = diag(e^gam) Q S + (Q K^T * exp(gam_i - gam_j) on/below diag) Vnew
      S   <- e^{gam_n} S + (diag(e^{gam_n - gam}) K)^T Vnew
    """
    T = K.shape[0]
    S = S0.copy()
    O = np.zeros((T, V.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        q, k, v, b = Q[sl], K[sl], V[sl], beta[sl]
        gam = np.cumsum(g[sl])
        n = k.shape[0]
        Dm = np.exp(gam[:, None] - gam[None, :])
        low = np.tril(np.ones((n, n)), -1)
        A = (b[:, None] * (k @ k.T) * Dm) * low
        Tm = np.linalg.solve(np.eye(n) + A, np.diag(b))
        W = Tm @ (np.exp(gam)[:, None] * k)
        U = Tm @ v
        Vn = U - W @ S
        P = (q @ k.T) * Dm * np.tril(np.ones((n, n)))
        O[sl] = np.exp(gam)[:, None] * (q @ S) + P @ Vn
        S = np.exp(gam[-1]) * S + (np.exp(gam[-1] - gam)[:, None] * k).T @ Vn
    return O, S


@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunked_form_equals_oracle(oracle_lib, C):
    rng = np.random.default_rng(20 + C)
    T, d = 150, 32
    Q, K, V = rng.standard_normal((3, T, d))
    Q /= np.linalg.norm(Q, axis=1, keepdims=True)
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    g = -0.1 * np.log1p(np.exp(rng.standard_normal(T)))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((d, d)) * 0.05
    o_ref, S_ref = oracle_lib.recurrence(Q, K, V, np.exp(g), beta, S0=S0)
    o, S = chunked_form(Q, K, V, g, beta, S0, C)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, atol=1e-12)


# --------------------------------------------------------------------------
# planted mistakes (in a copy of the oracle's update, on the CPU) are caught
# --------------------------------------------------------------------------
def _planted(Q, K, V, al, be, S0, mistake):
    S = S0.copy()
    outs = []
    for t in range(K.shape[0]):
        k, v, q = K[t], V[t], Q[t]
        if mistake != "alpha_after_predict":
            S = al[t] * S
        p = S.T @ k
        if mistake == "alpha_after_predict":
            S = al[t] * S
        sign = -1.0 if mistake == "sign" else 1.0
        S = S + be[t] * np.outer(k, v - sign * p)
        outs.append((S if mistake != "transposed" else S.T) .T @ q)
    return np.array(outs), S


@pytest.mark.parametrize("mistake", ["sign", "alpha_after_predict", "transposed"])
def test_planted_mistakes_fail_dense_pin(mistake):
    rng = np.random.default_rng(31)
    T, d = 6, 8
    K = rng.standard_normal((T, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    Q, V = rng.standard_normal((2, T, d))
    S0 = rng.standard_normal((d, d))
    al, be = rng.uniform(0.5, 0.9, T), rng.uniform(0.2, 1.0, T)
    o_ref, S_ref = _dense_unrolled(S0, Q, K, V, al, be)
    o_ok, S_ok = _planted(Q, K, V, al, be, S0, "none")
    np.testing.assert_allclose(o_ok, o_ref, atol=1e-12)
    o_bad, S_bad = _planted(Q, K, V, al, be, S0, mistake)
    assert not (np.allclose(o_bad, o_ref, atol=1e-6) and np.allclose(S_bad, S_ref, atol=1e-6))
