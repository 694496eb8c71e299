"""Pins of the oracle's backward (gradients of the whole mixer), on the CPU.

The backward is reverse-mode differentiation of the token recurrence written
out by hand.  Nothing here reuses its formulas: every gradient is checked
against central finite differences of the *forward* oracle (run with all
inputs in float64), along a random direction per input tensor, on small
packed batches that include sequences shorter than the conv window.  A
closed form (no decay, no write: o_t = q_scale S_0^T q_t) pins the state
gradient exactly, and planted mistakes, compiled into a scratch copy of the
oracle, must fail the finite-difference pin.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

from linear_attention_sequence_gdn_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

TENSORS = ("q", "k", "v", "a", "b", "conv_w", "conv_state", "state")


def _problem(seed, lens, Hqk, Hv, d, gate_scale=0.3, q_scale=0.7):
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, N = int(cu[-1]), len(lens)
    C = 2 * Hqk * d + Hv * d
    x = {
        "q": rng.normal(size=(T, Hqk, d)), "k": rng.normal(size=(T, Hqk, d)),
        "v": rng.normal(size=(T, Hv, d)), "a": rng.normal(size=(T, Hv)),
        "b": rng.normal(size=(T, Hv)), "conv_w": rng.normal(0, 0.5, size=(C, 4)),
        "conv_state": rng.normal(size=(N, 3, C)), "state": rng.normal(0, 0.5, size=(N, Hv, d, d)),
    }
    d_o = rng.normal(size=(T, Hv, d))
    d_S = rng.normal(size=(N, Hv, d, d))
    kw = dict(Hqk=Hqk, Hv=Hv, gate_scale=gate_scale, q_scale=q_scale)
    return x, cu, d_o, d_S, kw


def _loss(oracle, x, cu, d_o, d_S, kw):
    o, S = oracle.prefill_f64(x["q"], x["k"], x["v"], x["a"], x["b"], x["conv_w"], cu,
                              state_in=x["state"], conv_state_in=x["conv_state"], **kw)
    return float(np.sum(o * d_o) + np.sum(S * d_S))


def _grads(oracle, x, cu, d_o, d_S, kw):
    return oracle.prefill_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["conv_w"], cu, d_o,
                                   state_in=x["state"], conv_state_in=x["conv_state"],
                                   d_state_out=d_S, f64=True, **kw)


def _fd_check(oracle, grads, x, cu, d_o, d_S, kw, seed, h=1e-5):
    """Directional derivative along a random direction, per input tensor:
    returns {name: (finite difference, <grad, direction>)}."""
    rng = np.random.default_rng(seed)
    res = {}
    for name in TENSORS:
        dirn = rng.normal(size=x[name].shape)
        xp = dict(x); xp[name] = x[name] + h * dirn
        xm = dict(x); xm[name] = x[name] - h * dirn
        fd = (_loss(oracle, xp, cu, d_o, d_S, kw) - _loss(oracle, xm, cu, d_o, d_S, kw)) / (2 * h)
        res[name] = (fd, float(np.sum(grads[name] * dirn)))
    return res


def _assert_close(res, rtol=2e-6):
    for name, (fd, an) in res.items():
        assert abs(fd - an) <= rtol * max(abs(fd), abs(an)) + 1e-8, (name, fd, an)


@pytest.mark.parametrize("case", [
    dict(seed=1, lens=[5, 2, 9], Hqk=1, Hv=2, d=4),
    dict(seed=2, lens=[1, 12], Hqk=2, Hv=4, d=3),
    dict(seed=3, lens=[7, 0, 4], Hqk=2, Hv=2, d=5),
])
def test_backward_matches_finite_differences(oracle_lib, case):
    x, cu, d_o, d_S, kw = _problem(case["seed"], case["lens"], case["Hqk"], case["Hv"], case["d"])
    g = _grads(oracle_lib, x, cu, d_o, d_S, kw)
    _assert_close(_fd_check(oracle_lib, g, x, cu, d_o, d_S, kw, seed=100 + case["seed"]))


def test_backward_without_carries(oracle_lib):
    # no initial state, no conv history, no final-state gradient: the
    # entry points' None paths
    x, cu, d_o, _, kw = _problem(4, [6, 3], 1, 3, 4)
    g = oracle_lib.prefill_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["conv_w"], cu, d_o,
                                    f64=True, **kw)
    rng = np.random.default_rng(7)

    def loss(xx):
        o, _ = oracle_lib.prefill_f64(xx["q"], xx["k"], xx["v"], xx["a"], xx["b"], xx["conv_w"], cu, **kw)
        return float(np.sum(o * d_o))
    for name in ("q", "k", "v", "a", "b", "conv_w"):
        dirn = rng.normal(size=x[name].shape)
        xp = dict(x); xp[name] = x[name] + 1e-5 * dirn
        xm = dict(x); xm[name] = x[name] - 1e-5 * dirn
        fd = (loss(xp) - loss(xm)) / 2e-5
        an = float(np.sum(g[name] * dirn))
        assert abs(fd - an) <= 2e-6 * max(abs(fd), abs(an)) + 1e-8, (name, fd, an)
    # absent conv rows are zero rows: the same gradients, the rows' included
    z = oracle_lib.prefill_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["conv_w"], cu, d_o,
                                    conv_state_in=np.zeros_like(x["conv_state"]), f64=True, **kw)
    for name in TENSORS:
        assert np.array_equal(g[name], z[name]), name


def test_state_gradient_closed_form(oracle_lib):
    # gate_scale = 0 gives alpha = 1, and b = -40 gives beta ~ 4e-18: the state
    # never changes, o_t = q_scale S_0^T q^_t, so dL/dS_0 = q_scale sum_t q^_t dO_t^T + dS_T
    x, cu, d_o, d_S, kw = _problem(5, [11], 1, 2, 4, gate_scale=0.0, q_scale=0.6)
    x["b"][:] = -40.0
    g = _grads(oracle_lib, x, cu, d_o, d_S, kw)
    # q^ from the same definition, written out here: conv (with history), SiLU, L2 norm
    T, d = x["q"].shape[0], x["q"].shape[2]
    xq = np.concatenate([x["conv_state"][0, :, :d], x["q"][:, 0, :]], 0)
    y = sum(x["conv_w"][:d, j][None, :] * xq[j:j + T] for j in range(4))
    z = y / (1 + np.exp(-y))
    qh = z / np.sqrt(np.sum(z * z, 1, keepdims=True) + 1e-6)
    for h in range(2):
        want = 0.6 * qh.T @ d_o[:, h, :] + d_S[0, h]
        assert np.allclose(g["state"][0, h], want, rtol=1e-12, atol=1e-12)


def test_bf16_inputs_equal_f64_inputs(oracle_lib):
    # the input-kind switch only converts: bf16 / fp32 inputs give the same
    # gradients as the same values passed as float64
    inp = inputs.make_prefill(T_list=[40, 3], Hqk=1, Hv=2, seed=9, state_std=0.05,
                              conv_state_std=1.0, d=8, threads=1)
    q, k, v, a, b, cu = inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["cu_seqlens"]
    Tt, d = inp["T_tot"], inp["d"]
    rng = np.random.default_rng(3)
    d_o = rng.normal(size=(Tt, 2, d))
    kw = dict(Hqk=1, Hv=2, gate_scale=0.1)
    S0 = inp["state_in"].astype(np.float64)
    g16 = oracle_lib.prefill_backward(q, k, v, a, b, inp["conv_w"], cu, d_o, state_in=S0,
                                      conv_state_in=inp["conv_state_in"], **kw)
    f = lambda u: inputs.bf16_to_f32(u).astype(np.float64)
    g64 = oracle_lib.prefill_backward(f(q), f(k), f(v), a.astype(np.float64), b.astype(np.float64),
                                      f(inp["conv_w"]), cu, d_o, state_in=S0,
                                      conv_state_in=f(inp["conv_state_in"]), f64=True, **kw)
    for n in TENSORS:
        assert np.array_equal(g16[n], g64[n]), n


# ---- planted mistakes, in a scratch copy of the oracle compiled on the CPU

MISTAKES = {
    # the decay is not applied to the carried state gradient
    "no_decay_in_carry": ("G[(long)i * dv + j] = alpha[t] * dsd;", "G[(long)i * dv + j] = dsd;"),
    # the prediction's contribution to dk has the wrong sign
    "pred_sign": ("dkh[(long)t * dk + i] += beta[t] * gu - sdu;", "dkh[(long)t * dk + i] += beta[t] * gu + sdu;"),
    # q_scale dropped from dq
    "no_q_scale": ("dqh[(long)t * dk + i] += q_scale * acc;", "dqh[(long)t * dk + i] += acc;"),
    # the conv's weight gradient reads the wrong tap
    "conv_tap": ("gw[(long)c * 4 + j] += d * xv;", "gw[(long)c * 4 + (3 - j)] += d * xv;"),
}


@pytest.mark.parametrize("mistake", sorted(MISTAKES))
def test_planted_mistakes_fail_finite_differences(oracle_lib, mistake):
    src = open(os.path.join(ROOT, "oracle", "gdn_oracle.c")).read()
    a, b = MISTAKES[mistake]
    assert src.count(a) == 1
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "bad.c")
        so = os.path.join(tmp, "bad.so")
        open(c, "w").write(src.replace(a, b))
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-std=c99", "-o", so, c, "-lm"])
        bad = ctypes.CDLL(so)
        import oracle as good
        ref = good._load().gdn_ref_prefill_backward
        bad.gdn_ref_prefill_backward.restype = ref.restype
        bad.gdn_ref_prefill_backward.argtypes = ref.argtypes
        x, cu, d_o, d_S, kw = _problem(1, [5, 2, 9], 1, 2, 4)
        saved = good._lib
        try:
            # gradients from the planted copy, losses from the true forward
            good._lib = _Proxy(saved, bad)
            g = _grads(good, x, cu, d_o, d_S, kw)
        finally:
            good._lib = saved
        res = _fd_check(good, g, x, cu, d_o, d_S, kw, seed=101)
        with pytest.raises(AssertionError):
            _assert_close(res)


class _Proxy:
    """The true oracle library, except for the backward entry point."""

    def __init__(self, good, bad):
        self._good, self._bad = good, bad

    def __getattr__(self, name):
        if name == "gdn_ref_prefill_backward":
            return getattr(self._bad, name)
        return getattr(self._good, name)
