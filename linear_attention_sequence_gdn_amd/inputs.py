"""Seeded synthetic inputs for the Gated DeltaNet token mixer.

This module only draws random numbers and lays them out; it holds none of the
mixer's arithmetic.  Both the HIP path (through the binding) and the fp64 CPU
oracle consume the arrays it returns, so the two sides always see bit-identical
inputs.

Conventions
-----------
* bf16 tensors are returned as ``uint16`` arrays holding the bf16 bit pattern,
  produced from fp32 draws with round-to-nearest-even.
* Every (tensor, head) slice is drawn from its own PCG64 stream seeded with
  ``[seed, tensor_id, head]`` so that any subset of heads can be regenerated
  on its own and slices can be drawn in parallel threads.
* ``N(0, s)`` means standard deviation ``s``.

Layouts (row-major, innermost last)
-----------------------------------
* q, k: ``[T_tot][H_qk][d]``; v: ``[T_tot][H_v][d]`` (packed over sequences)
* a, b: ``[T_tot][H_v]`` fp32 raw gate pre-activations (a -> forget gate,
  b -> write strength)
* conv_w: ``[C_tot][4]`` bf16, channel order q | k | v, tap 3 multiplies the
  current token
* state: ``[N][H_v][d_k][d_v]`` fp32
* conv_state: ``[N][3][C_tot]`` bf16, oldest row first
* cu_seqlens: ``[N+1]`` int32
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids for the per-(tensor, head) streams
_TID = {"q": 1, "k": 2, "v": 3, "wq": 4, "wk": 5, "wv": 6, "b": 7, "a": 8,
        "state": 9, "conv_state": 10, "lengths": 11}

D = 128

# The five synthetic workloads.  Shapes and distributions follow the
# configuration list the mixer is graded on; sizes are in tokens.
CONFIGS = {
    0: dict(name="tiny_prefill_T512_2qk_6v", kind="prefill", B=1, T=512,
            Hqk=2, Hv=6, gate_scale=0.1, state_std=0.0),
    1: dict(name="layer_prefill_T8192_16qk_48v", kind="prefill", B=1, T=8192,
            Hqk=16, Hv=48, gate_scale=0.1, state_std=0.0),
    2: dict(name="native_ctx_prefill_T262144_16qk_48v", kind="prefill", B=1,
            T=262144, Hqk=16, Hv=48, gate_scale=0.02, state_std=0.0,
            oracle_heads=(0, 23, 47)),
    3: dict(name="decode_B256_x64steps_16qk_48v", kind="decode", B=256,
            steps=64, Hqk=16, Hv=48, gate_scale=0.1, state_std=0.05),
    4: dict(name="varlen_prefill_N64_logU128_32768_16qk_48v", kind="varlen",
            N=64, Lmin=128, Lmax=32768, Hqk=16, Hv=48, gate_scale=0.1,
            state_std=0.05),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> fp32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tensor: str, head: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), _TID[tensor], int(head)])


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_heads(out: np.ndarray, seed: int, tensor: str, heads, std: float,
                bf16: bool, pool: ThreadPoolExecutor) -> None:
    """out[..., h, :] (or out[:, h] for 2-D) <- N(0, std) from stream (tensor, h)."""
    def one(h):
        shape = out.shape[:-2] + out.shape[-1:] if out.ndim >= 3 else out.shape[:-1]
        x = _rng(seed, tensor, h).standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        if out.ndim >= 3:
            out[..., h, :] = bf16_bits(x) if bf16 else x
        else:
            out[:, h] = bf16_bits(x) if bf16 else x
    list(pool.map(one, heads))


def varlen_lengths(seed: int, n: int, lmin: int, lmax: int) -> np.ndarray:
    """Sequence lengths log-uniform in [lmin, lmax], rounded to integers."""
    r = _rng(seed, "lengths", 0)
    u = r.uniform(np.log(lmin), np.log(lmax), size=n)
    return np.clip(np.rint(np.exp(u)), lmin, lmax).astype(np.int64)


def make_prefill(*, T_list, Hqk, Hv, seed, gate_scale=0.1, state_std=0.0,
                 conv_state_std=None, d=D, heads=None, qk_heads=None,
                 threads=None):
    """Packed prefill inputs for sequences of lengths ``T_list``.

    ``heads`` / ``qk_heads`` restrict which V / QK head slices are drawn (the
    others stay zero), which lets a checker regenerate a subset of a very
    large workload bit-identically.
    """
    T_list = [int(t) for t in T_list]
    N = len(T_list)
    T_tot = int(sum(T_list))
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(T_list)
    heads = list(range(Hv)) if heads is None else list(heads)
    qk_heads = list(range(Hqk)) if qk_heads is None else list(qk_heads)
    C_tot = 2 * Hqk * d + Hv * d
    nthr = threads or _threads()
    with ThreadPoolExecutor(nthr) as pool:
        q = np.zeros((T_tot, Hqk, d), np.uint16)
        k = np.zeros((T_tot, Hqk, d), np.uint16)
        v = np.zeros((T_tot, Hv, d), np.uint16)
        _fill_heads(q, seed, "q", qk_heads, 1.0, True, pool)
        _fill_heads(k, seed, "k", qk_heads, 1.0, True, pool)
        _fill_heads(v, seed, "v", heads, 1.0, True, pool)
        w = np.zeros((C_tot, 4), np.uint16)
        wq = w[: Hqk * d].reshape(Hqk, d, 4)
        wk = w[Hqk * d: 2 * Hqk * d].reshape(Hqk, d, 4)
        wv = w[2 * Hqk * d:].reshape(Hv, d, 4)
        for g in range(Hqk):
            wq[g] = bf16_bits(_rng(seed, "wq", g).standard_normal((d, 4), dtype=np.float32) * np.float32(0.25))
            wk[g] = bf16_bits(_rng(seed, "wk", g).standard_normal((d, 4), dtype=np.float32) * np.float32(0.25))
        for h in range(Hv):
            wv[h] = bf16_bits(_rng(seed, "wv", h).standard_normal((d, 4), dtype=np.float32) * np.float32(0.25))
        b = np.zeros((T_tot, Hv), np.float32)
        a = np.zeros((T_tot, Hv), np.float32)
        _fill_heads(b, seed, "b", heads, 1.0, False, pool)
        _fill_heads(a, seed, "a", heads, 1.0, False, pool)
        state = None
        if state_std:
            state = np.zeros((N, Hv, d, d), np.float32)

            def st(h):
                x = _rng(seed, "state", h).standard_normal((N, d, d), dtype=np.float32)
                state[:, h] = x * np.float32(state_std)
            list(pool.map(st, heads))
        conv_state = None
        if conv_state_std:
            x = _rng(seed, "conv_state", 0).standard_normal((N, 3, C_tot), dtype=np.float32)
            conv_state = bf16_bits(x * np.float32(conv_state_std))
    return dict(q=q, k=k, v=v, a=a, b=b, conv_w=w, state_in=state,
                conv_state_in=conv_state, cu_seqlens=cu, T_list=T_list,
                N=N, T_tot=T_tot, Hqk=Hqk, Hv=Hv, d=d,
                gate_scale=float(gate_scale), q_scale=1.0)


def make_decode(*, B, steps, Hqk, Hv, seed, gate_scale=0.1, state_std=0.05,
                d=D, threads=None):
    """Inputs of ``steps`` consecutive single-token decode steps for B sequences."""
    C_tot = 2 * Hqk * d + Hv * d
    nthr = threads or _threads()
    with ThreadPoolExecutor(nthr) as pool:
        q = np.zeros((steps, B, Hqk, d), np.uint16)
        k = np.zeros((steps, B, Hqk, d), np.uint16)
        v = np.zeros((steps, B, Hv, d), np.uint16)
        _fill_heads(q, seed, "q", range(Hqk), 1.0, True, pool)
        _fill_heads(k, seed, "k", range(Hqk), 1.0, True, pool)
        _fill_heads(v, seed, "v", range(Hv), 1.0, True, pool)
        b = np.zeros((steps * B, Hv), np.float32)
        a = np.zeros((steps * B, Hv), np.float32)
        _fill_heads(b, seed, "b", range(Hv), 1.0, False, pool)
        _fill_heads(a, seed, "a", range(Hv), 1.0, False, pool)
        w = np.zeros((C_tot, 4), np.uint16)
        for g in range(Hqk):
            w[g * d:(g + 1) * d] = bf16_bits(_rng(seed, "wq", g).standard_normal((d, 4), dtype=np.float32) * np.float32(0.25))
            w[(Hqk + g) * d:(Hqk + g + 1) * d] = bf16_bits(_rng(seed, "wk", g).standard_normal((d, 4), dtype=np.float32) * np.float32(0.25))
        for h in range(Hv):
            o = 2 * Hqk * d + h * d
            w[o:o + d] = bf16_bits(_rng(seed, "wv", h).standard_normal((d, 4), dtype=np.float32) * np.float32(0.25))
        state = np.zeros((B, Hv, d, d), np.float32)

        def st(h):
            x = _rng(seed, "state", h).standard_normal((B, d, d), dtype=np.float32)
            state[:, h] = x * np.float32(state_std)
        list(pool.map(st, range(Hv)))
        x = _rng(seed, "conv_state", 0).standard_normal((B, 3, C_tot), dtype=np.float32)
        conv_state = bf16_bits(x)
    return dict(q=q, k=k, v=v, a=a.reshape(steps, B, Hv), b=b.reshape(steps, B, Hv),
                conv_w=w, state=state, conv_state=conv_state, B=B, steps=steps,
                Hqk=Hqk, Hv=Hv, d=d, gate_scale=float(gate_scale), q_scale=1.0)


def make_config(idx: int, seed: int | None = None, *, heads=None, qk_heads=None,
                T_override=None, N_override=None):
    """Inputs of one of the five synthetic workloads (seed = 1000 + idx)."""
    c = CONFIGS[idx]
    seed = 1000 + idx if seed is None else seed
    if c["kind"] == "prefill":
        T = T_override or c["T"]
        return make_prefill(T_list=[T] * c["B"], Hqk=c["Hqk"], Hv=c["Hv"], seed=seed,
                            gate_scale=c["gate_scale"], state_std=c["state_std"],
                            heads=heads, qk_heads=qk_heads)
    if c["kind"] == "decode":
        return make_decode(B=N_override or c["B"], steps=c["steps"], Hqk=c["Hqk"],
                           Hv=c["Hv"], seed=seed, gate_scale=c["gate_scale"],
                           state_std=c["state_std"])
    lengths = varlen_lengths(seed, c["N"], c["Lmin"], c["Lmax"])
    if N_override:
        lengths = lengths[:N_override]
    return make_prefill(T_list=lengths, Hqk=c["Hqk"], Hv=c["Hv"], seed=seed,
                        gate_scale=c["gate_scale"], state_std=c["state_std"],
                        heads=heads, qk_heads=qk_heads)
