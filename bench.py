#!/usr/bin/env python3
"""GDN token mixer benchmark on one MI355X.

A step is one chunked prefill of the model-layer workload (B = 1, T = 8192,
16 QK / 48 V heads, d = 128, seeded synthetic bf16 inputs already resident in
HBM).  The decode workload (B = 256 sequences, 64 consecutive in-place steps)
is timed in the same run and reported under "decode", and the training
backward of the prefill workload under "backward".  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--calibrate-copy]
  python bench.py --traffic-report FETCH_CSV WRITE_CSV

--calibrate-copy ends the run with a plain 256 MiB device-to-device copy, so
that a rocprofv3 --pmc pass over this command also reads its counters for a
transfer of known size.  --traffic-report turns two such passes (FETCH_SIZE,
then WRITE_SIZE; rocprofv3's counter_collection.csv files) into HBM bytes per
launch of each kernel, scaled by what the counters read for the copy, and
writes them to profiles/traffic.json tagged with the digest of the kernel
sources they were taken on.

Timing: HIP events on the stream the library launches on.  The step time is
K plain gdn_prefill calls between two events; the same K steps are then run
through gdn_prefill_with_events, which records an event after each of its
kernels (chunk-table setup, parallel pass, sequential pass), for the
per-kernel times the roofline uses.  Each recorded event costs the stream a
few microseconds; the interval before the first kernel, empty for a uniform
batch, measures that cost, and it is subtracted from the kernels' intervals
(the raw intervals are reported too).  The default 200 warm-up steps (about
70 ms of GPU work) let the clocks settle: after 30 the prefill still runs
about 10 % slower.  The 64 decode steps run back to back between two
events.  The CPU baseline is the fp64 oracle, as it stands, on a bounded
sample of the same prefill workload.
"""
import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s (T=8192, 16QK/48V heads, d=128); decode μs/step at B=256"
PEAK_MFMA_F16 = 2.5e15      # dense fp16/bf16 matrix-core FLOP/s
PEAK_HBM = 8.0e12           # bytes/s
PEAK_VALU_F32 = 157.3e12    # fp32 vector FLOP/s (the published figure counts packed fp32)
D = 128
CHUNK = 64


# ---------------------------------------------------------------------------
# algorithmic work (chunk form, C = 64, counted per full chunk)
# ---------------------------------------------------------------------------
# gdn_prefill_with_events records an event before the first kernel and after
# each of these, in launch order
PREFILL_KERNELS = ("setup_kernel", "prep_kernel", "chain_kernel")
N_EVENTS = len(PREFILL_KERNELS) + 1


def prefill_flops(T, Hqk, Hv, n=CHUNK, d=D):
    """(prep, chain) algorithmic FLOP of one prefill of T tokens (T % 64 == 0).

    prep: K K^T and K Q^T per QK head (2 x 2 n^2 d), the triangular inverse
    per V head (n^3 / 3); chain, per V head: K S, Q S and the state update
    (3 x 2 n d^2), T' times the bracket and P Vnew (2 x 2 n^2 d)."""
    chunks = T // n
    prep = chunks * (Hqk * 4 * n * n * d + Hv * n ** 3 / 3)
    chain = chunks * Hv * (6 * n * d * d + 4 * n * n * d)
    return prep, chain


def prefill_bytes(T, Hqk, Hv, d=D):
    """Compulsory HBM bytes of one prefill (zero initial state, no conv carry)."""
    per_tok = 2 * (2 * Hqk * d + Hv * d) + 2 * 4 * Hv + 2 * Hv * d
    return T * per_tok + Hv * d * d * 4 + (2 * Hqk * d + Hv * d) * 4 * 2


def backward_flops(T, Hqk, Hv, n=CHUNK, d=D):
    """Algorithmic FLOP of the training backward per sequence of T tokens,
    counted per full chunk and V head (2 per multiply-add; triangular n x n
    factors at half):

      recomputed forward   K S, Ks^T Vn: 4 n d^2;          T' Vt: n^2 d
      state-gradient pass  Ks dS', (Gam Q)^T dO', (Gam K)^T dVt: 6 n d^2;
                           P^T dO', T'^T dVn: 2 n^2 d
      chunk-local          K K^T, Q K^T: 2 n^2 d;   (I + A)^-1: n^3 / 3
      per-chunk gradients  Vn dS'^T, dO' S^T, dVt S^T: 6 n d^2;
                           dO' Vn^T, dVn Vt^T: 2 n^2 d (full); dQK K, dQK^T Q,
                           K K^T, (dKK + dKK^T) K: 5 n^2 d; X^T dX X^T: 2 n^3 / 3
    """
    per = 16 * n * d * d + 12 * n * n * d + n ** 3
    return per * (T // n) * Hv


def decode_bytes(B, Hqk, Hv, d=D, T=1):
    """Compulsory HBM bytes of one decode call of T tokens per sequence: the
    fp32 state read and written once, per token the q/k/v rows, o and the
    gates, and the conv rows read and written once."""
    C_tot = 2 * Hqk * d + Hv * d
    state = 2 * B * Hv * d * d * 4
    per_tok = 2 * (2 * Hqk * d + Hv * d) + 2 * Hv * d + 2 * 4 * Hv
    return state + B * (T * per_tok + 2 * 3 * C_tot * 2)


# ---------------------------------------------------------------------------
# HIP events through the runtime torch already loaded
# ---------------------------------------------------------------------------
class Hip:
    def __init__(self):
        import torch
        cands = glob.glob(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so*"))
        self.L = ctypes.CDLL(cands[0] if cands else "libamdhip64.so")
        self.L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.L.hipEventCreate(ctypes.byref(e))
        assert rc == 0, f"hipEventCreate failed ({rc})"
        return e

    def record(self, e, stream):
        assert self.L.hipEventRecord(e, stream) == 0

    def ms(self, a, b):
        self.L.hipEventSynchronize(b)
        out = ctypes.c_float()
        assert self.L.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return float(out.value)


# kernel sources behind each group of measured kernels
FWD_SOURCES = ("gdn_common.h", "gdn_prefill.h", "gdn_prefill.hip", "gdn_decode.hip")
BWD_SOURCES = ("gdn_common.h", "gdn_backward.hip")


def source_digest(files=FWD_SOURCES):
    h = hashlib.sha256()
    for f in sorted(files):
        h.update(open(os.path.join(ROOT, "linear_attention_sequence_gdn_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


COPY_BYTES = 256 << 20
TRAFFIC_KERNELS = {"prefill_chain": "chain_kernel", "prefill_prep": "prep_kernel",
                   "prefill_setup": "setup_kernel", "decode": "decode_step_kernel",
                   "decode_conv_shift": "conv_shift_qk_kernel<1>",
                   "decode_multi": "decode_head_kernel<4>", "decode_multi_conv_shift": "conv_shift_qk_kernel<4>"}
BWD_KERNELS = ("bwd_prep_kernel", "bwd_local_kernel", "bwd_fwd_kernel", "bwd_chain_kernel", "bwd_grad_kernel",
               "bwd_dy_kernel", "bwd_conv_kernel", "bwd_dw_kernel")
TRAFFIC_KERNELS.update({"backward_" + k_[4:-7]: k_ for k_ in BWD_KERNELS})


def _counter_rows(path, counter):
    """(dispatch id, value) rows of `counter` by kernel name, from a rocprofv3
    counter_collection.csv."""
    import csv
    acc = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            acc.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return acc


def traffic_report(fetch_csv, write_csv):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) -> calibrated bytes per launch.
    The calibration copy is the run's last device-to-device copy dispatch."""
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")

    def named(k_, sub):  # the kernel itself, not one whose name contains it
        return ("::" + sub + "(") in k_ or k_.startswith(sub + "(")

    def rows(table, sub):
        hits = [v_ for k_, v_ in table.items() if named(k_, sub)]
        if len(hits) != 1:
            raise SystemExit(f"traffic report: {len(hits)} kernels match {sub!r}")
        return hits[0]

    def mean(table, sub):
        r = rows(table, sub)
        return sum(v_ for _, v_ in r) / len(r)

    def copy_rows(table):
        hits = [v_ for k_, v_ in table.items() if "copyBuffer" in k_]
        if len(hits) != 1:
            raise SystemExit(f"traffic report: {len(hits)} copy kernels")
        return hits[0]

    f_copy = max(copy_rows(fetch))[1] * 1024
    w_copy = max(copy_rows(write))[1] * 1024
    f_scale, w_scale = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    digest, bwd_digest = source_digest(), source_digest(BWD_SOURCES)
    out = {"_calibration": {"copy_bytes": COPY_BYTES, "fetch_counter_bytes": f_copy,
                            "write_counter_bytes": w_copy, "fetch_scale": f_scale,
                            "write_scale": w_scale}}
    for name, sub in TRAFFIC_KERNELS.items():
        if not any(named(k_, sub) for k_ in fetch):
            print(f"{sub:22s} not launched in this run")
            continue
        rd = mean(fetch, sub) * 1024 * f_scale
        wr = mean(write, sub) * 1024 * w_scale
        out[name] = {"kernel": sub, "read_bytes": rd, "write_bytes": wr, "bytes_per_launch": rd + wr,
                     "source_digest": bwd_digest if name.startswith("backward") else digest}
        print(f"{sub:22s} read {rd / 2**20:10.2f} MiB  write {wr / 2**20:10.2f} MiB per launch")
    print(f"copy calibration: FETCH_SIZE x{f_scale:.3f}, WRITE_SIZE x{w_scale:.3f}")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print("wrote", path)


def _sum_or_none(*xs):
    return None if any(x_ is None for x_ in xs) else sum(xs)


def load_traffic(name, digest):
    """HBM traffic measured by rocprofv3 counters for `name`, if the committed
    measurement was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(name)
    except (ValueError, AttributeError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
def bench_prefill(hip, steps, warmup):
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    from linear_attention_sequence_gdn_amd import inputs

    x = inputs.make_config(1)
    T, Hqk, Hv = 8192, 16, 48

    def dev(a, bf):
        import numpy as np
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if bf else np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf else t).cuda()

    q = dev(x["q"].reshape(1, T, Hqk, D), True)
    k = dev(x["k"].reshape(1, T, Hqk, D), True)
    v = dev(x["v"].reshape(1, T, Hv, D), True)
    a = dev(x["a"].reshape(1, T, Hv), False)
    b = dev(x["b"].reshape(1, T, Hv), False)
    w = dev(x["conv_w"], True)
    o = torch.empty((1, T, Hv, D), dtype=torch.bfloat16, device="cuda")
    so = torch.empty((1, Hv, D, D), dtype=torch.float32, device="cuda")
    need = gdn.gdn_prefill_workspace_size(1, T, Hqk, Hv)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    L = gdn.lib()
    L.gdn_prefill.restype = ctypes.c_int
    L.gdn_prefill.argtypes = [ctypes.c_void_p] * 11 + [ctypes.c_int] * 6 + \
        [ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.gdn_prefill_with_events.restype = ctypes.c_int
    L.gdn_prefill_with_events.argtypes = [ctypes.c_void_p] * 11 + [ctypes.c_int] * 6 + \
        [ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    evs = [[hip.event() for _ in range(N_EVENTS)] for _ in range(steps)]
    arrs = [(ctypes.c_void_p * N_EVENTS)(*[e.value for e in ev]) for ev in evs]
    warm = (ctypes.c_void_p * N_EVENTS)(*[hip.event().value for _ in range(N_EVENTS)])

    def run(arr=None):
        if arr is None:
            rc = L.gdn_prefill(P(q), P(k), P(v), P(a), P(b), P(w), None, None, None, P(so), P(o),
                               1, T, Hqk, Hv, D, D, 0.1, 1.0, P(ws), need, sp)
        else:
            rc = L.gdn_prefill_with_events(P(q), P(k), P(v), P(a), P(b), P(w), None, None, None, P(so), P(o),
                                           1, T, Hqk, Hv, D, D, 0.1, 1.0, P(ws), need, sp, arr)
        assert rc == 0, gdn.gdn_status_string(rc)

    for _ in range(warmup):
        run()
        run(warm)
    torch.cuda.synchronize()
    # the step time: plain calls, nothing recorded between the kernels
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, sp)
    for i in range(steps):
        run()
    hip.record(t1, sp)
    torch.cuda.synchronize()
    total_ms = hip.ms(t0, t1)
    # per-kernel times: the same steps again with an event after every kernel
    # (each recorded event costs the stream a few microseconds, which these
    # intervals include)
    for i in range(steps):
        run(arrs[i])
    torch.cuda.synchronize()
    stage = {name: 0.0 for name in PREFILL_KERNELS}
    for ev in evs:
        for i, name in enumerate(PREFILL_KERNELS):
            stage[name] += hip.ms(ev[i], ev[i + 1])
    stage = {k_: v_ / steps for k_, v_ in stage.items()}
    return dict(ms_per_step=total_ms / steps, stage_ms=stage, T=T, Hqk=Hqk, Hv=Hv)


def bench_decode(hip, steps=64):
    import numpy as np
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    from linear_attention_sequence_gdn_amd import inputs

    x = inputs.make_config(3)
    B, Hqk, Hv = x["B"], x["Hqk"], x["Hv"]

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = bf(x["q"]), bf(x["k"]), bf(x["v"])
    a = torch.from_numpy(x["a"]).cuda()
    b = torch.from_numpy(x["b"]).cuda()
    w = bf(x["conv_w"])
    conv0 = bf(x["conv_state"])
    st0 = torch.from_numpy(x["state"]).cuda()
    conv, st = conv0.clone(), st0.clone()
    o = torch.empty((B, Hv, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    L = gdn.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def step(i):
        rc = L.gdn_decode_step(P(q[i]), P(k[i]), P(v[i]), P(a[i]), P(b[i]), P(w), P(conv), P(st), P(st),
                               P(o), B, Hqk, Hv, D, D, 0.1, 1.0, sp)
        assert rc == 0, gdn.gdn_status_string(rc)

    for i in range(16):  # warm-up, then restore the initial state
        step(i)
    torch.cuda.synchronize()
    conv.copy_(conv0)
    st.copy_(st0)
    torch.cuda.synchronize()
    # the steps back to back between two events (an event between steps would
    # add its own cost to every step)
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, sp)
    for i in range(steps):
        step(i)
    hip.record(t1, sp)
    torch.cuda.synchronize()
    return dict(us_per_step=hip.ms(t0, t1) * 1e3 / steps, B=B, Hqk=Hqk, Hv=Hv, steps=steps)


def bench_decode_multi(hip, T=4, steps=32):
    """B = 256 sequences, T tokens each per call (multi-token decode): the
    state is read and written once per call, so the per-token cost falls."""
    import numpy as np
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    from linear_attention_sequence_gdn_amd import inputs

    c = inputs.CONFIGS[3]
    B, Hqk, Hv = c["B"], c["Hqk"], c["Hv"]
    x = inputs.make_decode(B=B, steps=T, Hqk=Hqk, Hv=Hv, seed=1003, gate_scale=c["gate_scale"])

    def dev(arr, bf):
        t = torch.from_numpy(np.ascontiguousarray(np.swapaxes(arr, 0, 1)))
        return (t.view(torch.int16).view(torch.bfloat16) if bf else t).cuda()

    q, k, v = dev(x["q"].view(np.int16), True), dev(x["k"].view(np.int16), True), dev(x["v"].view(np.int16), True)
    a, b = dev(x["a"], False), dev(x["b"], False)
    w = torch.from_numpy(x["conv_w"].view(np.int16)).view(torch.bfloat16).cuda()
    conv = torch.from_numpy(x["conv_state"].view(np.int16)).view(torch.bfloat16).cuda()
    st = torch.from_numpy(x["state"]).cuda()
    o = torch.empty((B, T, Hv, D), dtype=torch.bfloat16, device="cuda")
    for _ in range(4):
        gdn.gdn_decode_multi(q, k, v, a, b, w, conv, st, o=o, gate_scale=c["gate_scale"])
    torch.cuda.synchronize()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, sp)
    for _ in range(steps):
        gdn.gdn_decode_multi(q, k, v, a, b, w, conv, st, o=o, gate_scale=c["gate_scale"])
    hip.record(t1, sp)
    torch.cuda.synchronize()
    us = hip.ms(t0, t1) * 1e3 / steps
    nbytes = decode_bytes(B, Hqk, Hv, T=T)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"metric": f"multi-token decode (B=256, T={T} tokens per sequence per call, 16QK/48V)",
            "us_per_call": us, "us_per_token_step": us / T, "tokens_per_s": B * T / (us * 1e-6),
            "roofline": {"bound": "hbm", "kernel": "decode_head_kernel<4> + conv_shift_qk_kernel<4>",
                         "achieved": gbs, "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": gbs * 1e9 / PEAK_HBM,
                         "traffic": _sum_or_none(load_traffic("decode_multi", source_digest()),
                                                 load_traffic("decode_multi_conv_shift", source_digest())),
                         "algorithmic_bytes_per_launch": nbytes}}


def bench_backward(hip, steps=10, warmup=3):
    """gdn_prefill_backward on the prefill workload (same seeded inputs, a
    seeded bf16 output gradient and final-state gradient), K calls between
    two events."""
    import numpy as np
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    from linear_attention_sequence_gdn_amd import inputs

    c = inputs.CONFIGS[1]
    B, T, Hqk, Hv = c["B"], c["T"], c["Hqk"], c["Hv"]
    x = inputs.make_prefill(T_list=[T], Hqk=Hqk, Hv=Hv, seed=1001, gate_scale=c["gate_scale"])
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    rng = np.random.default_rng(2001)
    g_o = bf(inputs.bf16_bits(rng.standard_normal((B, T, Hv, D), dtype=np.float32)))
    g_S = f32(rng.standard_normal((B, Hv, D, D), dtype=np.float32))
    args = (bf(x["q"].reshape(B, T, Hqk, D)), bf(x["k"].reshape(B, T, Hqk, D)), bf(x["v"].reshape(B, T, Hv, D)),
            f32(x["a"].reshape(B, T, Hv)), f32(x["b"].reshape(B, T, Hv)), bf(x["conv_w"]), g_o)
    ws = torch.empty(gdn.gdn_prefill_backward_workspace_size(B, T, Hqk, Hv), dtype=torch.uint8, device="cuda")
    run = lambda: gdn.gdn_prefill_backward(*args, gate_scale=c["gate_scale"], grad_state_out=g_S, workspace=ws)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, sp)
    for _ in range(steps):
        run()
    hip.record(t1, sp)
    torch.cuda.synchronize()
    ms = hip.ms(t0, t1) / steps
    flop = backward_flops(T, Hqk, Hv)
    tf = flop / (ms * 1e-3) / 1e12
    return {"metric": "training backward tokens/s (B=1, T=8192, 16QK/48V; all gradients, fp32)",
            "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_call": ms, "steps": steps,
            "roofline": {"bound": "alu", "kernel": "whole backward (eight launches)", "achieved": tf,
                         "peak": PEAK_VALU_F32 / 1e12, "unit": "TFLOP/s", "frac": tf * 1e12 / PEAK_VALU_F32,
                         "traffic": None, "algorithmic_flop_per_call": flop}}


def cpu_baseline(min_seconds=12.0, max_reps=60):
    import oracle
    from linear_attention_sequence_gdn_amd import inputs
    x = inputs.make_config(1)
    oracle.build(force=False)
    reps, t0 = 0, time.perf_counter()
    while reps < max_reps:
        oracle.prefill(x["q"], x["k"], x["v"], x["a"], x["b"], x["conv_w"], x["cu_seqlens"],
                       Hqk=16, Hv=48, gate_scale=0.1)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": 8192 * reps / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"fp64 token-by-token oracle on the full T=8192, 16QK/48V workload, "
                      f"{reps} run(s) in {dt:.1f} s wall"}


def cpu_baseline_backward(T_sample=1024, min_seconds=4.0, max_reps=20):
    """The oracle's backward (fp64, token by token) on the first T_sample
    tokens of the backward workload, all heads; its cost per token does not
    depend on T, so tokens/s carries over to the whole sequence."""
    import numpy as np
    import oracle
    from linear_attention_sequence_gdn_amd import inputs
    c = inputs.CONFIGS[1]
    Hqk, Hv = c["Hqk"], c["Hv"]
    x = inputs.make_prefill(T_list=[T_sample], Hqk=Hqk, Hv=Hv, seed=1001, gate_scale=c["gate_scale"])
    rng = np.random.default_rng(2001)
    g_o = rng.standard_normal((T_sample, Hv, D))
    oracle.build(force=False)
    reps, t0 = 0, time.perf_counter()
    while reps < max_reps:
        oracle.prefill_backward(x["q"], x["k"], x["v"], x["a"], x["b"], x["conv_w"], x["cu_seqlens"], g_o,
                                Hqk=Hqk, Hv=Hv, gate_scale=c["gate_scale"])
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": T_sample * reps / dt, "unit": "tokens/s", "cores": min(oracle.num_threads(), Hqk),
            "kind": "oracle",
            "sample": f"fp64 token-by-token oracle backward on the first {T_sample} tokens of the workload, "
                      f"16QK/48V, parallel over the 16 QK groups; {reps} run(s) in {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--traffic-report", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    args = ap.parse_args()
    if args.traffic_report:
        traffic_report(*args.traffic_report)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    gdn.lib()
    hip = Hip()
    digest = source_digest()

    pf = bench_prefill(hip, args.steps, args.warmup)
    dc = bench_decode(hip)
    dm = bench_decode_multi(hip)
    bw = bench_backward(hip)
    bw["roofline"]["traffic"] = _sum_or_none(*(load_traffic("backward_" + k_[4:-7], source_digest(BWD_SOURCES))
                                               for k_ in BWD_KERNELS))
    T, Hqk, Hv = pf["T"], pf["Hqk"], pf["Hv"]
    flop_prep, flop_chain = prefill_flops(T, Hqk, Hv)
    tok_s = T / (pf["ms_per_step"] * 1e-3)

    # dominant prefill kernel (the longer of the two that carry the matrix
    # products), priced against the fp16 dense matrix-core peak
    # Each recorded event costs the stream about as much as the interval
    # before the first kernel, which is empty here (a uniform batch launches
    # no setup kernel); it is subtracted from the kernels' intervals.
    raw = pf["stage_ms"]
    event_ms = raw["setup_kernel"]
    km = {k_: max(v_ - event_ms, 0.0) for k_, v_ in raw.items() if k_ != "setup_kernel"}
    dom = "chain_kernel" if km["chain_kernel"] >= km["prep_kernel"] else "prep_kernel"
    dom_flop = flop_chain if dom == "chain_kernel" else flop_prep
    dom_ms = km[dom]
    achieved = dom_flop / (dom_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": dom, "achieved": achieved,
            "peak": PEAK_MFMA_F16 / 1e12, "unit": "TFLOP/s", "frac": achieved * 1e12 / PEAK_MFMA_F16,
            "traffic": load_traffic("prefill_chain" if dom == "chain_kernel" else "prefill_prep", digest),
            "algorithmic_flop_per_launch": dom_flop, "avg_launch_ms": dom_ms}
    path_flop = flop_prep + flop_chain
    dec_bytes = decode_bytes(dc["B"], dc["Hqk"], dc["Hv"])
    dec_gbs = dec_bytes / (dc["us_per_step"] * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA operands, f32 accumulate/state, bf16 I/O",
        "data": "synthetic (seeded, inputs resident in HBM)",
        "config": {"workload": "layer_prefill_T8192_16qk_48v", "B": 1, "T": T, "Hqk": Hqk, "Hv": Hv,
                   "d": D, "chunk": CHUNK, "seed": 1001},
        "roofline": roof,
        "path": {"algorithmic_flop": path_flop,
                 "mfma_frac": path_flop / (pf["ms_per_step"] * 1e-3) / PEAK_MFMA_F16,
                 "compulsory_bytes": prefill_bytes(T, Hqk, Hv),
                 "hbm_frac": prefill_bytes(T, Hqk, Hv) / (pf["ms_per_step"] * 1e-3) / PEAK_HBM,
                 "kernel_ms": km,
                 "event_intervals_ms": raw,
                 "other_kernel": {"kernel": "prep_kernel" if dom == "chain_kernel" else "chain_kernel",
                                  "tflops": (flop_prep if dom == "chain_kernel" else flop_chain) /
                                  (km["prep_kernel" if dom == "chain_kernel" else "chain_kernel"] * 1e-3) / 1e12}},
        "decode": {"metric": "decode us/step (B=256, 16QK/48V, 64 in-place steps)",
                   "value": dc["us_per_step"], "unit": "us/step", "higher_is_better": False,
                   "roofline": {"bound": "hbm", "kernel": "decode step (decode_step_kernel + conv_shift_qk_kernel<1>)",
                                "achieved": dec_gbs, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                                "frac": dec_gbs * 1e9 / PEAK_HBM,
                                "traffic": _sum_or_none(load_traffic("decode", digest),
                                                        load_traffic("decode_conv_shift", digest)),
                                "algorithmic_bytes_per_launch": dec_bytes}},
        "decode_multi": dm,
        "backward": bw,
        "source_digest": digest,
    }
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
        line["backward"]["cpu_baseline"] = cpu_baseline_backward()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
