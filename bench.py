#!/usr/bin/env python3
"""GDN token mixer benchmark on one MI355X.

A step is one chunked prefill of the model-layer workload (B = 1, T = 8192,
16 QK / 48 V heads, d = 128, seeded synthetic bf16 inputs already resident in
HBM).  The decode workload (B = 256 sequences, 64 consecutive in-place steps)
is timed in the same run and reported under "decode", the training backward
of the prefill workload under "backward", and the other prefill workloads
(the tiny 2 QK / 6 V one, the 262,144-token one, the 64-sequence packed one)
under "configs".  Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                  [--no-cpu-baseline] [--only LEG ...] [--calibrate-copy]
  python bench.py --traffic-report FETCH_CSV WRITE_CSV
  python bench.py --counter-report OUT_MD DB [DB ...] [--counter-command CMD]
  python bench.py --trace-report OUT_MD DB [--counter-command CMD]

--only restricts the run to some legs (prefill, decode, decode_multi,
backward, backward_windows, configs, segments), for profiling; the JSON line
then holds those legs.  "segments" times a tensor-parallel shard's head shape
(2 QK / 6 V) at T = 8192 and 262,144 with and without the sequential pass's
sequence split.  "backward_windows" times the backward with a workspace short
of the one-pass size (T = 8192 in 512 MiB, T = 262,144 in 3 GiB), which runs
in windows.
--calibrate-copy ends the run with a plain 256 MiB device-to-device copy, so
that a rocprofv3 --pmc pass over this command also reads its counters for a
transfer of known size.  --traffic-report turns two such passes (FETCH_SIZE,
then WRITE_SIZE; rocprofv3's counter_collection.csv files) into HBM bytes per
launch of each kernel, scaled by what the counters read for the copy, and
writes them to profiles/traffic.json tagged with the digest of the kernel
sources they were taken on.  --counter-report summarises rocprofv3 --pmc
databases (one per pass) per kernel: matrix-core busy fraction and FLOP, LDS
instructions, bank conflicts and issue waits.

Timing: HIP events on the stream the library launches on.  Before anything is
timed, each leg runs its own work back to back until at least --settle-ms of
GPU time (default 400 ms) has passed, whatever --warmup says: the GPU's
clocks ramp up under load, and a prefill timed after 30 steps (5 ms) ran
about 10 % slower than one timed after 200.  The step time is K plain
gdn_prefill calls between two events; the same K steps are then run through
gdn_prefill_with_events, which records an event after each of its kernels
(chunk-table setup, parallel pass, sequential pass), for the per-kernel times
the roofline uses.  Each recorded event costs the stream a few microseconds;
the interval before the first kernel, empty for a uniform batch, measures
that cost, and it is subtracted from the kernels' intervals (the raw
intervals are reported too).  The 64 decode steps run back to back between
two events.  The GPU's shader clock is sampled from the driver while the legs
run.  The CPU baselines are the fp64 oracle, as it stands, on bounded samples
of the same workloads.
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


def method_flops(lengths, Hqk, Hv, n=CHUNK, d=D):
    """Algorithmic FLOP of the chunked method over sequences of the given
    lengths, C fixed at 64 and a partial last chunk counted with its own n:
    per chunk and V head 6 n d^2 (W S, K^T Vnew, Q S) + 6 n^2 d (W, U', P
    Vnew) + n^3 / 3 (the triangular inverse); per chunk and QK head 4 n^2 d
    (K K^T, Q K^T).  7,667,712 FLOP per token at 16 QK / 48 V heads."""
    total = 0.0
    for L in lengths:
        L = int(L)
        full, rem = divmod(L, n)
        for m, cnt in ((n, full), (rem, 1 if rem else 0)):
            total += cnt * (Hv * (6 * m * d * d + 6 * m * m * d + m ** 3 / 3) + Hqk * 4 * m * m * d)
    return total


# bytes per (chunk, QK group) of the q^ and k^ operands, and per (chunk, V
# head) of the T' / P / gates record, that the parallel pass hands over
QK_FRAG_BYTES = 2 * 16 * 1024
REC_BYTES = 11 * 1024


def prep_bytes(T, Hqk, Hv, d=D):
    """Bytes the parallel pass moves by its design: q and k read (bf16), a and
    b read (fp32), the conv taps of q and k, and its hand-over written.  Its
    arithmetic (about 20 FLOP per byte) is far below the fp16 matrix-core
    ridge (2.5 PFLOP/s / 8 TB/s = 312 FLOP per byte), so HBM bounds it."""
    chunks = -(-T // CHUNK)
    read = 2 * T * Hqk * d * 2 + 2 * T * Hv * 4 + 2 * Hqk * d * 4 * 2
    write = chunks * (Hqk * QK_FRAG_BYTES + Hv * REC_BYTES)
    return read + write


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


def settle(hip, stream, work, settle_ms, batch=20):
    """Run `work` back to back, `batch` calls between two events, until at
    least settle_ms of GPU time has passed (the clocks ramp up under load).
    Returns (GPU ms spent, calls made)."""
    spent, calls = 0.0, 0
    t0, t1 = hip.event(), hip.event()
    while spent < settle_ms:
        hip.record(t0, stream)
        for _ in range(batch):
            work()
        hip.record(t1, stream)
        spent += hip.ms(t0, t1)
        calls += batch
    return spent, calls


class ClockSampler:
    """Samples the GPU's shader clock (MHz) from the driver in a background
    thread while legs run: the amdgpu sysfs DPM table where it is readable,
    else rocm-smi.  Reports None where neither answers."""

    def __init__(self, period_s=0.05):
        import threading
        self.samples = []
        self.source = None
        self._stop = threading.Event()
        self._sysfs = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self._thread = threading.Thread(target=self._run, args=(period_s,), daemon=True)

    def _read(self):
        import re
        import subprocess
        for path in self._sysfs:
            try:
                for line in open(path):
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        if m:
                            self.source = "sysfs pp_dpm_sclk"
                            return float(m.group(1))
            except OSError:
                pass
        try:
            out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                                 timeout=10).stdout
            m = re.search(r"sclk.*?\((\d+)\s*[Mm][Hh]z\)", out)
            if m:
                self.source = "rocm-smi --showclocks"
                return float(m.group(1))
        except (OSError, subprocess.SubprocessError):
            pass
        return None

    def _run(self, period_s):
        while not self._stop.is_set():
            v = self._read()
            if v is None:
                return
            self.samples.append(v)
            self._stop.wait(period_s if self.source and self.source.startswith("sysfs") else 1.0)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=15)

    def summary(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        return {"sclk_mhz_median": xs[len(xs) // 2], "sclk_mhz_max": xs[-1], "samples": len(xs),
                "source": self.source}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


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
                   "prefill_setup": "setup_kernel", "decode": "decode_persist_kernel",
                   "decode_conv_shift": "conv_shift_qk_kernel<1>",
                   "decode_multi": "decode_tokens_kernel<4>", "decode_multi_conv_shift": "conv_shift_qk_kernel<4>"}
BWD_KERNELS = ("bwd_prep_kernel", "bwd_local_kernel", "bwd_fwd_kernel", "bwd_chain_kernel", "bwd_grad_kernel",
               "bwd_dyconv_kernel", "bwd_dw_kernel")
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


XCDS, CUS, SIMDS_PER_CU = 8, 256, 4


def counter_report(out_md, dbs, command=""):
    """Per-kernel averages (per dispatch) of the counters in rocprofv3
    databases (one --pmc pass each), and what follows from them:

    * MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI cycles x 256 CUs x 4 SIMDs),
      the fraction of the kernel's time the matrix cores are busy.
      GRBM_GUI_ACTIVE reads the sum over the 8 XCDs, so one XCD's active
      cycles are a eighth of it.
    * matrix-core FLOP = 512 per MOP (SQ_INSTS_VALU_MFMA_MOPS_*); dense peaks
      per CU-cycle: 4096 fp16/bf16, 256 fp32.
    * LDS: instructions, bank-conflict cycles per CU as a fraction of the
      active cycles, and the share of wave cycles spent waiting to issue an
      LDS instruction (SQ_WAIT_INST_LDS) or any instruction (SQ_WAIT_INST_ANY).
    Inputs are rocprofv3 databases or --output-format csv counter files.
    Writes a markdown table to out_md."""
    import collections
    import re
    import sqlite3
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for db in dbs:
        if db.endswith(".csv"):  # --output-format csv: one row per (dispatch, counter)
            import csv
            per = collections.defaultdict(float)
            for r_ in csv.DictReader(open(db)):
                per[(r_["Kernel_Name"], r_["Dispatch_Id"], r_["Counter_Name"])] += float(r_["Counter_Value"])
            rows_ = [(k_, c_, v_) for (k_, _, c_), v_ in per.items()]
        else:
            rows_ = sqlite3.connect(db).execute("select kernel_name, counter_name, value from counters_collection")
        for kname, ctr, val in rows_:
            m = re.search(r"(\w+(?:<[^>]*>)?)\(", kname)
            acc[m.group(1) if m else kname][ctr].append(float(val))
    lines = ["# Counter summary", "", "Command(s):", ""] + [f"    {c_}" for c_ in command.split(" ;; ") if c_] + [""]
    for k_, ctrs in sorted(acc.items()):
        avg = {c_: sum(v_) / len(v_) for c_, v_ in ctrs.items()}
        n = min(len(v_) for v_ in ctrs.values())
        lines += [f"## {k_} ({n} dispatches per pass)", "", "| counter | mean per dispatch |", "|---|---|"]
        lines += [f"| {c_} | {v_:,.0f} |" for c_, v_ in sorted(avg.items())]
        gui = avg.get("GRBM_GUI_ACTIVE")
        der = []
        if gui:
            cyc = gui / XCDS
            der.append(("active cycles per XCD", f"{cyc:,.0f}"))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                der.append(("MFMA busy (of all SIMDs' cycles)",
                            f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * CUS * SIMDS_PER_CU):.3f}"))
            f16 = 512 * (avg.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0) + avg.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0))
            if f16:
                der.append(("fp16/bf16 matrix-core FLOP per dispatch", f"{f16 / 1e9:.2f} G"))
                der.append(("fp16/bf16 FLOP per cycle / dense peak (4096 per CU-cycle)",
                            f"{f16 / (cyc * CUS * 4096):.3f}"))
            f32 = 512 * avg.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0)
            if f32:
                der.append(("fp32 matrix-core FLOP per dispatch", f"{f32 / 1e9:.2f} G"))
                der.append(("fp32 FLOP per cycle / dense peak (256 per CU-cycle)",
                            f"{f32 / (cyc * CUS * 256):.3f}"))
            if "SQ_LDS_BANK_CONFLICT" in avg:
                der.append(("LDS bank-conflict cycles per CU / active cycles",
                            f"{avg['SQ_LDS_BANK_CONFLICT'] / CUS / cyc:.3f}"))
        if "SQ_WAVE_CYCLES" in avg:
            wc = avg["SQ_WAVE_CYCLES"]
            for c_, name in (("SQ_WAIT_INST_LDS", "wave cycles waiting to issue LDS"),
                             ("SQ_WAIT_INST_ANY", "wave cycles waiting to issue any instruction"),
                             ("SQ_ACTIVE_INST_VALU", "wave cycles issuing VALU (incl. MFMA)")):
                if c_ in avg:
                    der.append((name, f"{avg[c_] / wc:.3f}"))
        if der:
            lines += ["", "| derived | value |", "|---|---|"] + [f"| {a_} | {b_} |" for a_, b_ in der]
        lines.append("")
    open(out_md, "w").write("\n".join(lines))
    print("\n".join(lines))


def trace_report(out_md, db, command="", tail=40):
    """Per-kernel dispatch count and mean / min / max duration from a
    rocprofv3 --kernel-trace database, as a markdown table in out_md, with the
    mean over each kernel's last `tail` dispatches: the bench's timed steps
    (K plain calls, then K with events) come last, after the settle phase."""
    import re
    import sqlite3
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), avg(duration), min(duration), max(duration), sum(duration) "
                       "from kernels group by name order by sum(duration) desc").fetchall()
    total = sum(r[5] for r in rows) or 1.0
    lines = ["# Kernel trace summary", "", "Command:", "", f"    {command}", "",
             f"| kernel | dispatches | mean us | mean of the last {tail} us | min us | max us | share of kernel time |",
             "|---|---|---|---|---|---|---|"]
    for name, n, avg, mn, mx, tot in rows:
        m = re.search(r"(\w+(?:<[^>]*>)?)\(", name)
        last = [r[0] for r in con.execute("select duration from kernels where name = ? order by start desc limit ?",
                                          (name, tail))]
        lines.append(f"| {m.group(1) if m else name} | {n} | {avg / 1e3:.2f} | {sum(last) / len(last) / 1e3:.2f} | "
                     f"{mn / 1e3:.2f} | {mx / 1e3:.2f} | {tot / total:.3f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


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
def bench_prefill(hip, steps, warmup, settle_ms):
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
    settle_gpu_ms, settle_calls = settle(hip, sp, run, settle_ms)
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
    return dict(ms_per_step=total_ms / steps, stage_ms=stage, T=T, Hqk=Hqk, Hv=Hv,
                settle_gpu_ms=settle_gpu_ms, settle_calls=settle_calls + warmup)


def bench_decode(hip, settle_ms, steps=64):
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
    it = iter(range(1 << 30))
    settle(hip, sp, lambda: step(next(it) % steps), settle_ms, batch=64)
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


def bench_decode_multi(hip, settle_ms, T=4, steps=32):
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
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    settle(hip, sp, lambda: gdn.gdn_decode_multi(q, k, v, a, b, w, conv, st, o=o, gate_scale=c["gate_scale"]),
           settle_ms, batch=16)
    torch.cuda.synchronize()
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
            "roofline": {"bound": "hbm", "kernel": "decode_tokens_kernel<4> + conv_shift_qk_kernel<4>",
                         "achieved": gbs, "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": gbs * 1e9 / PEAK_HBM,
                         "traffic": _sum_or_none(load_traffic("decode_multi", source_digest()),
                                                 load_traffic("decode_multi_conv_shift", source_digest())),
                         "algorithmic_bytes_per_launch": nbytes}}


def bench_backward(hip, settle_ms, steps=10, warmup=3):
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
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(warmup):
        run()
    settle(hip, sp, run, settle_ms, batch=4)
    torch.cuda.synchronize()
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
            "roofline": {"bound": "alu", "kernel": "whole backward (seven launches)", "achieved": tf,
                         "peak": PEAK_VALU_F32 / 1e12, "unit": "TFLOP/s", "frac": tf * 1e12 / PEAK_VALU_F32,
                         "traffic": None, "algorithmic_flop_per_call": flop}}


def bench_backward_windows(hip):
    """The backward in a workspace short of the one-pass size: T = 8192 in
    512 MiB (the cost of the windows at the same length) and the native-context
    length T = 262,144 (one pass: ~83 GB) in 3 GiB."""
    import numpy as np
    import torch
    from linear_attention_sequence_gdn_amd import inputs

    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    out = {}
    for idx, seed, ws_bytes, steps in ((1, 1001, 512 << 20, 3), (2, 1002, 3 << 30, 2)):
        c = inputs.CONFIGS[idx]
        B, T, Hqk, Hv = 1, c["T"], c["Hqk"], c["Hv"]
        x = inputs.make_prefill(T_list=[T], Hqk=Hqk, Hv=Hv, seed=seed, gate_scale=c["gate_scale"])
        gen = torch.Generator(device="cuda").manual_seed(2000 + idx)
        g_o = torch.randn((B, T, Hv, D), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        g_S = torch.randn((B, Hv, D, D), generator=gen, device="cuda", dtype=torch.float32)
        args = (bf(x["q"].reshape(B, T, Hqk, D)), bf(x["k"].reshape(B, T, Hqk, D)), bf(x["v"].reshape(B, T, Hv, D)),
                f32(x["a"].reshape(B, T, Hv)), f32(x["b"].reshape(B, T, Hv)), bf(x["conv_w"]), g_o)
        del x
        out[f"T{T}"] = bench_backward_bounded(hip, args, g_S, T, Hqk, Hv, c["gate_scale"], ws_bytes, steps)
        del args, g_o
        torch.cuda.empty_cache()
    return out


def bench_backward_bounded(hip, args, g_S, T, Hqk, Hv, gate_scale, ws_bytes, steps):
    """gdn_prefill_backward with a workspace of ws_bytes, short of the one-pass
    size: the sequence runs in windows (forward sweep for the window states,
    then the windows' backwards from the last).  One warm-up call, then K
    calls between two events."""
    import torch
    import linear_attention_sequence_gdn_amd as gdn

    tw = gdn.gdn_prefill_backward_windows(1, T, Hqk, Hv, ws_bytes)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    run = lambda: gdn.gdn_prefill_backward(*args, gate_scale=gate_scale, grad_state_out=g_S, workspace=ws)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    run()
    torch.cuda.synchronize()
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, sp)
    for _ in range(steps):
        run()
    hip.record(t1, sp)
    torch.cuda.synchronize()
    ms = hip.ms(t0, t1) / steps
    return {"T": T, "workspace_bytes": ws_bytes,
            "one_pass_workspace_bytes": gdn.gdn_prefill_backward_workspace_size(1, T, Hqk, Hv),
            "window_tokens": tw, "windows": -(-T // tw), "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "calls": steps}


def bench_config(hip, idx, settle_ms, steps):
    """One of the other prefill workloads, timed as the step is: the tiny
    2 QK / 6 V prefill (T = 512), the native-context prefill (T = 262,144,
    long memory) and the packed batch of 64 sequences (log-uniform lengths
    128..32768, nonzero initial states).  Whole calls between two events."""
    import numpy as np
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    from linear_attention_sequence_gdn_amd import inputs

    x = inputs.make_config(idx)
    Hqk, Hv, N, T_tot = x["Hqk"], x["Hv"], x["N"], x["T_tot"]
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    lengths = np.diff(x["cu_seqlens"])
    uniform = idx != 4
    st = None if x["state_in"] is None else f32(x["state_in"])
    w = bf(x["conv_w"])
    if uniform:
        T = int(lengths[0])
        args = (bf(x["q"].reshape(N, T, Hqk, D)), bf(x["k"].reshape(N, T, Hqk, D)), bf(x["v"].reshape(N, T, Hv, D)),
                f32(x["a"].reshape(N, T, Hv)), f32(x["b"].reshape(N, T, Hv)), w)
        need = gdn.gdn_prefill_workspace_size(N, T, Hqk, Hv)
    else:
        args = (bf(x["q"]), bf(x["k"]), bf(x["v"]), f32(x["a"]), f32(x["b"]), w,
                torch.from_numpy(x["cu_seqlens"]).cuda())
        need = gdn.gdn_prefill_varlen_workspace_size(N, T_tot, Hqk, Hv)
    del x
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    so = torch.empty((N, Hv, D, D), dtype=torch.float32, device="cuda")
    o = torch.empty((T_tot * Hv * D,), dtype=torch.bfloat16, device="cuda")
    o = o.view(N, -1, Hv, D) if uniform else o.view(T_tot, Hv, D)
    fn = gdn.gdn_prefill if uniform else gdn.gdn_prefill_varlen
    gs = inputs.CONFIGS[idx]["gate_scale"]
    run = lambda: fn(*args, gate_scale=gs, state_in=st, state_out=so, o=o, workspace=ws)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    run()
    settle(hip, sp, run, settle_ms, batch=max(1, min(20, int(20 * 8192 / max(T_tot, 1)))))
    k = max(3, min(steps, int(steps * 8192 * 4 / max(T_tot, 1))))
    t0, t1 = hip.event(), hip.event()
    hip.record(t0, sp)
    for _ in range(k):
        run()
    hip.record(t1, sp)
    torch.cuda.synchronize()
    ms = hip.ms(t0, t1) / k
    flop = method_flops(lengths, Hqk, Hv)
    names = {0: "tiny_prefill_T512_2qk_6v", 2: "native_context_prefill_T262144_16qk_48v",
             4: "varlen_prefill_64seq_16qk_48v"}
    out = {"workload": names[idx], "tokens": int(T_tot), "sequences": int(N), "ms_per_call": ms, "calls": k,
           "tokens_per_s": T_tot / (ms * 1e-3), "algorithmic_flop": flop,
           "mfma_frac": flop / (ms * 1e-3) / PEAK_MFMA_F16}
    if uniform and need > gdn.gdn_prefill_noalloc_max_workspace():
        # the same call with its workspace bounded to the no-alloc array's
        # size: the library runs it in windows of whole chunks
        bound = gdn.gdn_prefill_noalloc_max_workspace()
        ws_b = ws[:bound]
        # the window the library picks: the largest whole-chunk window whose
        # workspace fits beside the two state buffers it hands states through
        sb = (N * Hv * D * D * 4 + 255) // 256 * 256
        tw = 64
        while tw + 64 <= T and gdn.gdn_prefill_workspace_size(N, tw + 64, Hqk, Hv) <= (bound - 2 * sb) // 256 * 256:
            tw += 64
        run_b = lambda: fn(*args, gate_scale=gs, state_in=st, state_out=so, o=o, workspace=ws_b)
        run_b()
        kb = max(3, k // 2)
        hip.record(t0, sp)
        for _ in range(kb):
            run_b()
        hip.record(t1, sp)
        torch.cuda.synchronize()
        msb = hip.ms(t0, t1) / kb
        out["bounded_workspace"] = {"workspace_bytes": bound, "window_tokens": tw, "windows": -(-T // tw),
                                    "ms_per_call": msb, "tokens_per_s": T_tot / (msb * 1e-3)}
    return out


def bench_segments(hip, settle_ms, steps):
    """What intra-card sequence parallelism buys at a tensor-parallel shard's
    head shape (2 QK / 6 V heads: 48 V heads over 8 GPUs), T = 8192 and
    T = 262,144: the prefill with the library's segment split against the
    same call with every sequence run as one segment (gdn_prefill_with_options).
    Both again with no decay on any head (a = -30: alpha = 1 to fp32
    precision): every later segment then misses its warm-up bound and goes
    through its transition matrix and the in-order combine."""
    import numpy as np
    import torch
    import linear_attention_sequence_gdn_amd as gdn
    from linear_attention_sequence_gdn_amd import inputs

    L = gdn.lib()
    Hqk, Hv = 2, 6
    out = {}
    for T, decay in ((8192, True), (262144, True), (8192, False), (262144, False)):
        x = inputs.make_prefill(T_list=[T], Hqk=Hqk, Hv=Hv, seed=1100, gate_scale=0.1)
        if not decay:
            x["a"][:] = -30.0
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
        q, k, v = bf(x["q"]), bf(x["k"]), bf(x["v"])
        a, b, w = f32(x["a"]), f32(x["b"]), bf(x["conv_w"])
        del x
        o = torch.empty((T, Hv, D), dtype=torch.bfloat16, device="cuda")
        so = torch.empty((1, Hv, D, D), dtype=torch.float32, device="cuda")
        need = gdn.gdn_prefill_workspace_size(1, T, Hqk, Hv)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        P = lambda t_: ctypes.c_void_p(t_.data_ptr())
        res = {}
        for name, segc in (("auto", 0), ("one_segment", (T + CHUNK - 1) // CHUNK)):
            run = lambda: L.gdn_prefill_with_options(P(q), P(k), P(v), P(a), P(b), P(w), None, None, None, P(so),
                                                     P(o), 1, T, Hqk, Hv, D, D, 0.1, 1.0, P(ws), need, sp, segc, None)
            assert run() == 0
            settle(hip, sp, run, settle_ms / 2, batch=max(1, 20 * 8192 // T))
            kk = max(3, min(steps, steps * 8192 // T * 4))
            t0, t1 = hip.event(), hip.event()
            hip.record(t0, sp)
            for _ in range(kk):
                run()
            hip.record(t1, sp)
            ms = hip.ms(t0, t1) / kk
            res[name] = {"ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3)}
        res["speedup_of_segments"] = res["one_segment"]["ms_per_call"] / res["auto"]["ms_per_call"]
        out[f"T{T}_2qk_6v" + ("" if decay else "_no_decay")] = res
        del q, k, v, o, ws
    return out


def cpu_baseline_config(idx, min_seconds=4.0, max_reps=20):
    """The oracle on a bounded sample of config idx's workload."""
    import numpy as np
    import oracle
    from linear_attention_sequence_gdn_amd import inputs
    oracle.build(force=False)
    c = inputs.CONFIGS[idx]
    heads = None
    if idx == 2:  # the first 16384 tokens, V heads 0, 23, 47 (the parity test's heads)
        x = inputs.make_config(2, heads=[0, 23, 47], qk_heads=[0, 7, 15], T_override=16384)
        heads = [0, 23, 47]
        what = "first 16384 tokens of the T=262144 workload, V heads 0, 23, 47 (3 of 48)"
    elif idx == 4:  # four of the 64 packed sequences
        full = inputs.make_config(4)
        cu = full["cu_seqlens"]
        pick = [3, 17, 40, 63]
        idxs = np.concatenate([np.arange(cu[s_], cu[s_ + 1]) for s_ in pick])
        x = dict(full)
        for key in ("q", "k", "v", "a", "b"):
            x[key] = np.ascontiguousarray(full[key][idxs])
        L = np.diff(cu)[pick]
        x["cu_seqlens"] = np.concatenate([[0], np.cumsum(L)]).astype(np.int32)
        x["state_in"] = np.ascontiguousarray(full["state_in"][pick])
        del full
        what = f"sequences 3, 17, 40, 63 of the 64-sequence packed workload ({int(L.sum())} tokens), all heads"
    else:
        x = inputs.make_config(idx)
        what = "the whole workload"
    T = int(x["cu_seqlens"][-1])
    reps, t0 = 0, time.perf_counter()
    while reps < max_reps:
        oracle.prefill(x["q"], x["k"], x["v"], x["a"], x["b"], x["conv_w"], x["cu_seqlens"], Hqk=c["Hqk"],
                       Hv=c["Hv"], gate_scale=c["gate_scale"], state_in=x["state_in"], heads=heads)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    threads = oracle.num_threads() if heads is None else min(oracle.num_threads(), len(heads))
    return {"value": T * reps / dt, "unit": "tokens/s" + (" (3 of 48 V heads)" if heads else ""),
            "cores": threads, "kind": "oracle", "sample": f"fp64 oracle on {what}; {reps} run(s) in {dt:.1f} s wall"}


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


LEGS = ("prefill", "decode", "decode_multi", "backward", "backward_windows", "configs", "segments")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-ms", type=float, default=400.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", nargs="+", choices=LEGS)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--traffic-report", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--counter-report", nargs="+", metavar=("OUT_MD", "DB"))
    ap.add_argument("--counter-command", default="")
    ap.add_argument("--trace-report", nargs=2, metavar=("OUT_MD", "DB"))
    args = ap.parse_args()
    if args.traffic_report:
        traffic_report(*args.traffic_report)
        return
    if args.trace_report:
        trace_report(*args.trace_report, command=args.counter_command)
        return
    if args.counter_report:
        counter_report(args.counter_report[0], args.counter_report[1:], args.counter_command)
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
    legs = set(args.only or LEGS)
    settle_ms = args.settle_ms

    line = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f16 MFMA operands, f32 accumulate/state, bf16 I/O",
            "data": "synthetic (seeded, inputs resident in HBM)",
            "config": {"workload": "layer_prefill_T8192_16qk_48v", "B": 1, "T": 8192, "Hqk": 16, "Hv": 48,
                       "d": D, "chunk": CHUNK, "seed": 1001}}
    with ClockSampler() as clock:
        if "prefill" in legs:
            pf = bench_prefill(hip, args.steps, args.warmup, settle_ms)
            T, Hqk, Hv = pf["T"], pf["Hqk"], pf["Hv"]
            flop_prep, flop_chain = prefill_flops(T, Hqk, Hv)
            # dominant prefill kernel (the longer of the two that carry the
            # matrix products), priced against the fp16 dense matrix-core
            # peak.  Each recorded event costs the stream about as much as
            # the interval before the first kernel, which is empty here (a
            # uniform batch launches no setup kernel); it is subtracted from
            # the kernels' intervals.
            raw = pf["stage_ms"]
            event_ms = raw["setup_kernel"]
            km = {k_: max(v_ - event_ms, 0.0) for k_, v_ in raw.items() if k_ != "setup_kernel"}
            dom = "chain_kernel" if km["chain_kernel"] >= km["prep_kernel"] else "prep_kernel"
            other = "prep_kernel" if dom == "chain_kernel" else "chain_kernel"
            kflop = {"chain_kernel": flop_chain, "prep_kernel": flop_prep}
            achieved = kflop[dom] / (km[dom] * 1e-3) / 1e12
            path_flop = method_flops([T], Hqk, Hv)
            line.update({
                "value": T / (pf["ms_per_step"] * 1e-3),
                "ms_per_step": pf["ms_per_step"],
                "warmup_gpu_ms": pf["settle_gpu_ms"],
                "warmup_steps_run": pf["settle_calls"],
                "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved,
                             "peak": PEAK_MFMA_F16 / 1e12, "unit": "TFLOP/s",
                             "frac": achieved * 1e12 / PEAK_MFMA_F16,
                             "traffic": load_traffic("prefill_chain" if dom == "chain_kernel" else "prefill_prep",
                                                     digest),
                             "algorithmic_flop_per_launch": kflop[dom], "avg_launch_ms": km[dom]},
                "path": {"algorithmic_flop": path_flop,
                         "mfma_frac": path_flop / (pf["ms_per_step"] * 1e-3) / PEAK_MFMA_F16,
                         "compulsory_bytes": prefill_bytes(T, Hqk, Hv),
                         "hbm_frac": prefill_bytes(T, Hqk, Hv) / (pf["ms_per_step"] * 1e-3) / PEAK_HBM,
                         "kernel_ms": km, "event_intervals_ms": raw,
                         "other_kernel": {"kernel": other,
                                          "tflops": kflop[other] / (km[other] * 1e-3) / 1e12},
                         "prep_hbm_roofline": {
                             "bound": "hbm", "kernel": "prep_kernel",
                             "achieved": prep_bytes(T, Hqk, Hv) / (km["prep_kernel"] * 1e-3) / 1e9,
                             "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                             "frac": prep_bytes(T, Hqk, Hv) / (km["prep_kernel"] * 1e-3) / PEAK_HBM,
                             "design_bytes_per_launch": prep_bytes(T, Hqk, Hv),
                             "traffic": load_traffic("prefill_prep", digest)}}})
        if "decode" in legs:
            dc = bench_decode(hip, settle_ms)
            dec_bytes = decode_bytes(dc["B"], dc["Hqk"], dc["Hv"])
            dec_gbs = dec_bytes / (dc["us_per_step"] * 1e-6) / 1e9
            line["decode"] = {
                "metric": "decode us/step (B=256, 16QK/48V, 64 in-place steps)",
                "value": dc["us_per_step"], "unit": "us/step", "higher_is_better": False,
                "roofline": {"bound": "hbm", "kernel": "decode step (decode_persist_kernel + conv_shift_qk_kernel<1>)",
                             "achieved": dec_gbs, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                             "frac": dec_gbs * 1e9 / PEAK_HBM,
                             "traffic": _sum_or_none(load_traffic("decode", digest),
                                                     load_traffic("decode_conv_shift", digest)),
                             "algorithmic_bytes_per_launch": dec_bytes}}
        if "decode_multi" in legs:
            line["decode_multi"] = bench_decode_multi(hip, settle_ms)
        if "backward" in legs:
            bw = bench_backward(hip, settle_ms)
            bw["roofline"]["traffic"] = _sum_or_none(
                *(load_traffic("backward_" + k_[4:-7], source_digest(BWD_SOURCES)) for k_ in BWD_KERNELS))
            line["backward"] = bw
        if "backward_windows" in legs:
            line.setdefault("backward", {})["bounded_workspace"] = bench_backward_windows(hip)
        if "configs" in legs:
            line["configs"] = {str(i): bench_config(hip, i, settle_ms, args.steps) for i in (0, 2, 4)}
        if "segments" in legs:
            line["segments"] = bench_segments(hip, settle_ms, args.steps)
    line["gpu_clock"] = clock.summary()
    line["source_digest"] = digest
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        if "prefill" in legs:
            line["cpu_baseline"] = cpu_baseline()
            line["cpu_baseline"]["cpu_model"] = cpu_model()
        if "backward" in legs:
            line["backward"]["cpu_baseline"] = cpu_baseline_backward()
        if "configs" in legs:
            for i in (0, 2, 4):
                line["configs"][str(i)]["cpu_baseline"] = cpu_baseline_config(i)
    line["cpu_model"] = cpu_model()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
