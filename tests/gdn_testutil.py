"""Helpers shared by the GPU parity tests: host<->device marshalling and the
tolerance checks.  No mixer arithmetic lives here.

Tolerances (fp32 accumulation, bf16 I/O):
  * relative L2 of the output            <= 1e-2
  * relative L2 of the final fp32 state  <= 1e-3
  * per element |o_gpu - o_ref| <= 3e-2 * RMS(o_ref) + half a bf16 ulp of o_ref
    (the output is bf16, so its own rounding is excused; only error beyond
    the format's rounding counts against the 3e-2 * RMS bound)
"""
import numpy as np

from linear_attention_sequence_gdn_amd import inputs

OUT_REL_L2 = 1e-2
STATE_REL_L2 = 1e-3
MAX_ABS_RMS = 3e-2


def dev_bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def dev_i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host_bf16(t):
    """bf16 torch tensor -> float64 numpy."""
    import torch
    u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return inputs.bf16_to_f32(u).astype(np.float64)


def host_u16(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def half_ulp_bf16(x):
    x = np.asarray(x, np.float64)
    _, e = np.frexp(np.abs(x))  # |x| = m 2^e, m in [0.5, 1)
    h = np.ldexp(1.0, e - 9)
    return np.where(x == 0, 0.0, h)


def rel_l2(got, ref):
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(np.asarray(got, np.float64) - ref)
    return num / den if den > 0 else num


def check_output(got, ref, what="o"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    r = rel_l2(got, ref)
    rms = np.sqrt(np.mean(ref ** 2))
    excess = np.abs(got - ref) - half_ulp_bf16(ref)
    worst = float(excess.max()) / rms if rms > 0 else float(excess.max())
    assert r <= OUT_REL_L2, f"{what}: relL2 {r:.3e} > {OUT_REL_L2}"
    assert worst <= MAX_ABS_RMS, f"{what}: max-abs excess {worst:.3e} RMS > {MAX_ABS_RMS}"
    return r, worst


def check_state(got, ref, what="state"):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    r = rel_l2(got, ref)
    assert r <= STATE_REL_L2, f"{what}: relL2 {r:.3e} > {STATE_REL_L2}"
    return r
