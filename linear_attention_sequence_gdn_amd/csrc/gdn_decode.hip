// gdn_decode.hip -- one decode step of the GDN mixer on gfx950.
//
// One token per sequence: the work is streaming every (sequence, V head)
// state once from HBM and once back (64 KiB each way per head at d = 128),
// with a few hundred flops per state column, so the kernel is HBM-bound and
// is laid out for coalesced 16-byte accesses and few bytes of traffic beyond
// the state itself.
//
// The state update of the local-inference walkthrough (section 2.1) for one
// token, with p = alpha S^T k^ and u = beta (v^ - p):
//     S' = alpha S + k^ u^T,      o = S'^T q^ = alpha S^T q^ + u (k^ . q^)
// so both reductions over the d_k rows (S^T k^ and S^T q^) come from one read
// of the old state, and the new state is written in the same pass.
#include "gdn_common.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;

struct DecodeArgs {
    const uint16_t *q, *k, *v;
    const float *a, *b;
    const uint16_t *conv_w;
    uint16_t *conv_state;
    const float *state_in;
    float *state_out;
    uint16_t *o;
    int B, Hqk, Hv;
    float gate_scale, q_scale;
};

// conv (width 4) + SiLU of one channel, and the in-place shift of its rows
__device__ __forceinline__ float conv_channel(const DecodeArgs &p, int b, long C_tot, long c,
                                              uint16_t x)
{
    uint16_t *cs = p.conv_state + (long)b * 3 * C_tot + c;
    uint16_t h0 = cs[0], h1 = cs[C_tot], h2 = cs[2 * C_tot];
    uint2 w = *reinterpret_cast<const uint2 *>(p.conv_w + c * 4);
    float y = bf16_lo(w.x) * bf16_to_f32(h0) + bf16_hi(w.x) * bf16_to_f32(h1) +
              bf16_lo(w.y) * bf16_to_f32(h2) + bf16_hi(w.y) * bf16_to_f32(x);
    cs[0] = h1;
    cs[C_tot] = h2;
    cs[2 * C_tot] = x;
    return silu_f(y);
}

// One workgroup per (sequence b, V head h), so that each streams a single
// 64 KiB state (many short workgroups keep more of HBM busy than a few long
// ones).  q^ and k^ of the head's QK group are computed by each of the group's
// workgroups from the conv rows as they were before the step, which stay
// untouched here; only the workgroup's own v channels are shifted in place,
// and conv_shift_qk_kernel shifts the q and k rows afterwards (same stream).
__device__ __forceinline__ float conv_channel_ro(const DecodeArgs &p, int b, long C_tot, long c, uint16_t x)
{
    const uint16_t *cs = p.conv_state + (long)b * 3 * C_tot + c;
    const uint2 w = *reinterpret_cast<const uint2 *>(p.conv_w + c * 4);
    const float y = bf16_lo(w.x) * bf16_to_f32(cs[0]) + bf16_hi(w.x) * bf16_to_f32(cs[C_tot]) +
                    bf16_lo(w.y) * bf16_to_f32(cs[2 * C_tot]) + bf16_hi(w.y) * bf16_to_f32(x);
    return silu_f(y);
}

__global__ __launch_bounds__(kThreads) void decode_head_kernel(DecodeArgs p)
{
    __shared__ float s_q[kD], s_k[kD], s_v[kD];
    __shared__ float s_red[4];
    __shared__ float s_ab[2];
    __shared__ float s_kq;
    __shared__ f32x4 s_part[8][32][2];  // [row group][col group][k^/q^ partial]

    const int t = threadIdx.x;
    const int h = blockIdx.x % p.Hv;
    const int b = blockIdx.x / p.Hv;
    const int g = h / (p.Hv / p.Hqk);
    const long C_tot = 2L * p.Hqk * kD + (long)p.Hv * kD;
    const int lane = t & 63, wave = t >> 6;

    // the state is requested first, so that its latency covers the prologue:
    // thread owns columns 4cg..4cg+3, rows rg + 8i
    const int cg = t & 31, rg = t >> 5;
    const long head0 = ((long)b * p.Hv + h) * kD * kD;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(p.state_in + head0) + rg * 32 + cg;
    f32x4 *dst = reinterpret_cast<f32x4 *>(p.state_out + head0) + rg * 32 + cg;
    f32x4 st[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = __builtin_nontemporal_load(src + i * 256);

    // ---- prologue: q_g (threads 0..127) and k_g (128..255), read-only conv
    //      rows; v_h (threads 0..127) with its in-place shift; the gates
    {
        const bool isq = t < kD;
        const int ch = t & (kD - 1);
        const long c = isq ? (long)g * kD + ch : (long)p.Hqk * kD + (long)g * kD + ch;
        const uint16_t x = isq ? p.q[((long)b * p.Hqk + g) * kD + ch] : p.k[((long)b * p.Hqk + g) * kD + ch];
        const float z = conv_channel_ro(p, b, C_tot, c, x);
        const float ss = wave_sum(z * z);
        if (lane == 0) s_red[wave] = ss;
        if (isq) s_q[ch] = z; else s_k[ch] = z;
        if (isq) {
            const long cv = 2L * p.Hqk * kD + (long)h * kD + ch;
            s_v[ch] = conv_channel(p, b, C_tot, cv, p.v[((long)b * p.Hv + h) * kD + ch]);
        }
        if (t == kD) {
            s_ab[0] = __expf(-p.gate_scale * softplus_f(p.a[(long)b * p.Hv + h]));
            s_ab[1] = sigmoid_f(p.b[(long)b * p.Hv + h]);
        }
    }
    __syncthreads();
    if (t < kD) {
        s_q[t] *= rsqrtf(s_red[0] + s_red[1] + 1e-6f);
        s_k[t] *= rsqrtf(s_red[2] + s_red[3] + 1e-6f);
    }
    __syncthreads();
    if (wave == 0) {
        float kq = s_k[lane] * s_q[lane] + s_k[lane + 64] * s_q[lane + 64];
        kq = wave_sum(kq);
        if (lane == 0) s_kq = kq;
    }
    // ---- S^T k^ and S^T q^
    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float kr = s_k[rg + 8 * i], qr = s_q[rg + 8 * i];
        pk += st[i] * kr;
        pq += st[i] * qr;
    }
    s_part[rg][cg][0] = pk;
    s_part[rg][cg][1] = pq;
    __syncthreads();
    f32x4 PK = {0.f, 0.f, 0.f, 0.f}, PQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        PK += s_part[r][cg][0];
        PQ += s_part[r][cg][1];
    }
    const float al = s_ab[0], be = s_ab[1], kq = s_kq;
    f32x4 u, ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        u[e] = be * (s_v[4 * cg + e] - al * PK[e]);
        ov[e] = (al * PQ[e] + u[e] * kq) * p.q_scale;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float kr = s_k[rg + 8 * i];
        __builtin_nontemporal_store(st[i] * al + u * kr, dst + i * 256);
    }
    if (rg == 0) {
        uint2 packed;
        packed.x = pack_bf16x2(ov[0], ov[1]);
        packed.y = pack_bf16x2(ov[2], ov[3]);
        *reinterpret_cast<uint2 *>(p.o + ((long)b * p.Hv + h) * kD + 4 * cg) = packed;
    }
}

// The in-place shift of the q and k conv rows, after decode_head_kernel has
// read them: rows (r0, r1, r2) <- (r1, r2, x), two channels per thread.
__global__ __launch_bounds__(kThreads) void conv_shift_qk_kernel(DecodeArgs p)
{
    const long nqk = 2L * p.Hqk * kD;  // q and k channels per sequence
    const long C_tot = nqk + (long)p.Hv * kD;
    const long i = ((long)blockIdx.x * kThreads + threadIdx.x) * 2;
    if (i >= (long)p.B * nqk) return;
    const int b = (int)(i / nqk);
    const long c = i % nqk;  // q channels first, then k
    const long qk = (long)p.Hqk * kD;
    const uint16_t *x = c < qk ? p.q + (long)b * qk + c : p.k + (long)b * qk + (c - qk);
    uint32_t *cs = reinterpret_cast<uint32_t *>(p.conv_state + (long)b * 3 * C_tot + c);
    const uint32_t r1 = cs[C_tot / 2], r2 = cs[C_tot];
    cs[0] = r1;
    cs[C_tot / 2] = r2;
    cs[C_tot] = *reinterpret_cast<const uint32_t *>(x);
}

}  // namespace

hipError_t launch_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                         const float *b, const uint16_t *conv_w, uint16_t *conv_state,
                         const float *state_in, float *state_out, uint16_t *o, int B, int Hqk,
                         int Hv, float gate_scale, float q_scale, hipStream_t stream)
{
    DecodeArgs p{q, k, v, a, b, conv_w, conv_state, state_in, state_out, o,
                 B, Hqk, Hv, gate_scale, q_scale};
    if ((long)B * Hqk == 0) return hipSuccess;
    const long grid = (long)B * Hv;
    hipLaunchKernelGGL(decode_head_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long pairs = (long)B * Hqk * kD;  // 2 * Hqk * kD channels, two per thread
    hipLaunchKernelGGL(conv_shift_qk_kernel, dim3((unsigned)((pairs + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace gdn
