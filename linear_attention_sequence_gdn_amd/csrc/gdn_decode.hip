// gdn_decode.hip -- one decode step of the GDN mixer on gfx950.
//
// One token per sequence: the work is streaming every (sequence, V head)
// state once from HBM and once back (64 KiB each way per head at d = 128),
// with a few hundred flops per state column, so the kernel is HBM-bound and
// is laid out for coalesced 16-byte accesses and few bytes of traffic beyond
// the state itself.
//
// Workgroup = one (sequence b, QK head g) and its G = Hv/Hqk V heads.  It
// owns every conv channel it reads (q_g, k_g and the v channels of its V
// heads), so the in-place conv-state shift is race-free.
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
constexpr int kMaxG = 16;  // V heads per QK head handled by one workgroup

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

__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs p)
{
    __shared__ float s_q[kD], s_k[kD];
    __shared__ float s_v[kMaxG][kD];
    __shared__ float s_alpha[kMaxG], s_beta[kMaxG];
    __shared__ float s_red[4];
    __shared__ float s_kq;
    __shared__ f32x4 s_part[2][8][32][2];  // [buffer][row group][col group][k^/q^ partial]

    const int t = threadIdx.x;
    const int g = blockIdx.x % p.Hqk;
    const int b = blockIdx.x / p.Hqk;
    const int G = p.Hv / p.Hqk;
    const long C_tot = 2L * p.Hqk * kD + (long)p.Hv * kD;
    const int lane = t & 63, wave = t >> 6;

    // ---- prologue: conv + SiLU of q_g (threads 0..127) and k_g (128..255)
    {
        const bool isq = t < kD;
        const int ch = t & (kD - 1);
        const long c = isq ? (long)g * kD + ch : (long)p.Hqk * kD + (long)g * kD + ch;
        const uint16_t x = isq ? p.q[((long)b * p.Hqk + g) * kD + ch]
                               : p.k[((long)b * p.Hqk + g) * kD + ch];
        float z = conv_channel(p, b, C_tot, c, x);
        float ss = wave_sum(z * z);
        if (lane == 0) s_red[wave] = ss;
        __syncthreads();
        float tot = isq ? s_red[0] + s_red[1] : s_red[2] + s_red[3];
        z *= rsqrtf(tot + 1e-6f);
        if (isq) s_q[ch] = z; else s_k[ch] = z;
    }
    // v channels of the G V heads, and the gates
    for (int i = t; i < G * kD; i += kThreads) {
        const int j = i / kD, ch = i % kD;
        const int h = g * G + j;
        const long c = 2L * p.Hqk * kD + (long)h * kD + ch;
        s_v[j][ch] = conv_channel(p, b, C_tot, c, p.v[((long)b * p.Hv + h) * kD + ch]);
    }
    if (t < G) {
        const int h = g * G + t;
        const float av = p.a[(long)b * p.Hv + h], bv = p.b[(long)b * p.Hv + h];
        s_alpha[t] = __expf(-p.gate_scale * softplus_f(av));
        s_beta[t] = sigmoid_f(bv);
    }
    __syncthreads();
    if (wave == 0) {
        float kq = s_k[lane] * s_q[lane] + s_k[lane + 64] * s_q[lane + 64];
        kq = wave_sum(kq);
        if (lane == 0) s_kq = kq;
    }

    // ---- state streaming: thread owns columns 4cg..4cg+3, rows rg + 8i
    const int cg = t & 31, rg = t >> 5;
    const long head0 = ((long)b * p.Hv + (long)g * G) * kD * kD;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(p.state_in + head0) + rg * 32 + cg;
    f32x4 *dst = reinterpret_cast<f32x4 *>(p.state_out + head0) + rg * 32 + cg;

    f32x4 cur[16], nxt[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) cur[i] = __builtin_nontemporal_load(src + i * 256);

    for (int j = 0; j < G; ++j) {
        f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float kr = s_k[rg + 8 * i], qr = s_q[rg + 8 * i];
            pk += cur[i] * kr;
            pq += cur[i] * qr;
        }
        s_part[j & 1][rg][cg][0] = pk;
        s_part[j & 1][rg][cg][1] = pq;
        if (j + 1 < G) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                nxt[i] = __builtin_nontemporal_load(src + (long)(j + 1) * (kD * kD / 4) + i * 256);
        }
        __syncthreads();
        f32x4 PK = {0.f, 0.f, 0.f, 0.f}, PQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            PK += s_part[j & 1][r][cg][0];
            PQ += s_part[j & 1][r][cg][1];
        }
        const float al = s_alpha[j], be = s_beta[j], kq = s_kq;
        f32x4 u, ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[e] = be * (s_v[j][4 * cg + e] - al * PK[e]);
            ov[e] = (al * PQ[e] + u[e] * kq) * p.q_scale;
        }
        f32x4 *d = dst + (long)j * (kD * kD / 4);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float kr = s_k[rg + 8 * i];
            __builtin_nontemporal_store(cur[i] * al + u * kr, d + i * 256);
        }
        if (rg == 0) {
            uint2 packed;
            packed.x = pack_bf16x2(ov[0], ov[1]);
            packed.y = pack_bf16x2(ov[2], ov[3]);
            *reinterpret_cast<uint2 *>(p.o + ((long)b * p.Hv + g * G + j) * kD + 4 * cg) = packed;
        }
        if (j + 1 < G) {
#pragma unroll
            for (int i = 0; i < 16; ++i) cur[i] = nxt[i];
        }
    }
}

}  // namespace

int max_decode_group() { return kMaxG; }

hipError_t launch_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                         const float *b, const uint16_t *conv_w, uint16_t *conv_state,
                         const float *state_in, float *state_out, uint16_t *o, int B, int Hqk,
                         int Hv, float gate_scale, float q_scale, hipStream_t stream)
{
    DecodeArgs p{q, k, v, a, b, conv_w, conv_state, state_in, state_out, o,
                 B, Hqk, Hv, gate_scale, q_scale};
    const long grid = (long)B * Hqk;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
