// gdn_decode.hip -- decode steps of the GDN mixer on gfx950: T = 1..4 new
// tokens for each of B sequences, the state read once, advanced token by
// token in registers and written once.
//
// The work is streaming every (sequence, V head) state once from HBM and once
// back (64 KiB each way per head at d = 128), with a few hundred flops per
// state column and token, so the kernel is HBM-bound and is laid out for
// coalesced 16-byte accesses and few bytes of traffic beyond the state.
//
// The state update of the local-inference walkthrough (section 2.1) for one
// token, with p = alpha S^T k^ and u = beta (v^ - p):
//     S' = alpha S + k^ u^T,      o = S'^T q^ = alpha S^T q^ + u (k^ . q^)
// so both reductions over the d_k rows (S^T k^ and S^T q^) come from one pass
// over the old state, and the new state follows in the same pass.
//
// Sequences may address their state and conv rows through a slot table (a
// serving engine's state cache): sequence b then reads and writes row
// slots[b] of the pools.
#include "gdn_common.h"

namespace gdn {

namespace {

constexpr int kThreads = 256;

struct DecodeArgs {
    const uint16_t *q, *k, *v;  // [B][T][Hqk|Hv][d]
    const float *a, *b;         // [B][T][Hv]
    const uint16_t *conv_w;
    uint16_t *conv_state;       // [rows][3][C_tot]
    const float *state_in;      // [rows][Hv][d][d]
    float *state_out;
    uint16_t *o;                // [B][T][Hv][d]
    const int32_t *slots;       // [B] pool row of each sequence, or NULL: row b
    int n_rows;                 // rows in the pools (slots must lie in [0, n_rows))
    int B, T, Hqk, Hv;
    float gate_scale, q_scale;
};

__device__ __forceinline__ int pool_row(const DecodeArgs &p, int b)
{
    if (!p.slots) return b;
    const int r = p.slots[b];
    return (r >= 0 && r < p.n_rows) ? r : -1;
}

// Conv (width 4, tap 3 = current token) + SiLU of one channel over its three
// carried rows and the step's T new values: z[t] for t < T.  hist: the three
// raw rows (oldest first), x: the new raw values.
template <int TM>
__device__ __forceinline__ void conv_tokens(const uint16_t (&win)[3 + TM], const uint16_t *w4, int T, float (&z)[TM])
{
    const uint2 w = *reinterpret_cast<const uint2 *>(w4);
    const float w0 = bf16_lo(w.x), w1 = bf16_hi(w.x), w2 = bf16_lo(w.y), w3 = bf16_hi(w.y);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const float y = w0 * bf16_to_f32(win[t]) + w1 * bf16_to_f32(win[t + 1]) + w2 * bf16_to_f32(win[t + 2]) +
                        w3 * bf16_to_f32(win[t + 3]);
        z[t] = t < T ? silu_f(y) : 0.f;
    }
}

// One workgroup per (sequence b, V head h), so that each streams a single
// 64 KiB state (many short workgroups keep more of HBM busy than a few long
// ones).  q^ and k^ of the head's QK group are computed by each of the group's
// workgroups from the conv rows as they were before the step, which stay
// untouched here; only the workgroup's own v channels are shifted in place,
// and conv_shift_qk_kernel shifts the q and k rows afterwards (same stream).
// TM: tokens the kernel is built for (the step has T <= TM)
template <int TM>
__global__ __launch_bounds__(kThreads) void decode_head_kernel(DecodeArgs p)
{
    __shared__ float s_q[TM][kD], s_k[TM][kD], s_v[TM][kD];
    __shared__ float s_red[TM][4];
    __shared__ float s_ab[TM][2];
    __shared__ float s_kq[TM];
    __shared__ f32x4 s_part[2][8][32][2];  // [buffer][row group][col group][k^/q^ partial]

    const int t = threadIdx.x;
    const int h = blockIdx.x % p.Hv;
    const int b = blockIdx.x / p.Hv;
    const int row = pool_row(p, b);
    if (row < 0) return;  // slot out of range: the sequence is skipped
    const int g = h / (p.Hv / p.Hqk);
    const int T = TM == 1 ? 1 : p.T;
    const long C_tot = 2L * p.Hqk * kD + (long)p.Hv * kD;
    const int lane = t & 63, wave = t >> 6;

    // the state is requested first, so that its latency covers the prologue:
    // thread owns columns 4cg..4cg+3, rows rg + 8i
    const int cg = t & 31, rg = t >> 5;
    const long head0 = ((long)row * p.Hv + h) * kD * kD;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(p.state_in + head0) + rg * 32 + cg;
    f32x4 *dst = reinterpret_cast<f32x4 *>(p.state_out + head0) + rg * 32 + cg;
    f32x4 st[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = __builtin_nontemporal_load(src + i * 256);

    // ---- prologue: q_g (threads 0..127) and k_g (128..255) from read-only
    //      conv rows; v_h (threads 0..127) with its in-place shift; the gates
    {
        const bool isq = t < kD;
        const int ch = t & (kD - 1);
        const long c = isq ? (long)g * kD + ch : (long)p.Hqk * kD + (long)g * kD + ch;
        const uint16_t *cs = p.conv_state + (long)row * 3 * C_tot + c;
        uint16_t win[3 + TM];
        win[0] = cs[0];
        win[1] = cs[C_tot];
        win[2] = cs[2 * C_tot];
        const uint16_t *x = (isq ? p.q : p.k) + ((long)b * T * p.Hqk + g) * kD + ch;
#pragma unroll
        for (int i = 0; i < TM; ++i) win[3 + i] = i < T ? x[(long)i * p.Hqk * kD] : 0;
        float z[TM];
        conv_tokens<TM>(win, p.conv_w + c * 4, T, z);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const float ss = wave_sum(z[i] * z[i]);
            if (lane == 0) s_red[i][wave] = ss;
            if (isq) s_q[i][ch] = z[i]; else s_k[i][ch] = z[i];
        }
        if (isq) {
            const long cv = 2L * p.Hqk * kD + (long)h * kD + ch;
            uint16_t *csv = p.conv_state + (long)row * 3 * C_tot + cv;
            uint16_t wv[3 + TM];
            wv[0] = csv[0];
            wv[1] = csv[C_tot];
            wv[2] = csv[2 * C_tot];
            const uint16_t *xv = p.v + ((long)b * T * p.Hv + h) * kD + ch;
#pragma unroll
            for (int i = 0; i < TM; ++i) wv[3 + i] = i < T ? xv[(long)i * p.Hv * kD] : 0;
            float zv[TM];
            conv_tokens<TM>(wv, p.conv_w + cv * 4, T, zv);
#pragma unroll
            for (int i = 0; i < TM; ++i) s_v[i][ch] = zv[i];
            // the last three raw rows become the carried rows
            csv[0] = wv[T];
            csv[C_tot] = wv[T + 1];
            csv[2 * C_tot] = wv[T + 2];
        } else if (ch < T) {
            const long ab = ((long)b * T + ch) * p.Hv + h;
            s_ab[ch][0] = __expf(-p.gate_scale * softplus_f(p.a[ab]));
            s_ab[ch][1] = sigmoid_f(p.b[ab]);
        }
    }
    __syncthreads();
    if (t < kD) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            s_q[i][t] *= rsqrtf(s_red[i][0] + s_red[i][1] + 1e-6f);
            s_k[i][t] *= rsqrtf(s_red[i][2] + s_red[i][3] + 1e-6f);
        }
    }
    __syncthreads();
    if (wave < T) {
        float kq = s_k[wave][lane] * s_q[wave][lane] + s_k[wave][lane + 64] * s_q[wave][lane + 64];
        kq = wave_sum(kq);
        if (lane == 0) s_kq[wave] = kq;
    }

    // ---- the tokens in order, the state in registers
    for (int i = 0; i < T; ++i) {
        f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float kr = s_k[i][rg + 8 * r], qr = s_q[i][rg + 8 * r];
            pk += st[r] * kr;
            pq += st[r] * qr;
        }
        // (the same summation order as the single-token build)
        s_part[i & 1][rg][cg][0] = pk;
        s_part[i & 1][rg][cg][1] = pq;
        __syncthreads();
        f32x4 PK = {0.f, 0.f, 0.f, 0.f}, PQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            PK += s_part[i & 1][r][cg][0];
            PQ += s_part[i & 1][r][cg][1];
        }
        const float al = s_ab[i][0], be = s_ab[i][1], kq = s_kq[i];
        f32x4 u, ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[e] = be * (s_v[i][4 * cg + e] - al * PK[e]);
            ov[e] = (al * PQ[e] + u[e] * kq) * p.q_scale;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = st[r] * al + u * s_k[i][rg + 8 * r];
        if (rg == 0) {
            uint2 packed;
            packed.x = pack_bf16x2(ov[0], ov[1]);
            packed.y = pack_bf16x2(ov[2], ov[3]);
            *reinterpret_cast<uint2 *>(p.o + (((long)b * T + i) * p.Hv + h) * kD + 4 * cg) = packed;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) __builtin_nontemporal_store(st[r], dst + r * 256);
}

// ---- one token, no slot table: the lean build the single-step entry point
//      uses (fewest registers, so the most resident waves for the stream)

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

__device__ __forceinline__ float conv_channel_ro(const DecodeArgs &p, int b, long C_tot, long c, uint16_t x)
{
    const uint16_t *cs = p.conv_state + (long)b * 3 * C_tot + c;
    const uint2 w = *reinterpret_cast<const uint2 *>(p.conv_w + c * 4);
    const float y = bf16_lo(w.x) * bf16_to_f32(cs[0]) + bf16_hi(w.x) * bf16_to_f32(cs[C_tot]) +
                    bf16_lo(w.y) * bf16_to_f32(cs[2 * C_tot]) + bf16_hi(w.y) * bf16_to_f32(x);
    return silu_f(y);
}

__global__ __launch_bounds__(kThreads) void decode_step_kernel(DecodeArgs p)
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
// read them: the last three of (r0, r1, r2, x_0 .. x_{T-1}) become the rows,
// two channels per thread.
template <int TM>
__global__ __launch_bounds__(kThreads) void conv_shift_qk_kernel(DecodeArgs p)
{
    const long nqk = 2L * p.Hqk * kD;  // q and k channels per sequence
    const long C_tot = nqk + (long)p.Hv * kD;
    const long i = ((long)blockIdx.x * kThreads + threadIdx.x) * 2;
    if (i >= (long)p.B * nqk) return;
    const int b = (int)(i / nqk);
    const int row = pool_row(p, b);
    if (row < 0) return;
    const long c = i % nqk;  // q channels first, then k
    const long qk = (long)p.Hqk * kD;
    const int T = p.T;
    const uint16_t *x = c < qk ? p.q + (long)b * T * qk + c : p.k + (long)b * T * qk + (c - qk);
    uint32_t *cs = reinterpret_cast<uint32_t *>(p.conv_state + (long)row * 3 * C_tot + c);
    uint32_t win[3 + TM];
    win[0] = cs[0];
    win[1] = cs[C_tot / 2];
    win[2] = cs[C_tot];
#pragma unroll
    for (int j = 0; j < TM; ++j)
        win[3 + j] = j < T ? *reinterpret_cast<const uint32_t *>(x + (long)j * qk) : 0u;
    cs[0] = win[T];
    cs[C_tot / 2] = win[T + 1];
    cs[C_tot] = win[T + 2];
}

}  // namespace

hipError_t launch_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                         const float *b, const uint16_t *conv_w, uint16_t *conv_state,
                         const float *state_in, float *state_out, uint16_t *o, const int32_t *slots,
                         int n_rows, int B, int T, int Hqk, int Hv, float gate_scale, float q_scale,
                         hipStream_t stream)
{
    DecodeArgs p{q, k, v, a, b, conv_w, conv_state, state_in, state_out, o, slots, n_rows,
                 B, T, Hqk, Hv, gate_scale, q_scale};
    if ((long)B * Hqk == 0 || T == 0) return hipSuccess;
    const long grid = (long)B * Hv;
    const long pairs = (long)B * Hqk * kD;  // 2 * Hqk * kD channels, two per thread
    const dim3 shift_grid((unsigned)((pairs + kThreads - 1) / kThreads));
    // a single token takes a lean build (fewer registers, more resident waves)
    if (T == 1 && !slots)
        hipLaunchKernelGGL(decode_step_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    else if (T == 1)
        hipLaunchKernelGGL(decode_head_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(decode_head_kernel<kMaxDecodeTokens>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (T == 1)
        hipLaunchKernelGGL(conv_shift_qk_kernel<1>, shift_grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(conv_shift_qk_kernel<kMaxDecodeTokens>, shift_grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
