// gdn_decode.hip -- decode steps of the GDN mixer on gfx950: T = 1..4 new
// tokens for each of B sequences, the state read once and written once.
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
// over the old state, and the new state follows in the same pass.  Several
// tokens unroll the same way (decode_tokens_kernel).
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

// T = 2..4 tokens per sequence in one pass over the state, on the fp32
// matrix cores.  With S_0 the state before the step, A_i the product of the
// decays of tokens 0..i and r_ji that of tokens j+1..i, the one-token update
// unrolls (the chunk form of the local-inference walkthrough, section 2.1,
// for one chunk of T tokens) to
//   alpha_i S_{i-1}^T k_i = A_i S_0^T k_i + sum_{j<i}  r_ji (k_j . k_i) u_j
//   u_i = beta_i (v_i - alpha_i S_{i-1}^T k_i)
//   o_i = S_i^T q_i       = A_i S_0^T q_i + sum_{j<=i} r_ji (k_j . q_i) u_j
//   S_{T-1} = A_{T-1} S_0 + sum_j r_j,T-1 k_j u_j^T
// so one product [k_0..k_3 q_0..q_3]^T S_0 gives all that the tokens need of
// the old state, the tokens themselves need only a few scalars per state
// column, and the new state is S_0 scaled plus one rank-T product.  Wave w
// holds rows 64 (w / 2) + 4 s + lq (s < 16) of columns 64 (w % 2) + 4 lr ..
// + 3, lane = 16 lq + lr, as one 16-byte piece per s.  Element e of piece s
// is the B operand of step s of a 16x16x4 product over the wave's rows for
// the columns 64 (w % 2) + 4 c + e, c < 16; and pieces 4 tt .. 4 tt + 3 hold,
// element e, the accumulator tile of rows 64 (w / 2) + 16 tt + 4 i + q
// (tile row 4 q + i) of those columns, which the rank-T product updates in
// place.  So the state is loaded and stored in 256-byte runs and is never
// exchanged between lanes.  One workgroup per (sequence, V head): q^ and k^
// of the head's QK group come from the conv rows as they were before the
// step, which stay untouched here; only the workgroup's own v channels are
// shifted in place, and conv_shift_qk_kernel shifts the q and k rows
// afterwards (same stream).
template <int TM>
// Five waves per SIMD (96 registers, five workgroups per CU): the state's
// loads are issued after the prologue, whose registers are free by then, so
// that nothing spills; the other workgroups' streams cover their latency.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(5, 5))) void decode_tokens_kernel(DecodeArgs p)
{
    constexpr int kXS = kD + 4;     // s_x row stride: the A reads of a step hit distinct banks
    __shared__ float s_x[8][kXS];   // k^_0..k^_3, q^_0..q^_3 (zero beyond T)
    __shared__ float s_v[TM][kD];
    __shared__ float s_red[TM][4];
    __shared__ float s_ab[TM][2];
    __shared__ float s_g[2][4][4];  // k^_j . k^_i and k^_j . q^_i
    __shared__ float s_P[2][8][kD]; // [row half][x][column]: the halves of x^T S_0
    __shared__ float s_u[4][kD];    // r_j,T-1 u_j (zero beyond T)

    const int t = threadIdx.x;
    const int h = blockIdx.x % p.Hv;
    const int b = blockIdx.x / p.Hv;
    const int row = pool_row(p, b);
    if (row < 0) return;  // slot out of range: the sequence is skipped
    const int g = h / (p.Hv / p.Hqk);
    const int T = p.T;
    const long C_tot = 2L * p.Hqk * kD + (long)p.Hv * kD;
    const int lane = t & 63, wave = t >> 6, lq = lane >> 4, lr = lane & 15;
    const int r0 = 64 * (wave >> 1), c0 = 64 * (wave & 1);

    const long piece0 = ((long)row * p.Hv + h) * kD * kD + (long)(r0 + lq) * kD + c0 + 4 * lr;

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
            s_x[(isq ? 4 : 0) + i][ch] = z[i];
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
    // the state
    f32x4 st[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
        st[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p.state_in + piece0 + 4L * s * kD));
    __syncthreads();
    if (t < kD) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            s_x[4 + i][t] *= rsqrtf(s_red[i][0] + s_red[i][1] + 1e-6f);
            s_x[i][t] *= rsqrtf(s_red[i][2] + s_red[i][3] + 1e-6f);
        }
    }
    __syncthreads();
    // the Gram scalars k^_j . k^_i and k^_j . q^_i, eight lanes each
    {
        const int pr = t >> 3, part = t & 7, kind = pr >> 4, j = (pr >> 2) & 3, i = pr & 3;
        const float *xa = s_x[j], *xb = s_x[4 * kind + i];
        float acc = 0.f;
#pragma unroll
        for (int n = 0; n < 16; ++n) acc += xa[part + 8 * n] * xb[part + 8 * n];
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        acc += __shfl_xor(acc, 4, 64);
        if (part == 0) s_g[kind][j][i] = acc;
    }
    // x^T S_0 over the wave's 64 rows: lane (lq, lr) supplies x_lr (lr < 8)
    // at row r0 + 4 s + lq and the state at that row, column c0 + 4 lr + e;
    // it receives x_(4 lq + i) . S_0[rows][c0 + 4 lr + e] as element i of D[e]
    f32x4 D[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) D[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const float xa = lr < 8 ? s_x[lr][r0 + 4 * s + lq] : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) D[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, st[s][e], D[e], 0, 0, 0);
    }
    if (lq < 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_P[wave >> 1][4 * lq + i][c0 + 4 * lr + e] = D[e][i];
    }
    __syncthreads();
    // ---- the tokens in order, one state column per thread
    float al[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) al[i] = i < T ? s_ab[i][0] : 1.f;
    if (t < kD) {
        float u[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            u[i] = 0.f;
            if (i >= T) continue;
            float A = al[0];
#pragma unroll
            for (int l = 1; l <= i; ++l) A *= al[l];
            float c = A * (s_P[0][i][t] + s_P[1][i][t]);
            float o = A * (s_P[0][4 + i][t] + s_P[1][4 + i][t]);
#pragma unroll
            for (int j = 0; j < i; ++j) {
                float r = 1.f;
#pragma unroll
                for (int l = j + 1; l <= i; ++l) r *= al[l];
                c += r * s_g[0][j][i] * u[j];
                o += r * s_g[1][j][i] * u[j];
            }
            u[i] = s_ab[i][1] * (s_v[i][t] - c);
            o += s_g[1][i][i] * u[i];
            p.o[(((long)b * T + i) * p.Hv + h) * kD + t] = (uint16_t)f32_to_bf16(o * p.q_scale);
        }
#pragma unroll
        for (int j = 0; j < TM; ++j) {
            float r = 1.f;
#pragma unroll
            for (int l = j + 1; l < TM; ++l) r *= al[l];
            s_u[j][t] = r * u[j];
        }
    }
    __syncthreads();
    // ---- S' = A_(T-1) S_0 + sum_j r_j,T-1 k_j u_j^T, tile by tile in place
    float AT = al[0];
#pragma unroll
    for (int l = 1; l < TM; ++l) AT *= al[l];
    float ub[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ub[e] = s_u[lq][c0 + 4 * lr + e];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const float ka = s_x[lq][r0 + 16 * tt + 4 * (lr & 3) + (lr >> 2)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f32x4 c = {st[4 * tt][e] * AT, st[4 * tt + 1][e] * AT, st[4 * tt + 2][e] * AT, st[4 * tt + 3][e] * AT};
            c = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, ub[e], c, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) st[4 * tt + i][e] = c[i];
        }
    }
#pragma unroll
    for (int s = 0; s < 16; ++s)
        __builtin_nontemporal_store(st[s], reinterpret_cast<f32x4 *>(p.state_out + piece0 + 4L * s * kD));
}

// One token per sequence: a persistent workgroup walks the (sequence, V head)
// items blockIdx.x, blockIdx.x + gridDim.x, ..., and requests the next item's
// state into a second set of registers while it works on the current one, so
// that state loads stay in flight through the prologue and the update (a
// one-item workgroup leaves HBM idle while it computes).  Two workgroups per
// CU.
__device__ __forceinline__ void decode_one(const DecodeArgs &p, int item, int row, f32x4 (&st)[16],
                                           f32x4 (&sn)[16], int next_item, int next_row, float *s_q, float *s_k,
                                           float *s_v, float *s_red, float *s_ab, float *s_kq,
                                           f32x4 (*s_part)[8][32])
{
    const int t = threadIdx.x;
    const int h = item % p.Hv;
    const int b = item / p.Hv;
    const int g = h / (p.Hv / p.Hqk);
    const long C_tot = 2L * p.Hqk * kD + (long)p.Hv * kD;
    const int lane = t & 63, wave = t >> 6;
    const int cg = t & 31, rg = t >> 5;
    f32x4 *dst = reinterpret_cast<f32x4 *>(p.state_out + ((long)row * p.Hv + h) * kD * kD) + rg * 32 + cg;

    // ---- prologue loads: q_g (threads 0..127) and k_g (128..255) from the
    //      read-only conv rows; v_h (threads 0..127); the gates
    const bool isq = t < kD;
    const int ch = t & (kD - 1);
    const long c = isq ? (long)g * kD + ch : (long)p.Hqk * kD + (long)g * kD + ch;
    const uint16_t *cs = p.conv_state + (long)row * 3 * C_tot + c;
    uint16_t win[4];
    win[0] = cs[0];
    win[1] = cs[C_tot];
    win[2] = cs[2 * C_tot];
    win[3] = (isq ? p.q : p.k)[((long)b * p.Hqk + g) * kD + ch];
    const long cv = 2L * p.Hqk * kD + (long)h * kD + ch;
    uint16_t *csv = p.conv_state + (long)row * 3 * C_tot + cv;
    uint16_t wv[4];
    float av = 0.f, bv = 0.f;
    if (isq) {
        wv[0] = csv[0];
        wv[1] = csv[C_tot];
        wv[2] = csv[2 * C_tot];
        wv[3] = p.v[((long)b * p.Hv + h) * kD + ch];
    } else if (ch == 0) {
        av = p.a[(long)b * p.Hv + h];
        bv = p.b[(long)b * p.Hv + h];
    }
    // ---- the next item's state, after the prologue loads (loads complete in
    //      order, so waiting for the prologue does not wait for these)
    if (next_row >= 0) {
        const f32x4 *srcn = reinterpret_cast<const f32x4 *>(p.state_in + ((long)next_row * p.Hv + next_item % p.Hv) *
                                                                            kD * kD) + rg * 32 + cg;
#pragma unroll
        for (int i = 0; i < 16; ++i) sn[i] = __builtin_nontemporal_load(srcn + i * 256);
    }
    {
        float z[1];
        conv_tokens<1>(win, p.conv_w + c * 4, 1, z);
        const float ss = wave_sum(z[0] * z[0]);
        if (lane == 0) s_red[wave] = ss;
        if (isq) s_q[ch] = z[0]; else s_k[ch] = z[0];
        if (isq) {
            float zv[1];
            conv_tokens<1>(wv, p.conv_w + cv * 4, 1, zv);
            s_v[ch] = zv[0];
            // the last three raw rows become the carried rows
            csv[0] = wv[1];
            csv[C_tot] = wv[2];
            csv[2 * C_tot] = wv[3];
        } else if (ch == 0) {
            s_ab[0] = __expf(-p.gate_scale * softplus_f(av));
            s_ab[1] = sigmoid_f(bv);
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
        if (lane == 0) s_kq[0] = kq;
    }
    // ---- S^T k^ and S^T q^, the output and the new state
    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float kr = s_k[rg + 8 * r], qr = s_q[rg + 8 * r];
        pk += st[r] * kr;
        pq += st[r] * qr;
    }
    s_part[0][rg][cg] = pk;
    s_part[1][rg][cg] = pq;
    __syncthreads();
    f32x4 PK = {0.f, 0.f, 0.f, 0.f}, PQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        PK += s_part[0][r][cg];
        PQ += s_part[1][r][cg];
    }
    const float al = s_ab[0], be = s_ab[1], kq = s_kq[0];
    f32x4 u, ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        u[e] = be * (s_v[4 * cg + e] - al * PK[e]);
        ov[e] = (al * PQ[e] + u[e] * kq) * p.q_scale;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) __builtin_nontemporal_store(st[r] * al + u * s_k[rg + 8 * r], dst + r * 256);
    if (rg == 0) {
        uint2 packed;
        packed.x = pack_bf16x2(ov[0], ov[1]);
        packed.y = pack_bf16x2(ov[2], ov[3]);
        *reinterpret_cast<uint2 *>(p.o + ((long)b * p.Hv + h) * kD + 4 * cg) = packed;
    }
    __syncthreads();  // the next item rewrites the LDS arrays
}

__global__ __launch_bounds__(kThreads, 2) void decode_persist_kernel(DecodeArgs p)
{
    __shared__ float s_q[kD], s_k[kD], s_v[kD];
    __shared__ float s_red[4];
    __shared__ float s_ab[2];
    __shared__ float s_kq[1];
    __shared__ f32x4 s_part[2][8][32];  // [k^/q^ partial][row group][col group]: a wave's 16-byte
                                        // accesses are consecutive (no bank conflicts)

    const int items = p.B * p.Hv;
    const int t = threadIdx.x, cg = t & 31, rg = t >> 5;
    int item = blockIdx.x;
    if (item >= items) return;
    int row = pool_row(p, item / p.Hv);
    f32x4 st[16], sn[16];
    if (row >= 0) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(p.state_in + ((long)row * p.Hv + item % p.Hv) * kD * kD) +
                           rg * 32 + cg;
#pragma unroll
        for (int i = 0; i < 16; ++i) st[i] = __builtin_nontemporal_load(src + i * 256);
    }
    for (; item < items; item += gridDim.x) {
        const int next = item + gridDim.x;
        const int next_row = next < items ? pool_row(p, next / p.Hv) : -1;
        if (row >= 0)  // else the slot lies outside the pool: the sequence is skipped
            decode_one(p, item, row, st, sn, next, next_row, s_q, s_k, s_v, s_red, s_ab, s_kq, s_part);
        else if (next_row >= 0) {
            const f32x4 *srcn = reinterpret_cast<const f32x4 *>(p.state_in + ((long)next_row * p.Hv + next % p.Hv) *
                                                                                kD * kD) + rg * 32 + cg;
#pragma unroll
            for (int i = 0; i < 16; ++i) sn[i] = __builtin_nontemporal_load(srcn + i * 256);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) st[i] = sn[i];
        row = next_row;
    }
}

// The in-place shift of the q and k conv rows, after the decode kernel has
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
    if (T == 1) {
        // persistent: two workgroups per CU, each walking items gridDim apart
        int dev = 0, cus = 0;
        hipError_t e0 = hipGetDevice(&dev);
        if (e0 == hipSuccess) e0 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e0 != hipSuccess) return e0;
        const unsigned pg = (unsigned)(grid < 2L * cus ? grid : 2L * cus);
        hipLaunchKernelGGL(decode_persist_kernel, dim3(pg), dim3(kThreads), 0, stream, p);
    } else {
        hipLaunchKernelGGL(decode_tokens_kernel<kMaxDecodeTokens>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (T == 1)
        hipLaunchKernelGGL(conv_shift_qk_kernel<1>, shift_grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(conv_shift_qk_kernel<kMaxDecodeTokens>, shift_grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gdn
