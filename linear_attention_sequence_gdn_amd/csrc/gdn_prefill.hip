// gdn_prefill.hip -- chunked prefill of the GDN mixer on gfx950.
//
// The state update of the local-inference walkthrough (section 2.1) is
// evaluated in its chunk-parallel (WY) form, which the same section names as
// the way the method becomes GPU-friendly.  Per chunk of n <= 64 tokens of one
// (sequence, V head), with in-chunk log decays gam_i = sum_{j<=i} log alpha_j,
// Gam = e^gam and D_ij = e^{gam_i - gam_j}:
//
//   A    = strict_lower( diag(beta) (K K^T) * D )          (n x n)
//   T'   = (I + A)^-1 diag(beta)
//   W    = T' diag(Gam) K,   U' = T' V                     (n x d)
//   Vnew = U' - W S                                        (S: state entering)
//   O    = diag(Gam) Q S + (Q K^T * D, lower incl. diag) Vnew
//   S   <- Gam_n S + (diag(Gam_n / Gam) K)^T Vnew
//
// which equals the token-by-token recurrence up to rounding order.
//
// Three launches:
//   setup  -- chunk and sequence tables from cu_seqlens (device-side, no host
//             sync), longest sequences first;
//   prep   -- fully parallel over (chunk, QK group): conv + SiLU, L2 norm,
//             gates, K K^T and K Q^T on the matrix cores, the blocked
//             unit-lower-triangular inverse, W and U' on the matrix cores;
//             writes every operand the sequential pass needs in the register
//             order of the matrix-core instruction that consumes it;
//   chain  -- sequential over the chunks of a sequence, parallel over
//             (sequence, V head, 16-column slice of the state): the columns
//             of S evolve independently, so each wave carries a 128 x 16
//             fp32 slice of S in registers through the whole sequence with no
//             synchronisation at all.
#include "gdn_prefill.h"

namespace gdn {

namespace {

constexpr int kPrepThreads = 256;
constexpr int kQ_LD = 136;  // fp16 row stride of the token-major q^ / k^ tiles
constexpr int kT_LD = 72;   // fp16 row stride of 64-token rows (k^T, v^T, T')

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// operand loaders
// ---------------------------------------------------------------------------

// 16x32 fp16 operand fragment from a row-major LDS matrix M[row][k]:
// lane l takes row r0 + l%16 and contraction indices k0 + kappa(l/16, 0..7).
// Serves A operands (M = A) and B operands (M[col][k] = B[k][col]).
__device__ __forceinline__ half8 lds_frag(const _Float16 *M, int ld, int r0, int k0, int lane)
{
    const _Float16 *row = M + (r0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
    const half4 lo = *reinterpret_cast<const half4 *>(row);
    const half4 hi = *reinterpret_cast<const half4 *>(row + 16);
    half8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}

__device__ __forceinline__ uint32_t ld_pair(const uint16_t *p) { return *reinterpret_cast<const uint32_t *>(p); }

// Causal width-4 conv + SiLU of channels (2*pp, 2*pp+1) of one 128-channel
// plane, rows r0 .. r0+15 of the chunk.  x points at the chunk's first token
// (row stride ld); rows < 0 come from the previous chunk of the same sequence
// (first == false), from the carried conv rows `hist` (row stride C_tot), or
// are zero.  Rows >= n are padding and produce zeros.
__device__ __forceinline__ void conv_plane(const uint16_t *__restrict__ x, long ld, int n, bool first,
                                           const uint16_t *hist, long C_tot,
                                           const uint16_t *__restrict__ w, int pp, int r0,
                                           float (&z0)[16], float (&z1)[16])
{
    const uint2 wa = *reinterpret_cast<const uint2 *>(w + (2 * pp) * 4);
    const uint2 wb = *reinterpret_cast<const uint2 *>(w + (2 * pp + 1) * 4);
    const float a0 = bf16_lo(wa.x), a1 = bf16_hi(wa.x), a2 = bf16_lo(wa.y), a3 = bf16_hi(wa.y);
    const float b0 = bf16_lo(wb.x), b1 = bf16_hi(wb.x), b2 = bf16_lo(wb.y), b3 = bf16_hi(wb.y);
    uint32_t win[19];
#pragma unroll
    for (int i = 0; i < 19; ++i) {
        const int r = r0 - 3 + i;
        uint32_t val = 0;
        if (r >= 0) {
            if (r < n) val = ld_pair(x + (long)r * ld + 2 * pp);
        } else if (!first) {
            val = ld_pair(x + (long)r * ld + 2 * pp);
        } else if (hist) {
            val = ld_pair(hist + (long)(3 + r) * C_tot + 2 * pp);
        }
        win[i] = val;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float ya = a0 * bf16_lo(win[i]) + a1 * bf16_lo(win[i + 1]) + a2 * bf16_lo(win[i + 2]) +
                         a3 * bf16_lo(win[i + 3]);
        const float yb = b0 * bf16_hi(win[i]) + b1 * bf16_hi(win[i + 1]) + b2 * bf16_hi(win[i + 2]) +
                         b3 * bf16_hi(win[i + 3]);
        const bool valid = r0 + i < n;
        z0[i] = valid ? silu_f(ya) : 0.0f;
        z1[i] = valid ? silu_f(yb) : 0.0f;
    }
}

// ---------------------------------------------------------------------------
// setup: chunk / sequence tables
// ---------------------------------------------------------------------------
// Sequence bounds, clamped into [0, T_tot] so that a malformed cu_seqlens
// cannot send any kernel outside the caller's buffers.
__device__ __forceinline__ int seq_start(const PrefillArgs &p, int s)
{
    return p.cu_seqlens ? min(max(p.cu_seqlens[s], 0), p.T_tot) : s * p.T_uniform;
}
__device__ __forceinline__ int seq_len(const PrefillArgs &p, int s)
{
    if (!p.cu_seqlens) return p.T_uniform;
    const int t0 = seq_start(p, s);
    return min(max(p.cu_seqlens[s + 1] - t0, 0), p.T_tot - t0);
}

__global__ __launch_bounds__(1024) void setup_kernel(PrefillArgs p, Workspace ws)
{
    __shared__ int s_scan[1024];
    const int t = threadIdx.x;
    const int per = (p.N + 1023) / 1024;
    const int s0 = min(p.N, t * per), s1 = min(p.N, s0 + per);
    int local = 0;
    for (int s = s0; s < s1; ++s) local += (seq_len(p, s) + kChunk - 1) / kChunk;
    s_scan[t] = local;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int add = t >= off ? s_scan[t - off] : 0;
        __syncthreads();
        s_scan[t] += add;
        __syncthreads();
    }
    int base = s_scan[t] - local;
    const int total = s_scan[1023];
    for (int s = s0; s < s1; ++s) {
        const int L = seq_len(p, s), t0 = seq_start(p, s);
        // chunks beyond the workspace bound (only with a malformed cu_seqlens) are dropped
        const int nch = max(0, min((L + kChunk - 1) / kChunk, p.max_chunks - base));
        ws.seq_info[s] = make_int4(base, nch, t0, min(L, nch * kChunk));
        for (int j = 0; j < nch; ++j)
            ws.chunk_info[base + j] = make_int4(s, t0 + j * kChunk, min(kChunk, L - j * kChunk), j == 0);
        base += nch;
    }
    for (int c = min(total, p.max_chunks) + t; c < p.max_chunks; c += 1024) ws.chunk_info[c] = make_int4(0, 0, 0, 0);
    // longest first (ties by index): rank of each sequence
    for (int s = t; s < p.N; s += 1024) {
        const int Ls = seq_len(p, s);
        int rank = 0;
        for (int j2 = 0; j2 < p.N; ++j2) {
            const int Lj = seq_len(p, j2);
            rank += (Lj > Ls) || (Lj == Ls && j2 < s);
        }
        ws.order[rank] = s;
    }
}

// ---------------------------------------------------------------------------
// prep: everything that does not depend on the carried state
// ---------------------------------------------------------------------------
constexpr int kAL = 68;        // fp32 row stride of A (16-byte aligned rows)

// Sum over the 64 lanes of each of 16 per-lane values, by recursive halving
// (reduce-scatter): 17 lane exchanges instead of 16 separate all-reduces.
// Lanes 4r .. 4r+3 end up holding the total of value r.
__device__ __forceinline__ float reduce_scatter16(const float (&v)[16], int lane)
{
    float u[8], w4[4], w2[2];
    const bool hi32 = lane & 32, hi16 = lane & 16, hi8 = lane & 8, hi4 = lane & 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float keep = hi32 ? v[8 + i] : v[i], send = hi32 ? v[i] : v[8 + i];
        u[i] = keep + __shfl_xor(send, 32, 64);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = hi16 ? u[4 + i] : u[i], send = hi16 ? u[i] : u[4 + i];
        w4[i] = keep + __shfl_xor(send, 16, 64);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = hi8 ? w4[2 + i] : w4[i], send = hi8 ? w4[i] : w4[2 + i];
        w2[i] = keep + __shfl_xor(send, 8, 64);
    }
    float x = (hi4 ? w2[1] : w2[0]) + __shfl_xor(hi4 ? w2[0] : w2[1], 4, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 1, 64);
    return x;
}

// prepA: per (chunk, QK group) -- conv + SiLU + L2 norm of q and k, written
// as matrix-core operands: q^ and k^ token-major, k^T d-major.
__global__ __launch_bounds__(kPrepThreads) void prep_qk_kernel(PrefillArgs p, Workspace ws)
{
    __shared__ __attribute__((aligned(16))) _Float16 Qs[64 * kQ_LD];
    __shared__ __attribute__((aligned(16))) _Float16 Ks[64 * kQ_LD];
    __shared__ __attribute__((aligned(16))) _Float16 KTs[128 * kT_LD];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int c = blockIdx.x / p.Hqk, g = blockIdx.x % p.Hqk;
    const int4 ci = ws.chunk_info[c];
    const int n = ci.z;
    if (n == 0) return;  // empty chunk slot (whole workgroup)
    const int s = ci.x, t0 = ci.y;
    const bool first = ci.w != 0;
    const int Hqk = p.Hqk;
    const long C_tot = 2L * Hqk * kD + (long)p.Hv * kD;
    const uint16_t *hist = (first && p.conv_state_in) ? p.conv_state_in + (long)s * 3 * C_tot : nullptr;
    const int r0 = 16 * wave;
    {
        float z0[16], z1[16];
        const long ldqk = (long)Hqk * kD;
#pragma unroll
        for (int plane = 0; plane < 2; ++plane) {
            const long ch0 = plane == 0 ? (long)g * kD : (long)Hqk * kD + (long)g * kD;
            const uint16_t *x = (plane == 0 ? p.q : p.k) + (long)t0 * ldqk + (long)g * kD;
            conv_plane(x, ldqk, n, first, hist ? hist + ch0 : nullptr, C_tot, p.conv_w + ch0 * 4, lane, r0,
                       z0, z1);
            float ss[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) ss[i] = z0[i] * z0[i] + z1[i] * z1[i];
            const float inv_mine = rsqrtf(reduce_scatter16(ss, lane) + 1e-6f);  // row (lane >> 2)
            _Float16 *dst = plane == 0 ? Qs : Ks;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv_mine), 4 * i));
                const _Float16 h0 = (_Float16)(z0[i] * inv), h1 = (_Float16)(z1[i] * inv);
                dst[(r0 + i) * kQ_LD + 2 * lane] = h0;
                dst[(r0 + i) * kQ_LD + 2 * lane + 1] = h1;
                if (plane == 1) {
                    KTs[(2 * lane) * kT_LD + r0 + i] = h0;
                    KTs[(2 * lane + 1) * kT_LD + r0 + i] = h1;
                }
            }
        }
    }
    __syncthreads();
    const long gc = (long)c * Hqk + g;
    half8 *qf = reinterpret_cast<half8 *>(ws.qfrag + gc * kQFragBytes);
    half8 *kt = reinterpret_cast<half8 *>(ws.ktok + gc * kKTokFragBytes);
    half8 *kf = reinterpret_cast<half8 *>(ws.kfrag + gc * kKFragBytes);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        qf[(wave * 4 + kb) * 64 + lane] = lds_frag(Qs, kQ_LD, 16 * wave, 32 * kb, lane);
        kt[(wave * 4 + kb) * 64 + lane] = lds_frag(Ks, kQ_LD, 16 * wave, 32 * kb, lane);
    }
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int rt = 2 * wave + rr;
            kf[(rt * 2 + kb) * 64 + lane] = lds_frag(KTs, kT_LD, 16 * rt, 32 * kb, lane);
        }
}

// Forward substitution for column `lane` of X = (I + A)^-1, A strictly lower
// (row stride kAL): x_i = delta(i, lane) - sum_{m<i} A[i][m] x_m.  Expanded at
// compile time so that x stays in registers.
template <int I, int M0>
struct SolveDot {
    static __device__ __forceinline__ void run(float &acc, const float (&x)[64], const float *Arow)
    {
        if constexpr (M0 < I) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(Arow + M0);
            if constexpr (M0 + 0 < I) acc -= a[0] * x[M0 + 0];
            if constexpr (M0 + 1 < I) acc -= a[1] * x[M0 + 1];
            if constexpr (M0 + 2 < I) acc -= a[2] * x[M0 + 2];
            if constexpr (M0 + 3 < I) acc -= a[3] * x[M0 + 3];
            SolveDot<I, M0 + 4>::run(acc, x, Arow);
        }
    }
};
template <int I>
struct SolveRow {
    static __device__ __forceinline__ void run(float (&x)[64], const float *As, int lane)
    {
        if constexpr (I < 64) {
            float acc = I == lane ? 1.f : 0.f;
            SolveDot<I, 0>::run(acc, x, As + I * kAL);
            x[I] = acc;
            SolveRow<I + 1>::run(x, As, lane);
        }
    }
};

// prepB: per (chunk, V head) -- gates, conv + SiLU of v, K K^T and K Q^T,
// A, P, the unit-lower-triangular solve, T', U' = T' V and -W.
constexpr int kH_LD = 68;  // fp16 row stride of v^T, T', T' diag(Gam) (8-byte aligned rows)

__global__ __launch_bounds__(kPrepThreads) void prep_head_kernel(PrefillArgs p, Workspace ws)
{
    __shared__ __attribute__((aligned(16))) float As[64 * kAL];
    __shared__ __attribute__((aligned(16))) _Float16 VTs[128 * kH_LD];
    __shared__ __attribute__((aligned(16))) _Float16 Th[64 * kH_LD];
    __shared__ __attribute__((aligned(16))) _Float16 TGh[64 * kH_LD];
    __shared__ float s_gam2[64], s_beta[64];

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int q4 = lane >> 4, c16 = lane & 15;
    const int Hqk = p.Hqk, Hv = p.Hv, G = Hv / Hqk;
    // block -> (chunk, group, head in group); the G heads of one (chunk, group)
    // share an XCD, so the q^ / k^ operands they all read come from one L2
    const int bid = blockIdx.x;
    const int u = (bid / (8 * G)) * 8 + (bid & 7);
    const int j = (bid >> 3) % G;
    if (u >= p.max_chunks * Hqk) return;
    const int c = u / Hqk, g = u % Hqk;
    const int h = g * G + j;
    const int4 ci = ws.chunk_info[c];
    const int n = ci.z;
    if (n == 0) return;
    const int s = ci.x, t0 = ci.y;
    const bool first = ci.w != 0;
    const long C_tot = 2L * Hqk * kD + (long)Hv * kD;
    const uint16_t *hist = (first && p.conv_state_in) ? p.conv_state_in + (long)s * 3 * C_tot : nullptr;
    const long hc = (long)c * Hv + h, gc = (long)c * Hqk + g;
    const int r0 = 16 * wave;

    // operands from the q/k pass (straight into registers)
    const half8 *qf = reinterpret_cast<const half8 *>(ws.qfrag + gc * kQFragBytes) + lane;
    const half8 *kt = reinterpret_cast<const half8 *>(ws.ktok + gc * kKTokFragBytes) + lane;
    const half8 *kf = reinterpret_cast<const half8 *>(ws.kfrag + gc * kKFragBytes) + lane;
    half8 ktA[4][4], kOwn[4], qB[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) ktA[rt][kb] = kt[(rt * 4 + kb) * 64];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        kOwn[kb] = kt[(wave * 4 + kb) * 64];
        qB[kb] = qf[(wave * 4 + kb) * 64];
    }

    // gates (wave 0): gam = in-chunk cumulative log decay (log2 units), beta
    if (wave == 0) {
        const bool valid = lane < n;
        const long ti = (long)(t0 + lane) * Hv + h;
        const float av = valid ? p.a[ti] : 0.f, bv = valid ? p.b[ti] : 0.f;
        const float gl = valid ? -p.gate_scale * kLog2e * softplus_f(av) : 0.f;
        const float be = valid ? sigmoid_f(bv) : 0.f;
        float gam = gl;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(gam, off, 64);
            if (lane >= off) gam += y;
        }
        const float gam_n = __shfl(gam, n - 1, 64);
        s_gam2[lane] = gam;
        s_beta[lane] = be;
        // slot 0: q_scale * Gam (only the output uses it); slot 1: Gam_n / Gam; slot 2: Gam_n
        float *gt = ws.gates + hc * kGateFloats;
        gt[lane] = p.q_scale * __builtin_amdgcn_exp2f(gam);
        gt[64 + lane] = valid ? __builtin_amdgcn_exp2f(gam_n - gam) : 0.f;
        if (lane == 0) gt[128] = __builtin_amdgcn_exp2f(gam_n);
    }
    // v^ of head h: conv + SiLU -> v^T in LDS
    {
        float z0[16], z1[16];
        const long ldv = (long)Hv * kD;
        const long cv = 2L * Hqk * kD + (long)h * kD;
        const uint16_t *xv = p.v + (long)t0 * ldv + (long)h * kD;
        conv_plane(xv, ldv, n, first, hist ? hist + cv : nullptr, C_tot, p.conv_w + cv * 4, lane, r0, z0, z1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            VTs[(2 * lane) * kH_LD + r0 + i] = (_Float16)z0[i];
            VTs[(2 * lane + 1) * kH_LD + r0 + i] = (_Float16)z1[i];
        }
    }
    // K K^T (rows 16*wave.., column tiles ct <= wave) and K Q^T (query tile
    // `wave`, key tiles jt <= wave)
    f32x4 kk[4], kq[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acq = {0.f, 0.f, 0.f, 0.f};
        if (ct <= wave) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                acc = mfma16(kOwn[kb], ktA[ct][kb], acc);
                acq = mfma16(ktA[ct][kb], qB[kb], acq);
            }
        }
        kk[ct] = acc;
        kq[ct] = acq;
    }
    __syncthreads();
    // A = strict_lower(diag(beta) K K^T * D) -> LDS; P = (K Q^T)^T * D (lower) -> global
    {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            if (ct > wave) continue;
            const int jj = 16 * ct + c16;
            const float gj = s_gam2[jj];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * wave + 4 * q4 + e;
                if (i > jj) As[i * kAL + jj] = s_beta[i] * kk[ct][e] * __builtin_amdgcn_exp2f(s_gam2[i] - gj);
            }
        }
        half8 *pf = reinterpret_cast<half8 *>(ws.pfrag + hc * kPFragBytes);
        const int i = 16 * wave + c16;
        const float gi = s_gam2[i];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            half8 fr;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int jt = 2 * kb + (e >> 2);
                const int jj = 16 * jt + 4 * q4 + (e & 3);
                float val = 0.f;
                if (jt <= wave && i >= jj)
                    val = p.q_scale * kq[jt][e & 3] * __builtin_amdgcn_exp2f(gi - s_gam2[jj]);
                fr[e] = (_Float16)val;
            }
            pf[(wave * 2 + kb) * 64 + lane] = fr;
        }
    }
    __syncthreads();
    // (I + A) X = I by forward substitution (wave 0; lane = column of X, X in
    // registers), then T' = X diag(beta) and T' diag(Gam) into LDS
    if (wave == 0) {
        float x[64];
        SolveRow<0>::run(x, As, lane);
        const float bc = s_beta[lane];
        const float gcl = bc * __builtin_amdgcn_exp2f(s_gam2[lane]);
#pragma unroll
        for (int i = 0; i < 64; ++i) {
            Th[i * kH_LD + lane] = (_Float16)(x[i] * bc);
            TGh[i * kH_LD + lane] = (_Float16)(x[i] * gcl);
        }
    }
    __syncthreads();
    // U' = T' V: column tiles 2*wave, 2*wave+1; stored in accumulator order
    {
        half4 *uf = reinterpret_cast<half4 *>(ws.ufrag + hc * kUBytes);
        half8 ta[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            ta[rt][0] = lds_frag(Th, kH_LD, 16 * rt, 0, lane);
            ta[rt][1] = lds_frag(Th, kH_LD, 16 * rt, 32, lane);
        }
#pragma unroll
        for (int cti = 0; cti < 2; ++cti) {
            const int ct = 2 * wave + cti;
            const half8 b0 = lds_frag(VTs, kH_LD, 16 * ct, 0, lane);
            const half8 b1 = lds_frag(VTs, kH_LD, 16 * ct, 32, lane);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma16(ta[rt][0], b0, acc);
                if (rt >= 2) acc = mfma16(ta[rt][1], b1, acc);
                half4 hv;
                hv[0] = (_Float16)acc[0]; hv[1] = (_Float16)acc[1];
                hv[2] = (_Float16)acc[2]; hv[3] = (_Float16)acc[3];
                uf[(ct * 4 + rt) * 64 + lane] = hv;
            }
        }
    }
    // W^T = K^T diag(Gam) T'^T: token tile `wave`, all eight d tiles; -W stored as A operand
    {
        half8 *wf = reinterpret_cast<half8 *>(ws.wfrag + hc * kWFragBytes);
        const half8 b0 = lds_frag(TGh, kH_LD, 16 * wave, 0, lane);
        const half8 b1 = lds_frag(TGh, kH_LD, 16 * wave, 32, lane);
        f32x4 wt[8];
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mfma16(kf[(rt * 2 + 0) * 64], b0, acc);
            if (wave >= 2) acc = mfma16(kf[(rt * 2 + 1) * 64], b1, acc);
            wt[rt] = acc;
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) wf[(wave * 4 + kb) * 64 + lane] = pack_h8(-wt[2 * kb], -wt[2 * kb + 1]);
    }
}

// ---------------------------------------------------------------------------
// chain: the sequential state carry
// ---------------------------------------------------------------------------
// Workgroup = kChainWaves waves = one (sequence, V head) and 16*kChainWaves
// columns of its state; each wave carries a 128 x 16 fp32 slice of S in its
// accumulators through the whole sequence.  The operands of a chunk that
// every wave needs (-W, q^, k^T, P, gates) and the waves' U' tiles are
// brought into LDS with direct-to-LDS loads, double-buffered: chunk c+1 is in
// flight while chunk c is computed, with one workgroup barrier per chunk.
constexpr int kChainWaves = 2;

template <int NW>
struct ChainStage {
    static constexpr int kW = 0, kQ = 16 * 1024, kK = 32 * 1024, kP = 48 * 1024, kG = 56 * 1024,
                         kU = 57 * 1024;
    static constexpr int kBlocks = 57 + 2 * NW;  // 1-KiB blocks per stage
    static constexpr int kBytes = kBlocks * 1024;
};


// Issue the direct-to-LDS loads of chunk c into `stage`.  Every region is a
// whole number of 1-KiB blocks; wave w (uniform) moves blocks w, w+NW, ... of
// each region (lane l: bytes 16l .. 16l+15 of a block).  Buffer loads carry
// the block offset in a scalar register, so issuing costs no vector ALU work.
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t region_rsrc(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}

template <int NW, int kBlocks>
__device__ __forceinline__ void issue_region(const void *src, uint8_t *dst, int wave, int lane)
{
    const __amdgpu_buffer_rsrc_t r = region_rsrc(src);
#pragma unroll
    for (int i = 0; i < kBlocks / NW; ++i) {
        const int blk = i * NW + wave;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst + blk * 1024), 16, lane * 16, blk * 1024, 0, 0);
    }
}

template <int NW>
__device__ __forceinline__ void chain_issue(const Workspace &ws, uint8_t *stage, long c, int h, int g,
                                            int Hqk, int Hv, int cb, int wave, int lane)
{
    using St = ChainStage<NW>;
    const long hc = c * Hv + h, gc = c * Hqk + g;
    issue_region<NW, 16>(ws.wfrag + hc * kWFragBytes, stage + St::kW, wave, lane);
    issue_region<NW, 16>(ws.qfrag + gc * kQFragBytes, stage + St::kQ, wave, lane);
    issue_region<NW, 16>(ws.kfrag + gc * kKFragBytes, stage + St::kK, wave, lane);
    issue_region<NW, 8>(ws.pfrag + hc * kPFragBytes, stage + St::kP, wave, lane);
    issue_region<NW, 2 * NW>(ws.ufrag + hc * kUBytes + (long)cb * NW * 2048, stage + St::kU, wave, lane);
    if (wave == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(region_rsrc(ws.gates + hc * kGateFloats),
                                                 (lds_void_t *)(stage + St::kG), 16, lane * 16, 0, 0, 0);
}

template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chain_kernel(PrefillArgs p, Workspace ws)
{
    using St = ChainStage<NW>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * St::kBytes + NW * 2048];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int q4 = lane >> 4, c16 = lane & 15;
    const int Hqk = p.Hqk, Hv = p.Hv, G = Hv / Hqk;
    constexpr int kBlocksPerHead = 8 / NW;
    // block -> (rank, group, head-in-group, column block); all workgroups of
    // one (sequence, QK group) land on the same XCD (same L2)
    const int per_group = G * kBlocksPerHead;
    const int bid = blockIdx.x;
    const int gu = (bid / (8 * per_group)) * 8 + (bid & 7);
    const int inner = (bid >> 3) % per_group;
    if (gu >= p.N * Hqk) return;
    const int rank = gu / Hqk, g = gu % Hqk;
    const int j = inner / kBlocksPerHead, cb = inner % kBlocksPerHead;
    const int h = g * G + j;
    const int ct = cb * NW + wave;
    const int s = ws.order[rank];
    const int4 si = ws.seq_info[s];  // chunk0, nchunks, t0, L
    const int col = 16 * ct + c16;
    uint16_t *ostage = reinterpret_cast<uint16_t *>(smem + 2 * St::kBytes + wave * 2048);

    // state slice S[:, 16ct .. 16ct+15] in accumulator layout: tile rt holds rows 16rt + 4q4 + e
    f32x4 S[8];
    const long sbase = ((long)s * Hv + h) * kD * kD;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[rt][e] = p.state_in ? p.state_in[sbase + (long)(16 * rt + 4 * q4 + e) * kD + col] : 0.f;

    if (si.y > 0) chain_issue<NW>(ws, smem, si.x, h, g, Hqk, Hv, cb, wave, lane);
    for (int cc = 0; cc < si.y; ++cc) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (cc + 1 < si.y)
            chain_issue<NW>(ws, smem + ((cc + 1) & 1) * St::kBytes, si.x + cc + 1, h, g, Hqk, Hv, cb, wave, lane);
        const uint8_t *st = smem + (cc & 1) * St::kBytes;
        const half8 *Wf = reinterpret_cast<const half8 *>(st + St::kW) + lane;
        const half8 *Qf = reinterpret_cast<const half8 *>(st + St::kQ) + lane;
        const half8 *Kf = reinterpret_cast<const half8 *>(st + St::kK) + lane;
        const half8 *Pf = reinterpret_cast<const half8 *>(st + St::kP) + lane;
        const float *gt = reinterpret_cast<const float *>(st + St::kG);
        const half4 *Uf = reinterpret_cast<const half4 *>(st + St::kU) + wave * 4 * 64 + lane;
        const int n = min(kChunk, si.w - cc * kChunk);
        const int tok0 = si.z + cc * kChunk;

        // state as the B operand (fp16), contraction over d_k
        half8 Sb[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Sb[kb] = pack_h8(S[2 * kb], S[2 * kb + 1]);

        // Vnew = U' - W S ;  QS = Q S   (eight independent accumulators per
        // k-block, operands read one k-block ahead)
        f32x4 Vn[4], QS[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const half4 u = Uf[rt * 64];
            Vn[rt] = f32x4{(float)u[0], (float)u[1], (float)u[2], (float)u[3]};
            QS[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        half8 wA[4], qA[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            wA[rt] = Wf[(rt * 4) * 64];
            qA[rt] = Qf[(rt * 4) * 64];
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            half8 wN[4], qN[4];
            if (kb < 3) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    wN[rt] = Wf[(rt * 4 + kb + 1) * 64];
                    qN[rt] = Qf[(rt * 4 + kb + 1) * 64];
                }
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                Vn[rt] = mfma16(wA[rt], Sb[kb], Vn[rt]);
                QS[rt] = mfma16(qA[rt], Sb[kb], QS[rt]);
            }
            if (kb < 3) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    wA[rt] = wN[rt];
                    qA[rt] = qN[rt];
                }
            }
        }
        // Vnew as B operands: plain (for P Vnew) and scaled by Gam_n / Gam (for the state)
        half8 Vb[2], Vr[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const f32x4 r_lo = *reinterpret_cast<const f32x4 *>(gt + 64 + 32 * kb + 4 * q4);
            const f32x4 r_hi = *reinterpret_cast<const f32x4 *>(gt + 64 + 32 * kb + 16 + 4 * q4);
            Vb[kb] = pack_h8(Vn[2 * kb], Vn[2 * kb + 1]);
            Vr[kb] = pack_h8(Vn[2 * kb] * r_lo, Vn[2 * kb + 1] * r_hi);
        }
        // O = q_scale (diag(Gam) Q S + P Vnew) (q_scale is folded into Gam and
        // P), staged through LDS for 16-byte row stores
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 gam = *reinterpret_cast<const f32x4 *>(gt + 16 * rt + 4 * q4);
            f32x4 acc = QS[rt] * gam;
            acc = mfma16(Pf[(rt * 2 + 0) * 64], Vb[0], acc);
            if (rt >= 2) acc = mfma16(Pf[(rt * 2 + 1) * 64], Vb[1], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) ostage[(16 * rt + 4 * q4 + e) * 16 + c16] = (uint16_t)f32_to_bf16(acc[e]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < n) {
            const uint4 *srow = reinterpret_cast<const uint4 *>(ostage + lane * 16);
            uint4 *drow = reinterpret_cast<uint4 *>(p.o + ((long)(tok0 + lane) * Hv + h) * kD + 16 * ct);
            drow[0] = srow[0];
            drow[1] = srow[1];
        }
        // S <- Gam_n S + K^T (r * Vnew): the dependency into the next chunk,
        // last so that its matrix-core work overlaps the next chunk's wait
        const float gn = gt[128];
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) S[rt] = S[rt] * gn;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) S[rt] = mfma16(Kf[(rt * 2 + kb) * 64], Vr[kb], S[rt]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }

#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) p.state_out[sbase + (long)(16 * rt + 4 * q4 + e) * kD + col] = S[rt][e];

    // carried conv rows: the last three raw rows of the sequence (v channels of
    // head h; the first head of the group also writes the q and k channels)
    if (p.conv_state_out && cb == 0 && wave == 0) {
        const long C_tot = 2L * Hqk * kD + (long)Hv * kD;
        const int L = si.w, t0 = si.z;
        for (int plane = (j == 0 ? 0 : 2); plane < 3; ++plane) {
            const long ch0 = plane == 0 ? (long)g * kD : plane == 1 ? (long)Hqk * kD + (long)g * kD
                                                                  : 2L * Hqk * kD + (long)h * kD;
            const uint16_t *src = plane == 0 ? p.q + (long)g * kD : plane == 1 ? p.k + (long)g * kD
                                                                              : p.v + (long)h * kD;
            const long ld = plane == 2 ? (long)Hv * kD : (long)Hqk * kD;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const int tau = L - 3 + r;
                uint32_t val = 0;
                if (tau >= 0)
                    val = ld_pair(src + (long)(t0 + tau) * ld + 2 * lane);
                else if (p.conv_state_in)
                    val = ld_pair(p.conv_state_in + ((long)s * 3 + 3 + tau) * C_tot + ch0 + 2 * lane);
                *reinterpret_cast<uint32_t *>(p.conv_state_out + ((long)s * 3 + r) * C_tot + ch0 + 2 * lane) = val;
            }
        }
    }
}

}  // namespace

size_t prefill_workspace_bytes(int max_chunks, int N, int Hqk, int Hv)
{
    const size_t C = (size_t)max_chunks;
    size_t total = 0;
    total += align256(C * sizeof(int4));
    total += align256((size_t)N * sizeof(int4));
    total += align256((size_t)N * sizeof(int));
    total += align256(C * Hqk * kQFragBytes);
    total += align256(C * Hqk * kKFragBytes);
    total += align256(C * Hqk * kKTokFragBytes);
    total += align256(C * Hv * kWFragBytes);
    total += align256(C * Hv * kUBytes);
    total += align256(C * Hv * kPFragBytes);
    total += align256(C * Hv * kGateFloats * sizeof(float));
    return total;
}

Workspace carve_workspace(void *base, int max_chunks, int N, int Hqk, int Hv)
{
    const size_t C = (size_t)max_chunks;
    uint8_t *ptr = static_cast<uint8_t *>(base);
    Workspace ws;
    auto take = [&](size_t bytes) {
        uint8_t *r = ptr;
        ptr += align256(bytes);
        return r;
    };
    ws.chunk_info = reinterpret_cast<int4 *>(take(C * sizeof(int4)));
    ws.seq_info = reinterpret_cast<int4 *>(take((size_t)N * sizeof(int4)));
    ws.order = reinterpret_cast<int *>(take((size_t)N * sizeof(int)));
    ws.qfrag = take(C * Hqk * kQFragBytes);
    ws.kfrag = take(C * Hqk * kKFragBytes);
    ws.ktok = take(C * Hqk * kKTokFragBytes);
    ws.wfrag = take(C * Hv * kWFragBytes);
    ws.ufrag = take(C * Hv * kUBytes);
    ws.pfrag = take(C * Hv * kPFragBytes);
    ws.gates = reinterpret_cast<float *>(take(C * Hv * kGateFloats * sizeof(float)));
    return ws;
}

hipError_t launch_prefill(const PrefillArgs &p, void *workspace, hipStream_t stream,
                          hipEvent_t const *events)
{
    const Workspace ws = carve_workspace(workspace, p.max_chunks, p.N, p.Hqk, p.Hv);
    hipError_t e;
    auto mark = [&](int i) { return events ? hipEventRecord(events[i], stream) : hipSuccess; };
    if ((e = mark(0)) != hipSuccess) return e;
    hipLaunchKernelGGL(setup_kernel, dim3(1), dim3(1024), 0, stream, p, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = mark(1)) != hipSuccess) return e;
    if (p.max_chunks > 0) {
        const long units = (long)p.max_chunks * p.Hqk;
        hipLaunchKernelGGL(prep_qk_kernel, dim3((unsigned)units), dim3(kPrepThreads), 0, stream, p, ws);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const long blocks = ((units + 7) / 8) * 8L * (p.Hv / p.Hqk);
        hipLaunchKernelGGL(prep_head_kernel, dim3((unsigned)blocks), dim3(kPrepThreads), 0, stream, p, ws);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = mark(2)) != hipSuccess) return e;
    const int G = p.Hv / p.Hqk;
    const long groups = (long)p.N * p.Hqk;
    const long blocks = ((groups + 7) / 8) * 8L * G * (8 / kChainWaves);
    hipLaunchKernelGGL(chain_kernel<kChainWaves>, dim3((unsigned)blocks), dim3(64 * kChainWaves), 0, stream, p,
                       ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark(3);
}

}  // namespace gdn
