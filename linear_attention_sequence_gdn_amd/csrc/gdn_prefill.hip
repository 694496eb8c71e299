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

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// raw buffer resource over `base` (offsets are bounds-checked against 2^31 - 1)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t region_rsrc(const void *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, 0x7fffffff, 0x00020000);
}

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

// Raw rows r0-3 .. r0+15 of channels (2*pp, 2*pp+1) of one 128-channel plane
// for the causal width-4 conv.  x points at the chunk's first token (row
// stride ld); rows < 0 come from the previous chunk of the same sequence
// (first == false), from the carried conv rows `hist` (row stride C_tot), or
// are zero.  Rows >= n are padding and read as zero.
__device__ __forceinline__ void conv_window(const uint16_t *__restrict__ x, long ld, int n, bool first,
                                            const uint16_t *hist, long C_tot, int pp, int r0, uint32_t (&win)[19])
{
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
}

// Conv (tap 3 = current token) + SiLU over a loaded window; rows >= n give 0.
__device__ __forceinline__ void conv_silu(const uint32_t (&win)[19], const uint16_t *__restrict__ w, int pp, int r0,
                                          int n, float (&z0)[16], float (&z1)[16])
{
    const uint2 wa = *reinterpret_cast<const uint2 *>(w + (2 * pp) * 4);
    const uint2 wb = *reinterpret_cast<const uint2 *>(w + (2 * pp + 1) * 4);
    const float a0 = bf16_lo(wa.x), a1 = bf16_hi(wa.x), a2 = bf16_lo(wa.y), a3 = bf16_hi(wa.y);
    const float b0 = bf16_lo(wb.x), b1 = bf16_hi(wb.x), b2 = bf16_lo(wb.y), b3 = bf16_hi(wb.y);
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

__device__ __forceinline__ void conv_plane(const uint16_t *__restrict__ x, long ld, int n, bool first,
                                           const uint16_t *hist, long C_tot,
                                           const uint16_t *__restrict__ w, int pp, int r0,
                                           float (&z0)[16], float (&z1)[16])
{
    uint32_t win[19];
    conv_window(x, ld, n, first, hist, C_tot, pp, r0, win);
    conv_silu(win, w, pp, r0, n, z0, z1);
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
    for (int s = s0; s < s1; ++s) {
        const int L = seq_len(p, s), t0 = seq_start(p, s);
        // chunks beyond the workspace bound (only with a malformed cu_seqlens) are dropped
        const int nch = max(0, min((L + kChunk - 1) / kChunk, p.max_chunks - base));
        ws.seq_info[s] = make_int4(base, nch, t0, min(L, nch * kChunk));
        base += nch;
    }
    // chunk table, one chunk per thread: chunk c lies in the sequence range of
    // the first thread whose inclusive count exceeds c
    const int total = min(s_scan[1023], p.max_chunks);
    for (int c = t; c < p.max_chunks; c += 1024) {
        int4 info = make_int4(0, 0, 0, 0);
        if (c < total) {
            int lo = 0, hi = 1023;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_scan[mid] > c) hi = mid;
                else lo = mid + 1;
            }
            int b = lo > 0 ? s_scan[lo - 1] : 0;
            for (int s = lo * per; s < min(p.N, lo * per + per); ++s) {
                const int L = seq_len(p, s), nch = (L + kChunk - 1) / kChunk;
                if (c < b + nch) {
                    const int j = c - b;
                    info = make_int4(s, seq_start(p, s) + j * kChunk, min(kChunk, L - j * kChunk), j == 0);
                    break;
                }
                b += nch;
            }
        }
        ws.chunk_info[c] = info;
    }
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

// Forward substitution for column c of the inverse of a 16 x 16 unit
// lower-triangular block I + A (A strictly lower, row stride kAL):
// y_i = delta(i, c) - sum_{m<i} A[i][m] y_m.  Expanded at compile time so that
// y stays in registers.
template <int I, int M0>
struct SolveDot16 {
    static __device__ __forceinline__ void run(float &acc, const float (&y)[16], const float *Arow)
    {
        if constexpr (M0 < I) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(Arow + M0);
            if constexpr (M0 + 0 < I) acc -= a[0] * y[M0 + 0];
            if constexpr (M0 + 1 < I) acc -= a[1] * y[M0 + 1];
            if constexpr (M0 + 2 < I) acc -= a[2] * y[M0 + 2];
            if constexpr (M0 + 3 < I) acc -= a[3] * y[M0 + 3];
            SolveDot16<I, M0 + 4>::run(acc, y, Arow);
        }
    }
};
template <int I>
struct SolveRow16 {
    static __device__ __forceinline__ void run(float (&y)[16], const float *A, int c)
    {
        if constexpr (I < 16) {
            float acc = I == c ? 1.f : 0.f;
            SolveDot16<I, 0>::run(acc, y, A + I * kAL);
            y[I] = acc;
            SolveRow16<I + 1>::run(y, A, c);
        }
    }
};

// acc += A_blk @ B_blk for 16 x 16 fp32 blocks of row-major LDS matrices, on
// the fp32 matrix cores (four 16x16x4 steps).  Lane l supplies A[l%16][k] and
// B[k][l%16] for k = 4kb + l/16; acc is in accumulator layout.
__device__ __forceinline__ f32x4 mm16_f32(const float *Ab, int lda, const float *Bb, int ldb, f32x4 acc, int lane)
{
    const int r = lane & 15, k = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Ab[r * lda + 4 * kb + k], Bb[(4 * kb + k) * ldb + r], acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ void st16_f32(float *Db, int ldd, f32x4 v, int lane)
{
    const int c = lane & 15, q = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) Db[(4 * q + e) * ldd + c] = v[e];
}

// prepB: per (chunk, V head) -- gates, conv + SiLU of v, K K^T and K Q^T,
// A, P, the unit-lower-triangular inverse, T', U' = T' V and -W.
constexpr int kH_LD = 68;  // fp16 row stride of v^T, T', T' diag(Gam) (8-byte aligned rows)

__global__ __launch_bounds__(kPrepThreads) void prep_head_kernel(PrefillArgs p, Workspace ws)
{
    // LDS plan: [F] k^ operands (16 KiB) -> X = (I+A)^-1 (fp32) -> v^T (fp16);
    //           [A] A (fp32) -> T' and T' diag(Gam) (fp16); scratch; gates
    __shared__ __attribute__((aligned(16))) uint8_t regF[64 * kAL * 4];
    __shared__ __attribute__((aligned(16))) uint8_t regA[64 * kAL * 4];
    __shared__ __attribute__((aligned(16))) float Msc[3][256];
    __shared__ float s_gam2[64], s_beta[64], s_bg[64];
    const half8 *Fk = reinterpret_cast<const half8 *>(regF);  // k^ token-major: [rt*4+kb][lane]
    float *Xs = reinterpret_cast<float *>(regF);
    _Float16 *VTs = reinterpret_cast<_Float16 *>(regF);
    float *As = reinterpret_cast<float *>(regA);
    _Float16 *Th = reinterpret_cast<_Float16 *>(regA);
    _Float16 *TGh = Th + 64 * kH_LD;
    static_assert(128 * kH_LD * 2 <= 64 * kAL * 4, "v^T fits over X");
    static_assert(2 * 64 * kH_LD * 2 <= 64 * kAL * 4, "T' and T' diag(Gam) fit over A");

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
    const long ldv = (long)Hv * kD;
    const long cv = 2L * Hqk * kD + (long)h * kD;

    // ---- every global read of the workgroup is issued first
    {
        const __amdgpu_buffer_rsrc_t rk = region_rsrc(ws.ktok + gc * kKTokFragBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int blk = i * 4 + wave;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t *)(regF + blk * 1024), 16, lane * 16, blk * 1024, 0, 0);
        }
    }
    half8 qB[4], kT[4];
    {
        const half8 *qf = reinterpret_cast<const half8 *>(ws.qfrag + gc * kQFragBytes) + lane;
        const half8 *kf = reinterpret_cast<const half8 *>(ws.kfrag + gc * kKFragBytes) + lane;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            qB[kb] = qf[(wave * 4 + kb) * 64];
            kT[kb] = kf[(wave * 4 + kb) * 64];  // k^T row tiles 2w, 2w+1, k-blocks 0..1
        }
    }
    uint32_t vwin[19];
    conv_window(p.v + (long)t0 * ldv + (long)h * kD, ldv, n, first, hist ? hist + cv : nullptr, C_tot, lane, r0, vwin);
    float av = 0.f, bv = 0.f;
    if (wave == 0 && lane < n) {
        const long ti = (long)(t0 + lane) * Hv + h;
        av = p.a[ti];
        bv = p.b[ti];
    }

    // ---- gates (wave 0): gam = in-chunk cumulative log decay (log2 units), beta
    if (wave == 0) {
        const bool valid = lane < n;
        const float gl = valid ? -p.gate_scale * kLog2e * softplus_f(av) : 0.f;
        const float be = valid ? sigmoid_f(bv) : 0.f;
        float gam = gl;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(gam, off, 64);
            if (lane >= off) gam += y;
        }
        const float gam_n = __shfl(gam, n - 1, 64);
        const float Gam = __builtin_amdgcn_exp2f(gam);
        s_gam2[lane] = gam;
        s_beta[lane] = be;
        s_bg[lane] = be * Gam;
        // slot 0: q_scale * Gam (only the output uses it); slot 1: Gam_n / Gam; slot 2: Gam_n
        float *gt = ws.gates + hc * kGateFloats;
        gt[lane] = p.q_scale * Gam;
        gt[64 + lane] = valid ? __builtin_amdgcn_exp2f(gam_n - gam) : 0.f;
        if (lane == 0) gt[128] = __builtin_amdgcn_exp2f(gam_n);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // ---- K K^T (rows 16*wave.., column tiles ct <= wave) and K Q^T (query
    //      tile `wave`, key tiles jt <= wave)
    f32x4 kk[4], kq[4];
    {
        half8 kOwn[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) kOwn[kb] = Fk[(wave * 4 + kb) * 64 + lane];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acq = {0.f, 0.f, 0.f, 0.f};
            if (ct <= wave) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const half8 kc = Fk[(ct * 4 + kb) * 64 + lane];
                    acc = mfma16(kOwn[kb], kc, acc);
                    acq = mfma16(kc, qB[kb], acq);
                }
            }
            kk[ct] = acc;
            kq[ct] = acq;
        }
    }
    // ---- A = strict_lower(diag(beta) K K^T * D) -> LDS; P = (K Q^T)^T * D (lower) -> global
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
    // ---- X = (I + A)^-1, blocked by 16: diagonal blocks by forward
    //      substitution (wave b, block b), then the blocks below the diagonal
    //      level by level, X_ij = -X_ii sum_{k=j}^{i-1} A_ik X_kj, on the fp32
    //      matrix cores
    {
        float y[16];
        const int bo = 16 * wave;
        SolveRow16<0>::run(y, As + bo * kAL + bo, c16);
        if (lane < 16) {
#pragma unroll
            for (int i = 0; i < 16; ++i) Xs[(bo + i) * kAL + bo + c16] = y[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int lvl = 1; lvl <= 3; ++lvl) {
        if (wave < 4 - lvl) {
            const int bi = wave + lvl, bj = wave;
            f32x4 m = {0.f, 0.f, 0.f, 0.f};
            for (int bk = bj; bk < bi; ++bk)
                m = mm16_f32(As + 16 * bi * kAL + 16 * bk, kAL, Xs + 16 * bk * kAL + 16 * bj, kAL, m, lane);
            st16_f32(Msc[wave], 16, m, lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            x = mm16_f32(Xs + 16 * bi * kAL + 16 * bi, kAL, Msc[wave], 16, x, lane);
            st16_f32(Xs + 16 * bi * kAL + 16 * bj, kAL, -x, lane);
        }
        __syncthreads();
    }
    // ---- T' = X diag(beta) and T' diag(Gam) (fp16, lower) over A's storage
    {
        float tv[16], tg[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int e = t + k * kPrepThreads;
            const int i = e >> 6, jj = e & 63;
            const float xv = jj <= i ? Xs[i * kAL + jj] : 0.f;
            tv[k] = xv * s_beta[jj];
            tg[k] = xv * s_bg[jj];
        }
        __syncthreads();  // A and X are dead from here on
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int e = t + k * kPrepThreads;
            const int i = e >> 6, jj = e & 63;
            Th[i * kH_LD + jj] = (_Float16)tv[k];
            TGh[i * kH_LD + jj] = (_Float16)tg[k];
        }
    }
    // ---- v^ of head h: conv + SiLU from the window loaded at the start -> v^T over X
    {
        float z0[16], z1[16];
        conv_silu(vwin, p.conv_w + cv * 4, lane, r0, n, z0, z1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            VTs[(2 * lane) * kH_LD + r0 + i] = (_Float16)z0[i];
            VTs[(2 * lane + 1) * kH_LD + r0 + i] = (_Float16)z1[i];
        }
    }
    __syncthreads();
    // ---- U' = T' V: column tiles 2*wave, 2*wave+1; stored in accumulator order
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
    // ---- W^T = K^T diag(Gam) T'^T: d tiles 2*wave, 2*wave+1 (k-block `wave`
    //      of -W), all four token tiles; -W stored as A operand
    {
        half8 *wf = reinterpret_cast<half8 *>(ws.wfrag + hc * kWFragBytes);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const half8 b0 = lds_frag(TGh, kH_LD, 16 * ct, 0, lane);
            const half8 b1 = lds_frag(TGh, kH_LD, 16 * ct, 32, lane);
            f32x4 w2[2];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma16(kT[2 * rr + 0], b0, acc);
                if (ct >= 2) acc = mfma16(kT[2 * rr + 1], b1, acc);
                w2[rr] = acc;
            }
            wf[(ct * 4 + wave) * 64 + lane] = pack_h8(-w2[0], -w2[1]);
        }
    }
}

// ---------------------------------------------------------------------------
// chain: the sequential state carry
// ---------------------------------------------------------------------------
// Workgroup = 4 waves = one (sequence, V head) and 16*kChainTiles columns of
// its state.  Every product of a chunk is split over the four waves by rows:
//   wave w computes Vnew and Q S for the chunk's tokens 16w .. 16w+15, owns
//   (and updates) the state rows 32w .. 32w+31, and writes the outputs of
//   its 16 tokens,
// so each wave reads only its quarter of -W, q^, k^T and P.  Those operands
// come straight from L2/HBM into registers, prefetched two chunks ahead; the
// only exchanges are the fp16 copy of the state (B operand of W S and Q S)
// and the two fp16 copies of Vnew (B operands of P Vnew and of the state
// update), through small LDS buffers, with two barriers per chunk.
constexpr int kChainTiles = 2;                         // 16-column tiles per workgroup
constexpr int kChainBlocksPerHead = 8 / kChainTiles;   // workgroups per (sequence, V head)
constexpr int kChainPrefetch = 2;                      // chunks in flight ahead of the one computed

__device__ __forceinline__ half8 ld_frag(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// this wave's operands of one chunk
template <int CT>
struct ChainOps {
    half8 W[4];   // -W  rows 16w.., k-blocks 0..3 over d_k
    half8 Q[4];   // q^  rows 16w.., k-blocks 0..3 over d_k
    half8 K[4];   // k^T rows 32w + 16rr.., k-blocks 0..1 over tokens: index 2rr + kb
    half8 P[2];   // P   rows 16w.., k-blocks 0..1 over tokens
    half4 U[CT];  // U'  rows 16w.., column tiles of the workgroup
    f32x4 gam;    // q_scale * Gam of rows 16w + 4q4 + e
    f32x4 r;      // Gam_n / Gam of the same rows
    float gn;     // Gam_n
};

template <int CT>
__device__ __forceinline__ void chain_load(ChainOps<CT> &op, const Workspace &ws, long c, int h, int g, int Hqk,
                                           int Hv, int ct0, int wave, int lane)
{
    const long hc = c * Hv + h, gc = c * Hqk + g;
    const __amdgpu_buffer_rsrc_t rw = region_rsrc(ws.wfrag + hc * kWFragBytes);
    const __amdgpu_buffer_rsrc_t rq = region_rsrc(ws.qfrag + gc * kQFragBytes);
    const __amdgpu_buffer_rsrc_t rk = region_rsrc(ws.kfrag + gc * kKFragBytes);
    const __amdgpu_buffer_rsrc_t rp = region_rsrc(ws.pfrag + hc * kPFragBytes);
    const __amdgpu_buffer_rsrc_t ru = region_rsrc(ws.ufrag + hc * kUBytes);
    const __amdgpu_buffer_rsrc_t rg = region_rsrc(ws.gates + hc * kGateFloats);
    const int v16 = lane * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        op.W[i] = ld_frag(rw, v16, (wave * 4 + i) * 1024);
        op.Q[i] = ld_frag(rq, v16, (wave * 4 + i) * 1024);
        op.K[i] = ld_frag(rk, v16, (wave * 4 + i) * 1024);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) op.P[i] = ld_frag(rp, v16, (wave * 2 + i) * 1024);
#pragma unroll
    for (int x = 0; x < CT; ++x)
        op.U[x] = __builtin_bit_cast(half4, __builtin_amdgcn_raw_buffer_load_b64(ru, lane * 8, ((ct0 + x) * 4 + wave) * 512, 0));
    const int row4 = (16 * wave + 4 * (lane >> 4)) * 4;
    op.gam = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, row4, 0, 0));
    op.r = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, row4, 256, 0));
    op.gn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, 0, 512, 0));
}

template <int CT>
struct ChainLds {
    half8 sx[4 * CT * 64];      // state as B operand: [k-block over d_k][tile][lane]
    half8 vb[2 * CT * 64];      // Vnew as B operand:  [k-block over tokens][tile][lane]
    half8 vr[2 * CT * 64];      // (Gam_n / Gam) Vnew as B operand
    uint16_t os[4][16 * 16 * CT];  // output rows of each wave, bf16
};

// one chunk: consumes `op`, and issues the loads of chunk c + kChainPrefetch into `nxt`
template <int CT>
__device__ __forceinline__ void chain_step(const PrefillArgs &p, const Workspace &ws, ChainLds<CT> &L,
                                           f32x4 (&S)[CT][2], const ChainOps<CT> &op, ChainOps<CT> &nxt,
                                           const int4 &si, int cc, int h, int g, int ct0, int wave, int lane)
{
    const int Hqk = p.Hqk, Hv = p.Hv;
    const int q4 = lane >> 4, c16 = lane & 15;
    // always issued (past the end it re-reads the last chunk), so that every
    // chunk has the same memory operations in flight and the waits stay exact
    chain_load<CT>(nxt, ws, si.x + min(cc + kChainPrefetch, si.y - 1), h, g, Hqk, Hv, ct0, wave, lane);

    // 1. this wave's state rows 32w .. 32w+31 are k-block w of the B operand
#pragma unroll
    for (int x = 0; x < CT; ++x) L.sx[(wave * CT + x) * 64 + lane] = pack_h8(S[x][0], S[x][1]);
    __syncthreads();
    // 2. Vnew = U' - W S and Q S for tokens 16w .. 16w+15
    f32x4 Vn[CT], QS[CT];
#pragma unroll
    for (int x = 0; x < CT; ++x) {
        Vn[x] = f32x4{(float)op.U[x][0], (float)op.U[x][1], (float)op.U[x][2], (float)op.U[x][3]};
        QS[x] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int x = 0; x < CT; ++x) {
            const half8 sb = L.sx[(kb * CT + x) * 64 + lane];
            Vn[x] = mfma16(op.W[kb], sb, Vn[x]);
            QS[x] = mfma16(op.Q[kb], sb, QS[x]);
        }
    // 3. publish Vnew (plain and scaled) as half of a token k-block of the B operands
    {
        const int kbt = wave >> 1, half = wave & 1;
#pragma unroll
        for (int x = 0; x < CT; ++x) {
            const f32x4 vs = Vn[x] * op.r;
            half4 hb, hr;
            hb[0] = (_Float16)Vn[x][0]; hb[1] = (_Float16)Vn[x][1]; hb[2] = (_Float16)Vn[x][2]; hb[3] = (_Float16)Vn[x][3];
            hr[0] = (_Float16)vs[0]; hr[1] = (_Float16)vs[1]; hr[2] = (_Float16)vs[2]; hr[3] = (_Float16)vs[3];
            reinterpret_cast<half4 *>(&L.vb[(kbt * CT + x) * 64 + lane])[half] = hb;
            reinterpret_cast<half4 *>(&L.vr[(kbt * CT + x) * 64 + lane])[half] = hr;
        }
    }
    __syncthreads();
    // 4. state rows 32w + 16rr: S <- Gam_n S + k^T (r Vnew)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < CT; ++x) {
            const half8 vr = L.vr[(kb * CT + x) * 64 + lane];
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                if (kb == 0) S[x][rr] = S[x][rr] * op.gn;
                S[x][rr] = mfma16(op.K[2 * rr + kb], vr, S[x][rr]);
            }
        }
    // 5. outputs of tokens 16w .. 16w+15: q_scale (diag(Gam) Q S + P Vnew)
    const int tok0 = si.z + cc * kChunk;
    const int n = min(kChunk, si.w - cc * kChunk);
#pragma unroll
    for (int x = 0; x < CT; ++x) {
        f32x4 acc = QS[x] * op.gam;
        acc = mfma16(op.P[0], L.vb[(0 * CT + x) * 64 + lane], acc);
        if (wave >= 2) acc = mfma16(op.P[1], L.vb[(1 * CT + x) * 64 + lane], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) L.os[wave][(4 * q4 + e) * (16 * CT) + 16 * x + c16] = (uint16_t)f32_to_bf16(acc[e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
        // 16 rows x (32 CT bytes): lane -> (row, 16-byte piece).  A buffer
        // store whose range ends at the chunk's last valid token drops the
        // rows of a partial chunk without a branch.
        static_assert(CT == 2, "one 16-byte piece per lane");
        constexpr int kPieces = 2 * CT;
        const int row = lane / kPieces, piece = lane % kPieces;
        const i32x4 v = reinterpret_cast<const i32x4 *>(&L.os[wave][row * 16 * CT])[piece];
        const int rowb = Hv * kD * 2;  // bytes per token row of o
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            p.o + ((long)tok0 * Hv + h) * kD + 16 * ct0, 0, n * rowb, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, (16 * wave + row) * rowb + piece * 16, 0, 0);
    }
}

template <int CT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chain_kernel(PrefillArgs p, Workspace ws)
{
    __shared__ ChainLds<CT> L;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int q4 = lane >> 4, c16 = lane & 15;
    const int Hqk = p.Hqk, Hv = p.Hv, G = Hv / Hqk;
    constexpr int kPerHead = 8 / CT;
    // block -> (rank, group, head-in-group, column block); all workgroups of
    // one (sequence, QK group) land on the same XCD (same L2)
    const int per_group = G * kPerHead;
    const int bid = blockIdx.x;
    const int gu = (bid / (8 * per_group)) * 8 + (bid & 7);
    const int inner = (bid >> 3) % per_group;
    if (gu >= p.N * Hqk) return;
    const int rank = gu / Hqk, g = gu % Hqk;
    const int j = inner / kPerHead, cb = inner % kPerHead;
    const int h = g * G + j;
    const int ct0 = cb * CT;
    const int s = ws.order[rank];
    const int4 si = ws.seq_info[s];  // chunk0, nchunks, t0, L

    // state rows 32w + 16rr + 4q4 + e, columns 16(ct0 + x) + c16
    f32x4 S[CT][2];
    const long sbase = ((long)s * Hv + h) * kD * kD;
#pragma unroll
    for (int x = 0; x < CT; ++x)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[x][rr][e] = p.state_in ? p.state_in[sbase + (long)(32 * wave + 16 * rr + 4 * q4 + e) * kD +
                                                      16 * (ct0 + x) + c16]
                                         : 0.f;

    if (si.y > 0) {
        // three operand sets rotate: chunk cc is computed while cc+1 and cc+2 load
        ChainOps<CT> o0, o1, o2;
        chain_load<CT>(o0, ws, si.x, h, g, Hqk, Hv, ct0, wave, lane);
        chain_load<CT>(o1, ws, si.x + min(1, si.y - 1), h, g, Hqk, Hv, ct0, wave, lane);
        int cc = 0;
        for (; cc + 3 <= si.y; cc += 3) {
            chain_step<CT>(p, ws, L, S, o0, o2, si, cc, h, g, ct0, wave, lane);
            chain_step<CT>(p, ws, L, S, o1, o0, si, cc + 1, h, g, ct0, wave, lane);
            chain_step<CT>(p, ws, L, S, o2, o1, si, cc + 2, h, g, ct0, wave, lane);
        }
        if (cc < si.y) chain_step<CT>(p, ws, L, S, o0, o2, si, cc, h, g, ct0, wave, lane);
        if (cc + 1 < si.y) chain_step<CT>(p, ws, L, S, o1, o0, si, cc + 1, h, g, ct0, wave, lane);
    }

#pragma unroll
    for (int x = 0; x < CT; ++x)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.state_out[sbase + (long)(32 * wave + 16 * rr + 4 * q4 + e) * kD + 16 * (ct0 + x) + c16] = S[x][rr][e];

    // carried conv rows: the last three raw rows of the sequence (v channels of
    // head h; the first head of the group also writes the q and k channels)
    if (p.conv_state_out && cb == 0 && wave == 0) {
        const long C_tot = 2L * Hqk * kD + (long)Hv * kD;
        const int Ls = si.w, t0 = si.z;
        for (int plane = (j == 0 ? 0 : 2); plane < 3; ++plane) {
            const long ch0 = plane == 0 ? (long)g * kD : plane == 1 ? (long)Hqk * kD + (long)g * kD
                                                                  : 2L * Hqk * kD + (long)h * kD;
            const uint16_t *src = plane == 0 ? p.q + (long)g * kD : plane == 1 ? p.k + (long)g * kD
                                                                              : p.v + (long)h * kD;
            const long ld = plane == 2 ? (long)Hv * kD : (long)Hqk * kD;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const int tau = Ls - 3 + r;
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
    const long blocks = ((groups + 7) / 8) * 8L * G * kChainBlocksPerHead;
    hipLaunchKernelGGL(chain_kernel<kChainTiles>, dim3((unsigned)blocks), dim3(256), 0, stream, p, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark(3);
}

}  // namespace gdn
