// gdn_backward.hip -- gradients of the chunked GDN prefill (training
// backward), for B sequences of equal length T or packed sequences of any
// lengths, on gfx950.
//
// The forward, per chunk of n <= 64 tokens of one (sequence, V head), with S
// the state entering the chunk, gamma the in-chunk cumulative log decay (Gam =
// e^gamma, gamma_n = gamma of the last token), beta the write strengths:
//   A   = strict_lower(diag(beta) K K^T * D),   D_ij = e^(gamma_i - gamma_j)
//   X   = (I + A)^-1,   T' = X diag(beta)
//   Vt  = V - diag(Gam) K S                      (what the state mispredicts)
//   Vn  = T' Vt
//   O   = q_scale (diag(Gam) Q S + P Vn),        P = Q K^T * D, lower incl. diagonal
//   S'  = Gam_n S + Ks^T Vn,                      Ks = diag(e^(gamma_n - gamma)) K
// (the WY / chunk-parallel form of the update of the local-inference
// walkthrough, section 2.1; section 9 of the architecture deep dive on
// alwayszhang.cn describes FlashQLA's forward and backward kernels of this
// chunked form).  The backward applies the chain rule to each of these
// lines in reverse; the derivative of the inverse is dL = -X^T dX X^T.  All
// arithmetic is fp32: the two sequential passes multiply on the fp32 matrix
// cores, everything else on the vector ALUs.
//
// Passes (one launch each):
//   bwd_setup_kernel   (packed calls) chunk and sequence tables from cu_seqlens
//   bwd_prep_kernel    conv + SiLU (+ L2 norm) of q, k, v; gates and gamma
//   bwd_local_kernel   per (chunk, QK group): P and X = (I + A)^-1 of its V heads
//   bwd_fwd_kernel     per (sequence, V head, 32 state columns), in order:
//                      the state entering every chunk, Vt and Vn
//   bwd_chain_kernel   per (sequence, V head, 32 columns), in reverse: the
//                      state gradient at every chunk end, dVn and dVt (= dv^)
//   bwd_grad_kernel    per (chunk, V head): dq^, dk^ (per V head), dgamma,
//                      dbeta -> grad_a, grad_b
//   bwd_dy_kernel      per (chunk, channel plane): back through the L2 norm
//                      and SiLU to the conv output
//   bwd_conv_kernel    per (chunk, channel plane): back through the conv to
//                      q, k, v, the carried conv rows and per-chunk partial
//                      conv weight gradients
//   bwd_dw_kernel      the conv weight gradient, summed over chunks in order
// The state columns are independent in the update, so the two sequential
// passes split them over four workgroups per (sequence, V head); the twelve
// workgroups of one (sequence, QK group) run on one XCD and share its L2.
#include "../../include/gdn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_common.h"

namespace gdn {
namespace {

constexpr int kBT = 256;  // threads of every backward workgroup
constexpr int kCB = 32;   // state columns per workgroup of the sequential passes
constexpr int kLK = 132;  // LDS row stride of 64 x 128 fp32 tiles (16-byte rows, 4-bank skew)
constexpr int kLN = 68;   // LDS row stride of 64 x 64 fp32 tiles
constexpr int kLC = kCB;  // LDS row stride of kCB-column slices (read as broadcasts)
constexpr int kNCB = kD / kCB;
constexpr int kST = 512;  // threads of a sequential-pass workgroup: eight waves, two per SIMD
constexpr int kSD = kNCB * (kST / 64);  // <dS', S> partials per (chunk, V head): one per wave

struct BwdArgs {
    const uint16_t *q, *k, *v;
    const float *a, *b;
    const uint16_t *conv_w, *conv_state_in;
    const float *state_in;
    const uint16_t *grad_o;
    const float *grad_state_out;
    float *grad_q, *grad_k, *grad_v, *grad_a, *grad_b, *grad_conv_w, *grad_conv_state_in, *grad_state_in;
    const int32_t *cu_seqlens;  // packed calls: sequence bounds (device); else NULL
    int N;                      // sequences
    int T, nc;                  // uniform calls: tokens and chunks per sequence
    int T_tot, max_chunks;      // all tokens; chunk slots
    int Hqk, Hv;
    float gate_scale, q_scale;
};

// Workspace (fp32).  tok = s*T + t; rows of a chunk beyond its length are
// never written or read.
struct BwdWs {
    int4 *chunk_info;   // [chunk slot] {sequence, its first token, length, index in it} (packed calls)
    int4 *seq_info;     // [sequence] {first chunk slot, chunks, first token, length} (packed calls)
    float *qh, *kh;     // [tok][Hqk][128]  q^, k^
    float *vh;          // [tok][Hv][128]   v^
    float *gam, *beta;  // [tok][Hv]        gamma (natural log), beta
    float *X, *P;       // [chunk][Hv][64][64]
    float *Sc, *dSc;    // [chunk][Hv][128][128]  state entering / gradient leaving
    float *vt, *vn;     // [tok][Hv][128]   Vt, Vn
    float *dvn, *dvh;   // [tok][Hv][128]   dVn, dVt = dv^
    float *dqp, *dkp;   // [tok][Hv][128]   dq^, dk^ of each V head
    float *dy;          // [tok][C_tot]     gradient of the conv outputs
    float *sdot;        // [chunk][Hv][kSD] <dS', S> of each (column block, wave): state
                        //                   gradient leaving the chunk, state entering it
    float *dwp;         // [chunk][C_tot][4] conv weight gradient of each chunk
};

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

// Sequential-pass block id -> (sequence, V head, column block), so that the
// G * kNCB blocks of one (sequence, QK group), which read the same k^ and q^
// rows chunk after chunk, get ids of one residue mod 8: they run on the same
// XCD (blocks are dealt to the eight XCDs round-robin) and share its L2.  A
// tail of fewer than eight groups maps plainly.
__device__ __forceinline__ void seq_block(const BwdArgs &p, int b, int &s, int &h, int &cb)
{
    const int G = p.Hv / p.Hqk, P = G * kNCB, N = gridDim.x;
    const int full = N / (8 * P) * (8 * P);
    int unit, member;
    if (b < full) {
        unit = 8 * ((b >> 3) / P) + (b & 7);
        member = (b >> 3) % P;
    } else {
        unit = b / P;
        member = b % P;
    }
    s = unit / p.Hqk;
    h = (unit % p.Hqk) * G + member / kNCB;
    cb = member % kNCB;
}
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void st4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }

// {sequence, its first token, chunk length (0: empty slot), chunk index in the sequence}
__device__ __forceinline__ int4 bchunk(const BwdArgs &p, const BwdWs &ws, int cidx)
{
    if (p.cu_seqlens) return ws.chunk_info[cidx];
    const int s = cidx / p.nc, j = cidx % p.nc;
    return make_int4(s, s * p.T, min(kChunk, p.T - j * kChunk), j);
}
// {first chunk slot, chunks, first token, length}
__device__ __forceinline__ int4 bseq(const BwdArgs &p, const BwdWs &ws, int s)
{
    if (p.cu_seqlens) return ws.seq_info[s];
    return make_int4(s * p.nc, p.nc, s * p.T, p.T);
}
__device__ __forceinline__ float silu_grad(float y)
{
    const float s = sigm(y);
    return s * (1.0f + y * (1.0f - s));
}

// channel plane -> tensor, head and conv channel base
struct Plane {
    int kind, head;  // kind 0 q, 1 k, 2 v
    long ch0;        // first conv channel
    long ld;         // elements per token row of the tensor
};
__device__ __forceinline__ Plane plane_of(const BwdArgs &p, int pl)
{
    if (pl < p.Hqk) return Plane{0, pl, (long)pl * kD, (long)p.Hqk * kD};
    if (pl < 2 * p.Hqk) return Plane{1, pl - p.Hqk, (long)p.Hqk * kD + (long)(pl - p.Hqk) * kD, (long)p.Hqk * kD};
    const int h = pl - 2 * p.Hqk;
    return Plane{2, h, 2L * p.Hqk * kD + (long)h * kD, (long)p.Hv * kD};
}
__device__ __forceinline__ const uint16_t *plane_src(const BwdArgs &p, const Plane &P)
{
    return (P.kind == 0 ? p.q : P.kind == 1 ? p.k : p.v) + (long)P.head * kD;
}

// The conv rows a thread needs, held in registers: thread (channel c, half
// rh) of a chunk takes its rows 32 rh .. 32 rh + 31 (sequence positions
// tb .. tb + 31), and the window holds the raw rows tb - 3 .. tb + 31 of
// channel c (carried rows, or zeros, before the sequence; zeros past it).
constexpr int kWin = 35;
__device__ __forceinline__ void x_window(const BwdArgs &p, const Plane &P, const uint16_t *x, int s, long seq0,
                                         int tb, int L, int c, long C_tot, float (&xw)[kWin])
{
    // all rows are loaded first, clamped into the sequence, so that the loads
    // are in flight together; rows outside it are then replaced
    uint16_t raw[kWin];
#pragma unroll
    for (int i = 0; i < kWin; ++i) raw[i] = x[(seq0 + min(max(tb - 3 + i, 0), L - 1)) * P.ld + c];
#pragma unroll
    for (int i = 0; i < kWin; ++i) {
        const int tau = tb - 3 + i;
        float v = 0.f;
        if (tau >= 0 && tau < L)
            v = bf16_to_f32(raw[i]);
        else if (tau < 0 && p.conv_state_in)
            v = bf16_to_f32(p.conv_state_in[((long)s * 3 + 3 + tau) * C_tot + P.ch0 + c]);
        xw[i] = v;
    }
}
// conv output of the window's row r (sequence position tb + r): taps in order
__device__ __forceinline__ float conv_at(const float (&w)[4], const float (&xw)[kWin], int r)
{
    float y = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) y = fmaf(w[j], xw[r + j], y);
    return y;
}

// ---------------------------------------------------------------------------
// 1. q^, k^, v^, gamma, beta
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBT) void bwd_prep_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ float zs[64 * kLK];
    __shared__ float nrm[64];
    const int4 ci = bchunk(p, ws, blockIdx.x);
    const int s = ci.x, n = ci.z, j = ci.w;
    if (n == 0) return;  // empty chunk slot
    const long seq0 = ci.y, t0 = seq0 + (long)j * kChunk;
    const int L = bseq(p, ws, s).w;
    const long C_tot = 2L * p.Hqk * kD + (long)p.Hv * kD;
    const Plane P = plane_of(p, blockIdx.y);
    const uint16_t *x = plane_src(p, P);
    const int t = threadIdx.x, c = t & 127, rh = t >> 7, rb = 32 * rh;
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_to_f32(p.conv_w[(P.ch0 + c) * 4 + i]);
    float xw[kWin];
    x_window(p, P, x, s, seq0, j * kChunk + rb, L, c, C_tot, xw);
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        if (rb + r < n) {
            const float y = conv_at(w, xw, r);
            const float z = y * sigm(y);
            if (P.kind == 2)
                ws.vh[((t0 + rb + r) * p.Hv + P.head) * kD + c] = z;
            else
                zs[(rb + r) * kLK + c] = z;
        }
    }
    if (P.kind == 2) {
        // gates of this V head, lane = token: g = -c softplus(a), gamma = in-chunk prefix sum
        if (t < 64) {
            float g = 0.f, be = 0.f;
            if (t < n) {
                const long ti = (t0 + t) * p.Hv + P.head;
                const float av = p.a[ti];
                g = -p.gate_scale * (fmaxf(av, 0.f) + log1pf(expf(-fabsf(av))));
                be = sigm(p.b[ti]);
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float u = __shfl_up(g, off, 64);
                if (t >= off) g += u;
            }
            if (t < n) {
                ws.gam[(t0 + t) * p.Hv + P.head] = g;
                ws.beta[(t0 + t) * p.Hv + P.head] = be;
            }
        }
        return;
    }
    __syncthreads();
    {
        const int r = t >> 2, part = t & 3;
        float ss = 0.f;
        if (r < n)
            for (int i = 0; i < 32; ++i) {
                const float z = zs[r * kLK + part * 32 + i];
                ss = fmaf(z, z, ss);
            }
        ss += __shfl_xor(ss, 1, 64);
        ss += __shfl_xor(ss, 2, 64);
        if (part == 0) nrm[r] = sqrtf(ss + 1e-6f);
    }
    __syncthreads();
    float *dst = P.kind == 0 ? ws.qh : ws.kh;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        if (rb + r < n) {
            dst[((t0 + rb + r) * p.Hqk + P.head) * kD + c] = zs[(rb + r) * kLK + c] / nrm[rb + r];
        }
    }
}

// ---------------------------------------------------------------------------
// 2. P and X = (I + A)^-1 per (chunk, QK group)
// ---------------------------------------------------------------------------
// Column of (I + A)^-1 for a strictly lower A (row stride kLN), y = e_c on
// entry: right-looking substitution, expanded at compile time so that y
// stays in registers.
template <int M>
struct SolveCol64 {
    static __device__ __forceinline__ void run(float (&y)[64], const float *A)
    {
        if constexpr (M < 63) {
#pragma unroll
            for (int ii = M + 1; ii < 64; ++ii) y[ii] = fmaf(-A[ii * kLN + M], y[M], y[ii]);
            SolveCol64<M + 1>::run(y, A);
        }
    }
};

// One workgroup per (chunk, QK group): K^K^T and Q^K^T once, then the
// group's V heads four at a time (their A matrices reuse the LDS of the k^ /
// q^ rows), wave w solving head w.
constexpr int kLocalR = 4 * 64 * kLN;  // >= 2 * 64 * kLK: the k^ and q^ rows, or four A matrices
static_assert(kLocalR >= 2 * 64 * kLK, "the A matrices overlay the k^ and q^ rows");

__global__ __launch_bounds__(kBT) void bwd_local_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ __attribute__((aligned(16))) float R[kLocalR];
    __shared__ float KK[64 * kLN], QK[64 * kLN];
    __shared__ float gam[4][64], bet[4][64];
    const int Hv = p.Hv, Hqk = p.Hqk, G = Hv / Hqk;
    const int cidx = blockIdx.x / Hqk, g = blockIdx.x % Hqk;
    const int4 ci = bchunk(p, ws, cidx);
    const int n = ci.z;
    if (n == 0) return;
    const long t0 = (long)ci.y + (long)ci.w * kChunk;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    float *Ks = R, *Qs = R + 64 * kLK;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int idx = t + kBT * e, r = idx >> 5, q = idx & 31;
        const long src = ((t0 + r) * Hqk + g) * kD + 4 * q;
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        st4(Ks + r * kLK + 4 * q, r < n ? ld4(ws.kh + src) : z);
        st4(Qs + r * kLK + 4 * q, r < n ? ld4(ws.qh + src) : z);
    }
    __syncthreads();
    {
        // row i, columns (t & 3) + 4m
        const int i = t >> 2;
        float kk[16], qk[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) kk[m] = qk[m] = 0.f;
        for (int d = 0; d < kD; ++d) {
            const float ki = Ks[i * kLK + d], qi = Qs[i * kLK + d];
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float kj = Ks[((t & 3) + 4 * m) * kLK + d];
                kk[m] = fmaf(ki, kj, kk[m]);
                qk[m] = fmaf(qi, kj, qk[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            KK[i * kLN + (t & 3) + 4 * m] = kk[m];
            QK[i * kLN + (t & 3) + 4 * m] = qk[m];
        }
    }
    __syncthreads();  // the k^ / q^ rows are dead from here on
    for (int j0 = 0; j0 < G; j0 += 4) {
        const int jn = min(4, G - j0);
        if (w < jn) {
            const int h = g * G + j0 + w;
            gam[w][lane] = lane < n ? ws.gam[(t0 + lane) * Hv + h] : 0.f;
            bet[w][lane] = lane < n ? ws.beta[(t0 + lane) * Hv + h] : 0.f;
        }
        __syncthreads();
        // A (strict lower) into LDS and P (lower incl. the diagonal) to the workspace, for each head
        for (int idx = t; idx < jn * 4096; idx += kBT) {
            const int jh = idx >> 12, i = (idx >> 6) & 63, jj = idx & 63;
            const float D = expf(gam[jh][i] - gam[jh][jj]);
            R[jh * 64 * kLN + i * kLN + jj] = (jj < i && i < n) ? bet[jh][i] * KK[i * kLN + jj] * D : 0.f;
            const long mo = ((long)cidx * Hv + g * G + j0 + jh) * 4096;
            ws.P[mo + i * 64 + jj] = (jj <= i && i < n) ? QK[i * kLN + jj] * D : 0.f;
        }
        __syncthreads();
        // unit lower-triangular inverse of head w's I + A, lane c takes column c in
        // registers: once x_m is final it is removed from every later row
        if (w < jn) {
            float y[64];
#pragma unroll
            for (int ii = 0; ii < 64; ++ii) y[ii] = ii == lane ? 1.f : 0.f;
            SolveCol64<0>::run(y, R + w * 64 * kLN);
            const long mo = ((long)cidx * Hv + g * G + j0 + w) * 4096;
#pragma unroll
            for (int ii = 0; ii < 64; ++ii) ws.X[mo + ii * 64 + lane] = y[ii];
        }
        __syncthreads();  // the next round rewrites the gates and the A matrices
    }
}

// Per-chunk operands of the sequential passes in LDS
struct SeqTile {
    float K[64 * kLK];
    float X[64 * kLN];
    float gam[64], bet[64], eg[64], en[64];
};


// A chunk's operands for the sequential passes, held in registers: they are
// requested before the current chunk's products and written to LDS after
// them, so that their load latency overlaps the arithmetic.  kChain: the
// backward pass (q^, P and dO as well; else V).
constexpr int kPrK = 2048 / kST, kPrX = 1024 / kST, kPrS = 64 * kCB / 4 / kST;
template <bool kChain>
struct SeqPref {
    float4 k[kPrK], q[kChain ? kPrK : 1], x[kPrX], pm[kChain ? kPrX : 1], v[kChain ? 1 : kPrS];
    uint2 o[kChain ? kPrS : 1];
    float gam, gl, bet;
    int n;
    long t0;
};
template <bool kChain>
__device__ __forceinline__ void seq_fetch(const BwdArgs &p, const BwdWs &ws, SeqPref<kChain> &f, int cidx, long t0,
                                          int n, int h, int g, int col0)
{
    const int t = threadIdx.x, Hv = p.Hv;
    const long mo = ((long)cidx * Hv + h) * 64 * 64;
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    f.n = n;
    f.t0 = t0;
#pragma unroll
    for (int e = 0; e < kPrK; ++e) {
        const int idx = t + kST * e, r = idx >> 5, q = idx & 31;
        const long src = (t0 + r) * p.Hqk * kD + (long)g * kD + 4 * q;
        f.k[e] = r < n ? ld4(ws.kh + src) : z4;
        if constexpr (kChain) f.q[e] = r < n ? ld4(ws.qh + src) : z4;
    }
#pragma unroll
    for (int e = 0; e < kPrX; ++e) {
        const int idx = t + kST * e;
        f.x[e] = ld4(ws.X + mo + 4 * idx);
        if constexpr (kChain) f.pm[e] = ld4(ws.P + mo + 4 * idx);
    }
    constexpr int Q = kCB / 4;
#pragma unroll
    for (int e = 0; e < kPrS; ++e) {
        const int idx = t + kST * e, r = idx / Q, q = idx % Q;
        const long src = ((t0 + r) * Hv + h) * kD + col0 + 4 * q;
        if constexpr (kChain)
            f.o[e] = r < n ? *reinterpret_cast<const uint2 *>(p.grad_o + src) : make_uint2(0u, 0u);
        else
            f.v[e] = r < n ? ld4(ws.vh + src) : z4;
    }
    if (t < 64) {
        f.gl = ws.gam[(t0 + n - 1) * Hv + h];
        f.gam = t < n ? ws.gam[(t0 + t) * Hv + h] : 0.f;
        f.bet = t < n ? ws.beta[(t0 + t) * Hv + h] : 0.f;
    }
}
template <bool kChain>
__device__ __forceinline__ void seq_commit(const BwdArgs &p, const SeqPref<kChain> &f, SeqTile &L, float *Qs,
                                           float *Ps, float *slice)
{
    const int t = threadIdx.x, n = f.n;
#pragma unroll
    for (int e = 0; e < kPrK; ++e) {
        const int idx = t + kST * e, r = idx >> 5, q = idx & 31;
        st4(L.K + r * kLK + 4 * q, f.k[e]);
        if constexpr (kChain) st4(Qs + r * kLK + 4 * q, f.q[e]);
    }
#pragma unroll
    for (int e = 0; e < kPrX; ++e) {
        const int idx = t + kST * e, r = idx >> 4, q = idx & 15;
        st4(L.X + r * kLN + 4 * q, f.x[e]);
        if constexpr (kChain) st4(Ps + r * kLN + 4 * q, f.pm[e]);
    }
    constexpr int Q = kCB / 4;
#pragma unroll
    for (int e = 0; e < kPrS; ++e) {
        const int idx = t + kST * e, r = idx / Q, q = idx % Q;
        if constexpr (kChain) {
            const uint2 u = f.o[e];
            st4(slice + r * kLC + 4 * q, make_float4(p.q_scale * bf16_lo(u.x), p.q_scale * bf16_hi(u.x),
                                                     p.q_scale * bf16_lo(u.y), p.q_scale * bf16_hi(u.y)));
        } else {
            st4(slice + r * kLC + 4 * q, f.v[e]);
        }
    }
    if (t < 64) {
        L.gam[t] = f.gam;
        L.bet[t] = f.bet;
        L.eg[t] = t < n ? expf(f.gam) : 0.f;
        L.en[t] = t < n ? expf(f.gl - f.gam) : 0.f;
    }
}

// ---------------------------------------------------------------------------
// 3. forward again, keeping the state entering every chunk, Vt and Vn
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The sequential passes multiply on the fp32 matrix cores in 16 x 16 tiles:
// lane l supplies A[16 tile + l%16][k] and B[k][16 tile + l%16] for
// k = 4 kb + l/16, and holds rows 4 (l/16) .. +3 of column l%16 of its tile.
// The state (or its gradient), 128 x 32: wave w holds row tile w in both
// column tiles.  A 64 x 32 slice: wave w holds tile (w / 2, w % 2).
__global__ __launch_bounds__(kST) void bwd_fwd_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ SeqTile L;
    __shared__ __attribute__((aligned(16))) float Ss[kD * kLC], Vs[64 * kLC], Vts[64 * kLC], Vns[64 * kLC];
    const int Hv = p.Hv, G = Hv / p.Hqk;
    int s, h, cb;
    seq_block(p, blockIdx.x, s, h, cb);
    const int g = h / G, col0 = cb * kCB;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, lr = lane & 15, lq = lane >> 4;
    const int srow = 16 * w + 4 * lq;                      // state rows srow .. srow + 3
    const int vrt = w >> 1, vrow = 16 * vrt + 4 * lq, vcol = 16 * (w & 1) + lr;  // slice tile
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 S[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[ct][e] = p.state_in ? p.state_in[(((long)s * Hv + h) * kD + srow + e) * kD + col0 + 16 * ct + lr] : 0.f;
    const int4 sq = bseq(p, ws, s);  // {first chunk slot, chunks, first token, length}
    const int nch = sq.y;
    SeqPref<false> f;
    if (nch > 0) {
        seq_fetch<false>(p, ws, f, sq.x, sq.z, min(kChunk, sq.w), h, g, col0);
        seq_commit<false>(p, f, L, nullptr, nullptr, Vs);
    }
    for (int j = 0; j < nch; ++j) {
        const int cidx = sq.x + j, n = min(kChunk, sq.w - j * kChunk);
        const long t0 = (long)sq.z + (long)j * kChunk;
        float *sc = ws.Sc + ((long)cidx * Hv + h) * kD * kD + col0;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sc[(long)(srow + e) * kD + 16 * ct + lr] = S[ct][e];
                Ss[(srow + e) * kLC + 16 * ct + lr] = S[ct][e];
            }
        if (j + 1 < nch) seq_fetch<false>(p, ws, f, cidx + 1, t0 + kChunk, min(kChunk, sq.w - (j + 1) * kChunk), h, g, col0);
        __syncthreads();
        // Vt = V - diag(Gam) K S
        f32x4 acc = z4;
#pragma unroll 8
        for (int kb = 0; kb < kD / 4; ++kb)
            acc = mfma4(L.K[(16 * vrt + lr) * kLK + 4 * kb + lq], Ss[(4 * kb + lq) * kLC + vcol], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = vrow + e;
            const float vt = r < n ? Vs[r * kLC + vcol] - L.eg[r] * acc[e] : 0.f;
            Vts[r * kLC + vcol] = vt;
            if (r < n) ws.vt[((t0 + r) * Hv + h) * kD + col0 + vcol] = vt;
        }
        __syncthreads();
        // Vn = X diag(beta) Vt (X lower: k < 16 (vrt + 1))
        acc = z4;
        for (int kb = 0; kb < 4 * vrt + 4; ++kb) {
            const int k = 4 * kb + lq;
            acc = mfma4(L.X[(16 * vrt + lr) * kLN + k] * L.bet[k], Vts[k * kLC + vcol], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = vrow + e;
            const float vn = r < n ? acc[e] : 0.f;
            Vns[r * kLC + vcol] = vn;
            if (r < n) ws.vn[((t0 + r) * Hv + h) * kD + col0 + vcol] = vn;
        }
        __syncthreads();
        // S <- Gam_n S + Ks^T Vn
        const float egn = L.eg[n - 1];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[ct][e] *= egn;
#pragma unroll 4
        for (int kb = 0; kb < 16; ++kb) {
            const int k = 4 * kb + lq;
            const float a = L.en[k] * L.K[k * kLK + 16 * w + lr];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) S[ct] = mfma4(a, Vns[k * kLC + 16 * ct + lr], S[ct]);
        }
        __syncthreads();
        if (j + 1 < nch) seq_commit<false>(p, f, L, nullptr, nullptr, Vs);
    }
}

// ---------------------------------------------------------------------------
// 4. the state gradient, chunk by chunk from the last
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kST) void bwd_chain_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ SeqTile L;
    __shared__ __attribute__((aligned(16))) float Qs[64 * kLK], Ps[64 * kLN];
    __shared__ __attribute__((aligned(16))) float dSs[kD * kLC], dOs[64 * kLC], dVns[64 * kLC], dVts[64 * kLC];
    const int Hv = p.Hv, G = Hv / p.Hqk;
    int s, h, cb;
    seq_block(p, blockIdx.x, s, h, cb);
    const int g = h / G, col0 = cb * kCB;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, lr = lane & 15, lq = lane >> 4;
    const int srow = 16 * w + 4 * lq;
    const int vrt = w >> 1, vrow = 16 * vrt + 4 * lq, vcol = 16 * (w & 1) + lr;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const long so = ((long)s * Hv + h) * kD * kD + col0;
    f32x4 dS[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dS[ct][e] = p.grad_state_out ? p.grad_state_out[so + (long)(srow + e) * kD + 16 * ct + lr] : 0.f;
    const int4 sq = bseq(p, ws, s);  // {first chunk slot, chunks, first token, length}
    const int nch = sq.y;
    SeqPref<true> f;
    // this block's columns of the state entering a chunk, loaded one chunk
    // ahead, for <dS', S> (the gate gradient's Gam_n S term)
    float sv[8];
    auto load_sv = [&](int c) {
        const float *sc = ws.Sc + ((long)c * Hv + h) * kD * kD + col0;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) sv[4 * ct + e] = sc[(long)(srow + e) * kD + 16 * ct + lr];
    };
    if (nch > 0) {
        load_sv(sq.x + nch - 1);
        seq_fetch<true>(p, ws, f, sq.x + nch - 1, sq.z + (long)(nch - 1) * kChunk, sq.w - (nch - 1) * kChunk, h, g,
                        col0);
        seq_commit<true>(p, f, L, Qs, Ps, dOs);
    }
    for (int j = nch - 1; j >= 0; --j) {
        const int cidx = sq.x + j, n = min(kChunk, sq.w - j * kChunk);
        const long t0 = (long)sq.z + (long)j * kChunk;
        float *dsc = ws.dSc + ((long)cidx * Hv + h) * kD * kD + col0;
        float part = 0.f;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dsc[(long)(srow + e) * kD + 16 * ct + lr] = dS[ct][e];
                dSs[(srow + e) * kLC + 16 * ct + lr] = dS[ct][e];
                part = fmaf(dS[ct][e], sv[4 * ct + e], part);
            }
        part = wave_sum(part);
        if (lane == 0) ws.sdot[((long)cidx * Hv + h) * kSD + (kST / 64) * cb + w] = part;
        if (j > 0) load_sv(cidx - 1);
        if (j > 0) seq_fetch<true>(p, ws, f, cidx - 1, t0 - kChunk, kChunk, h, g, col0);
        __syncthreads();
        // dVn = diag(en) K dS' + P^T dO'  (P^T upper: k >= 16 vrt)
        f32x4 acc = z4;
#pragma unroll 8
        for (int kb = 0; kb < kD / 4; ++kb)
            acc = mfma4(L.K[(16 * vrt + lr) * kLK + 4 * kb + lq], dSs[(4 * kb + lq) * kLC + vcol], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= L.en[vrow + e];
        for (int kb = 4 * vrt; kb < 16; ++kb) {
            const int k = 4 * kb + lq;
            acc = mfma4(Ps[k * kLN + 16 * vrt + lr], dOs[k * kLC + vcol], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = vrow + e;
            const float v = r < n ? acc[e] : 0.f;
            dVns[r * kLC + vcol] = v;
            if (r < n) ws.dvn[((t0 + r) * Hv + h) * kD + col0 + vcol] = v;
        }
        __syncthreads();
        // dVt = T'^T dVn = diag(beta) X^T dVn
        acc = z4;
        for (int kb = 4 * vrt; kb < 16; ++kb) {
            const int k = 4 * kb + lq;
            acc = mfma4(L.X[k * kLN + 16 * vrt + lr], dVns[k * kLC + vcol], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = vrow + e;
            const float v = r < n ? L.bet[r] * acc[e] : 0.f;
            dVts[r * kLC + vcol] = v;
            if (r < n) ws.dvh[((t0 + r) * Hv + h) * kD + col0 + vcol] = v;
        }
        __syncthreads();
        // dS <- Gam_n dS' + (Gam Q)^T dO' - (Gam K)^T dVt
        const float egn = L.eg[n - 1];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) dS[ct][e] *= egn;
#pragma unroll 4
        for (int kb = 0; kb < 16; ++kb) {
            const int k = 4 * kb + lq;
            const float aq = L.eg[k] * Qs[k * kLK + 16 * w + lr], ak = -L.eg[k] * L.K[k * kLK + 16 * w + lr];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                dS[ct] = mfma4(aq, dOs[k * kLC + 16 * ct + lr], dS[ct]);
                dS[ct] = mfma4(ak, dVts[k * kLC + 16 * ct + lr], dS[ct]);
            }
        }
        __syncthreads();
        if (j > 0) seq_commit<true>(p, f, L, Qs, Ps, dOs);
    }
    if (p.grad_state_in) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.grad_state_in[so + (long)(srow + e) * kD + 16 * ct + lr] = dS[ct][e];
    }
}

// ---------------------------------------------------------------------------
// 5. per-chunk gradients
// ---------------------------------------------------------------------------
// acc[ri][m] += sum_k A(r0 + ri, k) B(k, cc + 16 m) for k < K (a multiple
// of 32), r0 = 4 (t / 16), cc = t % 16, m < NC: a 64 x (16 NC) product,
// staged through LDS 32 deep.  The sources are read 16 bytes at a time along
// their contiguous dimension: fa4(r, k) is A(r, k..k+3) when AK, else
// A(r..r+3, k); fb4(k, c) is B(k..k+3, c) when BK, else B(k, c..c+3).
template <int NC, bool AK, bool BK, class FA4, class FB4>
__device__ __forceinline__ void gemm64(float (&acc)[4][8], int K, FA4 fa4, FB4 fb4, float *sA, float *sB)
{
    const int t = threadIdx.x, r0 = 4 * (t >> 4), cc = t & 15;
    constexpr int NCOL = 16 * NC, LB = NCOL + 1;
    for (int k0 = 0; k0 < K; k0 += 32) {
        float4 va[2], vb[NC / 2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int idx = t + kBT * e;
            va[e] = AK ? fa4(idx >> 3, k0 + 4 * (idx & 7)) : fa4(4 * (idx & 15), k0 + (idx >> 4));
        }
#pragma unroll
        for (int e = 0; e < NC / 2; ++e) {
            const int idx = t + kBT * e;
            vb[e] = BK ? fb4(k0 + 4 * (idx & 7), idx >> 3) : fb4(k0 + idx / (NCOL / 4), 4 * (idx % (NCOL / 4)));
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int idx = t + kBT * e;
            const float v[4] = {va[e].x, va[e].y, va[e].z, va[e].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (AK)
                    sA[(idx >> 3) * 33 + 4 * (idx & 7) + i] = v[i];
                else
                    sA[(4 * (idx & 15) + i) * 33 + (idx >> 4)] = v[i];
            }
        }
#pragma unroll
        for (int e = 0; e < NC / 2; ++e) {
            const int idx = t + kBT * e;
            const float v[4] = {vb[e].x, vb[e].y, vb[e].z, vb[e].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (BK)
                    sB[(4 * (idx & 7) + i) * LB + (idx >> 3)] = v[i];
                else
                    sB[(idx / (NCOL / 4)) * LB + 4 * (idx % (NCOL / 4)) + i] = v[i];
            }
        }
        __syncthreads();
#pragma unroll 2
        for (int kk = 0; kk < 32; ++kk) {
            float av[4], bv[NC];
#pragma unroll
            for (int ri = 0; ri < 4; ++ri) av[ri] = sA[(r0 + ri) * 33 + kk];
#pragma unroll
            for (int m = 0; m < NC; ++m) bv[m] = sB[kk * LB + cc + 16 * m];
#pragma unroll
            for (int ri = 0; ri < 4; ++ri)
#pragma unroll
                for (int m = 0; m < NC; ++m) acc[ri][m] = fmaf(av[ri], bv[m], acc[ri][m]);
        }
        __syncthreads();
    }
}

__device__ __forceinline__ void zero(float (&acc)[4][8])
{
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[ri][m] = 0.f;
}

// sum over the 16 lanes of a row group
__device__ __forceinline__ float sum16(float v)
{
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    v += __shfl_xor(v, 8, 64);
    return v;
}

__global__ __launch_bounds__(kBT) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_grad_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ float sA[64 * 33], sB[32 * 129];
    __shared__ float Em[64 * kLN], Wm[64 * kLN], Ym[64 * kLN];
    __shared__ float gam[64], bet[64], eg[64], en[64], dgam[64], dbet[64], rowv[64];
    const int Hv = p.Hv, Hqk = p.Hqk, G = Hv / Hqk;
    // the G blocks of one (chunk, QK group), which read the same k^ and q^
    // rows, get ids of one residue mod 8: the same XCD, one L2
    int cidx, h;
    {
        const int b = blockIdx.x, full = (int)gridDim.x / (8 * G) * (8 * G);
        const int unit = b < full ? 8 * ((b >> 3) / G) + (b & 7) : b / G;
        const int member = b < full ? (b >> 3) % G : b % G;
        cidx = unit / Hqk;
        h = (unit % Hqk) * G + member;
    }
    const int g = h / G;
    const int4 ci = bchunk(p, ws, cidx);
    const int n = ci.z;
    if (n == 0) return;
    const long t0 = (long)ci.y + (long)ci.w * kChunk;
    const int t = threadIdx.x, r0 = 4 * (t >> 4), cc = t & 15;
    const long mo = ((long)cidx * Hv + h) * 64 * 64;
    const float *Sc = ws.Sc + ((long)cidx * Hv + h) * kD * kD;
    const float *dSc = ws.dSc + ((long)cidx * Hv + h) * kD * kD;
    if (t < 64) {
        const float gl = ws.gam[(t0 + n - 1) * Hv + h];
        const float gr = t < n ? ws.gam[(t0 + t) * Hv + h] : 0.f;
        gam[t] = gr;
        bet[t] = t < n ? ws.beta[(t0 + t) * Hv + h] : 0.f;
        eg[t] = t < n ? expf(gr) : 0.f;
        en[t] = t < n ? expf(gl - gr) : 0.f;
        dgam[t] = 0.f;
        dbet[t] = 0.f;
    }
    __syncthreads();
    auto KH = [&](int r, int d) { return r < n ? ws.kh[((t0 + r) * Hqk + g) * kD + d] : 0.f; };
    auto QH = [&](int r, int d) { return r < n ? ws.qh[((t0 + r) * Hqk + g) * kD + d] : 0.f; };
    // 16-byte sources: four consecutive elements of a row (rows >= n read as zero)
    auto KH4 = [&](int r, int d) { return r < n ? ld4(ws.kh + ((t0 + r) * Hqk + g) * kD + d) : make_float4(0.f, 0.f, 0.f, 0.f); };
    auto QH4 = [&](int r, int d) { return r < n ? ld4(ws.qh + ((t0 + r) * Hqk + g) * kD + d) : make_float4(0.f, 0.f, 0.f, 0.f); };
    auto V4 = [&](const float *base, int r, int c) { return r < n ? ld4(base + ((t0 + r) * Hv + h) * kD + c) : make_float4(0.f, 0.f, 0.f, 0.f); };
    auto DO4 = [&](int r, int c) {
        if (r >= n) return make_float4(0.f, 0.f, 0.f, 0.f);
        const uint2 u = *reinterpret_cast<const uint2 *>(p.grad_o + ((t0 + r) * Hv + h) * kD + c);
        return make_float4(p.q_scale * bf16_lo(u.x), p.q_scale * bf16_hi(u.x), p.q_scale * bf16_lo(u.y),
                           p.q_scale * bf16_hi(u.y));
    };
    auto L4 = [](const float *q) { return *reinterpret_cast<const float4 *>(q); };
    // rows of this thread's group: apply coef[r] * rowsum to dgam (one writer per row)
    auto row_apply = [&](float (&part)[4], float *dst, const float *coef, float sign) {
#pragma unroll
        for (int ri = 0; ri < 4; ++ri) {
            const float v = sum16(part[ri]);
            const int r = r0 + ri;
            if (cc == 0 && r < n) dst[r] += sign * (coef ? coef[r] : 1.f) * v;
        }
    };
    float acc[4][8];
    {
        // ---- dq^ first, so that its registers are free before dk^ is formed
        float dQ[4][8];
        zero(dQ);
        // (c) O = q_scale (diag(Gam) Q S + ...): E1 = dO' S^T
        zero(acc);
        gemm64<8, true, true>(acc, kD, DO4, [&](int c, int i) { return ld4(Sc + i * kD + c); }, sA, sB);
        float part[4];
#pragma unroll
        for (int ri = 0; ri < 4; ++ri) {
            const int r = r0 + ri;
            part[ri] = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                dQ[ri][m] += eg[r] * acc[ri][m];
                part[ri] = fmaf(acc[ri][m], QH(r, cc + 16 * m), part[ri]);
            }
        }
        row_apply(part, dgam, eg, 1.f);
        // (d) P = Q K^T * D * M: dP = dO' Vn^T (lower); Em = dP * P; Wm = dP * D
        zero(acc);
        gemm64<4, true, true>(acc, kD, DO4, [&](int c, int jj) { return V4(ws.vn, jj, c); }, sA, sB);
#pragma unroll
        for (int ri = 0; ri < 4; ++ri)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = r0 + ri, jj = cc + 16 * m;
                const bool in = jj <= r && r < n;
                Em[r * kLN + jj] = in ? acc[ri][m] * ws.P[mo + r * 64 + jj] : 0.f;
                Wm[r * kLN + jj] = in ? acc[ri][m] * expf(gam[r] - gam[jj]) : 0.f;
            }
        __syncthreads();
        gemm64<8, true, false>(dQ, 64, [&](int r, int jj) { return L4(Wm + r * kLN + jj); }, KH4, sA, sB);
#pragma unroll
        for (int ri = 0; ri < 4; ++ri) {
            const int r = r0 + ri;
            if (r >= n) continue;
#pragma unroll
            for (int m = 0; m < 8; ++m) ws.dqp[((t0 + r) * Hv + h) * kD + cc + 16 * m] = dQ[ri][m];
        }
    }
    float dK[4][8];
    zero(dK);
    // (d) continued: dk^ += dQK^T q^
    gemm64<8, false, false>(dK, 64, [&](int r, int jj) { return L4(Wm + jj * kLN + r); }, QH4, sA, sB);

    // (a) Ks = diag(en) K enters S' = ... + Ks^T Vn: dKs = Vn dS'^T
    zero(acc);
    gemm64<8, true, true>(acc, kD, [&](int r, int c) { return V4(ws.vn, r, c); },
                          [&](int c, int i) { return ld4(dSc + i * kD + c); }, sA, sB);
    {
        float part[4];
#pragma unroll
        for (int ri = 0; ri < 4; ++ri) {
            const int r = r0 + ri;
            part[ri] = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                dK[ri][m] += en[r] * acc[ri][m];
                part[ri] = fmaf(acc[ri][m], KH(r, cc + 16 * m), part[ri]);
            }
        }
#pragma unroll
        for (int ri = 0; ri < 4; ++ri) {
            const float v = sum16(part[ri]);
            if (cc == 0) rowv[r0 + ri] = r0 + ri < n ? en[r0 + ri] * v : 0.f;
        }
    }
    // <dS', S> for the Gam_n S term: the state-gradient pass left it per column block
    __syncthreads();
    if (t == 0) {
        float tot = 0.f, sd = 0.f;
        for (int r = 0; r < n; ++r) tot += rowv[r];
        for (int i = 0; i < kSD; ++i) sd += ws.sdot[((long)cidx * Hv + h) * kSD + i];
        dgam[n - 1] += tot + eg[n - 1] * sd;
    }
    __syncthreads();
    if (t < n) dgam[t] -= rowv[t];
    __syncthreads();
    // (e) Vt = V - diag(Gam) K S: E2 = dVt S^T
    zero(acc);
    gemm64<8, true, true>(acc, kD, [&](int r, int c) { return V4(ws.dvh, r, c); },
                          [&](int c, int i) { return ld4(Sc + i * kD + c); }, sA, sB);
    {
        float part[4];
#pragma unroll
        for (int ri = 0; ri < 4; ++ri) {
            const int r = r0 + ri;
            part[ri] = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                dK[ri][m] -= eg[r] * acc[ri][m];
                part[ri] = fmaf(acc[ri][m], KH(r, cc + 16 * m), part[ri]);
            }
        }
        row_apply(part, dgam, eg, -1.f);
    }
    __syncthreads();
    // (f) Vn = T' Vt: dT' = dVn Vt^T (lower incl. diagonal); dbeta_j += sum_i dT'_ij X_ij; dX = dT' diag(beta)
    zero(acc);
    gemm64<4, true, true>(acc, kD, [&](int r, int c) { return V4(ws.dvn, r, c); },
                          [&](int c, int jj) { return V4(ws.vt, jj, c); }, sA, sB);
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = r0 + ri, jj = cc + 16 * m;
            const bool in = jj <= r && r < n;
            Ym[r * kLN + jj] = in ? acc[ri][m] * ws.X[mo + r * 64 + jj] : 0.f;
            Wm[r * kLN + jj] = in ? acc[ri][m] * bet[jj] : 0.f;
        }
    __syncthreads();
    if (t < n) {
        float cs = 0.f;
        for (int r = t; r < n; ++r) cs += Ym[r * kLN + t];
        dbet[t] += cs;
    }
    __syncthreads();
    // (g) X = (I + A)^-1: dA = strict_lower(-X^T dX X^T)
    zero(acc);
    gemm64<4, false, false>(acc, 64, [&](int r, int m) { return ld4(ws.X + mo + m * 64 + r); },
                            [&](int m, int jj) { return L4(Wm + m * kLN + jj); }, sA, sB);
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
        for (int m = 0; m < 4; ++m) Ym[(r0 + ri) * kLN + cc + 16 * m] = acc[ri][m];
    __syncthreads();
    zero(acc);
    gemm64<4, true, true>(acc, 64, [&](int r, int m) { return L4(Ym + r * kLN + m); },
                          [&](int m, int jj) { return ld4(ws.X + mo + jj * 64 + m); }, sA, sB);
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = r0 + ri, jj = cc + 16 * m;
            Wm[r * kLN + jj] = (jj < r && r < n) ? -acc[ri][m] : 0.f;
        }
    __syncthreads();
    // (h) A = diag(beta) K K^T * D (strict lower): dbeta_i, Em += dA * A, dKK -> Ym
    zero(acc);
    gemm64<4, true, true>(acc, kD, KH4, [&](int d, int jj) { return KH4(jj, d); }, sA, sB);
    {
        float part[4];
#pragma unroll
        for (int ri = 0; ri < 4; ++ri) {
            part[ri] = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int r = r0 + ri, jj = cc + 16 * m;
                const bool in = jj < r && r < n;
                const float D = expf(gam[r] - gam[jj]);
                const float dA = Wm[r * kLN + jj];
                if (in) {
                    Em[r * kLN + jj] += dA * bet[r] * acc[ri][m] * D;
                    part[ri] = fmaf(dA, acc[ri][m] * D, part[ri]);
                }
                Ym[r * kLN + jj] = in ? dA * bet[r] * D : 0.f;
            }
        }
        row_apply(part, dbet, nullptr, 1.f);
    }
    __syncthreads();
    gemm64<8, true, false>(dK, 64, [&](int r, int jj) {
        const float4 u = L4(Ym + r * kLN + jj);
        return make_float4(u.x + Ym[jj * kLN + r], u.y + Ym[(jj + 1) * kLN + r], u.z + Ym[(jj + 2) * kLN + r],
                           u.w + Ym[(jj + 3) * kLN + r]);
    }, KH4, sA, sB);
    // gamma: rows of Em count +, columns -; then dg = reverse prefix sum
    if (t < n) {
        float v = 0.f;
        for (int jj = 0; jj < 64; ++jj) v += Em[t * kLN + jj] - Em[jj * kLN + t];
        dgam[t] += v;
    }
    __syncthreads();
    if (t < n) {
        float dg = 0.f;
        for (int r = n - 1; r >= t; --r) dg += dgam[r];
        const long ti = (t0 + t) * Hv + h;
        p.grad_a[ti] = dg * (-p.gate_scale * sigm(p.a[ti]));
        p.grad_b[ti] = dbet[t] * bet[t] * (1.f - bet[t]);
    }
#pragma unroll
    for (int ri = 0; ri < 4; ++ri) {
        const int r = r0 + ri;
        if (r >= n) continue;
#pragma unroll
        for (int m = 0; m < 8; ++m) ws.dkp[((t0 + r) * Hv + h) * kD + cc + 16 * m] = dK[ri][m];
    }
}

// ---------------------------------------------------------------------------
// 6. back through the L2 norm and SiLU to the conv outputs
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBT) void bwd_dy_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ float zs[64 * kLK], ds[64 * kLK];
    __shared__ float nrm[64], zd[64];
    const int4 ci = bchunk(p, ws, blockIdx.x);
    const int s = ci.x, n = ci.z, j = ci.w;
    if (n == 0) return;
    const long seq0 = ci.y, t0 = seq0 + (long)j * kChunk;
    const int L = bseq(p, ws, s).w;
    const long C_tot = 2L * p.Hqk * kD + (long)p.Hv * kD;
    const int G = p.Hv / p.Hqk;
    const Plane P = plane_of(p, blockIdx.y);
    const uint16_t *x = plane_src(p, P);
    const int t = threadIdx.x, c = t & 127, rh = t >> 7, rb = 32 * rh;
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_to_f32(p.conv_w[(P.ch0 + c) * 4 + i]);
    float xw[kWin];
    x_window(p, P, x, s, seq0, j * kChunk + rb, L, c, C_tot, xw);
    // the 32 rows' gradient loads are issued together: rows past the chunk's
    // end read its last row (in bounds) and are not used
    const long hs = (long)p.Hv * kD;
    if (P.kind == 2) {
        const float *gv = ws.dvh + t0 * hs + (long)P.head * kD + c;
        float gr[32];
#pragma unroll
        for (int r = 0; r < 32; ++r) gr[r] = gv[min(rb + r, n - 1) * hs];
#pragma unroll
        for (int r = 0; r < 32; ++r)
            if (rb + r < n) ws.dy[(t0 + rb + r) * C_tot + P.ch0 + c] = gr[r] * silu_grad(conv_at(w, xw, r));
        return;
    }
    float dsum[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) dsum[r] = 0.f;
    for (int jh = 0; jh < G; ++jh) {
        const float *pj = (P.kind == 0 ? ws.dqp : ws.dkp) + t0 * hs + (long)(P.head * G + jh) * kD + c;
#pragma unroll
        for (int r = 0; r < 32; ++r) dsum[r] += pj[min(rb + r, n - 1) * hs];
    }
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        if (rb + r < n) {
            const float y = conv_at(w, xw, r);
            zs[(rb + r) * kLK + c] = y * sigm(y);
            ds[(rb + r) * kLK + c] = dsum[r];
        }
    }
    __syncthreads();
    {
        const int r = t >> 2, pt = t & 3;
        float ss = 0.f, sd = 0.f;
        if (r < n)
            for (int i = 0; i < 32; ++i) {
                const float z = zs[r * kLK + pt * 32 + i];
                ss = fmaf(z, z, ss);
                sd = fmaf(z, ds[r * kLK + pt * 32 + i], sd);
            }
        ss += __shfl_xor(ss, 1, 64);
        ss += __shfl_xor(ss, 2, 64);
        sd += __shfl_xor(sd, 1, 64);
        sd += __shfl_xor(sd, 2, 64);
        if (pt == 0) {
            nrm[r] = sqrtf(ss + 1e-6f);
            zd[r] = sd;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        const int rr = rb + r;
        if (rr < n) {
            const float rn = nrm[rr];
            const float dz = ds[rr * kLK + c] / rn - zs[rr * kLK + c] * zd[rr] / (rn * rn * rn);
            ws.dy[(t0 + rr) * C_tot + P.ch0 + c] = dz * silu_grad(conv_at(w, xw, r));
        }
    }
}

// ---------------------------------------------------------------------------
// 7. back through the conv
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBT) void bwd_conv_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ float wpart[2][kD][4];
    const int cidx = blockIdx.x;
    const int4 ci = bchunk(p, ws, cidx);
    const int s = ci.x, n = ci.z, j = ci.w;
    const long C_tot = 2L * p.Hqk * kD + (long)p.Hv * kD;
    const Plane P = plane_of(p, blockIdx.y);
    if (n == 0) {  // an empty chunk slot contributes nothing to the weight gradient
        if (threadIdx.x < kD)
            for (int jj = 0; jj < 4; ++jj) ws.dwp[((long)cidx * C_tot + P.ch0 + threadIdx.x) * 4 + jj] = 0.f;
        return;
    }
    const long seq0 = ci.y, t0 = seq0 + (long)j * kChunk;
    const int L = bseq(p, ws, s).w;  // sequence length
    const uint16_t *x = plane_src(p, P);
    float *gx = (P.kind == 0 ? p.grad_q : P.kind == 1 ? p.grad_k : p.grad_v) + (long)P.head * kD;
    const int t = threadIdx.x, c = t & 127, rh = t >> 7, rb = 32 * rh, tb = j * kChunk + rb;
    const long ch = P.ch0 + c;
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_to_f32(p.conv_w[ch * 4 + i]);
    // dy of sequence positions tb .. tb + 34 (zero past the sequence), and the raw rows tb - 3 .. tb + 31
    const float *dy = ws.dy + seq0 * C_tot + ch;
    float dw[kWin], xw[kWin];
#pragma unroll
    for (int i = 0; i < kWin; ++i) dw[i] = dy[(long)min(tb + i, L - 1) * C_tot];
#pragma unroll
    for (int i = 0; i < kWin; ++i) dw[i] = tb + i < L ? dw[i] : 0.f;
    x_window(p, P, x, s, seq0, tb, L, c, C_tot, xw);
    float gw[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 32; ++r) {
        if (rb + r < n) {
            // x[tau] feeds y[tau + 3 - jj] through tap jj; y[tau] reads x[tau - 3 + jj]
            float gxv = 0.f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) gxv = fmaf(w[jj], dw[r + 3 - jj], gxv);
            gx[(t0 + rb + r) * P.ld + c] = gxv;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) gw[jj] = fmaf(dw[r], xw[r + jj], gw[jj]);
        }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) wpart[rh][c][jj] = gw[jj];
    __syncthreads();
    if (rh == 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            ws.dwp[((long)cidx * C_tot + ch) * 4 + jj] = wpart[0][c][jj] + wpart[1][c][jj];
        // the carried rows x[-3..-1] feed the sequence's first tokens
        if (j == 0 && p.grad_conv_state_in) {
#pragma unroll
            for (int rr = 0; rr < 3; ++rr) {
                float gv = 0.f;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (rr - jj >= 0) gv = fmaf(w[jj], dw[rr - jj], gv);  // token rr - jj reads row rr through tap jj
                p.grad_conv_state_in[((long)s * 3 + rr) * C_tot + ch] = gv;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 8. conv weight gradient: per-chunk parts summed in chunk order
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBT) void bwd_dw_kernel(BwdArgs p, BwdWs ws, long n_elems, int n_chunks)
{
    const long e = (long)blockIdx.x * kBT + threadIdx.x;
    if (e >= n_elems) return;
    float acc = 0.f;
    for (int c = 0; c < n_chunks; ++c) acc += ws.dwp[(long)c * n_elems + e];
    p.grad_conv_w[e] = acc;
}

__global__ __launch_bounds__(kBT) void bwd_fill_kernel(float *dst, long n)
{
    const long e = (long)blockIdx.x * kBT + threadIdx.x;
    if (e < n) dst[e] = 0.f;
}

// Packed calls: chunk and sequence tables from cu_seqlens, one workgroup.
// Sequence bounds are clamped into [0, T_tot] and chunk slots to max_chunks,
// so that a malformed cu_seqlens cannot send any kernel outside the buffers.
__global__ __launch_bounds__(1024) void bwd_setup_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ int scan[1024];
    __shared__ int base_chunk;
    const int t = threadIdx.x;
    if (t == 0) base_chunk = 0;
    __syncthreads();
    for (int s0 = 0; s0 < p.N; s0 += 1024) {
        const int s = s0 + t;
        int start = 0, len = 0;
        if (s < p.N) {
            start = min(max(p.cu_seqlens[s], 0), p.T_tot);
            len = max(min(max(p.cu_seqlens[s + 1], 0), p.T_tot) - start, 0);
        }
        const int nch = (len + kChunk - 1) / kChunk;
        scan[t] = nch;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int v = t >= off ? scan[t - off] : 0;
            __syncthreads();
            scan[t] += v;
            __syncthreads();
        }
        if (s < p.N) {
            const int first = min(base_chunk + scan[t] - nch, p.max_chunks);
            const int cnt = min(nch, p.max_chunks - first);
            ws.seq_info[s] = make_int4(first, cnt, start, min(len, cnt * kChunk));
            for (int j = 0; j < cnt; ++j) ws.chunk_info[first + j] = make_int4(s, start, min(kChunk, len - j * kChunk), j);
        }
        __syncthreads();
        if (t == 0) base_chunk += scan[1023];
        __syncthreads();
    }
    for (int c = min(base_chunk, p.max_chunks) + t; c < p.max_chunks; c += 1024) ws.chunk_info[c] = make_int4(0, 0, 0, 0);
}

// Workspace carve-up: sizes in floats, each region 64-byte aligned
struct BwdLayout {
    long off[20];
    long total;
};
BwdLayout bwd_layout(int N, int T_tot, int max_chunks, int Hqk, int Hv)
{
    const long tok = T_tot, chunks = max_chunks;
    const long C_tot = 2L * Hqk * kD + (long)Hv * kD;
    const long sizes[20] = {chunks * 4, (long)N * 4,  // int4 tables
                            tok * Hqk * kD, tok * Hqk * kD, tok * Hv * kD, tok * Hv, tok * Hv,
                            chunks * Hv * 4096, chunks * Hv * 4096, chunks * Hv * kD * kD, chunks * Hv * kD * kD,
                            tok * Hv * kD, tok * Hv * kD, tok * Hv * kD, tok * Hv * kD, tok * Hv * kD,
                            tok * Hv * kD, tok * C_tot, chunks * C_tot * 4, chunks * Hv * kSD};
    BwdLayout L{};
    long o = 0;
    for (int i = 0; i < 20; ++i) {
        L.off[i] = o;
        o += (sizes[i] + 15) / 16 * 16;
    }
    L.total = o;
    return L;
}

int bwd_max_chunks(const int32_t *cu_seqlens, int N, int T_tot)
{
    // uniform: N sequences of T_tot / N tokens; packed: sum of ceil(L_i / 64) <= T_tot / 64 + N
    if (cu_seqlens) return T_tot / kChunk + N;
    return N == 0 ? 0 : N * ((T_tot / N + kChunk - 1) / kChunk);
}

}  // namespace

size_t backward_workspace_bytes(int N, int T_tot, bool packed, int Hqk, int Hv)
{
    if (N == 0 || T_tot == 0) return 0;
    const int mc = packed ? T_tot / kChunk + N : bwd_max_chunks(nullptr, N, T_tot);
    return (size_t)bwd_layout(N, T_tot, mc, Hqk, Hv).total * sizeof(float);
}

// Uniform calls: cu_seqlens NULL, N sequences of T tokens (T_tot = N T).
// Packed calls: cu_seqlens (device) with N + 1 bounds over T_tot tokens.
hipError_t launch_backward(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                           const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                           const float *state_in, const uint16_t *grad_o, const float *grad_state_out,
                           float *grad_q, float *grad_k, float *grad_v, float *grad_a, float *grad_b,
                           float *grad_conv_w, float *grad_conv_state_in, float *grad_state_in,
                           const int32_t *cu_seqlens, int N, int T, int T_tot, int Hqk, int Hv, float gate_scale,
                           float q_scale, void *workspace, hipStream_t stream)
{
    BwdArgs p{};
    p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.conv_w = conv_w; p.conv_state_in = conv_state_in;
    p.state_in = state_in; p.grad_o = grad_o; p.grad_state_out = grad_state_out;
    p.grad_q = grad_q; p.grad_k = grad_k; p.grad_v = grad_v; p.grad_a = grad_a; p.grad_b = grad_b;
    p.grad_conv_w = grad_conv_w; p.grad_conv_state_in = grad_conv_state_in; p.grad_state_in = grad_state_in;
    p.cu_seqlens = cu_seqlens; p.N = N; p.T = T; p.nc = (T + kChunk - 1) / kChunk;
    p.T_tot = T_tot; p.max_chunks = T_tot > 0 ? bwd_max_chunks(cu_seqlens, N, T_tot) : 0;
    p.Hqk = Hqk; p.Hv = Hv; p.gate_scale = gate_scale; p.q_scale = q_scale;
    const long C_tot = 2L * Hqk * kD + (long)Hv * kD;
    BwdWs ws{};
    if (T_tot > 0) {
        const BwdLayout L = bwd_layout(N, T_tot, p.max_chunks, Hqk, Hv);
        float *base = static_cast<float *>(workspace);
        ws.chunk_info = reinterpret_cast<int4 *>(base + L.off[0]);
        ws.seq_info = reinterpret_cast<int4 *>(base + L.off[1]);
        float **slots[18] = {&ws.qh, &ws.kh, &ws.vh, &ws.gam, &ws.beta, &ws.X, &ws.P, &ws.Sc, &ws.dSc,
                             &ws.vt, &ws.vn, &ws.dvn, &ws.dvh, &ws.dqp, &ws.dkp, &ws.dy, &ws.dwp, &ws.sdot};
        for (int i = 0; i < 18; ++i) *slots[i] = base + L.off[i + 2];
    } else {
        p.cu_seqlens = nullptr;  // nothing to tabulate: every sequence is empty
        p.T = 0;
        p.nc = 0;
    }
    const int chunks = p.max_chunks, planes = 2 * Hqk + Hv;
    if (chunks > 0) {
        if (p.cu_seqlens) hipLaunchKernelGGL(bwd_setup_kernel, dim3(1), dim3(1024), 0, stream, p, ws);
        hipLaunchKernelGGL(bwd_prep_kernel, dim3(chunks, planes), dim3(kBT), 0, stream, p, ws);
        hipLaunchKernelGGL(bwd_local_kernel, dim3(chunks * Hqk), dim3(kBT), 0, stream, p, ws);
        hipLaunchKernelGGL(bwd_fwd_kernel, dim3(N * Hv * kNCB), dim3(kST), 0, stream, p, ws);
    }
    // also with no tokens: the state gradient passes straight through
    hipLaunchKernelGGL(bwd_chain_kernel, dim3(N * Hv * kNCB), dim3(kST), 0, stream, p, ws);
    if (grad_conv_state_in && (chunks == 0 || p.cu_seqlens)) {
        // rows of sequences without a first chunk (empty ones) stay zero
        const long nh = (long)N * 3 * C_tot;
        hipLaunchKernelGGL(bwd_fill_kernel, dim3((nh + kBT - 1) / kBT), dim3(kBT), 0, stream, grad_conv_state_in, nh);
    }
    const long nw = C_tot * 4;
    if (chunks > 0) {
        hipLaunchKernelGGL(bwd_grad_kernel, dim3(chunks * Hv), dim3(kBT), 0, stream, p, ws);
        hipLaunchKernelGGL(bwd_dy_kernel, dim3(chunks, planes), dim3(kBT), 0, stream, p, ws);
        hipLaunchKernelGGL(bwd_conv_kernel, dim3(chunks, planes), dim3(kBT), 0, stream, p, ws);
        hipLaunchKernelGGL(bwd_dw_kernel, dim3((nw + kBT - 1) / kBT), dim3(kBT), 0, stream, p, ws, nw, chunks);
    } else {
        hipLaunchKernelGGL(bwd_fill_kernel, dim3((nw + kBT - 1) / kBT), dim3(kBT), 0, stream, grad_conv_w, nw);
    }
    return hipGetLastError();
}

}  // namespace gdn
