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
// arithmetic is fp32: the products of the two sequential passes, the
// chunk-local pass and the per-chunk gradients run on the fp32 matrix cores,
// the conv, norm and gate steps on the vector ALUs.
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
//   bwd_dyconv_kernel  per (chunk, channel plane): back through the L2 norm
//                      and SiLU to the conv output (in LDS, with the three
//                      rows after the chunk), then through the conv to q, k,
//                      v, the carried conv rows and per-chunk partial conv
//                      weight gradients
//   bwd_dw_kernel      the conv weight gradient, summed over chunks in order
// A uniform call short of its one-pass workspace runs sequence by sequence in
// windows of whole chunks; bwd_hist_kernel, bwd_addrows_kernel and
// bwd_accum_kernel carry the conv rows, their gradients and the conv weight
// gradient between windows.
// The state columns are independent in the update, so the two sequential
// passes split them over four workgroups per (sequence, V head); the twelve
// workgroups of one (sequence, QK group) run on one XCD and share its L2.
// Long sequences are further cut into segments, run in parallel, each after
// a warm-up whose decay bounds what its zero start drops.
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
constexpr int kLC = kCB;  // LDS row stride of kCB-column slices
// Element (k, c) of a kCB-column slice in LDS.  The sequential passes read
// slices at rows k = 4 kb + lq, lane group lq = 0..3, 16 columns per group:
// rows of one parity share a half of the 64 banks, so the 16-column halves
// of rows 4 kb + 2, 4 kb + 3 are swapped to keep the four groups apart.
__device__ __forceinline__ int sl(int k, int c) { return k * kLC + (c ^ (((k >> 1) & 1) << 4)); }
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
    int nseg;                   // workgroups (segments) per sequence in the two sequential passes
    float *state_final;         // optional [N][Hv][128][128]: the state after each sequence's last
                                // chunk, from the recomputed forward (NULL: not written)
    bool forward_only;          // the recomputed forward for state_final alone: it stores no
                                // per-chunk state, Vt or Vn
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
    float *sdot;        // [chunk][Hv][kSD] <dS', S> of each (column block, wave): state
                        //                   gradient leaving the chunk, state entering it
    float *dwp;         // [chunk][C_tot][4] conv weight gradient of each chunk
    float *KK;          // [chunk][Hqk][64][64] k^ k^T of each (chunk, QK group)
};

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

// Sequential-pass block id -> (segment, sequence, V head, column block), so
// that the G * kNCB blocks of one (segment, sequence, QK group), which read
// the same k^ and q^ rows chunk after chunk, get ids of one residue mod 8:
// they run on the same XCD (blocks are dealt to the eight XCDs round-robin)
// and share its L2.  A tail of fewer than eight groups maps plainly.
__device__ __forceinline__ void seq_block(const BwdArgs &p, int &seg, int &s, int &h, int &cb)
{
    const int G = p.Hv / p.Hqk, P = G * kNCB, N = gridDim.x / p.nseg;
    const int b = blockIdx.x % N;
    seg = blockIdx.x / N;
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
// Segments of the two sequential passes.  A sequence of nch chunks is cut
// into ns <= p.nseg segments, each run by its own workgroups, in parallel.
// Segment 0 (the first chunks in the forward pass, the last ones in the
// state-gradient pass) starts from the given state or state gradient and is
// kBwdLead chunks longer; every other segment starts from zero a few chunks
// before its own (its warm-up, which stores nothing).  Each token's
// transition alpha (I - beta k k^T), and so its transpose, has spectral norm
// <= alpha (beta in (0,1), |k| = 1), so what a zero start drops reaches the
// segment scaled by at most the product of the warm-up chunks' decays.  The
// warm-up is the shortest one whose product is <= 2^-24, below fp32
// resolution of what it drops.  When a segment finds none within 64 chunks
// (weak or no decay), segment 0 runs the whole sequence and the others exit.
constexpr int kBwdLead = 4, kBwdMinSeg = 8, kBwdMaxSeg = 8;
constexpr float kBwdWarmLn = -16.6355323f;  // ln 2^-24

__device__ __forceinline__ int seg_count(const BwdArgs &p, int nch)
{
    return min(p.nseg, max(1, (nch - kBwdLead) / kBwdMinSeg));
}
// first chunk of segment k counted from the pass's start (k = ns: nch)
__device__ __forceinline__ int seg_bound(int nch, int ns, int k)
{
    if (k == 0) return 0;
    if (k >= ns) return nch;
    const int L = (nch - kBwdLead + ns - 1) / ns;
    return min(nch, kBwdLead + k * L);
}
// natural log of chunk c's decay: gamma at its last token
__device__ __forceinline__ float chunk_logdecay(const BwdArgs &p, const BwdWs &ws, int4 sq, int c, int h)
{
    const int n = min(kChunk, sq.w - c * kChunk);
    return ws.gam[((long)sq.z + (long)c * kChunk + n - 1) * p.Hv + h];
}
// Warm-up start of a segment.  kRev = false: the segment starts at chunk e,
// and the pass runs forward from the chunk returned (0: from the sequence
// start, exactly).  kRev = true: the segment ends before chunk e, and the
// pass runs backward from the chunk returned (nch - 1: from the sequence
// end, exactly).  -1: no warm-up within 64 chunks meets the bound.
// Wave-uniform.
template <bool kRev>
__device__ int seg_warm_start(const BwdArgs &p, const BwdWs &ws, int4 sq, int h, int e, int lane)
{
    const int nch = sq.y;
    const int c = kRev ? e + lane : e - 1 - lane;
    const bool in = kRev ? c < nch : c >= 0;
    float g = in ? chunk_logdecay(p, ws, sq, c, h) : 0.f;
    // inclusive prefix over lanes: log of the decay of the lane + 1 chunks next to the segment
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(g, off, 64);
        if (lane >= off) g += y;
    }
    const unsigned long long hit = __ballot(in && g <= kBwdWarmLn);
    int w;
    if (kRev) w = hit ? e + (int)__builtin_ctzll(hit) : (nch - e <= 64 ? nch - 1 : -1);
    else w = hit ? e - 1 - (int)__builtin_ctzll(hit) : (e <= 64 ? 0 : -1);
    return __builtin_amdgcn_readfirstlane(w);
}
// A workgroup's chunks: its own [lo, hi), which it stores, and j0, where its
// pass starts (kRev: going down), from the given state or state gradient
// when `exact`, else from zero.  false: nothing to do.
struct SegPlan {
    int lo, hi, j0;
    bool exact;
};
template <bool kRev>
__device__ bool seg_plan(const BwdArgs &p, const BwdWs &ws, int4 sq, int h, int seg, SegPlan &pl)
{
    __shared__ int wstart[kBwdMaxSeg];
    const int nch = sq.y, ns = seg_count(p, nch);
    if (seg >= ns) return false;
    if (ns > 1) {
        // wave k tests segment k; every workgroup of the sequence decides alike
        const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (w >= 1 && w < ns) {
            const int e = kRev ? nch - seg_bound(nch, ns, w) : seg_bound(nch, ns, w);
            const int st = seg_warm_start<kRev>(p, ws, sq, h, e, lane);
            if (lane == 0) wstart[w] = st;
        }
        __syncthreads();
        bool ok = true;
        for (int k = 1; k < ns; ++k) ok = ok && wstart[k] >= 0;
        if (!ok) {
            if (seg > 0) return false;
            pl.lo = 0;
            pl.hi = nch;
            pl.j0 = kRev ? nch - 1 : 0;
            pl.exact = true;
            return true;
        }
    }
    const int a = seg_bound(nch, ns, seg), b = seg_bound(nch, ns, seg + 1);
    pl.lo = kRev ? nch - b : a;
    pl.hi = kRev ? nch - a : b;
    if (seg == 0) {
        pl.j0 = kRev ? nch - 1 : 0;
        pl.exact = true;
    } else {
        pl.j0 = wstart[seg];
        pl.exact = pl.j0 == (kRev ? nch - 1 : 0);
    }
    return true;
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
// acc += A_blk B_blk for 16 x 16 blocks of row-major LDS matrices (row
// strides lda, ldb), on the fp32 matrix cores: lane l supplies A[l%16][k] and
// B[k][l%16] for k = 4 kb + l/16; acc in accumulator layout (lane (q, c):
// rows 4q .. 4q+3 of column c).
__device__ __forceinline__ f32x4 blk_mm(const float *Ab, int lda, const float *Bb, int ldb, f32x4 acc, int lane)
{
    const int r = lane & 15, k = lane >> 4;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Ab[r * lda + 4 * kb + k], Bb[(4 * kb + k) * ldb + r], acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ void blk_st(float *Db, int ldd, f32x4 v, int lane)
{
    const int c = lane & 15, q = lane >> 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) Db[(4 * q + e) * ldd + c] = v[e];
}

// Column c of the inverse of the 16 x 16 unit lower-triangular block I + A
// (A strictly lower, row stride kLN), y = e_c on entry: right-looking
// substitution, expanded at compile time so that y stays in registers.
template <int M>
struct SolveCol16b {
    static __device__ __forceinline__ void run(float (&y)[16], const float *A)
    {
        if constexpr (M < 15) {
#pragma unroll
            for (int ii = M + 1; ii < 16; ++ii) y[ii] = fmaf(-A[ii * kLN + M], y[M], y[ii]);
            SolveCol16b<M + 1>::run(y, A);
        }
    }
};

// X = (I + A)^-1 of one 64 x 64 strictly lower A (row stride kLN), in place,
// by one wave with wave-level synchronisation only: the four diagonal 16 x 16
// blocks by substitution (lane (q, c) takes column c of block q), then the
// blocks below them by the 2 x 2 block recursion
// [[X_a, 0], [L_ba, X_b]]^-1 = [[X_a, 0], [-X_b L_ba X_a, X_b]], within and
// across the 32 x 32 halves.  Block (0, 1), above the diagonal, holds the
// intermediate products; the blocks above the diagonal are left to the caller.
__device__ __forceinline__ void inverse64(float *H, int lane)
{
    auto B = [&](int i, int j) { return H + 16 * i * kLN + 16 * j; };
    auto wave_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    {
        const int q = lane >> 4, c = lane & 15;
        float y[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = i == c ? 1.f : 0.f;
        SolveCol16b<0>::run(y, B(q, q));
        wave_sync();
#pragma unroll
        for (int i = 0; i < 16; ++i) B(q, q)[i * kLN + c] = y[i];
        wave_sync();
    }
    float *tmp = B(0, 1);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    // X_10 = -X_11 (A_10 X_00), X_32 = -X_33 (A_32 X_22)
    blk_st(tmp, kLN, blk_mm(B(1, 0), kLN, B(0, 0), kLN, z, lane), lane);
    wave_sync();
    blk_st(B(1, 0), kLN, -blk_mm(B(1, 1), kLN, tmp, kLN, z, lane), lane);
    wave_sync();
    blk_st(tmp, kLN, blk_mm(B(3, 2), kLN, B(2, 2), kLN, z, lane), lane);
    wave_sync();
    blk_st(B(3, 2), kLN, -blk_mm(B(3, 3), kLN, tmp, kLN, z, lane), lane);
    wave_sync();
    // M_i0 = A_i0 X_00 + A_i1 X_10, M_i1 = A_i1 X_11 (i = 2, 3), over the A blocks
#pragma unroll
    for (int i = 2; i < 4; ++i) {
        f32x4 m = blk_mm(B(i, 0), kLN, B(0, 0), kLN, z, lane);
        m = blk_mm(B(i, 1), kLN, B(1, 0), kLN, m, lane);
        const f32x4 m1 = blk_mm(B(i, 1), kLN, B(1, 1), kLN, z, lane);
        wave_sync();
        blk_st(B(i, 0), kLN, m, lane);
        blk_st(B(i, 1), kLN, m1, lane);
        wave_sync();
    }
    // X_31 = -(X_32 M_21 + X_33 M_31), X_21 = -X_22 M_21
    {
        f32x4 x = blk_mm(B(3, 2), kLN, B(2, 1), kLN, z, lane);
        x = blk_mm(B(3, 3), kLN, B(3, 1), kLN, x, lane);
        const f32x4 x21 = blk_mm(B(2, 2), kLN, B(2, 1), kLN, z, lane);
        wave_sync();
        blk_st(B(3, 1), kLN, -x, lane);
        blk_st(B(2, 1), kLN, -x21, lane);
        wave_sync();
    }
    // X_30 = -(X_32 M_20 + X_33 M_30), X_20 = -X_22 M_20
    {
        f32x4 x = blk_mm(B(3, 2), kLN, B(2, 0), kLN, z, lane);
        x = blk_mm(B(3, 3), kLN, B(3, 0), kLN, x, lane);
        const f32x4 x20 = blk_mm(B(2, 2), kLN, B(2, 0), kLN, z, lane);
        wave_sync();
        blk_st(B(3, 0), kLN, -x, lane);
        blk_st(B(2, 0), kLN, -x20, lane);
        wave_sync();
    }
}

// One workgroup per (chunk, QK group): K^K^T and Q^K^T once (their lower
// 16 x 16 tiles on the fp32 matrix cores), then the group's V heads four at
// a time (their A matrices reuse the LDS of the k^ / q^ rows), wave w
// inverting head w's I + A.
constexpr int kLocalR = 4 * 64 * kLN;  // >= 2 * 64 * kLK: the k^ and q^ rows, or four A matrices
static_assert(kLocalR >= 2 * 64 * kLK, "the A matrices overlay the k^ and q^ rows");

__global__ __launch_bounds__(kBT) void bwd_local_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ __attribute__((aligned(16))) float R[kLocalR];
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
    // lower tiles (I, J <= I): K K^T by waves 0 (row blocks 0, 3) and 1
    // (1, 2), Q K^T by waves 2 and 3 likewise; lane (lq, lr) contracts
    // k = 32 lq .. 32 lq + 31 (a permutation of the 16x16x4 steps' k).  A
    // wave keeps its five tiles in registers (element e: row 16 I + 4 lq + e,
    // column 16 J + lr) until it has formed the A (or P) tiles of every head.
    constexpr int kTi[2][5] = {{0, 3, 3, 3, 3}, {1, 1, 2, 2, 2}}, kTj[2][5] = {{0, 0, 1, 2, 3}, {0, 1, 0, 1, 2}};
    const int lq = lane >> 4, lr = lane & 15, par = w & 1;
    const bool isk = w < 2;  // K K^T (then A) or Q K^T (then P)
    f32x4 tl[5];
    {
        const float *Asrc = isk ? Ks : Qs;
        float *kkg = ws.KK + ((long)cidx * Hqk + g) * 4096;
#pragma unroll
        for (int kt = 0; kt < 5; ++kt) {
            const int I = kTi[par][kt], J = kTj[par][kt];
            float a[32], b[32];
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                const float4 u = ld4(Asrc + (16 * I + lr) * kLK + 32 * lq + 4 * v);
                a[4 * v] = u.x; a[4 * v + 1] = u.y; a[4 * v + 2] = u.z; a[4 * v + 3] = u.w;
                const float4 u2 = ld4(Ks + (16 * J + lr) * kLK + 32 * lq + 4 * v);
                b[4 * v] = u2.x; b[4 * v + 1] = u2.y; b[4 * v + 2] = u2.z; b[4 * v + 3] = u2.w;
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 32; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], b[st], acc, 0, 0, 0);
            tl[kt] = acc;
            if (isk) {
#pragma unroll
                for (int e = 0; e < 4; ++e)  // for the per-head gradient kernel (lower tiles)
                    kkg[(16 * I + 4 * lq + e) * 64 + 16 * J + lr] = acc[e];
            }
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
        // A (strict lower) into LDS from the K K^T tiles, P (lower incl. the
        // diagonal) to the workspace from the Q K^T tiles, for each head;
        // the A tiles above the diagonal are never read, the P tiles above
        // it are written as zeros
        for (int jh = 0; jh < jn; ++jh) {
            const long mo = ((long)cidx * Hv + g * G + j0 + jh) * 4096;
#pragma unroll
            for (int kt = 0; kt < 5; ++kt) {
                const int I = kTi[par][kt], J = kTj[par][kt], jj = 16 * J + lr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * I + 4 * lq + e;
                    const float D = expf(gam[jh][i] - gam[jh][jj]);
                    if (isk)
                        R[jh * 64 * kLN + i * kLN + jj] = (jj < i && i < n) ? bet[jh][i] * tl[kt][e] * D : 0.f;
                    else
                        ws.P[mo + i * 64 + jj] = (jj <= i && i < n) ? tl[kt][e] * D : 0.f;
                }
            }
        }
        for (int idx = t; idx < jn * 1024; idx += kBT) {
            const int jh = idx >> 10, i = (idx >> 4) & 63, c4 = 4 * (idx & 15);
            if (c4 >= 16 * (i / 16 + 1))
                st4(ws.P + ((long)cidx * Hv + g * G + j0 + jh) * 4096 + i * 64 + c4, make_float4(0.f, 0.f, 0.f, 0.f));
        }
        __syncthreads();
        // X = (I + A)^-1 of head w, in place; written out whole, zero above the diagonal
        if (w < jn) {
            float *H = R + w * 64 * kLN;
            inverse64(H, lane);
            const long mo = ((long)cidx * Hv + g * G + j0 + w) * 4096;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int idx = lane + 64 * e, r = idx >> 4, c4 = 4 * (idx & 15);
                const float4 v = c4 >= 16 * (r / 16 + 1) ? make_float4(0.f, 0.f, 0.f, 0.f)
                                                         : *reinterpret_cast<const float4 *>(H + r * kLN + c4);
                st4(ws.X + mo + r * 64 + c4, v);
            }
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
            st4(slice + sl(r, 4 * q), make_float4(p.q_scale * bf16_lo(u.x), p.q_scale * bf16_hi(u.x),
                                                     p.q_scale * bf16_lo(u.y), p.q_scale * bf16_hi(u.y)));
        } else {
            st4(slice + sl(r, 4 * q), f.v[e]);
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
    int seg, s, h, cb;
    seq_block(p, seg, s, h, cb);
    const int g = h / G, col0 = cb * kCB;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, lr = lane & 15, lq = lane >> 4;
    const int srow = 16 * w + 4 * lq;                      // state rows srow .. srow + 3
    const int vrt = w >> 1, vrow = 16 * vrt + 4 * lq, vcol = 16 * (w & 1) + lr;  // slice tile
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const int4 sq = bseq(p, ws, s);  // {first chunk slot, chunks, first token, length}
    SegPlan pl;
    if (!seg_plan<false>(p, ws, sq, h, seg, pl)) return;
    f32x4 S[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[ct][e] = pl.exact && p.state_in
                           ? p.state_in[(((long)s * Hv + h) * kD + srow + e) * kD + col0 + 16 * ct + lr]
                           : 0.f;
    SeqPref<false> f;
    if (pl.j0 < pl.hi) {
        seq_fetch<false>(p, ws, f, sq.x + pl.j0, sq.z + (long)pl.j0 * kChunk, min(kChunk, sq.w - pl.j0 * kChunk),
                         h, g, col0);
        seq_commit<false>(p, f, L, nullptr, nullptr, Vs);
    }
    for (int j = pl.j0; j < pl.hi; ++j) {
        const int cidx = sq.x + j, n = min(kChunk, sq.w - j * kChunk);
        const long t0 = (long)sq.z + (long)j * kChunk;
        const bool own = j >= pl.lo && !p.forward_only;  // else a warm-up chunk: nothing stored
        float *sc = ws.Sc + ((long)cidx * Hv + h) * kD * kD + col0;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (own) sc[(long)(srow + e) * kD + 16 * ct + lr] = S[ct][e];
                Ss[sl(srow + e, 16 * ct + lr)] = S[ct][e];
            }
        if (j + 1 < pl.hi)
            seq_fetch<false>(p, ws, f, cidx + 1, t0 + kChunk, min(kChunk, sq.w - (j + 1) * kChunk), h, g, col0);
        __syncthreads();
        // Vt = V - diag(Gam) K S
        f32x4 acc = z4;
#pragma unroll 8
        for (int kb = 0; kb < kD / 4; ++kb)
            acc = mfma4(L.K[(16 * vrt + lr) * kLK + 4 * kb + lq], Ss[sl(4 * kb + lq, vcol)], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = vrow + e;
            const float vt = r < n ? Vs[sl(r, vcol)] - L.eg[r] * acc[e] : 0.f;
            Vts[sl(r, vcol)] = vt;
            if (own && r < n) ws.vt[((t0 + r) * Hv + h) * kD + col0 + vcol] = vt;
        }
        __syncthreads();
        // Vn = X diag(beta) Vt (X lower: k < 16 (vrt + 1))
        acc = z4;
        for (int kb = 0; kb < 4 * vrt + 4; ++kb) {
            const int k = 4 * kb + lq;
            acc = mfma4(L.X[(16 * vrt + lr) * kLN + k] * L.bet[k], Vts[sl(k, vcol)], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = vrow + e;
            const float vn = r < n ? acc[e] : 0.f;
            Vns[sl(r, vcol)] = vn;
            if (own && r < n) ws.vn[((t0 + r) * Hv + h) * kD + col0 + vcol] = vn;
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
            for (int ct = 0; ct < 2; ++ct) S[ct] = mfma4(a, Vns[sl(k, 16 * ct + lr)], S[ct]);
        }
        __syncthreads();
        if (j + 1 < pl.hi) seq_commit<false>(p, f, L, nullptr, nullptr, Vs);
    }
    // the workgroup that ends at the sequence's last chunk leaves the final state
    if (p.state_final && pl.hi == sq.y) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.state_final[(((long)s * Hv + h) * kD + srow + e) * kD + col0 + 16 * ct + lr] = S[ct][e];
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
    int seg, s, h, cb;
    seq_block(p, seg, s, h, cb);
    const int g = h / G, col0 = cb * kCB;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, lr = lane & 15, lq = lane >> 4;
    const int srow = 16 * w + 4 * lq;
    const int vrt = w >> 1, vrow = 16 * vrt + 4 * lq, vcol = 16 * (w & 1) + lr;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const long so = ((long)s * Hv + h) * kD * kD + col0;
    const int4 sq = bseq(p, ws, s);  // {first chunk slot, chunks, first token, length}
    SegPlan pl;
    if (!seg_plan<true>(p, ws, sq, h, seg, pl)) return;
    f32x4 dS[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dS[ct][e] = pl.exact && p.grad_state_out ? p.grad_state_out[so + (long)(srow + e) * kD + 16 * ct + lr]
                                                     : 0.f;
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
    if (pl.j0 >= pl.lo) {
        load_sv(sq.x + pl.j0);
        seq_fetch<true>(p, ws, f, sq.x + pl.j0, sq.z + (long)pl.j0 * kChunk, min(kChunk, sq.w - pl.j0 * kChunk), h,
                        g, col0);
        seq_commit<true>(p, f, L, Qs, Ps, dOs);
    }
    for (int j = pl.j0; j >= pl.lo; --j) {
        const int cidx = sq.x + j, n = min(kChunk, sq.w - j * kChunk);
        const long t0 = (long)sq.z + (long)j * kChunk;
        const bool own = j < pl.hi;  // else a warm-up chunk: nothing stored
        float *dsc = ws.dSc + ((long)cidx * Hv + h) * kD * kD + col0;
        float part = 0.f;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (own) dsc[(long)(srow + e) * kD + 16 * ct + lr] = dS[ct][e];
                dSs[sl(srow + e, 16 * ct + lr)] = dS[ct][e];
                part = fmaf(dS[ct][e], sv[4 * ct + e], part);
            }
        part = wave_sum(part);
        if (own && lane == 0) ws.sdot[((long)cidx * Hv + h) * kSD + (kST / 64) * cb + w] = part;
        if (j > pl.lo) load_sv(cidx - 1);
        if (j > pl.lo) seq_fetch<true>(p, ws, f, cidx - 1, t0 - kChunk, kChunk, h, g, col0);
        __syncthreads();
        // dVn = diag(en) K dS' + P^T dO'  (P^T upper: k >= 16 vrt)
        f32x4 acc = z4;
#pragma unroll 8
        for (int kb = 0; kb < kD / 4; ++kb)
            acc = mfma4(L.K[(16 * vrt + lr) * kLK + 4 * kb + lq], dSs[sl(4 * kb + lq, vcol)], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= L.en[vrow + e];
        for (int kb = 4 * vrt; kb < 16; ++kb) {
            const int k = 4 * kb + lq;
            acc = mfma4(Ps[k * kLN + 16 * vrt + lr], dOs[sl(k, vcol)], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = vrow + e;
            const float v = r < n ? acc[e] : 0.f;
            dVns[sl(r, vcol)] = v;
            if (own && r < n) ws.dvn[((t0 + r) * Hv + h) * kD + col0 + vcol] = v;
        }
        __syncthreads();
        // dVt = T'^T dVn = diag(beta) X^T dVn
        acc = z4;
        for (int kb = 4 * vrt; kb < 16; ++kb) {
            const int k = 4 * kb + lq;
            acc = mfma4(L.X[k * kLN + 16 * vrt + lr], dVns[sl(k, vcol)], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = vrow + e;
            const float v = r < n ? L.bet[r] * acc[e] : 0.f;
            dVts[sl(r, vcol)] = v;
            if (own && r < n) ws.dvh[((t0 + r) * Hv + h) * kD + col0 + vcol] = v;
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
                dS[ct] = mfma4(aq, dOs[sl(k, 16 * ct + lr)], dS[ct]);
                dS[ct] = mfma4(ak, dVts[sl(k, 16 * ct + lr)], dS[ct]);
            }
        }
        __syncthreads();
        if (j > pl.lo) seq_commit<true>(p, f, L, Qs, Ps, dOs);
    }
    if (p.grad_state_in && pl.lo == 0) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.grad_state_in[so + (long)(srow + e) * kD + 16 * ct + lr] = dS[ct][e];
    }
}

// ---------------------------------------------------------------------------
// 5. per-chunk gradients
// ---------------------------------------------------------------------------
// acc[m][ri] += sum_k A(r0 + ri, k) B(k, cc + 16 m) for k < K (a multiple
// of 32), r0 = 4 (t / 16), cc = t % 16, m < NC: a 64 x (16 NC) product on
// the fp32 matrix cores (16x16x4 steps), staged through LDS 32 deep.  Wave w
// computes row tile w: its accumulator layout (lane (q, c) holds rows
// 4q .. 4q+3 of column c) is exactly the thread layout above, so acc[m] is
// the accumulator of column tile m.  The sources are read 16 bytes at a time
// along their contiguous dimension: fa4(r, k) is A(r, k..k+3) when AK, else
// A(r..r+3, k); fb4(k, c) is B(k..k+3, c) when BK, else B(k, c..c+3).
// Staged slices hold A by rows and B by columns, 32 k-values (128 bytes) per
// row, the eight 16-byte pieces of row (or column) x stored at piece
// p ^ ((x >> 1) & 7): a lane reads the 8 k-values 8q .. 8q+7 of its row as
// two 16-byte pieces, and the sixteen lanes of a quarter wave then cover all
// 64 banks.  Step s of a slice contracts k = 8q + s in lane group q (the
// same permutation of k for A and B).
__device__ __forceinline__ int gslot(int x, int k) { return x * 32 + ((((k >> 2) ^ (x >> 1)) & 7) << 2) + (k & 3); }

template <int NC, bool AK, bool BK>
__device__ __forceinline__ void gemm_stage(const float4 (&va)[2], const float4 (&vb)[NC / 2], float *sA, float *sB)
{
    const int t = threadIdx.x;
    constexpr int NCOL = 16 * NC;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int idx = t + kBT * e;
        if (AK) {
            *reinterpret_cast<float4 *>(sA + gslot(idx >> 3, 4 * (idx & 7))) = va[e];
        } else {
            const int r = 4 * (idx & 15), k = idx >> 4;
            sA[gslot(r, k)] = va[e].x;
            sA[gslot(r + 1, k)] = va[e].y;
            sA[gslot(r + 2, k)] = va[e].z;
            sA[gslot(r + 3, k)] = va[e].w;
        }
    }
#pragma unroll
    for (int e = 0; e < NC / 2; ++e) {
        const int idx = t + kBT * e;
        if (BK) {
            *reinterpret_cast<float4 *>(sB + gslot(idx >> 3, 4 * (idx & 7))) = vb[e];
        } else {
            const int k = idx / (NCOL / 4), c = 4 * (idx % (NCOL / 4));
            sB[gslot(c, k)] = vb[e].x;
            sB[gslot(c + 1, k)] = vb[e].y;
            sB[gslot(c + 2, k)] = vb[e].z;
            sB[gslot(c + 3, k)] = vb[e].w;
        }
    }
}

// The eight k-values 8q .. 8q+7 of staged row x
__device__ __forceinline__ void gemm_frag(const float *src, int x, int q, float (&v)[8])
{
    const float4 lo = *reinterpret_cast<const float4 *>(src + gslot(x, 8 * q));
    const float4 hi = *reinterpret_cast<const float4 *>(src + gslot(x, 8 * q + 4));
    v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
    v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
}

// One staged slice: acc (column tiles m < NC of the wave's row tile) += A B
template <int NC>
__device__ __forceinline__ void gemm_slice(f32x4 (&acc)[NC], const float *sA, const float *sB)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, q = lane >> 4, r16 = lane & 15;
    float a[8], b[2][8];
    gemm_frag(sA, 16 * w + r16, q, a);
    gemm_frag(sB, r16, q, b[0]);
#pragma unroll
    for (int m = 0; m < NC; ++m) {
        if (m + 1 < NC) gemm_frag(sB, 16 * (m + 1) + r16, q, b[(m + 1) & 1]);  // the next tile's column in flight
#pragma unroll
        for (int st = 0; st < 8; ++st)
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], b[m & 1][st], acc[m], 0, 0, 0);
    }
}

template <int NC, bool AK, bool BK, class FA4, class FB4>
__device__ __forceinline__ void gemm64(f32x4 (&acc)[8], int K, FA4 fa4, FB4 fb4, float *sA, float *sB)
{
    const int t = threadIdx.x;
    constexpr int NCOL = 16 * NC;
    // the sources of slice k0 + 32 are requested before slice k0's products,
    // so that their latency overlaps them
    float4 va[2], vb[NC / 2];
    auto fetch = [&](int k0) {
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
    };
    f32x4 (&d)[NC] = reinterpret_cast<f32x4 (&)[NC]>(acc);
    fetch(0);
    for (int k0 = 0; k0 < K; k0 += 32) {
        gemm_stage<NC, AK, BK>(va, vb, sA, sB);
        __syncthreads();
        if (k0 + 32 < K) fetch(k0 + 32);
        gemm_slice<NC>(d, sA, sB);
        __syncthreads();
    }
}

// Two 64-row products over the same B: acc1 += A1 B and acc2 += A2 B, with
// the B slice staged once per 32-deep step (A row-major sources, B k-major,
// as gemm64<8, true, true>).
template <class FA4, class FA4b, class FB4>
__device__ __forceinline__ void gemm64x2(f32x4 (&acc1)[8], f32x4 (&acc2)[8], int K, FA4 fa1, FA4b fa2, FB4 fb4,
                                         float *sA1, float *sA2, float *sB)
{
    const int t = threadIdx.x;
    float4 va1[2], va2[2], vb[4];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int idx = t + kBT * e;
            va1[e] = fa1(idx >> 3, k0 + 4 * (idx & 7));
            va2[e] = fa2(idx >> 3, k0 + 4 * (idx & 7));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = t + kBT * e;
            vb[e] = fb4(k0 + 4 * (idx & 7), idx >> 3);
        }
    };
    f32x4 (&d1)[8] = acc1, (&d2)[8] = acc2;
    fetch(0);
    for (int k0 = 0; k0 < K; k0 += 32) {
        gemm_stage<8, true, true>(va1, vb, sA1, sB);
#pragma unroll
        for (int e = 0; e < 2; ++e)
            *reinterpret_cast<float4 *>(sA2 + gslot((t + kBT * e) >> 3, 4 * ((t + kBT * e) & 7))) = va2[e];
        __syncthreads();
        if (k0 + 32 < K) fetch(k0 + 32);
        gemm_slice<8>(d1, sA1, sB);
        gemm_slice<8>(d2, sA2, sB);
        __syncthreads();
    }
}

__device__ __forceinline__ void zero(f32x4 (&acc)[8])
{
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
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
    __shared__ __attribute__((aligned(16))) float sA[64 * 32], sB[128 * 32];
    __shared__ __attribute__((aligned(16))) float Em[64 * kLN], Wm[64 * kLN], Ym[64 * kLN];
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
    f32x4 acc[8], dK[8];  // [column tile m][row ri]: the accumulator layout
    {
        // ---- dq^ first, so that its registers are free before the rest of dk^ is formed
        f32x4 dQ[8];
        zero(dQ);
        // (c) O = q_scale (diag(Gam) Q S + ...): E1 = dO' S^T, and (e) Vt = V -
        //     diag(Gam) K S: E2 = dVt S^T, in one pass over S (the second A
        //     slice is staged in Ym, which is free until (f))
        zero(acc);
        zero(dK);
        gemm64x2(acc, dK, kD, DO4, [&](int r, int c) { return V4(ws.dvh, r, c); },
                 [&](int c, int i) { return ld4(Sc + i * kD + c); }, sA, Ym, sB);
        {
            float part[4];
#pragma unroll
            for (int ri = 0; ri < 4; ++ri) {
                const int r = r0 + ri;
                part[ri] = 0.f;
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    part[ri] = fmaf(dK[m][ri], KH(r, cc + 16 * m), part[ri]);
                    dK[m][ri] *= -eg[r];
                }
            }
            row_apply(part, dgam, eg, -1.f);
        }
        float part[4];
#pragma unroll
        for (int ri = 0; ri < 4; ++ri) {
            const int r = r0 + ri;
            part[ri] = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                dQ[m][ri] += eg[r] * acc[m][ri];
                part[ri] = fmaf(acc[m][ri], QH(r, cc + 16 * m), part[ri]);
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
                Em[r * kLN + jj] = in ? acc[m][ri] * ws.P[mo + r * 64 + jj] : 0.f;
                Wm[r * kLN + jj] = in ? acc[m][ri] * expf(gam[r] - gam[jj]) : 0.f;
            }
        __syncthreads();
        gemm64<8, true, false>(dQ, 64, [&](int r, int jj) { return L4(Wm + r * kLN + jj); }, KH4, sA, sB);
#pragma unroll
        for (int ri = 0; ri < 4; ++ri) {
            const int r = r0 + ri;
            if (r >= n) continue;
#pragma unroll
            for (int m = 0; m < 8; ++m) ws.dqp[((t0 + r) * Hv + h) * kD + cc + 16 * m] = dQ[m][ri];
        }
    }
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
                dK[m][ri] += en[r] * acc[m][ri];
                part[ri] = fmaf(acc[m][ri], KH(r, cc + 16 * m), part[ri]);
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
            Ym[r * kLN + jj] = in ? acc[m][ri] * ws.X[mo + r * 64 + jj] : 0.f;
            Wm[r * kLN + jj] = in ? acc[m][ri] * bet[jj] : 0.f;
        }
    __syncthreads();
    if (t < n) {
        // column t below the diagonal, rows t .. n-1 in order (a fixed-count
        // loop, so that its reads go out together; rows outside add nothing)
        float cs = 0.f;
#pragma unroll 16
        for (int r = 0; r < 64; ++r) {
            const float y = Ym[r * kLN + t];
            cs = r >= t && r < n ? cs + y : cs;
        }
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
        for (int m = 0; m < 4; ++m) Ym[(r0 + ri) * kLN + cc + 16 * m] = acc[m][ri];
    __syncthreads();
    zero(acc);
    gemm64<4, true, true>(acc, 64, [&](int r, int m) { return L4(Ym + r * kLN + m); },
                          [&](int m, int jj) { return ld4(ws.X + mo + jj * 64 + m); }, sA, sB);
#pragma unroll
    for (int ri = 0; ri < 4; ++ri)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int r = r0 + ri, jj = cc + 16 * m;
            Wm[r * kLN + jj] = (jj < r && r < n) ? -acc[m][ri] : 0.f;
        }
    __syncthreads();
    // (h) A = diag(beta) K K^T * D (strict lower): dbeta_i, Em += dA * A, dKK -> Ym;
    //     K K^T of the QK group as the chunk-local pass formed it (the same
    //     multiply-adds in the same order)
    {
        const float *kkg = ws.KK + ((long)cidx * Hqk + g) * 4096;
#pragma unroll
        for (int ri = 0; ri < 4; ++ri)
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[m][ri] = kkg[(r0 + ri) * 64 + cc + 16 * m];
    }
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
                    Em[r * kLN + jj] += dA * bet[r] * acc[m][ri] * D;
                    part[ri] = fmaf(dA, acc[m][ri] * D, part[ri]);
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
        float dg = 0.f;  // rows n-1 down to t, in that order
#pragma unroll 16
        for (int r = 63; r >= 0; --r) {
            const float v = dgam[r];
            dg = r >= t && r < n ? dg + v : dg;
        }
        const long ti = (t0 + t) * Hv + h;
        p.grad_a[ti] = dg * (-p.gate_scale * sigm(p.a[ti]));
        p.grad_b[ti] = dbet[t] * bet[t] * (1.f - bet[t]);
    }
#pragma unroll
    for (int ri = 0; ri < 4; ++ri) {
        const int r = r0 + ri;
        if (r >= n) continue;
#pragma unroll
        for (int m = 0; m < 8; ++m) ws.dkp[((t0 + r) * Hv + h) * kD + cc + 16 * m] = dK[m][ri];
    }
}

// ---------------------------------------------------------------------------
// 6. back through the L2 norm and SiLU to the conv outputs, then through the
//    conv, per (chunk, channel plane)
// ---------------------------------------------------------------------------
// The conv-output gradient dy of the chunk's rows and of the three rows after
// it (which the conv backward of its last rows reads) is formed into LDS and
// consumed there: row x of the conv input feeds outputs x .. x + 3.  The three
// rows after the chunk are formed again by the next chunk's workgroup; the
// arithmetic is the same, so both see the same values.
constexpr int kDyRows = kChunk + 3;
constexpr int kDyHalf = (kDyRows + 1) / 2;  // rows per thread half when forming dy
constexpr int kDyWin = kDyHalf + 3;         // their conv input window

// Raw rows tb - 3 .. tb - 3 + NW - 1 of channel c of a plane (carried rows,
// or zeros, before the sequence; zeros past it), loaded together
template <int NW>
__device__ __forceinline__ void x_window_n(const BwdArgs &p, const Plane &P, const uint16_t *x, int s, long seq0,
                                           int tb, int L, int c, long C_tot, float (&xw)[NW])
{
    uint16_t raw[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) raw[i] = x[(seq0 + min(max(tb - 3 + i, 0), L - 1)) * P.ld + c];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int tau = tb - 3 + i;
        float v = 0.f;
        if (tau >= 0 && tau < L)
            v = bf16_to_f32(raw[i]);
        else if (tau < 0 && p.conv_state_in)
            v = bf16_to_f32(p.conv_state_in[((long)s * 3 + 3 + tau) * C_tot + P.ch0 + c]);
        xw[i] = v;
    }
}

__global__ __launch_bounds__(kBT) void bwd_dyconv_kernel(BwdArgs p, BwdWs ws)
{
    __shared__ float zs[kDyRows * kLK], ds[kDyRows * kLK];  // SiLU output, its gradient, then dy
    __shared__ float nrm[kDyRows], zd[kDyRows];
    __shared__ float wpart[2][kD][4];
    const int cidx = blockIdx.x;
    const int4 ci = bchunk(p, ws, cidx);
    const int s = ci.x, n = ci.z, j = ci.w;
    const long C_tot = 2L * p.Hqk * kD + (long)p.Hv * kD;
    const Plane P = plane_of(p, blockIdx.y);
    const int t = threadIdx.x, c = t & 127, rh = t >> 7;
    const long ch = P.ch0 + c;
    if (n == 0) {  // an empty chunk slot contributes nothing to the weight gradient
        if (t < kD)
            for (int jj = 0; jj < 4; ++jj) ws.dwp[((long)cidx * C_tot + P.ch0 + t) * 4 + jj] = 0.f;
        return;
    }
    const long seq0 = ci.y, t0 = seq0 + (long)j * kChunk;
    const int L = bseq(p, ws, s).w;
    const int m = min(n + 3, L - j * kChunk);  // rows of dy formed: the chunk's, and up to three after it
    const int G = p.Hv / p.Hqk;
    const uint16_t *x = plane_src(p, P);
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_to_f32(p.conv_w[ch * 4 + i]);
    {
        // ---- dy of rows rb .. rb + kDyHalf - 1 (those below m) of channel c
        const int rb = kDyHalf * rh;
        float xw[kDyWin];
        x_window_n<kDyWin>(p, P, x, s, seq0, j * kChunk + rb, L, c, C_tot, xw);
        const long hs = (long)p.Hv * kD;
        float dsum[kDyHalf];
        // rows past m read row m - 1 (in bounds) and are not used
        if (P.kind == 2) {
            const float *gv = ws.dvh + t0 * hs + (long)P.head * kD + c;
#pragma unroll
            for (int r = 0; r < kDyHalf; ++r) dsum[r] = gv[min(rb + r, m - 1) * hs];
        } else {
#pragma unroll
            for (int r = 0; r < kDyHalf; ++r) dsum[r] = 0.f;
            for (int jh = 0; jh < G; ++jh) {
                const float *pj = (P.kind == 0 ? ws.dqp : ws.dkp) + t0 * hs + (long)(P.head * G + jh) * kD + c;
#pragma unroll
                for (int r = 0; r < kDyHalf; ++r) dsum[r] += pj[min(rb + r, m - 1) * hs];
            }
        }
        // v: dy = dv^ SiLU'(y).  q, k: the SiLU output z and its gradient, for the norm
#pragma unroll
        for (int r = 0; r < kDyHalf; ++r) {
            if (rb + r < m) {
                float y = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) y = fmaf(w[i], xw[r + i], y);
                if (P.kind == 2) {
                    ds[(rb + r) * kLK + c] = dsum[r] * silu_grad(y);
                } else {
                    zs[(rb + r) * kLK + c] = y * sigm(y);
                    ds[(rb + r) * kLK + c] = dsum[r];
                }
            }
        }
        __syncthreads();
        if (P.kind != 2) {
            // ---- q, k: back through the L2 norm, row by row (four threads a row)
            for (int r0 = 0; r0 < m; r0 += kBT / 4) {
                const int r = r0 + (t >> 2), pt = t & 3;
                float ss = 0.f, sd = 0.f;
                if (r < m)
                    for (int i = 0; i < 32; ++i) {
                        const float z = zs[r * kLK + pt * 32 + i];
                        ss = fmaf(z, z, ss);
                        sd = fmaf(z, ds[r * kLK + pt * 32 + i], sd);
                    }
                ss += __shfl_xor(ss, 1, 64);
                ss += __shfl_xor(ss, 2, 64);
                sd += __shfl_xor(sd, 1, 64);
                sd += __shfl_xor(sd, 2, 64);
                if (pt == 0 && r < m) {
                    nrm[r] = sqrtf(ss + 1e-6f);
                    zd[r] = sd;
                }
            }
            __syncthreads();
            // dy = (dz / |z| - z <z, dz> / |z|^3) SiLU'(y), over ds in place
#pragma unroll
            for (int r = 0; r < kDyHalf; ++r) {
                const int rr = rb + r;
                if (rr < m) {
                    float y = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) y = fmaf(w[i], xw[r + i], y);
                    const float rn = nrm[rr];
                    const float dz = ds[rr * kLK + c] / rn - zs[rr * kLK + c] * zd[rr] / (rn * rn * rn);
                    ds[rr * kLK + c] = dz * silu_grad(y);
                }
            }
        }
        __syncthreads();
    }
    // ---- back through the conv: thread (c, rh) takes rows 32 rh .. 32 rh + 31
    float *gx = (P.kind == 0 ? p.grad_q : P.kind == 1 ? p.grad_k : p.grad_v) + (long)P.head * kD;
    const int rb = 32 * rh, tb = j * kChunk + rb;
    float dw[kWin], xw[kWin];
#pragma unroll
    for (int i = 0; i < kWin; ++i) dw[i] = rb + i < m ? ds[(rb + i) * kLK + c] : 0.f;  // zero past the sequence
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
    // sixteen chunks' loads in flight at a time, added in chunk order
    float acc = 0.f;
    int c = 0;
    for (; c + 16 <= n_chunks; c += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = ws.dwp[(long)(c + u) * n_elems + e];
#pragma unroll
        for (int u = 0; u < 16; ++u) acc += v[u];
    }
    for (; c < n_chunks; ++c) acc += ws.dwp[(long)c * n_elems + e];
    p.grad_conv_w[e] = acc;
}

__global__ __launch_bounds__(kBT) void bwd_fill_kernel(float *dst, long n)
{
    const long e = (long)blockIdx.x * kBT + threadIdx.x;
    if (e < n) dst[e] = 0.f;
}

// ---------------------------------------------------------------------------
// Windows of one sequence (a backward run in pieces of whole chunks)
// ---------------------------------------------------------------------------
// dst[e] += src[e]
__global__ __launch_bounds__(kBT) void bwd_accum_kernel(float *dst, const float *src, long n)
{
    const long e = (long)blockIdx.x * kBT + threadIdx.x;
    if (e < n) dst[e] += src[e];
}

// The three raw rows before a window, tokens tok0 .. tok0 + 2 of q, k and v,
// as conv history rows [3][C_tot] (channel order q | k | v)
__global__ __launch_bounds__(kBT) void bwd_hist_kernel(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                                       uint16_t *rows, long tok0, int Hqk, int Hv)
{
    const long nq = (long)Hqk * kD, C_tot = 2 * nq + (long)Hv * kD;
    const long e = (long)blockIdx.x * kBT + threadIdx.x;
    if (e >= 3 * C_tot) return;
    const long r = e / C_tot, c = e % C_tot, tok = tok0 + r;
    rows[e] = c < nq ? q[tok * nq + c] : c < 2 * nq ? k[tok * nq + c - nq] : v[tok * Hv * kD + c - 2 * nq];
}

// The gradient of a window's history rows [3][C_tot] added into the gradients
// of the raw rows tok0 .. tok0 + 2, which the window before it has written
__global__ __launch_bounds__(kBT) void bwd_addrows_kernel(const float *g, float *gq, float *gk, float *gv,
                                                          long tok0, int Hqk, int Hv)
{
    const long nq = (long)Hqk * kD, C_tot = 2 * nq + (long)Hv * kD;
    const long e = (long)blockIdx.x * kBT + threadIdx.x;
    if (e >= 3 * C_tot) return;
    const long r = e / C_tot, c = e % C_tot, tok = tok0 + r;
    float *dst = c < nq ? gq + tok * nq + c : c < 2 * nq ? gk + tok * nq + c - nq : gv + tok * Hv * kD + c - 2 * nq;
    *dst += g[e];
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
constexpr int kBwdRegions = 20;  // two int4 tables and the eighteen float regions of BwdWs
struct BwdLayout {
    long off[kBwdRegions];
    long total;
};
BwdLayout bwd_layout(int N, int T_tot, int max_chunks, int Hqk, int Hv)
{
    const long tok = T_tot, chunks = max_chunks;
    const long C_tot = 2L * Hqk * kD + (long)Hv * kD;
    const long sizes[kBwdRegions] = {chunks * 4, (long)N * 4,  // int4 tables
                            tok * Hqk * kD, tok * Hqk * kD, tok * Hv * kD, tok * Hv, tok * Hv,
                            chunks * Hv * 4096, chunks * Hv * 4096, chunks * Hv * kD * kD, chunks * Hv * kD * kD,
                            tok * Hv * kD, tok * Hv * kD, tok * Hv * kD, tok * Hv * kD, tok * Hv * kD,
                            tok * Hv * kD, chunks * C_tot * 4, chunks * Hv * kSD, chunks * Hqk * 4096};
    BwdLayout L{};
    long o = 0;
    for (int i = 0; i < kBwdRegions; ++i) {
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

// Segments per sequence of the two sequential passes, from a makespan model
// for sequences of the mean length: blocks = units x segments, run in rounds
// of 256 resident blocks (one per CU), each round as long as a segment plus
// its warm-up (taken as kBwdLead chunks; segment 0, that much longer, has
// none).  The cheapest cut wins; ties go to fewer segments.
int bwd_choose_nseg(int N, int T_tot, int Hv)
{
    constexpr long kSlots = 256;
    if (N <= 0 || T_tot <= 0) return 1;
    const int nch = (int)(((long)T_tot / N + kChunk - 1) / kChunk);
    const long units = (long)N * Hv * kNCB;
    long best_cost = -1;
    int best = 1;
    for (int ns = 1; ns <= kBwdMaxSeg; ++ns) {
        if (ns > 1 && (nch - kBwdLead) / kBwdMinSeg < ns) break;
        const long L = ns == 1 ? nch : (nch - kBwdLead + ns - 1) / ns;
        const long rounds = (units * ns + kSlots - 1) / kSlots;
        const long cost = rounds * (L + (ns > 1 ? kBwdLead : 0));
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = ns;
        }
    }
    return best;
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
                           float q_scale, float *state_final, bool forward_only, void *workspace,
                           hipStream_t stream)
{
    BwdArgs p{};
    p.state_final = state_final;
    p.forward_only = forward_only;
    p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.conv_w = conv_w; p.conv_state_in = conv_state_in;
    p.state_in = state_in; p.grad_o = grad_o; p.grad_state_out = grad_state_out;
    p.grad_q = grad_q; p.grad_k = grad_k; p.grad_v = grad_v; p.grad_a = grad_a; p.grad_b = grad_b;
    p.grad_conv_w = grad_conv_w; p.grad_conv_state_in = grad_conv_state_in; p.grad_state_in = grad_state_in;
    p.cu_seqlens = cu_seqlens; p.N = N; p.T = T; p.nc = (T + kChunk - 1) / kChunk;
    p.T_tot = T_tot; p.max_chunks = T_tot > 0 ? bwd_max_chunks(cu_seqlens, N, T_tot) : 0;
    p.Hqk = Hqk; p.Hv = Hv; p.gate_scale = gate_scale; p.q_scale = q_scale;
    p.nseg = bwd_choose_nseg(N, T_tot, Hv);
    const long C_tot = 2L * Hqk * kD + (long)Hv * kD;
    BwdWs ws{};
    if (T_tot > 0) {
        const BwdLayout L = bwd_layout(N, T_tot, p.max_chunks, Hqk, Hv);
        float *base = static_cast<float *>(workspace);
        ws.chunk_info = reinterpret_cast<int4 *>(base + L.off[0]);
        ws.seq_info = reinterpret_cast<int4 *>(base + L.off[1]);
        float **slots[kBwdRegions - 2] = {&ws.qh, &ws.kh, &ws.vh, &ws.gam, &ws.beta, &ws.X, &ws.P, &ws.Sc, &ws.dSc,
                             &ws.vt, &ws.vn, &ws.dvn, &ws.dvh, &ws.dqp, &ws.dkp, &ws.dwp, &ws.sdot, &ws.KK};
        for (int i = 0; i < kBwdRegions - 2; ++i) *slots[i] = base + L.off[i + 2];
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
        hipLaunchKernelGGL(bwd_fwd_kernel, dim3(N * Hv * kNCB * p.nseg), dim3(kST), 0, stream, p, ws);
    }
    if (forward_only) return hipGetLastError();  // the recomputed forward alone (state_final)
    // also with no tokens: the state gradient passes straight through
    hipLaunchKernelGGL(bwd_chain_kernel, dim3(N * Hv * kNCB * p.nseg), dim3(kST), 0, stream, p, ws);
    if (grad_conv_state_in && (chunks == 0 || p.cu_seqlens)) {
        // rows of sequences without a first chunk (empty ones) stay zero
        const long nh = (long)N * 3 * C_tot;
        hipLaunchKernelGGL(bwd_fill_kernel, dim3((nh + kBT - 1) / kBT), dim3(kBT), 0, stream, grad_conv_state_in, nh);
    }
    const long nw = C_tot * 4;
    if (chunks > 0) {
        hipLaunchKernelGGL(bwd_grad_kernel, dim3(chunks * Hv), dim3(kBT), 0, stream, p, ws);
        hipLaunchKernelGGL(bwd_dyconv_kernel, dim3(chunks, planes), dim3(kBT), 0, stream, p, ws);
        hipLaunchKernelGGL(bwd_dw_kernel, dim3((nw + kBT - 1) / kBT), dim3(kBT), 0, stream, p, ws, nw, chunks);
    } else {
        hipLaunchKernelGGL(bwd_fill_kernel, dim3((nw + kBT - 1) / kBT), dim3(kBT), 0, stream, grad_conv_w, nw);
    }
    return hipGetLastError();
}

// The window kernels of a backward run in pieces (one sequence at a time)
hipError_t launch_bwd_accum(float *dst, const float *src, long n, hipStream_t stream)
{
    hipLaunchKernelGGL(bwd_accum_kernel, dim3((n + kBT - 1) / kBT), dim3(kBT), 0, stream, dst, src, n);
    return hipGetLastError();
}

hipError_t launch_bwd_hist(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *rows, long tok0,
                           int Hqk, int Hv, hipStream_t stream)
{
    const long n = 3 * (2L * Hqk * kD + (long)Hv * kD);
    hipLaunchKernelGGL(bwd_hist_kernel, dim3((n + kBT - 1) / kBT), dim3(kBT), 0, stream, q, k, v, rows, tok0, Hqk,
                       Hv);
    return hipGetLastError();
}

hipError_t launch_bwd_addrows(const float *g, float *gq, float *gk, float *gv, long tok0, int Hqk, int Hv,
                              hipStream_t stream)
{
    const long n = 3 * (2L * Hqk * kD + (long)Hv * kD);
    hipLaunchKernelGGL(bwd_addrows_kernel, dim3((n + kBT - 1) / kBT), dim3(kBT), 0, stream, g, gq, gk, gv, tok0,
                       Hqk, Hv);
    return hipGetLastError();
}

}  // namespace gdn
