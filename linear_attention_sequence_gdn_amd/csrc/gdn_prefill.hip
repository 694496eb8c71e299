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
//   Vnew = T' (V - diag(Gam) K S)                          (S: state entering)
//   O    = diag(Gam) Q S + (Q K^T * D, lower incl. diag) Vnew
//   S   <- Gam_n S + (diag(Gam_n / Gam) K)^T Vnew
//
// which equals the token-by-token recurrence up to rounding order.  (The
// usual W = T' diag(Gam) K and U' = T' V are never formed: Vnew is one more
// 64 x 64 product of the sequential pass, which spares writing both to HBM
// and reading them back.)
//
// Launches:
//   setup     -- chunk, sequence and segment tables from cu_seqlens
//                (device-side, no host sync); uniform batches compute the
//                same entries arithmetically and skip it;
//   prep      -- per (chunk, QK group): conv + SiLU + L2 norm of q and k,
//                written as matrix-core operands; K K^T and K Q^T on the
//                matrix cores; per V head of the group: gates, A, P, the
//                blocked unit-lower-triangular inverse, T';
//   chain     -- the sequential pass over (segment, V head): conv + SiLU of v
//                and every product that involves the state; each wave
//                carries 16 columns of S in registers.  A segment whose
//                warm-up bound fails carries its transition matrix as well;
//                the last workgroup of a (sequence, V head) to finish chains
//                the segments' affine maps in order, and extra workgroups
//                form those segments' outputs from the states it hands them.
#include "gdn_prefill.h"

namespace gdn {

namespace {

constexpr int kPrepThreads = 256;
constexpr int kQ_LD = 136;  // fp16 row stride of the token-major q^ / k^ tiles

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

// The q^ and k^ operand fragments the sequential pass reads hold their two
// 8-byte halves in swapped order in the lanes of odd lane groups (lane / 16
// odd): element i of such a lane is contraction index kappa(q, i ^ 4).  The
// state operand they meet is packed the same way, so the products are
// unchanged; what it buys is that the transposed reads of k^ (which read one
// half of each 16-byte lane slot, and whose half-wave touches two slots of
// every bank group) fetch the two slots of a bank group from opposite halves:
// no bank conflicts.
__device__ __forceinline__ half8 swap_halves_if(half8 f, bool odd)
{
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 u = __builtin_bit_cast(u32x4, f);
    const u32x4 w = odd ? u32x4{u[2], u[3], u[0], u[1]} : u;
    return __builtin_bit_cast(half8, w);
}

// Conv taps of channels (2*pp, 2*pp+1), tap 3 = current token
struct ConvW {
    float a[4], b[4];
};
__device__ __forceinline__ ConvW conv_weights(const uint16_t *__restrict__ w, int pp)
{
    const uint2 wa = *reinterpret_cast<const uint2 *>(w + (2 * pp) * 4);
    const uint2 wb = *reinterpret_cast<const uint2 *>(w + (2 * pp + 1) * 4);
    return ConvW{{bf16_lo(wa.x), bf16_hi(wa.x), bf16_lo(wa.y), bf16_hi(wa.y)},
                 {bf16_lo(wb.x), bf16_hi(wb.x), bf16_lo(wb.y), bf16_hi(wb.y)}};
}

// Conv + SiLU over a loaded window; rows >= n give 0.  Each raw row is
// unpacked once and added into the (up to) four outputs it reaches, in tap
// order, so every output is the same chain of multiply-adds as the plain
// four-term sum.  The mask is only applied in a partial chunk (wave-uniform).
__device__ __forceinline__ void conv_silu(const uint32_t (&win)[19], const ConvW &cw, int r0, int n,
                                          float (&z0)[16], float (&z1)[16])
{
#pragma unroll
    for (int i = 0; i < 19; ++i) {
        const float lo = bf16_lo(win[i]), hi = bf16_hi(win[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = i - j;
            if (r < 0 || r >= 16) continue;
            if (j == 0) {
                z0[r] = cw.a[0] * lo;
                z1[r] = cw.b[0] * hi;
            } else {
                z0[r] = __builtin_fmaf(cw.a[j], lo, z0[r]);
                z1[r] = __builtin_fmaf(cw.b[j], hi, z1[r]);
            }
        }
    }
    if (r0 + 16 <= n) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            z0[i] = silu_f(z0[i]);
            z1[i] = silu_f(z1[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bool valid = r0 + i < n;
            z0[i] = valid ? silu_f(z0[i]) : 0.0f;
            z1[i] = valid ? silu_f(z1[i]) : 0.0f;
        }
    }
}

// Raw rows r0-3 .. r0+15 of channels (2*pp, 2*pp+1) of one 128-channel plane
// for the causal width-4 conv (one bf16 pair per row), through range-checked
// buffer loads without branches.  x points at the chunk's first token; one
// range covers the rows taken from x (the chunk's n rows, and the three
// before unless the chunk starts the sequence) and rows outside it read as
// zero.  The three earlier rows of a sequence's first chunk come from the
// carried conv rows `hist` (zeros without them), selected per row so that
// each register receives one load.  ldb / ldh: bytes per row of x / of hist.
__device__ __forceinline__ void conv_window_rc(const uint16_t *x, int ldb, int n, bool first, const uint16_t *hist,
                                               int ldh, int pp, int r0, uint32_t (&win)[19])
{
    const int lo = first ? 0 : -3;  // first row taken from x
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(x) + (long)lo * (ldb / 2), 0, (n - lo) * ldb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rh =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(hist), 0, hist ? 3 * ldh : 0, 0x00020000);
    const int voff = (r0 - 3 - lo) * ldb + 4 * pp;  // negative offsets fail the range check too
    const bool carried = first && r0 == 0;
#pragma unroll
    for (int i = 0; i < 19; ++i) {
        if (i < 3)
            win[i] = __builtin_amdgcn_raw_buffer_load_b32(carried ? rh : rx,
                                                          carried ? 4 * pp + i * ldh : voff + i * ldb, 0, 0);
        else
            win[i] = __builtin_amdgcn_raw_buffer_load_b32(rx, voff + i * ldb, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// setup: chunk / sequence tables
// ---------------------------------------------------------------------------
// Sequence bounds, clamped into [0, T_tot] so that a malformed cu_seqlens
// cannot send any kernel outside the caller's buffers.
__device__ __forceinline__ int seq_start(const PrefillArgs &p, int s)
{
    return p.cu_seqlens ? min(max(p.cu_seqlens[s], 0), p.T_tot) : s * p.T_stride + p.t_off;
}
__device__ __forceinline__ int seq_len(const PrefillArgs &p, int s)
{
    if (!p.cu_seqlens) return p.T_uniform;
    const int t0 = seq_start(p, s);
    return min(max(p.cu_seqlens[s + 1] - t0, 0), p.T_tot - t0);
}

// Inclusive prefix sum over the 1024 threads of the block: within each wave by
// lane shifts, then across the 16 wave totals.
__device__ __forceinline__ int block_scan1024(int x, int *s_wsum)
{
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[w] = x;
    __syncthreads();
    int pre = 0;
    for (int i = 0; i < w; ++i) pre += s_wsum[i];
    __syncthreads();  // s_wsum may be reused
    return x + pre;
}

__global__ __launch_bounds__(1024) void setup_kernel(PrefillArgs p, Workspace ws)
{
    __shared__ int s_scan[1024];
    __shared__ int s_wsum[16];
    const int t = threadIdx.x;
    const int per = (p.N + 1023) / 1024;
    const int s0 = min(p.N, t * per), s1 = min(p.N, s0 + per);
    int local = 0;
    for (int s = s0; s < s1; ++s) local += (seq_len(p, s) + kChunk - 1) / kChunk;
    s_scan[t] = block_scan1024(local, s_wsum);
    __syncthreads();
    int base = s_scan[t] - local;
    const int Lseg = p.seg_chunks;
    int segs_local = 0;
    for (int s = s0; s < s1; ++s) {
        const int L = seq_len(p, s), t0 = seq_start(p, s);
        // chunks beyond the workspace bound (only with a malformed cu_seqlens) are dropped
        const int nch = max(0, min((L + kChunk - 1) / kChunk, p.max_chunks - base));
        ws.seq_info[s] = make_int4(base, nch, t0, min(L, nch * kChunk));
        base += nch;
        segs_local += seg_count(nch, Lseg);
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
    // segments of the sequential pass, in sequence order
    const int segs_incl = block_scan1024(segs_local, s_wsum);
    if (t == 1023) s_wsum[0] = segs_incl;
    __syncthreads();
    const int segs_total = s_wsum[0];
    int sb = segs_incl - segs_local;
    for (int s = s0; s < s1; ++s) {
        const int4 si = ws.seq_info[s];
        const int ns = seg_count(si.y, Lseg);
        ws.seq_seg[s] = make_int4(sb, ns, 0, 0);
        for (int i = 0; i < ns && sb + i < p.max_segs; ++i) {
            const int cb = si.x + seg_begin(i, Lseg), ce = si.x + seg_end(i, si.y, Lseg);
            ws.seg_info[sb + i] = make_int4(s, cb, ce, (i == 0 ? 1 : 0) | (i == ns - 1 ? 2 : 0));
        }
        sb += ns;
    }
    for (int k = min(segs_total, p.max_segs) + t; k < p.max_segs; k += 1024) ws.seg_info[k] = make_int4(-1, 0, 0, 0);
    // The order in which the sequential pass takes the segments: longest
    // first (a counting sort by chunk count, descending; ties in any order),
    // so that the short segments of short sequences fill the tail of the
    // launch instead of long ones starting last.  Slots past the segments
    // keep their own index (unused segments).
    __syncthreads();  // the segment table is complete
    const int nsegs = min(segs_total, p.max_segs);
    s_scan[t] = 0;
    __syncthreads();
    for (int k = t; k < nsegs; k += 1024) {
        const int4 sk = ws.seg_info[k];
        atomicAdd(&s_scan[1023 - min(sk.z - sk.y, 1023)], 1);
    }
    __syncthreads();
    const int cnt = s_scan[t];
    const int before = block_scan1024(cnt, s_wsum) - cnt;  // segments in longer bins
    s_scan[t] = before;
    __syncthreads();
    for (int k = t; k < nsegs; k += 1024) {
        const int4 sk = ws.seg_info[k];
        ws.seg_order[atomicAdd(&s_scan[1023 - min(sk.z - sk.y, 1023)], 1)] = k;
    }
    for (int k = nsegs + t; k < p.max_segs; k += 1024) ws.seg_order[k] = k;
}

// Table lookups.  Packed (varlen) calls read the tables setup_kernel built;
// uniform batches (B sequences of T tokens) compute the same entries directly,
// so that they need no setup launch.
struct Tables {
    static __device__ __forceinline__ int chunks_per_seq(const PrefillArgs &p) { return (p.T_uniform + kChunk - 1) / kChunk; }
    static __device__ __forceinline__ int segs_per_seq(const PrefillArgs &p)
    {
        return seg_count(chunks_per_seq(p), p.seg_chunks);
    }
    // {sequence, first token, length, is-first}
    static __device__ __forceinline__ int4 chunk(const PrefillArgs &p, const Workspace &ws, int c)
    {
        if (p.cu_seqlens) return ws.chunk_info[c];
        const int per = chunks_per_seq(p), s = c / per, j = c % per;
        return make_int4(s, s * p.T_stride + p.t_off + j * kChunk, min(kChunk, p.T_uniform - j * kChunk),
                         j == 0 && !p.cont);
    }
    // {first chunk, chunks, first token, length}
    static __device__ __forceinline__ int4 seq(const PrefillArgs &p, const Workspace &ws, int s)
    {
        if (p.cu_seqlens) return ws.seq_info[s];
        const int per = chunks_per_seq(p);
        return make_int4(s * per, per, s * p.T_stride + p.t_off, p.T_uniform);
    }
    // {sequence or -1, first chunk, end chunk, 1: first of sequence | 2: last}
    static __device__ __forceinline__ int4 seg(const PrefillArgs &p, const Workspace &ws, int k)
    {
        if (p.cu_seqlens) return ws.seg_info[k];
        const int per = chunks_per_seq(p), ns = segs_per_seq(p);
        const int s = k / ns, i = k % ns;
        if (s >= p.N) return make_int4(-1, 0, 0, 0);
        const int cb = s * per + seg_begin(i, p.seg_chunks), ce = s * per + seg_end(i, per, p.seg_chunks);
        return make_int4(s, cb, ce, (i == 0 ? 1 : 0) | (i == ns - 1 ? 2 : 0));
    }
    // {first segment, segments}
    static __device__ __forceinline__ int2 seq_segs(const PrefillArgs &p, const Workspace &ws, int s)
    {
        if (p.cu_seqlens) return make_int2(ws.seq_seg[s].x, ws.seq_seg[s].y);
        const int ns = segs_per_seq(p);
        return make_int2(s * ns, ns);
    }
};

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

// Column c of the inverse of a 16 x 16 unit lower-triangular block I + A (A
// strictly lower, row stride LD), by right-looking substitution: once y_m is
// final it is removed from every later row, y_i -= A[i][m] y_m, so the chain
// of dependent operations is one multiply-add per row.  Expanded at compile
// time so that y stays in registers.
template <int M, int LD>
struct SolveCol16 {
    static __device__ __forceinline__ void run(float (&y)[16], const float *A)
    {
        if constexpr (M < 15) {
#pragma unroll
            for (int i = M + 1; i < 16; ++i) y[i] -= A[i * LD + M] * y[M];
            SolveCol16<M + 1, LD>::run(y, A);
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

// Index of fragment (row tile rt, key block kb <= rt / 2) of a lower-triangular
// 64 x 64 operand in its compact order
__host__ __device__ constexpr int tri_frag(int rt, int kb) { return rt < 2 ? rt : 2 * rt - 2 + kb; }

// Gates of one (chunk, V head), by one wave (lane = token): gam = in-chunk
// cumulative log decay (log2 units) and beta into LDS; the sequential pass's
// per-chunk floats into the workspace
__device__ __forceinline__ void prep_gates(const PrefillArgs &p, float av, float bv, int n, float *gt,
                                           float *s_gam2, float *s_beta, int lane)
{
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
    gt[lane] = p.q_scale * Gam;
    gt[64 + lane] = valid ? __builtin_amdgcn_exp2f(gam_n - gam) : 0.f;
    gt[192 + lane] = Gam;
    if (lane == 0) {
        gt[128] = __builtin_amdgcn_exp2f(gam_n);
        gt[129] = gam_n;
    }
}

// prep: per (chunk, QK group), everything that does not depend on the carried
// state.  q and k: conv + SiLU + L2 norm, written as matrix-core operands (q^
// and k^ token-major, k^T d-major); K K^T and K Q^T once, on the matrix cores;
// then for each V head of the group: gates, A, P, the unit-lower-triangular
// inverse and T'.
constexpr int kPrepTile = 64 * kAL * 4;  // one fp32 64 x 64 tile (row stride kAL)
static_assert(64 * kQ_LD * 2 <= kPrepTile, "a token-major q^ / k^ tile fits in an fp32 tile");


// Lower 16 x 16 tiles of K K^T (row tile, column tile) and of K Q^T (query
// tile, key tile) computed by each wave: five per wave.  Wave w's first K K^T
// tile is the diagonal tile (w, w), whose block of the inverse the wave then
// solves itself.  The K Q^T tiles of a P fragment (query tile rt, key block
// kb) stay within one wave, except for fragment (3, 1), whose two halves come
// from waves 1 and 3.
__device__ constexpr int kPrepKK[4][3][2] = {{{0, 0}, {1, 0}, {3, 2}}, {{1, 1}, {2, 0}, {0, 0}},
                                             {{2, 2}, {2, 1}, {3, 1}}, {{3, 3}, {3, 0}, {0, 0}}};
__device__ constexpr int kPrepKQ[4][3][2] = {{{1, 0}, {1, 1}, {0, 0}}, {{0, 0}, {2, 2}, {3, 2}},
                                             {{2, 0}, {2, 1}, {0, 0}}, {{3, 0}, {3, 1}, {3, 3}}};
__device__ constexpr int kPrepNKK[4] = {3, 2, 3, 2}, kPrepNKQ[4] = {2, 3, 2, 3};

// The per-head phase works on up to kPrepHeads V heads at a time, each in a
// region of its own: the ten 16 x 16 tiles (i, j), i >= j, of its lower
// triangle (first A, then, in place, X = (I + A)^-1) and one temporary tile,
// fp32 with row stride kHLD (17: the column reads of the fp32 products fall in
// distinct banks).  The regions reuse the LDS of the q^ / k^ tiles.
constexpr int kPrepHeads = 3;
constexpr int kHLD = 17;
constexpr int kHTile = 16 * kHLD;                    // floats per tile slot
constexpr int kHSlots = 11;                          // ten lower tiles and a temporary
__host__ __device__ constexpr int htri(int i, int j) { return i * (i + 1) / 2 + j; }
constexpr int kPrepR = 2 * kPrepTile > kPrepHeads * kHSlots * kHTile * 4 ? 2 * kPrepTile
                                                                        : kPrepHeads * kHSlots * kHTile * 4;

// Four resident workgroups per CU (at most 128 VGPRs): the per-head phases
// are short stretches between barriers, and other workgroups fill the waits.
__global__ __launch_bounds__(kPrepThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void prep_kernel(PrefillArgs p, Workspace ws)
{
    // LDS plan: q^ and k^ (fp16 token-major tiles), then, reusing them, the
    // head regions of the per-head phase; the gates of kPrepHeads heads
    __shared__ __attribute__((aligned(16))) uint8_t R[kPrepR];
    __shared__ __attribute__((aligned(16))) float s_gam2[kPrepHeads * 64];
    __shared__ __attribute__((aligned(16))) float s_beta[kPrepHeads * 64];
    _Float16 *Qs = reinterpret_cast<_Float16 *>(R), *Ks = reinterpret_cast<_Float16 *>(R + kPrepTile);
    float *Hs = reinterpret_cast<float *>(R);

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int q4 = lane >> 4, c16 = lane & 15;
    const int Hqk = p.Hqk, Hv = p.Hv, G = Hv / Hqk;
    const int c = blockIdx.x / Hqk, g = blockIdx.x % Hqk;
    // the sequential pass's per-(sequence, V head) segment counters and flags
    if (blockIdx.x == 0)
        for (int i = t; i < p.N * Hv; i += kPrepThreads) ws.seg_done[i] = ws.seg_ready[i] = 0;
    const int4 ci = Tables::chunk(p, ws, c);
    const int n = ci.z;
    if (n == 0) return;  // empty chunk slot (whole workgroup)
    const int s = ci.x, t0 = ci.y;
    const bool first = ci.w != 0;
    const long C_tot = 2L * Hqk * kD + (long)Hv * kD;
    const int row = seq_row(p, s);
    const uint16_t *hist = (first && p.conv_state_in && row >= 0) ? p.conv_state_in + (long)row * 3 * C_tot : nullptr;
    const int r0 = 16 * wave;
    const long gc = (long)c * Hqk + g;

    // gate inputs of the group's first four V heads (wave w: head w, lane = token)
    float av = 0.f, bv = 0.f;
    if (wave < G && lane < n) {
        const long ti = (long)(t0 + lane) * Hv + g * G + wave;
        av = p.a[ti];
        bv = p.b[ti];
    }
    // ---- q^, k^ of the chunk: conv + SiLU, L2 norm per token.  The raw
    //      rows of both planes are requested before either is used, so that
    //      the k loads are in flight while q is formed.
    {
        float z0[16], z1[16];
        const long ldqk = (long)Hqk * kD;
        uint32_t win[2][19];
#pragma unroll
        for (int plane = 0; plane < 2; ++plane) {
            const long ch0 = plane == 0 ? (long)g * kD : (long)Hqk * kD + (long)g * kD;
            const uint16_t *x = (plane == 0 ? p.q : p.k) + (long)t0 * ldqk + (long)g * kD;
            conv_window_rc(x, (int)ldqk * 2, n, first, hist ? hist + ch0 : nullptr, (int)C_tot * 2, lane, r0,
                           win[plane]);
        }
#pragma unroll
        for (int plane = 0; plane < 2; ++plane) {
            const long ch0 = plane == 0 ? (long)g * kD : (long)Hqk * kD + (long)g * kD;
            conv_silu(win[plane], conv_weights(p.conv_w + ch0 * 4, lane), r0, n, z0, z1);
            float ss[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) ss[i] = z0[i] * z0[i] + z1[i] * z1[i];
            const float inv_mine = rsqrtf(reduce_scatter16(ss, lane) + 1e-6f);  // row (lane >> 2)
            _Float16 *dst = plane == 0 ? Qs : Ks;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv_mine), 4 * i));
                typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
                *reinterpret_cast<half2_t *>(dst + (r0 + i) * kQ_LD + 2 * lane) =
                    half2_t{(_Float16)(z0[i] * inv), (_Float16)(z1[i] * inv)};
            }
        }
    }
    __syncthreads();
    // ---- operands of the sequential pass (q^ fragments of row tile `wave`,
    //      k^ fragments), then the lower 16 x 16 tiles of K K^T and K Q^T, five per
    //      wave: K K^T tile (rt, ct) with ct <= rt, and K Q^T tile (query rt,
    //      key jt) with jt <= rt, kept in registers for every head
    f32x4 kk[3], kq[3];
    const int nkk = kPrepNKK[wave], nkq = kPrepNKQ[wave];
    {
        half8 *qf = reinterpret_cast<half8 *>(ws.qfrag + gc * kQFragBytes);
        half8 *kf = reinterpret_cast<half8 *>(ws.kfrag + gc * kKFragBytes);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            qf[(wave * 4 + kb) * 64 + lane] = swap_halves_if(lds_frag(Qs, kQ_LD, 16 * wave, 32 * kb, lane), q4 & 1);
            kf[(wave * 4 + kb) * 64 + lane] = swap_halves_if(lds_frag(Ks, kQ_LD, 16 * wave, 32 * kb, lane), q4 & 1);
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acq = {0.f, 0.f, 0.f, 0.f};
            if (i < nkk) {
                const int rt = kPrepKK[wave][i][0], ct = kPrepKK[wave][i][1];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    acc = mfma16(lds_frag(Ks, kQ_LD, 16 * rt, 32 * kb, lane), lds_frag(Ks, kQ_LD, 16 * ct, 32 * kb, lane),
                                 acc);
            }
            if (i < nkq) {
                const int rt = kPrepKQ[wave][i][0], jt = kPrepKQ[wave][i][1];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                    acq = mfma16(lds_frag(Ks, kQ_LD, 16 * jt, 32 * kb, lane), lds_frag(Qs, kQ_LD, 16 * rt, 32 * kb, lane),
                                 acq);
            }
            kk[i] = acc;
            kq[i] = acq;
            __builtin_amdgcn_sched_barrier(0);  // one tile's operands in flight at a time
        }
    }
    __syncthreads();  // the q^ / k^ tiles are dead from here on

    for (int j0 = 0; j0 < G; j0 += kPrepHeads) {
        const int jn = min(kPrepHeads, G - j0);
        // gates of heads j0 .. j0 + jn - 1 of the group (wave w: head j0 + w)
        if (wave < jn) {
            if (j0 > 0) {
                av = bv = 0.f;
                if (lane < n) {
                    const long ti = (long)(t0 + lane) * Hv + g * G + j0 + wave;
                    av = p.a[ti];
                    bv = p.b[ti];
                }
            }
            const long hc = (long)c * Hv + g * G + j0 + wave;
            prep_gates(p, av, bv, n, reinterpret_cast<float *>(ws.hrec + hc * kRecBytes + kRecG), s_gam2 + 64 * wave,
                       s_beta + 64 * wave, lane);
        }
        __syncthreads();
        // ---- A = strict_lower(diag(beta) K K^T * D) of every head of the
        //      round, from the K K^T tiles this wave holds (a lane's four rows
        //      are adjacent: one 16-byte read each of gam and beta per tile);
        //      the diagonal tiles' entries on and above the diagonal are never
        //      read.  P = (K Q^T)^T * D, lower incl. the diagonal, to the
        //      records, from the K Q^T tiles: each gives half of a fragment
        //      (key tile jt: elements 4 (jt % 2) .. +3); a diagonal tile of an
        //      even key tile (fragments (0, 0) and (2, 1)) also writes the
        //      zero half
        for (int jj = 0; jj < jn; ++jj) {
            const float *gam2 = s_gam2 + 64 * jj, *beta = s_beta + 64 * jj;
            float *Hh = Hs + jj * kHSlots * kHTile;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                if (i >= nkk) continue;
                const int rt = kPrepKK[wave][i][0], ct = kPrepKK[wave][i][1];
                const int jc = 16 * ct + c16;
                const f32x4 gr = *reinterpret_cast<const f32x4 *>(gam2 + 16 * rt + 4 * q4);
                const f32x4 br = *reinterpret_cast<const f32x4 *>(beta + 16 * rt + 4 * q4);
                const float gj = gam2[jc];
                float *tile = Hh + htri(rt, ct) * kHTile;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float a = br[e] * kk[i][e] * __builtin_amdgcn_exp2f(gr[e] - gj);
                    tile[(4 * q4 + e) * kHLD + c16] = (rt > ct || 4 * q4 + e > c16) ? a : 0.f;
                }
            }
            const long hc = (long)c * Hv + g * G + j0 + jj;
            uint8_t *pf = ws.hrec + hc * kRecBytes + kRecP;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                if (i >= nkq) continue;
                const int rt = kPrepKQ[wave][i][0], jt = kPrepKQ[wave][i][1];
                const int qi = 16 * rt + c16;
                const float gi = gam2[qi];
                const f32x4 gk = *reinterpret_cast<const f32x4 *>(gam2 + 16 * jt + 4 * q4);
                half4 hv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int jc = 16 * jt + 4 * q4 + e;
                    const float pv = p.q_scale * kq[i][e] * __builtin_amdgcn_exp2f(gi - gk[e]);
                    hv[e] = (_Float16)(qi >= jc ? pv : 0.f);
                }
                *reinterpret_cast<half4 *>(pf + tri_off(tri_frag(rt, jt >> 1), jt & 1, lane)) = hv;
            }
        }
        __syncthreads();
        // ---- X = (I + A)^-1 of head j0 + w by wave w alone, in place in its
        //      region, with wave-level synchronisation only: the four diagonal
        //      blocks by forward substitution (lane (q, c) takes column c of
        //      block q), then the blocks below them by the 2 x 2 block
        //      recursion L^-1 = [[X_a, 0], [-X_b L_ba X_a, X_b]] within and
        //      across the 32 x 32 halves, on the fp32 matrix cores; then T' =
        //      X diag(beta) as A operands (rows = tokens i, contraction =
        //      tokens j) to the record
        if (wave < jn) {
            float *Hh = Hs + wave * kHSlots * kHTile;
            auto T = [&](int i, int j) { return Hh + htri(i, j) * kHTile; };
            float *tmp = Hh + 10 * kHTile;
            auto wave_sync = [] {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            };
            {
                float y[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) y[i] = i == c16 ? 1.f : 0.f;
                const float *Ad = q4 == 0 ? T(0, 0) : q4 == 1 ? T(1, 1) : q4 == 2 ? T(2, 2) : T(3, 3);
                SolveCol16<0, kHLD>::run(y, Ad);
                wave_sync();
                float *Xd = const_cast<float *>(Ad);
#pragma unroll
                for (int i = 0; i < 16; ++i) Xd[i * kHLD + c16] = y[i];
                wave_sync();
            }
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            // X_10 = -X_11 (A_10 X_00), X_32 = -X_33 (A_32 X_22)
            st16_f32(tmp, kHLD, mm16_f32(T(1, 0), kHLD, T(0, 0), kHLD, z, lane), lane);
            wave_sync();
            st16_f32(T(1, 0), kHLD, -mm16_f32(T(1, 1), kHLD, tmp, kHLD, z, lane), lane);
            wave_sync();
            st16_f32(tmp, kHLD, mm16_f32(T(3, 2), kHLD, T(2, 2), kHLD, z, lane), lane);
            wave_sync();
            st16_f32(T(3, 2), kHLD, -mm16_f32(T(3, 3), kHLD, tmp, kHLD, z, lane), lane);
            wave_sync();
            // M_20 = A_20 X_00 + A_21 X_10, M_21 = A_21 X_11, M_30, M_31 likewise, each over its A tile
#pragma unroll
            for (int i = 2; i < 4; ++i) {
                f32x4 m = mm16_f32(T(i, 0), kHLD, T(0, 0), kHLD, z, lane);
                m = mm16_f32(T(i, 1), kHLD, T(1, 0), kHLD, m, lane);
                const f32x4 m1 = mm16_f32(T(i, 1), kHLD, T(1, 1), kHLD, z, lane);
                wave_sync();
                st16_f32(T(i, 0), kHLD, m, lane);
                st16_f32(T(i, 1), kHLD, m1, lane);
                wave_sync();
            }
            // X_31 = -(X_32 M_21 + X_33 M_31) (via tmp), X_21 = -X_22 M_21
            {
                f32x4 x = mm16_f32(T(3, 2), kHLD, T(2, 1), kHLD, z, lane);
                x = mm16_f32(T(3, 3), kHLD, T(3, 1), kHLD, x, lane);
                const f32x4 x21 = mm16_f32(T(2, 2), kHLD, T(2, 1), kHLD, z, lane);
                wave_sync();
                st16_f32(T(3, 1), kHLD, -x, lane);
                st16_f32(T(2, 1), kHLD, -x21, lane);
                wave_sync();
            }
            // X_30 = -(X_32 M_20 + X_33 M_30), X_20 = -X_22 M_20
            {
                f32x4 x = mm16_f32(T(3, 2), kHLD, T(2, 0), kHLD, z, lane);
                x = mm16_f32(T(3, 3), kHLD, T(3, 0), kHLD, x, lane);
                const f32x4 x20 = mm16_f32(T(2, 2), kHLD, T(2, 0), kHLD, z, lane);
                wave_sync();
                st16_f32(T(3, 0), kHLD, -x, lane);
                st16_f32(T(2, 0), kHLD, -x20, lane);
                wave_sync();
            }
            // T' = X diag(beta), the six fragments (row tile rt, key block kb);
            // entries above the diagonal are selected away
            const float *beta = s_beta + 64 * wave;
            const long hc = (long)c * Hv + g * G + j0 + wave;
            uint8_t *tf = ws.hrec + hc * kRecBytes + kRecT;
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                const int rt = f < 2 ? f : (f + 2) >> 1, kb = f < 2 ? 0 : f & 1;
                const int i = 16 * rt + c16;
                half8 fr;
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int cb = 2 * kb + hb, j0c = 16 * cb + 4 * q4;
                    const f32x4 bb = *reinterpret_cast<const f32x4 *>(beta + j0c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float xv = cb <= rt ? T(rt, cb <= rt ? cb : 0)[c16 * kHLD + 4 * q4 + e] : 0.f;
                        fr[4 * hb + e] = (_Float16)(j0c + e <= i ? xv * bb[e] : 0.f);
                    }
                }
                if (tri_half_only(f))
                    *reinterpret_cast<half4 *>(tf + tri_off(f, 0, lane)) = half4{fr[0], fr[1], fr[2], fr[3]};
                else
                    *reinterpret_cast<half8 *>(tf + tri_off(f, 0, lane)) = fr;
            }
        }
        if (j0 + kPrepHeads < G) __syncthreads();  // the next round rewrites the gates and the regions
    }
}

// ---------------------------------------------------------------------------
// chain: the sequential state carry
// ---------------------------------------------------------------------------
// Workgroup = one (segment, V head), 8 waves (kChainCT = 1); wave w owns the
// state columns kCW w .. kCW w + kCW - 1 (kChainCT 16-column tiles) in every
// product of a chunk:
//   v^ = SiLU(conv v)                  64 tokens x kCW channels, over 4 taps
//   X = K S,  Q S                      64 tokens x kCW columns, over d_k
//   Vnew = T' (v^ - diag(Gam) X)       64 tokens x kCW columns, over the chunk
//   S <- Gam_n S + k^T (r Vnew)        d_k x kCW columns, over the chunk
//   O = diag(q_scale Gam) Q S + P Vnew
// The B operands of these products are the wave's own accumulators: with the
// kappa k-mapping, a lane's accumulator rows 4q..4q+3 of two vertically
// adjacent 16-row tiles are exactly its eight B-operand elements of the
// 32-deep block they form, so the state, X and Vnew never leave the wave.
// The width-4 causal conv of v runs on the matrix cores as well, as a product
// with a block-diagonal tap matrix, which leaves v^ in the accumulator layout
// of X.  The waves share the chunk's operands (k^, q^, k^T, P, T', gates, raw
// v rows), which the workgroup stages in LDS with direct-to-LDS loads into
// two buffers, one barrier per chunk.  Waiting for a chunk's operands never
// waits for the output stores: they are the only memory operations issued
// after the operand loads (a warm-up step, which stores nothing, waits for
// its operand loads at its end).
constexpr int kChainBlocksPerHead = 1;
constexpr int kVTileRows = 68;  // raw v rows of a chunk: 1 unused, 3 before the chunk, 64
struct ChainBuf {
    // k^, q^ (operand order), the head record (P, T', gates), raw v
    static constexpr int kK = 0, kQ = 16384, kRec = 32768;
    static constexpr int kP = kRec + (int)kRecP, kT = kRec + (int)kRecT, kG = kRec + (int)kRecG;
    static constexpr int kV = kRec + (int)kRecBytes;
    static constexpr int kBytes = kV + kVTileRows * kD * 2;
};
constexpr int kRecPieces = (int)(kRecBytes / 1024);  // 1 KiB pieces of the head record
static_assert(kRecBytes % 1024 == 0, "the head record moves in 1 KiB pieces");
// 16-column tiles of the state per wave: 1 gives eight waves of 16 columns
// (two per SIMD, which hide each other's latencies), 2 gives four waves of 32.
constexpr int kChainCT = 1;
constexpr int kChainWaves = 8 / kChainCT;
constexpr int kChainThreads = 64 * kChainWaves;
constexpr int kCW = 16 * kChainCT;                      // state columns (and v channels) per wave
constexpr int kChainStageRows = 64;                    // token rows of the output staging (the chunk)
constexpr int kChainStage = kChainStageRows * kCW * 2;  // output staging of one wave (bf16)

// Byte offset in a wave's output staging of token row R, 16-byte piece p of
// the row, 8-byte half e.  The pieces of rows 8..15 of each 16-row tile are
// swapped in pairs (p ^ 1 with 32-byte rows, p ^ 2 with 64-byte ones), so
// that the staging writes (a lane per (row, 8 bytes), sixteen rows at a time)
// hit distinct banks in each half of the wave; a read of whole rows is a
// permutation within them.
__device__ __forceinline__ int stage_offset(int R, int p, int e)
{
    return R * (2 * kCW) + ((p ^ (((R >> 3) & 1) * kChainCT)) << 4) + (e << 3);
}

// k^ in LDS: the sixteen operand fragments (token tile rt, d block kb) in
// order, the 64 16-byte lane slots of each stored permuted: lane (q, r)
// (row r of the tile, d = 32kb + 4q .. +3 and +16) sits in slot
// 16q + (r ^ 4q).  A fragment read touches all 64 slots, so any permutation
// is conflict-free; the permutation makes the transposed reads of the
// d-major operand conflict-free too (their sixteen lanes touch four rows r
// and the four slots q of each).
__device__ __forceinline__ int kslot(int q4, int r) { return 16 * q4 + (r ^ (4 * q4)); }

// Raw v tile: tile row R holds chunk row R - 4 (rows 1..3: the three rows
// before the chunk); its 16-byte pieces are stored XOR-swizzled by R mod 16,
// so that the sixteen lanes of a conv operand, which read sixteen consecutive
// rows at the same channels, hit sixteen different bank groups.
__device__ __forceinline__ int vtile_offset(int R, int byte_in_row)
{
    return R * (kD * 2) + ((((byte_in_row >> 4) ^ R) & 15) << 4) + (byte_in_row & 15);
}

// Chunk c's operands into one LDS buffer: 60 pieces of 1 KiB; with four
// waves, wave w moves pieces 4i + w of k^, q^ and of the raw v tile (i < 4)
// and of the head record (4i + w < 11), and wave 3 the last piece of the v
// tile.
// Issued in four groups (i = 0..3), spread through a chunk step so that the
// memory unit takes them while the matrix cores work.
struct ChainDma {
    __amdgpu_buffer_rsrc_t rk, rq, rh, rv, rvh;
    int ldb, ldh;  // bytes per row of v and of the rows before the chunk
};

// Chunk range of one run of the sequential pass: chunks [c_from, c_to) of a
// sequence whose chunk 0 is c0 (first token t0, L tokens); chunks before c_out
// only advance the state (their output stores are dropped).  v is the head's
// v at the sequence's first token, hist its carried conv rows (or NULL).
struct ChainRun {
    int c0, t0, L;
    int c_from, c_to, c_out;
    const uint16_t *v, *hist;
};

__device__ __forceinline__ ChainDma chain_dma_plan(const PrefillArgs &p, const Workspace &ws, const ChainRun &run,
                                                   long c, int h, int g)
{
    const int Hqk = p.Hqk, Hv = p.Hv;
    const long hc = c * Hv + h, gc = c * Hqk + g;
    // raw v: the chunk's n rows (rows past its end read as zero), and the three
    // rows before it -- of v, or the carried rows of the sequence (zeros
    // without them) for its first chunk
    const int rel = ((int)c - run.c0) * kChunk;
    const int n = min(kChunk, run.L - rel);
    const int ldb = Hv * kD * 2, ldc = (2 * Hqk * kD + Hv * kD) * 2;
    const bool first = (int)c == run.c0 && !p.cont;  // a continuation reads its own earlier rows
    uint16_t *vc = const_cast<uint16_t *>(run.v) + (long)rel * (ldb / 2);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(vc, 0, n * ldb, 0x00020000);
    const __amdgpu_buffer_rsrc_t rvh =
        first ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(run.hist), 0, run.hist ? 3 * ldc : 0,
                                                  0x00020000)
              : __builtin_amdgcn_make_buffer_rsrc(vc - 3 * (ldb / 2), 0, 3 * ldb, 0x00020000);
    return ChainDma{region_rsrc(ws.kfrag + gc * kKFragBytes), region_rsrc(ws.qfrag + gc * kQFragBytes),
                    region_rsrc(ws.hrec + hc * kRecBytes), rv, rvh, ldb, first ? ldc : ldb};
}

// Piece f of the raw v tile (tile rows 4f .. 4f+3): lane L fills 16-byte slot
// L % 16 of tile row 4f + L / 16, i.e. the row's logical piece (L % 16) ^ R.
__device__ __forceinline__ void chain_dma_v(const ChainDma &d, uint8_t *buf, int f, int lane)
{
    const int R = 4 * f + (lane >> 4), piece = (lane ^ R) & 15;
    uint8_t *dst = buf + ChainBuf::kV + f * 1024;
    if (f == 0)  // tile row 0 is unused: a negative offset reads zero
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rvh, (lds_void_t *)dst, 16, (R - 1) * d.ldh + piece * 16, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rv, (lds_void_t *)dst, 16, (R - 4) * d.ldb + piece * 16, 0, 0, 0);
}

// k^ fragment f: LDS slot L receives lane (L / 16, (L % 16) ^ 4 (L / 16)) of
// the fragment, the lane that kslot places there
__device__ __forceinline__ void chain_dma_k(const ChainDma &d, uint8_t *buf, int f, int lane)
{
    const int q4 = lane >> 4, r = (lane & 15) ^ (4 * q4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rk, (lds_void_t *)(buf + ChainBuf::kK + f * 1024), 16,
                                             f * 1024 + (16 * q4 + r) * 16, 0, 0, 0);
}

template <int I>
__device__ __forceinline__ void chain_dma_group(const ChainDma &d, uint8_t *buf, int wave, int lane)
{
    const int v16 = lane * 16;
    if constexpr (kChainWaves == 4) {
        const int f = 4 * I + wave;
        chain_dma_k(d, buf, f, lane);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rq, (lds_void_t *)(buf + ChainBuf::kQ + f * 1024), 16, v16, f * 1024, 0, 0);
        chain_dma_v(d, buf, f, lane);
        // head record: T' 0-4, P 5-9, gates 10
        if (f < kRecPieces)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rh, (lds_void_t *)(buf + ChainBuf::kRec + f * 1024), 16, v16, f * 1024, 0, 0);
        if (I == 1 && wave == 3) chain_dma_v(d, buf, 16, lane);
    } else {
        // eight waves: group 0 k^, 1 q^, 2 raw v, 3 the head record; pieces
        // wave and wave + 8 of each
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int f = 8 * jj + wave;
            if (I == 0) chain_dma_k(d, buf, f, lane);
            if (I == 1)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rq, (lds_void_t *)(buf + ChainBuf::kQ + f * 1024), 16, v16, f * 1024, 0, 0);
            if (I == 2) chain_dma_v(d, buf, f, lane);
            if (I == 3 && f < kRecPieces)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rh, (lds_void_t *)(buf + ChainBuf::kRec + f * 1024), 16, v16, f * 1024, 0, 0);
        }
        if (I == 2 && wave == 0) chain_dma_v(d, buf, 16, lane);
    }
}

__device__ __forceinline__ void chain_dma(const PrefillArgs &p, const Workspace &ws, const ChainRun &run,
                                          uint8_t *buf, long c, int h, int g, int wave, int lane)
{
    const ChainDma d = chain_dma_plan(p, ws, run, c, h, g);
    chain_dma_group<0>(d, buf, wave, lane);
    chain_dma_group<1>(d, buf, wave, lane);
    chain_dma_group<2>(d, buf, wave, lane);
    chain_dma_group<3>(d, buf, wave, lane);
}

// Conv tap operands (B) of the wave's channel tile x and tap pair m: the
// contraction index kappa(q, i) stands for (tap 2m + (i >= 4), channel
// 4q + i % 4) of the tile, so lane (q, c) holds tap 2m / 2m+1 of channel c
// where 4q + i % 4 == c and zero elsewhere.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 conv_tap_frag(const uint16_t *__restrict__ w, int ch, int m, int lane)
{
    const int q4 = lane >> 4, c16 = lane & 15;
    const uint16_t *wc = w + (long)ch * 4;  // taps of channel ch (= the tile's channel c16)
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const bool on = 4 * q4 + (i & 3) == c16;
        const uint16_t bits = on ? wc[2 * m + (i >> 2)] : (uint16_t)0;
        r[i] = __builtin_bit_cast(__bf16, bits);
    }
    return r;
}

// Conv operand (A) of token tile rt, channel tile x, tap pair m: lane (q, r)
// takes the raw rows of token 16rt + r shifted by taps 2m and 2m+1 (tile rows
// 16rt + r + 1 + 2m and + 2 + 2m), channels 4q .. 4q+3 of the tile.
__device__ __forceinline__ bf16x8 conv_row_frag(const uint8_t *vt, int rt, int x, int m, int wave, int lane)
{
    const int q4 = lane >> 4, r = lane & 15;
    const int byte = (kCW * wave + 16 * x + 4 * q4) * 2;
    const int R = 16 * rt + r + 1 + 2 * m;
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 lo = *reinterpret_cast<const u32x2 *>(vt + vtile_offset(R, byte));
    const u32x2 hi = *reinterpret_cast<const u32x2 *>(vt + vtile_offset(R + 1, byte));
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x8, (u32x4){lo[0], lo[1], hi[0], hi[1]});
}

// k^ as the A operand of K S (token tile rt, d block kb): one 16-byte read
__device__ __forceinline__ half8 ktile_frag(const uint8_t *kt, int rt, int kb, int lane)
{
    return *reinterpret_cast<const half8 *>(kt + (rt * 4 + kb) * 1024 + kslot(lane >> 4, lane & 15) * 16);
}

// k^T as the A operand of the state update (d tile dt, token block tb):
// lane (q, r) needs d = 16dt + r at tokens 32tb + 4q .. +3 and 32tb + 16 + 4q
// .. +3.  A transposed read hands lane i of each 16-lane group element i % 4
// of the 8 bytes that lane 4j + i / 4 of the group addressed, as its element
// j; so lane s of group q addresses token row R = 32tb + 4q + s / 4, d
// columns 16dt + 4 (s % 4) .. +3: half dt % 2 of slot (s % 4, R % 16) of
// fragment (R / 16, dt / 2), stored as half (dt + s) % 2 (the halves of odd
// lane groups are swapped, see swap_halves_if).
__device__ __forceinline__ half8 ktile_frag_t(const uint8_t *kt, int dt, int tb, int lane)
{
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int q4 = lane >> 4, s = lane & 15;
    const int R = 32 * tb + 4 * q4 + (s >> 2);
    const uint8_t *p0 = kt + ((R >> 4) * 4 + (dt >> 1)) * 1024 + kslot(s & 3, R & 15) * 16 + 8 * ((dt ^ s) & 1);
    const uint8_t *p1 = p0 + 4 * 1024;  // token rows + 16: the next token tile
    const half4 lo = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(__attribute__((address_space(3))) uint8_t *)(p0)));
    const half4 hi = __builtin_bit_cast(half4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                   (lds_s16x4 *)(__attribute__((address_space(3))) uint8_t *)(p1)));
    return half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// VMEM operations a wave issues after a chunk's operand DMA and before the
// step that consumes it: the previous chunk's output stores (4).  Waiting
// down to this count waits for the DMA (vector memory operations complete in
// issue order) and leaves the stores in flight.
constexpr int kChainVmemAfterDma = 4;

// s_waitcnt immediate that waits for vector memory operations only, until at
// most n (< 64) are outstanding: vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt at their no-wait maxima
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }

// Fragment f of a compact lower-triangular operand in LDS (T' or P)
__device__ __forceinline__ half8 tri_frag_ld(const uint8_t *base, int f, int lane)
{
    if (tri_half_only(f)) {
        const half4 lo = *reinterpret_cast<const half4 *>(base + tri_off(f, 0, lane));
        return half8{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    }
    return *reinterpret_cast<const half8 *>(base + tri_off(f, 0, lane));
}

// One chunk from operand buffer `cur`; loads the next chunk's operands into
// `nxt`.  kOut = false: a warm-up chunk, which only advances the state (no
// Q S, no output); it waits for its own DMA at its end, since it issues no
// output stores after it.
//   Z, X, Vn [rt][x]  tokens 16rt.. x columns 16x..  (accumulator rows = tokens)
//   QST      [x][rt]  (Q S)^T, columns 16x.. x tokens 16rt.. (accumulator rows = columns)
// The output is formed transposed, O^T = S^T Q^T diag(q_scale Gam) + Vnew^T P^T,
// so that a lane holds four adjacent columns of one token (8-byte LDS writes
// into the row staging).  The fragment layout is the same for A and B
// operands, so the packed state and Vnew serve as A operands unchanged.
template <bool kOut>
__device__ __forceinline__ void chain_step(const PrefillArgs &p, const Workspace &ws, uint8_t *cur, uint8_t *nxt,
                                           uint8_t *stage, f32x4 (&S)[8][kChainCT], const bf16x8 (&wb)[kChainCT][2],
                                           const ChainRun &run, int cc, int h, int g, int wave, int lane)
{
    const int Hv = p.Hv;
    const int q4 = lane >> 4, c16 = lane & 15;
    // chunk cc's operands have landed for every wave, and every wave is done
    // with the buffer the next chunk's DMA overwrites
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kChainVmemAfterDma));
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    const int cn = min(cc + 1, run.c_to - 1);  // the last step repeats its own chunk
    const ChainDma dn = chain_dma_plan(p, ws, run, cn, h, g);

    const uint8_t *kt = cur + ChainBuf::kK;
    const half8 *Qf = reinterpret_cast<const half8 *>(cur + ChainBuf::kQ) + lane;
    const uint8_t *Pf = cur + ChainBuf::kP, *Tf = cur + ChainBuf::kT;
    const float *gt = reinterpret_cast<const float *>(cur + ChainBuf::kG);
    const uint8_t *vt = cur + ChainBuf::kV;

    // K S and (Q S)^T over the four 32-row blocks of the state; the LDS
    // fragments of block kb+1 are read while block kb multiplies, the next
    // chunk's DMA goes out one group per block.  The conv of v at the wave's
    // channels (pre-activation, on the matrix cores) goes out after the first
    // block's products, its operands read with that block's; SiLU of conv
    // tile kb-1 runs on the vector ALUs during block kb, of tile 3 after.
    f32x4 Z[4][kChainCT];
    f32x4 X[4][kChainCT], QST[kChainCT][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int x = 0; x < kChainCT; ++x) {
            X[rt][x] = f32x4{0.f, 0.f, 0.f, 0.f};
            QST[x][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        half8 ak[4], aq[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            ak[rt] = ktile_frag(kt, rt, kb, lane);
            if (kOut) aq[rt] = Qf[(rt * 4 + kb) * 64];
        }
        bf16x8 cv[4][kChainCT][2];
        if (kb == 0) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int x = 0; x < kChainCT; ++x)
#pragma unroll
                    for (int m = 0; m < 2; ++m) cv[rt][x][m] = conv_row_frag(vt, rt, x, m, wave, lane);
        }
        if (kb == 0) chain_dma_group<0>(dn, nxt, wave, lane);
        if (kb == 1) chain_dma_group<1>(dn, nxt, wave, lane);
        if (kb == 2) chain_dma_group<2>(dn, nxt, wave, lane);
        if (kb == 3) chain_dma_group<3>(dn, nxt, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
        half8 sb[kChainCT];
#pragma unroll
        for (int x = 0; x < kChainCT; ++x) sb[x] = swap_halves_if(pack_h8(S[2 * kb][x], S[2 * kb + 1][x]), q4 & 1);
        // per token tile: the X products of the wave's column tiles, then the
        // (Q S)^T ones; SiLU of conv tile kb, one value per slot
#pragma unroll
        for (int sl = 0; sl < 8 * kChainCT; ++sl) {
            const int rt = sl / (2 * kChainCT), r = sl % (2 * kChainCT);
            if (r < kChainCT) X[rt][r] = mfma16(ak[rt], sb[r], X[rt][r]);
            else if (kOut) QST[r - kChainCT][rt] = mfma16(sb[r - kChainCT], aq[rt], QST[r - kChainCT][rt]);
            if (kb > 0 && sl < 4 * kChainCT) Z[kb - 1][sl >> 2][sl & 3] = silu_f(Z[kb - 1][sl >> 2][sl & 3]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (kb == 0) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int x = 0; x < kChainCT; ++x) {
                    Z[rt][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv[rt][x][0], wb[x][0], f32x4{0.f, 0.f, 0.f, 0.f},
                                                                       0, 0, 0);
                    Z[rt][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cv[rt][x][1], wb[x][1], Z[rt][x], 0, 0, 0);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int sl = 0; sl < 4 * kChainCT; ++sl) Z[3][sl >> 2][sl & 3] = silu_f(Z[3][sl >> 2][sl & 3]);
    // Vnew = T' (v^ - diag(Gam) X): the bracket as B operands over the chunk's
    // two 32-token blocks, T' lower triangular
    half8 tf[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) tf[i] = tri_frag_ld(Tf, i, lane);
    f32x4 Vn[4][kChainCT];
    {
        f32x4 gg[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) gg[rt] = *reinterpret_cast<const f32x4 *>(gt + 192 + 16 * rt + 4 * q4);
        half8 yb[2][kChainCT];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int x = 0; x < kChainCT; ++x)
                yb[tb][x] = pack_h8(Z[2 * tb][x] - gg[2 * tb] * X[2 * tb][x],
                                    Z[2 * tb + 1][x] - gg[2 * tb + 1] * X[2 * tb + 1][x]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int x = 0; x < kChainCT; ++x) {
                Vn[rt][x] = mfma16(tf[tri_frag(rt, 0)], yb[0][x], f32x4{0.f, 0.f, 0.f, 0.f});
                if (rt >= 2) Vn[rt][x] = mfma16(tf[tri_frag(rt, 1)], yb[1][x], Vn[rt][x]);
            }
    }
    // k^T fragments of the first two 16-row state tiles, P, and the gates
    half8 kf[2][2][2];  // [buffer][tile in pair][token block]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) kf[0][i][tb] = ktile_frag_t(kt, i, tb, lane);
    half8 pf[6];
    if (kOut) {
#pragma unroll
        for (int i = 0; i < 6; ++i) pf[i] = tri_frag_ld(Pf, i, lane);
    }
    f32x4 rg[4];
    float gm[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        rg[rt] = *reinterpret_cast<const f32x4 *>(gt + 64 + 16 * rt + 4 * q4);
        if (kOut) gm[rt] = gt[16 * rt + c16];
    }
    const float gn = gt[128];
    __builtin_amdgcn_sched_barrier(0);
    // Vnew and (Gam_n / Gam) Vnew as operands over the chunk's two 32-token blocks
    half8 vb[2][kChainCT], vr[2][kChainCT];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int x = 0; x < kChainCT; ++x) {
            if (kOut) vb[tb][x] = pack_h8(Vn[2 * tb][x], Vn[2 * tb + 1][x]);
            vr[tb][x] = pack_h8(Vn[2 * tb][x] * rg[2 * tb], Vn[2 * tb + 1][x] * rg[2 * tb + 1]);
        }
    // O = diag(q_scale Gam) Q S + P Vnew (P lower triangular), formed
    // transposed: (Q S)^T tile (x, rt) lane (q, c) holds columns 16x + 4q ..
    // +3 of token 16rt + c.  Its products go out before the state update, and
    // its packing and LDS staging run between the update's products, so that
    // the two overlap; the staged rows are stored after the update.
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    f32x4 oacc[4][kChainCT];
    if (kOut) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int x = 0; x < kChainCT; ++x) {
                oacc[rt][x] = mfma16(vb[0][x], pf[tri_frag(rt, 0)], QST[x][rt] * gm[rt]);
                if (rt >= 2) oacc[rt][x] = mfma16(vb[1][x], pf[tri_frag(rt, 1)], oacc[rt][x]);
            }
    }
    uint16_t *os = reinterpret_cast<uint16_t *>(stage);
    static_assert(kChainStageRows == kChunk, "the whole chunk is staged at once");
    // S <- Gam_n S + k^T (r Vnew), two state tiles at a time, the next pair's
    // fragments read while this pair multiplies
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
        const int cb = pr & 1;
        if (pr < 3) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) kf[cb ^ 1][i][tb] = ktile_frag_t(kt, 2 * pr + 2 + i, tb, lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int dt = 2 * pr + i;
#pragma unroll
            for (int x = 0; x < kChainCT; ++x) {
                S[dt][x] = mfma16(kf[cb][i][0], vr[0][x], S[dt][x] * gn);
                S[dt][x] = mfma16(kf[cb][i][1], vr[1][x], S[dt][x]);
            }
        }
        if (kOut && pr >= 1) {  // output token tiles 2 (pr - 1) .. +1 into the staging
#pragma unroll
            for (int rt = 2 * (pr - 1); rt < 2 * pr && rt < 4; ++rt)
#pragma unroll
                for (int x = 0; x < kChainCT; ++x)
                    *reinterpret_cast<u32x2 *>(os + stage_offset(16 * rt + c16, 2 * x + (q4 >> 1), q4 & 1) / 2) =
                        u32x2{pack_bf16x2(oacc[rt][x][0], oacc[rt][x][1]), pack_bf16x2(oacc[rt][x][2], oacc[rt][x][3])};
        }
    }
    if (!kOut) {
        // the operands of the next chunk have landed (no output stores follow)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        return;
    }
    // the staged rows to o: the buffer range of the stores ends at the
    // chunk's last valid token, so the rows of a partial chunk are dropped
    // without a branch
    const int rel = (cc - run.c0) * kChunk;
    const int n = min(kChunk, run.L - rel);
    const int rowb = Hv * kD * 2;  // bytes per token row of o
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        p.o + ((long)(run.t0 + rel) * Hv + h) * kD + kCW * wave, 0, n * rowb, 0x00020000);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 16 rows of 2 kCW bytes per store: lane -> (row lane/4, piece lane%4 of kCW/2 bytes)
    const int row = lane >> 2, piece = lane & 3;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        if constexpr (kChainCT == 2) {
            const i32x4 v = *reinterpret_cast<const i32x4 *>(stage + stage_offset(16 * rt + row, piece, 0));
            __builtin_amdgcn_raw_buffer_store_b128(v, ro, (16 * rt + row) * rowb + piece * 16, 0, 0);
        } else {
            typedef int i32x2 __attribute__((ext_vector_type(2)));
            const i32x2 v = *reinterpret_cast<const i32x2 *>(stage + stage_offset(16 * rt + row, piece >> 1, piece & 1));
            __builtin_amdgcn_raw_buffer_store_b64(v, ro, (16 * rt + row) * rowb + piece * 8, 0, 0);
        }
    }
    // the staging is rewritten by the next step only after its block barrier
}

// The chunks of one run, the state carried in registers.
__device__ __forceinline__ void chain_run(const PrefillArgs &p, const Workspace &ws, uint8_t *buf0, uint8_t *buf1,
                                          uint8_t *stage, f32x4 (&S)[8][kChainCT],
                                          const bf16x8 (&wb)[kChainCT][2], const ChainRun &run, int h, int g, int wave,
                                          int lane)
{
    if (run.c_to <= run.c_from) return;
    chain_dma(p, ws, run, buf0, run.c_from, h, g, wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    int cc = run.c_from;
    // warm-up chunks [c_from, c_out): the state only
    const int cw = min(run.c_out, run.c_to);
    for (; cc + 2 <= cw; cc += 2) {
        chain_step<false>(p, ws, buf0, buf1, stage, S, wb, run, cc, h, g, wave, lane);
        chain_step<false>(p, ws, buf1, buf0, stage, S, wb, run, cc + 1, h, g, wave, lane);
    }
    if (cc < cw) {  // an odd warm-up: the next chunk sits in buf1
        chain_step<false>(p, ws, buf0, buf1, stage, S, wb, run, cc, h, g, wave, lane);
        ++cc;
        if (cc < run.c_to) {
            chain_step<true>(p, ws, buf1, buf0, stage, S, wb, run, cc, h, g, wave, lane);
            ++cc;
        }
    }
    for (; cc + 2 <= run.c_to; cc += 2) {
        chain_step<true>(p, ws, buf0, buf1, stage, S, wb, run, cc, h, g, wave, lane);
        chain_step<true>(p, ws, buf1, buf0, stage, S, wb, run, cc + 1, h, g, wave, lane);
    }
    if (cc < run.c_to) chain_step<true>(p, ws, buf0, buf1, stage, S, wb, run, cc, h, g, wave, lane);
    // the last step's DMA into the other buffer is still in flight
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
}

// Warm-up bound of the segmented sequential pass.  Every token's transition
// alpha (I - beta k k^T) has spectral norm <= alpha (beta in (0,1), |k| <= 1),
// so a state that enters w chunks before a segment reaches the segment's start
// scaled by at most the product of those chunks' gates.  A segment therefore
// starts from a zero state at the latest chunk w for which that product is
// <= 2^-24 -- what it drops is below single-precision resolution of the state
// it came from -- or from the sequence's own initial state when the sequence
// start is within reach.
constexpr float kWarmLog2 = -24.0f;
constexpr int kMaxWarm = 64;  // chunks a segment looks back at most (one per lane)

// First chunk of the run of the segment that starts at chunk cb (sequence
// chunk 0 = c0): c0 (exact start from the initial state), a chunk in
// (c0, cb) (start from zero), or -1 when the bound is not met within
// kMaxWarm chunks.  Wave-uniform, and identical in every block that asks.
// In two steps, so that several segments' gate loads can be in flight together:
// warm_gate loads log2 of chunk cb-1-lane's decay, warm_pick decides.
__device__ __forceinline__ float warm_gate(const Workspace &ws, int h, int Hv, int cb, int c0, int lane)
{
    const int c = cb - 1 - lane;
    return c >= c0 ? reinterpret_cast<const float *>(ws.hrec + ((long)c * Hv + h) * kRecBytes + kRecG)[129] : 0.f;
}
__device__ __forceinline__ int warm_pick(float gsum, int cb, int c0, int lane)
{
    if (cb <= c0) return c0;
    const bool in = cb - 1 - lane >= c0;
    // inclusive prefix over lanes: log2 of the decay of chunks cb-1-lane .. cb-1
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(gsum, off, 64);
        if (lane >= off) gsum += y;
    }
    const unsigned long long hit = __ballot(in && gsum <= kWarmLog2);
    int w;
    if (hit) w = cb - 1 - __builtin_ctzll(hit);
    else w = (cb - c0 <= kMaxWarm) ? c0 : -1;
    return __builtin_amdgcn_readfirstlane(w);
}
__device__ __forceinline__ int warm_start(const Workspace &ws, int h, int Hv, int cb, int c0, int lane)
{
    return warm_pick(cb > c0 ? warm_gate(ws, h, Hv, cb, c0, lane) : 0.f, cb, c0, lane);
}

// state columns kCW w .. kCW w + kCW - 1 of one (sequence, head): tile (dt, x)
// element e is row 16dt + 4q + e, column kCW w + 16x + c16
__device__ __forceinline__ void state_load(f32x4 (&S)[8][kChainCT], const float *src, int wave, int lane)
{
    const int q4 = lane >> 4, c16 = lane & 15;
    if (!src) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int x = 0; x < kChainCT; ++x) S[dt][x] = f32x4{0.f, 0.f, 0.f, 0.f};
        return;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int x = 0; x < kChainCT; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[dt][x][e] = src[(long)(16 * dt + 4 * q4 + e) * kD + kCW * wave + 16 * x + c16];
}
__device__ __forceinline__ void state_store(const f32x4 (&S)[8][kChainCT], float *dst, int wave, int lane)
{
    const int q4 = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int x = 0; x < kChainCT; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dst[(long)(16 * dt + 4 * q4 + e) * kD + kCW * wave + 16 * x + c16] = S[dt][x][e];
}

// The identity in the state layout: where a segment's transition-matrix run
// starts (the map from the state entering the segment to the state leaving
// it is S -> M S + S0, M the product of the chunks' linear parts; carrying
// the identity through the chunks with v^ = 0 gives M)
__device__ __forceinline__ void state_identity(f32x4 (&S)[8][kChainCT], int wave, int lane)
{
    const int q4 = lane >> 4, c16 = lane & 15;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int x = 0; x < kChainCT; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[dt][x][e] = 16 * dt + 4 * q4 + e == kCW * wave + 16 * x + c16 ? 1.f : 0.f;
}

// S <- M S + S0 for the wave's state columns, M (d_k x d_k) and S0 (a state)
// row-major fp32, on the fp32 matrix cores.  M arrives in registers (mreg:
// thread t holds rows (t + 512 i) / 32, float4 column block (t + 512 i) % 32,
// as m_fetch requests them) and the workgroup stages it in LDS (rows 0..63 in
// lo, 64..127 in hi, kMLD floats apart: the sixteen rows a quarter wave reads
// fall in distinct banks); mreg is then free, and `next` (if not NULL) is
// requested into it while the products run.  Output tile (rt, x) sums 32
// four-deep steps (dt, e), whose A operand is M[16 rt + r][16 dt + 4q + e]
// (lane (q, r)) and whose B operand is S[16 dt + 4q + e][column]: the lane's
// own element S[dt][x][e].  Called by the whole workgroup.
constexpr int kMLD = 132;
constexpr int kMRegs = 128 * 32 / kChainThreads;  // float4 blocks of M per thread
static_assert(64 * kMLD * 4 <= ChainBuf::kBytes, "half of M fits in an operand buffer");
__device__ __forceinline__ void m_fetch(f32x4 (&mreg)[kMRegs], const float *M)
{
#pragma unroll
    for (int i = 0; i < kMRegs; ++i) {
        const int idx = (int)threadIdx.x + kChainThreads * i;
        mreg[i] = *reinterpret_cast<const f32x4 *>(M + (long)(idx >> 5) * kD + 4 * (idx & 31));
    }
}
__device__ __forceinline__ void state_affine(f32x4 (&S)[8][kChainCT], f32x4 (&mreg)[kMRegs], const float *next,
                                             const float *S0, uint8_t *lo, uint8_t *hi, int wave, int lane)
{
    const int q4 = lane >> 4, c16 = lane & 15;
    float s0[8][kChainCT][4];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int x = 0; x < kChainCT; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e) s0[rt][x][e] = S0[(long)(16 * rt + 4 * q4 + e) * kD + kCW * wave + 16 * x + c16];
    __syncthreads();  // the buffers may hold the previous product's M
#pragma unroll
    for (int i = 0; i < kMRegs; ++i) {
        const int idx = (int)threadIdx.x + kChainThreads * i, r = idx >> 5, c4 = idx & 31;
        *reinterpret_cast<f32x4 *>((r < 64 ? lo : hi) + ((r & 63) * kMLD + 4 * c4) * 4) = mreg[i];
    }
    __syncthreads();
    if (next) m_fetch(mreg, next);
    f32x4 acc[8][kChainCT];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
        const uint8_t *mrow = (rt < 4 ? lo : hi) + ((16 * rt + c16) & 63) * kMLD * 4 + 16 * q4;
#pragma unroll
        for (int x = 0; x < kChainCT; ++x) acc[rt][x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(mrow + 64 * dt);
#pragma unroll
            for (int x = 0; x < kChainCT; ++x)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[rt][x] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[e], S[dt][x][e], acc[rt][x], 0, 0, 0);
        }
    }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int x = 0; x < kChainCT; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[rt][x][e] = acc[rt][x][e] + s0[rt][x][e];
}

// Polls of the flag that tells an extra workgroup its segment's incoming
// state is ready (a load and a short sleep each, about 1-2 us: a bound of
// one to two seconds).  The flag is set by a workgroup of lower id, which
// the dispatcher has started before this one, so the wait ends long before.
constexpr int kReadyPolls = 1 << 20;

// The carried conv rows of one sequence (pool row `row`), planes [pl0, pl1)
// of q | k | v for QK head g / V head h, one wave: the last three raw rows,
// reaching back into the incoming rows when the sequence is shorter than
// three tokens (into the input's earlier rows when the call is a window that
// continues its sequences).  In place, a lane reads each incoming row before it writes
// it: row r is written from row r + L (L < 3), which is read first.
__device__ __forceinline__ void write_conv_rows(const PrefillArgs &p, const int4 &si, int row, int g, int h,
                                                int pl0, int pl1, int lane)
{
    const int Hqk = p.Hqk, Hv = p.Hv;
    const long C_tot = 2L * Hqk * kD + (long)Hv * kD;
    const int Ls = si.w, t0 = si.z;
    for (int plane = pl0; plane < pl1; ++plane) {
        const long ch0 = plane == 0 ? (long)g * kD : plane == 1 ? (long)Hqk * kD + (long)g * kD
                                                              : 2L * Hqk * kD + (long)h * kD;
        const uint16_t *src = plane == 0 ? p.q + (long)g * kD : plane == 1 ? p.k + (long)g * kD : p.v + (long)h * kD;
        const long ld = plane == 2 ? (long)Hv * kD : (long)Hqk * kD;
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int tau = Ls - 3 + r;
            uint32_t val = 0;
            if (tau >= 0 || p.cont)  // a window that continues its sequence has its earlier rows in the input
                val = ld_pair(src + (long)(t0 + tau) * ld + 2 * lane);
            else if (p.conv_state_in)
                val = ld_pair(p.conv_state_in + ((long)row * 3 + 3 + tau) * C_tot + ch0 + 2 * lane);
            *reinterpret_cast<uint32_t *>(p.conv_state_out + ((long)row * 3 + r) * C_tot + ch0 + 2 * lane) = val;
        }
    }
}

// Sequential pass: one workgroup per (segment, V head); segments run in
// parallel, each from its warm-up start.  Every workgroup makes the warm-up
// test of all segments of its sequence.  A segment that misses its bound
// forms instead the affine map S -> M S + S0 from the state entering it to
// the one leaving it (two runs without output).  If a segment misses its
// bound, or the call is in place, the last workgroup of the (sequence, V
// head) to finish -- a device-scope counter per pair, zeroed by the parallel
// pass -- walks the sequence's segments in order, applies the maps to the
// states the previous segments hand over, hands a sequence of several
// segments its final state, and sets the pair's flag, on which the extra
// workgroups of the missed segments (the second half of the grid) wait
// before they form those segments' outputs.  Only a workgroup whose parked
// state the walk will read publishes it with a device-scope fence; the
// common case (no failed bound, out of place) needs no counter at all.
__global__ __launch_bounds__(kChainThreads) __attribute__((amdgpu_waves_per_eu(kChainWaves / 4, kChainWaves / 4)))
void chain_kernel(PrefillArgs p, Workspace ws)
{
    __shared__ __attribute__((aligned(16))) uint8_t buf0[ChainBuf::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t buf1[ChainBuf::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t stage_all[kChainWaves * kChainStage];
    __shared__ int s_total;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    uint8_t *stage = stage_all + wave * kChainStage;
    const int Hqk = p.Hqk, Hv = p.Hv, G = Hv / Hqk;
    // block -> (segment, group, head in group); the G heads of one (segment,
    // QK group) land on the same XCD (same L2).  The second half of the grid
    // are the extra workgroups, one per (segment, V head) again (same XCD as
    // the main one): they form the output of a segment that misses its
    // warm-up bound, once the in-order combine has its incoming state.
    const int n_main = ((p.max_segs * Hqk + 7) / 8) * 8 * G;
    const bool extra = (int)blockIdx.x >= n_main;
    const int bid = extra ? (int)blockIdx.x - n_main : (int)blockIdx.x;
    const int gu = (bid / (8 * G)) * 8 + (bid & 7);
    const int j = (bid >> 3) % G;
    if (gu >= p.max_segs * Hqk) return;
    // packed calls take the segments longest first (setup_kernel's order)
    const int k = p.cu_seqlens ? ws.seg_order[gu / Hqk] : gu / Hqk, g = gu % Hqk;
    const int h = g * G + j;
    const long C_tot = 2L * Hqk * kD + (long)Hv * kD, cv = 2L * Hqk * kD + (long)h * kD;
    const int4 sg = Tables::seg(p, ws, k);  // seq, first chunk, end chunk, flags
    if (sg.x < 0) return;                   // no segment in this slot
    const int s = sg.x;
    const int row = seq_row(p, s);          // pool row of the sequence's state and conv rows
    if (row < 0) return;                    // its slot lies outside the pool: skipped
    const int4 si = Tables::seq(p, ws, s);  // chunk0, nchunks, t0, L
    const bool first = sg.w & 1, last = sg.w & 2;
    const long sbase = ((long)row * Hv + h) * kD * kD;
    const uint16_t *hist = p.conv_state_in ? p.conv_state_in + (long)row * 3 * C_tot + cv : nullptr;
    const uint16_t *vs = p.v + (long)si.z * Hv * kD + (long)h * kD;
    f32x4 S[8][kChainCT];

    const int2 ss = Tables::seq_segs(p, ws, s);  // first segment, segments
    const int nseg = min(ss.y, p.max_segs - ss.x), i_seg = k - ss.x;
    int w = sg.y;
    bool any_bad = false, next_bad = false;
    if (extra) {
        if (first) return;  // a sequence's first segment always starts from the true state
        if (warm_start(ws, h, Hv, sg.y, si.x, lane) >= 0) return;  // its main workgroup wrote its output
        if (t == 0) {
            int ok = 0;
            for (int n = 0; n < kReadyPolls && !ok; ++n) {
                ok = __hip_atomic_load(ws.seg_ready + (long)s * Hv + h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (!ok) __builtin_amdgcn_s_sleep(8);
            }
            s_total = ok;
        }
        __syncthreads();
        if (!s_total) {
            // not reached (the combine's workgroup has a lower id and waits
            // on nothing); should the bound ever expire, the segment's output
            // rows are NaN instead of left unwritten
            const int rel0 = (sg.y - si.x) * kChunk, rel1 = min((sg.z - si.x) * kChunk, si.w);
            const uint16_t nan16 = 0x7fc0;
            for (long i = t; i < (long)(rel1 - rel0) * kD; i += kChainThreads)
                p.o[((long)(si.z + rel0 + i / kD) * Hv + h) * kD + i % kD] = nan16;
            return;
        }
        __threadfence();
    } else {
        // The warm-up test of every segment of the sequence, the same in
        // every workgroup of it (gate loads of four segments in flight
        // together): this segment's start, whether the next one misses its
        // bound, and whether any does.
        for (int i0 = 1; i0 < nseg; i0 += 4) {
            int cb[4];
            float gv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u;
                cb[u] = i < nseg ? Tables::seg(p, ws, ss.x + i).y : si.x;
                gv[u] = i < nseg ? warm_gate(ws, h, Hv, cb[u], si.x, lane) : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u;
                if (i >= nseg) continue;
                const int wi = warm_pick(gv[u], cb[u], si.x, lane);
                any_bad |= wi < 0;
                if (i == i_seg) w = wi;
                if (i == i_seg + 1) next_bad = wi < 0;
            }
        }
    }
    // The workgroup's runs:
    //  - main, bound met: from the initial state at the sequence start, or
    //    from zero at its warm-up start, with output from the segment start.
    //    Every segment but the last parks its final state for the in-order
    //    pass, which hands it to the next segment if that one misses its
    //    bound.  The last segment writes state_out, unless state_out is
    //    state_in and other blocks of the sequence may still be reading it:
    //    then it parks its state as well and the in-order pass moves it.
    //  - main, bound missed: the map from the state that enters the segment
    //    to the one that leaves it, S -> M S + S0: S0 from zero, then M from
    //    the identity with v^ = 0 (zero conv taps: SiLU(0) = 0), both without
    //    output and parked; the in-order pass applies the map.
    //  - extra: from the state the in-order pass parked for the segment, with
    //    output.
    const bool missed = !extra && w < 0;
    {
        const float *src = nullptr;
        float *dst = nullptr;
        int c_from = sg.y, c_out = sg.y;
        if (extra) {
            src = ws.bstate + ((long)(k - 1) * Hv + h) * kStateFloats;
        } else if (!missed) {
            const bool direct = last && (first || !p.defer_final);
            src = w == si.x && p.state_in ? p.state_in + sbase : nullptr;
            dst = direct ? p.state_out + sbase : ws.bstate + ((long)k * Hv + h) * kStateFloats;
            c_from = w;
        } else {
            dst = ws.bstate + ((long)k * Hv + h) * kStateFloats;
            c_out = sg.z;
        }
        // conv taps of the wave's channel tiles
        bf16x8 taps[kChainCT][2];
#pragma unroll
        for (int x = 0; x < kChainCT; ++x)
#pragma unroll
            for (int m = 0; m < 2; ++m) taps[x][m] = conv_tap_frag(p.conv_w, cv + kCW * wave + 16 * x + (lane & 15), m, lane);
        state_load(S, src, wave, lane);
        chain_run(p, ws, buf0, buf1, stage, S, taps, ChainRun{si.x, si.z, si.w, c_from, sg.z, c_out, vs, hist}, h, g,
                  wave, lane);
        if (dst) state_store(S, dst, wave, lane);
    }
    if (missed) {
        const bf16x8 zero_taps[kChainCT][2] = {};
        state_identity(S, wave, lane);
        chain_run(p, ws, buf0, buf1, stage, S, zero_taps, ChainRun{si.x, si.z, si.w, sg.y, sg.z, sg.z, vs, hist}, h,
                  g, wave, lane);
        state_store(S, ws.mstate + ((long)k * Hv + h) * kStateFloats, wave, lane);
    }
    if (extra) return;
    // carried conv rows: the last three raw rows of the sequence (v channels
    // of head h; the first head of the group also writes the q and k
    // channels).  In place, the v rows wait for every workgroup of the
    // (sequence, head) that may read them (a later segment whose warm-up
    // reaches back to the sequence start does), so the in-order walk below
    // writes them; the q and k rows were read by the parallel pass only.
    if (first && p.conv_state_out && wave == 0)
        write_conv_rows(p, si, row, g, h, j == 0 ? 0 : 2, (p.defer_conv && nseg > 1) ? 2 : 3, lane);

    // The in-order walk, if any segment missed its bound or the call is in
    // place: the last workgroup of the sequence to finish does it.  A
    // workgroup publishes what it parked first if the walk will read it (its
    // own segment or the next one missed the bound, or the final state of an
    // in-place call).
    if (nseg <= 1 || (!any_bad && !p.defer_final && !p.defer_conv)) return;
    if (w < 0 || next_bad || (i_seg == nseg - 1 && p.defer_final)) __threadfence();
    __syncthreads();
    if (t == 0) s_total = atomicAdd(ws.seg_done + (long)s * Hv + h, 1) + 1;
    __syncthreads();
    if (s_total != nseg) return;  // not the last to finish
    __threadfence();
    bool carry = false;   // S holds the final state of the previous segment
    bool m_next = false;  // mreg holds (or is receiving) the M of segment ss.x + i
    f32x4 mreg[kMRegs];
    for (int i = 1; any_bad && i < nseg; ++i) {  // a sequence's first segment always meets its bound
        const int kk = ss.x + i;
        const int4 sk = Tables::seg(p, ws, kk);
        if (warm_start(ws, h, Hv, sk.y, si.x, lane) >= 0) {
            carry = m_next = false;
            continue;
        }
        // S <- M S + S0: the state leaving segment kk from the one entering
        // it, which its extra workgroup reads from the previous slot; the
        // next segment's M is requested meanwhile, in case it is needed
        float *park = ws.bstate + ((long)kk * Hv + h) * kStateFloats;
        if (!carry) state_load(S, ws.bstate + ((long)(kk - 1) * Hv + h) * kStateFloats, wave, lane);
        if (!m_next) m_fetch(mreg, ws.mstate + ((long)kk * Hv + h) * kStateFloats);
        m_next = i < nseg - 1;
        state_affine(S, mreg, m_next ? ws.mstate + ((long)(kk + 1) * Hv + h) * kStateFloats : nullptr, park, buf0,
                     buf1, wave, lane);
        if (i < nseg - 1) state_store(S, park, wave, lane);
        carry = true;
    }
    // the extra workgroups of the segments that missed their bounds may start
    if (any_bad) {
        __threadfence();
        __syncthreads();
        if (t == 0) __hip_atomic_store(ws.seg_ready + (long)s * Hv + h, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the final state, when the walk formed the last segment's or it was parked
    if (carry || p.defer_final) {
        if (!carry) state_load(S, ws.bstate + ((long)(ss.x + nseg - 1) * Hv + h) * kStateFloats, wave, lane);
        state_store(S, p.state_out + sbase, wave, lane);
    }
    // the v rows of an in-place conv carry, now that no workgroup reads them
    if (p.defer_conv && p.conv_state_out && wave == 0) write_conv_rows(p, si, row, g, h, 2, 3, lane);
}

}  // namespace

int choose_seg_chunks(int max_chunks, int N, int Hv)
{
    // Makespan model of the segmented sequential pass, for sequences of the
    // mean length: blocks = segments x Hv, run in rounds of kSlots resident
    // blocks (256 CUs, one block each), each round as long as a segment plus
    // its warm-up chunks (the first segment, kSegLead chunks longer, has
    // none).  The cheapest cut wins; ties go to longer segments.
    constexpr long kSlots = 256;
    constexpr int kWarmGuess = kSegLead, kMinSeg = 8;
    if (N <= 0 || max_chunks <= 0) return kMinSeg;
    const int nch = (max_chunks + N - 1) / N;
    if (nch <= kMinSeg) return kMinSeg;
    const long units = (long)N * Hv * kChainBlocksPerHead;
    long best_cost = -1;
    int best = nch;
    // for a given number of segments the shortest even cut is the best one
    for (int nseg = 1;; ++nseg) {
        const int Ls = nseg == 1 ? nch : (nch - kSegLead + nseg - 1) / nseg;
        if (nseg > 1 && Ls < kMinSeg) break;
        const long rounds = (units * nseg + kSlots - 1) / kSlots;
        const long cost = rounds * (Ls + (nseg > 1 ? kWarmGuess : 0));
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = Ls;
        }
    }
    return best;
}

size_t prefill_workspace_bytes(int max_chunks, int N, int Hqk, int Hv)
{
    const size_t C = (size_t)max_chunks;
    const size_t M = (size_t)max_segments(max_chunks, N, choose_seg_chunks(max_chunks, N, Hv));
    size_t total = 0;
    total += align256(C * sizeof(int4));
    total += align256((size_t)N * sizeof(int4));
    total += align256(C * Hqk * kQFragBytes);
    total += align256(C * Hqk * kKFragBytes);
    total += align256(C * Hv * kRecBytes);
    total += align256(M * sizeof(int4));
    total += align256(M * sizeof(int));
    total += align256((size_t)N * sizeof(int4));
    total += align256(M * Hv * kStateFloats * sizeof(float));
    total += align256(M * Hv * kStateFloats * sizeof(float));
    total += align256((size_t)N * Hv * sizeof(int));
    total += align256((size_t)N * Hv * sizeof(int));
    return total;
}

Workspace carve_workspace(void *base, int max_chunks, int N, int Hqk, int Hv)
{
    const size_t C = (size_t)max_chunks;
    const size_t M = (size_t)max_segments(max_chunks, N, choose_seg_chunks(max_chunks, N, Hv));
    uint8_t *ptr = static_cast<uint8_t *>(base);
    Workspace ws;
    auto take = [&](size_t bytes) {
        uint8_t *r = ptr;
        ptr += align256(bytes);
        return r;
    };
    ws.chunk_info = reinterpret_cast<int4 *>(take(C * sizeof(int4)));
    ws.seq_info = reinterpret_cast<int4 *>(take((size_t)N * sizeof(int4)));
    ws.qfrag = take(C * Hqk * kQFragBytes);
    ws.kfrag = take(C * Hqk * kKFragBytes);
    ws.hrec = take(C * Hv * kRecBytes);
    ws.seg_info = reinterpret_cast<int4 *>(take(M * sizeof(int4)));
    ws.seg_order = reinterpret_cast<int *>(take(M * sizeof(int)));
    ws.seq_seg = reinterpret_cast<int4 *>(take((size_t)N * sizeof(int4)));
    ws.bstate = reinterpret_cast<float *>(take(M * Hv * kStateFloats * sizeof(float)));
    ws.mstate = reinterpret_cast<float *>(take(M * Hv * kStateFloats * sizeof(float)));
    ws.seg_done = reinterpret_cast<int *>(take((size_t)N * Hv * sizeof(int)));
    ws.seg_ready = reinterpret_cast<int *>(take((size_t)N * Hv * sizeof(int)));
    return ws;
}

hipError_t launch_prefill(const PrefillArgs &p, void *workspace, hipStream_t stream,
                          hipEvent_t const *events)
{
    const Workspace ws = carve_workspace(workspace, p.max_chunks, p.N, p.Hqk, p.Hv);
    hipError_t e;
    auto mark = [&](int i) { return events ? hipEventRecord(events[i], stream) : hipSuccess; };
    if ((e = mark(0)) != hipSuccess) return e;
    if (p.cu_seqlens) {
        hipLaunchKernelGGL(setup_kernel, dim3(1), dim3(1024), 0, stream, p, ws);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = mark(1)) != hipSuccess) return e;
    if (p.max_chunks > 0) {
        const long units = (long)p.max_chunks * p.Hqk;
        hipLaunchKernelGGL(prep_kernel, dim3((unsigned)units), dim3(kPrepThreads), 0, stream, p, ws);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = mark(2)) != hipSuccess) return e;
    const int G = p.Hv / p.Hqk;
    const long seg_groups = (long)p.max_segs * p.Hqk;
    const long seg_blocks = ((seg_groups + 7) / 8) * 8L * G;
    // main workgroups, then as many extra ones (started after every main one)
    hipLaunchKernelGGL(chain_kernel, dim3((unsigned)(2 * seg_blocks)), dim3(kChainThreads), 0, stream, p, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark(3);
}

}  // namespace gdn
