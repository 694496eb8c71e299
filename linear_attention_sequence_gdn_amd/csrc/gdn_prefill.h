// gdn_prefill.h -- internal interface of the chunked prefill (not the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn_common.h"

namespace gdn {

struct PrefillArgs {
    const uint16_t *q, *k, *v;
    const float *a, *b;
    const uint16_t *conv_w;
    const uint16_t *conv_state_in;
    uint16_t *conv_state_out;
    const float *state_in;
    float *state_out;
    uint16_t *o;
    const int32_t *cu_seqlens;  // NULL: N sequences of T_uniform tokens
    int N, T_uniform, T_tot;
    // uniform calls: sequence s's tokens start at s * T_stride + t_off (a
    // window of T_uniform tokens of longer sequences; T_stride = T_uniform,
    // t_off = 0 for a whole call); cont: the window continues its sequences,
    // so the rows before its first chunk are the sequences' own earlier rows
    int T_stride, t_off, cont;
    int Hqk, Hv;
    float gate_scale, q_scale;
    int max_chunks;
    int seg_chunks;  // chunks per segment of the sequential pass
    int max_segs;    // bound of the number of segments
    int defer_final; // state_out is state_in: final states go through the in-order pass
    int defer_conv;  // conv_state_out is conv_state_in: the v rows are written by the in-order pass
    const int32_t *slots;  // NULL, or DEVICE [N]: sequence s reads and writes row slots[s] of the
    int n_rows;            // state and conv-row pools of n_rows rows (out of range: skipped)
};

// Pool row of sequence s (s itself without a slot table), or -1 when its slot
// lies outside the pool.
__device__ __forceinline__ int seq_row(const PrefillArgs &p, int s)
{
    if (!p.slots) return s;
    const int r = p.slots[s];
    return (r >= 0 && r < p.n_rows) ? r : -1;
}

// Upper bound of the number of 64-token chunks.
inline int max_chunks_uniform(int B, int T) { return B * ((T + kChunk - 1) / kChunk); }
inline int max_chunks_varlen(int N, int T_tot)
{
    return (int)(((long)T_tot + (long)(kChunk - 1) * N) / kChunk);
}

// Per-chunk hand-over from the parallel prep pass to the sequential pass, in
// bytes.  The fp16 operands are stored in the register order of the
// matrix-core instruction that consumes them.
constexpr size_t kFragBytes = 64 * 16;               // one 16x32 fp16 operand
constexpr size_t kQFragBytes = 16 * kFragBytes;      // q^ of a chunk     [64 x 128]
constexpr size_t kKFragBytes = 16 * kFragBytes;      // k^ of a chunk     [64 x 128]
// Per (chunk, V head) record: P, T', gates.  The two lower-triangular 64 x 64
// matrices keep the six 16x32 fragments that are not structurally zero: (row
// tile, key block) (0,0) (1,0) (2,0) (2,1) (3,0) (3,1), f = 0..5 in that
// order.  Fragments 0 and 3 are zero in their upper halves (elements 4..7 of
// every lane), so each matrix is stored compactly in 5 KiB: fragments 1, 2, 4,
// 5 whole (16 bytes per lane), then the lower halves of fragments 0 and 3 (8
// bytes per lane each); tri_off gives the place of a lane's half.  Gate
// floats: [0,64) q_scale Gamma, [64,128) Gamma_n / Gamma, 128 Gamma_n, 129
// log2 Gamma_n, [192,256) Gamma.
constexpr size_t kTriBytes = 5 * kFragBytes;         // a compact lower-triangular operand [64 x 64]
constexpr size_t kGateFloats = 256;
constexpr size_t kRecT = 0, kRecP = kTriBytes, kRecG = 2 * kTriBytes;
constexpr size_t kRecBytes = kRecG + kGateFloats * 4;  // 11 KiB
__host__ __device__ constexpr bool tri_half_only(int f) { return f == 0 || f == 3; }
// byte offset of 8-byte half hb (0 for fragments 0 and 3) of lane `lane` of fragment f
__host__ __device__ constexpr int tri_off(int f, int hb, int lane)
{
    return tri_half_only(f) ? 4096 + 512 * (f == 3) + 8 * lane : 1024 * (f - 1 - (f > 3)) + 16 * lane + 8 * hb;
}
constexpr size_t kStateFloats = 128 * 128;          // one fp32 state

struct Workspace {
    int4 *chunk_info;   // [max_chunks] {seq, t0, n, first}
    int4 *seq_info;     // [N] {chunk0, nchunks, t0, L}
    uint8_t *qfrag;     // [max_chunks][Hqk]
    uint8_t *kfrag;     // [max_chunks][Hqk]  k^ (token rows, d contraction)
    uint8_t *hrec;      // [max_chunks][Hv] P, T', gates
    int4 *seg_info;     // [max_segs] {seq, first chunk, end chunk, 1: first of seq | 2: last of seq}; seq -1 = unused
    int *seg_order;     // [max_segs] segments longest first: the sequential pass's order (packed calls only)
    int4 *seq_seg;      // [N] {first segment, segments, -, -}
    float *bstate;      // [max_segs][Hv][128][128] final state of a segment (read by the in-order combine and by the
                        // extra workgroup of its successor); a segment that misses its warm-up bound parks here its
                        // final state from a zero start, which the combine replaces by the true one
    float *mstate;      // [max_segs][Hv][128][128] transition matrix of a segment that misses its warm-up bound
    int *seg_done;      // [N][Hv] segments of the pair finished, when the in-order walk is needed (zeroed by the parallel pass)
    int *seg_ready;     // [N][Hv] the pair's in-order combine is done (zeroed by the parallel pass)
};

// Segments of the sequential pass: each sequence's chunks are cut into runs
// that proceed in parallel, seg_chunks long (chosen from the sizes alone, so
// that the workspace size is a function of the arguments), except that the
// first run of a sequence takes kSegLead more chunks: it starts from the
// sequence's own initial state and needs no warm-up, while every later run
// first re-runs a few chunks before its start (typically four, each about
// 0.7 of a full chunk step since it forms no output: about three steps).
int choose_seg_chunks(int max_chunks, int N, int Hv);
inline int max_segments(int max_chunks, int N, int seg_chunks) { return max_chunks / seg_chunks + N; }
constexpr int kSegLead = 3;
// segments of a sequence of nch chunks, and the chunk range [begin, end) of
// segment i (relative to the sequence's first chunk)
__host__ __device__ inline int seg_count(int nch, int seg_chunks)
{
    const int r = (nch - kSegLead + seg_chunks - 1) / seg_chunks;
    return r > 1 ? r : 1;
}
__host__ __device__ inline int seg_begin(int i, int seg_chunks) { return i == 0 ? 0 : i * seg_chunks + kSegLead; }
__host__ __device__ inline int seg_end(int i, int nch, int seg_chunks)
{
    const int e = (i + 1) * seg_chunks + kSegLead;
    return e < nch ? e : nch;
}

size_t prefill_workspace_bytes(int max_chunks, int N, int Hqk, int Hv);
Workspace carve_workspace(void *base, int max_chunks, int N, int Hqk, int Hv);
// events: NULL, or kPrefillEvents events recorded before the first kernel and
// after each of the three (setup, prep, chain).
constexpr int kPrefillEvents = 4;
hipError_t launch_prefill(const PrefillArgs &p, void *workspace, hipStream_t stream,
                          hipEvent_t const *events = nullptr);

}  // namespace gdn
