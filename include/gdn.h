/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet (GDN) token mixer.
 *
 * The mixer (local-inference walkthrough, bjdmk.com.cn, section 2.1; hybrid-
 * attention explainer, jianying88.com, section 3) keeps one fixed-size state
 * matrix S (d_k x d_v, fp32) per (sequence, V head) and, for every token t:
 *
 *   1. short causal depthwise conv of width 4 over the raw q, k, v channels,
 *      then SiLU; q^ and k^ are L2-normalised per (token, QK head), eps = 1e-6
 *      inside the square root; v^ is not normalised;
 *   2. beta_t = sigmoid(b_t) (write strength), alpha_t = exp(-gate_scale *
 *      softplus(a_t)) (forget gate), one scalar each per (token, V head);
 *   3. S_t = alpha_t (I - beta_t k^_t k^_t^T) S_{t-1} + beta_t k^_t v^_t^T;
 *   4. o_t = q_scale * S_t^T q^_t.
 *
 * V head h reads QK head h / (Hv / Hqk): contiguous groups of Hv / Hqk V heads
 * share one QK head (16 QK heads for 48 V heads in the explainer's config).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, row-major, innermost last.
 *    bf16 tensors are passed as uint16_t bit patterns.
 *  - Conv channels are ordered q | k | v: C_tot = 2*Hqk*d_k + Hv*d_v.
 *    conv_w is [C_tot][4] bf16; tap 3 multiplies the current token, taps
 *    0..2 the three previous tokens.  Conv states are [.][3][C_tot] bf16 raw
 *    (pre-conv) rows, oldest first.
 *  - The library allocates nothing, keeps no pointer after it returns and
 *    holds no global state.  All work is enqueued on `stream` (a hipStream_t;
 *    NULL = the default stream); the call returns before the GPU finishes,
 *    and every buffer must stay valid until the stream has passed the work.
 *  - Arguments are validated before any HIP call: on an error status nothing
 *    is launched and no output is touched.  Device faults are asynchronous
 *    and surface at the caller's next stream synchronisation.
 *  - Supported shapes: d_k = d_v = 128, Hv a multiple of Hqk, every pointer
 *    16-byte aligned except a, b, cu_seqlens (4-byte).
 *  - Numerics: bf16 I/O, fp32 state, fp32 accumulation; the chunked prefill
 *    feeds its dense products to the matrix cores as fp16 operands (see the
 *    repository's design notes for the error budget).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, size <= 0, misaligned */
    GDN_ERR_UNSUPPORTED = 2,      /* d_k or d_v != 128, Hv % Hqk != 0 */
    GDN_ERR_WORKSPACE_TOO_SMALL = 3,
    GDN_ERR_HIP = 4               /* a HIP launch or query failed */
};

/* Human-readable name of a status code (static storage, never NULL). */
const char *gdn_status_string(int status);

/* Bytes of device workspace gdn_prefill needs to run these sizes at once
 * (with less, down to the size for T = 64, it runs in windows). */
size_t gdn_prefill_workspace_size(int B, int T, int Hqk, int Hv, int dk, int dv);

/*
 * Chunked prefill of B sequences of equal length T (the WY / chunk-parallel
 * evaluation of the update that the walkthrough's section 2.1 names; exact up
 * to rounding order).
 *
 *   q, k           [B][T][Hqk][dk] bf16, raw (pre-conv)
 *   v              [B][T][Hv][dv]  bf16, raw (pre-conv)
 *   a, b           [B][T][Hv] fp32 raw gate pre-activations (a -> alpha, b -> beta)
 *   conv_w         [C_tot][4] bf16
 *   conv_state_in  [B][3][C_tot] bf16 history rows, or NULL (zero history)
 *   conv_state_out [B][3][C_tot] bf16, or NULL (not written): the last three
 *                  raw rows of each sequence (reaching into conv_state_in when
 *                  T < 3); may equal conv_state_in (in place), any other
 *                  overlap is undefined
 *   state_in       [B][Hv][dk][dv] fp32 initial state, or NULL (zeros)
 *   state_out      [B][Hv][dk][dv] fp32 final state; may equal state_in
 *                  (in place), any other overlap is undefined
 *   o              [B][T][Hv][dv] bf16 output (round to nearest even)
 *   workspace      device scratch, 16-byte aligned (a misaligned one is
 *                  rejected with GDN_ERR_INVALID_ARGUMENT); its contents on
 *                  entry are irrelevant.  With gdn_prefill_workspace_size(B,
 *                  T, ...) bytes or more the call runs at once.  With less,
 *                  but at least gdn_prefill_workspace_size(B, 64, ...), it
 *                  runs in windows of Tw tokens of every sequence, Tw the
 *                  largest multiple of 64 whose workspace fits.  Each window
 *                  continues the sequences from the state (handed over in
 *                  two state buffers at the workspace's end, or, when they
 *                  do not fit, in state_out in place) and the input rows the
 *                  previous one left, so the chunk grid is the call's own
 *                  and the result equals the one-window result up to
 *                  rounding.  The workspace then stays bounded whatever T is:
 *                  the explainer (section 3) stresses the mixer's fixed-size
 *                  state.  With less than one 64-token window's worth it
 *                  returns GDN_ERR_WORKSPACE_TOO_SMALL, nothing launched.
 * T = 0 copies state_in to state_out (zeros if state_in is NULL).
 */
int gdn_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                const float *a, const float *b, const uint16_t *conv_w,
                const uint16_t *conv_state_in, uint16_t *conv_state_out,
                const float *state_in, float *state_out, uint16_t *o,
                int B, int T, int Hqk, int Hv, int dk, int dv,
                float gate_scale, float q_scale,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Measurement variant of gdn_prefill: the same work on the same stream, and
 * additionally records four caller-created HIP events (events[i] is a
 * hipEvent_t), so that the caller can time each of the three kernels with
 * hipEventElapsedTime: events[0] before the first kernel, then one after each
 * of the chunk-table setup (nothing is launched for uniform batches), the
 * parallel per-chunk pass and the segmented sequential pass (which includes
 * the in-order combine of the segments that miss their warm-up bound).  events must not be NULL and must hold
 * four events.
 */
int gdn_prefill_with_events(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const float *a, const float *b, const uint16_t *conv_w,
                            const uint16_t *conv_state_in, uint16_t *conv_state_out,
                            const float *state_in, float *state_out, uint16_t *o,
                            int B, int T, int Hqk, int Hv, int dk, int dv,
                            float gate_scale, float q_scale,
                            void *workspace, size_t workspace_bytes, void *stream,
                            void *const *events);

/*
 * gdn_prefill for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels as gdn_prefill, with the workspace taken from
 * a file-scope device array of the library instead of a caller's buffer.  It
 * calls no hipMalloc, hipFree or other allocating routine.
 *
 *   - Every other argument is as for gdn_prefill; there is no workspace.
 *   - The array holds gdn_prefill_noalloc_max_workspace() bytes (192 MiB)
 *     on each GPU the library runs on, until the process ends.  A call
 *     longer than the array holds runs in windows, as gdn_prefill does with
 *     a short workspace (at 16 QK / 48 V heads and B = 1: at once up to
 *     T = 8192, in windows beyond).  A batch whose 64-token window alone
 *     exceeds the array returns GDN_ERR_WORKSPACE_TOO_SMALL, nothing
 *     launched.
 *   - The array of the CURRENT device is used (hipGetDevice), which must be
 *     the device of `stream`.  Its address is looked up with
 *     hipGetSymbolAddress on the first call on each device and kept: this
 *     entry point, unlike the others, keeps that per-device address.
 *   - All calls on one GPU share its array, and the array keeps the last
 *     call's contents (the kernels clear what must start at zero): two calls
 *     that overlap in time on one GPU (on different streams, or on one
 *     stream from several host threads without ordering) race and give
 *     undefined results.  Calls ordered on one stream are safe.
 */
int gdn_prefill_noalloc(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const float *a, const float *b, const uint16_t *conv_w,
                        const uint16_t *conv_state_in, uint16_t *conv_state_out,
                        const float *state_in, float *state_out, uint16_t *o,
                        int B, int T, int Hqk, int Hv, int dk, int dv,
                        float gate_scale, float q_scale, void *stream);

/* Bytes of the device array gdn_prefill_noalloc uses as its workspace. */
size_t gdn_prefill_noalloc_max_workspace(void);

/*
 * Measurement variant of gdn_prefill with a choice of how the sequential
 * pass splits each sequence (the intra-card sequence parallelism that the
 * architecture deep dive, alwayszhang.cn, section 9, names among FlashQLA's
 * features for TP, long-sequence and few-head settings): seg_chunks = 0 lets
 * the library choose, as gdn_prefill does; a positive value makes every
 * segment at least that many 64-token chunks long (never more segments than
 * the library's choice, so the workspace of gdn_prefill_workspace_size
 * suffices); a value at least the sequence's chunk count runs each sequence
 * as one segment.  The results are those of gdn_prefill up to rounding order
 * (bit for bit when the split is the same).  events: NULL, or four events as
 * for gdn_prefill_with_events.
 */
int gdn_prefill_with_options(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *a, const float *b, const uint16_t *conv_w,
                             const uint16_t *conv_state_in, uint16_t *conv_state_out,
                             const float *state_in, float *state_out, uint16_t *o,
                             int B, int T, int Hqk, int Hv, int dk, int dv,
                             float gate_scale, float q_scale,
                             void *workspace, size_t workspace_bytes, void *stream,
                             int seg_chunks, void *const *events);

/* Bytes of device workspace gdn_prefill_varlen needs (any lengths summing to
 * T_tot over N sequences). */
size_t gdn_prefill_varlen_workspace_size(int N, int T_tot, int Hqk, int Hv, int dk, int dv);

/*
 * Packed variable-length prefill with state carry-in: the continuation of a
 * prefix.  The local-inference walkthrough (bjdmk.com.cn) serves the model
 * with chunked prefill and prefix caching switched on (section 3, the engine
 * configuration; section 5, chunked prefill against out-of-memory errors;
 * section 6, prefix caching for repeated long prompts).  Both resume a
 * sequence from the state and the conv rows a previous call left, which is
 * what state_in and conv_state_in carry.  Same as gdn_prefill, except:
 *
 *   q, k           [T_tot][Hqk][dk], v [T_tot][Hv][dv], a, b [T_tot][Hv],
 *                  o [T_tot][Hv][dv]: tokens of all sequences packed
 *   cu_seqlens     DEVICE int32 [N+1], cu_seqlens[0] = 0, non-decreasing,
 *                  cu_seqlens[N] = T_tot; read on the device only (no host
 *                  synchronisation).  Values outside that contract are
 *                  undefined behaviour.
 *   conv_state_*   [N][3][C_tot];  state_*  [N][Hv][dk][dv]
 * Sequences never see each other's tokens: each starts from its own
 * state_in / conv_state_in row (or zeros).  Empty sequences copy their state.
 */
int gdn_prefill_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const float *a, const float *b, const uint16_t *conv_w,
                       const uint16_t *conv_state_in, uint16_t *conv_state_out,
                       const float *state_in, float *state_out, uint16_t *o,
                       const int32_t *cu_seqlens, int N, int T_tot,
                       int Hqk, int Hv, int dk, int dv,
                       float gate_scale, float q_scale,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * gdn_prefill_varlen with a slot table into state and conv-row pools: the
 * prefill side of a serving engine's state cache (prefix caching and chunked
 * prefill resume a sequence from the cache row its previous call left;
 * walkthrough, bjdmk.com.cn, sections 3 and 6).  Same as gdn_prefill_varlen,
 * except:
 *
 *   slots          DEVICE int32 [N] (required): sequence s reads row slots[s]
 *                  of state_in and conv_state_in and writes row slots[s] of
 *                  state_out and conv_state_out
 *   n_rows         rows of each pool: state_* [n_rows][Hv][dk][dv],
 *                  conv_state_* [n_rows][3][C_tot]
 * A sequence whose slot lies outside [0, n_rows) is skipped: none of its
 * outputs (o rows, state, conv rows) is written.  Two sequences must not
 * share a slot.  The pools may be updated in place (state_out == state_in,
 * conv_state_out == conv_state_in); rows no sequence names are untouched.
 */
int gdn_prefill_varlen_slots(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *a, const float *b, const uint16_t *conv_w,
                             const uint16_t *conv_state_in, uint16_t *conv_state_out,
                             const float *state_in, float *state_out, uint16_t *o,
                             const int32_t *cu_seqlens, const int32_t *slots, int n_rows,
                             int N, int T_tot, int Hqk, int Hv, int dk, int dv,
                             float gate_scale, float q_scale,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode step: one new token for each of B independent sequences (the
 * pages' constant-cost decode: a token only reads and updates the fixed-size
 * memory; hybrid-attention explainer, section 3).
 *
 *   q, k        [B][Hqk][dk] bf16 raw;  v [B][Hv][dv] bf16 raw
 *   a, b        [B][Hv] fp32
 *   conv_state  [B][3][C_tot] bf16, updated IN PLACE: rows shift up by one
 *               and the new raw token becomes row 2
 *   state_in    [B][Hv][dk][dv] fp32
 *   state_out   [B][Hv][dk][dv] fp32; may equal state_in (in place)
 *   o           [B][Hv][dv] bf16
 * No workspace.  B = 0 is a no-op.
 */
int gdn_decode_step(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *a, const float *b, const uint16_t *conv_w,
                    uint16_t *conv_state, const float *state_in, float *state_out,
                    uint16_t *o, int B, int Hqk, int Hv, int dk, int dv,
                    float gate_scale, float q_scale, void *stream);

/*
 * Multi-token decode with an optional slot table: T = 1..4 new tokens for
 * each of B sequences, processed in order, the state read once and written
 * once.  This is the verification step of speculative decoding with the
 * model's multi-token-prediction head: the walkthrough (bjdmk.com.cn) serves
 * with num_speculative_tokens = 3 (section 3) and measures its gain (section
 * 4); the architecture deep dive (alwayszhang.cn, section 7) describes the MTP
 * head and its use for speculative decoding.  The slot table addresses the
 * state and conv caches of a serving engine (walkthrough, sections 3 and 6:
 * prefix caching keeps those caches across requests).  The same result as T
 * successive calls of gdn_decode_step up to fp32 rounding: for T >= 2 the
 * tokens are taken from one pass over the state (the one-token update
 * unrolled over the T tokens), so its sums run in another order; T = 1 is
 * gdn_decode_step's own computation.
 *
 *   q, k        [B][T][Hqk][dk] bf16 raw;  v [B][T][Hv][dv] bf16 raw
 *   a, b        [B][T][Hv] fp32
 *   o           [B][T][Hv][dv] bf16: the output of every token
 *   slots       DEVICE int32 [B], or NULL.  With a table, sequence b reads and
 *               writes row slots[b] of state_in / state_out ([n_rows][Hv][dk][dv])
 *               and of conv_state ([n_rows][3][C_tot]), the state cache of a
 *               serving engine; a sequence whose slot lies outside
 *               [0, n_rows) is skipped (its outputs are not written).  Two
 *               sequences must not share a slot.  Without a table, row b and
 *               n_rows is ignored.
 *   conv_state  updated IN PLACE: its rows become the last three raw rows
 *   state_out   may equal state_in (in place).  To take back the tokens a
 *               verifier rejects, keep state_in and conv rows separate from the
 *               outputs (state_out != state_in and a copy of the conv rows),
 *               then advance the accepted prefix with a second call.
 * T < 1 is invalid; T > 4 is unsupported.
 */
int gdn_decode_multi(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const float *a, const float *b, const uint16_t *conv_w,
                     uint16_t *conv_state, const float *state_in, float *state_out,
                     uint16_t *o, const int32_t *slots, int n_rows,
                     int B, int T, int Hqk, int Hv, int dk, int dv,
                     float gate_scale, float q_scale, void *stream);

/* Bytes of device workspace gdn_prefill_backward needs for these sizes (0 when
 * B * T = 0; about 0.36 MB per token at Hqk = 16, Hv = 48). */
size_t gdn_prefill_backward_workspace_size(int B, int T, int Hqk, int Hv, int dk, int dv);

/*
 * Training backward of gdn_prefill: the gradients of
 *     L = sum_t <grad_o_t, o_t> + <grad_state_out, state_out>
 * with respect to every input, for B sequences of equal length T.  The
 * chunked form of the update (the WY / chunk-parallel evaluation of the
 * walkthrough's section 2.1; section 9 of the architecture deep dive on
 * alwayszhang.cn describes FlashQLA's forward and backward kernels of this
 * chunked training form) is
 * differentiated line by line; all arithmetic is fp32.
 *
 *   q, k, v, a, b, conv_w, conv_state_in, state_in, gate_scale, q_scale:
 *                    the forward call's inputs (conv_state_in, state_in may
 *                    be NULL: zero history / zero state)
 *   grad_o           [B][T][Hv][dv] bf16 gradient of o
 *   grad_state_out   [B][Hv][dk][dv] fp32 gradient of state_out, or NULL (zero)
 *   grad_q, grad_k   [B][T][Hqk][dk] fp32  (of the raw, pre-conv q, k)
 *   grad_v           [B][T][Hv][dv] fp32
 *   grad_a, grad_b   [B][T][Hv] fp32
 *   grad_conv_w      [C_tot][4] fp32, summed over the batch
 *   grad_conv_state_in [B][3][C_tot] fp32, or NULL (not computed): the
 *                    gradient of the history rows (of zero rows when
 *                    conv_state_in is NULL)
 *   grad_state_in    [B][Hv][dk][dv] fp32, or NULL (not computed)
 *   workspace        device scratch, 16-byte aligned; its contents on entry
 *                    are irrelevant.  With gdn_prefill_backward_workspace_size
 *                    bytes or more the batch runs at once.  With less, it runs
 *                    sequence by sequence, each in windows of Tw tokens (Tw a
 *                    multiple of 64, the largest whose plan fits; the chunk
 *                    grid is the one-pass grid): a forward sweep keeps the
 *                    state entering every window (Hv x 64 KiB each), then the
 *                    windows' backwards run from the last, each handing its
 *                    state gradient and the gradient of its three history
 *                    rows to the window before it.  The result equals the
 *                    one-pass result up to rounding (the conv weight gradient
 *                    is summed in another order).  gdn_prefill_backward_windows
 *                    reports Tw; when not even 64-token windows fit it
 *                    returns GDN_ERR_WORKSPACE_TOO_SMALL, nothing launched.
 *                    The workspace then stays bounded by one window's
 *                    backward plus the window states, whatever T is (the
 *                    explainer, section 3, stresses the mixer's fixed-size
 *                    state).
 * Every gradient is overwritten (not accumulated).  Outputs must not overlap
 * each other, the inputs or the workspace.  Pointers 4-byte aligned, grad_o
 * 8-byte aligned.  With
 * T = 0, grad_state_in = grad_state_out (or zeros) and the conv gradients
 * are zero.
 */
int gdn_prefill_backward(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const float *a, const float *b, const uint16_t *conv_w,
                         const uint16_t *conv_state_in, const float *state_in,
                         const uint16_t *grad_o, const float *grad_state_out,
                         float *grad_q, float *grad_k, float *grad_v,
                         float *grad_a, float *grad_b, float *grad_conv_w,
                         float *grad_conv_state_in, float *grad_state_in,
                         int B, int T, int Hqk, int Hv, int dk, int dv,
                         float gate_scale, float q_scale,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Window length gdn_prefill_backward takes with workspace_bytes of workspace
 * for these sizes: *window_tokens = T when the whole batch runs at once (also
 * when B * T = 0), else the window length Tw of its sequence-by-sequence run.
 * Returns GDN_OK, or GDN_ERR_WORKSPACE_TOO_SMALL when not even 64-token
 * windows fit (GDN_ERR_INVALID_ARGUMENT / GDN_ERR_UNSUPPORTED for bad sizes,
 * as gdn_prefill_backward).  Host only: no HIP call.
 */
int gdn_prefill_backward_windows(int B, int T, int Hqk, int Hv, int dk, int dv, size_t workspace_bytes,
                                 int *window_tokens);

/* Bytes of device workspace gdn_prefill_backward_varlen needs (an upper bound
 * over every split of T_tot tokens into N sequences; 0 when T_tot = 0). */
size_t gdn_prefill_backward_varlen_workspace_size(int N, int T_tot, int Hqk, int Hv, int dk, int dv);

/*
 * Training backward of gdn_prefill_varlen: the same gradients as
 * gdn_prefill_backward for N packed sequences of any lengths (chunking
 * restarts at every sequence start; empty sequences pass their state
 * gradient through).  cu_seqlens is the forward call's DEVICE int32 [N+1];
 * q, k, v, grad_q, grad_k, grad_v are [T_tot][H][d]; a, b, grad_a, grad_b
 * [T_tot][Hv]; grad_o [T_tot][Hv][dv]; states and their gradients
 * [N][Hv][dk][dv]; conv rows and their gradient [N][3][C_tot].  Bounds
 * outside [0, T_tot] are clamped.  The workspace must hold the whole call
 * (a caller with a memory budget splits the batch into calls, or uses
 * gdn_prefill_backward sequence by sequence).  Other rules as
 * gdn_prefill_backward.
 */
int gdn_prefill_backward_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *a, const float *b, const uint16_t *conv_w,
                                const uint16_t *conv_state_in, const float *state_in,
                                const uint16_t *grad_o, const float *grad_state_out,
                                float *grad_q, float *grad_k, float *grad_v,
                                float *grad_a, float *grad_b, float *grad_conv_w,
                                float *grad_conv_state_in, float *grad_state_in,
                                const int32_t *cu_seqlens, int N, int T_tot,
                                int Hqk, int Hv, int dk, int dv,
                                float gate_scale, float q_scale,
                                void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
