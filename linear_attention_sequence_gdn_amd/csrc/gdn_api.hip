// gdn_api.hip -- the C ABI (include/gdn.h): argument validation, workspace
// carving and kernel launches on the caller's stream.
//
// Validation runs before any HIP call, so every error path returns with
// nothing launched and no output touched.
#include "../../include/gdn.h"

#include <hip/hip_runtime.h>

#include "gdn_prefill.h"

namespace gdn {
hipError_t launch_decode(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                         const float *b, const uint16_t *conv_w, uint16_t *conv_state,
                         const float *state_in, float *state_out, uint16_t *o, const int32_t *slots,
                         int n_rows, int B, int T, int Hqk, int Hv, float gate_scale, float q_scale,
                         hipStream_t stream);
size_t backward_workspace_bytes(int N, int T_tot, bool packed, int Hqk, int Hv);
hipError_t launch_backward(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                           const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                           const float *state_in, const uint16_t *grad_o, const float *grad_state_out,
                           float *grad_q, float *grad_k, float *grad_v, float *grad_a, float *grad_b,
                           float *grad_conv_w, float *grad_conv_state_in, float *grad_state_in,
                           const int32_t *cu_seqlens, int N, int T, int T_tot, int Hqk, int Hv, float gate_scale,
                           float q_scale, void *workspace, hipStream_t stream);
}  // namespace gdn

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_dims(int Hqk, int Hv, int dk, int dv)
{
    if (Hqk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0) return GDN_ERR_INVALID_ARGUMENT;
    if (dk != gdn::kD || dv != gdn::kD) return GDN_ERR_UNSUPPORTED;
    if (Hv % Hqk != 0) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_status_string(int status)
{
    switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "GDN_ERR_WORKSPACE_TOO_SMALL";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    default: return "GDN_ERR_UNKNOWN";
    }
}

int gdn_decode_multi(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                     const float *b, const uint16_t *conv_w, uint16_t *conv_state,
                     const float *state_in, float *state_out, uint16_t *o, const int32_t *slots,
                     int n_rows, int B, int T, int Hqk, int Hv, int dk, int dv, float gate_scale,
                     float q_scale, void *stream)
{
    if (B < 0 || T < 1) return GDN_ERR_INVALID_ARGUMENT;
    if (T > gdn::kMaxDecodeTokens) return GDN_ERR_UNSUPPORTED;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if (slots && n_rows < 0) return GDN_ERR_INVALID_ARGUMENT;
    if (B == 0) return GDN_OK;
    if (!q || !k || !v || !a || !b || !conv_w || !conv_state || !state_in || !state_out || !o)
        return GDN_ERR_INVALID_ARGUMENT;
    if (!aligned(state_in, 16) || !aligned(state_out, 16) || !aligned(conv_w, 8) ||
        !aligned(o, 8) || !aligned(q, 4) || !aligned(k, 4) || !aligned(v, 2) ||
        !aligned(conv_state, 4) || !aligned(a, 4) || !aligned(b, 4) || (slots && !aligned(slots, 4)))
        return GDN_ERR_INVALID_ARGUMENT;
    hipError_t e = gdn::launch_decode(q, k, v, a, b, conv_w, conv_state, state_in, state_out, o, slots,
                                      slots ? n_rows : B, B, T, Hqk, Hv, gate_scale, q_scale,
                                      reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_decode_step(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                    const float *b, const uint16_t *conv_w, uint16_t *conv_state,
                    const float *state_in, float *state_out, uint16_t *o, int B, int Hqk, int Hv,
                    int dk, int dv, float gate_scale, float q_scale, void *stream)
{
    return gdn_decode_multi(q, k, v, a, b, conv_w, conv_state, state_in, state_out, o, nullptr, 0, B, 1,
                            Hqk, Hv, dk, dv, gate_scale, q_scale, stream);
}

size_t gdn_prefill_workspace_size(int B, int T, int Hqk, int Hv, int dk, int dv)
{
    if (B < 0 || T < 0 || check_dims(Hqk, Hv, dk, dv) != GDN_OK) return 0;
    return gdn::prefill_workspace_bytes(gdn::max_chunks_uniform(B, T), B, Hqk, Hv);
}

size_t gdn_prefill_varlen_workspace_size(int N, int T_tot, int Hqk, int Hv, int dk, int dv)
{
    if (N < 0 || T_tot < 0 || check_dims(Hqk, Hv, dk, dv) != GDN_OK) return 0;
    return gdn::prefill_workspace_bytes(gdn::max_chunks_varlen(N, T_tot), N, Hqk, Hv);
}

static int prefill_common(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                          const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                          uint16_t *conv_state_out, const float *state_in, float *state_out,
                          uint16_t *o, const int32_t *cu_seqlens, int N, int T_uniform,
                          int T_tot, int Hqk, int Hv, float gate_scale, float q_scale,
                          void *workspace, size_t workspace_bytes, void *stream,
                          void *const *events = nullptr)
{
    if (!state_out || !conv_w) return GDN_ERR_INVALID_ARGUMENT;
    if (T_tot > 0 && (!q || !k || !v || !a || !b || !o)) return GDN_ERR_INVALID_ARGUMENT;
    const void *al16[] = {q, k, v, conv_w, conv_state_in, conv_state_out, state_in, state_out, o,
                          workspace};
    for (const void *ptr : al16)
        if (ptr && !aligned(ptr, 16)) return GDN_ERR_INVALID_ARGUMENT;
    if ((a && !aligned(a, 4)) || (b && !aligned(b, 4)) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return GDN_ERR_INVALID_ARGUMENT;
    if (conv_state_in && conv_state_out == conv_state_in) return GDN_ERR_INVALID_ARGUMENT;
    const int max_chunks = cu_seqlens ? gdn::max_chunks_varlen(N, T_tot)
                                      : gdn::max_chunks_uniform(N, T_uniform);
    const size_t need = gdn::prefill_workspace_bytes(max_chunks, N, Hqk, Hv);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE_TOO_SMALL;
    if (N == 0) return GDN_OK;

    gdn::PrefillArgs p{};
    p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.conv_w = conv_w;
    p.conv_state_in = conv_state_in; p.conv_state_out = conv_state_out;
    p.state_in = state_in; p.state_out = state_out; p.o = o;
    p.cu_seqlens = cu_seqlens; p.N = N; p.T_uniform = T_uniform; p.T_tot = T_tot;
    p.Hqk = Hqk; p.Hv = Hv; p.gate_scale = gate_scale; p.q_scale = q_scale;
    p.max_chunks = max_chunks;
    p.seg_chunks = gdn::choose_seg_chunks(max_chunks, N, Hv);
    p.max_segs = gdn::max_segments(max_chunks, N, p.seg_chunks);
    p.defer_final = state_in != nullptr && state_in == state_out;
    hipError_t e = gdn::launch_prefill(p, workspace, reinterpret_cast<hipStream_t>(stream),
                                       reinterpret_cast<hipEvent_t const *>(events));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_prefill(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                uint16_t *conv_state_out, const float *state_in, float *state_out, uint16_t *o,
                int B, int T, int Hqk, int Hv, int dk, int dv, float gate_scale, float q_scale,
                void *workspace, size_t workspace_bytes, void *stream)
{
    if (B < 0 || T < 0) return GDN_ERR_INVALID_ARGUMENT;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if ((long)B * T > 0x7fffffffL) return GDN_ERR_UNSUPPORTED;
    return prefill_common(q, k, v, a, b, conv_w, conv_state_in, conv_state_out, state_in,
                          state_out, o, nullptr, B, T, B * T, Hqk, Hv, gate_scale, q_scale,
                          workspace, workspace_bytes, stream);
}

int gdn_prefill_with_events(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                            const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                            uint16_t *conv_state_out, const float *state_in, float *state_out,
                            uint16_t *o, int B, int T, int Hqk, int Hv, int dk, int dv,
                            float gate_scale, float q_scale, void *workspace,
                            size_t workspace_bytes, void *stream, void *const *events)
{
    if (!events) return GDN_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < gdn::kPrefillEvents; ++i)
        if (!events[i]) return GDN_ERR_INVALID_ARGUMENT;
    if (B < 0 || T < 0) return GDN_ERR_INVALID_ARGUMENT;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if ((long)B * T > 0x7fffffffL) return GDN_ERR_UNSUPPORTED;
    return prefill_common(q, k, v, a, b, conv_w, conv_state_in, conv_state_out, state_in,
                          state_out, o, nullptr, B, T, B * T, Hqk, Hv, gate_scale, q_scale,
                          workspace, workspace_bytes, stream, events);
}

int gdn_prefill_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                       const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                       uint16_t *conv_state_out, const float *state_in, float *state_out,
                       uint16_t *o, const int32_t *cu_seqlens, int N, int T_tot, int Hqk, int Hv,
                       int dk, int dv, float gate_scale, float q_scale, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    if (N < 0 || T_tot < 0) return GDN_ERR_INVALID_ARGUMENT;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if (!cu_seqlens) return GDN_ERR_INVALID_ARGUMENT;
    return prefill_common(q, k, v, a, b, conv_w, conv_state_in, conv_state_out, state_in,
                          state_out, o, cu_seqlens, N, 0, T_tot, Hqk, Hv, gate_scale, q_scale,
                          workspace, workspace_bytes, stream);
}

size_t gdn_prefill_backward_workspace_size(int B, int T, int Hqk, int Hv, int dk, int dv)
{
    if (B < 0 || T < 0 || check_dims(Hqk, Hv, dk, dv) != GDN_OK) return 0;
    if ((long)B * T > 0x7fffffffL) return 0;
    return gdn::backward_workspace_bytes(B, B * T, false, Hqk, Hv);
}

size_t gdn_prefill_backward_varlen_workspace_size(int N, int T_tot, int Hqk, int Hv, int dk, int dv)
{
    if (N < 0 || T_tot < 0 || check_dims(Hqk, Hv, dk, dv) != GDN_OK) return 0;
    return gdn::backward_workspace_bytes(N, T_tot, true, Hqk, Hv);
}

static int backward_common(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                           const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                           const float *state_in, const uint16_t *grad_o, const float *grad_state_out,
                           float *grad_q, float *grad_k, float *grad_v, float *grad_a, float *grad_b,
                           float *grad_conv_w, float *grad_conv_state_in, float *grad_state_in,
                           const int32_t *cu_seqlens, int N, int T, int T_tot, int Hqk, int Hv,
                           float gate_scale, float q_scale, void *workspace, size_t workspace_bytes,
                           void *stream)
{
    if (!conv_w || !grad_conv_w) return GDN_ERR_INVALID_ARGUMENT;
    if (T_tot > 0 && (!q || !k || !v || !a || !b || !grad_o || !grad_q || !grad_k || !grad_v ||
                      !grad_a || !grad_b))
        return GDN_ERR_INVALID_ARGUMENT;
    const void *al4[] = {q, k, v, a, b, conv_w, conv_state_in, state_in, grad_o, grad_state_out,
                         grad_q, grad_k, grad_v, grad_a, grad_b, grad_conv_w, grad_conv_state_in,
                         grad_state_in, cu_seqlens};
    for (const void *ptr : al4)
        if (ptr && !aligned(ptr, 4)) return GDN_ERR_INVALID_ARGUMENT;
    if ((workspace && !aligned(workspace, 16)) || (grad_o && !aligned(grad_o, 8))) return GDN_ERR_INVALID_ARGUMENT;
    const size_t need = gdn::backward_workspace_bytes(N, T_tot, cu_seqlens != nullptr, Hqk, Hv);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE_TOO_SMALL;
    if (N == 0) return GDN_OK;
    hipError_t e = gdn::launch_backward(q, k, v, a, b, conv_w, conv_state_in, state_in, grad_o, grad_state_out,
                                        grad_q, grad_k, grad_v, grad_a, grad_b, grad_conv_w, grad_conv_state_in,
                                        grad_state_in, cu_seqlens, N, T, T_tot, Hqk, Hv, gate_scale, q_scale,
                                        workspace, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_prefill_backward(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                         const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                         const float *state_in, const uint16_t *grad_o, const float *grad_state_out,
                         float *grad_q, float *grad_k, float *grad_v, float *grad_a, float *grad_b,
                         float *grad_conv_w, float *grad_conv_state_in, float *grad_state_in, int B, int T,
                         int Hqk, int Hv, int dk, int dv, float gate_scale, float q_scale, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    if (B < 0 || T < 0) return GDN_ERR_INVALID_ARGUMENT;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if ((long)B * T > 0x7fffffffL) return GDN_ERR_UNSUPPORTED;
    return backward_common(q, k, v, a, b, conv_w, conv_state_in, state_in, grad_o, grad_state_out, grad_q,
                           grad_k, grad_v, grad_a, grad_b, grad_conv_w, grad_conv_state_in, grad_state_in,
                           nullptr, B, T, B * T, Hqk, Hv, gate_scale, q_scale, workspace, workspace_bytes, stream);
}

int gdn_prefill_backward_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                                const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                                const float *state_in, const uint16_t *grad_o, const float *grad_state_out,
                                float *grad_q, float *grad_k, float *grad_v, float *grad_a, float *grad_b,
                                float *grad_conv_w, float *grad_conv_state_in, float *grad_state_in,
                                const int32_t *cu_seqlens, int N, int T_tot, int Hqk, int Hv, int dk, int dv,
                                float gate_scale, float q_scale, void *workspace, size_t workspace_bytes,
                                void *stream)
{
    if (N < 0 || T_tot < 0) return GDN_ERR_INVALID_ARGUMENT;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if (!cu_seqlens) return GDN_ERR_INVALID_ARGUMENT;
    return backward_common(q, k, v, a, b, conv_w, conv_state_in, state_in, grad_o, grad_state_out, grad_q,
                           grad_k, grad_v, grad_a, grad_b, grad_conv_w, grad_conv_state_in, grad_state_in,
                           cu_seqlens, N, 0, T_tot, Hqk, Hv, gate_scale, q_scale, workspace, workspace_bytes,
                           stream);
}

}  // extern "C"
