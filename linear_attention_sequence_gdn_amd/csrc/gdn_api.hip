// gdn_api.hip -- the C ABI (include/gdn.h): argument validation, workspace
// carving and kernel launches on the caller's stream.
//
// Validation runs before any HIP call, so every error path returns with
// nothing launched and no output touched.
#include "../../include/gdn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

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
                           float q_scale, float *state_final, bool forward_only, void *workspace,
                           hipStream_t stream);
hipError_t launch_bwd_accum(float *dst, const float *src, long n, hipStream_t stream);
hipError_t launch_bwd_hist(const uint16_t *q, const uint16_t *k, const uint16_t *v, uint16_t *rows, long tok0,
                           int Hqk, int Hv, hipStream_t stream);
hipError_t launch_bwd_addrows(const float *g, float *gq, float *gk, float *gv, long tok0, int Hqk, int Hv,
                              hipStream_t stream);
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

// Checks of the arguments every prefill entry point shares, apart from the
// workspace (no HIP call).
static int prefill_check(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                         const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                         uint16_t *conv_state_out, const float *state_in, float *state_out, uint16_t *o,
                         const int32_t *cu_seqlens, int T_tot)
{
    if (!state_out || !conv_w) return GDN_ERR_INVALID_ARGUMENT;
    if (T_tot > 0 && (!q || !k || !v || !a || !b || !o)) return GDN_ERR_INVALID_ARGUMENT;
    const void *al16[] = {q, k, v, conv_w, conv_state_in, conv_state_out, state_in, state_out, o};
    for (const void *ptr : al16)
        if (ptr && !aligned(ptr, 16)) return GDN_ERR_INVALID_ARGUMENT;
    if ((a && !aligned(a, 4)) || (b && !aligned(b, 4)) || (cu_seqlens && !aligned(cu_seqlens, 4)))
        return GDN_ERR_INVALID_ARGUMENT;
    return GDN_OK;
}

static int prefill_common(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                          const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                          uint16_t *conv_state_out, const float *state_in, float *state_out,
                          uint16_t *o, const int32_t *cu_seqlens, int N, int T_uniform,
                          int T_tot, int Hqk, int Hv, float gate_scale, float q_scale,
                          void *workspace, size_t workspace_bytes, void *stream,
                          void *const *events = nullptr, const int32_t *slots = nullptr, int n_rows = 0,
                          int seg_chunks_min = 0)
{
    const int rc = prefill_check(q, k, v, a, b, conv_w, conv_state_in, conv_state_out, state_in, state_out, o,
                                 cu_seqlens, T_tot);
    if (rc != GDN_OK) return rc;
    if (workspace && !aligned(workspace, 16)) return GDN_ERR_INVALID_ARGUMENT;
    const int max_chunks = cu_seqlens ? gdn::max_chunks_varlen(N, T_tot)
                                      : gdn::max_chunks_uniform(N, T_uniform);
    const size_t need = gdn::prefill_workspace_bytes(max_chunks, N, Hqk, Hv);
    // A uniform call whose workspace holds less than the whole call runs in
    // windows of Tw tokens (a multiple of the chunk), the largest that fits:
    // each window continues the sequences from the state and rows the
    // previous one left, so the chunk grid and the result (up to rounding)
    // are those of one call.
    int Tw = T_uniform;
    float *ping[2] = {nullptr, nullptr};  // the states handed from window to window
    if (need > 0 && (!workspace || workspace_bytes < need)) {
        if (cu_seqlens || slots || events || seg_chunks_min > 0 || !workspace) return GDN_ERR_WORKSPACE_TOO_SMALL;
        // chunks per window whose workspace fits in `budget`: lo fits, hi does not
        auto window_chunks = [&](size_t budget) {
            int lo = 0, hi = (T_uniform + gdn::kChunk - 1) / gdn::kChunk;
            while (hi - lo > 1) {
                const int mid = (lo + hi) / 2;
                if (gdn::prefill_workspace_bytes(gdn::max_chunks_uniform(N, mid * gdn::kChunk), N, Hqk, Hv) <= budget)
                    lo = mid;
                else
                    hi = mid;
            }
            return lo;
        };
        // preferably with two state buffers at the workspace's end, so that no
        // window updates a state in place (which routes every final state
        // through the sequential pass's in-order walk); else in place in state_out
        const size_t sbytes = (size_t)N * Hv * gdn::kStateFloats * sizeof(float);
        const size_t tail = 2 * ((sbytes + 255) & ~(size_t)255);
        int lo = 0;
        if (workspace_bytes > tail) lo = window_chunks((workspace_bytes - tail) & ~(size_t)255);
        if (lo > 0) {
            uint8_t *base = static_cast<uint8_t *>(workspace) + (((workspace_bytes - tail) & ~(size_t)255));
            ping[0] = reinterpret_cast<float *>(base);
            ping[1] = reinterpret_cast<float *>(base + tail / 2);
        } else {
            lo = window_chunks(workspace_bytes);
        }
        if (lo == 0) return GDN_ERR_WORKSPACE_TOO_SMALL;
        Tw = lo * gdn::kChunk;
    }
    if (N == 0) return GDN_OK;

    for (int t_off = 0; t_off < T_uniform || (t_off == 0 && T_uniform == 0); t_off += Tw) {
        const int len = T_uniform - t_off < Tw ? T_uniform - t_off : Tw;
        const bool first_w = t_off == 0, last_w = t_off + len >= T_uniform;
        const int wchunks = cu_seqlens ? max_chunks : gdn::max_chunks_uniform(N, len);
        gdn::PrefillArgs p{};
        p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.conv_w = conv_w;
        // later windows start from the state the previous one wrote, and read
        // their sequences' earlier rows from the input; only the last writes
        // the carried rows
        p.conv_state_in = first_w ? conv_state_in : nullptr;
        p.conv_state_out = last_w ? conv_state_out : nullptr;
        const int w_idx = t_off / (Tw > 0 ? Tw : 1);
        if (ping[0]) {
            p.state_in = first_w ? state_in : ping[(w_idx - 1) & 1];
            p.state_out = last_w ? state_out : ping[w_idx & 1];
        } else {
            p.state_in = first_w ? state_in : state_out;
            p.state_out = state_out;
        }
        p.o = o;
        p.cu_seqlens = cu_seqlens; p.N = N; p.T_uniform = len; p.T_tot = T_tot;
        p.T_stride = T_uniform; p.t_off = t_off; p.cont = !first_w;
        p.Hqk = Hqk; p.Hv = Hv; p.gate_scale = gate_scale; p.q_scale = q_scale;
        p.max_chunks = wchunks;
        p.seg_chunks = gdn::choose_seg_chunks(wchunks, N, Hv);
        // a caller's longer segments (fewer of them: the workspace still fits)
        if (seg_chunks_min > p.seg_chunks) p.seg_chunks = seg_chunks_min;
        p.max_segs = gdn::max_segments(wchunks, N, p.seg_chunks);
        p.defer_final = p.state_in != nullptr && p.state_in == p.state_out;
        p.defer_conv = p.conv_state_in != nullptr && p.conv_state_in == p.conv_state_out;
        p.slots = slots;
        p.n_rows = n_rows;
        hipError_t e = gdn::launch_prefill(p, workspace, reinterpret_cast<hipStream_t>(stream),
                                           reinterpret_cast<hipEvent_t const *>(events));
        if (e != hipSuccess) return GDN_ERR_HIP;
        if (cu_seqlens || T_uniform == 0) break;
    }
    return GDN_OK;
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

}  // extern "C"

// ---------------------------------------------------------------------------
// gdn_prefill_noalloc: gdn_prefill with its workspace in a file-scope device
// array instead of a caller's buffer, for callers that cannot allocate.  The
// array lives in the library's code object: each GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// must not pass the array's name to a kernel (on the host it names a host-side
// stand-in); the device address is looked up once per device with
// hipGetSymbolAddress and kept in kScratchDevAddr.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)192 << 20;  // the T = 8192, 16 / 48-head prefill needs 166 MiB
constexpr int kScratchMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex kScratchMutex;
void *kScratchDevAddr[kScratchMaxDevices];

// Device address of the current device's scratch array, looked up on the
// first call on that device.
int scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_HIP;
    if (dev < 0 || dev >= kScratchMaxDevices) return GDN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(kScratchMutex);
    if (!kScratchDevAddr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GDN_ERR_HIP;
        kScratchDevAddr[dev] = ptr;
    }
    *out = kScratchDevAddr[dev];
    return GDN_OK;
}

}  // namespace

extern "C" {

size_t gdn_prefill_noalloc_max_workspace(void) { return kScratchBytes; }

int gdn_prefill_noalloc(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                        const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                        uint16_t *conv_state_out, const float *state_in, float *state_out, uint16_t *o,
                        int B, int T, int Hqk, int Hv, int dk, int dv, float gate_scale, float q_scale,
                        void *stream)
{
    if (B < 0 || T < 0) return GDN_ERR_INVALID_ARGUMENT;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if ((long)B * T > 0x7fffffffL) return GDN_ERR_UNSUPPORTED;
    rc = prefill_check(q, k, v, a, b, conv_w, conv_state_in, conv_state_out, state_in, state_out, o, nullptr,
                       B * T);
    if (rc != GDN_OK) return rc;
    // one 64-token window of the batch must fit in the array; longer calls run
    // in windows (prefill_common)
    if (gdn::prefill_workspace_bytes(gdn::max_chunks_uniform(B, T < gdn::kChunk ? T : gdn::kChunk), B, Hqk, Hv) >
        kScratchBytes)
        return GDN_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != GDN_OK) return rc;
    return prefill_common(q, k, v, a, b, conv_w, conv_state_in, conv_state_out, state_in, state_out, o, nullptr,
                          B, T, B * T, Hqk, Hv, gate_scale, q_scale, ws, kScratchBytes, stream);
}

int gdn_prefill_with_options(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                             const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                             uint16_t *conv_state_out, const float *state_in, float *state_out,
                             uint16_t *o, int B, int T, int Hqk, int Hv, int dk, int dv,
                             float gate_scale, float q_scale, void *workspace,
                             size_t workspace_bytes, void *stream, int seg_chunks, void *const *events)
{
    if (events)
        for (int i = 0; i < gdn::kPrefillEvents; ++i)
            if (!events[i]) return GDN_ERR_INVALID_ARGUMENT;
    if (B < 0 || T < 0 || seg_chunks < 0) return GDN_ERR_INVALID_ARGUMENT;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if ((long)B * T > 0x7fffffffL) return GDN_ERR_UNSUPPORTED;
    return prefill_common(q, k, v, a, b, conv_w, conv_state_in, conv_state_out, state_in,
                          state_out, o, nullptr, B, T, B * T, Hqk, Hv, gate_scale, q_scale,
                          workspace, workspace_bytes, stream, events, nullptr, 0, seg_chunks);
}

int gdn_prefill_with_events(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                            const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                            uint16_t *conv_state_out, const float *state_in, float *state_out,
                            uint16_t *o, int B, int T, int Hqk, int Hv, int dk, int dv,
                            float gate_scale, float q_scale, void *workspace,
                            size_t workspace_bytes, void *stream, void *const *events)
{
    if (!events) return GDN_ERR_INVALID_ARGUMENT;
    return gdn_prefill_with_options(q, k, v, a, b, conv_w, conv_state_in, conv_state_out, state_in, state_out, o,
                                    B, T, Hqk, Hv, dk, dv, gate_scale, q_scale, workspace, workspace_bytes, stream,
                                    0, events);
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

int gdn_prefill_varlen_slots(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                             const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                             uint16_t *conv_state_out, const float *state_in, float *state_out, uint16_t *o,
                             const int32_t *cu_seqlens, const int32_t *slots, int n_rows, int N, int T_tot,
                             int Hqk, int Hv, int dk, int dv, float gate_scale, float q_scale, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    if (N < 0 || T_tot < 0) return GDN_ERR_INVALID_ARGUMENT;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if (!cu_seqlens || !slots || n_rows < 0 || !aligned(slots, 4)) return GDN_ERR_INVALID_ARGUMENT;
    return prefill_common(q, k, v, a, b, conv_w, conv_state_in, conv_state_out, state_in, state_out, o,
                          cu_seqlens, N, 0, T_tot, Hqk, Hv, gate_scale, q_scale, workspace, workspace_bytes,
                          stream, nullptr, slots, n_rows);
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

// ---- the backward of a uniform batch in pieces ---------------------------
// A call whose workspace is short of the one-pass size runs sequence by
// sequence, each cut into windows of Tw tokens (a multiple of 64, so the
// chunk grid is the one-pass grid).  A forward sweep (the backward's own fp32
// recomputation) leaves the state entering every window; a reverse sweep then
// runs the whole backward of each window from that state, with the raw rows
// before the window as its conv history, and the state gradient the window
// after it handed back as its grad_state_out.  Each window's gradient of its
// history rows is added into the gradients of those rows once the window
// before has written them, and the conv weight gradients are summed in a
// fixed order.
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static size_t bwd_state_bytes(int Hv) { return (size_t)Hv * gdn::kD * gdn::kD * sizeof(float); }
static size_t bwd_ctot(int Hqk, int Hv) { return (size_t)(2 * Hqk + Hv) * gdn::kD; }

// Workspace of one sequence of T tokens in windows of Tw: one window's
// backward, the states entering windows 1 .. nw-1, two state-gradient
// buffers, a window's history rows, two buffers of their gradient, and one
// conv weight gradient.
static size_t bwd_window_bytes(int T, int Tw, int Hqk, int Hv)
{
    const size_t nw = (size_t)((T + Tw - 1) / Tw), st = bwd_state_bytes(Hv), C_tot = bwd_ctot(Hqk, Hv);
    return align256(gdn::backward_workspace_bytes(1, Tw, false, Hqk, Hv)) + (nw + 1) * st +
           align256(3 * C_tot * sizeof(uint16_t)) + 2 * align256(3 * C_tot * sizeof(float)) +
           align256(4 * C_tot * sizeof(float));
}

// Window length a uniform backward takes with W bytes of workspace: T when
// the whole batch runs at once; else the longest window (fewest windows)
// whose plan fits; 0 when not even 64-token windows fit.
static int bwd_window_tokens(int B, int T, int Hqk, int Hv, size_t W)
{
    if (B == 0 || T == 0 || W >= gdn::backward_workspace_bytes(B, B * T, false, Hqk, Hv)) return T;
    const size_t st = bwd_state_bytes(Hv);
    const int max_nw = (T + gdn::kChunk - 1) / gdn::kChunk;
    for (int nw = 1; nw <= max_nw; ++nw) {
        if ((size_t)(nw + 1) * st > W) break;  // the states alone no longer fit
        const int Tw = nw == 1 ? T : ((T + nw - 1) / nw + gdn::kChunk - 1) / gdn::kChunk * gdn::kChunk;
        if (bwd_window_bytes(T, Tw, Hqk, Hv) <= W) return Tw;
    }
    return 0;
}

static hipError_t backward_windows(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *a,
                                   const float *b, const uint16_t *conv_w, const uint16_t *conv_state_in,
                                   const float *state_in, const uint16_t *grad_o, const float *grad_state_out,
                                   float *grad_q, float *grad_k, float *grad_v, float *grad_a, float *grad_b,
                                   float *grad_conv_w, float *grad_conv_state_in, float *grad_state_in, int B,
                                   int T, int Tw, int Hqk, int Hv, float gate_scale, float q_scale, void *workspace,
                                   hipStream_t st)
{
    const long nq = (long)Hqk * gdn::kD, nv = (long)Hv * gdn::kD, C_tot = (long)bwd_ctot(Hqk, Hv);
    const long sfl = (long)Hv * gdn::kD * gdn::kD;  // floats of one sequence's states
    const int nw = (T + Tw - 1) / Tw;
    uint8_t *base = static_cast<uint8_t *>(workspace);
    size_t off = 0;
    auto carve = [&](size_t bytes) {
        uint8_t *r = base + off;
        off += align256(bytes);
        return r;
    };
    void *wbwd = carve(gdn::backward_workspace_bytes(1, Tw, false, Hqk, Hv));
    float *states = reinterpret_cast<float *>(carve((size_t)(nw - 1) * bwd_state_bytes(Hv)));
    float *ds[2] = {reinterpret_cast<float *>(carve(bwd_state_bytes(Hv))),
                    reinterpret_cast<float *>(carve(bwd_state_bytes(Hv)))};
    uint16_t *hist = reinterpret_cast<uint16_t *>(carve(3 * C_tot * sizeof(uint16_t)));
    float *hg[2] = {reinterpret_cast<float *>(carve(3 * C_tot * sizeof(float))),
                    reinterpret_cast<float *>(carve(3 * C_tot * sizeof(float)))};
    float *dw = reinterpret_cast<float *>(carve(4 * C_tot * sizeof(float)));
    auto slot = [&](int w) { return (nw - 1 - w) & 1; };  // window w's buffer of a ping-pong pair
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t r) { return (e = r) == hipSuccess; };
    bool first_dw = true;
    for (int s = 0; s < B; ++s) {
        const long so = (long)s * T;  // the sequence's first token in the batch
        const float *s_in = state_in ? state_in + s * sfl : nullptr;
        const uint16_t *c_in = conv_state_in ? conv_state_in + s * 3 * C_tot : nullptr;
        const float *gs_out = grad_state_out ? grad_state_out + s * sfl : nullptr;
        float *gs_in = grad_state_in ? grad_state_in + s * sfl : nullptr;
        float *gc_in = grad_conv_state_in ? grad_conv_state_in + s * 3 * C_tot : nullptr;
        // forward sweep: the states entering windows 1 .. nw-1
        for (int w = 0; w + 1 < nw; ++w) {
            const long t0 = so + (long)w * Tw;
            if (w > 0 && !ok(gdn::launch_bwd_hist(q, k, v, hist, t0 - 3, Hqk, Hv, st))) return e;
            if (!ok(gdn::launch_backward(q + t0 * nq, k + t0 * nq, v + t0 * nv, a + t0 * Hv, b + t0 * Hv, conv_w,
                                         w == 0 ? c_in : hist, w == 0 ? s_in : states + (w - 1) * sfl,
                                         grad_o + t0 * nv, nullptr, grad_q + t0 * nq, grad_k + t0 * nq,
                                         grad_v + t0 * nv, grad_a + t0 * Hv, grad_b + t0 * Hv, grad_conv_w, nullptr,
                                         nullptr, nullptr, 1, Tw, Tw, Hqk, Hv, gate_scale, q_scale,
                                         states + w * sfl, true, wbwd, st)))
                return e;
        }
        // reverse sweep
        for (int w = nw - 1; w >= 0; --w) {
            const long t0 = so + (long)w * Tw;
            const int Lw = (int)std::min<long>(Tw, T - (long)w * Tw);
            if (w > 0 && !ok(gdn::launch_bwd_hist(q, k, v, hist, t0 - 3, Hqk, Hv, st))) return e;
            float *dwo = first_dw ? grad_conv_w : dw;
            if (!ok(gdn::launch_backward(q + t0 * nq, k + t0 * nq, v + t0 * nv, a + t0 * Hv, b + t0 * Hv, conv_w,
                                         w == 0 ? c_in : hist, w == 0 ? s_in : states + (w - 1) * sfl,
                                         grad_o + t0 * nv, w == nw - 1 ? gs_out : ds[slot(w + 1)],
                                         grad_q + t0 * nq, grad_k + t0 * nq, grad_v + t0 * nv, grad_a + t0 * Hv,
                                         grad_b + t0 * Hv, dwo, w == 0 ? gc_in : hg[slot(w)],
                                         w == 0 ? gs_in : ds[slot(w)], nullptr, 1, Lw, Lw, Hqk, Hv, gate_scale,
                                         q_scale, nullptr, false, wbwd, st)))
                return e;
            if (!first_dw && !ok(gdn::launch_bwd_accum(grad_conv_w, dw, 4 * C_tot, st))) return e;
            first_dw = false;
            // the window after this one reached into its last three rows
            if (w + 1 < nw && !ok(gdn::launch_bwd_addrows(hg[slot(w + 1)], grad_q, grad_k, grad_v,
                                                          so + (long)(w + 1) * Tw - 3, Hqk, Hv, st)))
                return e;
        }
    }
    return e;
}

int gdn_prefill_backward_windows(int B, int T, int Hqk, int Hv, int dk, int dv, size_t workspace_bytes,
                                 int *window_tokens)
{
    if (B < 0 || T < 0 || !window_tokens) return GDN_ERR_INVALID_ARGUMENT;
    int rc = check_dims(Hqk, Hv, dk, dv);
    if (rc != GDN_OK) return rc;
    if ((long)B * T > 0x7fffffffL) return GDN_ERR_UNSUPPORTED;
    const int Tw = bwd_window_tokens(B, T, Hqk, Hv, workspace_bytes);
    if (Tw == 0 && (long)B * T > 0) return GDN_ERR_WORKSPACE_TOO_SMALL;
    *window_tokens = Tw;
    return GDN_OK;
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
    if (need > 0 && (!workspace || workspace_bytes < need)) {
        // a uniform batch runs sequence by sequence, in windows of whole chunks
        const int Tw = cu_seqlens || !workspace ? 0 : bwd_window_tokens(N, T, Hqk, Hv, workspace_bytes);
        if (Tw == 0) return GDN_ERR_WORKSPACE_TOO_SMALL;
        hipError_t e = backward_windows(q, k, v, a, b, conv_w, conv_state_in, state_in, grad_o, grad_state_out,
                                        grad_q, grad_k, grad_v, grad_a, grad_b, grad_conv_w, grad_conv_state_in,
                                        grad_state_in, N, T, Tw, Hqk, Hv, gate_scale, q_scale, workspace,
                                        reinterpret_cast<hipStream_t>(stream));
        return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
    }
    if (N == 0) return GDN_OK;
    hipError_t e = gdn::launch_backward(q, k, v, a, b, conv_w, conv_state_in, state_in, grad_o, grad_state_out,
                                        grad_q, grad_k, grad_v, grad_a, grad_b, grad_conv_w, grad_conv_state_in,
                                        grad_state_in, cu_seqlens, N, T, T_tot, Hqk, Hv, gate_scale, q_scale,
                                        nullptr, false, workspace, reinterpret_cast<hipStream_t>(stream));
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
