// gdn_abi.hip -- the C ABI of include/gdn.h: argument checks, then launches.
//
// Every check runs on the host before the first HIP call, so a rejected call
// enqueues nothing and needs no device.
#include <stdint.h>
#include <mutex>
#include <string.h>

#include "gdn.h"
#include "gdn_internal.h"
#include <stdio.h>

namespace gdn {
namespace {

constexpr int kD = 128;

__global__ void fill_zero_kernel(uint4 *p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Shape checks shared by every entry point.  T is checked only when `use_T`.
int check_shape(const gdn_shape *s, bool use_T) {
    if (!s) return GDN_EINVAL;
    if (s->B < 1 || s->Hk < 1 || s->Hv < 1 || (use_T && s->T < 1)) return GDN_EINVAL;
    if (s->Hv % s->Hk != 0) return GDN_EINVAL;
    if (s->Dk != kD || s->Dv != kD) return GDN_EUNSUPPORTED;
    if (s->conv_width != 0 && s->conv_width != 4) return GDN_EUNSUPPORTED;
    if (s->flags & ~(GDN_NO_NORM | GDN_PACKED)) return GDN_EINVAL;
    if (!(s->eps_l2 >= 0.0f) || !(s->eps_norm >= 0.0f)) return GDN_EINVAL;
    if (s->prefill_segments < 0 || ((s->flags & GDN_PACKED) && s->prefill_segments > 1)) return GDN_EINVAL;
    // sizes must fit the kernels' 32-bit token and head indices
    if ((long long)s->B * s->Hv * kD > 0x7fffffffLL || (use_T && (long long)s->T * kD > 0x7fffffffLL))
        return GDN_EINVAL;
    return GDN_OK;
}

size_t conv_channels(const gdn_shape *s) { return (size_t)2 * s->Hk * kD + (size_t)s->Hv * kD; }

} // namespace
} // namespace gdn

using namespace gdn;

extern "C" {

const char *gdn_status_string(int status) {
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument (null or misaligned pointer, bad size, or overlapping buffers)";
    case GDN_EUNSUPPORTED: return "unsupported shape (head width must be 128, conv width 0 or 4)";
    case GDN_EHIP: return "a HIP call or kernel launch failed";
    case GDN_EWORKSPACE: return "workspace too small";
    case GDN_ETIMEOUT: return "a bounded wait between workgroups timed out: the prefill outputs are wrong";
    case GDN_ESKIPPED: return "a packed sequence with invalid bounds was skipped";
    default: return "unknown status";
    }
}

int gdn_state_init(const gdn_shape *shape, float *state, uint16_t *conv_state, void *stream) {
    int rc = check_shape(shape, false);
    if (rc) return rc;
    if (!state || !aligned(state, 16) || (conv_state && !aligned(conv_state, 16))) return GDN_EINVAL;
    if (conv_state && shape->conv_width == 0) return GDN_EINVAL;
    const size_t n_state = (size_t)shape->B * shape->Hv * kD * kD;
    const size_t n_conv = conv_state ? (size_t)shape->B * 3 * conv_channels(shape) : 0;
    return launch_state_init(state, n_state, conv_state, n_conv, static_cast<hipStream_t>(stream)) ? GDN_EHIP
                                                                                                   : GDN_OK;
}

int gdn_prefill_workspace_size(const gdn_shape *shape, size_t *bytes) {
    int rc = check_shape(shape, true);
    if (rc) return rc;
    if (!bytes) return GDN_EINVAL;
    PrefillPlan plan;
    plan_prefill(shape->B, shape->T, shape->Hk, shape->Hv, (shape->flags & GDN_PACKED) != 0, shape->prefill_segments,
                 &plan);
    if (plan.nslots * shape->Hk > 0x7fffffffLL) return GDN_EINVAL;
    *bytes = plan.total_bytes;
    return GDN_OK;
}

int gdn_prefill_check(const void *workspace, size_t workspace_bytes, void *stream) {
    if (!workspace || workspace_bytes < kHeaderBytes || !aligned(workspace, 16)) return GDN_EINVAL;
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail("hipStreamSynchronize", e), GDN_EHIP;
    unsigned int word = 0;
    e = hipMemcpy(&word, static_cast<const unsigned char *>(workspace) + kErrOffset, sizeof word, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail("hipMemcpy(error word)", e), GDN_EHIP;
    if (word & 1u) return GDN_ETIMEOUT;
    if (word & 2u) return GDN_ESKIPPED;
    return GDN_OK;
}

} // extern "C"

namespace {

// ---------------------------------------------------------------- static scratch
// The workspace of gdn_prefill_no_workspace: a file-scope device array of
// kStaticScratchBytes that every GPU the library runs on holds until the process ends.
// In host code `scratch` is only a stand-in for the symbol; the array's address on a
// device comes from hipGetSymbolAddress, looked up once per device with that device
// current, and that address is what the kernels get.  Every call on a GPU shares the
// array; the prep kernel clears the part that must start at zero on every call.
constexpr size_t kStaticScratchBytes = GDN_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices] = {};

// The current device's address of `scratch`, or nullptr (with the reason recorded) when
// it cannot be had.
void *static_scratch_address() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail("hipGetDevice", e), nullptr;
    if (dev < 0 || dev >= kMaxDevices) return fail("gdn_prefill_no_workspace: device index out of range"), nullptr;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail("hipGetSymbolAddress(scratch)", e), nullptr;
        if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255)) return fail("hipGetSymbolAddress(scratch): unaligned"), nullptr;
        g_scratch_addr[dev] = ptr;
    }
    return g_scratch_addr[dev];
}

// g, beta are the gate logits a, b when A_log and dt_bias are given (both or neither);
// cu_seqlens is given exactly when the shape carries GDN_PACKED.
int prefill_impl(const gdn_shape *s, const int32_t *cu_seqlens, const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                 const float *beta, const float *A_log, const float *dt_bias, const uint16_t *z,
                 const uint16_t *conv_w, const uint16_t *norm_w, const float *state_in,
                 const uint16_t *conv_state_in, uint16_t *o, float *state_out, uint16_t *conv_state_out,
                 void *workspace, size_t workspace_bytes, void *stream, bool static_scratch = false) {
    int rc = check_shape(s, true);
    if (rc) return rc;
    const bool packed = (s->flags & GDN_PACKED) != 0;
    // The static scratch is the library's own array: it is neither null nor misaligned nor
    // shared with any caller buffer, and its address is only looked up once every host check
    // has passed.  Here it stands in as a placeholder for those checks.
    alignas(256) static const unsigned char placeholder[256] = {};
    if (static_scratch) workspace = const_cast<unsigned char *>(placeholder), workspace_bytes = kStaticScratchBytes;
    if (packed != (cu_seqlens != nullptr)) return GDN_EINVAL;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return GDN_EINVAL;
    if ((A_log == nullptr) != (dt_bias == nullptr)) return GDN_EINVAL;
    if (A_log && (!aligned(A_log, 4) || !aligned(dt_bias, 4))) return GDN_EINVAL;
    const bool norm = !(s->flags & GDN_NO_NORM);
    const bool conv = s->conv_width == 4;
    if (!q || !k || !v || !g || !beta || !o || !state_out || !workspace) return GDN_EINVAL;
    if (norm && (!z || !norm_w)) return GDN_EINVAL;
    if (conv != (conv_w != nullptr)) return GDN_EINVAL;
    if (!conv && (conv_state_in || conv_state_out)) return GDN_EINVAL;
    const void *a16[] = {q, k, v, z, conv_w, norm_w, state_in, conv_state_in, o, state_out, conv_state_out, workspace};
    for (const void *p : a16)
        if (p && !aligned(p, 16)) return GDN_EINVAL;
    if (!aligned(g, 4) || !aligned(beta, 4)) return GDN_EINVAL;

    const size_t B = s->B, Hk = s->Hk, Hv = s->Hv, Cc = conv_channels(s);
    const size_t rows = packed ? (size_t)s->T : B * s->T;  // token rows of q, k, v, z, g, beta and o
    const size_t nqk = rows * Hk * kD * 2, nv = rows * Hv * kD * 2, ngb = rows * Hv * 4;
    const size_t nst = B * Hv * kD * kD * 4, ncs = B * 3 * Cc * 2;
    const size_t nw = conv ? Cc * 4 * 2 : 0, nn = norm ? kD * 2 : 0;
    const struct {
        const void *p;
        size_t n;
    } inputs[] = {{q, nqk}, {k, nqk}, {v, nv}, {g, ngb}, {beta, ngb}, {norm ? z : nullptr, nv},
                  {conv_w, nw}, {norm_w, nn}, {state_in, nst}, {conv_state_in, ncs},
                  {A_log, Hv * 4}, {dt_bias, Hv * 4}, {cu_seqlens, (B + 1) * 4}};
    const size_t wsb = static_scratch ? 0 : workspace_bytes;  // overlap() ignores empty ranges
    for (const auto &in : inputs)
        if (overlap(o, nv, in.p, in.n) || overlap(workspace, wsb, in.p, in.n)) return GDN_EINVAL;
    if (overlap(conv_state_out, ncs, conv_state_in, ncs)) return GDN_EINVAL;
    // state_out may be state_in exactly, but must not partly overlap anything else
    if (state_out != state_in && overlap(state_out, nst, state_in, nst)) return GDN_EINVAL;
    for (const auto &in : inputs)
        if (in.p != state_in && overlap(state_out, nst, in.p, in.n)) return GDN_EINVAL;
    if (overlap(o, nv, state_out, nst) || overlap(o, nv, conv_state_out, ncs) ||
        overlap(workspace, wsb, o, nv) || overlap(workspace, wsb, state_out, nst) ||
        overlap(workspace, wsb, conv_state_out, ncs) || overlap(state_out, nst, conv_state_out, ncs))
        return GDN_EINVAL;

    PrefillPlan plan;
    plan_prefill(s->B, s->T, s->Hk, s->Hv, packed, s->prefill_segments, &plan);
    // the static scratch: where the library's own choice of the two-level scan does not fit,
    // the plain sequential pass (the smaller workspace) may
    if (static_scratch && s->prefill_segments == 0 && plan.nseg > 1 && plan.total_bytes > kStaticScratchBytes)
        plan_prefill(s->B, s->T, s->Hk, s->Hv, packed, 1, &plan);
    if (plan.nslots * s->Hk > 0x7fffffffLL) return GDN_EINVAL;
    if (workspace_bytes < plan.total_bytes) return GDN_EWORKSPACE;
    if (static_scratch && !(workspace = static_scratch_address())) return GDN_EHIP;

    PrefillParams p;
    p.q = q; p.k = k; p.v = v; p.z = norm ? z : nullptr; p.conv_w = conv_w; p.norm_w = norm ? norm_w : nullptr;
    p.conv_state_in = conv_state_in; p.g = g; p.beta = beta; p.A_log = A_log; p.dt_bias = dt_bias;
    p.state_in = state_in;
    p.o = o; p.conv_state_out = conv_state_out; p.state_out = state_out; p.workspace = workspace;
    p.cu_seqlens = cu_seqlens;
    p.B = s->B; p.T = s->T; p.Hk = s->Hk; p.Hv = s->Hv; p.conv_width = s->conv_width; p.norm = norm;
    p.eps_l2 = s->eps_l2; p.eps_norm = s->eps_norm;
    return launch_prefill(p, plan, static_cast<hipStream_t>(stream)) ? GDN_EHIP : GDN_OK;
}

// T tokens per sequence (1 for gdn_decode_step); the snapshots are used only when T > 1.
int decode_impl(const gdn_shape *s, int T, const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                const float *beta, const float *A_log, const float *dt_bias, const uint16_t *z,
                const uint16_t *conv_w, const uint16_t *norm_w, float *state, uint16_t *conv_state, uint16_t *o,
                float *state_snaps, uint16_t *conv_snaps, void *stream) {
    int rc = check_shape(s, false);
    if (rc) return rc;
    if (T < 1 || T > kMaxDecodeTokens) return GDN_EINVAL;
    if (T == 1) state_snaps = nullptr, conv_snaps = nullptr;
    if (s->flags & GDN_PACKED) return GDN_EINVAL;  // one token per sequence: nothing to pack
    if ((A_log == nullptr) != (dt_bias == nullptr)) return GDN_EINVAL;
    if (A_log && (!aligned(A_log, 4) || !aligned(dt_bias, 4))) return GDN_EINVAL;
    const bool norm = !(s->flags & GDN_NO_NORM);
    const bool conv = s->conv_width == 4;
    if (!q || !k || !v || !g || !beta || !o || !state) return GDN_EINVAL;
    if (norm && (!z || !norm_w)) return GDN_EINVAL;
    if (conv != (conv_w != nullptr) || conv != (conv_state != nullptr)) return GDN_EINVAL;
    if (!conv && conv_snaps) return GDN_EINVAL;
    const void *a16[] = {q, k, v, z, conv_w, norm_w, state, conv_state, o, state_snaps, conv_snaps};
    for (const void *p : a16)
        if (p && !aligned(p, 16)) return GDN_EINVAL;
    if (!aligned(g, 4) || !aligned(beta, 4)) return GDN_EINVAL;
    if (s->Hv / s->Hk > 64) return GDN_EUNSUPPORTED;  // the r value heads' conv outputs must fit one workgroup's LDS
    if (decode_lds_bytes(T, s->Hv / s->Hk) > 160 * 1024) return GDN_EUNSUPPORTED;

    const size_t B = s->B, Hk = s->Hk, Hv = s->Hv, Cc = conv_channels(s);
    const size_t nqk = B * T * Hk * kD * 2, nv = B * T * Hv * kD * 2, ngb = B * T * Hv * 4;
    const size_t nst = B * Hv * kD * kD * 4, ncs = B * 3 * Cc * 2;
    const size_t nw = conv ? Cc * 4 * 2 : 0, nn = norm ? kD * 2 : 0;
    const size_t nss = (T - 1) * nst, ncss = (T - 1) * ncs;
    const struct {
        const void *p;
        size_t n;
    } ro[] = {{q, nqk}, {k, nqk}, {v, nv}, {g, ngb}, {beta, ngb}, {norm ? z : nullptr, nv},
              {conv_w, nw}, {norm_w, nn}, {A_log, Hv * 4}, {dt_bias, Hv * 4}};
    const struct {
        const void *p;
        size_t n;
    } rw[] = {{o, nv}, {state, nst}, {conv_state, ncs}, {state_snaps, nss}, {conv_snaps, ncss}};
    for (const auto &out : rw)
        for (const auto &in : ro)
            if (overlap(out.p, out.n, in.p, in.n)) return GDN_EINVAL;
    for (size_t i = 0; i < 5; ++i)
        for (size_t j = i + 1; j < 5; ++j)
            if (overlap(rw[i].p, rw[i].n, rw[j].p, rw[j].n)) return GDN_EINVAL;

    DecodeParams p;
    p.q = q; p.k = k; p.v = v; p.z = norm ? z : nullptr; p.conv_w = conv_w; p.norm_w = norm ? norm_w : nullptr;
    p.g = g; p.beta = beta; p.A_log = A_log; p.dt_bias = dt_bias;
    p.state = state; p.conv_state = conv_state; p.o = o; p.state_snaps = state_snaps; p.conv_snaps = conv_snaps;
    p.B = s->B; p.T = T; p.Hk = s->Hk; p.Hv = s->Hv; p.conv_width = s->conv_width; p.norm = norm;
    p.eps_l2 = s->eps_l2; p.eps_norm = s->eps_norm;
    return launch_decode(p, static_cast<hipStream_t>(stream)) ? GDN_EHIP : GDN_OK;
}

} // namespace

extern "C" {

int gdn_prefill(const gdn_shape *s, const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                const float *beta, const uint16_t *z, const uint16_t *conv_w, const uint16_t *norm_w,
                const float *state_in, const uint16_t *conv_state_in, uint16_t *o, float *state_out,
                uint16_t *conv_state_out, void *workspace, size_t workspace_bytes, void *stream) {
    return prefill_impl(s, nullptr, q, k, v, g, beta, nullptr, nullptr, z, conv_w, norm_w, state_in, conv_state_in,
                        o, state_out, conv_state_out, workspace, workspace_bytes, stream);
}

int gdn_prefill_no_workspace(const gdn_shape *s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const float *g, const float *beta, const uint16_t *z, const uint16_t *conv_w,
                             const uint16_t *norm_w, const float *state_in, const uint16_t *conv_state_in,
                             uint16_t *o, float *state_out, uint16_t *conv_state_out, void *stream) {
    return prefill_impl(s, nullptr, q, k, v, g, beta, nullptr, nullptr, z, conv_w, norm_w, state_in, conv_state_in,
                        o, state_out, conv_state_out, nullptr, 0, stream, true);
}

int gdn_prefill_gate_logits(const gdn_shape *s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                            const float *a, const float *b, const float *A_log, const float *dt_bias,
                            const uint16_t *z, const uint16_t *conv_w, const uint16_t *norm_w,
                            const float *state_in, const uint16_t *conv_state_in, uint16_t *o, float *state_out,
                            uint16_t *conv_state_out, void *workspace, size_t workspace_bytes, void *stream) {
    if (!A_log || !dt_bias) return GDN_EINVAL;
    return prefill_impl(s, nullptr, q, k, v, a, b, A_log, dt_bias, z, conv_w, norm_w, state_in, conv_state_in, o,
                        state_out, conv_state_out, workspace, workspace_bytes, stream);
}

int gdn_prefill_packed(const gdn_shape *s, const int32_t *cu_seqlens, const uint16_t *q, const uint16_t *k,
                       const uint16_t *v, const float *g, const float *beta, const uint16_t *z,
                       const uint16_t *conv_w, const uint16_t *norm_w, const float *state_in,
                       const uint16_t *conv_state_in, uint16_t *o, float *state_out, uint16_t *conv_state_out,
                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!cu_seqlens) return GDN_EINVAL;
    return prefill_impl(s, cu_seqlens, q, k, v, g, beta, nullptr, nullptr, z, conv_w, norm_w, state_in,
                        conv_state_in, o, state_out, conv_state_out, workspace, workspace_bytes, stream);
}

int gdn_prefill_packed_gate_logits(const gdn_shape *s, const int32_t *cu_seqlens, const uint16_t *q,
                                   const uint16_t *k, const uint16_t *v, const float *a, const float *b,
                                   const float *A_log, const float *dt_bias, const uint16_t *z,
                                   const uint16_t *conv_w, const uint16_t *norm_w, const float *state_in,
                                   const uint16_t *conv_state_in, uint16_t *o, float *state_out,
                                   uint16_t *conv_state_out, void *workspace, size_t workspace_bytes,
                                   void *stream) {
    if (!cu_seqlens || !A_log || !dt_bias) return GDN_EINVAL;
    return prefill_impl(s, cu_seqlens, q, k, v, a, b, A_log, dt_bias, z, conv_w, norm_w, state_in, conv_state_in,
                        o, state_out, conv_state_out, workspace, workspace_bytes, stream);
}

int gdn_decode_step(const gdn_shape *s, const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                    const float *beta, const uint16_t *z, const uint16_t *conv_w, const uint16_t *norm_w,
                    float *state, uint16_t *conv_state, uint16_t *o, void *stream) {
    return decode_impl(s, 1, q, k, v, g, beta, nullptr, nullptr, z, conv_w, norm_w, state, conv_state, o, nullptr,
                       nullptr, stream);
}

int gdn_decode_step_gate_logits(const gdn_shape *s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *a, const float *b, const float *A_log, const float *dt_bias,
                                const uint16_t *z, const uint16_t *conv_w, const uint16_t *norm_w, float *state,
                                uint16_t *conv_state, uint16_t *o, void *stream) {
    if (!A_log || !dt_bias) return GDN_EINVAL;
    return decode_impl(s, 1, q, k, v, a, b, A_log, dt_bias, z, conv_w, norm_w, state, conv_state, o, nullptr, nullptr,
                       stream);
}

int gdn_decode_multi(const gdn_shape *s, const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                     const float *beta, const uint16_t *z, const uint16_t *conv_w, const uint16_t *norm_w,
                     float *state, uint16_t *conv_state, uint16_t *o, float *state_snaps, uint16_t *conv_snaps,
                     void *stream) {
    if (!s) return GDN_EINVAL;
    return decode_impl(s, s->T, q, k, v, g, beta, nullptr, nullptr, z, conv_w, norm_w, state, conv_state, o,
                       state_snaps, conv_snaps, stream);
}

int gdn_decode_multi_gate_logits(const gdn_shape *s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 const float *a, const float *b, const float *A_log, const float *dt_bias,
                                 const uint16_t *z, const uint16_t *conv_w, const uint16_t *norm_w, float *state,
                                 uint16_t *conv_state, uint16_t *o, float *state_snaps, uint16_t *conv_snaps,
                                 void *stream) {
    if (!s || !A_log || !dt_bias) return GDN_EINVAL;
    return decode_impl(s, s->T, q, k, v, a, b, A_log, dt_bias, z, conv_w, norm_w, state, conv_state, o, state_snaps,
                       conv_snaps, stream);
}

} // extern "C"

namespace gdn {

namespace {
thread_local char g_last_error[256] = "";
}

int fail(const char *what, hipError_t e) {
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return -1;
}

int fail(const char *what) {
    snprintf(g_last_error, sizeof g_last_error, "%s", what);
    return -1;
}

int launch_state_init(float *state, size_t n_state, uint16_t *conv_state, size_t n_conv, hipStream_t stream) {
    uint4 *ps = reinterpret_cast<uint4 *>(state);
    size_t n16s = n_state * sizeof(float) / 16;
    void *args_s[] = {&ps, &n16s};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fill_zero_kernel), dim3(1024), dim3(256), args_s, 0,
                                   stream);
    if (e != hipSuccess) return fail("hipLaunchKernel(fill_zero_kernel, state)", e);
    if (conv_state && n_conv) {
        uint4 *pc = reinterpret_cast<uint4 *>(conv_state);
        size_t n16c = n_conv * sizeof(uint16_t) / 16;
        void *args_c[] = {&pc, &n16c};
        e = hipLaunchKernel(reinterpret_cast<const void *>(fill_zero_kernel), dim3(256), dim3(256), args_c, 0, stream);
        if (e != hipSuccess) return fail("hipLaunchKernel(fill_zero_kernel, conv state)", e);
    }
    return 0;
}
} // namespace gdn

extern "C" const char *gdn_last_error(void) { return gdn::g_last_error; }
