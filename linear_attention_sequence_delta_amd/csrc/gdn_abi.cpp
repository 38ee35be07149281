// gdn_abi.cpp -- the extern "C" entry points declared in include/gdn.h:
// host-side argument validation, error reporting and kernel dispatch.
// No HIP call is made before every host-side check has passed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_last_error[0] = '\0';
    return GDN_OK;
}

// GDN_DEBUG=1: device-side precondition checks and a synchronisation after
// every call.  Read at every call, so a process can switch it on and off.
bool debug_env() {
    const char *e = std::getenv("GDN_DEBUG");
    return e && e[0] && std::strcmp(e, "0") != 0;
}

bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

// The checks synchronise the stream, which a stream under graph capture must
// not do: on a capturing stream debug mode checks nothing.
bool debug_mode(hipStream_t s) { return debug_env() && !capturing(s); }

int hip_fail(hipError_t e, const char *what) {
    return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Report a launch error, and in debug mode wait for the stream and report
// asynchronous faults too.
int finish(hipError_t e, hipStream_t s, const char *what) {
    if (e != hipSuccess) return hip_fail(e, what);
    if (debug_mode(s)) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, what);
    }
    return ok();
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
    return pa < pb + nb && pb < pa + na;
}

int check_heads(int H_qk, int H_v, int d_k, int d_v) {
    if (H_qk < 1 || H_v < 1) return fail(GDN_ERR_INVALID_ARG, "head counts must be >= 1 (H_qk=%d, H_v=%d)", H_qk, H_v);
    if (H_v % H_qk != 0) return fail(GDN_ERR_INVALID_ARG, "H_v (%d) must be a multiple of H_qk (%d)", H_v, H_qk);
    if (d_k != gdn::kD || d_v != gdn::kD)
        return fail(GDN_ERR_UNSUPPORTED, "only d_k = d_v = 128 is built (got d_k=%d, d_v=%d)", d_k, d_v);
    if ((long long)H_v * gdn::kD > (1LL << 24) || (long long)H_qk * gdn::kD > (1LL << 24))
        return fail(GDN_ERR_INVALID_ARG, "head count too large");
    return GDN_OK;
}

int check_seqs(const int32_t *cu_seqlens, int N, int T) {
    if (T < 0) return fail(GDN_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
    if (N < 1) return fail(GDN_ERR_INVALID_ARG, "N must be >= 1 (got %d)", N);
    if (!cu_seqlens && N != 1)
        return fail(GDN_ERR_INVALID_ARG, "cu_seqlens is NULL but N = %d (must be 1)", N);
    return GDN_OK;
}

int device_check_cu(const int32_t *cu_seqlens, int N, int T, hipStream_t s) {
    if (!debug_mode(s) || !cu_seqlens) return GDN_OK;
    int bad = 0;
    hipError_t e = gdn::debug_check_cu_seqlens(cu_seqlens, N, T, s, &bad);
    if (e != hipSuccess) return hip_fail(e, "cu_seqlens check");
    if (bad) return fail(GDN_ERR_DEVICE_CHECK, "cu_seqlens is not non-decreasing from 0 to T=%d", T);
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_last_error(void) { return g_last_error; }

int gdn_conv_prelude(const void *x_raw, const void *conv_w, const int32_t *cu_seqlens, int N,
                     int T, int H_qk, int H_v, int d_k, int d_v, float l2_eps, void *q, void *k,
                     void *v, void *stream) {
    int rc;
    if ((rc = check_heads(H_qk, H_v, d_k, d_v))) return rc;
    if ((rc = check_seqs(cu_seqlens, N, T))) return rc;
    if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps))
        return fail(GDN_ERR_INVALID_ARG, "l2_eps must be finite and >= 0");
    if (T == 0) return ok();
    if (!x_raw || !conv_w || !q || !k || !v)
        return fail(GDN_ERR_INVALID_ARG, "x_raw, conv_w, q, k and v must be non-NULL");
    const size_t craw = (size_t)(2 * H_qk + H_v) * gdn::kD;
    const size_t nx = (size_t)T * craw * 2, nq = (size_t)T * H_qk * gdn::kD * 2,
                 nv = (size_t)T * H_v * gdn::kD * 2;
    if (overlaps(q, nq, x_raw, nx) || overlaps(k, nq, x_raw, nx) || overlaps(v, nv, x_raw, nx) ||
        overlaps(q, nq, k, nq) || overlaps(q, nq, v, nv) || overlaps(k, nq, v, nv))
        return fail(GDN_ERR_INVALID_ARG, "prelude outputs must not overlap each other or x_raw");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = device_check_cu(cu_seqlens, N, T, s))) return rc;
    hipError_t e = gdn::launch_conv_prelude(x_raw, conv_w, cu_seqlens, N, T, H_qk, H_v, l2_eps,
                                            q, k, v, s);
    return finish(e, s, "gdn_conv_prelude launch");
}

size_t gdn_prefill_workspace_size(int io_dtype, int N, int T, int H_qk, int H_v, int d_k,
                                  int d_v) {
    (void)d_k;
    (void)d_v;
    if (io_dtype != GDN_BF16 || N < 1 || T < 1 || H_qk < 1 || H_v < 1) return 0;
    return gdn::chunked_workspace_bytes(N, T, H_qk, H_v, false);
}

}  // extern "C"

namespace {

// gdn_prefill, with chunk_states (bf16 only) gdn_prefill_save_states, and with
// no_alloc gdn_prefill_no_alloc (the workspace in the library's fixed scratch).
int prefill_impl(int io_dtype, const void *q, const void *k, const void *v, const float *g,
                 const float *beta, const float *initial_state, float *final_state,
                 const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k, int d_v,
                 float scale, void *o, void *chunk_states, size_t cs_bytes, void *workspace,
                 size_t ws_bytes, void *stream, bool no_alloc = false) {
    int rc;
    if (io_dtype != GDN_F32 && io_dtype != GDN_BF16)
        return fail(GDN_ERR_UNSUPPORTED, "io_dtype must be GDN_F32 or GDN_BF16 (got %d)", io_dtype);
    if ((rc = check_heads(H_qk, H_v, d_k, d_v))) return rc;
    if ((rc = check_seqs(cu_seqlens, N, T))) return rc;
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    if (io_dtype == GDN_BF16 && H_v / H_qk > gdn::kMaxPrepGroup)
        return fail(GDN_ERR_UNSUPPORTED, "bf16 prefill supports at most %d V-heads per QK head (got %d)",
                    gdn::kMaxPrepGroup, H_v / H_qk);
    const size_t esz = io_dtype == GDN_F32 ? 4 : 2;
    const size_t nqk = (size_t)T * H_qk * gdn::kD * esz, nv = (size_t)T * H_v * gdn::kD * esz;
    const size_t ng = (size_t)T * H_v * 4, ns = (size_t)N * H_v * gdn::kD * gdn::kD * 4;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o))
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta and o must be non-NULL");
    if (overlaps(o, nv, q, nqk) || overlaps(o, nv, k, nqk) || overlaps(o, nv, v, nv) ||
        overlaps(o, nv, g, ng) || overlaps(o, nv, beta, ng) || overlaps(o, nv, initial_state, ns) ||
        overlaps(o, nv, final_state, ns))
        return fail(GDN_ERR_INVALID_ARG, "o must not overlap any input or state");
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, ns, initial_state, ns))
        return fail(GDN_ERR_INVALID_ARG, "final_state must equal initial_state or not overlap it");
    if (final_state && (overlaps(final_state, ns, q, nqk) || overlaps(final_state, ns, k, nqk) ||
                        overlaps(final_state, ns, v, nv) || overlaps(final_state, ns, g, ng) ||
                        overlaps(final_state, ns, beta, ng)))
        return fail(GDN_ERR_INVALID_ARG, "final_state must not overlap q, k, v, g or beta");
    const size_t need = gdn_prefill_workspace_size(io_dtype, N, T, H_qk, H_v, d_k, d_v);
    if (no_alloc && need > gdn::chunked_scratch_bytes())
        return fail(GDN_ERR_WORKSPACE, "the prefill needs %zu bytes of scratch, the library holds %zu",
                    need, gdn::chunked_scratch_bytes());
    if (!no_alloc && (ws_bytes < need || (need > 0 && !workspace)))
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    if (need > 0 && (overlaps(workspace, need, o, nv) || overlaps(workspace, need, q, nqk) ||
                     overlaps(workspace, need, k, nqk) || overlaps(workspace, need, v, nv) ||
                     overlaps(workspace, need, final_state, ns) ||
                     overlaps(workspace, need, initial_state, ns)))
        return fail(GDN_ERR_INVALID_ARG, "workspace must not overlap inputs or outputs");
    if (chunk_states) {
        const size_t ncs = gdn_chunk_states_size(N, T, H_v, d_k, d_v);
        if (cs_bytes < ncs)
            return fail(GDN_ERR_INVALID_ARG, "chunk_states of %zu bytes given, %zu needed", cs_bytes, ncs);
        const struct { const void *p; size_t n; } other[] = {
            {q, nqk}, {k, nqk}, {v, nv}, {g, ng}, {beta, ng}, {initial_state, ns}, {final_state, ns},
            {o, nv}, {workspace, need}, {cu_seqlens, (size_t)(N + 1) * 4}};
        for (const auto &x : other)
            if (overlaps(chunk_states, ncs, x.p, x.n))
                return fail(GDN_ERR_INVALID_ARG, "chunk_states must not overlap any other argument");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = device_check_cu(cu_seqlens, N, T, s))) return rc;
    hipError_t e;
    if (io_dtype == GDN_F32 || T == 0)   // T = 0: only the final state (no workspace)
        e = gdn::launch_recurrent_prefill(io_dtype == GDN_F32 ? gdn::kIoF32 : gdn::kIoBF16, q, k,
                                          v, g, beta, initial_state, final_state, cu_seqlens, N,
                                          T, H_qk, H_v, scale, o, s);
    else if (no_alloc)
        e = gdn::launch_chunked_prefill_no_alloc(q, k, v, g, beta, initial_state, final_state,
                                                 cu_seqlens, N, T, H_qk, H_v, scale, o, s);
    else
        e = gdn::launch_chunked_prefill(q, k, v, g, beta, initial_state, final_state, cu_seqlens,
                                        N, T, H_qk, H_v, scale, o, chunk_states, workspace, s);
    return finish(e, s, no_alloc ? "gdn_prefill_no_alloc launch" : "gdn_prefill launch");
}

}  // namespace

extern "C" {

int gdn_prefill(int io_dtype, const void *q, const void *k, const void *v, const float *g,
                const float *beta, const float *initial_state, float *final_state,
                const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k, int d_v,
                float scale, void *o, void *workspace, size_t ws_bytes, void *stream) {
    return prefill_impl(io_dtype, q, k, v, g, beta, initial_state, final_state, cu_seqlens, N, T,
                        H_qk, H_v, d_k, d_v, scale, o, nullptr, 0, workspace, ws_bytes, stream);
}

int gdn_prefill_no_alloc(int io_dtype, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *initial_state,
                         float *final_state, const int32_t *cu_seqlens, int N, int T, int H_qk,
                         int H_v, int d_k, int d_v, float scale, void *o, void *stream) {
    return prefill_impl(io_dtype, q, k, v, g, beta, initial_state, final_state, cu_seqlens, N, T,
                        H_qk, H_v, d_k, d_v, scale, o, nullptr, 0, nullptr, 0, stream, true);
}

size_t gdn_chunk_states_size(int N, int T, int H_v, int d_k, int d_v) {
    if (N < 1 || T < 0 || H_v < 1 || d_k != gdn::kD || d_v != gdn::kD) return 0;
    return gdn::chunk_states_bytes(N, T, H_v);
}

int gdn_prefill_save_states(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state, float *final_state,
                            const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k,
                            int d_v, float scale, void *o, void *chunk_states, size_t cs_bytes,
                            void *workspace, size_t ws_bytes, void *stream) {
    if (!chunk_states) return fail(GDN_ERR_INVALID_ARG, "chunk_states must be non-NULL");
    return prefill_impl(GDN_BF16, q, k, v, g, beta, initial_state, final_state, cu_seqlens, N, T,
                        H_qk, H_v, d_k, d_v, scale, o, chunk_states, cs_bytes, workspace, ws_bytes,
                        stream);
}


size_t gdn_prefill_raw_workspace_size(int N, int T, int H_qk, int H_v, int d_k, int d_v) {
    (void)d_k;
    (void)d_v;
    if (N < 1 || T < 1 || H_qk < 1 || H_v < 1) return 0;
    return gdn::chunked_workspace_bytes(N, T, H_qk, H_v, true);
}

}  // extern "C"

namespace {

// Host-side checks of a prefill from raw projections (nothing is enqueued).
int check_prefill_raw(const void *x_raw, const void *conv_w, float l2_eps, const float *g,
                      const float *beta, const float *initial_state, const float *final_state,
                      const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k, int d_v,
                      float scale, const void *o, const void *workspace, size_t ws_bytes,
                      bool gated = false) {
    int rc;
    if ((rc = check_heads(H_qk, H_v, d_k, d_v))) return rc;
    if ((rc = check_seqs(cu_seqlens, N, T))) return rc;
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps))
        return fail(GDN_ERR_INVALID_ARG, "l2_eps must be finite and >= 0");
    if (H_v / H_qk > gdn::kMaxPrepGroup)
        return fail(GDN_ERR_UNSUPPORTED, "bf16 prefill supports at most %d V-heads per QK head (got %d)",
                    gdn::kMaxPrepGroup, H_v / H_qk);
    const size_t craw = (size_t)(2 * H_qk + H_v) * gdn::kD;
    const size_t nx = (size_t)T * craw * 2, nw = craw * 4 * 2, nv = (size_t)T * H_v * gdn::kD * 2;
    const size_t ng = (size_t)T * H_v * 4, ns = (size_t)N * H_v * gdn::kD * gdn::kD * 4;
    if (T > 0 && (!x_raw || !conv_w || !g || !beta || !o))
        return fail(GDN_ERR_INVALID_ARG, "x_raw, conv_w, g, beta and o must be non-NULL");
    if (overlaps(o, nv, x_raw, nx) || overlaps(o, nv, conv_w, nw) || overlaps(o, nv, g, ng) ||
        overlaps(o, nv, beta, ng) || overlaps(o, nv, initial_state, ns) ||
        overlaps(o, nv, final_state, ns))
        return fail(GDN_ERR_INVALID_ARG, "o must not overlap any input or state");
    if (final_state && initial_state && final_state != initial_state &&
        overlaps(final_state, ns, initial_state, ns))
        return fail(GDN_ERR_INVALID_ARG, "final_state must equal initial_state or not overlap it");
    if (final_state && (overlaps(final_state, ns, x_raw, nx) || overlaps(final_state, ns, conv_w, nw) ||
                        overlaps(final_state, ns, g, ng) || overlaps(final_state, ns, beta, ng)))
        return fail(GDN_ERR_INVALID_ARG, "final_state must not overlap x_raw, conv_w, g or beta");
    const size_t need = !gated ? gdn_prefill_raw_workspace_size(N, T, H_qk, H_v, d_k, d_v)
                        : T > 0    ? gdn::chunked_gated_workspace_bytes(N, T, H_qk, H_v)
                                   : 0;
    if (ws_bytes < need || (need > 0 && !workspace))
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    if (need > 0 && (overlaps(workspace, need, o, nv) || overlaps(workspace, need, x_raw, nx) ||
                     overlaps(workspace, need, conv_w, nw) || overlaps(workspace, need, g, ng) ||
                     overlaps(workspace, need, beta, ng) ||
                     overlaps(workspace, need, final_state, ns) ||
                     overlaps(workspace, need, initial_state, ns)))
        return fail(GDN_ERR_INVALID_ARG, "workspace must not overlap inputs or outputs");
    return GDN_OK;
}

}  // namespace

namespace {
// Backward of the layer: the workspace holds g, b, dg, dbeta, q, k, dq, dk,
// v, dv, the dw partial sums and the gate-sum partials (each 256-byte
// aligned), then the chunked backward's workspace.
struct LayerBwdWs {
    size_t g, q, v, part, gpart, total;
};
LayerBwdWs layer_bwd_ws(int N, int T, int H_qk, int H_v, bool saved) {
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    LayerBwdWs w;
    w.g = al((size_t)T * H_v * 4);
    w.q = al((size_t)T * H_qk * gdn::kD * 2);
    w.v = al((size_t)T * H_v * gdn::kD * 2);
    w.part = al(gdn::prelude_bwd_partial_bytes(T, H_qk, H_v));
    w.gpart = al(gdn::gates_bwd_partial_bytes(H_v));
    w.total = 4 * w.g + 4 * w.q + 2 * w.v + w.part + w.gpart +
              gdn::chunked_backward_workspace_bytes(N, T, H_qk, H_v, saved);
    return w;
}
}  // namespace

extern "C" {

}  // extern "C"

namespace {

// gdn_prefill_raw, and with chunk_states gdn_prefill_raw_save_states.
int prefill_raw_impl(const void *x_raw, const void *conv_w, float l2_eps, const float *g,
                     const float *beta, const float *initial_state, float *final_state,
                     const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k, int d_v,
                     float scale, void *o, void *chunk_states, size_t cs_bytes, void *workspace,
                     size_t ws_bytes, void *stream) {
    int rc = check_prefill_raw(x_raw, conv_w, l2_eps, g, beta, initial_state, final_state,
                               cu_seqlens, N, T, H_qk, H_v, d_k, d_v, scale, o, workspace, ws_bytes);
    if (rc) return rc;
    if (chunk_states) {
        const size_t craw = (size_t)(2 * H_qk + H_v) * gdn::kD;
        const size_t nx = (size_t)T * craw * 2, nw = craw * 4 * 2, nv = (size_t)T * H_v * gdn::kD * 2;
        const size_t ng = (size_t)T * H_v * 4, ns = (size_t)N * H_v * gdn::kD * gdn::kD * 4;
        const size_t need = gdn_prefill_raw_workspace_size(N, T, H_qk, H_v, d_k, d_v);
        const size_t ncs = gdn_chunk_states_size(N, T, H_v, d_k, d_v);
        if (cs_bytes < ncs)
            return fail(GDN_ERR_INVALID_ARG, "chunk_states of %zu bytes given, %zu needed", cs_bytes, ncs);
        const struct { const void *p; size_t n; } other[] = {
            {x_raw, nx}, {conv_w, nw}, {g, ng}, {beta, ng}, {initial_state, ns}, {final_state, ns},
            {o, nv}, {workspace, need}, {cu_seqlens, (size_t)(N + 1) * 4}};
        for (const auto &x : other)
            if (overlaps(chunk_states, ncs, x.p, x.n))
                return fail(GDN_ERR_INVALID_ARG, "chunk_states must not overlap any other argument");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = device_check_cu(cu_seqlens, N, T, s))) return rc;
    hipError_t e;
    if (T == 0)   // only the final state (no workspace; nothing else is read)
        e = gdn::launch_recurrent_prefill(gdn::kIoBF16, nullptr, nullptr, nullptr, g, beta,
                                          initial_state, final_state, cu_seqlens, N, T, H_qk, H_v,
                                          scale, o, s);
    else
        e = gdn::launch_chunked_prefill_raw(x_raw, conv_w, l2_eps, g, beta, initial_state,
                                            final_state, cu_seqlens, N, T, H_qk, H_v, scale, o,
                                            chunk_states, workspace, s);
    return finish(e, s, "gdn_prefill_raw launch");
}

}  // namespace

extern "C" {

int gdn_prefill_raw(const void *x_raw, const void *conv_w, float l2_eps, const float *g,
                    const float *beta, const float *initial_state, float *final_state,
                    const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k, int d_v,
                    float scale, void *o, void *workspace, size_t ws_bytes, void *stream) {
    return prefill_raw_impl(x_raw, conv_w, l2_eps, g, beta, initial_state, final_state, cu_seqlens,
                            N, T, H_qk, H_v, d_k, d_v, scale, o, nullptr, 0, workspace, ws_bytes,
                            stream);
}

int gdn_prefill_raw_save_states(const void *x_raw, const void *conv_w, float l2_eps,
                                const float *g, const float *beta, const float *initial_state,
                                float *final_state, const int32_t *cu_seqlens, int N, int T,
                                int H_qk, int H_v, int d_k, int d_v, float scale, void *o,
                                void *chunk_states, size_t cs_bytes, void *workspace,
                                size_t ws_bytes, void *stream) {
    if (!chunk_states) return fail(GDN_ERR_INVALID_ARG, "chunk_states must be non-NULL");
    return prefill_raw_impl(x_raw, conv_w, l2_eps, g, beta, initial_state, final_state, cu_seqlens,
                            N, T, H_qk, H_v, d_k, d_v, scale, o, chunk_states, cs_bytes, workspace,
                            ws_bytes, stream);
}

size_t gdn_prefill_backward_workspace_size(int N, int T, int H_qk, int H_v, int d_k, int d_v) {
    (void)d_k;
    (void)d_v;
    if (N < 1 || T < 0 || H_qk < 1 || H_v < 1) return 0;
    return gdn::chunked_backward_workspace_bytes(N, T, H_qk, H_v, false);
}

size_t gdn_prefill_backward_saved_workspace_size(int N, int T, int H_qk, int H_v, int d_k,
                                                 int d_v) {
    (void)d_k;
    (void)d_v;
    if (N < 1 || T < 0 || H_qk < 1 || H_v < 1) return 0;
    return gdn::chunked_backward_workspace_bytes(N, T, H_qk, H_v, true);
}

}  // extern "C"

namespace {

// gdn_prefill_backward (the states recomputed: chunk_states NULL, initial_state
// read) and gdn_prefill_backward_saved (the states of an earlier forward pass).
int backward_impl(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  const float *initial_state, const void *chunk_states, size_t cs_bytes,
                  const int32_t *cu_seqlens, const void *d_o, const float *d_final_state, int N,
                  int T, int H_qk, int H_v, int d_k, int d_v, float scale, void *dq, void *dk,
                  void *dv, float *dg, float *dbeta, float *d_initial_state, void *workspace,
                  size_t ws_bytes, void *stream) {
    int rc;
    if ((rc = check_heads(H_qk, H_v, d_k, d_v))) return rc;
    if ((rc = check_seqs(cu_seqlens, N, T))) return rc;
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    if (H_v / H_qk > gdn::kMaxPrepGroup)
        return fail(GDN_ERR_UNSUPPORTED, "bf16 prefill supports at most %d V-heads per QK head (got %d)",
                    gdn::kMaxPrepGroup, H_v / H_qk);
    if (T > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
        return fail(GDN_ERR_INVALID_ARG,
                    "q, k, v, g, beta, d_o, dq, dk, dv, dg and dbeta must be non-NULL");
    const size_t nqk = (size_t)T * H_qk * gdn::kD * 2, nv = (size_t)T * H_v * gdn::kD * 2;
    const size_t ng = (size_t)T * H_v * 4, ns = (size_t)N * H_v * gdn::kD * gdn::kD * 4;
    const bool saved = chunk_states != nullptr;
    const size_t ncs = saved ? gdn_chunk_states_size(N, T, H_v, d_k, d_v) : 0;
    if (saved && cs_bytes < ncs)
        return fail(GDN_ERR_INVALID_ARG, "chunk_states of %zu bytes given, %zu needed", cs_bytes, ncs);
    const size_t need = saved ? gdn_prefill_backward_saved_workspace_size(N, T, H_qk, H_v, d_k, d_v)
                              : gdn_prefill_backward_workspace_size(N, T, H_qk, H_v, d_k, d_v);
    if (ws_bytes < need || !workspace)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    const struct { const void *p; size_t n; } in[] = {
        {q, nqk}, {k, nqk}, {v, nv}, {g, ng}, {beta, ng}, {initial_state, ns}, {d_o, nv},
        {d_final_state, ns}, {cu_seqlens, (size_t)(N + 1) * 4}, {chunk_states, ncs}};
    const struct { const void *p; size_t n; } out[] = {
        {dq, nqk}, {dk, nqk}, {dv, nv}, {dg, ng}, {dbeta, ng}, {d_initial_state, ns},
        {workspace, need}};
    for (const auto &o : out) {
        for (const auto &i : in)
            if (overlaps(o.p, o.n, i.p, i.n))
                return fail(GDN_ERR_INVALID_ARG, "gradients and workspace must not overlap any input");
        for (const auto &o2 : out)
            if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n))
                return fail(GDN_ERR_INVALID_ARG, "gradients and workspace must not overlap each other");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = device_check_cu(cu_seqlens, N, T, s))) return rc;
    hipError_t e = gdn::launch_chunked_backward(q, k, v, g, beta, saved ? nullptr : initial_state,
                                                cu_seqlens, N, T, H_qk, H_v, scale, d_o,
                                                d_final_state, dq, dk, dv, dg, dbeta,
                                                d_initial_state, chunk_states, workspace, s);
    return finish(e, s, "gdn_prefill_backward launch");
}

}  // namespace

extern "C" {

int gdn_prefill_backward(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                         const void *d_o, const float *d_final_state, int N, int T, int H_qk,
                         int H_v, int d_k, int d_v, float scale, void *dq, void *dk, void *dv,
                         float *dg, float *dbeta, float *d_initial_state, void *workspace,
                         size_t ws_bytes, void *stream) {
    return backward_impl(q, k, v, g, beta, initial_state, nullptr, 0, cu_seqlens, d_o,
                         d_final_state, N, T, H_qk, H_v, d_k, d_v, scale, dq, dk, dv, dg, dbeta,
                         d_initial_state, workspace, ws_bytes, stream);
}

int gdn_prefill_backward_saved(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const void *chunk_states, size_t cs_bytes,
                               const int32_t *cu_seqlens, const void *d_o,
                               const float *d_final_state, int N, int T, int H_qk, int H_v,
                               int d_k, int d_v, float scale, void *dq, void *dk, void *dv,
                               float *dg, float *dbeta, float *d_initial_state, void *workspace,
                               size_t ws_bytes, void *stream) {
    if (!chunk_states) return fail(GDN_ERR_INVALID_ARG, "chunk_states must be non-NULL");
    return backward_impl(q, k, v, g, beta, nullptr, chunk_states, cs_bytes, cu_seqlens, d_o,
                         d_final_state, N, T, H_qk, H_v, d_k, d_v, scale, dq, dk, dv, dg, dbeta,
                         d_initial_state, workspace, ws_bytes, stream);
}

size_t gdn_layer_prefill_backward_workspace_size(int N, int T, int H_qk, int H_v, int d_k,
                                                 int d_v) {
    (void)d_k;
    (void)d_v;
    if (N < 1 || T < 0 || H_qk < 1 || H_v < 1) return 0;
    return layer_bwd_ws(N, T, H_qk, H_v, false).total;
}

}  // extern "C"

namespace {

// gdn_layer_prefill_backward, and with chunk_states gdn_layer_prefill_backward_saved.
int layer_backward_impl(const void *x_raw, const void *conv_w, const float *a, const float *b,
                        const float *A_log, const float *dt_bias, float l2_eps,
                        const float *initial_state, const void *chunk_states, size_t cs_bytes,
                        const int32_t *cu_seqlens, const void *d_o, const float *d_final_state,
                        int N, int T, int H_qk, int H_v, int d_k, int d_v, float scale,
                        void *dx_raw, float *dconv_w, float *da, float *db, float *dA_log,
                        float *ddt_bias, float *d_initial_state, void *workspace, size_t ws_bytes,
                        void *stream) {
    int rc;
    if ((rc = check_heads(H_qk, H_v, d_k, d_v))) return rc;
    if ((rc = check_seqs(cu_seqlens, N, T))) return rc;
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps))
        return fail(GDN_ERR_INVALID_ARG, "l2_eps must be finite and >= 0");
    if (H_v / H_qk > gdn::kMaxPrepGroup)
        return fail(GDN_ERR_UNSUPPORTED, "bf16 prefill supports at most %d V-heads per QK head (got %d)",
                    gdn::kMaxPrepGroup, H_v / H_qk);
    if (!conv_w || !A_log || !dt_bias || !dconv_w || !dA_log || !ddt_bias)
        return fail(GDN_ERR_INVALID_ARG,
                    "conv_w, A_log, dt_bias, dconv_w, dA_log and ddt_bias must be non-NULL");
    if (T > 0 && (!x_raw || !a || !b || !d_o || !dx_raw || !da || !db))
        return fail(GDN_ERR_INVALID_ARG, "x_raw, a, b, d_o, dx_raw, da and db must be non-NULL");
    const bool saved = chunk_states != nullptr;
    const size_t ncs = saved ? gdn_chunk_states_size(N, T, H_v, d_k, d_v) : 0;
    if (saved && cs_bytes < ncs)
        return fail(GDN_ERR_INVALID_ARG, "chunk_states of %zu bytes given, %zu needed", cs_bytes, ncs);
    const LayerBwdWs L = layer_bwd_ws(N, T, H_qk, H_v, saved);
    if (ws_bytes < L.total || !workspace)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, L.total);
    const size_t craw = (size_t)(2 * H_qk + H_v) * gdn::kD;
    const size_t nx = (size_t)T * craw * 2, nw = craw * 4 * 2, nwf = craw * 4 * 4;
    const size_t ng = (size_t)T * H_v * 4, nh = (size_t)H_v * 4, nv = (size_t)T * H_v * gdn::kD * 2;
    const size_t ns = (size_t)N * H_v * gdn::kD * gdn::kD * 4;
    const struct { const void *p; size_t n; } in[] = {
        {x_raw, nx}, {conv_w, nw}, {a, ng}, {b, ng}, {A_log, nh}, {dt_bias, nh},
        {initial_state, ns}, {d_o, nv}, {d_final_state, ns}, {cu_seqlens, (size_t)(N + 1) * 4},
        {chunk_states, ncs}};
    const struct { const void *p; size_t n; } out[] = {
        {dx_raw, nx}, {dconv_w, nwf}, {da, ng}, {db, ng}, {dA_log, nh}, {ddt_bias, nh},
        {d_initial_state, ns}, {workspace, L.total}};
    for (const auto &o : out) {
        for (const auto &i : in)
            if (overlaps(o.p, o.n, i.p, i.n))
                return fail(GDN_ERR_INVALID_ARG, "gradients and workspace must not overlap any input");
        for (const auto &o2 : out)
            if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n))
                return fail(GDN_ERR_INVALID_ARG, "gradients and workspace must not overlap each other");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = device_check_cu(cu_seqlens, N, T, s))) return rc;
    char *p = static_cast<char *>(workspace);
    float *g = reinterpret_cast<float *>(p), *beta = reinterpret_cast<float *>(p + L.g);
    float *dg = reinterpret_cast<float *>(p + 2 * L.g), *dbeta = reinterpret_cast<float *>(p + 3 * L.g);
    p += 4 * L.g;
    void *q = p, *k = p + L.q, *dq = p + 2 * L.q, *dk = p + 3 * L.q;
    p += 4 * L.q;
    void *v = p, *dv = p + L.v;
    p += 2 * L.v;
    float *part = reinterpret_cast<float *>(p);
    float *gpart = reinterpret_cast<float *>(p + L.part);
    void *rest = p + L.part + L.gpart;
    hipError_t e = hipSuccess;
    if (T > 0) {
        if ((e = gdn::launch_gates(a, b, A_log, dt_bias, T, H_v, g, beta, s)) == hipSuccess)
            e = gdn::launch_conv_prelude(x_raw, conv_w, cu_seqlens, N, T, H_qk, H_v, l2_eps, q, k, v, s);
    }
    if (e == hipSuccess)
        e = gdn::launch_chunked_backward(q, k, v, g, beta, saved ? nullptr : initial_state,
                                         cu_seqlens, N, T, H_qk, H_v, scale, d_o, d_final_state,
                                         dq, dk, dv, dg, dbeta, d_initial_state, chunk_states,
                                         rest, s);
    if (e == hipSuccess)
        e = gdn::launch_prelude_bwd(x_raw, conv_w, cu_seqlens, N, T, H_qk, H_v, l2_eps, dq, dk, dv,
                                    dx_raw, dconv_w, part, s);
    if (e == hipSuccess)
        e = gdn::launch_gates_bwd(a, b, A_log, dt_bias, dg, dbeta, T, H_v, da, db, dA_log, ddt_bias,
                                  gpart, s);
    return finish(e, s, "gdn_layer_prefill_backward launch");
}

}  // namespace

extern "C" {

int gdn_layer_prefill_backward(const void *x_raw, const void *conv_w, const float *a,
                               const float *b, const float *A_log, const float *dt_bias,
                               float l2_eps, const float *initial_state,
                               const int32_t *cu_seqlens, const void *d_o,
                               const float *d_final_state, int N, int T, int H_qk, int H_v,
                               int d_k, int d_v, float scale, void *dx_raw, float *dconv_w,
                               float *da, float *db, float *dA_log, float *ddt_bias,
                               float *d_initial_state, void *workspace, size_t ws_bytes,
                               void *stream) {
    return layer_backward_impl(x_raw, conv_w, a, b, A_log, dt_bias, l2_eps, initial_state, nullptr,
                               0, cu_seqlens, d_o, d_final_state, N, T, H_qk, H_v, d_k, d_v, scale,
                               dx_raw, dconv_w, da, db, dA_log, ddt_bias, d_initial_state,
                               workspace, ws_bytes, stream);
}

size_t gdn_layer_prefill_backward_saved_workspace_size(int N, int T, int H_qk, int H_v, int d_k,
                                                       int d_v) {
    (void)d_k;
    (void)d_v;
    if (N < 1 || T < 0 || H_qk < 1 || H_v < 1) return 0;
    return layer_bwd_ws(N, T, H_qk, H_v, true).total;
}

int gdn_layer_prefill_backward_saved(const void *x_raw, const void *conv_w, const float *a,
                                     const float *b, const float *A_log, const float *dt_bias,
                                     float l2_eps, const void *chunk_states, size_t cs_bytes,
                                     const int32_t *cu_seqlens, const void *d_o,
                                     const float *d_final_state, int N, int T, int H_qk, int H_v,
                                     int d_k, int d_v, float scale, void *dx_raw, float *dconv_w,
                                     float *da, float *db, float *dA_log, float *ddt_bias,
                                     float *d_initial_state, void *workspace, size_t ws_bytes,
                                     void *stream) {
    if (!chunk_states) return fail(GDN_ERR_INVALID_ARG, "chunk_states must be non-NULL");
    return layer_backward_impl(x_raw, conv_w, a, b, A_log, dt_bias, l2_eps, nullptr, chunk_states,
                               cs_bytes, cu_seqlens, d_o, d_final_state, N, T, H_qk, H_v, d_k,
                               d_v, scale, dx_raw, dconv_w, da, db, dA_log, ddt_bias,
                               d_initial_state, workspace, ws_bytes, stream);
}

int gdn_gates(const float *a, const float *b, const float *A_log, const float *dt_bias, int T,
              int H_v, float *g, float *beta, void *stream) {
    if (T < 0 || H_v < 1) return fail(GDN_ERR_INVALID_ARG, "T must be >= 0 and H_v >= 1");
    if (T == 0) return ok();
    if (!a || !b || !A_log || !dt_bias || !g || !beta)
        return fail(GDN_ERR_INVALID_ARG, "a, b, A_log, dt_bias, g and beta must be non-NULL");
    const size_t n = (size_t)T * H_v * 4, nh = (size_t)H_v * 4;
    if (overlaps(g, n, beta, n) || overlaps(g, n, a, n) || overlaps(g, n, b, n) ||
        overlaps(beta, n, a, n) || overlaps(beta, n, b, n) || overlaps(g, n, A_log, nh) ||
        overlaps(g, n, dt_bias, nh) || overlaps(beta, n, A_log, nh) || overlaps(beta, n, dt_bias, nh))
        return fail(GDN_ERR_INVALID_ARG, "g and beta must not overlap each other or the inputs");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_gates(a, b, A_log, dt_bias, T, H_v, g, beta, s), s, "gdn_gates launch");
}

size_t gdn_layer_prefill_workspace_size(int N, int T, int H_qk, int H_v, int d_k, int d_v) {
    if (N < 1 || T < 1 || H_qk < 1 || H_v < 1) return 0;
    const size_t gate = ((size_t)T * H_v * 4 + 255) & ~size_t(255);
    return 2 * gate + gdn_prefill_raw_workspace_size(N, T, H_qk, H_v, d_k, d_v);
}

size_t gdn_layer_prefill_gated_workspace_size(int N, int T, int H_qk, int H_v, int d_k, int d_v) {
    (void)d_k;
    (void)d_v;
    if (N < 1 || T < 1 || H_qk < 1 || H_v < 1) return 0;
    const size_t gate = ((size_t)T * H_v * 4 + 255) & ~size_t(255);
    return 2 * gate + gdn::chunked_gated_workspace_bytes(N, T, H_qk, H_v);
}

}  // extern "C"

namespace {

// gdn_layer_prefill, and with chunk_states gdn_layer_prefill_save_states.
struct GateArgs {        // gdn_layer_prefill_gated's output gate
    const void *z;
    const float *norm_w;
    float norm_eps;
    void *y;
};

int layer_prefill_impl(const void *x_raw, const void *conv_w, const float *a, const float *b,
                       const float *A_log, const float *dt_bias, float l2_eps,
                       const float *initial_state, float *final_state, const void *conv_state_in,
                       void *conv_state_out,
                       const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k,
                       int d_v, float scale, void *o, void *chunk_states, size_t cs_bytes,
                       void *workspace, size_t ws_bytes, void *stream,
                       const GateArgs *gt = nullptr) {
    int rc;
    if ((rc = check_heads(H_qk, H_v, d_k, d_v))) return rc;
    if ((rc = check_seqs(cu_seqlens, N, T))) return rc;
    const size_t need = gt ? gdn_layer_prefill_gated_workspace_size(N, T, H_qk, H_v, d_k, d_v)
                             : gdn_layer_prefill_workspace_size(N, T, H_qk, H_v, d_k, d_v);
    if (ws_bytes < need || (need > 0 && !workspace))
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    if (T > 0 && (!a || !b || !A_log || !dt_bias))
        return fail(GDN_ERR_INVALID_ARG, "a, b, A_log and dt_bias must be non-NULL");
    const size_t craw = (size_t)(2 * H_qk + H_v) * gdn::kD;
    const size_t ng = (size_t)T * H_v * 4, nh = (size_t)H_v * 4, nc = (size_t)N * 3 * craw * 2;
    const size_t nx = (size_t)T * craw * 2, nv = (size_t)T * H_v * gdn::kD * 2;
    const size_t ns = (size_t)N * H_v * gdn::kD * gdn::kD * 4;
    if (need > 0 && (overlaps(workspace, need, a, ng) || overlaps(workspace, need, b, ng) ||
                     overlaps(workspace, need, A_log, nh) || overlaps(workspace, need, dt_bias, nh) ||
                     overlaps(workspace, need, conv_state_out, nc)))
        return fail(GDN_ERR_INVALID_ARG, "workspace must not overlap inputs or outputs");
    if (conv_state_out &&
        (overlaps(conv_state_out, nc, x_raw, nx) || overlaps(conv_state_out, nc, o, nv) ||
         overlaps(conv_state_out, nc, final_state, ns) || overlaps(conv_state_out, nc, initial_state, ns) ||
         overlaps(conv_state_out, nc, a, ng) || overlaps(conv_state_out, nc, b, ng)))
        return fail(GDN_ERR_INVALID_ARG, "conv_state_out must not overlap inputs or outputs");
    if (overlaps(o, nv, a, ng) || overlaps(o, nv, b, ng) ||
        (final_state && (overlaps(final_state, ns, a, ng) || overlaps(final_state, ns, b, ng))))
        return fail(GDN_ERR_INVALID_ARG, "o and final_state must not overlap a or b");
    if (conv_state_in) {
        // read through the whole call; conv_state_out may be the same buffer
        // (it is written last), but not a shifted view of it
        if (conv_state_out && conv_state_out != conv_state_in && overlaps(conv_state_out, nc, conv_state_in, nc))
            return fail(GDN_ERR_INVALID_ARG, "conv_state_in must be conv_state_out or not overlap it");
        if (overlaps(conv_state_in, nc, o, nv) || overlaps(conv_state_in, nc, final_state, ns) ||
            (need > 0 && overlaps(conv_state_in, nc, workspace, need)) ||
            (gt && overlaps(conv_state_in, nc, gt->y, nv)) ||
            (chunk_states && overlaps(conv_state_in, nc, chunk_states, cs_bytes)))
            return fail(GDN_ERR_INVALID_ARG, "conv_state_in must not overlap any output or the workspace");
    }
    // the gates go to the front of the workspace, the prefill's workspace follows
    const size_t gate = need > 0 ? ((size_t)T * H_v * 4 + 255) & ~size_t(255) : 0;
    float *g = need > 0 ? static_cast<float *>(workspace) : nullptr;
    float *beta = need > 0 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + gate) : nullptr;
    void *rest = need > 0 ? static_cast<char *>(workspace) + 2 * gate : nullptr;
    const size_t rest_bytes = need > 0 ? ws_bytes - 2 * gate : 0;
    rc = check_prefill_raw(x_raw, conv_w, l2_eps, T > 0 ? g : nullptr, T > 0 ? beta : nullptr,
                           initial_state, final_state, cu_seqlens, N, T, H_qk, H_v, d_k, d_v,
                           scale, o, rest, rest_bytes, gt != nullptr);
    if (rc) return rc;
    if (gt) {
        if (!(gt->norm_eps >= 0.f) || !std::isfinite(gt->norm_eps))
            return fail(GDN_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");
        if (T > 0 && (!gt->z || !gt->norm_w || !gt->y))
            return fail(GDN_ERR_INVALID_ARG, "z, norm_w and y must be non-NULL");
        const size_t nw = (size_t)gdn::kD * 4;
        const struct { const void *p; size_t n; } other[] = {
            {x_raw, nx}, {conv_w, craw * 4 * 2}, {a, ng}, {b, ng}, {A_log, nh}, {dt_bias, nh},
            {initial_state, ns}, {final_state, ns}, {conv_state_out, nc}, {o, nv}, {gt->z, nv},
            {gt->norm_w, nw}, {workspace, need}, {cu_seqlens, (size_t)(N + 1) * 4}};
        for (const auto &x : other)
            if (overlaps(gt->y, nv, x.p, x.n))
                return fail(GDN_ERR_INVALID_ARG, "y must not overlap any other argument");
        if (overlaps(o, nv, gt->z, nv) || overlaps(o, nv, gt->norm_w, nw) ||
            overlaps(workspace, need, gt->z, nv) || overlaps(workspace, need, gt->norm_w, nw))
            return fail(GDN_ERR_INVALID_ARG, "o and workspace must not overlap z or norm_w");
    }
    if (chunk_states) {
        const size_t ncs = gdn_chunk_states_size(N, T, H_v, d_k, d_v);
        if (cs_bytes < ncs)
            return fail(GDN_ERR_INVALID_ARG, "chunk_states of %zu bytes given, %zu needed", cs_bytes, ncs);
        const struct { const void *p; size_t n; } other[] = {
            {x_raw, nx}, {conv_w, craw * 4 * 2}, {a, ng}, {b, ng}, {A_log, nh}, {dt_bias, nh},
            {initial_state, ns}, {final_state, ns}, {conv_state_out, nc}, {o, nv},
            {workspace, need}, {cu_seqlens, (size_t)(N + 1) * 4}};
        for (const auto &x : other)
            if (overlaps(chunk_states, ncs, x.p, x.n))
                return fail(GDN_ERR_INVALID_ARG, "chunk_states must not overlap any other argument");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if ((rc = device_check_cu(cu_seqlens, N, T, s))) return rc;
    hipError_t e = hipSuccess;
    if (T == 0)
        e = gdn::launch_recurrent_prefill(gdn::kIoBF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                                          initial_state, final_state, cu_seqlens, N, T, H_qk, H_v,
                                          scale, o, s);
    else if ((e = gdn::launch_gates(a, b, A_log, dt_bias, T, H_v, g, beta, s)) == hipSuccess)
        e = gt ? gdn::launch_chunked_prefill_raw_gated(x_raw, conv_w, l2_eps, g, beta, initial_state,
                                                         final_state, cu_seqlens, N, T, H_qk, H_v,
                                                         scale, o, gt->z, gt->norm_w,
                                                         gt->norm_eps, gt->y, rest, s, conv_state_in)
                 : gdn::launch_chunked_prefill_raw(x_raw, conv_w, l2_eps, g, beta, initial_state,
                                                   final_state, cu_seqlens, N, T, H_qk, H_v, scale,
                                                   o, chunk_states, rest, s, conv_state_in);
    if (e == hipSuccess && conv_state_out)
        e = gdn::launch_conv_hist(x_raw, cu_seqlens, N, T, (int)craw, conv_state_in, conv_state_out, s);
    return finish(e, s, "gdn_layer_prefill launch");
}

}  // namespace

extern "C" {

int gdn_layer_prefill(const void *x_raw, const void *conv_w, const float *a, const float *b,
                      const float *A_log, const float *dt_bias, float l2_eps,
                      const float *initial_state, float *final_state, const void *conv_state_in,
                      void *conv_state_out, const int32_t *cu_seqlens, int N, int T, int H_qk,
                      int H_v, int d_k, int d_v, float scale, void *o, void *workspace,
                      size_t ws_bytes, void *stream) {
    return layer_prefill_impl(x_raw, conv_w, a, b, A_log, dt_bias, l2_eps, initial_state,
                              final_state, conv_state_in, conv_state_out, cu_seqlens, N, T, H_qk,
                              H_v, d_k, d_v,
                              scale, o, nullptr, 0, workspace, ws_bytes, stream);
}

int gdn_layer_prefill_gated(const void *x_raw, const void *conv_w, const float *a, const float *b,
                            const float *A_log, const float *dt_bias, float l2_eps, const void *z,
                            const float *norm_w, float norm_eps, const float *initial_state,
                            float *final_state, const void *conv_state_in, void *conv_state_out,
                            const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k,
                            int d_v, float scale, void *o, void *y, void *workspace, size_t ws_bytes,
                            void *stream) {
    const GateArgs gate{z, norm_w, norm_eps, y};
    return layer_prefill_impl(x_raw, conv_w, a, b, A_log, dt_bias, l2_eps, initial_state,
                              final_state, conv_state_in, conv_state_out, cu_seqlens, N, T, H_qk,
                              H_v, d_k, d_v,
                              scale, o, nullptr, 0, workspace, ws_bytes, stream, &gate);
}

int gdn_layer_prefill_save_states(const void *x_raw, const void *conv_w, const float *a,
                                  const float *b, const float *A_log, const float *dt_bias,
                                  float l2_eps, const float *initial_state, float *final_state,
                                  void *conv_state_out, const int32_t *cu_seqlens, int N, int T,
                                  int H_qk, int H_v, int d_k, int d_v, float scale, void *o,
                                  void *chunk_states, size_t cs_bytes, void *workspace,
                                  size_t ws_bytes, void *stream) {
    if (!chunk_states) return fail(GDN_ERR_INVALID_ARG, "chunk_states must be non-NULL");
    return layer_prefill_impl(x_raw, conv_w, a, b, A_log, dt_bias, l2_eps, initial_state,
                              final_state, nullptr, conv_state_out, cu_seqlens, N, T, H_qk, H_v,
                              d_k, d_v, scale, o, chunk_states, cs_bytes, workspace, ws_bytes,
                              stream);
}

int gdn_layer_decode_step(const void *x_raw, const void *conv_w, const float *a, const float *b,
                          const float *A_log, const float *dt_bias, float l2_eps,
                          void *conv_state_pool, float *state_pool, const int32_t *slot_idx, int B,
                          int P, int H_qk, int H_v, int d_k, int d_v, float scale, void *o,
                          void *stream) {
    int rc;
    if ((rc = check_heads(H_qk, H_v, d_k, d_v))) return rc;
    if (B < 0) return fail(GDN_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    if (P < 1) return fail(GDN_ERR_INVALID_ARG, "P must be >= 1 (got %d)", P);
    if (B > P) return fail(GDN_ERR_INVALID_ARG, "B (%d) distinct slots cannot fit a pool of P=%d", B, P);
    if ((long long)B * H_v > 0x7FFFFFFFLL) return fail(GDN_ERR_INVALID_ARG, "B * H_v too large");
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    if (!(l2_eps >= 0.f) || !std::isfinite(l2_eps))
        return fail(GDN_ERR_INVALID_ARG, "l2_eps must be finite and >= 0");
    if (B == 0) return ok();
    if (!x_raw || !conv_w || !a || !b || !A_log || !dt_bias || !conv_state_pool || !state_pool ||
        !slot_idx || !o)
        return fail(GDN_ERR_INVALID_ARG, "every pointer argument must be non-NULL");
    const size_t craw = (size_t)(2 * H_qk + H_v) * gdn::kD;
    const size_t nx = (size_t)B * craw * 2, nc = (size_t)P * 3 * craw * 2, nw = craw * 4 * 2;
    const size_t npool = (size_t)P * H_v * gdn::kD * gdn::kD * 4, no = (size_t)B * H_v * gdn::kD * 2;
    const size_t ng = (size_t)B * H_v * 4;
    if (overlaps(o, no, state_pool, npool) || overlaps(o, no, conv_state_pool, nc) ||
        overlaps(o, no, x_raw, nx) || overlaps(o, no, a, ng) || overlaps(o, no, b, ng))
        return fail(GDN_ERR_INVALID_ARG, "o must not overlap inputs or the pools");
    if (overlaps(conv_state_pool, nc, state_pool, npool) || overlaps(conv_state_pool, nc, x_raw, nx) ||
        overlaps(conv_state_pool, nc, conv_w, nw) || overlaps(state_pool, npool, x_raw, nx) ||
        overlaps(state_pool, npool, conv_w, nw))
        return fail(GDN_ERR_INVALID_ARG, "the pools must not overlap each other or the inputs");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode(s)) {
        int bad = 0;
        hipError_t e = gdn::debug_check_slots(slot_idx, B, P, s, &bad);
        if (e != hipSuccess) return hip_fail(e, "slot_idx check");
        if (bad) return fail(GDN_ERR_DEVICE_CHECK, "slot_idx has ids outside [0, %d) or repeated ids", P);
    }
    // the decode reads every addressed slot's history; the shift that follows
    // on the same stream rewrites it
    hipError_t e = gdn::launch_decode_step_raw(x_raw, conv_w, a, b, A_log, dt_bias, l2_eps,
                                               conv_state_pool, state_pool, slot_idx, B, H_qk, H_v,
                                               scale, o, s);
    if (e == hipSuccess) e = gdn::launch_conv_shift(x_raw, slot_idx, B, (int)craw, conv_state_pool, s);
    return finish(e, s, "gdn_layer_decode_step launch");
}

int gdn_decode_multi_step(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, float *state_pool, const int32_t *slot_idx, int B,
                          int P, int n_tok, int H_qk, int H_v, int d_k, int d_v, float scale,
                          void *o, float *snapshots, void *stream) {
    int rc;
    if ((rc = check_heads(H_qk, H_v, d_k, d_v))) return rc;
    if (B < 0) return fail(GDN_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    if (P < 1) return fail(GDN_ERR_INVALID_ARG, "P must be >= 1 (got %d)", P);
    if (n_tok < 1) return fail(GDN_ERR_INVALID_ARG, "n_tok must be >= 1 (got %d)", n_tok);
    if (B > P) return fail(GDN_ERR_INVALID_ARG, "B (%d) distinct slots cannot fit a pool of P=%d", B, P);
    if ((long long)B * H_v > 0x7FFFFFFFLL || (long long)B * n_tok * H_v > 0x7FFFFFFFLL)
        return fail(GDN_ERR_INVALID_ARG, "B * n_tok * H_v too large");
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    if (B == 0) return ok();
    if (!q || !k || !v || !g || !beta || !state_pool || !slot_idx || !o)
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta, state_pool, slot_idx and o must be non-NULL");
    const size_t st = (size_t)gdn::kD * gdn::kD * 4;
    const size_t npool = (size_t)P * H_v * st, nsnap = (size_t)B * n_tok * H_v * st;
    const size_t nqk = (size_t)B * n_tok * H_qk * gdn::kD * 2, nv = (size_t)B * n_tok * H_v * gdn::kD * 2;
    const size_t ng = (size_t)B * n_tok * H_v * 4;
    if (overlaps(o, nv, state_pool, npool) || overlaps(o, nv, q, nqk) || overlaps(o, nv, k, nqk) ||
        overlaps(o, nv, v, nv) || overlaps(o, nv, snapshots, nsnap))
        return fail(GDN_ERR_INVALID_ARG, "o must not overlap inputs, the pool or the snapshots");
    if (snapshots && (overlaps(snapshots, nsnap, state_pool, npool) || overlaps(snapshots, nsnap, q, nqk) ||
                      overlaps(snapshots, nsnap, k, nqk) || overlaps(snapshots, nsnap, v, nv) ||
                      overlaps(snapshots, nsnap, g, ng) || overlaps(snapshots, nsnap, beta, ng)))
        return fail(GDN_ERR_INVALID_ARG, "snapshots must not overlap the pool or the inputs");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode(s)) {
        int bad = 0;
        hipError_t e = gdn::debug_check_slots(slot_idx, B, P, s, &bad);
        if (e != hipSuccess) return hip_fail(e, "slot_idx check");
        if (bad) return fail(GDN_ERR_DEVICE_CHECK, "slot_idx has ids outside [0, %d) or repeated ids", P);
    }
    hipError_t e = gdn::launch_decode_multi(q, k, v, g, beta, state_pool, slot_idx, B, n_tok, H_qk,
                                            H_v, scale, o, snapshots, s);
    return finish(e, s, "gdn_decode_multi_step launch");
}

int gdn_state_rollback(const float *snapshots, const int32_t *n_keep, int n_tok, float *state_pool,
                       const int32_t *slot_idx, int B, int P, int H_v, int d_k, int d_v,
                       void *stream) {
    int rc;
    if ((rc = check_heads(1, H_v, d_k, d_v))) return rc;
    if (B < 0 || P < 1 || n_tok < 1 || B > P)
        return fail(GDN_ERR_INVALID_ARG, "need B >= 0, P >= 1, n_tok >= 1 and B <= P");
    if ((long long)B * n_tok * H_v > 0x7FFFFFFFLL) return fail(GDN_ERR_INVALID_ARG, "B * n_tok * H_v too large");
    if (B == 0) return ok();
    if (!snapshots || !n_keep || !state_pool || !slot_idx)
        return fail(GDN_ERR_INVALID_ARG, "snapshots, n_keep, state_pool and slot_idx must be non-NULL");
    const size_t st = (size_t)gdn::kD * gdn::kD * 4;
    if (overlaps(snapshots, (size_t)B * n_tok * H_v * st, state_pool, (size_t)P * H_v * st))
        return fail(GDN_ERR_INVALID_ARG, "snapshots must not overlap the pool");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode(s)) {
        int bad = 0;
        hipError_t e = gdn::debug_check_slots(slot_idx, B, P, s, &bad);
        if (e != hipSuccess) return hip_fail(e, "slot_idx check");
        if (bad) return fail(GDN_ERR_DEVICE_CHECK, "slot_idx has ids outside [0, %d) or repeated ids", P);
    }
    hipError_t e = gdn::launch_state_rollback(snapshots, n_keep, n_tok, state_pool, slot_idx, B, H_v, s);
    return finish(e, s, "gdn_state_rollback launch");
}

int gdn_gated_norm(const void *o, const void *z, const float *w, int rows, int d_v, float eps,
                   void *out, void *stream) {
    if (d_v != gdn::kD) return fail(GDN_ERR_UNSUPPORTED, "only d_v = 128 is built (got %d)", d_v);
    if (rows < 0) return fail(GDN_ERR_INVALID_ARG, "rows must be >= 0 (got %d)", rows);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(GDN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (rows == 0) return ok();
    if (!o || !z || !w || !out) return fail(GDN_ERR_INVALID_ARG, "o, z, w and out must be non-NULL");
    const size_t n = (size_t)rows * gdn::kD * 2;
    if ((out != o && overlaps(out, n, o, n)) || overlaps(out, n, z, n) ||
        overlaps(out, n, w, (size_t)gdn::kD * 4))
        return fail(GDN_ERR_INVALID_ARG, "out must equal o or not overlap it, and not overlap z or w");
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_gated_norm(o, z, w, rows, eps, out, s), s, "gdn_gated_norm launch");
}

size_t gdn_gated_norm_backward_workspace_size(int rows, int d_v) {
    if (rows < 0 || d_v != gdn::kD) return 0;
    return gdn::gated_norm_bwd_partial_bytes(rows);
}

int gdn_gated_norm_backward(const void *o, const void *z, const float *w, const void *dy,
                            int rows, int d_v, float eps, void *d_o, void *dz, float *dw,
                            void *workspace, size_t ws_bytes, void *stream) {
    if (d_v != gdn::kD) return fail(GDN_ERR_UNSUPPORTED, "only d_v = 128 is built (got %d)", d_v);
    if (rows < 0) return fail(GDN_ERR_INVALID_ARG, "rows must be >= 0 (got %d)", rows);
    if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(GDN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (!w || !dw) return fail(GDN_ERR_INVALID_ARG, "w and dw must be non-NULL");
    if (rows > 0 && (!o || !z || !dy || !d_o || !dz))
        return fail(GDN_ERR_INVALID_ARG, "o, z, dy, d_o and dz must be non-NULL");
    const size_t need = gdn_gated_norm_backward_workspace_size(rows, d_v);
    if (ws_bytes < need || !workspace)
        return fail(GDN_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws_bytes, need);
    const size_t n = (size_t)rows * gdn::kD * 2, nw = (size_t)gdn::kD * 4;
    const struct { const void *p; size_t n; } in[] = {{o, n}, {z, n}, {w, nw}, {dy, n}};
    const struct { const void *p; size_t n; } out[] = {{d_o, n}, {dz, n}, {dw, nw}, {workspace, need}};
    for (const auto &x : out) {
        for (const auto &i : in)
            if (overlaps(x.p, x.n, i.p, i.n))
                return fail(GDN_ERR_INVALID_ARG, "gradients and workspace must not overlap any input");
        for (const auto &x2 : out)
            if (&x2 != &x && overlaps(x.p, x.n, x2.p, x2.n))
                return fail(GDN_ERR_INVALID_ARG, "gradients and workspace must not overlap each other");
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_gated_norm_bwd(o, z, w, dy, rows, eps, d_o, dz, dw,
                                             static_cast<float *>(workspace), s),
                  s, "gdn_gated_norm_backward launch");
}

int gdn_decode_step(const void *q, const void *k, const void *v, const float *g,
                    const float *beta, float *state_pool, const int32_t *slot_idx, int B, int P,
                    int H_qk, int H_v, int d_k, int d_v, float scale, void *o, void *stream) {
    int rc;
    if ((rc = check_heads(H_qk, H_v, d_k, d_v))) return rc;
    if (B < 0) return fail(GDN_ERR_INVALID_ARG, "B must be >= 0 (got %d)", B);
    if (P < 1) return fail(GDN_ERR_INVALID_ARG, "P must be >= 1 (got %d)", P);
    if (B > P) return fail(GDN_ERR_INVALID_ARG, "B (%d) distinct slots cannot fit a pool of P=%d", B, P);
    if ((long long)B * H_v > 0x7FFFFFFFLL) return fail(GDN_ERR_INVALID_ARG, "B * H_v too large");
    if (!std::isfinite(scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
    if (B == 0) return ok();
    if (!q || !k || !v || !g || !beta || !state_pool || !slot_idx || !o)
        return fail(GDN_ERR_INVALID_ARG, "q, k, v, g, beta, state_pool, slot_idx and o must be non-NULL");
    const size_t npool = (size_t)P * H_v * gdn::kD * gdn::kD * 4, no = (size_t)B * H_v * gdn::kD * 2;
    if (overlaps(o, no, state_pool, npool) || overlaps(o, no, q, (size_t)B * H_qk * gdn::kD * 2) ||
        overlaps(o, no, k, (size_t)B * H_qk * gdn::kD * 2) || overlaps(o, no, v, no))
        return fail(GDN_ERR_INVALID_ARG, "o must not overlap inputs or the state pool");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_mode(s)) {
        int bad = 0;
        hipError_t e = gdn::debug_check_slots(slot_idx, B, P, s, &bad);
        if (e != hipSuccess) return hip_fail(e, "slot_idx check");
        if (bad) return fail(GDN_ERR_DEVICE_CHECK, "slot_idx has ids outside [0, %d) or repeated ids", P);
    }
    hipError_t e = gdn::launch_decode_step(q, k, v, g, beta, state_pool, slot_idx, B, H_qk, H_v,
                                           scale, o, s);
    return finish(e, s, "gdn_decode_step launch");
}

}  // extern "C"
