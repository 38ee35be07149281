// gdn_internal.h -- launchers shared between the kernel files and the C ABI.
// Internal header: not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kD = 128;       // d_k = d_v built
constexpr int kChunk = 64;    // prefill chunk length
constexpr int kMaxPrepGroup = 8;   // V-heads per QK head the bf16 prefill handles
constexpr int kIoF32 = 0;
constexpr int kIoBF16 = 1;

hipError_t launch_conv_prelude(const void *x, const void *w, const int32_t *cu_seqlens, int N,
                               int T, int H_qk, int H_v, float eps, void *q, void *k, void *v,
                               hipStream_t stream);

hipError_t launch_decode_step(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, float *pool, const int32_t *slot_idx, int B,
                              int H_qk, int H_v, float scale, void *o, hipStream_t stream);

hipError_t launch_recurrent_prefill(int io_dtype, const void *q, const void *k, const void *v,
                                    const float *g, const float *beta, const float *S0,
                                    float *S_final, const int32_t *cu_seqlens, int N, int T,
                                    int H_qk, int H_v, float scale, void *o, hipStream_t stream);

// Chunked bf16 prefill (64-token chunks, bf16 matrix-core products); `raw`:
// from the raw projections, with the conv prelude fused.  chunk_states (or
// NULL): bf16 [chunks][H_v][d_v][d_k], the state each chunk starts from, kept
// for a later backward (chunk_states_bytes of them).
size_t chunked_workspace_bytes(int N, int T, int H_qk, int H_v, bool raw);
size_t chunk_states_bytes(int N, int T, int H_v);
hipError_t launch_chunked_prefill(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *S0, float *S_final,
                                  const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v,
                                  float scale, void *o, void *chunk_states, void *workspace,
                                  hipStream_t stream);
// The bf16 chunked prefill with its workspace in a fixed device array of
// chunked_scratch_bytes() (for callers that cannot allocate); everything on
// `stream`.  hipErrorInvalidValue if the workspace would not fit.
size_t chunked_scratch_bytes();
hipError_t launch_chunked_prefill_no_alloc(const void *q, const void *k, const void *v,
                                           const float *g, const float *beta, const float *S0,
                                           float *S_final, const int32_t *cu_seqlens, int N, int T,
                                           int H_qk, int H_v, float scale, void *o,
                                           hipStream_t stream);
hipError_t launch_chunked_prefill_raw(const void *x, const void *w, float eps, const float *g,
                                      const float *beta, const float *S0, float *S_final,
                                      const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v,
                                      float scale, void *o, void *chunk_states, void *workspace,
                                      hipStream_t stream, const void *conv_hist_in = nullptr);
// The same with the output gate (o / sqrt(mean(o^2) + norm_eps) * norm_w *
// SiLU(z) per 128-wide row) fused into the scan's stores: o and y both
// written; the workspace holds chunked_gated_workspace_bytes.
size_t chunked_gated_workspace_bytes(int N, int T, int H_qk, int H_v);
hipError_t launch_chunked_prefill_raw_gated(const void *x, const void *w, float eps, const float *g,
                                            const float *beta, const float *S0, float *S_final,
                                            const int32_t *cu_seqlens, int N, int T, int H_qk,
                                            int H_v, float scale, void *o, const void *z,
                                            const float *norm_w, float norm_eps, void *y,
                                            void *workspace, hipStream_t stream,
                                            const void *conv_hist_in = nullptr);

// Gradients of the chunked bf16 prefill (dq, dk, dv bf16; dg, dbeta, dS0 fp32);
// `saved` / chunk_states: with the chunk states of an earlier forward pass.
size_t chunked_backward_workspace_bytes(int N, int T, int H_qk, int H_v, bool saved);
hipError_t launch_chunked_backward(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *S0, const int32_t *cu_seqlens,
                                   int N, int T, int H_qk, int H_v, float scale, const void *d_o,
                                   const float *dS_final, void *dq, void *dk, void *dv, float *dg,
                                   float *dbeta, float *dS0, const void *chunk_states,
                                   void *workspace, hipStream_t stream);
hipError_t launch_bwd_scan(const void *q, const void *k, const void *d_o, const float *dS_final,
                           const int32_t *cu_seqlens, const int32_t *chunk_base, int N, int T,
                           int H_qk, int H_v, float scale, const void *bws, void *dsw, void *duw,
                           void *dv, float *dS0, int c_lo, int c_hi, hipStream_t stream);
hipError_t launch_bwd_grad(const void *q, const void *k, const void *v, const void *d_o,
                           const void *dv, const float *beta, const int32_t *cu_seqlens,
                           const int32_t *chunk_base, int N, int T, int H_qk, int H_v,
                           float scale, const void *bws, const void *states, const void *dsw,
                           const void *duw, void *dq, void *dk, float *dg, float *dbeta,
                           int item_lo, int item_hi, int grid, hipStream_t stream);

// Gradients of the prelude (dx bf16, dw fp32 [C_raw][4]; `partial` holds
// prelude_bwd_partial_bytes) and of the gates (da, db fp32 [T][H_v]; dA_log,
// ddt_bias fp32 [H_v]; `partial` holds gates_bwd_partial_bytes).
size_t prelude_bwd_partial_bytes(int T, int H_qk, int H_v);
size_t gates_bwd_partial_bytes(int H_v);
// Gradients of the output gate (d_o, dz bf16; dw fp32 [128]; `partial` holds
// gated_norm_bwd_partial_bytes).
size_t gated_norm_bwd_partial_bytes(int rows);
hipError_t launch_gated_norm_bwd(const void *o, const void *z, const float *w, const void *dy,
                                 int rows, float eps, void *d_o, void *dz, float *dw,
                                 float *partial, hipStream_t stream);
hipError_t launch_prelude_bwd(const void *x, const void *w, const int32_t *cu_seqlens, int N, int T,
                              int H_qk, int H_v, float eps, const void *dq, const void *dk,
                              const void *dv, void *dx, float *dw, float *partial,
                              hipStream_t stream);
hipError_t launch_gates_bwd(const float *a, const float *b, const float *A_log,
                            const float *dt_bias, const float *dg, const float *dbeta, int T,
                            int H_v, float *da, float *db, float *dA_log, float *ddt_bias,
                            float *partial, hipStream_t stream);

// The layer's forward from raw projections: gates, conv history, decode.
hipError_t launch_gates(const float *a, const float *b, const float *A_log, const float *dt_bias,
                        int T, int H_v, float *g, float *beta, hipStream_t stream);
// Each sequence's last three raw rows into hist_out ([N][3][C_raw]); rows
// before a sequence's start come from hist_in (or are zero without it).
// hist_out may be hist_in.
hipError_t launch_conv_hist(const void *x, const int32_t *cu_seqlens, int N, int T, int C_raw,
                            const void *hist_in, void *hist_out, hipStream_t stream);
hipError_t launch_conv_shift(const void *x, const int32_t *slot_idx, int B, int C_raw, void *hist,
                             hipStream_t stream);
hipError_t launch_gated_norm(const void *o, const void *z, const float *w, int rows, float eps,
                             void *out, hipStream_t stream);
hipError_t launch_decode_step_raw(const void *x, const void *w, const float *a, const float *b,
                                  const float *A_log, const float *dt_bias, float eps,
                                  const void *conv_hist, float *pool, const int32_t *slot_idx,
                                  int B, int H_qk, int H_v, float scale, void *o,
                                  hipStream_t stream);

// n tokens per sequence with optional per-position state snapshots; rollback.
hipError_t launch_decode_multi(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, float *pool, const int32_t *slot_idx, int B,
                               int n, int H_qk, int H_v, float scale, void *o, float *snapshots,
                               hipStream_t stream);
hipError_t launch_state_rollback(const float *snapshots, const int32_t *n_keep, int n, float *pool,
                                 const int32_t *slot_idx, int B, int H_v, hipStream_t stream);

// Device-side precondition checks (GDN_DEBUG=1): launch a one-workgroup scan,
// wait for the stream, and return the violation bits in *result (0 = ok).
hipError_t debug_check_cu_seqlens(const int32_t *cu_seqlens, int N, int T, hipStream_t stream,
                                  int *result);
hipError_t debug_check_slots(const int32_t *slot_idx, int B, int P, hipStream_t stream,
                             int *result);

}  // namespace gdn
