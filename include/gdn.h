/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet layer library (libgdn.so).
 *
 * The layer keeps, per (sequence, V-head), a d_v x d_k fp32 state S and for each
 * token applies the gated delta rule
 *     S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t (scale * q_t)
 * with decay a_t = exp(g_t) and write strength b_t.
 *
 * Pages cited (title, site):
 *   [Dissect] "从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力"
 *             (www.2kiu.com): sec. 2.1 gives the layer shape (16 QK heads, 48 V heads,
 *             key and value head dim 128, short conv of width 4, the conv1d.weight,
 *             A_log and dt_bias weights) and the fp32 state dtype; sec. 2.2 gives the
 *             delta-rule update (the a_t = 1 case of the formula above) and its
 *             erase-then-write meaning.
 *   [OOM]     "Qwen3.8-27B 混合线性注意力到底解决了什么" (www.mhpn.cn): sec. 1.2 gives a
 *             per-token step taking (q_t, k_t, v_t, S_prev, two gates) and returning
 *             (o_t, S_t) -- the argument set of gdn_decode_step.
 *   [Local]   "Qwen3.8-27B：27B 如何打出千亿级效果，且塞进单张消费级显卡" (www.nzsm.cn):
 *             sec. 2.1 names a fused forward/backward kernel for the GDN layer
 *             (the reason gdn_prefill_backward exists).
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" are HIP device pointers (or host-coherent memory
 *     the device can address); the caller allocates and owns every buffer.  The
 *     library never allocates, frees or retains a caller buffer.
 *   - All arrays are dense, row-major, with the listed shapes.  bf16 arrays hold
 *     IEEE bfloat16 bit patterns (uint16); outputs are rounded to nearest even.
 *   - A state is [d_v][d_k] fp32 with d_k contiguous (the v k^T orientation of
 *     [Dissect sec. 2.2]).  V-head h reads QK head h / (H_v / H_qk).
 *   - The decay gate is passed as its logarithm g (a = exp(g)), fp32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns; nothing synchronises unless the
 *     environment variable GDN_DEBUG=1 is set (read at every call), in which
 *     case each call waits for its kernels and reports device-side failures.
 *   - Graph capture: every entry point may be captured into a HIP graph.  On a
 *     stream under capture the calls enqueue all their work on `stream` itself
 *     (no auxiliary stream, same results), and GDN_DEBUG checks are skipped
 *     (they would have to synchronise).
 *   - Return value: GDN_OK (0) or a negative gdn_status.  On failure nothing has
 *     been enqueued (argument errors are detected on the host before any launch)
 *     except for GDN_ERR_HIP, which reports a failing launch.  The text of the
 *     last failure on the calling thread is returned by gdn_last_error().
 *   - Only d_k = d_v = 128 is built; other head sizes return GDN_ERR_UNSUPPORTED.
 *   - Array contents are not inspected on the host (that would need a sync):
 *     cu_seqlens must be non-decreasing from 0 to T, slot ids distinct and in
 *     [0, P).  With GDN_DEBUG=1 these preconditions are checked on the device.
 *   - Thread safety: calls may be made concurrently from several threads.  The
 *     library's only mutable state is the per-thread error text and, per device,
 *     one auxiliary stream (default priority) with a few events, made on the
 *     first bf16 prefill of a long single sequence and kept until the process
 *     ends; the enqueues on it are serialised by a lock.  Such a prefill runs
 *     part of its work on that stream, forked from and joined back into
 *     `stream` with events, so to the caller it is ordered like any other call
 *     on `stream`.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 5

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = -1, /* NULL required pointer, bad size, H_v % H_qk != 0, ... */
    GDN_ERR_UNSUPPORTED = -2, /* head size or dtype not built */
    GDN_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    GDN_ERR_HIP = -4,         /* a HIP launch/runtime call failed (text in gdn_last_error) */
    GDN_ERR_DEVICE_CHECK = -5 /* GDN_DEBUG=1 only: a device-side precondition failed */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* ABI version of the loaded library (GDN_ABI_VERSION at build time). */
int gdn_abi_version(void);

/* Text describing the last failing call on this thread ("" if none). The string
 * is owned by the library and valid until the next call on the same thread. */
const char *gdn_last_error(void);

/*
 * gdn_conv_prelude -- short causal depthwise conv (width 4), SiLU, then split
 * into q, k, v and L2-normalise every q and k head.  [Dissect sec. 2.1]: the
 * conv kernel width 4 and the per-layer conv1d weight.
 *
 *   x_raw      device bf16 [T][C_raw], C_raw = 2*H_qk*d_k + H_v*d_v, channels
 *              ordered [q heads | k heads | v heads], each head's channels contiguous
 *   conv_w     device bf16 [C_raw][4]; tap 3 multiplies the current token, tap 0
 *              the token three steps back; no bias
 *   cu_seqlens device int32 [N+1] packed sequence offsets, or NULL for a single
 *              sequence (then N must be 1).  Conv taps before each sequence's first
 *              token read zero.
 *   l2_eps     q = y / sqrt(sum(y^2) + l2_eps) per head (same for k)
 *   q, k       device bf16 [T][H_qk][d_k] outputs;  v  device bf16 [T][H_v][d_v]
 * Outputs must not alias inputs.  T = 0 is a no-op.
 */
int gdn_conv_prelude(const void *x_raw, const void *conv_w, const int32_t *cu_seqlens, int N,
                     int T, int H_qk, int H_v, int d_k, int d_v, float l2_eps, void *q, void *k,
                     void *v, void *stream);

/*
 * gdn_prefill_workspace_size -- bytes of device workspace gdn_prefill needs for
 * the given sizes and io dtype (host-only; no device call).  It bounds the
 * number of 64-token chunks by ceil(T/64) + N, so it holds for any cu_seqlens.
 */
size_t gdn_prefill_workspace_size(int io_dtype, int N, int T, int H_qk, int H_v, int d_k,
                                  int d_v);

/*
 * gdn_prefill -- run the recurrence over packed sequences ([Dissect sec. 2.2],
 * gated by a_t = exp(g_t)), returning every o_t and each sequence's final state.
 *
 *   io_dtype       GDN_BF16: q, k, v, o are bf16; computed by the chunked (64-token)
 *                  kernels with bf16 matrix-core products and an fp32 state
 *                  (at most 8 V-heads per QK head, else GDN_ERR_UNSUPPORTED).
 *                  GDN_F32:  q, k, v, o are fp32; computed token by token in fp32.
 *   q, k           device [T][H_qk][d_k];  v  device [T][H_v][d_v]
 *   g, beta        device fp32 [T][H_v]: log decay (<= 0) and write strength
 *   initial_state  device fp32 [N][H_v][d_v][d_k], or NULL for zero states
 *   final_state    device fp32 [N][H_v][d_v][d_k] output, or NULL to skip it.
 *                  May alias initial_state exactly (in-place hand-off).
 *   cu_seqlens     device int32 [N+1], or NULL for one sequence of T tokens (N = 1)
 *   scale          multiplies q (1.0 in the layer as described on the pages)
 *   o              device [T][H_v][d_v] output (io dtype); must not alias inputs
 *   workspace      device scratch of at least gdn_prefill_workspace_size(...) bytes
 *                  (may be NULL when that size is 0); contents on entry are ignored
 */
int gdn_prefill(int io_dtype, const void *q, const void *k, const void *v, const float *g,
                const float *beta, const float *initial_state, float *final_state,
                const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k, int d_v,
                float scale, void *o, void *workspace, size_t ws_bytes, void *stream);

/*
 * gdn_prefill_no_alloc -- gdn_prefill for callers that cannot allocate device
 * memory or pass a workspace (code under stream capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and rules as
 * gdn_prefill without workspace / ws_bytes: the bf16 path keeps its workspace
 * in a scratch array the library holds on each device it runs on (64 MiB,
 * kept until the process ends), so the call allocates nothing.  The limit:
 * gdn_prefill_workspace_size(GDN_BF16, N, T, ...) must not exceed 64 MiB --
 * about 80 chunks of 64 tokens at 48 V-heads, e.g. one sequence of 4096
 * tokens -- else GDN_ERR_WORKSPACE and nothing is enqueued.  All work runs on
 * `stream` (no auxiliary stream).  Calls on the same device share the scratch:
 * calls that overlap in time on one device (two streams, or two threads) race
 * and give wrong results; order them on one stream.  GDN_F32 needs no scratch.
 */
int gdn_prefill_no_alloc(int io_dtype, const void *q, const void *k, const void *v,
                         const float *g, const float *beta, const float *initial_state,
                         float *final_state, const int32_t *cu_seqlens, int N, int T, int H_qk,
                         int H_v, int d_k, int d_v, float scale, void *o, void *stream);

/*
 * gdn_prefill_raw_workspace_size -- bytes of device workspace gdn_prefill_raw
 * needs (host-only; 0 when T = 0).  Bounds the chunk count as
 * gdn_prefill_workspace_size does; about 1.7 times its bf16 figure (the
 * normalised q and k rows are kept there as well).
 */
size_t gdn_prefill_raw_workspace_size(int N, int T, int H_qk, int H_v, int d_k, int d_v);

/*
 * gdn_prefill_raw -- the layer's prefill from its raw projections: the conv
 * prelude ([Dissect sec. 2.1]: width-4 causal depthwise conv, SiLU, L2 norm of
 * each q and k head) fused into the bf16 chunked prefill ([Dissect sec. 2.2],
 * gated by a_t = exp(g_t)).  The result is bit-identical to gdn_conv_prelude
 * followed by gdn_prefill(GDN_BF16, ...) on the same arguments; the
 * normalised q, k and the v that pass between the two are never written out
 * (q and k go through the workspace once, v stays on chip).
 *
 *   x_raw, conv_w, l2_eps   as for gdn_conv_prelude (bf16 [T][C_raw], bf16 [C_raw][4])
 *   g, beta, initial_state, final_state, cu_seqlens, scale, o
 *                           as for gdn_prefill with io_dtype GDN_BF16 (o is bf16
 *                           [T][H_v][d_v]; at most 8 V-heads per QK head)
 *   workspace      device scratch of at least gdn_prefill_raw_workspace_size(...)
 *                  bytes (may be NULL when that size is 0); contents on entry ignored
 */
int gdn_prefill_raw(const void *x_raw, const void *conv_w, float l2_eps, const float *g,
                    const float *beta, const float *initial_state, float *final_state,
                    const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k, int d_v,
                    float scale, void *o, void *workspace, size_t ws_bytes, void *stream);

/*
 * gdn_chunk_states_size -- bytes of the chunk-states buffer that
 * gdn_prefill_save_states and gdn_prefill_raw_save_states fill and
 * gdn_prefill_backward_saved reads (host-only; 0 for invalid sizes): one bf16
 * [d_v][d_k] state per (64-token chunk, V-head), for (T + 63) / 64 + N chunks
 * (an upper bound on the chunks of N packed sequences; 32 KiB per chunk and
 * V-head, 805 MB for one 32768-token sequence with 48 V-heads).
 */
size_t gdn_chunk_states_size(int N, int T, int H_v, int d_k, int d_v);

/*
 * gdn_prefill_save_states -- gdn_prefill (io_dtype GDN_BF16) that also keeps,
 * for a later gdn_prefill_backward_saved, the state each 64-token chunk starts
 * from, rounded to bf16 as the chunk's products use it.  A forward pass of a
 * training step calls it so that the backward need not recompute the forward
 * states ([Local sec. 2.1] names a fused forward and backward kernel for the
 * trained GDN layer).  o and final_state are bit-identical to gdn_prefill's.
 *
 *   q ... o, workspace, ws_bytes, stream   as for gdn_prefill (bf16)
 *   chunk_states   device bf16 [chunks][H_v][d_v][d_k] output, chunks counted
 *                  over the packed sequences in order (sequence n's chunks
 *                  follow those of sequences 0 .. n - 1); at least
 *                  gdn_chunk_states_size(N, T, H_v, d_k, d_v) = cs_bytes bytes;
 *                  must not overlap any other argument.  Owned by the caller;
 *                  entries past the sequences' chunk count are not written.
 * Returns as gdn_prefill; GDN_ERR_INVALID_ARG for a NULL or short chunk_states.
 */
int gdn_prefill_save_states(const void *q, const void *k, const void *v, const float *g,
                            const float *beta, const float *initial_state, float *final_state,
                            const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k,
                            int d_v, float scale, void *o, void *chunk_states, size_t cs_bytes,
                            void *workspace, size_t ws_bytes, void *stream);

/*
 * gdn_prefill_raw_save_states -- gdn_prefill_raw that also keeps the chunk
 * states, as gdn_prefill_save_states does.  The states are those of the
 * equivalent gdn_conv_prelude + gdn_prefill_save_states (bit for bit), so a
 * backward on the prelude's q, k, v may use them.
 *
 *   x_raw ... o, workspace, ws_bytes, stream   as for gdn_prefill_raw
 *   chunk_states, cs_bytes                     as for gdn_prefill_save_states
 */
int gdn_prefill_raw_save_states(const void *x_raw, const void *conv_w, float l2_eps,
                                const float *g, const float *beta, const float *initial_state,
                                float *final_state, const int32_t *cu_seqlens, int N, int T,
                                int H_qk, int H_v, int d_k, int d_v, float scale, void *o,
                                void *chunk_states, size_t cs_bytes, void *workspace,
                                size_t ws_bytes, void *stream);

/*
 * gdn_prefill_backward_workspace_size -- bytes of device workspace
 * gdn_prefill_backward needs (host-only; 0 for invalid sizes, > 0 for any
 * valid N >= 1, T >= 0).  It holds, per (64-token chunk, V-head), the
 * forward and backward chunk records and the bf16 state and state gradient
 * at the chunk's boundaries: about 110 KB per chunk and V-head (2.7 GB for
 * one 32768-token sequence with 48 V-heads).
 */
size_t gdn_prefill_backward_workspace_size(int N, int T, int H_qk, int H_v, int d_k, int d_v);

/*
 * gdn_prefill_backward -- gradients of gdn_prefill (io_dtype GDN_BF16) with
 * respect to all its inputs, given the gradients of the loss with respect to
 * its outputs.  [Local sec. 2.1] names a fused forward and backward kernel for
 * the GDN layer, which is trained.  The result is the derivative of the
 * recurrence of gdn_prefill; it is computed in the same 64-token chunked form
 * (bf16 matrix-core products, fp32 accumulation, fp32 state gradient): the
 * forward states at chunk boundaries are recomputed, then a reverse scan
 * carries the state gradient from the last chunk to the first.
 *
 *   q, k, v, g, beta, initial_state, cu_seqlens, N, T, H_qk, H_v, d_k, d_v, scale
 *                   the forward's inputs, as for gdn_prefill (bf16 q, k, v; at
 *                   most 8 V-heads per QK head)
 *   d_o             device bf16 [T][H_v][d_v]: gradient with respect to o
 *   d_final_state   device fp32 [N][H_v][d_v][d_k], or NULL (zero): gradient
 *                   with respect to the final states
 *   dq, dk          device bf16 [T][H_qk][d_k] outputs (summed over the V-heads
 *                   that read each QK head)
 *   dv              device bf16 [T][H_v][d_v] output
 *   dg, dbeta       device fp32 [T][H_v] outputs
 *   d_initial_state device fp32 [N][H_v][d_v][d_k] output, or NULL to skip it
 *                   (its value does not depend on whether initial_state is NULL)
 *   workspace       device scratch of at least gdn_prefill_backward_workspace_size
 *                   bytes; contents on entry ignored
 * Outputs and workspace must not overlap each other or any input.  T = 0
 * writes only d_initial_state (= d_final_state, or zero).
 */
int gdn_prefill_backward(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                         const void *d_o, const float *d_final_state, int N, int T, int H_qk,
                         int H_v, int d_k, int d_v, float scale, void *dq, void *dk, void *dv,
                         float *dg, float *dbeta, float *d_initial_state, void *workspace,
                         size_t ws_bytes, void *stream);

/*
 * gdn_prefill_backward_saved_workspace_size -- bytes of device workspace
 * gdn_prefill_backward_saved needs (host-only; 0 for invalid sizes): the
 * backward chunk records, the state gradients at chunk ends and dU, without
 * the forward records and states (about 70 KB per chunk and V-head).
 */
size_t gdn_prefill_backward_saved_workspace_size(int N, int T, int H_qk, int H_v, int d_k,
                                                 int d_v);

/*
 * gdn_prefill_backward_saved -- gdn_prefill_backward given the chunk states
 * kept by gdn_prefill_save_states (or gdn_prefill_raw_save_states) on the same
 * q, k, v, g, beta, initial_state and cu_seqlens: the forward pass over the
 * chunks is not repeated.  The gradients are bit-identical to
 * gdn_prefill_backward's on the same inputs.
 *
 *   q, k, v, g, beta, cu_seqlens, d_o, d_final_state, N ... scale, dq ...
 *   d_initial_state            as for gdn_prefill_backward (the initial state
 *                              itself is carried by chunk_states)
 *   chunk_states, cs_bytes     device bf16, as filled by the forward pass;
 *                              at least gdn_chunk_states_size(...) bytes; read only
 *   workspace, ws_bytes        device scratch of at least
 *                              gdn_prefill_backward_saved_workspace_size bytes
 * Outputs and workspace must not overlap each other or any input (chunk_states
 * included).  GDN_ERR_INVALID_ARG for a NULL or short chunk_states.
 */
int gdn_prefill_backward_saved(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const void *chunk_states, size_t cs_bytes,
                               const int32_t *cu_seqlens, const void *d_o,
                               const float *d_final_state, int N, int T, int H_qk, int H_v,
                               int d_k, int d_v, float scale, void *dq, void *dk, void *dv,
                               float *dg, float *dbeta, float *d_initial_state, void *workspace,
                               size_t ws_bytes, void *stream);

/*
 * gdn_layer_prefill_backward_workspace_size -- bytes of device workspace
 * gdn_layer_prefill_backward needs (host-only; 0 for invalid sizes):
 * gdn_prefill_backward_workspace_size plus the recomputed gates, q, k, v, their
 * gradients and per-run partial sums of the conv-weight gradient.
 */
size_t gdn_layer_prefill_backward_workspace_size(int N, int T, int H_qk, int H_v, int d_k,
                                                 int d_v);

/*
 * gdn_layer_prefill_backward -- gradients of the layer's prefill from raw
 * projections (gdn_layer_prefill: gates, conv prelude, recurrence) with respect
 * to all its inputs.  [Local sec. 2.1] names a fused forward and backward GDN
 * kernel; [Dissect sec. 2.1] the conv1d.weight, A_log and dt_bias weights
 * trained with it.  The gates and the prelude are recomputed (as gdn_gates and
 * gdn_conv_prelude form them), gdn_prefill_backward gives the gradients of q,
 * k, v, g and beta, and these are carried back through the L2 norm, SiLU and
 * conv, and through the gates:
 *     da = -dg exp(A_log) sigmoid(a + dt_bias), ddt_bias = sum over tokens of da,
 *     dA_log = sum over tokens of dg g,         db = dbeta beta (1 - beta).
 * Sums over tokens are reduced in a fixed order (results are reproducible).
 *
 *   x_raw, conv_w, a, b, A_log, dt_bias, l2_eps, initial_state, cu_seqlens,
 *   N, T, H_qk, H_v, d_k, d_v, scale   the forward's inputs, as for gdn_layer_prefill
 *   d_o             device bf16 [T][H_v][d_v]: gradient with respect to o
 *   d_final_state   device fp32 [N][H_v][d_v][d_k], or NULL (zero)
 *   dx_raw          device bf16 [T][C_raw] output
 *   dconv_w         device fp32 [C_raw][4] output (tap order as conv_w)
 *   da, db          device fp32 [T][H_v] outputs
 *   dA_log, ddt_bias  device fp32 [H_v] outputs
 *   d_initial_state device fp32 [N][H_v][d_v][d_k] output, or NULL to skip it
 *   workspace       at least gdn_layer_prefill_backward_workspace_size(...) bytes
 * Outputs and workspace must not overlap each other or any input.  T = 0
 * writes zero dconv_w, dA_log, ddt_bias and d_initial_state = d_final_state
 * (or zero).
 */
int gdn_layer_prefill_backward(const void *x_raw, const void *conv_w, const float *a,
                               const float *b, const float *A_log, const float *dt_bias,
                               float l2_eps, const float *initial_state,
                               const int32_t *cu_seqlens, const void *d_o,
                               const float *d_final_state, int N, int T, int H_qk, int H_v,
                               int d_k, int d_v, float scale, void *dx_raw, float *dconv_w,
                               float *da, float *db, float *dA_log, float *ddt_bias,
                               float *d_initial_state, void *workspace, size_t ws_bytes,
                               void *stream);

/*
 * gdn_layer_prefill_backward_saved_workspace_size,
 * gdn_layer_prefill_backward_saved -- gdn_layer_prefill_backward given the
 * chunk states that gdn_layer_prefill_save_states kept on the same inputs
 * (initial_state is then not an argument: the states carry it).  The forward
 * pass over the chunks is not repeated; the gradients are bit-identical.
 *
 *   chunk_states, cs_bytes   device bf16, at least gdn_chunk_states_size(...)
 *                            bytes, read only; other arguments as for
 *                            gdn_layer_prefill_backward
 * GDN_ERR_INVALID_ARG for a NULL or short chunk_states; the overlap rules of
 * gdn_layer_prefill_backward apply with chunk_states among the inputs.
 */
size_t gdn_layer_prefill_backward_saved_workspace_size(int N, int T, int H_qk, int H_v, int d_k,
                                                       int d_v);
int gdn_layer_prefill_backward_saved(const void *x_raw, const void *conv_w, const float *a,
                                     const float *b, const float *A_log, const float *dt_bias,
                                     float l2_eps, const void *chunk_states, size_t cs_bytes,
                                     const int32_t *cu_seqlens, const void *d_o,
                                     const float *d_final_state, int N, int T, int H_qk, int H_v,
                                     int d_k, int d_v, float scale, void *dx_raw, float *dconv_w,
                                     float *da, float *db, float *dA_log, float *ddt_bias,
                                     float *d_initial_state, void *workspace, size_t ws_bytes,
                                     void *stream);

/*
 * gdn_gates -- the layer's gates from its raw per-token projections a, b:
 *     g    = -softplus(a + dt_bias[h]) * exp(A_log[h])   (log decay, a_t = exp(g))
 *     beta = sigmoid(b)
 * [Dissect sec. 2.1] names the A_log and dt_bias weights of each layer.
 *
 *   a, b        device fp32 [T][H_v]
 *   A_log, dt_bias  device fp32 [H_v]
 *   g, beta     device fp32 [T][H_v] outputs (must not overlap the inputs)
 * T = 0 is a no-op.
 */
int gdn_gates(const float *a, const float *b, const float *A_log, const float *dt_bias, int T,
              int H_v, float *g, float *beta, void *stream);

/*
 * gdn_layer_prefill_workspace_size -- bytes of device workspace
 * gdn_layer_prefill needs (host-only; 0 when T = 0): the gates' 8 bytes per
 * token and V-head plus gdn_prefill_raw_workspace_size.
 */
size_t gdn_layer_prefill_workspace_size(int N, int T, int H_qk, int H_v, int d_k, int d_v);

/*
 * gdn_layer_prefill -- the layer's whole prefill from its raw projections
 * ([Dissect sec. 2.1, 2.2]): gdn_gates on a, b into the workspace, then
 * gdn_prefill_raw (conv prelude fused into the bf16 chunked prefill), then,
 * if conv_state_out is given, each sequence's conv history for decoding on:
 * its last three raw rows, oldest first, zero where the sequence is shorter.
 * Without conv_state_in, bit-identical to those calls made one after the
 * other.
 *
 * A prefill that resumes sequences (a prompt fed in several calls, or a
 * prefill after decode steps) passes their conv history as conv_state_in:
 * the conv window before each sequence's first token reads those three raw
 * rows instead of zeros, and a sequence shorter than three tokens takes the
 * rest of its conv_state_out from them.  With initial_state and
 * conv_state_in carried from a prefill of a sequence's first tokens, the
 * outputs of its remaining tokens are those of one prefill of the whole
 * sequence (bit for bit when the first part is a whole number of 64-token
 * chunks: the chunks then coincide).
 *
 *   x_raw, conv_w, l2_eps, initial_state, final_state, cu_seqlens, scale, o
 *                   as for gdn_prefill_raw
 *   a, b            device fp32 [T][H_v];  A_log, dt_bias  device fp32 [H_v]
 *   conv_state_in   device bf16 [N][3][C_raw], each sequence's three raw rows
 *                   before its first token, oldest first; or NULL (zeros).
 *                   May be conv_state_out itself (updated in place), but no
 *                   other output or the workspace.
 *   conv_state_out  device bf16 [N][3][C_raw] output, or NULL
 *   workspace       at least gdn_layer_prefill_workspace_size(...) bytes
 */
int gdn_layer_prefill(const void *x_raw, const void *conv_w, const float *a, const float *b,
                      const float *A_log, const float *dt_bias, float l2_eps,
                      const float *initial_state, float *final_state, const void *conv_state_in,
                      void *conv_state_out, const int32_t *cu_seqlens, int N, int T, int H_qk,
                      int H_v, int d_k, int d_v, float scale, void *o, void *workspace,
                      size_t ws_bytes, void *stream);

/*
 * gdn_layer_prefill_gated_workspace_size -- bytes of device workspace
 * gdn_layer_prefill_gated needs (host-only; 0 when T = 0): that of
 * gdn_layer_prefill plus 2 KiB per chunk and V-head.
 */
size_t gdn_layer_prefill_gated_workspace_size(int N, int T, int H_qk, int H_v, int d_k, int d_v);

/*
 * gdn_layer_prefill_gated -- gdn_layer_prefill with the layer's output gate
 * applied in the same call: besides o it writes
 *     y = o / sqrt(mean(o^2) + norm_eps) * norm_w * SiLU(z)
 * per (token, V-head) row of 128 outputs, the gate of gdn_gated_norm
 * ([Dissect sec. 2.1] names the layer's norm and in_proj_z weights; the gate's
 * form is the reading gdn_gated_norm documents).  When the chunked prefill's
 * grid fits on the device at once (one sequence: 4 * H_v workgroups, at most
 * the number of CUs), the gate is applied inside it, as each chunk's rows of
 * o are completed, not as a pass of its own; otherwise it runs as a pass
 * after the prefill.  Either way o and y are bit-identical to
 * gdn_layer_prefill followed by gdn_gated_norm(o, z, norm_w, norm_eps).
 *
 *   x_raw ... scale, o   as for gdn_layer_prefill (o is written as there)
 *   z               device bf16 [T][H_v][d_v], the gate projections
 *   norm_w          device fp32 [d_v];  norm_eps >= 0
 *   y               device bf16 [T][H_v][d_v] output, overlapping no other
 *                   argument
 *   workspace       at least gdn_layer_prefill_gated_workspace_size(...) bytes
 * T = 0 leaves y untouched (final_state as for gdn_layer_prefill).
 */
int gdn_layer_prefill_gated(const void *x_raw, const void *conv_w, const float *a, const float *b,
                            const float *A_log, const float *dt_bias, float l2_eps, const void *z,
                            const float *norm_w, float norm_eps, const float *initial_state,
                            float *final_state, const void *conv_state_in, void *conv_state_out,
                            const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, int d_k,
                            int d_v, float scale, void *o, void *y, void *workspace, size_t ws_bytes,
                            void *stream);

/*
 * gdn_layer_prefill_save_states -- gdn_layer_prefill that also keeps the
 * chunk states for gdn_layer_prefill_backward_saved (as
 * gdn_prefill_raw_save_states does; outputs bit-identical to gdn_layer_prefill
 * with no conv_state_in: the backward differentiates sequences that start
 * with zero conv history).
 *
 *   chunk_states, cs_bytes   device bf16 output of at least
 *                            gdn_chunk_states_size(N, T, H_v, d_k, d_v) bytes,
 *                            overlapping no other argument
 */
int gdn_layer_prefill_save_states(const void *x_raw, const void *conv_w, const float *a,
                                  const float *b, const float *A_log, const float *dt_bias,
                                  float l2_eps, const float *initial_state, float *final_state,
                                  void *conv_state_out, const int32_t *cu_seqlens, int N, int T,
                                  int H_qk, int H_v, int d_k, int d_v, float scale, void *o,
                                  void *chunk_states, size_t cs_bytes, void *workspace,
                                  size_t ws_bytes, void *stream);

/*
 * gdn_layer_decode_step -- one token for each of B sequences from its raw
 * projections: the conv window of sequence b is its slot's conv history (the
 * three previous raw rows) followed by x_raw[b]; conv, SiLU and q/k L2 norm as
 * in gdn_conv_prelude ([Dissect sec. 2.1]); gates as in gdn_gates; then the
 * update of gdn_decode_step ([OOM sec. 1.2], [Dissect sec. 2.2]).  Afterwards
 * the slot's history holds its rows 1, 2 and x_raw[b].  Bit-identical to
 * gdn_conv_prelude on each 4-row window, gdn_gates and gdn_decode_step.
 *
 *   x_raw           device bf16 [B][C_raw], the new token's raw projections
 *   conv_w, l2_eps  as for gdn_conv_prelude
 *   a, b            device fp32 [B][H_v];  A_log, dt_bias  device fp32 [H_v]
 *   conv_state_pool device bf16 [P][3][C_raw], updated in place for the
 *                   addressed slots (a prefill's conv_state_out rows fit here)
 *   state_pool, slot_idx, B, P, scale, o   as for gdn_decode_step
 * Slots not named in slot_idx are neither read nor written. B = 0 is a no-op.
 */
int gdn_layer_decode_step(const void *x_raw, const void *conv_w, const float *a, const float *b,
                          const float *A_log, const float *dt_bias, float l2_eps,
                          void *conv_state_pool, float *state_pool, const int32_t *slot_idx, int B,
                          int P, int H_qk, int H_v, int d_k, int d_v, float scale, void *o,
                          void *stream);

/*
 * gdn_decode_multi_step -- n_tok tokens for each of B sequences, applied in
 * order to the slot's state, as when a speculative decoder verifies n_tok
 * drafted tokens in one call ([Dissect sec. 2.2] update per token).  Token j
 * of sequence b sees the state after tokens 0..j-1; o is the output of every
 * token; the slot ends with the state after all n_tok tokens.
 *
 *   q, k        device bf16 [B][n_tok][H_qk][d_k];  v  device bf16 [B][n_tok][H_v][d_v]
 *   g, beta     device fp32 [B][n_tok][H_v]
 *   state_pool, slot_idx, B, P, scale   as for gdn_decode_step
 *   o           device bf16 [B][n_tok][H_v][d_v] output
 *   snapshots   device fp32 [B][n_tok][H_v][d_v][d_k] output, or NULL: entry
 *               [b][j] is the slot's state before token j (so after j tokens),
 *               for gdn_state_rollback
 * B = 0 is a no-op; n_tok >= 1.
 */
int gdn_decode_multi_step(const void *q, const void *k, const void *v, const float *g,
                          const float *beta, float *state_pool, const int32_t *slot_idx, int B,
                          int P, int n_tok, int H_qk, int H_v, int d_k, int d_v, float scale,
                          void *o, float *snapshots, void *stream);

/*
 * gdn_state_rollback -- after gdn_decode_multi_step, keep only the first
 * n_keep[b] tokens of sequence b: its slot takes snapshots[b][n_keep[b]]
 * when n_keep[b] < n_tok and is left alone when n_keep[b] = n_tok.
 *
 *   snapshots   device fp32 [B][n_tok][H_v][d_v][d_k] (from gdn_decode_multi_step)
 *   n_keep      device int32 [B], each in [0, n_tok] (clamped to it)
 *   state_pool, slot_idx, B, P   as for gdn_decode_step (same slot_idx as the
 *               gdn_decode_multi_step call)
 */
int gdn_state_rollback(const float *snapshots, const int32_t *n_keep, int n_tok, float *state_pool,
                       const int32_t *slot_idx, int B, int P, int H_v, int d_k, int d_v,
                       void *stream);

/*
 * gdn_gated_norm -- the layer's output gate on rows of d_v outputs (one row
 * per token and V-head): y = o / sqrt(mean(o^2) + eps) * w * SiLU(z).
 * [Dissect sec. 2.1] lists the layer's norm and in_proj_z weights; the pages
 * print no formula, and this per-head RMS norm gated by SiLU(z) is the reading
 * taken.  Apply it to the o of gdn_prefill / gdn_decode_step (rows = T * H_v
 * or B * H_v).
 *
 *   o, z    device bf16 [rows][d_v];  w  device fp32 [d_v] (the norm weight)
 *   out     device bf16 [rows][d_v]; may be o itself (in place)
 * Only d_v = 128 is built.  rows = 0 is a no-op.
 */
int gdn_gated_norm(const void *o, const void *z, const float *w, int rows, int d_v, float eps,
                   void *out, void *stream);

/*
 * gdn_gated_norm_backward_workspace_size -- bytes of device workspace
 * gdn_gated_norm_backward needs (host-only; 0 for invalid sizes): the per-
 * workgroup partial sums of dw, at most 512 KiB.
 */
size_t gdn_gated_norm_backward_workspace_size(int rows, int d_v);

/*
 * gdn_gated_norm_backward -- gradients of gdn_gated_norm with respect to o, z
 * and w, given dy (the gradient with respect to its output).  Per row, with
 * r = (mean(o^2) + eps)^(-1/2), n = o r, s = SiLU(z), u = dy w s:
 *     d_o = r (u - n mean(u n)),  dz = dy n w SiLU'(z),  dw = sum over rows dy n s
 * (dw reduced in a fixed order: results are reproducible).  The form of the
 * gate is the reading of [Dissect sec. 2.1]'s norm and in_proj_z weights that
 * gdn_gated_norm documents.
 *
 *   o, z, dy    device bf16 [rows][d_v]
 *   w           device fp32 [d_v]
 *   d_o, dz     device bf16 [rows][d_v] outputs
 *   dw          device fp32 [d_v] output
 *   workspace   at least gdn_gated_norm_backward_workspace_size(rows, d_v) bytes
 * Outputs and workspace must not overlap each other or any input.  rows = 0
 * writes dw = 0.
 */
int gdn_gated_norm_backward(const void *o, const void *z, const float *w, const void *dy,
                            int rows, int d_v, float eps, void *d_o, void *dz, float *dw,
                            void *workspace, size_t ws_bytes, void *stream);

/*
 * gdn_decode_step -- one token for each of B sequences whose states live in a
 * slot pool; each addressed state is read once and overwritten in place.
 * [OOM sec. 1.2] per-token step (q, k, v, S_prev, gates) -> (o, S); the update
 * is the gated delta rule above, and o uses the updated state.
 *
 *   q, k        device bf16 [B][H_qk][d_k];  v  device bf16 [B][H_v][d_v]
 *   g, beta     device fp32 [B][H_v]
 *   state_pool  device fp32 [P][H_v][d_v][d_k]; slots not named in slot_idx are
 *               neither read nor written
 *   slot_idx    device int32 [B], distinct values in [0, P)
 *   o           device bf16 [B][H_v][d_v] output
 * B = 0 is a no-op.
 */
int gdn_decode_step(const void *q, const void *k, const void *v, const float *g,
                    const float *beta, float *state_pool, const int32_t *slot_idx, int B, int P,
                    int H_qk, int H_v, int d_k, int d_v, float scale, void *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
