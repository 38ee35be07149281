// gdn_recurrent.hip -- state-in-registers kernels of the gated delta rule:
//   * the decode step over a state-slot pool (one token per sequence), and
//   * the token-by-token prefill used for fp32 io.
//
// Update per token and state row i (S is d_v x d_k, row i = S[i, :]):
//   a_i = S_i . k,   c_i = S_i . q,   d_i = beta (v_i - alpha a_i)
//   S_i <- alpha S_i + d_i k,        o_i = alpha c_i + d_i (k . q)
// which is S <- alpha S (I - beta k k^T) + beta v k^T followed by o = S q
// ("从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力", sec. 2.2,
// gated by alpha = exp(g)); both dot products use the old row, so each state
// row is read once and written once.
//
// Thread layout (256 threads = 4 waves own one 128 x 128 state): lane groups of
// 16 share a row; lane c of a group holds columns 4c..4c+3 and 64+4c..64+4c+3,
// so one row is two contiguous 256-byte segments and its dot products reduce
// inside one 16-lane DPP row.  Thread (wave w, group r) owns rows
// 32w + 4j + r for j = 0..7: 64 fp32 state values per thread, all loaded before
// any arithmetic so that 64 KiB per workgroup are in flight at once.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

struct RowMap {
    int wave, c16, r4;
    __device__ RowMap() {
        const int lane = threadIdx.x & 63;
        wave = threadIdx.x >> 6;
        c16 = lane & 15;
        r4 = lane >> 4;
    }
    __device__ int row(int j) const { return wave * 32 + j * 4 + r4; }
    __device__ int col(int half) const { return half * 64 + c16 * 4; }
};

template <typename T>
__device__ __forceinline__ void load_vec8(const T *base, const RowMap &m, float *d) {
    load4(base + m.col(0), d);
    load4(base + m.col(1), d + 4);
}

// The 8 state rows this thread owns (s[j][0..7] = row m.row(j), columns
// m.col(0)+0..3 and m.col(1)+0..3), read and written with non-temporal
// accesses: a decode call touches each state once, and cached fills and
// write-backs of the 805 MB of states per B = 256 step only cost bandwidth.
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load_state_rows(const float *S, const RowMap &m, float (&s)[8][8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(S + m.row(j) * kD + m.col(hh)));
            s[j][4 * hh] = x.x;
            s[j][4 * hh + 1] = x.y;
            s[j][4 * hh + 2] = x.z;
            s[j][4 * hh + 3] = x.w;
        }
}
__device__ __forceinline__ void store_state_rows(float *S, const RowMap &m, const float (&s)[8][8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            __builtin_nontemporal_store(f32x4v{s[j][4 * hh], s[j][4 * hh + 1], s[j][4 * hh + 2], s[j][4 * hh + 3]},
                                        reinterpret_cast<f32x4v *>(S + m.row(j) * kD + m.col(hh)));
}

// One token applied to the 8 rows this thread owns.  s[j][0..7] holds row
// m.row(j), columns (m.col(0)+0..3, m.col(1)+0..3).  vr[j] = v[m.row(j)].
// Returns, in lanes with c16 < 8, o of row m.row(c16).
__device__ __forceinline__ float delta_rows(float (&s)[8][8], const float *kk, const float *qq,
                                            const float *vr, float alpha, float beta,
                                            const RowMap &m) {
    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) kq += kk[e] * qq[e];
    kq = row16_sum(kq);
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float a = 0.f, c = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a += s[j][e] * kk[e];
            c += s[j][e] * qq[e];
        }
        a = row16_sum(a);
        c = row16_sum(c);
        const float d = beta * (vr[j] - alpha * a);
        const float oj = alpha * c + d * kq;
#pragma unroll
        for (int e = 0; e < 8; ++e) s[j][e] = alpha * s[j][e] + d * kk[e];
        mine = (m.c16 == j) ? oj : mine;
    }
    return mine;
}

// Decode from the raw projections: the new token's raw row, each slot's
// three previous raw rows (its conv history), the conv taps, the raw gate
// projections and the layer's A_log, dt_bias.
struct RawDecodeIn {
    const uint16_t *x;       // [B][C_raw] bf16
    const uint16_t *w;       // [C_raw][4] bf16
    const uint16_t *conv;    // [P][3][C_raw] bf16, read only here
    const float *a, *b;      // [B][H_v]
    const float *A_log, *dt_bias;   // [H_v]
    float eps;
};

// With kRaw, the workgroup first forms its own q, k (its QK head) and v (its
// V-head) from the raw rows with the conv prelude's arithmetic and lane layout
// (16 lanes x 8 channels per 128-channel block, the norm reduced over the
// 16-lane row), rounds them to bf16 as the prelude does, and hands them to the
// other threads through LDS; the gates come from the shared gate helpers.  The
// state loads are issued first, so this overlaps them.
template <bool kRaw>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ pool,
    const int32_t *__restrict__ slot_idx, int H_qk, int H_v, float scale,
    uint16_t *__restrict__ o, const RawDecodeIn raw) {
    const RowMap m;
    const int b = blockIdx.x / H_v;
    const int h = blockIdx.x - b * H_v;
    const int hq = h / (H_v / H_qk);
    const int slot = slot_idx[b];
    float *S = pool + ((size_t)slot * H_v + h) * (kD * kD);

    float s[8][8];
    load_state_rows(S, m, s);
    float kk[8], qq[8], vr[8];
    float alpha, bt;
    if constexpr (kRaw) {
        __shared__ __attribute__((aligned(16))) uint16_t sqkv[3][kD];   // q, k, v (bf16)
        if (threadIdx.x < 48) {                    // wave 0, lanes 0-15 q, 16-31 k, 32-47 v
            const int part = threadIdx.x >> 4, cg = threadIdx.x & 15;
            const size_t C = (size_t)(2 * H_qk + H_v) * kD;
            const size_t ch = (size_t)(part == 0 ? hq : part == 1 ? H_qk + hq : 2 * H_qk + h) * kD + 8 * cg;
            float wt[4][8];
            load_taps8(raw.w, ch, wt);
            const uint16_t *hist = raw.conv + (size_t)slot * 3 * C + ch;
            float xm[4][8];
#pragma unroll
            for (int j = 0; j < 3; ++j) unpack8(*reinterpret_cast<const uint4 *>(hist + j * C), xm[j]);
            unpack8(*reinterpret_cast<const uint4 *>(raw.x + (size_t)b * C + ch), xm[3]);
            float y[8], ss = 0.f;
            conv_silu8(wt, xm[0], xm[1], xm[2], xm[3], y, ss);
            const float rn = rsqrtf(row16_sum(ss) + raw.eps);   // full 16-lane rows: 0-15, 16-31, 32-47
            if (part < 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] *= rn;
            }
            *reinterpret_cast<uint4 *>(sqkv[part] + 8 * cg) = pack_bf8(y);
        }
        const size_t gi = (size_t)b * H_v + h;
        alpha = expf(gate_log_decay(raw.a[gi], raw.A_log[h], raw.dt_bias[h]));
        bt = gate_beta(raw.b[gi]);
        __syncthreads();
        load_vec8(sqkv[1], m, kk);
        load_vec8(sqkv[0], m, qq);
#pragma unroll
        for (int j = 0; j < 8; ++j) vr[j] = bf2f(sqkv[2][m.row(j)]);
    } else {
        load_vec8(k + ((size_t)b * H_qk + hq) * kD, m, kk);
        load_vec8(q + ((size_t)b * H_qk + hq) * kD, m, qq);
        const uint16_t *vb = v + ((size_t)b * H_v + h) * kD;
#pragma unroll
        for (int j = 0; j < 8; ++j) vr[j] = bf2f(vb[m.row(j)]);
        alpha = expf(g[(size_t)b * H_v + h]);
        bt = beta[(size_t)b * H_v + h];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) qq[e] *= scale;

    const float mine = delta_rows(s, kk, qq, vr, alpha, bt, m);

    store_state_rows(S, m, s);
    if (m.c16 < 8) o[((size_t)b * H_v + h) * kD + m.wave * 32 + m.c16 * 4 + m.r4] = f2bf(mine);
}

// n tokens per sequence (speculative-decoding verification): the state stays
// in registers across the tokens, each token's inputs are loaded during the
// previous token's arithmetic, and, when snapshots is given, the state before
// each token is stored there ([B][n][H_v][d_v][d_k]) so that a caller can
// return the slot to any prefix of the tokens.  Per (sequence, V-head): one
// state read, one state write, n snapshot writes.
__global__ __launch_bounds__(256) void decode_multi_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ pool,
    const int32_t *__restrict__ slot_idx, int n, int H_qk, int H_v, float scale,
    uint16_t *__restrict__ o, float *__restrict__ snapshots) {
    const RowMap m;
    const int b = blockIdx.x / H_v;
    const int h = blockIdx.x - b * H_v;
    const int hq = h / (H_v / H_qk);
    float *S = pool + ((size_t)slot_idx[b] * H_v + h) * (kD * kD);

    float s[8][8];
    load_state_rows(S, m, s);
    float kk[8], qq[8], vr[8], gt, bt;
    auto fetch = [&](int t, float *kd, float *qd, float *vd, float &gd, float &bd) {
        const size_t bt_ = (size_t)b * n + t;
        load_vec8(k + (bt_ * H_qk + hq) * kD, m, kd);
        load_vec8(q + (bt_ * H_qk + hq) * kD, m, qd);
        const uint16_t *vb = v + (bt_ * H_v + h) * kD;
#pragma unroll
        for (int j = 0; j < 8; ++j) vd[j] = bf2f(vb[m.row(j)]);
        gd = g[bt_ * H_v + h];
        bd = beta[bt_ * H_v + h];
    };
    fetch(0, kk, qq, vr, gt, bt);
    for (int t = 0; t < n; ++t) {
        if (snapshots) {
            store_state_rows(snapshots + (((size_t)b * n + t) * H_v + h) * (kD * kD), m, s);
        }
        float kn[8], qn[8], vn[8], gn, bn;
        fetch(min(t + 1, n - 1), kn, qn, vn, gn, bn);   // clamped: the last fetch is unused
#pragma unroll
        for (int e = 0; e < 8; ++e) qq[e] *= scale;
        const float mine = delta_rows(s, kk, qq, vr, expf(gt), bt, m);
        if (m.c16 < 8)
            o[(((size_t)b * n + t) * H_v + h) * kD + m.wave * 32 + m.c16 * 4 + m.r4] = f2bf(mine);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kk[e] = kn[e];
            qq[e] = qn[e];
            vr[e] = vn[e];
        }
        gt = gn;
        bt = bn;
    }
    store_state_rows(S, m, s);
}

// Return slot_idx[b] to the state after its first n_keep[b] tokens:
// snapshots[b][n_keep[b]] when n_keep[b] < n (clamped to [0, n]; n keeps it).
__global__ __launch_bounds__(256) void state_rollback_kernel(const float *__restrict__ snapshots,
                                                             const int32_t *__restrict__ n_keep,
                                                             int n, float *__restrict__ pool,
                                                             const int32_t *__restrict__ slot_idx,
                                                             int H_v) {
    const int b = blockIdx.x / H_v;
    const int h = blockIdx.x - b * H_v;
    const int keep = min(max(n_keep[b], 0), n);
    if (keep == n) return;
    const float4 *src = reinterpret_cast<const float4 *>(
        snapshots + (((size_t)b * n + keep) * H_v + h) * (kD * kD));
    float4 *dst = reinterpret_cast<float4 *>(pool + ((size_t)slot_idx[b] * H_v + h) * (kD * kD));
#pragma unroll
    for (int i = 0; i < kD * kD / 4 / 256; ++i) dst[i * 256 + threadIdx.x] = src[i * 256 + threadIdx.x];
}

// Token-by-token prefill: one workgroup per (sequence, V-head) carries the
// state through the sequence in registers.  The next token's inputs are
// loaded before the current token's arithmetic.
template <typename IO>
__global__ __launch_bounds__(256) void recurrent_prefill_kernel(
    const IO *__restrict__ q, const IO *__restrict__ k, const IO *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta,
    const float *initial_state, float *final_state, const int32_t *__restrict__ cu_seqlens,
    int T, int H_qk, int H_v, float scale, IO *__restrict__ o) {
    const RowMap m;
    const int n = blockIdx.x / H_v;
    const int h = blockIdx.x - n * H_v;
    const int hq = h / (H_v / H_qk);
    const int s0 = cu_seqlens ? cu_seqlens[n] : 0;
    const int s1 = cu_seqlens ? cu_seqlens[n + 1] : T;
    const size_t st_off = ((size_t)n * H_v + h) * (kD * kD);

    float s[8][8];
    if (initial_state) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            load4(initial_state + st_off + m.row(j) * kD + m.col(0), s[j]);
            load4(initial_state + st_off + m.row(j) * kD + m.col(1), s[j] + 4);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) s[j][e] = 0.f;
    }

    float kk[8], qq[8], vr[8], gt = 0.f, bt = 0.f;
    auto fetch = [&](int t, float *kd, float *qd, float *vd, float &gd, float &bd) {
        load_vec8(k + ((size_t)t * H_qk + hq) * kD, m, kd);
        load_vec8(q + ((size_t)t * H_qk + hq) * kD, m, qd);
        const IO *vb = v + ((size_t)t * H_v + h) * kD;
#pragma unroll
        for (int j = 0; j < 8; ++j) vd[j] = load1(vb + m.row(j));
        gd = g[(size_t)t * H_v + h];
        bd = beta[(size_t)t * H_v + h];
    };
    if (s0 < s1) fetch(s0, kk, qq, vr, gt, bt);
    for (int t = s0; t < s1; ++t) {
        float kn[8], qn[8], vn[8], gn = 0.f, bn = 0.f;
        if (t + 1 < s1) fetch(t + 1, kn, qn, vn, gn, bn);
#pragma unroll
        for (int e = 0; e < 8; ++e) qq[e] *= scale;
        const float mine = delta_rows(s, kk, qq, vr, expf(gt), bt, m);
        if (m.c16 < 8) store1(o + ((size_t)t * H_v + h) * kD + m.wave * 32 + m.c16 * 4 + m.r4, mine);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kk[e] = kn[e];
            qq[e] = qn[e];
            vr[e] = vn[e];
        }
        gt = gn;
        bt = bn;
    }
    if (final_state) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            *reinterpret_cast<float4 *>(final_state + st_off + m.row(j) * kD + m.col(0)) =
                make_float4(s[j][0], s[j][1], s[j][2], s[j][3]);
            *reinterpret_cast<float4 *>(final_state + st_off + m.row(j) * kD + m.col(1)) =
                make_float4(s[j][4], s[j][5], s[j][6], s[j][7]);
        }
    }
}

}  // namespace

hipError_t launch_decode_step(const void *q, const void *k, const void *v, const float *g,
                              const float *beta, float *pool, const int32_t *slot_idx, int B,
                              int H_qk, int H_v, float scale, void *o, hipStream_t stream) {
    hipLaunchKernelGGL(decode_step_kernel<false>, dim3(B * H_v), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), g, beta, pool, slot_idx, H_qk, H_v,
                       scale, static_cast<uint16_t *>(o), RawDecodeIn{});
    return hipGetLastError();
}

hipError_t launch_decode_multi(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, float *pool, const int32_t *slot_idx, int B,
                               int n, int H_qk, int H_v, float scale, void *o, float *snapshots,
                               hipStream_t stream) {
    hipLaunchKernelGGL(decode_multi_kernel, dim3(B * H_v), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), g, beta, pool, slot_idx, n, H_qk, H_v,
                       scale, static_cast<uint16_t *>(o), snapshots);
    return hipGetLastError();
}

hipError_t launch_state_rollback(const float *snapshots, const int32_t *n_keep, int n, float *pool,
                                 const int32_t *slot_idx, int B, int H_v, hipStream_t stream) {
    hipLaunchKernelGGL(state_rollback_kernel, dim3(B * H_v), dim3(256), 0, stream, snapshots,
                       n_keep, n, pool, slot_idx, H_v);
    return hipGetLastError();
}

hipError_t launch_decode_step_raw(const void *x, const void *w, const float *a, const float *b,
                                  const float *A_log, const float *dt_bias, float eps,
                                  const void *conv_hist, float *pool, const int32_t *slot_idx,
                                  int B, int H_qk, int H_v, float scale, void *o,
                                  hipStream_t stream) {
    const RawDecodeIn raw{static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w),
                          static_cast<const uint16_t *>(conv_hist), a, b, A_log, dt_bias, eps};
    hipLaunchKernelGGL(decode_step_kernel<true>, dim3(B * H_v), dim3(256), 0, stream, nullptr,
                       nullptr, nullptr, nullptr, nullptr, pool, slot_idx, H_qk, H_v, scale,
                       static_cast<uint16_t *>(o), raw);
    return hipGetLastError();
}

hipError_t launch_recurrent_prefill(int io_dtype, const void *q, const void *k, const void *v,
                                    const float *g, const float *beta, const float *S0,
                                    float *S_final, const int32_t *cu_seqlens, int N, int T,
                                    int H_qk, int H_v, float scale, void *o,
                                    hipStream_t stream) {
    if (io_dtype == kIoF32) {
        hipLaunchKernelGGL(recurrent_prefill_kernel<float>, dim3(N * H_v), dim3(256), 0, stream,
                           static_cast<const float *>(q), static_cast<const float *>(k),
                           static_cast<const float *>(v), g, beta, S0, S_final, cu_seqlens, T,
                           H_qk, H_v, scale, static_cast<float *>(o));
    } else {
        hipLaunchKernelGGL(recurrent_prefill_kernel<uint16_t>, dim3(N * H_v), dim3(256), 0,
                           stream, static_cast<const uint16_t *>(q),
                           static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), g,
                           beta, S0, S_final, cu_seqlens, T, H_qk, H_v, scale,
                           static_cast<uint16_t *>(o));
    }
    return hipGetLastError();
}

}  // namespace gdn
