// gdn_prelude.hip -- fused short causal conv (width 4) + SiLU + q/k L2 norm.
//
// "从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力", sec. 2.1:
// each linear-attention layer has a depthwise conv of width 4 (conv1d.weight)
// over its projected q/k/v channels.  Per channel c and token t of a sequence
// starting at s0:
//   xc[t, c] = sum_{j=0..3} w[c, j] * x[t - 3 + j, c]   (terms with t-3+j < s0 are 0)
//   y = xc * sigmoid(xc)
// then q and k heads are scaled by 1 / sqrt(sum y^2 + eps); v passes through.
//
// HBM-bound (20 KiB read + 20 KiB written per token at the standard shape), so
// the kernel reads every raw value once, in 256-byte rows: a group of 16 lanes
// owns one 128-channel head block (8 channels = 16 bytes per lane) and walks a
// run of kRun tokens, keeping the last four inputs in registers.  The head's
// sum of squares reduces inside the 16-lane DPP row.  Four groups of a wave take
// four neighbouring head blocks, so each wave reads 1 KiB contiguous per token.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kRun = 32;          // tokens walked by one lane group
constexpr int kBatch = 8;         // rows loaded together
constexpr int kGroupsPerBlock = 16;

__global__ __launch_bounds__(256) void conv_prelude_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const int32_t *__restrict__ cu_seqlens, int N, int T, int H_qk, int H_v, float eps,
    uint16_t *__restrict__ q, uint16_t *__restrict__ k, uint16_t *__restrict__ v) {
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int grp = threadIdx.x >> 4;                  // 0..15
    const int n_blocks = 2 * H_qk + H_v;               // 128-channel head blocks
    const int cb = blockIdx.y * kGroupsPerBlock + grp;
    if (cb >= n_blocks) return;
    const int t0 = blockIdx.x * kRun;
    const int t1 = min(T, t0 + kRun);
    const int C = n_blocks * kD;
    const int ch0 = cb * kD + c16 * 8;                 // first of this lane's 8 channels

    float wt[4][8];
    load_taps8(w, (size_t)ch0, wt);

    // Sequence containing t0: largest n with cu[n] <= t0 (skipping empty ones).
    int n = 0, s0 = 0, s1 = T;
    if (cu_seqlens) {
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cu_seqlens[mid] <= t0) lo = mid; else hi = mid - 1;
        }
        n = lo;
        s0 = cu_seqlens[n];
        s1 = cu_seqlens[n + 1];
    }

    float win[3][8];                                   // x[t-3], x[t-2], x[t-1]
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int src = t0 - 3 + j;
        if (src >= s0 && src >= 0) {
            unpack8(*reinterpret_cast<const uint4 *>(x + (size_t)src * C + ch0), win[j]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
        }
    }

    uint16_t *dst;
    int dst_stride;
    if (cb < H_qk) {
        dst = q + (size_t)cb * kD + c16 * 8;
        dst_stride = H_qk * kD;
    } else if (cb < 2 * H_qk) {
        dst = k + (size_t)(cb - H_qk) * kD + c16 * 8;
        dst_stride = H_qk * kD;
    } else {
        dst = v + (size_t)(cb - 2 * H_qk) * kD + c16 * 8;
        dst_stride = H_v * kD;
    }
    const bool normalise = cb < 2 * H_qk;

    // the run's rows of x are read once and q, k, v written once: non-temporal.
    // Rows are loaded kBatch at a time, the next batch in flight while this
    // one is computed (rows past T are read clamped and not stored).
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    auto ldx = [&](int t) {
        const v4u a = __builtin_nontemporal_load(
            reinterpret_cast<const v4u *>(x + (size_t)min(t, T - 1) * C + ch0));
        return make_uint4(a.x, a.y, a.z, a.w);
    };
    uint4 buf[2][kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) buf[0][i] = ldx(t0 + i);
#pragma unroll
    for (int bi = 0; bi < kRun / kBatch; ++bi) {
        const int cur = bi & 1;
        if (bi + 1 < kRun / kBatch) {
#pragma unroll
            for (int i = 0; i < kBatch; ++i) buf[cur ^ 1][i] = ldx(t0 + (bi + 1) * kBatch + i);
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int t = t0 + bi * kBatch + i;
            if (t >= t1) break;
            float cur_x[8];
            unpack8(buf[cur][i], cur_x);
            if (cu_seqlens && t >= s1) {               // a new sequence starts at t
                while (n + 1 < N && cu_seqlens[n + 1] <= t) ++n;
                s1 = cu_seqlens[n + 1];
#pragma unroll
                for (int j = 0; j < 3; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
            }
            float y[8];
            float ss = 0.f;
            conv_silu8(wt, win[0], win[1], win[2], cur_x, y, ss);
            if (normalise) {
                const float r = rsqrtf(row16_sum(ss) + eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] *= r;
            }
            const uint4 pv = pack_bf8(y);
            __builtin_nontemporal_store(v4u{pv.x, pv.y, pv.z, pv.w},
                                        reinterpret_cast<v4u *>(dst + (size_t)t * dst_stride));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                win[0][e] = win[1][e];
                win[1][e] = win[2][e];
                win[2][e] = cur_x[e];
            }
        }
    }
}

}  // namespace

hipError_t launch_conv_prelude(const void *x, const void *w, const int32_t *cu_seqlens, int N,
                               int T, int H_qk, int H_v, float eps, void *q, void *k, void *v,
                               hipStream_t stream) {
    const int n_blocks = 2 * H_qk + H_v;
    dim3 grid((T + kRun - 1) / kRun, (n_blocks + kGroupsPerBlock - 1) / kGroupsPerBlock);
    hipLaunchKernelGGL(conv_prelude_kernel, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w),
                       cu_seqlens, N, T, H_qk, H_v, eps, static_cast<uint16_t *>(q),
                       static_cast<uint16_t *>(k), static_cast<uint16_t *>(v));
    return hipGetLastError();
}

}  // namespace gdn
