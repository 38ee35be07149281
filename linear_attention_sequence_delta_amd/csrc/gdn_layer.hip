// gdn_layer.hip -- the pieces that turn the kernels into the layer's forward
// from its raw projections ("从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力",
// sec. 2.1: the conv1d.weight, A_log and dt_bias weights of each linear-attention
// layer):
//   gates_kernel       g = -softplus(a + dt_bias) exp(A_log), beta = sigmoid(b)
//   conv_hist_kernel   each sequence's last three raw rows (its conv history for
//                      the next token), zero where the sequence is shorter
//   conv_shift_kernel  after a decode step: a slot's history drops its oldest
//                      row and takes the new token's row
//   gated_norm_kernel  the output gate: each (token, V-head) row of o divided
//                      by its root mean square, times the norm weight and
//                      SiLU(z) (the pages list the norm and in_proj_z
//                      weights; this is the reading taken of how they apply)
// All are elementwise copies or maps, HBM-bound; rows move in 16-byte pieces.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

__global__ __launch_bounds__(256) void gates_kernel(const float *__restrict__ a,
                                                    const float *__restrict__ b,
                                                    const float *__restrict__ A_log,
                                                    const float *__restrict__ dt_bias, int T,
                                                    int H_v, float *__restrict__ g,
                                                    float *__restrict__ beta) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * H_v) return;
    const int h = (int)(i % H_v);
    g[i] = gate_log_decay(a[i], A_log[h], dt_bias[h]);
    beta[i] = gate_beta(b[i]);
}

// grid (pieces per row / 256, N): piece p of sequence n's three history rows.
// Row j is raw row s1 - 3 + j, or, before the sequence start, row L + j of
// its incoming history (zero without one); each thread reads its three
// values before writing any, so hist_out may be hist_in.
__global__ __launch_bounds__(256) void conv_hist_kernel(const uint16_t *__restrict__ x,
                                                        const int32_t *__restrict__ cu, int T,
                                                        int pieces, const uint16_t *hist_in,
                                                        uint16_t *hist_out) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= pieces) return;
    const int n = blockIdx.y;
    const int s0 = cu ? cu[n] : 0, s1 = cu ? cu[n + 1] : T;
    uint4 val[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int t = s1 - 3 + j;
        val[j] = make_uint4(0, 0, 0, 0);
        if (t >= s0)
            val[j] = reinterpret_cast<const uint4 *>(x)[(size_t)t * pieces + p];
        else if (hist_in)
            val[j] = reinterpret_cast<const uint4 *>(hist_in)[((size_t)n * 3 + 3 + (t - s0)) * pieces + p];
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) reinterpret_cast<uint4 *>(hist_out)[((size_t)n * 3 + j) * pieces + p] = val[j];
}

// grid (pieces per row / 256, B): slot_idx[b]'s history <- rows 1, 2, x[b]
__global__ __launch_bounds__(256) void conv_shift_kernel(const uint16_t *__restrict__ x,
                                                         const int32_t *__restrict__ slot_idx,
                                                         int pieces, uint16_t *__restrict__ hist) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= pieces) return;
    const int b = blockIdx.y;
    uint4 *hs = reinterpret_cast<uint4 *>(hist) + (size_t)slot_idx[b] * 3 * pieces + p;
    const uint4 r1 = hs[pieces], r2 = hs[2 * (size_t)pieces];
    const uint4 xn = reinterpret_cast<const uint4 *>(x)[(size_t)b * pieces + p];
    hs[0] = r1;
    hs[pieces] = r2;
    hs[2 * (size_t)pieces] = xn;
}

// 16 lanes per 128-channel row (8 channels each), the sum of squares reduced
// over the 16-lane DPP row; 16 rows per 256-thread workgroup.  out may be o.
__global__ __launch_bounds__(256) void gated_norm_kernel(const uint16_t *o,
                                                         const uint16_t *__restrict__ z,
                                                         const float *__restrict__ w, int rows,
                                                         float eps, uint16_t *out) {
    const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int cg = threadIdx.x & 15;
    const int rr = min(row, rows - 1);              // a whole DPP row stays active
    const size_t off = (size_t)rr * kD + 8 * cg;
    // o and z are read once and out written once: non-temporal accesses
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u oa = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(o + off));
    const v4u za = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(z + off));
    const float4 w0 = *reinterpret_cast<const float4 *>(w + 8 * cg);
    const float4 w1 = *reinterpret_cast<const float4 *>(w + 8 * cg + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const uint4 pv = gate_row8(make_uint4(oa.x, oa.y, oa.z, oa.w), make_uint4(za.x, za.y, za.z, za.w), wv, eps);
    if (row < rows)
        __builtin_nontemporal_store(v4u{pv.x, pv.y, pv.z, pv.w}, reinterpret_cast<v4u *>(out + off));
}

}  // namespace

hipError_t launch_gated_norm(const void *o, const void *z, const float *w, int rows, float eps,
                             void *out, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(gated_norm_kernel, dim3((rows + 15) / 16), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(o), static_cast<const uint16_t *>(z), w,
                       rows, eps, static_cast<uint16_t *>(out));
    return hipGetLastError();
}

hipError_t launch_gates(const float *a, const float *b, const float *A_log, const float *dt_bias,
                        int T, int H_v, float *g, float *beta, hipStream_t stream) {
    const size_t n = (size_t)T * H_v;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(gates_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a, b,
                       A_log, dt_bias, T, H_v, g, beta);
    return hipGetLastError();
}

hipError_t launch_conv_hist(const void *x, const int32_t *cu_seqlens, int N, int T, int C_raw,
                            const void *hist_in, void *hist_out, hipStream_t stream) {
    const int pieces = C_raw / 8;
    hipLaunchKernelGGL(conv_hist_kernel, dim3((pieces + 255) / 256, N), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(x), cu_seqlens, T, pieces,
                       static_cast<const uint16_t *>(hist_in), static_cast<uint16_t *>(hist_out));
    return hipGetLastError();
}

hipError_t launch_conv_shift(const void *x, const int32_t *slot_idx, int B, int C_raw, void *hist,
                             hipStream_t stream) {
    const int pieces = C_raw / 8;
    if (B == 0) return hipSuccess;
    hipLaunchKernelGGL(conv_shift_kernel, dim3((pieces + 255) / 256, B), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(x), slot_idx, pieces,
                       static_cast<uint16_t *>(hist));
    return hipGetLastError();
}

}  // namespace gdn
