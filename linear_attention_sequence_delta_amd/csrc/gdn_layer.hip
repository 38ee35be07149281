// gdn_layer.hip -- the pieces that turn the kernels into the layer's forward
// from its raw projections ("从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力",
// sec. 2.1: the conv1d.weight, A_log and dt_bias weights of each linear-attention
// layer):
//   gates_kernel       g = -softplus(a + dt_bias) exp(A_log), beta = sigmoid(b)
//   conv_hist_kernel   each sequence's last three raw rows (its conv history for
//                      the next token), zero where the sequence is shorter
//   conv_shift_kernel  after a decode step: a slot's history drops its oldest
//                      row and takes the new token's row
// All three are elementwise copies or maps, HBM-bound and tiny next to the
// prefill and the decode step; rows move in 16-byte pieces.
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

// grid (pieces per row / 256, 3, N): row j of sequence n's history
__global__ __launch_bounds__(256) void conv_hist_kernel(const uint16_t *__restrict__ x,
                                                        const int32_t *__restrict__ cu, int T,
                                                        int pieces, uint16_t *__restrict__ hist) {
    const int p = blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= pieces) return;
    const int j = blockIdx.y, n = blockIdx.z;
    const int s0 = cu ? cu[n] : 0, s1 = cu ? cu[n + 1] : T;
    const int t = s1 - 3 + j;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (t >= s0) val = reinterpret_cast<const uint4 *>(x)[(size_t)t * pieces + p];
    reinterpret_cast<uint4 *>(hist)[((size_t)n * 3 + j) * pieces + p] = val;
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

}  // namespace

hipError_t launch_gates(const float *a, const float *b, const float *A_log, const float *dt_bias,
                        int T, int H_v, float *g, float *beta, hipStream_t stream) {
    const size_t n = (size_t)T * H_v;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(gates_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a, b,
                       A_log, dt_bias, T, H_v, g, beta);
    return hipGetLastError();
}

hipError_t launch_conv_hist(const void *x, const int32_t *cu_seqlens, int N, int T, int C_raw,
                            void *hist, hipStream_t stream) {
    const int pieces = C_raw / 8;
    hipLaunchKernelGGL(conv_hist_kernel, dim3((pieces + 255) / 256, 3, N), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(x), cu_seqlens, T, pieces,
                       static_cast<uint16_t *>(hist));
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
