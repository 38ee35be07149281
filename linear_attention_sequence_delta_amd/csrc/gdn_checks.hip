// gdn_checks.hip -- device-side precondition checks used when GDN_DEBUG=1.
// A single workgroup scans the index array and records the first violation in
// a file-scope device flag; the host reads the flag after synchronising.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

__device__ int g_check_flag;

// cu_seqlens must start at 0, end at T and never decrease.
__global__ void check_cu_kernel(const int32_t *cu, int N, int T) {
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    for (int i = threadIdx.x; i <= N; i += blockDim.x) {
        const int c = cu[i];
        if ((i == 0 && c != 0) || (i == N && c != T) || (i > 0 && c < cu[i - 1]) || c < 0 || c > T)
            atomicOr(&bad, 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) g_check_flag = bad;
}

// slot ids must lie in [0, P) and be pairwise distinct (quadratic scan; debug only).
__global__ void check_slots_kernel(const int32_t *slot, int B, int P) {
    __shared__ int bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
        const int s = slot[i];
        if (s < 0 || s >= P) atomicOr(&bad, 2);
        for (int j = i + 1; j < B; ++j)
            if (slot[j] == s) atomicOr(&bad, 4);
    }
    __syncthreads();
    if (threadIdx.x == 0) g_check_flag = bad;
}

}  // namespace

hipError_t debug_check_cu_seqlens(const int32_t *cu_seqlens, int N, int T, hipStream_t stream,
                                  int *result) {
    hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, stream, cu_seqlens, N, T);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipMemcpyFromSymbol(result, HIP_SYMBOL(g_check_flag), sizeof(int));
    return e;
}

hipError_t debug_check_slots(const int32_t *slot_idx, int B, int P, hipStream_t stream,
                             int *result) {
    hipLaunchKernelGGL(check_slots_kernel, dim3(1), dim3(256), 0, stream, slot_idx, B, P);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e == hipSuccess) e = hipMemcpyFromSymbol(result, HIP_SYMBOL(g_check_flag), sizeof(int));
    return e;
}

}  // namespace gdn
