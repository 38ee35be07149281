// gdn_layer_bwd.hip -- gradients of the layer's steps before the recurrence:
// the conv prelude (width-4 causal depthwise conv, SiLU, L2 norm of the q and
// k heads) and the gates, for training the layer from its raw projections
// ("从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力", sec. 2.1:
// the conv1d.weight, A_log and dt_bias weights; the fused forward/backward GDN
// kernel named in "Qwen3.8-27B：27B 如何打出千亿级效果，且塞进单张消费级显卡",
// sec. 2.1).
//
// Per token and channel, with y the conv output, a = SiLU(y) and, for a q or
// k head, n = a r with r = (sum a^2 + eps)^(-1/2):
//   da = r (dn - n (n . dn))  (v channels: da = dv)
//   dy = da sigmoid(y) (1 + y (1 - sigmoid(y)))
//   dx[s] = w3 dy[s] + w2 dy[s+1] + w1 dy[s+2] + w0 dy[s+3]   (same sequence)
//   dw[j] = sum_t x[t - 3 + j] dy[t]
// and for the gates g = -softplus(a + dt_bias) exp(A_log), beta = sigmoid(b):
//   da = -dg exp(A_log) sigmoid(a + dt_bias),  ddt_bias = sum_t da,
//   dA_log = sum_t dg g,  db = dbeta beta (1 - beta).
// The output gate after the recurrence (y = o r w SiLU(z) per (token, V-head)
// row, r = (mean o^2 + eps)^(-1/2), the reading taken of the norm and in_proj_z
// weights the first page lists) has, with n = o r, s = SiLU(z), u = dy w s:
//   do = r (u - n mean(u n)),  dz = dy n w SiLU'(z),  dw = sum over rows dy n s.
// All HBM-bound elementwise work; the sums over tokens go through per-run
// partials reduced in a fixed order (no atomics: results are reproducible).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kRunB = 128;         // tokens walked by one lane group
constexpr int kGroupsPerBlockB = 16;

// The prelude kernel's lane layout: 16 lanes own one 128-channel head block
// (8 channels each) and walk the tokens [t0, t0 + kRunB), recomputing the
// forward with its arithmetic; dx of token s is complete once dy of s + 3 is
// known, so the walk runs three tokens past its run (dy only).  Per-run
// partial sums of dw go to partial [run][C_raw][4].
__global__ __launch_bounds__(256) void prelude_bwd_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    const int32_t *__restrict__ cu_seqlens, int N, int T, int H_qk, int H_v, float eps,
    const uint16_t *__restrict__ dq, const uint16_t *__restrict__ dk,
    const uint16_t *__restrict__ dv, uint16_t *__restrict__ dx, float *__restrict__ partial) {
    const int lane = threadIdx.x & 63;
    const int c16 = lane & 15;
    const int grp = threadIdx.x >> 4;
    const int n_blocks = 2 * H_qk + H_v;
    const int cb = blockIdx.y * kGroupsPerBlockB + grp;
    if (cb >= n_blocks) return;                        // whole 16-lane groups leave together
    const int t0 = blockIdx.x * kRunB;
    const int t1 = min(T, t0 + kRunB);
    const int C = n_blocks * kD;
    const int ch0 = cb * kD + c16 * 8;

    float wt[4][8];
    load_taps8(w, (size_t)ch0, wt);

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
    const uint16_t *dn_base;
    int dn_stride;
    if (cb < H_qk) {
        dn_base = dq + (size_t)cb * kD + c16 * 8;
        dn_stride = H_qk * kD;
    } else if (cb < 2 * H_qk) {
        dn_base = dk + (size_t)(cb - H_qk) * kD + c16 * 8;
        dn_stride = H_qk * kD;
    } else {
        dn_base = dv + (size_t)(cb - 2 * H_qk) * kD + c16 * 8;
        dn_stride = H_v * kD;
    }
    const bool normalise = cb < 2 * H_qk;

    float dyw[3][8];                                   // dy of tokens t-3, t-2, t-1
    int endw[3] = {0, 0, 0};                           // end of their sequences
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) dyw[j][e] = 0.f;
    float dwacc[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) dwacc[j][e] = 0.f;

    const int t_end = t1 + 3;
    for (int t = t0; t < t_end; ++t) {
        float dy[8];
        int end_t = s1;
        if (t < T) {
            float cur[8];
            unpack8(*reinterpret_cast<const uint4 *>(x + (size_t)t * C + ch0), cur);
            if (cu_seqlens && t >= s1) {               // a new sequence starts at t
                while (n + 1 < N && cu_seqlens[n + 1] <= t) ++n;
                s1 = cu_seqlens[n + 1];
#pragma unroll
                for (int j = 0; j < 3; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
            }
            end_t = s1;
            // the forward's conv, SiLU and norm, in its order
            float yc[8], a[8], ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = wt[3][e] * cur[e];
                acc = __builtin_fmaf(wt[2][e], win[2][e], acc);
                acc = __builtin_fmaf(wt[1][e], win[1][e], acc);
                acc = __builtin_fmaf(wt[0][e], win[0][e], acc);
                yc[e] = acc;
                a[e] = silu(acc);
                ss = __builtin_fmaf(a[e], a[e], ss);
            }
            float dn[8];
            unpack8(*reinterpret_cast<const uint4 *>(dn_base + (size_t)t * dn_stride), dn);
            float da[8];
            if (normalise) {
                const float r = rsqrtf(row16_sum(ss) + eps);
                float nd = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) nd = __builtin_fmaf(a[e] * r, dn[e], nd);
                nd = row16_sum(nd);
#pragma unroll
                for (int e = 0; e < 8; ++e) da[e] = r * (dn[e] - a[e] * r * nd);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) da[e] = dn[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // the same reciprocal as silu(), so the exponential and the
                // reciprocal are shared with the recomputed forward
                const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-yc[e]));
                dy[e] = da[e] * sg * (1.f + yc[e] * (1.f - sg));
            }
            if (t < t1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    dwacc[3][e] = __builtin_fmaf(cur[e], dy[e], dwacc[3][e]);
                    dwacc[2][e] = __builtin_fmaf(win[2][e], dy[e], dwacc[2][e]);
                    dwacc[1][e] = __builtin_fmaf(win[1][e], dy[e], dwacc[1][e]);
                    dwacc[0][e] = __builtin_fmaf(win[0][e], dy[e], dwacc[0][e]);
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                win[0][e] = win[1][e];
                win[1][e] = win[2][e];
                win[2][e] = cur[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) dy[e] = 0.f;
        }
        // dx of token s = t - 3 (taps of later tokens of the same sequence)
        const int s = t - 3;
        if (s >= t0) {
            const int es = endw[0];
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = wt[3][e] * dyw[0][e];
                if (s + 1 < es) acc = __builtin_fmaf(wt[2][e], dyw[1][e], acc);
                if (s + 2 < es) acc = __builtin_fmaf(wt[1][e], dyw[2][e], acc);
                if (s + 3 < es) acc = __builtin_fmaf(wt[0][e], dy[e], acc);
                o[e] = acc;
            }
            *reinterpret_cast<uint4 *>(dx + (size_t)s * C + ch0) = pack_bf8(o);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            dyw[0][e] = dyw[1][e];
            dyw[1][e] = dyw[2][e];
            dyw[2][e] = dy[e];
        }
        endw[0] = endw[1];
        endw[1] = endw[2];
        endw[2] = end_t;
    }
    float4 *pp = reinterpret_cast<float4 *>(partial + ((size_t)blockIdx.x * C + ch0) * 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) pp[e] = make_float4(dwacc[0][e], dwacc[1][e], dwacc[2][e], dwacc[3][e]);
}

// dw[i] = sum over runs of partial[run][i]: wave j of a workgroup takes the
// runs r = j mod 4 for 64 consecutive i, spread over eight running sums (run
// r + 4 k of each group of 32 into sum k, the leftover runs into sum 0) so
// that eight loads are in flight; the sums and then the four waves are added
// in a fixed order.
__global__ __launch_bounds__(256) void sum_runs_kernel(const float *__restrict__ partial, int runs,
                                                       int n, float *__restrict__ out) {
    __shared__ float part[4][64];
    const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int i = blockIdx.x * 64 + lane;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (i < n) {
        int r = j;
        for (; r + 28 < runs; r += 32) {
#pragma unroll
            for (int k = 0; k < 8; ++k) a[k] += partial[(size_t)(r + 4 * k) * n + i];
        }
        for (; r < runs; r += 4) a[0] += partial[(size_t)r * n + i];
    }
    part[j][lane] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    __syncthreads();
    if (j == 0 && i < n) out[i] = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
}

__global__ __launch_bounds__(256) void gates_bwd_kernel(const float *__restrict__ a,
                                                        const float *__restrict__ b,
                                                        const float *__restrict__ A_log,
                                                        const float *__restrict__ dt_bias,
                                                        const float *__restrict__ dg,
                                                        const float *__restrict__ dbeta, int T,
                                                        int H_v, float *__restrict__ da,
                                                        float *__restrict__ db) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * H_v) return;
    const int h = (int)(i % H_v);
    const float sg = 1.f / (1.f + expf(-(a[i] + dt_bias[h])));
    da[i] = -dg[i] * expf(A_log[h]) * sg;
    const float be = gate_beta(b[i]);
    db[i] = dbeta[i] * be * (1.f - be);
}

// Workgroup (h, split): over the tokens of its split, dA_log = sum_t dg g and
// ddt_bias = sum_t da for V-head h (the gates recomputed as the forward forms
// them), into partial [split][H_v][2]; gates_sum_splits_kernel adds the
// splits.  Fixed order throughout.
constexpr int kGateSplits = 32;
__global__ __launch_bounds__(256) void gates_bwd_sum_kernel(const float *__restrict__ a,
                                                            const float *__restrict__ A_log,
                                                            const float *__restrict__ dt_bias,
                                                            const float *__restrict__ dg, int T,
                                                            int H_v, float *__restrict__ partial) {
    __shared__ float part[2][256];
    const int h = blockIdx.x, sp = blockIdx.y;
    const int ts = (int)((long long)T * sp / kGateSplits), te = (int)((long long)T * (sp + 1) / kGateSplits);
    const float al = A_log[h], dtb = dt_bias[h], ea = expf(al);
    float s1 = 0.f, s2 = 0.f;
    for (int t = ts + threadIdx.x; t < te; t += 256) {
        const size_t i = (size_t)t * H_v + h;
        const float g = gate_log_decay(a[i], al, dtb);
        s1 = __builtin_fmaf(dg[i], g, s1);
        s2 -= dg[i] * ea * (1.f / (1.f + expf(-(a[i] + dtb))));
    }
    part[0][threadIdx.x] = s1;
    part[1][threadIdx.x] = s2;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) {
            part[0][threadIdx.x] += part[0][threadIdx.x + off];
            part[1][threadIdx.x] += part[1][threadIdx.x + off];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        partial[((size_t)sp * H_v + h) * 2] = part[0][0];
        partial[((size_t)sp * H_v + h) * 2 + 1] = part[1][0];
    }
}

__global__ __launch_bounds__(64) void gates_sum_splits_kernel(const float *__restrict__ partial,
                                                              int H_v, float *__restrict__ dA_log,
                                                              float *__restrict__ ddt_bias) {
    const int h = blockIdx.x * 64 + threadIdx.x;
    if (h >= H_v) return;
    float s1 = 0.f, s2 = 0.f;
    for (int sp = 0; sp < kGateSplits; ++sp) {
        s1 += partial[((size_t)sp * H_v + h) * 2];
        s2 += partial[((size_t)sp * H_v + h) * 2 + 1];
    }
    dA_log[h] = s1;
    ddt_bias[h] = s2;
}

// Output gate: 16 lanes per 128-channel row (8 channels each, the forward's
// layout), 16 rows per step of a 256-thread workgroup, two steps' rows loaded
// before either is computed, the grid striding over the rows; each
// workgroup's share of dw goes to partial [block][128].  The rows are read
// and written once, with non-temporal loads and stores.
constexpr int kGateNormBlocks = 512;
constexpr int kGateNormSteps = 2;
__global__ __launch_bounds__(256) void gated_norm_bwd_kernel(
    const uint16_t *__restrict__ o, const uint16_t *__restrict__ z, const float *__restrict__ w,
    const uint16_t *__restrict__ dy, int rows, float eps, uint16_t *__restrict__ d_o,
    uint16_t *__restrict__ dz, float *__restrict__ partial) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    __shared__ float part[16][kD];
    const int cg = threadIdx.x & 15, rg = threadIdx.x >> 4;
    const float4 w0 = *reinterpret_cast<const float4 *>(w + 8 * cg);
    const float4 w1 = *reinterpret_cast<const float4 *>(w + 8 * cg + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto ld = [](const uint16_t *p) {
        const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
        return make_uint4(x.x, x.y, x.z, x.w);
    };
    auto st = [](uint16_t *p, uint4 x) {
        __builtin_nontemporal_store(v4u{x.x, x.y, x.z, x.w}, reinterpret_cast<v4u *>(p));
    };
    for (int base = blockIdx.x * 16 * kGateNormSteps; base < rows; base += gridDim.x * 16 * kGateNormSteps) {
        uint4 ou[kGateNormSteps], zu[kGateNormSteps], gu[kGateNormSteps];
#pragma unroll
        for (int u = 0; u < kGateNormSteps; ++u) {
            const size_t off = (size_t)min(base + 16 * u + rg, rows - 1) * kD + 8 * cg;   // whole DPP rows stay active
            ou[u] = ld(o + off);
            zu[u] = ld(z + off);
            gu[u] = ld(dy + off);
        }
#pragma unroll
        for (int u = 0; u < kGateNormSteps; ++u) {
            const int row = base + 16 * u + rg;
            const bool ok = row < rows;
            const size_t off = (size_t)min(row, rows - 1) * kD + 8 * cg;
            float ov[8], zv[8], gv[8];
            unpack8(ou[u], ov);
            unpack8(zu[u], zv);
            unpack8(gu[u], gv);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(ov[e], ov[e], ss);
            const float inv = rsqrtf(row16_sum(ss) * (1.f / kD) + eps);
            float n[8], sg[8], uu[8], un = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                n[e] = ov[e] * inv;
                sg[e] = __builtin_amdgcn_rcpf(1.f + __expf(-zv[e]));
                uu[e] = gv[e] * wv[e] * (zv[e] * sg[e]);
                un = __builtin_fmaf(uu[e], n[e], un);
            }
            const float m = row16_sum(un) * (1.f / kD);
            float go[8], gz[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                go[e] = inv * (uu[e] - n[e] * m);
                gz[e] = gv[e] * n[e] * wv[e] * sg[e] * (1.f + zv[e] * (1.f - sg[e]));
                if (ok) acc[e] = __builtin_fmaf(gv[e] * n[e], zv[e] * sg[e], acc[e]);
            }
            if (ok) {
                st(d_o + off, pack_bf8(go));
                st(dz + off, pack_bf8(gz));
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg][8 * cg + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < kD) {
        float s = 0.f;
        for (int r = 0; r < 16; ++r) s += part[r][threadIdx.x];
        partial[(size_t)blockIdx.x * kD + threadIdx.x] = s;
    }
}

}  // namespace

size_t gated_norm_bwd_partial_bytes(int rows) {
    const int blocks = max(1, min(kGateNormBlocks, (rows + 16 * kGateNormSteps - 1) / (16 * kGateNormSteps)));
    return (size_t)blocks * kD * sizeof(float);
}

hipError_t launch_gated_norm_bwd(const void *o, const void *z, const float *w, const void *dy,
                                 int rows, float eps, void *d_o, void *dz, float *dw,
                                 float *partial, hipStream_t stream) {
    const int blocks = max(1, min(kGateNormBlocks, (rows + 16 * kGateNormSteps - 1) / (16 * kGateNormSteps)));
    if (rows > 0) {
        hipLaunchKernelGGL(gated_norm_bwd_kernel, dim3(blocks), dim3(256), 0, stream,
                           static_cast<const uint16_t *>(o), static_cast<const uint16_t *>(z), w,
                           static_cast<const uint16_t *>(dy), rows, eps, static_cast<uint16_t *>(d_o),
                           static_cast<uint16_t *>(dz), partial);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sum_runs_kernel, dim3((kD + 63) / 64), dim3(256), 0, stream, partial,
                       rows > 0 ? blocks : 0, kD, dw);
    return hipGetLastError();
}

size_t gates_bwd_partial_bytes(int H_v) { return (size_t)kGateSplits * H_v * 2 * sizeof(float); }

size_t prelude_bwd_partial_bytes(int T, int H_qk, int H_v) {
    const size_t runs = (size_t)(T + kRunB - 1) / kRunB;
    return runs * (size_t)(2 * H_qk + H_v) * kD * 4 * sizeof(float);
}

hipError_t launch_prelude_bwd(const void *x, const void *w, const int32_t *cu_seqlens, int N, int T,
                              int H_qk, int H_v, float eps, const void *dq, const void *dk,
                              const void *dv, void *dx, float *dw, float *partial,
                              hipStream_t stream) {
    const int n_blocks = 2 * H_qk + H_v;
    const int runs = (T + kRunB - 1) / kRunB;
    const int nw = n_blocks * kD * 4;
    if (runs > 0) {
        dim3 grid(runs, (n_blocks + kGroupsPerBlockB - 1) / kGroupsPerBlockB);
        hipLaunchKernelGGL(prelude_bwd_kernel, grid, dim3(256), 0, stream,
                           static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w),
                           cu_seqlens, N, T, H_qk, H_v, eps, static_cast<const uint16_t *>(dq),
                           static_cast<const uint16_t *>(dk), static_cast<const uint16_t *>(dv),
                           static_cast<uint16_t *>(dx), partial);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sum_runs_kernel, dim3((nw + 63) / 64), dim3(256), 0, stream, partial, runs,
                       nw, dw);
    return hipGetLastError();
}

hipError_t launch_gates_bwd(const float *a, const float *b, const float *A_log,
                            const float *dt_bias, const float *dg, const float *dbeta, int T,
                            int H_v, float *da, float *db, float *dA_log, float *ddt_bias,
                            float *partial, hipStream_t stream) {
    const size_t n = (size_t)T * H_v;
    if (n > 0) {
        hipLaunchKernelGGL(gates_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                           a, b, A_log, dt_bias, dg, dbeta, T, H_v, da, db);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(gates_bwd_sum_kernel, dim3(H_v, kGateSplits), dim3(256), 0, stream, a, A_log,
                       dt_bias, dg, T, H_v, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gates_sum_splits_kernel, dim3((H_v + 63) / 64), dim3(64), 0, stream, partial,
                       H_v, dA_log, ddt_bias);
    return hipGetLastError();
}

}  // namespace gdn
