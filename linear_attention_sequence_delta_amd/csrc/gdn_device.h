// gdn_device.h -- device helpers shared by the gfx950 kernels of libgdn.
// Internal header: not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    return uint32_t(f2bf(lo)) | (uint32_t(f2bf(hi)) << 16);
}

// Sum over each aligned group of 16 lanes (one DPP row); every lane of the row
// receives the row's total.  quad_perm(1,0,3,2), quad_perm(2,3,0,1),
// row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
    return x;
}

// 8 bf16 (one 16-byte piece) -> fp32.
__device__ __forceinline__ void unpack8(uint4 u, float *d) {
    d[0] = __uint_as_float(u.x << 16); d[1] = __uint_as_float(u.x & 0xFFFF0000u);
    d[2] = __uint_as_float(u.y << 16); d[3] = __uint_as_float(u.y & 0xFFFF0000u);
    d[4] = __uint_as_float(u.z << 16); d[5] = __uint_as_float(u.z & 0xFFFF0000u);
    d[6] = __uint_as_float(u.w << 16); d[7] = __uint_as_float(u.w & 0xFFFF0000u);
}

__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Conv prelude arithmetic, shared by every kernel that applies it so that all
// of them produce the same bits.  wt[j][e] is tap j of channel e (tap 3 on the
// current token); xm3, xm2, xm1, x0 are the inputs 3, 2, 1 and 0 tokens back.
// y = SiLU(conv); ss accumulates y^2 over the 8 channels, in channel order.
__device__ __forceinline__ void conv_silu8(const float (&wt)[4][8], const float *xm3,
                                           const float *xm2, const float *xm1, const float *x0,
                                           float *y, float &ss) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float acc = wt[3][e] * x0[e];
        acc = __builtin_fmaf(wt[2][e], xm1[e], acc);
        acc = __builtin_fmaf(wt[1][e], xm2[e], acc);
        acc = __builtin_fmaf(wt[0][e], xm3[e], acc);
        y[e] = silu(acc);
        ss = __builtin_fmaf(y[e], y[e], ss);
    }
}

// The 4 conv taps of 8 consecutive channels starting at channel ch:
// w is [channels][4] bf16; wt[j][e] = w[ch + e][j].
__device__ __forceinline__ void load_taps8(const uint16_t *w, size_t ch, float (&wt)[4][8]) {
    const uint4 *wp = reinterpret_cast<const uint4 *>(w + ch * 4);
    float tmp[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack8(wp[i], tmp + 8 * i);
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) wt[j][e] = tmp[e * 4 + j];
}

__device__ __forceinline__ uint4 pack_bf8(const float *y) {
    uint4 out;
    out.x = pack_bf2(y[0], y[1]);
    out.y = pack_bf2(y[2], y[3]);
    out.z = pack_bf2(y[4], y[5]);
    out.w = pack_bf2(y[6], y[7]);
    return out;
}

// The output gate on one 128-wide row held by a 16-lane DPP row (8 channels,
// one 16-byte piece of o and of z per lane; wv the norm weight of the lane's
// channels): y = o / sqrt(mean(o^2) + eps) * w * SiLU(z).  Every lane of the
// row must be active.  Shared by every kernel that applies the gate.
__device__ __forceinline__ uint4 gate_row8(uint4 o8, uint4 z8, const float (&wv)[8], float eps) {
    float ov[8], zv[8];
    unpack8(o8, ov);
    unpack8(z8, zv);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(ov[e], ov[e], ss);
    const float inv = rsqrtf(row16_sum(ss) * (1.f / 128) + eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = ov[e] * inv * wv[e] * silu(zv[e]);
    return pack_bf8(y);
}

// Gates from the raw per-token projections a, b of a V-head and the layer's
// A_log, dt_bias: log decay g = -softplus(a + dt_bias) * exp(A_log) (softplus
// written max(x, 0) + log1p(exp(-|x|)), which cannot overflow) and write
// strength beta = sigmoid(b).  Shared by every kernel that forms gates.
__device__ __forceinline__ float gate_log_decay(float a, float A_log, float dt_bias) {
    const float x = a + dt_bias;
    const float softplus = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
    return -softplus * expf(A_log);
}
__device__ __forceinline__ float gate_beta(float b) { return 1.f / (1.f + expf(-b)); }

// Load 4 consecutive values (bf16 bits or fp32) as fp32.
__device__ __forceinline__ void load4(const uint16_t *p, float *d) {
    uint2 u = *reinterpret_cast<const uint2 *>(p);
    d[0] = __uint_as_float(u.x << 16);
    d[1] = __uint_as_float(u.x & 0xFFFF0000u);
    d[2] = __uint_as_float(u.y << 16);
    d[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const float *p, float *d) {
    float4 u = *reinterpret_cast<const float4 *>(p);
    d[0] = u.x; d[1] = u.y; d[2] = u.z; d[3] = u.w;
}
__device__ __forceinline__ float load1(const uint16_t *p) { return bf2f(*p); }
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ void store1(uint16_t *p, float x) { *p = f2bf(x); }
__device__ __forceinline__ void store1(float *p, float x) { *p = x; }

}  // namespace gdn
