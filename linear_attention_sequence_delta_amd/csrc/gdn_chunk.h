// gdn_chunk.h -- device helpers and layouts shared by the chunked kernels
// (forward prefill and its backward).  Internal header: not installed, not
// part of the ABI.
#pragma once

#include <stdint.h>

#include "gdn_device.h"

namespace gdn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 8 bf16, kept in registers without copies

constexpr int kKP = kD + 8;          // LDS row stride (bf16) of 128-wide rows
constexpr int kAP = kChunk + 4;      // LDS row stride (fp32) of 64-wide rows
constexpr int kRP = kChunk + 8;      // LDS row stride (bf16) of 64-wide rows
constexpr int kTileElems = kChunk * kChunk;   // one 64 x 64 bf16 matrix

template <class A, class B>
__device__ __forceinline__ f32x4 mfma32(A a, B b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 to_bf4(float a, float b, float c, float d) {
    s16x4 r;
    r[0] = (short)f2bf(a);
    r[1] = (short)f2bf(b);
    r[2] = (short)f2bf(c);
    r[3] = (short)f2bf(d);
    return r;
}
// fp32 -> bf16 (round to nearest even), two or four at a time
__device__ __forceinline__ uint32_t pk2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
}
__device__ __forceinline__ uint2 pk4(float a, float b, float c, float d) {
    return make_uint2(pk2(a, b), pk2(c, d));
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// if lane q points at row (r0 + q / 4), columns c0 + 4 (q % 4) .. + 3 of a
// row-major bf16 matrix, lane p receives column c0 + p, rows r0 .. r0 + 3:
// a 16 x 4 block read transposed.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *p) {
    typedef short s4v __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4v lds_s4v;
    const s4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s4v *)(__attribute__((address_space(3))) uint16_t *)p);
    return __builtin_bit_cast(uint2, r);
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ float wave_scan(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Make this wave's earlier LDS writes visible to its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

struct ChunkRange { int n, c0, len; };

// Largest n with chunk_base[n] <= gc (sequences with no chunks are skipped).
__device__ __forceinline__ int seq_of_chunk(const int32_t *chunk_base, int N, int gc) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_base[mid] <= gc) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Workspace record of one (chunk, V-head) of the forward prefill: T', then P,
// then the decays gamma_r = exp(G_r) and lambda_r = exp(G_L - G_r) as 64 fp32
// each (G the chunk's cumulative log decay, G_L its last row's; rows past a
// sequence's end repeat G_L).  T' and P (bf16 64 x 64)
// are stored as MFMA operand fragments: block (a, s) = 2 a + s holds, for lane
// (c, g4), the 16 bytes of row 16 a + c, columns 32 s + 8 g4 .. +7, lanes in
// order -- so a kernel loads each fragment as one contiguous 1 KiB block.  (A
// fragment read from a row-major tile would touch half of 16 cache lines,
// which halves the rate the vector memory pipe delivers.)
constexpr int kRecElems = 2 * kTileElems + 4 * kChunk;   // in bf16 units (16896 bytes)
constexpr int kRecGam = 2 * kTileElems;                  // gamma (fp32), then lambda
__device__ __forceinline__ int frag_off(int a, int s, int lane) { return ((2 * a + s) * 64 + lane) * 8; }

// Record of one (chunk, V-head) for the backward pass: the fragments of T'^T
// and P^T (same block layout as above, of the transposed matrices), T itself
// row-major (64 x 64 bf16, zero above the diagonal), then G as 64 fp32.
constexpr int kBwdRecElems = 3 * kTileElems + 2 * kChunk;   // in bf16 units (24832 bytes)
constexpr int kBwdTtOff = 0;                     // T'^T fragments
constexpr int kBwdPtOff = kTileElems;            // P^T fragments
constexpr int kBwdTOff = 2 * kTileElems;         // T, row-major
constexpr int kBwdGOff = 3 * kTileElems;         // G (fp32)

// Workgroup index -> work unit.  Workgroups are handed to the 8 XCDs
// round-robin; XCD x takes the contiguous range of units that starts at
// x * (G / 8) + min(x, G % 8), so consecutive units share an L2 (a bijection
// for any grid size G).
__device__ __forceinline__ int xcd_unit() {
    const int xcd = blockIdx.x & 7;
    return xcd * ((int)gridDim.x >> 3) + min(xcd, (int)gridDim.x & 7) + (int)(blockIdx.x >> 3);
}

// xcd_unit() for a grid of whole groups of gsz units (the workgroups of one QK
// group of one sequence): each XCD's contiguous share of positions is filled
// with the groups g = x, x + 8, x + 16, ... (x the share's first residue), so a
// group stays on one XCD while the groups of every sequence are spread over all
// eight.  (Positions are dealt out by residue of g mod 8, then by g / 8, then by
// unit within the group; a bijection on [0, gridDim.x) when gridDim.x is a
// multiple of gsz.)
__device__ __forceinline__ int xcd_group_unit(int gsz) {
    const int p = xcd_unit();
    const int ngroups = (int)gridDim.x / gsz;
    const int q = p / gsz, j = p - q * gsz;
    const int base = ngroups >> 3, rem = ngroups & 7;
    int r = 0;
#pragma unroll
    for (int k = 1; k < 8; ++k)
        if (q >= k * base + min(k, rem)) r = k;
    const int g = r + 8 * (q - (r * base + min(r, rem)));
    return g * gsz + j;
}

}  // namespace gdn
