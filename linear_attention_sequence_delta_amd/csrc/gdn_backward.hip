// gdn_backward.hip -- gradients of the bf16 chunked prefill (64-token chunks).
//
// The layer is trained, and the pages name a fused forward/backward kernel for
// it ("Qwen3.8-27B：27B 如何打出千亿级效果，且塞进单张消费级显卡", sec. 2.1).  The
// forward per chunk (gdn_chunked.hip), with S the state the chunk starts from,
// G the running sum of g inside the chunk, gamma = exp(G), lambda_r =
// exp(G_L - G_r), D_ri = exp(G_r - G_i):
//   A = strictly-lower(b_r D_ri k_r.k_i),  T = (I + A)^{-1},  T' = T diag(b)
//   P = lower-incl(scale D_ri q_r.k_i)
//   R = V - diag(gamma) K S^T,  U = T' R
//   O = scale diag(gamma) Q S^T + P U,  S' = gamma_L S + U^T diag(lambda) K
// is differentiated chunk by chunk.  With dS' the gradient with respect to
// the state the chunk hands on:
//   reverse scan (sequential over chunks, last to first):
//     dU = P^T dO + diag(lambda) K dS'^T,   dV = dR = T'^T dU
//     dS = gamma_L dS' + scale dO^T diag(gamma) Q - dR^T diag(gamma) K
//   per chunk, in parallel (S from a forward pass that stores it):
//     dQ = scale diag(gamma) dO S + M_P K
//     dK = -diag(gamma) dR S + diag(lambda) U dS' + M_P^T Q + M_A' K + M_A'^T K
//     with dP = dO U^T, M_P = dP * scale D (lower-incl),
//          dT' = dU R^T (lower-incl), dT = dT' diag(b), dA = -T^T dT T^T,
//          M_A = dA * D (strictly lower), M_A' = diag(b) M_A
//     db_i = sum_r dT'_ri T_ri + sum_j M_A,ij k_i.k_j
//     dG_r = scale gamma_r q_r.(dO S)_r - gamma_r dR_r.(K S^T)_r
//            - lambda_r k_r.(U dS')_r + rowsum_r - colsum_r of (dP * P) and
//            of (dA * A), and the last row also takes
//            gamma_L <dS', S> + sum_r lambda_r k_r.(U dS')_r
//     dg = the suffix sums of dG inside the chunk (G_r = g_0 + ... + g_r).
// All products are bf16 MFMA (16 x 16 x 32) with fp32 accumulation; the
// gradient of the state stays fp32 in registers through the reverse scan.
#include <stdint.h>

#include <type_traits>

#include "gdn_chunk.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kBSlab = 32;             // d_v columns per reverse-scan workgroup
constexpr int kBSlabs = kD / kBSlab;   // 4
constexpr int kSP = kBSlab + 8;        // LDS row stride (bf16) of slab-wide rows

// dU of a (chunk, V-head) is kept as 16 MFMA fragment blocks of 1 KiB: block
// (a, s) holds, for lane (c, g4) at 8 (16 g4 + c), row 16 a + c, columns
// 32 s + 8 g4 .. +7 -- the B operand the chunk-gradient kernel loads, one whole
// contiguous block per load instruction.  Offset (bf16 elements) of block (a, s):
__device__ __forceinline__ size_t dU_block(int chunk, int h, int H_v, int a, int s) {
    return (((size_t)chunk * H_v + h) * 16 + 4 * a + s) * 512;
}

// MFMA operands from row-major bf16 LDS matrices, for lane (c = lane % 16,
// g4 = lane / 16): frag_rows gives M[r0 + c][k0 + 8 g4 .. +7] (a row piece),
// frag_cols gives M[k0 + 8 g4 + j][c0 + c], j = 0..7 (a column piece, two
// transposing reads).  An operand's lane c indexes the output row (A) or
// column (B) and the 8 values run along the contraction.  `lane` is the
// caller's lane index (threadIdx.x % 64).
__device__ __forceinline__ uint4 frag_rows(const uint16_t *M, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const uint4 *>(M + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
__device__ __forceinline__ uint4 frag_cols(const uint16_t *M, int ld, int k0, int c0, int lane) {
    const int c = lane & 15;
    const uint16_t *base = M + (k0 + 8 * (lane >> 4) + (c >> 2)) * ld + c0 + 4 * (c & 3);
    const uint2 lo = lds_read_tr16(base), hi = lds_read_tr16(base + 4 * ld);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
__device__ __forceinline__ void unpack4(uint2 u, float *f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xFFFF0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// sum of the 8 products of two 8-wide bf16 pieces, plus acc (packed dot products)
__device__ __forceinline__ float dot8_acc(uint4 a, uint4 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), acc, false);
    return acc;
}
// Column sums of a 16-row tile held in the MFMA result layout: x[j] is row
// c, column 4 g4 + j of the lane (c, g4).  After the exchange, lanes with
// c % 4 == 0 hold the sum over the 16 rows for column 4 g4 + c / 4 (the
// lanes exchange half of what they hold with row_mirror, then half again
// with row_half_mirror, then sum each group of four).
__device__ __forceinline__ float col16_sums(f32x4 x, int c) {
    const bool h8 = c & 8, h4 = c & 4;
#define GDN_DPP(v, ctl) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctl, 0xF, 0xF, false))
    const float y0 = (h8 ? x[2] : x[0]) + GDN_DPP(h8 ? x[0] : x[2], 0x140);
    const float y1 = (h8 ? x[3] : x[1]) + GDN_DPP(h8 ? x[1] : x[3], 0x140);
    float z = (h4 ? y1 : y0) + GDN_DPP(h4 ? y0 : y1, 0x141);
    z += GDN_DPP(z, 0xB1);
    z += GDN_DPP(z, 0x4E);
#undef GDN_DPP
    return z;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// ------------------------------------------------------------ reverse scan
// Inputs of one chunk, loaded two chunks ahead into three rotating register
// sets.  Rows past the end of a sequence are clamped to its last row on load
// and replaced by zero in LDS.
struct RevState {     // waves 0-3
    u32x4 kr[4];      // K row 16 w + 4 i + lane / 16, d_k 8 (lane % 16) .. +7
    u32x4 tt[2];      // T'^T row 16 w + c, columns 32 s + 8 g4 .. +7
    float Gown;       // G of row 16 w + c
    float GL;         // G of the chunk's last row
};
struct RevHelp {      // waves 4-7
    u32x4 qr[4];      // Q row 16 w + 4 i + lane / 16, d_k 8 (lane % 16) .. +7
    u32x4 dor;        // dO row 16 w + lane / 4, slab columns 8 (lane % 4) .. +7
    u32x4 pt[2];      // P^T row 16 w + c, columns 32 s + 8 g4 .. +7
    float Gz;         // G of row 16 w + lane / 4
};

// One workgroup (512 threads) per (sequence, V-head, 32-column d_v slab).
// Waves 0-3 carry the fp32 state gradient from the last chunk to the first:
// wave w owns chunk rows 16 w .. +15 of Y = K dS'^T, dU and dR and d_k columns
// 32 w .. +31 of dS.  Waves 4-7 (same SIMDs) do everything off that chain:
// they form P^T dO of the next chunk and the update's Q term
// W = scale dO^T diag(gamma) Q (handed over in fp32 through LDS), and they
// write the results out of LDS: per chunk the bf16 dS' it starts from
// (dsw [chunk][H_v][d_v][d_k]), dU (duw, MFMA fragment blocks: see dU_block) and the dv
// rows.  (Global stores issued by the state waves lengthen their chain: the
// waits for their own prefetched loads would also cover the stores.)  Three
// barriers per chunk: (1) dU complete, (2) dR complete, (3) dS complete.  The
// state waves write the gradient with respect to the initial state.
__global__ __launch_bounds__(512) void bwd_scan_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ d_o,
    const float *dS_final, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_base, int N, int T, int H_qk, int H_v, float scale,
    const uint16_t *__restrict__ bws, uint16_t *__restrict__ dsw, uint16_t *__restrict__ duw,
    uint16_t *__restrict__ dv, float *dS0, int c_lo, int c_hi) {
    __shared__ __attribute__((aligned(16))) uint16_t sS[kBSlab * kKP];       // dS' (bf16), [v][k]
    __shared__ __attribute__((aligned(16))) uint16_t sKr[kChunk * kKP];      // K rows of the chunk
    __shared__ __attribute__((aligned(16))) uint16_t sQr[kChunk * kKP];      // Q rows (helpers)
    __shared__ __attribute__((aligned(16))) uint16_t sDO[kChunk * kSP];      // dO rows (slab)
    __shared__ __attribute__((aligned(16))) uint16_t sZq[kChunk * kSP];      // scale gamma_r dO_r
    __shared__ __attribute__((aligned(16))) uint16_t sDU[kChunk * kSP];      // dU rows (slab)
    __shared__ __attribute__((aligned(16))) uint16_t sZk[kChunk * kSP];      // -gamma_r dR_r
    __shared__ __attribute__((aligned(16))) uint16_t sDR[kChunk * kSP];      // dR rows (slab)
    __shared__ __attribute__((aligned(16))) float sW[4 * 4 * 64 * 4];        // W, in the state layout
    __shared__ __attribute__((aligned(16))) float sPd[4 * 2 * 64 * 4];      // P^T dO, in dU's layout

    const int u = xcd_group_unit((H_v / H_qk) * kBSlabs);
    const int slab = u % kBSlabs;
    const int nh = u / kBSlabs;
    const int h = nh % H_v, n = nh / H_v;
    const int hq = h / (H_v / H_qk);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = wave & 3;
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c = lane & 15;
    const int s0 = cu ? cu[n] : 0, s1 = cu ? cu[n + 1] : T;
    // chunks [c_lo, nch) of the sequence, last to first: the gradient enters as
    // dS_final and leaves as dS0, so a sequence can be walked in segments
    const int nch = min((s1 - s0 + kChunk - 1) / kChunk, c_hi);
    const int cbase = chunk_base[n];
    const int e0 = kBSlab * slab;
    const size_t st_off = ((size_t)n * H_v + h) * (kD * kD);
    auto chunk_len = [&](int ci) { return min(kChunk, s1 - (s0 + kChunk * ci)); };
    auto brec = [&](int ci) { return bws + ((size_t)(cbase + ci) * H_v + h) * kBwdRecElems; };
    // offset of row 16 w + 4 i + lane / 16 (clamped), 16-byte piece lane % 16,
    // of chunk ci in q or k
    auto qk_off = [&](int ci, int i) {
        const int r = min(16 * w + 4 * i + (lane >> 4), chunk_len(ci) - 1);
        return ((size_t)(s0 + kChunk * ci + r) * H_qk + hq) * kD + 8 * (lane & 15);
    };

    if (wave < 4) {
        // ---------------- state waves
        auto fetch = [&](int ci, RevState &R) {     // needs nch >= 1
            ci = max(ci, 0);                        // before the first chunk: loaded, never used
#pragma unroll
            for (int i = 0; i < 4; ++i) R.kr[i] = *reinterpret_cast<const u32x4 *>(k + qk_off(ci, i));
            const uint16_t *rec = brec(ci);
#pragma unroll
            for (int s = 0; s < 2; ++s) R.tt[s] = *reinterpret_cast<const u32x4 *>(rec + kBwdTtOff + frag_off(w, s, lane));
            const float *Gp = reinterpret_cast<const float *>(rec + kBwdGOff);
            R.Gown = Gp[16 * w + c];
            R.GL = Gp[kChunk - 1];
        };
        // st[t][nt] = dS[e0 + 16 nt + c][32 w + 16 t + 4 g4 + j]
        f32x4 st[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                if (dS_final) {
                    const float4 x = *reinterpret_cast<const float4 *>(
                        dS_final + st_off + (size_t)(e0 + 16 * nt + c) * kD + 32 * w + 16 * t + 4 * g4);
                    st[t][nt] = f32x4{x.x, x.y, x.z, x.w};
                } else {
                    st[t][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        auto write_state_lds = [&]() {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    *reinterpret_cast<uint2 *>(sS + (16 * nt + c) * kKP + 32 * w + 16 * t + 4 * g4) =
                        pk4(st[t][nt][0], st[t][nt][1], st[t][nt][2], st[t][nt][3]);
        };
        auto body = [&](int ci, const RevState &cur, RevState &pf) {
            const int L = chunk_len(ci);
            // this wave's K rows into LDS
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * i + (lane >> 4);
                *reinterpret_cast<u32x4 *>(sKr + r * kKP + 8 * (lane & 15)) =
                    r < L ? cur.kr[i] : u32x4{0u, 0u, 0u, 0u};
            }
            wave_lds_sync();
            uint4 kB[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) kB[s] = frag_rows(sKr, kKP, 16 * w, 32 * s, lane);
            fetch(ci - 2, pf);
            const float lam = __expf(cur.GL - cur.Gown), gam = __expf(cur.Gown), gamL = __expf(cur.GL);
            // dU = P^T dO + diag(lambda) K dS'^T: rows 16 w + c, slab columns 16 nt + 4 g4 + j
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) y = mfma32(frag_rows(sS, kKP, 16 * nt, 32 * s, lane), kB[s], y);
                const float4 pd = *reinterpret_cast<const float4 *>(sPd + ((w * 2 + nt) * 64 + lane) * 4);
                *reinterpret_cast<uint2 *>(sDU + (16 * w + c) * kSP + 16 * nt + 4 * g4) =
                    pk4(pd.x + lam * y[0], pd.y + lam * y[1], pd.z + lam * y[2], pd.w + lam * y[3]);
            }
            __syncthreads();                                    // (1) dU complete
            // dR = T'^T dU: the gradient of v
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (s >= (w >> 1)) d = mfma32(frag_cols(sDU, kSP, 32 * s, 16 * nt, lane), cur.tt[s], d);
                *reinterpret_cast<uint2 *>(sDR + (16 * w + c) * kSP + 16 * nt + 4 * g4) = pk4(d[0], d[1], d[2], d[3]);
                *reinterpret_cast<uint2 *>(sZk + (16 * w + c) * kSP + 16 * nt + 4 * g4) =
                    pk4(-gam * d[0], -gam * d[1], -gam * d[2], -gam * d[3]);
            }
            __syncthreads();                                    // (2) dR complete
            // dS = gamma_L dS' + W + (-diag(gamma) dR)^T K
            uint4 zk[2][2], ka[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) zk[nt][s] = frag_cols(sZk, kSP, 32 * s, 16 * nt, lane);
#pragma unroll
                for (int t = 0; t < 2; ++t) ka[t][s] = frag_cols(sKr, kKP, 32 * s, 32 * w + 16 * t, lane);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const float4 wq = *reinterpret_cast<const float4 *>(sW + ((w * 4 + t * 2 + nt) * 64 + lane) * 4);
                    f32x4 a = gamL * st[t][nt] + f32x4{wq.x, wq.y, wq.z, wq.w};
#pragma unroll
                    for (int s = 0; s < 2; ++s) a = mfma32(ka[t][s], zk[nt][s], a);
                    st[t][nt] = a;
                }
            write_state_lds();
            __syncthreads();                                    // (3) dS complete
        };

        RevState r0, r1, r2;
        if (nch > c_lo) {
            fetch(nch - 1, r0);
            fetch(nch - 2, r1);
        }
        write_state_lds();
        __syncthreads();                                        // helpers' first staging
        __syncthreads();                                        // helpers' first P^T dO
        for (int ci = nch - 1; ci >= c_lo; ci -= 3) {
            body(ci, r0, r2);
            if (ci == c_lo) break;
            body(ci - 1, r1, r0);
            if (ci - 1 == c_lo) break;
            body(ci - 2, r2, r1);
        }
        if (dS0) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    *reinterpret_cast<float4 *>(dS0 + st_off + (size_t)(e0 + 16 * nt + c) * kD + 32 * w + 16 * t + 4 * g4) =
                        make_float4(st[t][nt][0], st[t][nt][1], st[t][nt][2], st[t][nt][3]);
        }
    } else {
        // ---------------- helper waves
        auto fetch = [&](int ci, RevHelp &R) {      // needs nch >= 1
            ci = max(ci, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) R.qr[i] = *reinterpret_cast<const u32x4 *>(q + qk_off(ci, i));
            const int rd = min(16 * w + (lane >> 2), chunk_len(ci) - 1);
            R.dor = *reinterpret_cast<const u32x4 *>(d_o + ((size_t)(s0 + kChunk * ci + rd) * H_v + h) * kD + e0 + 8 * (lane & 3));
            const uint16_t *rec = brec(ci);
#pragma unroll
            for (int s = 0; s < 2; ++s) R.pt[s] = *reinterpret_cast<const u32x4 *>(rec + kBwdPtOff + frag_off(w, s, lane));
            R.Gz = reinterpret_cast<const float *>(rec + kBwdGOff)[16 * w + (lane >> 2)];
        };
        const int pr = 16 * w + (lane >> 2), pc = 8 * (lane & 3);    // this lane's dO row piece
        auto stage_do = [&](int ci, const RevHelp &R) {
            *reinterpret_cast<u32x4 *>(sDO + pr * kSP + pc) = pr < chunk_len(ci) ? R.dor : u32x4{0u, 0u, 0u, 0u};
        };
        // Q rows and scale gamma_r dO_r of chunk ci
        auto stage_qz = [&](int ci, const RevHelp &R) {
            const int L = chunk_len(ci);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * i + (lane >> 4);
                *reinterpret_cast<u32x4 *>(sQr + r * kKP + 8 * (lane & 15)) = r < L ? R.qr[i] : u32x4{0u, 0u, 0u, 0u};
            }
            float x[8];
            unpack8(__builtin_bit_cast(uint4, R.dor), x);
            const float gz = pr < L ? scale * __expf(R.Gz) : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= gz;
            *reinterpret_cast<uint4 *>(sZq + pr * kSP + pc) = pack_bf8(x);
        };
        // P^T dO of the staged chunk (rows 16 w + c, slab columns 16 nt + 4 g4 + j)
        auto pdo = [&](const RevHelp &R) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    if (s >= (w >> 1)) pd = mfma32(frag_cols(sDO, kSP, 32 * s, 16 * nt, lane), R.pt[s], pd);
                *reinterpret_cast<float4 *>(sPd + ((w * 2 + nt) * 64 + lane) * 4) = make_float4(pd[0], pd[1], pd[2], pd[3]);
            }
        };
        const int hl = lane + 64 * w;                               // 0..255
        auto body = [&](int ci, const RevHelp &nxt, RevHelp &pf) {
            // dS' of this chunk (bf16, as the state waves left it in LDS)
            {
                uint16_t *dsp = dsw + ((size_t)(cbase + ci) * H_v + h) * (kD * kD) + (size_t)e0 * kD;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int e = hl + 256 * m, r = e >> 4, pcs = 8 * (e & 15);
                    *reinterpret_cast<u32x4 *>(dsp + r * kD + pcs) = *reinterpret_cast<const u32x4 *>(sS + r * kKP + pcs);
                }
            }
            if (ci > c_lo) stage_do(ci - 1, nxt);
            fetch(ci - 2, pf);
            // W = scale dO^T diag(gamma) Q of chunk ci, in the state layout
            uint4 zq[2][2], qa[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) zq[nt][s] = frag_cols(sZq, kSP, 32 * s, 16 * nt, lane);
#pragma unroll
                for (int t = 0; t < 2; ++t) qa[t][s] = frag_cols(sQr, kKP, 32 * s, 32 * w + 16 * t, lane);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s) a = mfma32(qa[t][s], zq[nt][s], a);
                    *reinterpret_cast<float4 *>(sW + ((w * 4 + t * 2 + nt) * 64 + lane) * 4) = make_float4(a[0], a[1], a[2], a[3]);
                }
            __syncthreads();                                    // (1)
            if (ci > c_lo) {
                pdo(nxt);
                stage_qz(ci - 1, nxt);
            }
            {
                // block (a = hl / 64, s = slab); lane hl % 64 = (c, g4): row 16 a + c,
                // slab columns 8 g4 .. +7
                const int a = hl >> 6, fl = hl & 63;
                *reinterpret_cast<u32x4 *>(duw + dU_block(cbase + ci, h, H_v, a, slab) + 8 * fl) =
                    *reinterpret_cast<const u32x4 *>(sDU + (16 * a + (fl & 15)) * kSP + 8 * (fl >> 4));
            }
            __syncthreads();                                    // (2)
            {
                const int r = hl >> 2, pcs = 8 * (hl & 3);
                if (r < chunk_len(ci))
                    *reinterpret_cast<u32x4 *>(dv + ((size_t)(s0 + kChunk * ci + r) * H_v + h) * kD + e0 + pcs) =
                        *reinterpret_cast<const u32x4 *>(sDR + r * kSP + pcs);
            }
            __syncthreads();                                    // (3)
        };

        RevHelp r0, r1, r2;
        if (nch > c_lo) {
            fetch(nch - 1, r0);
            fetch(nch - 2, r1);
            stage_do(nch - 1, r0);
            stage_qz(nch - 1, r0);
        }
        __syncthreads();
        if (nch > c_lo) pdo(r0);
        __syncthreads();
        for (int ci = nch - 1; ci >= c_lo; ci -= 3) {
            body(ci, r1, r2);
            if (ci == c_lo) break;
            body(ci - 1, r2, r0);
            if (ci - 1 == c_lo) break;
            body(ci - 2, r0, r1);
        }
    }
}

// ------------------------------------------------------------ chunk gradients
// One workgroup (8 waves) per (chunk, QK head), looping over the V-heads of
// the group; dq and dk of the group accumulate in fp32 registers.  Waves w
// and w + 4 own chunk rows 16 (w % 4) .. +15 and split the column tiles of
// every product: half hf = w / 4 takes the 16-column tiles 4 hf .. 4 hf + 3
// of a 128-wide result and the tiles t with t % 2 = hf of a 64-wide one.
// Every row-wise result is held with lane (c, g4) on the row 16 (w % 4) + c,
// columns 16 t + 4 g4 .. +3 of each tile t, which an MFMA gives when the left
// factor's rows are its B operand and the right factor's columns its A
// operand.  A V-head's inputs are read in whole rows (every load instruction
// covers whole cache lines) and staged in LDS, each once for both halves; the
// column sums of the dG and db terms stay in registers until the end of the
// step and are reduced across the 16 rows of a tile by one exchange pass.
__global__ __launch_bounds__(512) void bwd_grad_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const uint16_t *__restrict__ d_o, const uint16_t *__restrict__ dv, const float *__restrict__ beta,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_base, int N, int T, int H_qk,
    int H_v, float scale, const uint16_t *__restrict__ bws, const uint16_t *__restrict__ states,
    const uint16_t *__restrict__ dsw, const uint16_t *__restrict__ duw, uint16_t *__restrict__ dq,
    uint16_t *__restrict__ dk, float *__restrict__ dg, float *__restrict__ dbeta, int item_lo,
    int item_hi) {
    __shared__ __attribute__((aligned(16))) uint16_t sQ[kChunk * kKP];
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * kKP];
    __shared__ __attribute__((aligned(16))) uint16_t sSt[kD * kKP];      // S, then dS' ([v][k])
    __shared__ __attribute__((aligned(16))) uint16_t sR[kChunk * kKP];   // R [r][v]
    __shared__ __attribute__((aligned(16))) uint16_t sU[kChunk * kKP];   // dR, then U [r][v]
    __shared__ __attribute__((aligned(16))) uint16_t sDO[kChunk * kKP];  // dO [r][v]
    __shared__ __attribute__((aligned(16))) uint16_t sT[kChunk * kRP];   // T
    __shared__ __attribute__((aligned(16))) uint16_t sM[kChunk * kRP];   // M_P, then M_A'
    __shared__ __attribute__((aligned(16))) uint16_t sM2[kChunk * kRP];  // dT
    __shared__ __attribute__((aligned(16))) uint16_t sF[kChunk * kRP];   // dT T^T
    __shared__ __attribute__((aligned(16))) float sG[kChunk];
    __shared__ __attribute__((aligned(16))) float sB[kChunk];
    __shared__ float sRowG[2][kChunk], sRowB[2][kChunk];
    __shared__ float sColG[4][kChunk], sColB[4][kChunk];
    __shared__ float sE[8];

    // items (chunk, QK head) item_lo + blockIdx.x, then every gridDim.x-th after it
    for (int item = item_lo + blockIdx.x; item < item_hi; item += gridDim.x) {
        __syncthreads();                                   // the previous item's LDS reads are done
        const int gc = item / H_qk, hq = item - gc * H_qk;
        if (gc >= chunk_base[N]) break;                    // so are the later items (same for the whole workgroup)
        const int n = seq_of_chunk(chunk_base, N, gc);
        const int s0 = cu ? cu[n] : 0, s1 = cu ? cu[n + 1] : T;
        const int c0 = s0 + kChunk * (gc - chunk_base[n]);
        const int L = min(kChunk, s1 - c0);
        const int group = H_v / H_qk;
        const int tid = threadIdx.x;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int w = wave & 3;
        const int lane = tid & 63, g4 = lane >> 4, c = lane & 15;
        const int row = 16 * w + c;                        // this lane's row
        const bool row_ok = row < L;
        const int wb = w >> 1;                             // 32-row block of this wave's rows

#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int e = tid + 512 * m, r = e >> 4, pc = e & 15;
            const size_t off = ((size_t)(c0 + min(r, L - 1)) * H_qk + hq) * kD + 8 * pc;
            uint4 kv = *reinterpret_cast<const uint4 *>(k + off), qv = *reinterpret_cast<const uint4 *>(q + off);
            if (r >= L) kv = qv = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(sK + r * kKP + 8 * pc) = kv;
            *reinterpret_cast<uint4 *>(sQ + r * kKP + 8 * pc) = qv;
        }
        __syncthreads();
        int ol = lane;
        // x_row . k_(16 t + 4 g4 + j) for the rows x of M (K or Q), tile t
        auto dot_k = [&](const uint16_t *M, int t) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) a = mfma32(frag_rows(sK, kKP, 16 * t, 32 * s, ol), frag_rows(M, kKP, 16 * w, 32 * s, ol), a);
            return a;
        };
        f32x4 dQa[4], dKa[4];                              // columns 16 (4 hf + i) + 4 g4 + j
#pragma unroll
        for (int i = 0; i < 4; ++i) dQa[i] = dKa[i] = f32x4{0.f, 0.f, 0.f, 0.f};

        // the V-head step, for a compile-time half (tile offsets fold into
        // instruction immediates); both halves pass the same barriers in order
        auto vhead = [&](int vv, auto half) {
            constexpr int hf = decltype(half)::value;
            const int h = hq * group + vv;
            // the lane index, opaque to the optimiser: LDS addresses are formed
            // inside each step instead of being kept in registers across steps
            ol = lane;
            asm volatile("" : "+v"(ol));
            const int c = ol & 15, g4 = ol >> 4, tid = 64 * wave + ol;
            const int row = 16 * w + c;
            const uint16_t *brec = bws + ((size_t)gc * H_v + h) * kBwdRecElems;
            const uint16_t *Sg = states + ((size_t)gc * H_v + h) * (kD * kD);
            const uint16_t *dSg = dsw + ((size_t)gc * H_v + h) * (kD * kD);
            // this V-head's inputs in flight together, all in whole rows: T, S,
            // G, b, and the rows of dO, dR and V (rows past the chunk's end read
            // as zero), written into LDS after the previous V-head's reads
            float e1 = 0.f;                                // this thread's share of <dS', S>
            {
                const u32x4 tv = *reinterpret_cast<const u32x4 *>(brec + kBwdTOff + (tid >> 3) * kChunk + 8 * (tid & 7));
                u32x4 sv[4], ov[2], rv[2], xv[2];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = tid + 512 * m;
                    sv[m] = *reinterpret_cast<const u32x4 *>(Sg + (e >> 4) * kD + 8 * (e & 15));
                }
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int e = tid + 512 * m;
                    const size_t off = ((size_t)(c0 + min(e >> 4, L - 1)) * H_v + h) * kD + 8 * (e & 15);
                    ov[m] = *reinterpret_cast<const u32x4 *>(d_o + off);
                    rv[m] = *reinterpret_cast<const u32x4 *>(dv + off);
                    xv[m] = *reinterpret_cast<const u32x4 *>(v + off);
                }
                float gl = 0.f, bl = 0.f;
                if (tid < kChunk) {
                    gl = reinterpret_cast<const float *>(brec + kBwdGOff)[tid];
                    bl = tid < L ? beta[(size_t)(c0 + tid) * H_v + h] : 0.f;
                }
                __syncthreads();                           // the previous V-head's LDS reads are done
                *reinterpret_cast<u32x4 *>(sT + (tid >> 3) * kRP + 8 * (tid & 7)) = tv;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = tid + 512 * m;
                    *reinterpret_cast<u32x4 *>(sSt + (e >> 4) * kKP + 8 * (e & 15)) = sv[m];
                }
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int e = tid + 512 * m, r = e >> 4, o = r * kKP + 8 * (e & 15);
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4 *>(sDO + o) = r < L ? ov[m] : z;
                    *reinterpret_cast<u32x4 *>(sU + o) = r < L ? rv[m] : z;
                    *reinterpret_cast<u32x4 *>(sR + o) = r < L ? xv[m] : z;
                }
                if (tid < kChunk) {
                    sG[tid] = gl;
                    sB[tid] = bl;
                }
            }
            __syncthreads();

            const float Gr = sG[row], GLast = sG[kChunk - 1];
            const float gam = __expf(Gr), lam = __expf(GLast - Gr), br = sB[row];
            float rowG = 0.f, rowB = 0.f, e2 = 0.f;
            f32x4 colG[2], colB[2];                        // column-sum terms of the wave's two tiles

            // X = K S^T -> R = V - diag(gamma) X
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int nt = 4 * hf + i;
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) x = mfma32(frag_rows(sSt, kKP, 16 * nt, 32 * s, ol), frag_rows(sK, kKP, 16 * w, 32 * s, ol), x);
                float vf[4];
                unpack4(*reinterpret_cast<const uint2 *>(sR + row * kKP + 16 * nt + 4 * g4), vf);
                *reinterpret_cast<uint2 *>(sR + row * kKP + 16 * nt + 4 * g4) =
                    pk4(vf[0] - gam * x[0], vf[1] - gam * x[1], vf[2] - gam * x[2], vf[3] - gam * x[3]);
            }
            // dO S and dR S: dQ += scale gamma dO S (dG: q_r . that), dK -= gamma dR S
            // (dG: -gamma_r dR_r . X_r = -gamma_r k_r . (dR S)_r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kt = 4 * hf + i;
                f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint4 sf = frag_cols(sSt, kKP, 32 * s, 16 * kt, ol);
                    a1 = mfma32(sf, frag_rows(sDO, kKP, 16 * w, 32 * s, ol), a1);
                    a2 = mfma32(sf, frag_rows(sU, kKP, 16 * w, 32 * s, ol), a2);
                }
                float qf[4], kf[4];
                unpack4(*reinterpret_cast<const uint2 *>(sQ + row * kKP + 16 * kt + 4 * g4), qf);
                unpack4(*reinterpret_cast<const uint2 *>(sK + row * kKP + 16 * kt + 4 * g4), kf);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float t = scale * gam * a1[j];
                    dQa[i][j] += t;
                    rowG += t * qf[j];
                    const float u = gam * a2[j];
                    dKa[i][j] -= u;
                    rowG -= u * kf[j];
                }
            }
            // the row-dot terms are finished here: left to the compiler they sink
            // to the end of the step and hold the products in registers until then
            asm volatile("" : "+v"(rowG));
            __syncthreads();                               // R complete; S no longer read
            uint4 dUf[4];                                  // row `row` of dU, columns 32 s + 8 g4 .. +7
#pragma unroll
            for (int s = 0; s < 4; ++s)
                dUf[s] = *reinterpret_cast<const uint4 *>(duw + dU_block(gc, h, H_v, w, s) + 8 * ol);
            {
                u32x4 dsv[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = tid + 512 * m;
                    dsv[m] = *reinterpret_cast<const u32x4 *>(dSg + (e >> 4) * kD + 8 * (e & 15));
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int e = tid + 512 * m;
                    u32x4 *p = reinterpret_cast<u32x4 *>(sSt + (e >> 4) * kKP + 8 * (e & 15));
                    e1 = dot8_acc(__builtin_bit_cast(uint4, *p), __builtin_bit_cast(uint4, dsv[m]), e1);
                    *p = dsv[m];
                }
            }
            asm volatile("" : "+v"(e1));
            // U = T' R (T'[row][i] = T[row][i] b_i)
            {
                uint4 tB[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    float tf[8];
                    unpack8(*reinterpret_cast<const uint4 *>(sT + row * kRP + 32 * s + 8 * g4), tf);
                    const float4 b0 = *reinterpret_cast<const float4 *>(sB + 32 * s + 8 * g4);
                    const float4 b1 = *reinterpret_cast<const float4 *>(sB + 32 * s + 8 * g4 + 4);
                    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) tf[e] *= bb[e];
                    tB[s] = pack_bf8(tf);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int nt = 4 * hf + i;
                    f32x4 ua = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        if (s <= wb) ua = mfma32(frag_cols(sR, kKP, 32 * s, 16 * nt, ol), tB[s], ua);
                    *reinterpret_cast<uint2 *>(sU + row * kKP + 16 * nt + 4 * g4) = pk4(ua[0], ua[1], ua[2], ua[3]);
                }
            }
            __syncthreads();                               // U and dS' complete

            // U dS': dK += lambda U dS'; dG: -lambda_r k_r . (U dS')_r (the last row gets the sum)
            {
                uint4 uB[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) uB[s] = frag_rows(sU, kKP, 16 * w, 32 * s, ol);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kt = 4 * hf + i;
                    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 4; ++s) a = mfma32(frag_cols(sSt, kKP, 32 * s, 16 * kt, ol), uB[s], a);
                    float kf[4];
                    unpack4(*reinterpret_cast<const uint2 *>(sK + row * kKP + 16 * kt + 4 * g4), kf);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        dKa[i][j] += lam * a[j];
                        const float t = lam * a[j] * kf[j];
                        rowG -= t;
                        e2 += t;
                    }
                }
            }
            asm volatile("" : "+v"(rowG), "+v"(e2));
            // dP = dO U^T -> M_P; dT' = dU R^T -> dT; row and column sums
            uint4 dOf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) dOf[s] = frag_rows(sDO, kKP, 16 * w, 32 * s, ol);
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                const int t = 2 * ti + hf;
                f32x4 dp = {0.f, 0.f, 0.f, 0.f}, dtp = dp, qk = dp;
                if (t <= w) {
                    qk = dot_k(sQ, t);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        dp = mfma32(frag_rows(sU, kKP, 16 * t, 32 * s, ol), dOf[s], dp);
                        dtp = mfma32(frag_rows(sR, kKP, 16 * t, 32 * s, ol), dUf[s], dtp);
                    }
                }
                const float4 Gi = *reinterpret_cast<const float4 *>(sG + 16 * t + 4 * g4);
                const float4 Bi = *reinterpret_cast<const float4 *>(sB + 16 * t + 4 * g4);
                const float gi[4] = {Gi.x, Gi.y, Gi.z, Gi.w}, bi[4] = {Bi.x, Bi.y, Bi.z, Bi.w};
                float tf[4];
                unpack4(*reinterpret_cast<const uint2 *>(sT + row * kRP + 16 * t + 4 * g4), tf);
                float mp[4], dt[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool lo = 16 * t + 4 * g4 + j <= row;
                    mp[j] = lo ? dp[j] * scale * __expf(Gr - gi[j]) : 0.f;
                    const float wp = lo ? mp[j] * qk[j] : 0.f;
                    rowG += wp;
                    colG[ti][j] = -wp;
                    dt[j] = lo ? dtp[j] * bi[j] : 0.f;
                    colB[ti][j] = lo ? dtp[j] * tf[j] : 0.f;
                }
                *reinterpret_cast<uint2 *>(sM + row * kRP + 16 * t + 4 * g4) = pk4(mp[0], mp[1], mp[2], mp[3]);
                *reinterpret_cast<uint2 *>(sM2 + row * kRP + 16 * t + 4 * g4) = pk4(dt[0], dt[1], dt[2], dt[3]);
            }
            __syncthreads();                               // M_P, dT complete

            // dQ += M_P K; dK += M_P^T Q; F = dT T^T
            {
                uint4 mB[2], mtB[2], dtB[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    mB[s] = frag_rows(sM, kRP, 16 * w, 32 * s, ol);
                    mtB[s] = frag_cols(sM, kRP, 32 * s, 16 * w, ol);
                    dtB[s] = frag_rows(sM2, kRP, 16 * w, 32 * s, ol);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kt = 4 * hf + i;
                    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        if (s <= wb) a = mfma32(frag_cols(sK, kKP, 32 * s, 16 * kt, ol), mB[s], a);
                        if (s >= wb) b = mfma32(frag_cols(sQ, kKP, 32 * s, 16 * kt, ol), mtB[s], b);
                    }
                    dQa[i] += a;
                    dKa[i] += b;
                }
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) {
                    const int t = 2 * ti + hf;
                    f32x4 f = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        if (s <= wb) f = mfma32(frag_rows(sT, kRP, 16 * t, 32 * s, ol), dtB[s], f);
                    *reinterpret_cast<uint2 *>(sF + row * kRP + 16 * t + 4 * g4) = pk4(f[0], f[1], f[2], f[3]);
                }
            }
            __syncthreads();                               // F complete; M_P no longer read

            // dA = -T^T F (strictly lower) -> M_A = dA * D; db: rows of M_A * KK^T;
            // dG: rows and columns of dA * A; M_A' = diag(b) M_A -> sM
            {
                uint4 ttB[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) ttB[s] = frag_cols(sT, kRP, 32 * s, 16 * w, ol);
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) {
                    const int t = 2 * ti + hf;
                    f32x4 da = {0.f, 0.f, 0.f, 0.f}, kk = da;
                    if (t <= w) {
                        kk = dot_k(sK, t);
#pragma unroll
                        for (int s = 0; s < 2; ++s)
                            if (s >= wb) da = mfma32(frag_cols(sF, kRP, 32 * s, 16 * t, ol), ttB[s], da);
                    }
                    const float4 Gj = *reinterpret_cast<const float4 *>(sG + 16 * t + 4 * g4);
                    const float gj[4] = {Gj.x, Gj.y, Gj.z, Gj.w};
                    float ma[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const bool lo = 16 * t + 4 * g4 + j < row;
                        const float m = lo ? -da[j] * __expf(Gr - gj[j]) : 0.f;
                        const float kkv = lo ? kk[j] : 0.f;
                        rowB += m * kkv;
                        const float wa = m * br * kkv;
                        rowG += wa;
                        colG[ti][j] -= wa;
                        ma[j] = m * br;
                    }
                    *reinterpret_cast<uint2 *>(sM + row * kRP + 16 * t + 4 * g4) = pk4(ma[0], ma[1], ma[2], ma[3]);
                }
            }
            rowG += __shfl_xor(rowG, 16, 64);
            rowG += __shfl_xor(rowG, 32, 64);
            rowB += __shfl_xor(rowB, 16, 64);
            rowB += __shfl_xor(rowB, 32, 64);
            if (g4 == 0) {
                sRowG[hf][row] = rowG;
                sRowB[hf][row] = rowB;
            }
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                const float zg = col16_sums(colG[ti], c), zb = col16_sums(colB[ti], c);
                if ((c & 3) == 0) {
                    sColG[w][16 * (2 * ti + hf) + 4 * g4 + (c >> 2)] = zg;
                    sColB[w][16 * (2 * ti + hf) + 4 * g4 + (c >> 2)] = zb;
                }
            }
            {
                const float ew = wave_sum(__expf(GLast) * e1 + e2);
                if (lane == 0) sE[wave] = ew;
            }
            __syncthreads();                               // M_A' and the sums complete

            // dK += M_A' K + M_A'^T K
            {
                uint4 mB[2], mtB[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    mB[s] = frag_rows(sM, kRP, 16 * w, 32 * s, ol);
                    mtB[s] = frag_cols(sM, kRP, 32 * s, 16 * w, ol);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kt = 4 * hf + i;
                    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const uint4 kf = frag_cols(sK, kKP, 32 * s, 16 * kt, ol);
                        if (s <= wb) a = mfma32(kf, mB[s], a);
                        if (s >= wb) a = mfma32(kf, mtB[s], a);
                    }
                    dKa[i] += a;
                }
            }
            // dg = suffix sums of dG inside the chunk; db
            if (wave == 0) {
                float dG = sRowG[0][lane] + sRowG[1][lane] + sColG[0][lane] + sColG[1][lane] +
                           sColG[2][lane] + sColG[3][lane];
                if (lane == kChunk - 1) {
#pragma unroll
                    for (int x = 0; x < 8; ++x) dG += sE[x];
                }
                const float db = sRowB[0][lane] + sRowB[1][lane] + sColB[0][lane] + sColB[1][lane] +
                                 sColB[2][lane] + sColB[3][lane];
                const float suf = wave_scan(__shfl(dG, 63 - lane, 64));
                const float dgr = __shfl(suf, 63 - lane, 64);
                if (lane < L) {
                    dg[(size_t)(c0 + lane) * H_v + h] = dgr;
                    dbeta[(size_t)(c0 + lane) * H_v + h] = db;
                }
            }
        };
        for (int vv = 0; vv < group; ++vv) {
            if (wave < 4) vhead(vv, std::integral_constant<int, 0>{});
            else vhead(vv, std::integral_constant<int, 1>{});
        }
        const int hf = wave >> 2;
        if (row_ok) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t off = ((size_t)(c0 + row) * H_qk + hq) * kD + 16 * (4 * hf + i) + 4 * g4;
                *reinterpret_cast<uint2 *>(dq + off) = pk4(dQa[i][0], dQa[i][1], dQa[i][2], dQa[i][3]);
                *reinterpret_cast<uint2 *>(dk + off) = pk4(dKa[i][0], dKa[i][1], dKa[i][2], dKa[i][3]);
            }
        }
    }
}

}  // namespace

hipError_t launch_bwd_scan(const void *q, const void *k, const void *d_o, const float *dS_final,
                           const int32_t *cu_seqlens, const int32_t *chunk_base, int N, int T,
                           int H_qk, int H_v, float scale, const void *bws, void *dsw, void *duw,
                           void *dv, float *dS0, int c_lo, int c_hi, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_scan_kernel, dim3(N * H_v * kBSlabs), dim3(512), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(d_o), dS_final, cu_seqlens, chunk_base, N, T,
                       H_qk, H_v, scale, static_cast<const uint16_t *>(bws),
                       static_cast<uint16_t *>(dsw), static_cast<uint16_t *>(duw),
                       static_cast<uint16_t *>(dv), dS0, c_lo, c_hi);
    return hipGetLastError();
}

hipError_t launch_bwd_grad(const void *q, const void *k, const void *v, const void *d_o,
                           const void *dv, const float *beta, const int32_t *cu_seqlens,
                           const int32_t *chunk_base, int N, int T, int H_qk, int H_v,
                           float scale, const void *bws, const void *states, const void *dsw,
                           const void *duw, void *dq, void *dk, float *dg, float *dbeta,
                           int item_lo, int item_hi, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_grad_kernel, dim3(grid), dim3(512), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), static_cast<const uint16_t *>(d_o),
                       static_cast<const uint16_t *>(dv), beta, cu_seqlens, chunk_base, N, T, H_qk,
                       H_v, scale, static_cast<const uint16_t *>(bws),
                       static_cast<const uint16_t *>(states), static_cast<const uint16_t *>(dsw),
                       static_cast<const uint16_t *>(duw), static_cast<uint16_t *>(dq),
                       static_cast<uint16_t *>(dk), dg, dbeta, item_lo, item_hi);
    return hipGetLastError();
}

}  // namespace gdn
