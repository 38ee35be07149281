// gdn_chunked.hip -- bf16 chunked prefill of the gated delta rule (chunk C = 64).
//
// The recurrence S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t
// ("从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力", sec. 2.2,
// with decay a_t = exp(g_t)) is rewritten per 64-token chunk.  With S the state
// at the chunk start, G_r = g_0 + ... + g_r, gamma_r = exp(G_r), L the last row:
//   A  = strictly-lower( b_r exp(G_r - G_i) k_r.k_i ),   T = (I + A)^{-1}
//   T' = T diag(b),   P = lower-incl( exp(G_r - G_i) scale q_r.k_i )
//   U  = T' (V - diag(gamma) K S^T)
//   O  = diag(gamma) scale Q S^T + P U
//   S' = gamma_L S + (diag(exp(G_L - G)) U)^T K
// (unrolling the token recurrence inside a chunk: every state is gamma_r S plus
// decayed rank-one terms u_i k_i^T whose coefficients solve a unit lower
// triangular system).  Exponents are always differences G_r - G_i with r >= i,
// so nothing overflows; gamma may underflow to 0, which is the exact limit.
//
// Three kernels:
//   plan  -- one workgroup: chunk offsets of every packed sequence.
//   prep  -- fully parallel, one wave per (chunk, QK head): K K^T and Q K^T on
//            bf16 MFMA (once, kept in registers); per V-head of the group the
//            gated A, its unit-lower-triangular inverse (fp32
//            substitution on the 16 x 16 diagonal blocks, bf16 MFMA for the
//            off-diagonal blocks), T', P and G, written to the workspace
//            (16.25 KiB per chunk and V-head).
//   scan  -- sequential over the chunks of one (sequence, V-head, 32-column slab
//            of d_v).  Four state waves split the 64 chunk rows (X = K S^T, R, U)
//            and the 128 d_k columns of the fp32 state (S' update, K^T read from
//            the K rows in LDS with transposing reads); four output waves on the
//            same SIMDs form O from the LDS copies of S and U, off the
//            recurrence's critical path.  The slab state never leaves the chip
//            between chunks: fp32 in MFMA accumulators, plus a bf16 copy in LDS
//            that feeds the next chunk's products.  Inputs are prefetched two
//            chunks ahead into three rotating register sets.
#include <stdint.h>

#include <mutex>

#include "gdn_chunk.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

// ------------------------------------------------------------------- plan
__global__ __launch_bounds__(256) void plan_kernel(const int32_t *__restrict__ cu, int N, int T,
                                                   int32_t *__restrict__ chunk_base) {
    __shared__ int part[256];
    int carry = 0;
    for (int base = 0; base < N; base += 256) {
        const int i = base + threadIdx.x;
        int cnt = 0;
        if (i < N) {
            const int s0 = cu ? cu[i] : 0, s1 = cu ? cu[i + 1] : T;
            cnt = (s1 - s0 + kChunk - 1) / kChunk;
        }
        part[threadIdx.x] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int y = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
            __syncthreads();
            part[threadIdx.x] += y;
            __syncthreads();
        }
        if (i < N) chunk_base[i] = carry + part[threadIdx.x] - cnt;
        carry += part[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) chunk_base[N] = carry;
}

// ------------------------------------------------------------------- prep
// Records (layout in gdn_chunk.h) are written with non-temporal stores: the
// scan reads them long after (a segment later, when prep and scan overlap),
// and they would otherwise displace the K and Q rows the scan's workgroups
// share through L2.

// One wave per (chunk, QK head) item; a workgroup holds 8 (forward) or 4
// (backward records) independent waves, each with its own LDS area, that step
// through the items [item_lo, item_hi) (item = chunk * H_qk + QK head) with
// the grid's stride.  A workgroup fills one CU, so a small grid stays on as
// many CUs as it has workgroups.  The K and Q rows of the chunk are loaded
// straight into MFMA operand registers: the A operand of a 16-row block and
// the B operand of K^T for the same block are the same fragment (row c of the
// block, 8 consecutive d_k), so K K^T and Q K^T need no LDS staging.  They are
// formed once, with the operands ordered so that each lane holds 4 consecutive
// columns of one row, and kept in registers for all V-heads of the QK head.
//
// With the prelude fused (kRaw), the wave first forms the chunk's K and Q rows
// from the raw projections: conv, SiLU and L2 norm with the conv prelude
// kernel's arithmetic and lane layout (16 lanes per row, 8 channels each, the
// norm reduced over the 16-lane row), so the rows come out bit-identical to
// the prelude's.  Each lane walks 16 consecutive rows, keeping the conv window
// in registers.  The normalised rows go to the workspace, where the scan reads
// them, and through LDS into the MFMA fragments.
//
// kRecs selects the records written per (chunk, V-head): the forward record
// (kRecFwd: T', P, G, read by the scan) and/or, for the backward pass, the
// backward record (kRecBwd, gdn_chunk.h: the fragments of T'^T and P^T, T
// row-major and G).
constexpr int kPrepWaves = 4;
constexpr int kRecFwd = 1, kRecBwd = 2;
static_assert(kChunk * kKP * sizeof(uint16_t) <= kChunk * kAP * sizeof(float),
              "a chunk's bf16 K or Q rows fit in a wave's A area");

struct RawIn {             // fused prelude inputs
    const uint16_t *x;     // [T][C_raw] bf16 raw projections, channels [q | k | v]
    const uint16_t *w;     // [C_raw][4] bf16 conv taps
    float eps;             // L2-norm epsilon
    uint16_t *kws, *qws;   // [chunks * 64][H_qk][128] bf16 normalised K and Q rows
    const uint16_t *hist;  // [N][3][C_raw] bf16: each sequence's three raw rows before its
                           // first token, oldest first (a resumed prefill), or null: zeros
};

struct GateIn {            // output gate fused into the scan's stores (kOutGated)
    const uint16_t *z;     // [T][H_v][128] bf16 gate projections
    const float *w;        // [128] norm weight
    float eps;             // norm epsilon
    uint16_t *y;           // [T][H_v][128] bf16 gated outputs
    uint64_t *part;        // [chunks][H_v][64 rows][4 slabs] tagged partial sums, zero on entry
};

// Waves per prep workgroup.  The forward-only prep keeps within 256 VGPRs and
// 18 KiB of LDS per wave, so a workgroup of 8 waves (two per SIMD, hiding each
// other's latency) fills one CU -- and, needing more than half of its LDS,
// never shares a CU with a second prep workgroup or a scan workgroup, so a
// prep grid of as many workgroups as idle CUs stays on at most that many
// CUs.  The backward forms need more registers: 4 waves, one per SIMD.
template <int kRecs> constexpr int kPrepWavesOf = kRecs == kRecFwd ? 8 : kPrepWaves;
template <bool kRaw, int kRecs = kRecFwd>
__global__ __launch_bounds__(64 * kPrepWavesOf<kRecs>) void prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const RawIn raw,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_base, int N, int T, int H_qk, int H_v, float scale,
    int item_lo, int item_hi, uint16_t *__restrict__ ws, uint16_t *__restrict__ bws = nullptr) {
    constexpr int kW = kPrepWavesOf<kRecs>;
    __shared__ __attribute__((aligned(16))) float sA_w[kW][kChunk * kAP];
    __shared__ __attribute__((aligned(16))) float sG_w[kW][kChunk];
    __shared__ __attribute__((aligned(16))) float sBt_w[kW][kChunk];

    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float *sA = sA_w[wv];
    uint16_t *sP = reinterpret_cast<uint16_t *>(sA);       // P (bf16 rows), before A is formed
    float *sG = sG_w[wv];
    float *sBt = sBt_w[wv];
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c = lane & 15;
    const int group = H_v / H_qk;
    const int hi = min(item_hi, chunk_base[N] * H_qk);
    for (int it = item_lo + (int)blockIdx.x * kW + wv; it < hi; it += (int)gridDim.x * kW) {
        const int gc = it / H_qk, hq = it - gc * H_qk;
        const int n = seq_of_chunk(chunk_base, N, gc);
        const int s0 = cu ? cu[n] : 0, s1 = cu ? cu[n + 1] : T;
        const int c0 = s0 + kChunk * (gc - chunk_base[n]);
        const int L = min(kChunk, s1 - c0);

        // gates of every V-head of the group (clamped indices: no load behind a branch)
        constexpr int kMaxGroup = kMaxPrepGroup;
        float graw[kMaxGroup], braw[kMaxGroup];
        const size_t grow = (size_t)(c0 + min(lane, L - 1)) * H_v + (size_t)hq * group;
#pragma unroll
        for (int vv = 0; vv < kMaxGroup; ++vv) {
            const int vc = min(vv, group - 1);
            graw[vv] = g[grow + vc];
            braw[vv] = beta[grow + vc];
        }

        // K and Q fragments: block I, k-step s -> row 16 I + c, d_k 32 s + 8 g4 .. +7
        uint4 kf[4][4], qf[4][4];
        if constexpr (kRaw) {
            // lane (sg, cg): rows 16 sg .. +15 of the chunk, channels 8 cg .. +7 of the head
            const int sg = lane >> 4, cg = lane & 15;
            const size_t C = (size_t)(2 * H_qk + H_v) * kD;
            uint16_t *rows = reinterpret_cast<uint16_t *>(sA);     // [64][kKP] bf16
#pragma unroll
            for (int m = 0; m < 2; ++m) {                           // K, then Q
                const size_t ch = (size_t)(m == 0 ? H_qk + hq : hq) * kD + 8 * cg;
                float wt[4][8];
                load_taps8(raw.w, ch, wt);
                // window x[r-3], x[r-2], x[r-1] for r = 16 sg; taps before the
                // sequence start read its history rows (zero without one)
                float win[3][8];
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const int r = 16 * sg - 3 + j;
                    const int rc = max(min(r, L - 1), s0 - c0);
                    const bool pre = c0 + r < s0;          // c0 + r - s0 in [-3, -1]
                    if (pre && !raw.hist) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
                    } else {
                        const uint16_t *src = pre ? raw.hist + ((size_t)n * 3 + 3 + (c0 + r - s0)) * C + ch
                                                  : raw.x + (size_t)(c0 + rc) * C + ch;
                        unpack8(*reinterpret_cast<const uint4 *>(src), win[j]);
                    }
                }
                uint16_t *dst = (m == 0 ? raw.kws : raw.qws) + ((size_t)gc * kChunk * H_qk + hq) * kD + 8 * cg;
                // the rows in two groups of 8, each in flight before its
                // arithmetic (the other wave on the SIMD hides the rest)
                u32x4 xr[8];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    if (j % 8 == 0) {
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            xr[i] = *reinterpret_cast<const u32x4 *>(raw.x + (size_t)(c0 + min(16 * sg + j + i, L - 1)) * C + ch);
                    }
                    const int r = 16 * sg + j;
                    float cur[8], y[8], ss = 0.f;
                    unpack8(__builtin_bit_cast(uint4, xr[j % 8]), cur);
                    conv_silu8(wt, win[0], win[1], win[2], cur, y, ss);
                    const float rn = rsqrtf(row16_sum(ss) + raw.eps);
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] *= rn;
                    const uint4 u = pack_bf8(y);
                    *reinterpret_cast<uint4 *>(dst + (size_t)r * H_qk * kD) = u;
                    *reinterpret_cast<uint4 *>(rows + r * kKP + 8 * cg) = u;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        win[0][e] = win[1][e];
                        win[1][e] = win[2][e];
                        win[2][e] = cur[e];
                    }
                }
                wave_lds_sync();
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const uint4 f = *reinterpret_cast<const uint4 *>(rows + (16 * I + c) * kKP + 32 * s + 8 * g4);
                        if (m == 0) kf[I][s] = f; else qf[I][s] = f;
                    }
                wave_lds_sync();                                    // read before the rows are rewritten
            }
        } else {
            const uint16_t *kc = k + (size_t)c0 * H_qk * kD;
            const uint16_t *qc = q + (size_t)c0 * H_qk * kD;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int off = (min(16 * I + c, L - 1) * H_qk + hq) * kD + 8 * g4;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    kf[I][s] = *reinterpret_cast<const uint4 *>(kc + off + 32 * s);
                    qf[I][s] = *reinterpret_cast<const uint4 *>(qc + off + 32 * s);
                }
            }
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const bool ok = 16 * I + c < L;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (!ok) kf[I][s] = make_uint4(0, 0, 0, 0);
                if (!ok) qf[I][s] = make_uint4(0, 0, 0, 0);
            }
        }

        // lower 16 x 16 tiles (J <= I); lane holds row 16 I + c, columns 16 J + 4 g4 + j:
        //   kk[I][J] = k_{16 I + c} . k_{16 J + 4 g4 + j}   (K K^T is symmetric)
        //   qk[I][J] = q_{16 I + c} . k_{16 J + 4 g4 + j}
        f32x4 kk[4][4], qk[4][4];
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                kk[I][J] = f32x4{0.f, 0.f, 0.f, 0.f};
                qk[I][J] = kk[I][J];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    kk[I][J] = mfma32(kf[J][s], kf[I][s], kk[I][J]);
                    qk[I][J] = mfma32(kf[J][s], qf[I][s], qk[I][J]);
                }
            }

#pragma unroll
        for (int vv = 0; vv < kMaxGroup; ++vv) {
            if (vv >= group) break;
            const int h = hq * group + vv;
            const float gl = lane < L ? graw[vv] : 0.f;
            const float bl = lane < L ? braw[vv] : 0.f;
            const float G = wave_scan(gl);
            sG[lane] = G;
            sBt[lane] = bl;
            constexpr bool kFwd = kRecs & kRecFwd, kBwd = kRecs & kRecBwd;
            uint16_t *rec = kFwd ? ws + ((size_t)gc * H_v + h) * kRecElems : nullptr;
            uint16_t *brec = kBwd ? bws + ((size_t)gc * H_v + h) * kBwdRecElems : nullptr;
            if constexpr (kFwd) {
                // the decays the scan applies, exponentiated once here
                const float GL = __shfl(G, kChunk - 1, 64);
                float *dec = reinterpret_cast<float *>(rec + kRecGam);
                __builtin_nontemporal_store(__expf(G), dec + lane);
                __builtin_nontemporal_store(__expf(GL - G), dec + kChunk + lane);
            }
            if constexpr (kBwd) reinterpret_cast<float *>(brec + kBwdGOff)[lane] = G;
            wave_lds_sync();

            // gated Q K^T -> P (bf16 rows in the wave's LDS area, zero above the
            // diagonal), stored out; then gated K K^T -> A (fp32 rows in the
            // same area, lower tiles)
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int row = 16 * I + c;
                const float Gr = sG[row];
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    if (J > I) {
                        *reinterpret_cast<uint2 *>(sP + row * kRP + 16 * J + 4 * g4) = make_uint2(0, 0);
                        continue;
                    }
                    const float4 Gv = *reinterpret_cast<const float4 *>(sG + 16 * J + 4 * g4);
                    const float gi[4] = {Gv.x, Gv.y, Gv.z, Gv.w};
                    float pv[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int col = 16 * J + 4 * g4 + j;
                        pv[j] = col <= row ? scale * __expf(Gr - gi[j]) * qk[I][J][j] : 0.f;
                    }
                    *reinterpret_cast<uint2 *>(sP + row * kRP + 16 * J + 4 * g4) = pk4(pv[0], pv[1], pv[2], pv[3]);
                }
            }
            wave_lds_sync();
            // P out as fragment blocks
            if constexpr (kFwd) {
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int a = qq >> 1, s = qq & 1;
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(sP + (16 * a + c) * kRP + 32 * s + 8 * g4),
                                                reinterpret_cast<u32x4 *>(rec + kTileElems + frag_off(a, s, lane)));
                }
            }
            if constexpr (kBwd) {
                // P^T block (a, s): lane (c, g4) holds P[32 s + 8 g4 + j][16 a + c], j = 0..7
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int a = qq >> 1, s = qq & 1;
                    uint16_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = sP[(32 * s + 8 * g4 + j) * kRP + 16 * a + c];
                    *reinterpret_cast<uint4 *>(brec + kBwdPtOff + frag_off(a, s, lane)) =
                        make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                                   e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
                }
            }
            wave_lds_sync();                                // P read before A overwrites it
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const int row = 16 * I + c;
                const float Gr = sG[row], br = sBt[row];
#pragma unroll
                for (int J = 0; J <= I; ++J) {
                    const float4 Gv = *reinterpret_cast<const float4 *>(sG + 16 * J + 4 * g4);
                    const float gi[4] = {Gv.x, Gv.y, Gv.z, Gv.w};
                    float av[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int col = 16 * J + 4 * g4 + j;
                        av[j] = col < row ? br * __expf(Gr - gi[j]) * kk[I][J][j] : 0.f;
                    }
                    *reinterpret_cast<float4 *>(sA + row * kAP + 16 * J + 4 * g4) = make_float4(av[0], av[1], av[2], av[3]);
                }
            }
            wave_lds_sync();

            float *A = sA;
            // Diagonal 16 x 16 blocks: lane (b, c) solves column c of block b by
            // forward substitution, T_bb = (I + A_bb)^{-1}, in fp32.
            {
                const int b = g4;
                float tc[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float acc = (r == c) ? 1.f : 0.f;
                    const float *Ar = A + (16 * b + r) * kAP + 16 * b;
#pragma unroll
                    for (int i = 0; i < r; ++i) acc -= Ar[i] * tc[i];
                    tc[r] = acc;
                }
                wave_lds_sync();
#pragma unroll
                for (int r = 0; r < 16; ++r) A[(16 * b + r) * kAP + 16 * b + c] = tc[r];
            }
            wave_lds_sync();

            // 16 x 16 x 16 MFMA operands from the fp32 block matrix: rows of block
            // (I, J) as an A operand, columns of block (I, J) as a B operand.
            auto rowop = [&](int I, int J) {
                const float *p = A + (16 * I + c) * kAP + 16 * J + 4 * g4;
                return to_bf4(p[0], p[1], p[2], p[3]);
            };
            auto colop = [&](int I, int J) {
                const float *p = A + (16 * I + 4 * g4) * kAP + 16 * J + c;
                return to_bf4(p[0], p[kAP], p[2 * kAP], p[3 * kAP]);
            };
            auto accop = [](f32x4 x) { return to_bf4(x[0], x[1], x[2], x[3]); };
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

            // Off-diagonal blocks of A are read before any is overwritten by T.
            const s16x4 a10 = rowop(1, 0), a21 = rowop(2, 1), a32 = rowop(3, 2);
            const s16x4 a20 = rowop(2, 0), a30 = rowop(3, 0), a31 = rowop(3, 1);

            // Blocks one below the diagonal: T_{I,I-1} = -T_II A_{I,I-1} T_{I-1,I-1}
            {
                const f32x4 y1 = mfma16(a10, colop(0, 0), z4);
                const f32x4 y2 = mfma16(a21, colop(1, 1), z4);
                const f32x4 y3 = mfma16(a32, colop(2, 2), z4);
                const f32x4 t10 = -mfma16(rowop(1, 1), accop(y1), z4);
                const f32x4 t21 = -mfma16(rowop(2, 2), accop(y2), z4);
                const f32x4 t32 = -mfma16(rowop(3, 3), accop(y3), z4);
                wave_lds_sync();
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    A[(16 + 4 * g4 + j) * kAP + c] = t10[j];
                    A[(32 + 4 * g4 + j) * kAP + 16 + c] = t21[j];
                    A[(48 + 4 * g4 + j) * kAP + 32 + c] = t32[j];
                }
            }
            wave_lds_sync();

            // Lower-left 32 x 32 block: T_[23][01] = -T_[23] A_[23][01] T_[01]
            {
                const f32x4 x20 = mfma16(a21, colop(1, 0), mfma16(a20, colop(0, 0), z4));
                const f32x4 x21 = mfma16(a21, colop(1, 1), z4);
                const f32x4 x30 = mfma16(a31, colop(1, 0), mfma16(a30, colop(0, 0), z4));
                const f32x4 x31 = mfma16(a31, colop(1, 1), z4);
                const s16x4 t22 = rowop(2, 2), t32r = rowop(3, 2), t33 = rowop(3, 3);
                const f32x4 t20 = -mfma16(t22, accop(x20), z4);
                const f32x4 t21b = -mfma16(t22, accop(x21), z4);
                const f32x4 t30 = -mfma16(t33, accop(x30), mfma16(t32r, accop(x20), z4));
                const f32x4 t31 = -mfma16(t33, accop(x31), mfma16(t32r, accop(x21), z4));
                wave_lds_sync();
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    A[(32 + 4 * g4 + j) * kAP + c] = t20[j];
                    A[(32 + 4 * g4 + j) * kAP + 16 + c] = t21b[j];
                    A[(48 + 4 * g4 + j) * kAP + c] = t30[j];
                    A[(48 + 4 * g4 + j) * kAP + 16 + c] = t31[j];
                }
            }
            wave_lds_sync();

            // T' = T diag(b) (zero above the diagonal blocks) out as fragment blocks
            if constexpr (kFwd) {
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int a = qq >> 1, s = qq & 1;
                    const int row = 16 * a + c, ca = 32 * s + 8 * g4, cb = ca + 4;
                    const float4 t0 = *reinterpret_cast<const float4 *>(A + row * kAP + ca);
                    const float4 t1 = *reinterpret_cast<const float4 *>(A + row * kAP + cb);
                    const float4 b0 = *reinterpret_cast<const float4 *>(sBt + ca);
                    const float4 b1 = *reinterpret_cast<const float4 *>(sBt + cb);
                    const bool la = (ca >> 4) <= a, lb = la;   // 8 columns in one 16-column block
                    const uint2 u0 = la ? pk4(t0.x * b0.x, t0.y * b0.y, t0.z * b0.z, t0.w * b0.w) : make_uint2(0, 0);
                    const uint2 u1 = lb ? pk4(t1.x * b1.x, t1.y * b1.y, t1.z * b1.z, t1.w * b1.w) : make_uint2(0, 0);
                    __builtin_nontemporal_store(u32x4{u0.x, u0.y, u1.x, u1.y},
                                                reinterpret_cast<u32x4 *>(rec + frag_off(a, s, lane)));
                }
            }
            if constexpr (kBwd) {
                // T'^T block (a, s): lane (c, g4) holds T'[r][16 a + c] for the rows
                // r = 32 s + 8 g4 + j (T' = T diag(b), rounded as above).  T is
                // held in the blocks at or below the diagonal; the rest is zero.
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int a = qq >> 1, s = qq & 1;
                    const int col = 16 * a + c;
                    const float bc = sBt[col];
                    float e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int r = 32 * s + 8 * g4 + j;
                        e[j] = (r >> 4) >= a ? A[r * kAP + col] * bc : 0.f;
                    }
                    const uint2 lo = pk4(e[0], e[1], e[2], e[3]), hi = pk4(e[4], e[5], e[6], e[7]);
                    *reinterpret_cast<uint4 *>(brec + kBwdTtOff + frag_off(a, s, lane)) =
                        make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
                // T row-major: lane r writes row r
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) {
                    const bool ok = (cb >> 1) <= (lane >> 4);
                    const float4 t0 = *reinterpret_cast<const float4 *>(A + lane * kAP + 8 * cb);
                    const float4 t1 = *reinterpret_cast<const float4 *>(A + lane * kAP + 8 * cb + 4);
                    const uint2 lo = ok ? pk4(t0.x, t0.y, t0.z, t0.w) : make_uint2(0, 0);
                    const uint2 hi = ok ? pk4(t1.x, t1.y, t1.z, t1.w) : make_uint2(0, 0);
                    *reinterpret_cast<uint4 *>(brec + kBwdTOff + lane * kChunk + 8 * cb) =
                        make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
            }
            wave_lds_sync();                 // T read before the next V-head's A is written
        }
    }
}

// ------------------------------------------------------------------- scan
constexpr int kSlabW = 32;                 // d_v columns per scan workgroup
constexpr int kSlabsW = kD / kSlabW;       // 4
constexpr int kVP = kSlabW + 8;            // LDS row stride (bf16) of the v staging rows

// Per-lane inputs of one chunk.  Every load reads a valid address (rows past
// the end of a sequence are clamped to its last row, chunk indices past the
// last chunk to the last chunk), so no load sits behind a branch; rows past
// the end only ever meet zero columns of T' and P, and results of the clamped
// chunks past the end are never used.
struct StateRegs {        // waves 0-3
    u32x4 kr[4];          // K row 16 w + 4 i + lane / 16, d_k 8 (lane % 16) .. +7
    u32x4 tA[2];          // T' row 16 w + c, columns 32 s + 8 g4 .. +7
    u32x4 vrow;           // v row 16 w + lane/4, slab columns 8 (lane%4) .. +7
    float4 gam4, lam4;    // gamma and lambda of rows 16 w + 4 g4 + j
    float gamL;           // gamma of the chunk's last row
};
struct OutRegs {          // waves 4-7
    u32x4 qr[4];          // Q row 16 w + 4 i + lane / 16, d_k 8 (lane % 16) .. +7
    u32x4 pA[2];          // P row 16 w + c, columns 32 s + 8 g4 .. +7
    float gown;           // gamma of row 16 w + c
    u32x4 xv, xvh;        // prelude fused: raw v row 16 w + lane / 4 and (lanes < 12)
                          // row 16 w - 3 + lane / 4, slab columns 8 (lane % 4) .. +7
    uint4 zr;             // gate fused: z of row 16 w + lane / 4, slab columns 8 (lane % 4) .. +7
};

// 512 threads: waves 0-3 carry the state through the chunks (X = K S^T, R,
// U = T' R, S' update), waves 4-7 produce the outputs (S Q^T, U^T P^T) from the
// LDS copies of S and U; waves w and w + 4 share a SIMD.  Wave w (mod 4) owns
// chunk rows 16 w .. +15 and d_k columns 32 w .. +31 of the state.  Three
// workgroup barriers per chunk: (1) R complete, (2) U complete, (3) S' complete.
// Inputs are loaded two chunks ahead into three rotating register sets.
//
// With the prelude fused (kRaw), K and Q rows come from prep's normalised rows
// in the workspace, and the output waves form the v slab: during chunk ci they
// apply conv and SiLU (the prelude's arithmetic) to the raw v rows of chunk
// ci + 1 and write them into the other half of a double-buffered v tile.
//
// kOut selects what the output waves write: kOutO the outputs o; kOutStates
// (the backward's own forward pass) no outputs but the bf16 state each chunk
// starts from (the values the chunk's products use), copied out of LDS into
// states [chunk][H_v][d_v][d_k]; kOutBoth both (a forward pass that keeps the
// states for a later backward); kOutGated o and the gated outputs y.  (Stores
// issued by the state waves would lengthen their chain: the waits for their
// own prefetched loads would also cover the stores.)
//
// kOutGated: the gate divides each 128-wide row of o by its RMS, and the
// four slab workgroups of a V-head each hold 32 columns.  Output wave w of
// each publishes, per row of its 16, the sum of squares of its 32 bf16
// outputs, summed exactly as the gated-norm kernel's 16-lane row sums them
// (per 8 channels a chained fma, then pairs, then the pair sums), as one 64-bit
// word (the chunk's index + 1 in the high half, the fp32 sum in the low half;
// the words are zeroed at the start of the call) stored with a
// relaxed device-scope atomic: each word is valid by itself, so no fence
// orders it against other memory.  Three chunks later the wave reads the four
// words of its rows (spinning, bounded, until all four tags are set), adds
// them as the row sum's last two levels do, and stores its 32 columns of y.
// A wave waits only for workgroups of the same launch; the launcher takes this
// path only when the whole grid fits on the device at once (one workgroup per
// CU), so every waited-for workgroup runs.
constexpr int kOutO = 0, kOutStates = 1, kOutBoth = 2, kOutGated = 3;
constexpr int kGateSpin = 1 << 22;    // bound on a wave's polls for the other slabs' sums
constexpr int kGateLag = 3;           // chunks between a chunk's outputs and its gate
template <bool kRaw, int kOut = kOutO>
__global__ __launch_bounds__(512) void scan_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const RawIn raw, const float *initial_state, float *final_state, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_base, int N, int T, int H_qk, int H_v, float scale,
    int c_lo, int c_hi, const uint16_t *__restrict__ ws, uint16_t *o,
    uint16_t *__restrict__ states = nullptr, const GateIn gate = GateIn{}) {
    constexpr int kVBufs = 2;
    __shared__ __attribute__((aligned(16))) uint16_t sS[kSlabW * kKP];
    __shared__ __attribute__((aligned(16))) uint16_t sR[kSlabW * kRP];
    __shared__ __attribute__((aligned(16))) uint16_t sU[kSlabW * kRP];
    __shared__ __attribute__((aligned(16))) uint16_t sUs[kSlabW * kRP];
    __shared__ __attribute__((aligned(16))) uint16_t sKr[2][kChunk * kKP];   // K rows of the chunk (double-buffered)
    __shared__ __attribute__((aligned(16))) uint16_t sV[kVBufs][kChunk * kVP];   // v rows of the chunk (slab columns)
    __shared__ __attribute__((aligned(16))) uint16_t sQ[4][16 * kKP];     // each output wave's Q rows
    __shared__ __attribute__((aligned(16))) uint16_t sXv[kRaw ? 4 : 1][20 * kVP];   // raw v rows per output wave
    constexpr int kGw = kOut == kOutGated ? 4 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t sGo[kGw][16 * kSlabW];   // kOutGated: a wave's o rows (row-major)
    __shared__ uint4 sGz[kGw][64];                 // and its z, output to state wave

    // Workgroup -> (sequence, V-head, slab): the workgroups of one QK group of
    // one sequence share an XCD's L2 (they read the same K and Q rows), and the
    // groups of every sequence are spread over the eight XCDs.
    const int u = xcd_group_unit((H_v / H_qk) * kSlabsW);
    const int slab = u % kSlabsW;
    const int nh = u / kSlabsW;
    const int h = nh % H_v, n = nh / H_v;
    const int hq = h / (H_v / H_qk);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = wave & 3;
    const int lane = threadIdx.x & 63, g4 = lane >> 4, c = lane & 15;
    const int s0 = cu ? cu[n] : 0, s1 = cu ? cu[n + 1] : T;
    // chunks [c_lo, c_end) of the sequence: the state enters as initial_state
    // and leaves as final_state, so a sequence can be scanned in segments
    const int c_end = min((s1 - s0 + kChunk - 1) / kChunk, c_hi);
    const int cbase = chunk_base[n];
    const int e0 = kSlabW * slab;           // first d_v column of the slab
    const size_t st_off = ((size_t)n * H_v + h) * (kD * kD);
    auto rec_of = [&](int ci) { return ws + ((size_t)(cbase + ci) * H_v + h) * kRecElems; };
    auto chunk_len = [&](int ci) { return min(kChunk, s1 - (s0 + kChunk * ci)); };
    // K and Q rows are loaded whole (16 lanes x 16 B per row, 4 rows per
    // instruction: every cache line fully used) and regrouped into MFMA
    // fragments through LDS.  Row 16 w + 4 i + lane / 16, 16-byte piece
    // lane % 16, of chunk ci: a chunk base common to the wave plus a 32-bit
    // lane offset.  Prep's chunk-aligned rows in the workspace are read as
    // they are (rows past a sequence's end hold finite values that meet only
    // zero columns of T' and P); rows of the caller's q, k are clamped into
    // the sequence.
    auto krow_ptr = [&](const uint16_t *base, int ci, int i) {
        const int r = 16 * w + 4 * i + (lane >> 4);
        const size_t row0 = kRaw ? (size_t)(cbase + ci) * kChunk : (size_t)(s0 + kChunk * ci);
        const int rc = kRaw ? r : min(r, chunk_len(ci) - 1);
        return reinterpret_cast<const u32x4 *>(base + row0 * H_qk * kD +
                                               (uint32_t)(__umul24(rc, H_qk * kD) + hq * kD + 8 * (lane & 15)));
    };
    const uint16_t *kin = kRaw ? raw.kws : k;
    const uint16_t *qin = kRaw ? raw.qws : q;

    // kOutGated: rows of a wave's o tile in the gated-norm kernel's lane layout
    const int gr = lane >> 2, gq = lane & 3;
    // x_l + x_(l^1), then + x_(l^2): the first two levels of the 16-lane row sum
    auto quad_sum = [](float x) {
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
        return x;
    };
    // publish the sum of squares of this slab's 32 columns of row 16 w + r
    auto publish = [&](int cj, const uint4 &o8) {
        float ov[8];
        unpack8(o8, ov);
        float l = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) l = __builtin_fmaf(ov[e], ov[e], l);
        const float sq = quad_sum(l);
        if (gq == 0) {
            uint64_t *pw = gate.part + (((size_t)(cbase + cj) * H_v + h) * kChunk + 16 * w + gr) * kSlabsW + slab;
            __hip_atomic_store(pw, (uint64_t(cbase + cj + 1) << 32) | __float_as_uint(sq),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    if (wave < 4) {
        // ---------------- state waves
        // st[t][nt] holds S[e0 + 16 nt + c][32 w + 16 t + 4 g4 + j] in fp32
        f32x4 st[2][2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                if (initial_state) {
                    const float4 x = *reinterpret_cast<const float4 *>(
                        initial_state + st_off + (size_t)(e0 + 16 * nt + c) * kD + 32 * w + 16 * t + 4 * g4);
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
        auto fetch_a = [&](int ci, StateRegs &R) {
            ci = min(ci, c_end - 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) R.kr[i] = *krow_ptr(kin, ci, i);
            const uint16_t *rec = rec_of(ci);
#pragma unroll
            for (int s = 0; s < 2; ++s)
                R.tA[s] = *reinterpret_cast<const u32x4 *>(rec + frag_off(w, s, lane));
        };
        auto fetch_b = [&](int ci, StateRegs &R) {
            ci = min(ci, c_end - 1);
            const float *dp = reinterpret_cast<const float *>(rec_of(ci) + kRecGam);
            R.gam4 = *reinterpret_cast<const float4 *>(dp + 16 * w + 4 * g4);
            R.lam4 = *reinterpret_cast<const float4 *>(dp + kChunk + 16 * w + 4 * g4);
            R.gamL = dp[kChunk - 1];
            if constexpr (!kRaw) {
                const int vr = min(16 * w + (lane >> 2), chunk_len(ci) - 1);
                const uint16_t *vb = v + ((size_t)(s0 + kChunk * ci) * H_v + h) * kD + e0;
                R.vrow = *reinterpret_cast<const u32x4 *>(vb + (uint32_t)(__umul24(vr, H_v * kD) + 8 * (lane & 3)));
            }
        };

        // kOutGated, run by state wave w on the outputs of output wave w,
        // handed over in LDS: lane (r, q) = (lane / 4, lane % 4) holds row
        // 16 w + r, slab columns 8 q .. +7 of o (bf16 as stored) and of z --
        // the gated-norm kernel's layout, so the row sum is its sum: each lane
        // chains its 8 squares, quads add pairs then pair sums.  gw: the norm
        // weight of the lane's columns.
        float gw[8];
        if constexpr (kOut == kOutGated) {
            const float4 t0 = *reinterpret_cast<const float4 *>(gate.w + e0 + 8 * gq);
            const float4 t1 = *reinterpret_cast<const float4 *>(gate.w + e0 + 8 * gq + 4);
            gw[0] = t0.x; gw[1] = t0.y; gw[2] = t0.z; gw[3] = t0.w;
            gw[4] = t1.x; gw[5] = t1.y; gw[6] = t1.z; gw[7] = t1.w;
        }
        auto part_of = [&](int cj) {   // this lane's word: row 16 w + r, slab q
            return gate.part + (((size_t)(cbase + cj) * H_v + h) * kChunk + 16 * w + gr) * kSlabsW + gq;
        };
        // wd: the lane's word as read earlier (polled again until all are set)
        auto apply_gate = [&](int cj, const uint4 &o8, const uint4 &z8, uint64_t wd) {
            const uint64_t *pw = part_of(cj);
            const uint32_t tag = (uint32_t)(cbase + cj + 1);
            // the first check outside the poll loop: it waits for this word's
            // own read only (a loop that rereads the word makes the compiler
            // wait for every vector memory operation in flight at its head)
            if (!__all((uint32_t)(wd >> 32) == tag)) {
                for (int t = 0; t < kGateSpin; ++t) {
                    __builtin_amdgcn_s_sleep(1);
                    wd = __hip_atomic_load(pw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (__all((uint32_t)(wd >> 32) == tag)) break;
                }
            }
            // slab q's sum in lane q of the quad; the row's total in every lane
            const float inv = rsqrtf(quad_sum(__uint_as_float((uint32_t)wd)) * (1.f / 128) + gate.eps);
            if (16 * w + gr < chunk_len(cj)) {
                float ov[8], zv[8], y[8];
                unpack8(o8, ov);
                unpack8(z8, zv);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = ov[e] * inv * gw[e] * silu(zv[e]);
                const uint4 yv = pack_bf8(y);
                uint16_t *yb = gate.y + ((size_t)(s0 + kChunk * cj) * H_v + h) * kD + e0;
                __builtin_nontemporal_store(u32x4{yv.x, yv.y, yv.z, yv.w},
                                            reinterpret_cast<u32x4 *>(yb + (uint32_t)(__umul24(16 * w + gr, H_v * kD) + 8 * gq)));
            }
        };
        // chunks whose gate is pending (kGateLag of them, oldest first), with
        // their o and z; a chunk is gated kGateLag chunks after its sums are
        // published, when the other slabs have long published theirs
        int pend[kGateLag];
        uint4 pend_o[kGateLag], pend_z[kGateLag];
#pragma unroll
        for (int i = 0; i < kGateLag; ++i) {
            pend[i] = -1;
            pend_o[i] = pend_z[i] = make_uint4(0, 0, 0, 0);
        }
        // the outputs of chunk cj (in LDS; their sums are published later in
        // the same body): gate the oldest pending chunk (gword: its words,
        // read earlier), then queue cj
        auto gate_step = [&](int cj, uint64_t gword) {
            const uint4 oc = *reinterpret_cast<const uint4 *>(sGo[w] + gr * kSlabW + 8 * gq);
            const uint4 zc = sGz[w][lane];
            if (pend[0] >= 0) apply_gate(pend[0], pend_o[0], pend_z[0], gword);
#pragma unroll
            for (int i = 0; i + 1 < kGateLag; ++i) {
                pend[i] = pend[i + 1];
                pend_o[i] = pend_o[i + 1];
                pend_z[i] = pend_z[i + 1];
            }
            pend[kGateLag - 1] = cj;
            pend_o[kGateLag - 1] = oc;
            pend_z[kGateLag - 1] = zc;
        };
        // the words of pending chunk i (device-scope reads are slow: the words
        // of the chunk gated in the next body are read in this one)
        auto gate_word = [&](int i) -> uint64_t {
            return pend[i] >= 0 ? __hip_atomic_load(part_of(pend[i]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : uint64_t(0);
        };
        uint64_t gword_next = 0;
        // this wave's 16 rows of K (and, prelude not fused, of v) of chunk cj
        // into LDS, row-major, written a chunk ahead (the output waves write
        // v when the prelude is fused)
        auto stage_rows = [&](int cj, const StateRegs &R) {
            if constexpr (!kRaw)
                *reinterpret_cast<u32x4 *>(sV[cj & 1] + (16 * w + (lane >> 2)) * kVP + 8 * (lane & 3)) = R.vrow;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4 *>(sKr[cj & 1] + (16 * w + 4 * i + (lane >> 4)) * kKP + 8 * (lane & 15)) = R.kr[i];
        };
        uint4 kA[4];              // K row 16 w + c, d_k 32 s + 8 g4 .. +7 of the chunk about to run
        auto read_ka = [&](int cj) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kA[s] = *reinterpret_cast<const uint4 *>(sKr[cj & 1] + (16 * w + c) * kKP + 32 * s + 8 * g4);
        };
        auto body = [&](int ci, StateRegs &cur, StateRegs &nxt, StateRegs &pf) {
            // the previous chunk's outputs (handed over before its barrier
            // (3)), gated first: a wait here finds only the previous chunk's
            // memory operations in flight (the next chunks' loads are issued
            // after it), and the output waves reach barrier (1) long after
            // this wave would otherwise; then the words of the chunk the next
            // body gates
            if constexpr (kOut == kOutGated) {
                if (ci > c_lo) gate_step(ci - 1, gword_next);
                gword_next = gate_word(0);
            }
            // K's MFMA fragments (kA) were read out of this wave's own rows,
            // staged in LDS, at the end of the previous chunk
            const uint16_t *sVc = sV[ci & 1];
            const uint16_t *sKc = sKr[ci & 1];
            fetch_a(ci + 2, pf);
            const float gam[4] = {cur.gam4.x, cur.gam4.y, cur.gam4.z, cur.gam4.w};
            const float dec[4] = {cur.lam4.x, cur.lam4.y, cur.lam4.z, cur.lam4.w};
            const float gamL = cur.gamL;

            // X = K S^T for chunk rows 16 w .. +15, both d_v tiles
            f32x4 ax[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    ax[nt] = mfma32(kA[s], *reinterpret_cast<const uint4 *>(sS + (16 * nt + c) * kKP + 32 * s + 8 * g4), ax[nt]);
            // R = V - diag(gamma) X, stored transposed ([d_v column][chunk row]);
            // v arrives in the C layout of X through a transposing read
            wave_lds_sync();
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const uint2 vv = lds_read_tr16(sVc + (16 * w + 4 * g4 + (c >> 2)) * kVP + 16 * nt + 4 * (c & 3));
                float r[4];
                r[0] = __uint_as_float(vv.x << 16) - gam[0] * ax[nt][0];
                r[1] = __uint_as_float(vv.x & 0xFFFF0000u) - gam[1] * ax[nt][1];
                r[2] = __uint_as_float(vv.y << 16) - gam[2] * ax[nt][2];
                r[3] = __uint_as_float(vv.y & 0xFFFF0000u) - gam[3] * ax[nt][3];
                *reinterpret_cast<uint2 *>(sR + (16 * nt + c) * kRP + 16 * w + 4 * g4) = pk4(r[0], r[1], r[2], r[3]);
            }
            // the sums of the previous chunk's outputs, published while the
            // output waves still form this chunk's O and v
            if constexpr (kOut == kOutGated)
                if (ci > c_lo) publish(ci - 1, pend_o[kGateLag - 1]);
            __syncthreads();                                   // (1) R complete
            // U = T' R (T' is lower triangular: k-steps up to this row block)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 au = mfma32(cur.tA[0], *reinterpret_cast<const uint4 *>(sR + (16 * nt + c) * kRP + 8 * g4),
                                  f32x4{0.f, 0.f, 0.f, 0.f});
                if (w >= 2)
                    au = mfma32(cur.tA[1], *reinterpret_cast<const uint4 *>(sR + (16 * nt + c) * kRP + 32 + 8 * g4), au);
                *reinterpret_cast<uint2 *>(sU + (16 * nt + c) * kRP + 16 * w + 4 * g4) = pk4(au[0], au[1], au[2], au[3]);
                *reinterpret_cast<uint2 *>(sUs + (16 * nt + c) * kRP + 16 * w + 4 * g4) =
                    pk4(dec[0] * au[0], dec[1] * au[1], dec[2] * au[2], dec[3] * au[3]);
            }
            fetch_b(ci + 2, pf);
            // the state update's K^T fragments and gamma_L S, ahead of barrier
            // (2): they do not depend on U.  K^T row 32 w + 16 t + c, chunk rows
            // 32 s + 8 g4 .. +7: two transposing reads
            uint4 ub[2][2], ka[2][2];
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const uint16_t *base = sKc + (32 * s + 8 * g4 + (c >> 2)) * kKP + 32 * w + 16 * t + 4 * (c & 3);
                    const uint2 lo = lds_read_tr16(base);
                    const uint2 hi = lds_read_tr16(base + 4 * kKP);
                    ka[t][s] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) st[t][nt] = gamL * st[t][nt];
            __syncthreads();                                   // (2) U complete
            // S' = gamma_L S + (diag(exp(G_L - G)) U)^T K   (d_k 32 w .. +31)
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    ub[nt][s] = *reinterpret_cast<const uint4 *>(sUs + (16 * nt + c) * kRP + 32 * s + 8 * g4);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f32x4 as = st[t][nt];
#pragma unroll
                    for (int s = 0; s < 2; ++s) as = mfma32(ka[t][s], ub[nt][s], as);
                    st[t][nt] = as;
                }
            stage_rows(ci + 1, nxt);       // the other buffers: last read in chunk ci - 1
            write_state_lds();
            wave_lds_sync();
            read_ka(ci + 1);
            __syncthreads();                                   // (3) S' complete
        };

        write_state_lds();
        StateRegs r0, r1, r2;
        if (c_lo < c_end) {
            fetch_a(c_lo, r0);
            fetch_b(c_lo, r0);
            fetch_a(c_lo + 1, r1);
            fetch_b(c_lo + 1, r1);
            stage_rows(c_lo, r0);
            wave_lds_sync();
            read_ka(c_lo);
        }
        __syncthreads();
        for (int ci = c_lo; ci < c_end; ci += 3) {
            body(ci, r0, r1, r2);
            if (ci + 1 >= c_end) break;
            body(ci + 1, r1, r2, r0);
            if (ci + 2 >= c_end) break;
            body(ci + 2, r2, r0, r1);
        }
        if constexpr (kOut == kOutGated) {
            if (c_lo < c_end) {                  // handed over before the last barrier
                gate_step(c_end - 1, gword_next);
                publish(c_end - 1, pend_o[kGateLag - 1]);
            }
#pragma unroll
            for (int i = 0; i < kGateLag; ++i)
                if (pend[i] >= 0)
                    apply_gate(pend[i], pend_o[i], pend_z[i],
                               __hip_atomic_load(part_of(pend[i]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        if (final_state) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    *reinterpret_cast<float4 *>(final_state + st_off + (size_t)(e0 + 16 * nt + c) * kD + 32 * w + 16 * t + 4 * g4) =
                        make_float4(st[t][nt][0], st[t][nt][1], st[t][nt][2], st[t][nt][3]);
        }
    } else if constexpr (kOut == kOutStates) {
        // ---------------- output waves, backward pass: the start states out
        const int ol = threadIdx.x - 256;
        __syncthreads();                                       // matches the state waves' first barrier
        for (int ci = c_lo; ci < c_end; ++ci) {
            // sS holds the state chunk ci starts from until its barrier (2)
            uint16_t *sp = states + ((size_t)(cbase + ci) * H_v + h) * (kD * kD) + (size_t)e0 * kD;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int e = ol + 256 * m, r = e >> 4, pcs = 8 * (e & 15);
                *reinterpret_cast<u32x4 *>(sp + r * kD + pcs) = *reinterpret_cast<const u32x4 *>(sS + r * kKP + pcs);
            }
            __syncthreads();                                   // (1)
            __syncthreads();                                   // (2)
            __syncthreads();                                   // (3)
        }
    } else {
        // ---------------- output waves
        // prelude fused: raw v rows of the slab, rows x row stride C
        const int C = (2 * H_qk + H_v) * kD;
        const size_t vch = (size_t)(2 * H_qk + h) * kD + e0 + 8 * (lane & 3);
        const int pr = lane >> 2;                  // this lane's row within the wave's 16
        auto fetch = [&](int ci, OutRegs &R) {
            ci = min(ci, c_end - 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) R.qr[i] = *krow_ptr(qin, ci, i);
            const uint16_t *rec = rec_of(ci);
#pragma unroll
            for (int s = 0; s < 2; ++s)
                R.pA[s] = *reinterpret_cast<const u32x4 *>(rec + kTileElems + frag_off(w, s, lane));
            R.gown = reinterpret_cast<const float *>(rec + kRecGam)[16 * w + c];
            if constexpr (kOut == kOutGated) {
                const int Lz = chunk_len(ci);
                const uint16_t *zb = gate.z + ((size_t)(s0 + kChunk * ci) * H_v + h) * kD + e0;
                R.zr = *reinterpret_cast<const uint4 *>(zb + __umul24(min(16 * w + (lane >> 2), Lz - 1), H_v * kD) +
                                                        8 * (lane & 3));
            }
            if constexpr (kRaw) {
                // rows clamped into the sequence; halo rows before its start
                // are replaced by zero when used
                const int Lc = chunk_len(ci), c0 = s0 + kChunk * ci;
                const int r = min(16 * w + pr, Lc - 1);
                const int rel = kChunk * ci + 16 * w - 3 + min(pr, 2);      // halo row, from the sequence start
                const int rh = max(min(16 * w - 3 + min(pr, 2), Lc - 1), -kChunk * ci);
                const uint16_t *xb = raw.x + (size_t)c0 * C + (2 * H_qk + h) * kD + e0;
                R.xv = *reinterpret_cast<const u32x4 *>(xb + (__mul24(r, C) + 8 * (lane & 3)));
                // a halo row before the sequence start comes from its history (rel in [-3, -1])
                const uint16_t *hsrc = rel < 0 && raw.hist
                                           ? raw.hist + ((size_t)n * 3 + 3 + max(rel, -3)) * C + (2 * H_qk + h) * kD + e0
                                           : xb + __mul24(rh, C);
                R.xvh = *reinterpret_cast<const u32x4 *>(hsrc + 8 * (lane & 3));
            }
        };
        // v of chunk cj (raw rows in R) -> conv, SiLU -> sV[cj & 1], rows 16 w .. +15
        float wv[4][8];
        if constexpr (kRaw) load_taps8(raw.w, vch, wv);
        auto v_conv = [&](int cj, const OutRegs &R) {
            uint16_t *xs = sXv[w];                 // rows 0-2: halo, 3-18: the wave's rows, 19: unused
            const int pc = 8 * (lane & 3);
            *reinterpret_cast<u32x4 *>(xs + (3 + pr) * kVP + pc) = R.xv;
            // ahead of the sequence start: its history row, or zero without one
            const bool before = kChunk * cj + 16 * w - 3 + pr < 0 && !raw.hist;
            *reinterpret_cast<u32x4 *>(xs + (lane < 12 ? pr : 19) * kVP + pc) =
                before ? u32x4{0u, 0u, 0u, 0u} : R.xvh;
            wave_lds_sync();
            float xm[4][8], y[8], ss = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) unpack8(*reinterpret_cast<const uint4 *>(xs + (pr + j) * kVP + pc), xm[j]);
            conv_silu8(wv, xm[0], xm[1], xm[2], xm[3], y, ss);
            *reinterpret_cast<uint4 *>(sV[cj & 1] + (16 * w + pr) * kVP + pc) = pack_bf8(y);
        };
        auto body = [&](int ci, OutRegs &cur, OutRegs &nxt, OutRegs &pf) {
            const int c0 = s0 + kChunk * ci;
            const int L = min(kChunk, s1 - c0);
            // this wave's Q rows through its LDS area into MFMA fragments
            uint16_t *q_lds = sQ[w];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<u32x4 *>(q_lds + (4 * i + (lane >> 4)) * kKP + 8 * (lane & 15)) = cur.qr[i];
            wave_lds_sync();
            uint4 qA[4];          // Q row 16 w + c, d_k 32 s + 8 g4 .. +7
#pragma unroll
            for (int s = 0; s < 4; ++s) qA[s] = *reinterpret_cast<const uint4 *>(q_lds + c * kKP + 32 * s + 8 * g4);
            // O^T = S Q^T (the S fragments are the A operand); lane holds
            // O[16 w + c][16 nt + 4 g4 + j]
            f32x4 ao[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    ao[nt] = mfma32(*reinterpret_cast<const uint4 *>(sS + (16 * nt + c) * kKP + 32 * s + 8 * g4), qA[s], ao[nt]);
            const float gsc = scale * cur.gown;
            // the next chunk's v slab (its buffer was last read before this
            // chunk began), before barrier (1): the state waves form X and R
            // meanwhile, and the VALU work then stays off the U phase, which
            // barrier (2) ends
            if constexpr (kRaw) v_conv(ci + 1, nxt);   // past the last chunk: written, never read
            __syncthreads();                                   // (1)
            // next loads issued while the state waves form U: the vector
            // memory pipe is then quiet while they form X and R
            fetch(ci + 2, pf);
            if constexpr (kOut == kOutBoth) {
                // sS holds the state chunk ci starts from until barrier (2); the
                // copy is read only by a later backward: non-temporal stores,
                // issued after this chunk's loads (1180 µs per 32768-token call
                // against 1240 with cached stores before barrier (1))
                uint16_t *sp = states + ((size_t)(cbase + ci) * H_v + h) * (kD * kD) + (size_t)e0 * kD;
                const int ol = threadIdx.x - 256;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int e = ol + 256 * m, r = e >> 4, pcs = 8 * (e & 15);
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(sS + r * kKP + pcs),
                                                reinterpret_cast<u32x4 *>(sp + r * kD + pcs));
                }
            }
            __syncthreads();                                   // (2) U complete
            // O^T += U^T P^T  (P is lower triangular: k-steps up to this row block)
            const bool row_ok = 16 * w + c < L;
            uint16_t *ob = o + ((size_t)c0 * H_v + h) * kD + e0;
            uint2 opk[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                f32x4 a = gsc * ao[nt];
                a = mfma32(*reinterpret_cast<const uint4 *>(sU + (16 * nt + c) * kRP + 8 * g4), cur.pA[0], a);
                if (w >= 2)
                    a = mfma32(*reinterpret_cast<const uint4 *>(sU + (16 * nt + c) * kRP + 32 + 8 * g4), cur.pA[1], a);
                opk[nt] = pk4(a[0], a[1], a[2], a[3]);
                if (row_ok)
                    *reinterpret_cast<uint2 *>(ob + (uint32_t)(__umul24(16 * w + c, H_v * kD) + 16 * nt + 4 * g4)) =
                        opk[nt];
            }
            if constexpr (kOut == kOutGated) {      // to state wave w, which gates them
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    *reinterpret_cast<uint2 *>(sGo[w] + c * kSlabW + 16 * nt + 4 * g4) = opk[nt];
                sGz[w][lane] = cur.zr;
            }
            __syncthreads();                                   // (3)
        };
        OutRegs r0, r1, r2;
        if (c_lo < c_end) {
            fetch(c_lo, r0);
            fetch(c_lo + 1, r1);
            if constexpr (kRaw) v_conv(c_lo, r0);
        }
        __syncthreads();                                       // matches the state waves' first barrier
        for (int ci = c_lo; ci < c_end; ci += 3) {
            body(ci, r0, r1, r2);
            if (ci + 1 >= c_end) break;
            body(ci + 1, r1, r2, r0);
            if (ci + 2 >= c_end) break;
            body(ci + 2, r2, r0, r1);
        }
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// A single sequence leaves CUs idle during the scan (one workgroup per
// (V-head, slab)).  Its chunks are then split into segments: the prep of
// segment i + 1 runs on the idle CUs, on an auxiliary stream, while segment i
// is scanned; only the first segment's prep runs alone.  Segment i holds a
// share of the chunks proportional to growth^i, with the count chosen so that
// the first segment is at most about kFirstSegChunks long.  The growth is a
// little below the ratio of the scan's time per chunk to the prep's on the
// idle CUs (about 1 / 0.85 for the prep alone), which leaves room for the
// event hand-over.  With the prelude fused the prep also forms K and Q and
// the ratio differs.
constexpr int kMaxSegments = 12;
constexpr double kSegGrowth = 1.1;
constexpr double kSegGrowthRaw = 1.0;
constexpr double kSegGrowthRev = 1.0;   // the backward's reverse scan (walked last to first)
constexpr int kFirstSegChunks = 128;
constexpr int kSegMinChunks = 64;     // shorter sequences are not split
constexpr int kMinIdleCUs = 32;       // fewer idle CUs: not split

// Segment bounds b[0] = 0 < b[1] < ... < b[count] = nch; returns count.
int segment_bounds(int nch, double growth, int *b) {
    int count = 2;
    double wsum = 1.0 + growth, wnext = growth * growth;
    while (count < kMaxSegments && nch / wsum > kFirstSegChunks) {
        wsum += wnext;
        wnext *= growth;
        ++count;
    }
    double w = 1.0, acc = 0.0;
    b[0] = 0;
    for (int i = 1; i < count; ++i, w *= growth) {
        acc += w;
        b[i] = max(b[i - 1] + 1, (int)(nch * acc / wsum));
    }
    b[count] = nch;
    return count;
}

// Events: one per segment, and two more for the backward's chunk gradients
// beside its reverse scan.
constexpr int kEvRscan = kMaxSegments, kEvGrad = kMaxSegments + 1, kAuxEvents = kMaxSegments + 2;
struct DeviceAux {           // per device, created on first use, never destroyed
    bool tried = false, ok = false;
    int cus = 0;
    hipStream_t stream = nullptr;
    hipEvent_t ev[kAuxEvents] = {};
};
constexpr int kMaxDevices = 64;
std::mutex g_aux_mu;         // guards g_aux and every enqueue on an auxiliary stream
DeviceAux g_aux[kMaxDevices];

// The current device's auxiliary stream (default priority) and events, or
// nullptr if they cannot be made or `s` is under graph capture (a captured
// call stays on the caller's stream: it runs unsegmented, with the same
// results, since segments hand the fp32 state over unchanged).  Caller holds
// g_aux_mu.
DeviceAux *device_aux(hipStream_t s) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    DeviceAux &a = g_aux[dev];
    if (!a.tried) {
        a.tried = true;
        bool ok = hipDeviceGetAttribute(&a.cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                  hipStreamCreateWithFlags(&a.stream, hipStreamNonBlocking) == hipSuccess;
        for (int i = 0; ok && i < kAuxEvents; ++i)
            ok = hipEventCreateWithFlags(&a.ev[i], hipEventDisableTiming | hipEventReleaseToDevice) ==
                 hipSuccess;
        a.ok = ok;
    }
    return a.ok ? &a : nullptr;
}

}  // namespace

namespace {

// Workspace: chunk offsets | chunk records | (prelude fused) K rows, Q rows |
// (one sequence) the state carried between segments | (gate fused) the
// tagged partial sums of squares.
struct Workspace {
    int32_t *chunk_base;
    uint16_t *rec, *kws, *qws;
    float *carry;
    uint64_t *part;
};
size_t workspace_layout(int N, int T, int H_qk, int H_v, bool raw, void *base, Workspace *wsp,
                        bool gated = false) {
    const size_t max_chunks = (size_t)(T + kChunk - 1) / kChunk + (size_t)N;
    const size_t head = align256((size_t)(N + 1) * sizeof(int32_t));
    const size_t rec = max_chunks * (size_t)H_v * kRecElems * sizeof(uint16_t);   // 256-byte multiple
    const size_t rows = raw ? max_chunks * kChunk * (size_t)H_qk * kD * sizeof(uint16_t) : 0;
    const size_t carry = N == 1 ? (size_t)H_v * kD * kD * sizeof(float) : 0;
    const size_t part = gated ? max_chunks * (size_t)H_v * kChunk * kSlabsW * sizeof(uint64_t) : 0;
    if (wsp) {
        char *p = static_cast<char *>(base);
        wsp->chunk_base = reinterpret_cast<int32_t *>(p);
        wsp->rec = reinterpret_cast<uint16_t *>(p + head);
        wsp->kws = reinterpret_cast<uint16_t *>(p + head + rec);
        wsp->qws = reinterpret_cast<uint16_t *>(p + head + rec + rows);
        wsp->carry = reinterpret_cast<float *>(p + head + rec + 2 * rows);
        wsp->part = gated ? reinterpret_cast<uint64_t *>(p + head + rec + 2 * rows + carry) : nullptr;
    }
    return head + rec + 2 * rows + carry + part;
}

__global__ __launch_bounds__(256) void zero_u64_kernel(uint64_t *p, size_t n) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// may_fork: a single long sequence may run in segments with part of the work
// on the device's auxiliary stream (created on first use).
// gate (prelude fused only): the output gate fused into the scan's stores.
template <bool kRaw>
hipError_t launch_impl(const uint16_t *q16, const uint16_t *k16, const uint16_t *v16, RawIn raw,
                       const float *g, const float *beta, const float *S0, float *S_final,
                       const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v, float scale,
                       uint16_t *o16, uint16_t *states, void *workspace, hipStream_t stream,
                       bool may_fork = true, const GateIn *gate = nullptr) {
    const size_t max_chunks = (size_t)(T + kChunk - 1) / kChunk + (size_t)N;
    Workspace W;
    workspace_layout(N, T, H_qk, H_v, kRaw, workspace, &W, gate != nullptr);
    GateIn gt{};
    if (gate) {
        gt = *gate;
        gt.part = W.part;
    }
    const int scan_grid = N * H_v * kSlabsW;
    // The fused gate makes workgroups wait for their V-head's other slabs, so
    // it is taken only when the whole grid is resident at once (one workgroup
    // per CU); otherwise the scan writes o and the gate runs as its own pass.
    bool fuse_gate = false;
    if (gate) {
        int dev = 0, cus = 0;
        hipError_t ge = hipGetDevice(&dev);
        if (ge == hipSuccess) ge = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (ge != hipSuccess) return ge;
        fuse_gate = scan_grid <= cus;
    }
    raw.kws = W.kws;
    raw.qws = W.qws;
    int32_t *chunk_base = W.chunk_base;
    uint16_t *ws = W.rec;
    auto prep = [&](int c_lo, int c_hi, int max_grid, hipStream_t s) {
        const int items = (c_hi - c_lo) * H_qk;
        constexpr int kW = kPrepWavesOf<kRecFwd>;
        const int grid = min((items + kW - 1) / kW, max_grid);
        hipLaunchKernelGGL(prep_kernel<kRaw>, dim3(grid), dim3(64 * kW), 0, s, q16, k16, raw,
                           g, beta, cu_seqlens, chunk_base, N, T, H_qk, H_v, scale, c_lo * H_qk,
                           c_hi * H_qk, ws);
        return hipGetLastError();
    };
    auto scan = [&](int c_lo, int c_hi, const float *init, float *fin) {
        if constexpr (kRaw) {
            if (fuse_gate) {
                hipLaunchKernelGGL((scan_kernel<true, kOutGated>), dim3(scan_grid), dim3(512), 0, stream,
                                   q16, k16, v16, raw, init, fin, cu_seqlens, chunk_base, N, T, H_qk,
                                   H_v, scale, c_lo, c_hi, ws, o16, nullptr, gt);
                return hipGetLastError();
            }
        }
        if (states)
            hipLaunchKernelGGL((scan_kernel<kRaw, kOutBoth>), dim3(scan_grid), dim3(512), 0, stream,
                               q16, k16, v16, raw, init, fin, cu_seqlens, chunk_base, N, T, H_qk,
                               H_v, scale, c_lo, c_hi, ws, o16, states);
        else
            hipLaunchKernelGGL((scan_kernel<kRaw, kOutO>), dim3(scan_grid), dim3(512), 0, stream,
                               q16, k16, v16, raw, init, fin, cu_seqlens, chunk_base, N, T, H_qk,
                               H_v, scale, c_lo, c_hi, ws, o16, nullptr);
        return hipGetLastError();
    };

    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu_seqlens, N, T, chunk_base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (fuse_gate) {     // tags cleared by a kernel (the call may be captured into a graph)
        const size_t n = max_chunks * (size_t)H_v * kChunk * kSlabsW;
        hipLaunchKernelGGL(zero_u64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, W.part, n);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    // the gate as its own pass when it could not be fused
    auto gate_pass = [&]() {
        if (!gate || fuse_gate) return hipSuccess;
        return launch_gated_norm(o16, gate->z, gate->w, T * H_v, gate->eps, gate->y, stream);
    };

    // one sequence (cu_seqlens, if given, is {0, T}): nch chunks known on the host
    const int nch = (T + kChunk - 1) / kChunk;
    std::unique_lock<std::mutex> lock(g_aux_mu);
    DeviceAux *aux = (may_fork && N == 1 && nch >= kSegMinChunks) ? device_aux(stream) : nullptr;
    const int idle = aux ? aux->cus - scan_grid : 0;
    if (idle < kMinIdleCUs) {
        lock.unlock();
        const int all = (int)max_chunks;
        if ((e = prep(0, all, INT32_MAX, stream)) != hipSuccess) return e;
        if ((e = scan(0, all, S0, S_final)) != hipSuccess) return e;
        return gate_pass();
    }

    // The state passes from segment to segment through final_state, or the
    // workspace's carry area when the caller wants no final state.  The last
    // wait joins the auxiliary stream back into the caller's stream.
    float *carry = S_final ? S_final : W.carry;
    int b[kMaxSegments + 1];
    const int nseg = segment_bounds(nch, kRaw ? kSegGrowthRaw : kSegGrowth, b);
    if ((e = prep(b[0], b[1], INT32_MAX, stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(aux->ev[0], stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(aux->stream, aux->ev[0], 0)) != hipSuccess) return e;
    for (int i = 1; i < nseg; ++i) {
        if ((e = prep(b[i], b[i + 1], idle, aux->stream)) != hipSuccess) return e;
        if ((e = hipEventRecord(aux->ev[i], aux->stream)) != hipSuccess) return e;
    }
    for (int i = 0; i < nseg; ++i) {
        if (i > 0 && (e = hipStreamWaitEvent(stream, aux->ev[i], 0)) != hipSuccess) return e;
        if ((e = scan(b[i], b[i + 1], i == 0 ? S0 : carry, i == nseg - 1 ? S_final : carry)) != hipSuccess)
            return e;
    }
    return gate_pass();
}

// Backward workspace: chunk offsets | forward records | backward records |
// bf16 state at each chunk start | bf16 state gradient at each chunk end |
// bf16 dU per (chunk, V-head) as MFMA fragment blocks.
struct BwdWorkspace {
    int32_t *chunk_base;
    uint16_t *rec, *brec, *states, *dsw, *duw;
    float *carry;     // the state gradient between segments of the reverse scan (one sequence)
};
// Given the chunk states of an earlier forward pass, the workspace has no
// states region and the forward records are not kept.
size_t bwd_workspace_layout(int N, int T, int H_v, bool saved, void *base, BwdWorkspace *wsp) {
    const size_t max_chunks = (size_t)(T + kChunk - 1) / kChunk + (size_t)N;
    const size_t head = align256((size_t)(N + 1) * sizeof(int32_t));
    const size_t rec = saved ? 0 : max_chunks * (size_t)H_v * kRecElems * sizeof(uint16_t);
    const size_t brec = max_chunks * (size_t)H_v * kBwdRecElems * sizeof(uint16_t);
    const size_t st = max_chunks * (size_t)H_v * kD * kD * sizeof(uint16_t);
    const size_t own = saved ? 0 : st;
    const size_t du = max_chunks * kChunk * (size_t)H_v * kD * sizeof(uint16_t);
    const size_t carry = N == 1 ? (size_t)H_v * kD * kD * sizeof(float) : 0;
    if (wsp) {
        char *p = static_cast<char *>(base);
        wsp->chunk_base = reinterpret_cast<int32_t *>(p);
        wsp->rec = saved ? nullptr : reinterpret_cast<uint16_t *>(p + head);
        wsp->brec = reinterpret_cast<uint16_t *>(p + head + rec);
        wsp->states = saved ? nullptr : reinterpret_cast<uint16_t *>(p + head + rec + brec);
        wsp->dsw = reinterpret_cast<uint16_t *>(p + head + rec + brec + own);
        wsp->duw = reinterpret_cast<uint16_t *>(p + head + rec + brec + own + st);
        wsp->carry = carry ? reinterpret_cast<float *>(p + head + rec + brec + own + st + du) : nullptr;
    }
    return head + rec + brec + own + st + du + carry;
}

}  // namespace

size_t chunked_backward_workspace_bytes(int N, int T, int H_qk, int H_v, bool saved) {
    (void)H_qk;
    return bwd_workspace_layout(N, T, H_v, saved, nullptr, nullptr);
}

size_t chunk_states_bytes(int N, int T, int H_v) {
    return ((size_t)(T + kChunk - 1) / kChunk + (size_t)N) * (size_t)H_v * kD * kD * sizeof(uint16_t);
}

// plan -> prep (forward and backward records) -> forward scan storing each
// chunk's start state -> reverse scan (dv, the initial-state gradient, dS' and
// dU per chunk) -> per-chunk gradients (dq, dk, dg, dbeta), all on `stream`.
// With chunk_states from an earlier forward pass (gdn_prefill with states
// kept), prep writes only the backward records and the forward scan is
// skipped.
//
// A single long sequence leaves CUs idle during both scans (one workgroup per
// (V-head, slab)); the work that needs neither scan's next result runs there,
// on the auxiliary stream, with grids no larger than the idle CUs (workgroups
// that loop over their items):
//   recomputing: forward records alone; then the forward scan, with the
//     backward records beside it (the reverse scan needs only those), those
//     of the first segment last: they are formed beside the reverse scan;
//   from kept states: the backward records of the last segment alone; the
//     reverse scan in segments walked last to first, with the records of the
//     earlier segments formed beside it;
//   both: the reverse scan in segments; once its last segment is done, that
//     segment's chunk gradients beside the rest of it.  The other segments'
//     gradients follow on the caller's stream, which then waits for the
//     auxiliary stream.
// (The two scans are independent, but 512-thread workgroups of both do not fit
// one CU together, so running them side by side gains nothing.)
hipError_t launch_chunked_backward(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *S0, const int32_t *cu_seqlens,
                                   int N, int T, int H_qk, int H_v, float scale, const void *d_o,
                                   const float *dS_final, void *dq, void *dk, void *dv, float *dg,
                                   float *dbeta, float *dS0, const void *chunk_states,
                                   void *workspace, hipStream_t stream) {
    const int max_chunks = (T + kChunk - 1) / kChunk + N;
    BwdWorkspace W;
    const bool saved = chunk_states != nullptr;
    bwd_workspace_layout(N, T, H_v, saved, workspace, &W);
    const uint16_t *q16 = static_cast<const uint16_t *>(q), *k16 = static_cast<const uint16_t *>(k);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu_seqlens, N, T, W.chunk_base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // records of chunks [c_lo, c_hi): forward, backward or both
    auto prep = [&](auto recs, int c_lo, int c_hi, int max_grid, hipStream_t s) {
        constexpr int kRecs = decltype(recs)::value, kW = kPrepWavesOf<kRecs>;
        const int it = (c_hi - c_lo) * H_qk;
        const int grid = min((it + kW - 1) / kW, max_grid);
        hipLaunchKernelGGL((prep_kernel<false, kRecs>), dim3(grid), dim3(64 * kW), 0, s, q16, k16,
                           RawIn{}, g, beta, cu_seqlens, W.chunk_base, N, T, H_qk, H_v, scale,
                           c_lo * H_qk, c_hi * H_qk, W.rec, W.brec);
        return hipGetLastError();
    };
    constexpr std::integral_constant<int, kRecFwd> fwd{};
    constexpr std::integral_constant<int, kRecBwd> bwd{};
    constexpr std::integral_constant<int, kRecFwd | kRecBwd> both{};
    auto fscan = [&]() {      // the forward scan, storing each chunk's start state
        hipLaunchKernelGGL((scan_kernel<false, kOutStates>), dim3(N * H_v * kSlabsW), dim3(512), 0,
                           stream, q16, k16, static_cast<const uint16_t *>(v), RawIn{}, S0, nullptr,
                           cu_seqlens, W.chunk_base, N, T, H_qk, H_v, scale, 0, max_chunks, W.rec,
                           nullptr, W.states);
        return hipGetLastError();
    };
    auto rscan = [&](int c_lo, int c_hi, const float *in, float *out) {
        return launch_bwd_scan(q, k, d_o, in, cu_seqlens, W.chunk_base, N, T, H_qk, H_v, scale,
                               W.brec, W.dsw, W.duw, dv, out, c_lo, c_hi, stream);
    };
    const void *states = saved ? chunk_states : W.states;
    auto grad = [&](int c_lo, int c_hi, int max_grid, hipStream_t s) {
        const int lo = c_lo * H_qk, hi = c_hi * H_qk;
        return launch_bwd_grad(q, k, v, d_o, dv, beta, cu_seqlens, W.chunk_base, N, T, H_qk, H_v,
                               scale, W.brec, states, W.dsw, W.duw, dq, dk, dg, dbeta, lo, hi,
                               min(hi - lo, max_grid), s);
    };

    const int nch = (T + kChunk - 1) / kChunk;
    const int scan_grid = N * H_v * kSlabsW;      // both scans: one workgroup per (V-head, slab)
    std::unique_lock<std::mutex> lock(g_aux_mu);
    DeviceAux *aux = (N == 1 && nch >= kSegMinChunks) ? device_aux(stream) : nullptr;
    const int idle = aux ? aux->cus - scan_grid : 0;
    if (idle < kMinIdleCUs) {
        lock.unlock();
        if (saved) {
            if ((e = prep(bwd, 0, max_chunks, INT32_MAX, stream)) != hipSuccess) return e;
        } else {
            if ((e = prep(both, 0, max_chunks, INT32_MAX, stream)) != hipSuccess) return e;
            if ((e = fscan()) != hipSuccess) return e;
        }
        if ((e = rscan(0, max_chunks, dS_final, dS0)) != hipSuccess) return e;
        return grad(0, max_chunks, INT32_MAX, stream);
    }

    int b[kMaxSegments + 1];
    const int nseg = segment_bounds(nch, kSegGrowthRev, b);
    const int last = nseg - 1;
    hipStream_t as = aux->stream;
    if (saved) {
        if ((e = prep(bwd, b[last], b[last + 1], INT32_MAX, stream)) != hipSuccess) return e;
        if ((e = hipEventRecord(aux->ev[last], stream)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(as, aux->ev[last], 0)) != hipSuccess) return e;
        for (int i = last - 1; i >= 0; --i) {
            if ((e = prep(bwd, b[i], b[i + 1], idle, as)) != hipSuccess) return e;
            if ((e = hipEventRecord(aux->ev[i], as)) != hipSuccess) return e;
        }
    } else {
        // the backward records of the sequence's first segment, which the
        // reverse scan reaches last, come after the others on the auxiliary
        // stream and are formed while the reverse scan starts
        if ((e = prep(fwd, 0, nch, INT32_MAX, stream)) != hipSuccess) return e;
        if ((e = hipEventRecord(aux->ev[0], stream)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(as, aux->ev[0], 0)) != hipSuccess) return e;
        if ((e = prep(bwd, b[1], nch, idle, as)) != hipSuccess) return e;
        if ((e = hipEventRecord(aux->ev[1], as)) != hipSuccess) return e;
        if ((e = prep(bwd, 0, b[1], idle, as)) != hipSuccess) return e;
        if ((e = hipEventRecord(aux->ev[2], as)) != hipSuccess) return e;
        if ((e = fscan()) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(stream, aux->ev[1], 0)) != hipSuccess) return e;
    }
    for (int i = last; i >= 0; --i) {
        // the records of segment i: from the auxiliary stream, except for the
        // last segment from kept states (formed on this stream)
        const int rec_ev = saved ? (i < last ? i : -1) : (i == 0 ? 2 : -1);
        if (rec_ev >= 0 && (e = hipStreamWaitEvent(stream, aux->ev[rec_ev], 0)) != hipSuccess) return e;
        if ((e = rscan(b[i], b[i + 1], i == last ? dS_final : W.carry, i == 0 ? dS0 : W.carry)) != hipSuccess)
            return e;
        if (i == last) {
            if ((e = hipEventRecord(aux->ev[kEvRscan], stream)) != hipSuccess) return e;
            if ((e = hipStreamWaitEvent(as, aux->ev[kEvRscan], 0)) != hipSuccess) return e;
            if ((e = grad(b[last], b[last + 1], idle, as)) != hipSuccess) return e;
            if ((e = hipEventRecord(aux->ev[kEvGrad], as)) != hipSuccess) return e;
        }
    }
    if ((e = grad(b[0], b[last], INT32_MAX, stream)) != hipSuccess) return e;
    return hipStreamWaitEvent(stream, aux->ev[kEvGrad], 0);
}

size_t chunked_workspace_bytes(int N, int T, int H_qk, int H_v, bool raw) {
    return workspace_layout(N, T, H_qk, H_v, raw, nullptr, nullptr);
}

size_t chunked_gated_workspace_bytes(int N, int T, int H_qk, int H_v) {
    return workspace_layout(N, T, H_qk, H_v, true, nullptr, nullptr, true);
}

hipError_t launch_chunked_prefill(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *S0, float *S_final,
                                  const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v,
                                  float scale, void *o, void *chunk_states, void *workspace,
                                  hipStream_t stream) {
    return launch_impl<false>(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                              static_cast<const uint16_t *>(v), RawIn{}, g, beta, S0, S_final,
                              cu_seqlens, N, T, H_qk, H_v, scale, static_cast<uint16_t *>(o),
                              static_cast<uint16_t *>(chunk_states), workspace, stream);
}

// Scratch for callers that cannot allocate (gdn_prefill_no_alloc): one array
// per device, holding the prefill workspace of one call.  Its device address
// is looked up once per device, with that device current; host code uses only
// that address.  Calls that overlap on one device share the array and race.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
struct ScratchAddr {
    bool tried = false;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
std::mutex g_scratch_mu;
ScratchAddr g_scratch[kMaxDevices];
}  // namespace

size_t chunked_scratch_bytes() { return kScratchBytes; }

hipError_t launch_chunked_prefill_no_alloc(const void *q, const void *k, const void *v,
                                           const float *g, const float *beta, const float *S0,
                                           float *S_final, const int32_t *cu_seqlens, int N, int T,
                                           int H_qk, int H_v, float scale, void *o,
                                           hipStream_t stream) {
    if (chunked_workspace_bytes(N, T, H_qk, H_v, false) > kScratchBytes) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        ScratchAddr &a = g_scratch[dev];
        if (!a.tried) {
            a.tried = true;
            a.err = hipGetSymbolAddress(&a.ptr, HIP_SYMBOL(scratch));
        }
        if (a.err != hipSuccess) return a.err;
        ws = a.ptr;
    }
    // everything on the caller's stream (no auxiliary stream, no events)
    return launch_impl<false>(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                              static_cast<const uint16_t *>(v), RawIn{}, g, beta, S0, S_final,
                              cu_seqlens, N, T, H_qk, H_v, scale, static_cast<uint16_t *>(o),
                              nullptr, ws, stream, false);
}

hipError_t launch_chunked_prefill_raw(const void *x, const void *w, float eps, const float *g,
                                      const float *beta, const float *S0, float *S_final,
                                      const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v,
                                      float scale, void *o, void *chunk_states, void *workspace,
                                      hipStream_t stream, const void *conv_hist_in) {
    RawIn raw{static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w), eps, nullptr, nullptr,
              static_cast<const uint16_t *>(conv_hist_in)};
    return launch_impl<true>(nullptr, nullptr, nullptr, raw, g, beta, S0, S_final, cu_seqlens, N, T,
                             H_qk, H_v, scale, static_cast<uint16_t *>(o),
                             static_cast<uint16_t *>(chunk_states), workspace, stream);
}

hipError_t launch_chunked_prefill_raw_gated(const void *x, const void *w, float eps, const float *g,
                                            const float *beta, const float *S0, float *S_final,
                                            const int32_t *cu_seqlens, int N, int T, int H_qk,
                                            int H_v, float scale, void *o, const void *z,
                                            const float *norm_w, float norm_eps, void *y,
                                            void *workspace, hipStream_t stream,
                                            const void *conv_hist_in) {
    RawIn raw{static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(w), eps, nullptr, nullptr,
              static_cast<const uint16_t *>(conv_hist_in)};
    const GateIn gate{static_cast<const uint16_t *>(z), norm_w, norm_eps, static_cast<uint16_t *>(y),
                      nullptr};
    return launch_impl<true>(nullptr, nullptr, nullptr, raw, g, beta, S0, S_final, cu_seqlens, N, T,
                             H_qk, H_v, scale, static_cast<uint16_t *>(o), nullptr, workspace, stream,
                             true, &gate);
}

}  // namespace gdn
