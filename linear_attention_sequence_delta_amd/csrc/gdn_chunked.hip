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
//   prep  -- fully parallel over (chunk, QK head): K K^T and Q K^T on bf16 MFMA
//            (shared by the V-heads of the QK head), then per V-head the gated A,
//            its unit-lower-triangular inverse (fp32 substitution on the 16 x 16
//            diagonal blocks, bf16 MFMA for the off-diagonal blocks), T' and P,
//            written to the workspace as bf16 (16 KiB per chunk and V-head).
//   scan  -- sequential over the chunks of one (sequence, V-head, 16-row slab of
//            d_v); four waves split the 64 chunk rows (X = K S^T, R, U, O) and the
//            128 d_k columns of the fp32 state (S' update).  The slab state never
//            leaves the chip between chunks: fp32 in MFMA accumulators, plus a bf16
//            copy in LDS that feeds the next chunk's products.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kSlab = 16;            // d_v rows per scan workgroup
constexpr int kSlabs = kD / kSlab;   // 8
constexpr int kKP = kD + 8;          // LDS row stride (bf16) of 128-wide rows
constexpr int kAP = kChunk + 4;      // LDS row stride (fp32) of 64-wide rows
constexpr int kRP = kChunk + 8;      // LDS row stride (bf16) of 64-wide rows
constexpr int kTileElems = kChunk * kChunk;   // one 64 x 64 bf16 matrix

__device__ __forceinline__ f32x4 mfma32(uint4 a, uint4 b, f32x4 c) {
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
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack_bf2(a, b), pack_bf2(c, d));
}
__device__ __forceinline__ uint16_t elem(uint4 u, int i) {
    const uint32_t w = i < 2 ? u.x : i < 4 ? u.y : i < 6 ? u.z : u.w;
    return (i & 1) ? uint16_t(w >> 16) : uint16_t(w & 0xFFFFu);
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
// Lower 16 x 16 tiles (I >= J) of a 64 x 64 product, in a fixed order.
__constant__ int8_t kTileI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int8_t kTileJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

__global__ __launch_bounds__(256) void prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ cu,
    const int32_t *__restrict__ chunk_base, int N, int T, int H_qk, int H_v, float scale,
    uint16_t *__restrict__ ws_tp) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[kChunk * kKP];
    __shared__ __attribute__((aligned(16))) uint16_t sQ[kChunk * kKP];
    __shared__ __attribute__((aligned(16))) float sKK[kChunk * kAP];
    __shared__ __attribute__((aligned(16))) float sQK[kChunk * kAP];
    __shared__ __attribute__((aligned(16))) float sA[4][kChunk * kAP];
    __shared__ float sG[4][kChunk];
    __shared__ float sB[4][kChunk];

    const int gc = blockIdx.x, hq = blockIdx.y;
    if (gc >= chunk_base[N]) return;
    const int n = seq_of_chunk(chunk_base, N, gc);
    const int s0 = cu ? cu[n] : 0, s1 = cu ? cu[n + 1] : T;
    const int c0 = s0 + kChunk * (gc - chunk_base[n]);
    const int L = min(kChunk, s1 - c0);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, c = lane & 15;

    // K and Q rows of the chunk (rows past the end read as zero)
    for (int idx = tid; idx < kChunk * 16; idx += 256) {
        const int r = idx >> 4, part = idx & 15;
        uint4 kv = make_uint4(0, 0, 0, 0), qv = kv;
        if (r < L) {
            const size_t off = ((size_t)(c0 + r) * H_qk + hq) * kD + part * 8;
            kv = *reinterpret_cast<const uint4 *>(k + off);
            qv = *reinterpret_cast<const uint4 *>(q + off);
        }
        *reinterpret_cast<uint4 *>(sK + r * kKP + part * 8) = kv;
        *reinterpret_cast<uint4 *>(sQ + r * kKP + part * 8) = qv;
    }
    __syncthreads();

    // K K^T and Q K^T, lower tiles only: 20 tiles of 16 x 16, 4 k-steps each
    for (int t = wave; t < 20; t += 4) {
        const bool isq = t >= 10;
        const int tt = isq ? t - 10 : t;
        const int I = kTileI[tt], J = kTileJ[tt];
        const uint16_t *X = isq ? sQ : sK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 a = *reinterpret_cast<const uint4 *>(X + (16 * I + c) * kKP + 32 * s + 8 * g4);
            const uint4 b = *reinterpret_cast<const uint4 *>(sK + (16 * J + c) * kKP + 32 * s + 8 * g4);
            acc = mfma32(a, b, acc);
        }
        float *D = isq ? sQK : sKK;
#pragma unroll
        for (int j = 0; j < 4; ++j) D[(16 * I + 4 * g4 + j) * kAP + 16 * J + c] = acc[j];
    }
    __syncthreads();

    const int group = H_v / H_qk;
    for (int vv = wave; vv < group; vv += 4) {
        const int h = hq * group + vv;
        float *A = sA[wave];
        const float gl = lane < L ? g[(size_t)(c0 + lane) * H_v + h] : 0.f;
        const float bl = lane < L ? beta[(size_t)(c0 + lane) * H_v + h] : 0.f;
        const float G = wave_scan(gl);
        sG[wave][lane] = G;
        sB[wave][lane] = bl;

        // A[r][i] = b_r exp(G_r - G_i) (k_r . k_i) for i < r, lower tiles only
        for (int r = 0; r < kChunk; ++r) {
            const float Gr = __shfl(G, r, 64), br = __shfl(bl, r, 64);
            const int i = lane;
            if ((i >> 4) <= (r >> 4))
                A[r * kAP + i] = i < r ? br * __expf(Gr - G) * sKK[r * kAP + i] : 0.f;
        }
        wave_lds_sync();

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

        // Operand loaders for 16 x 16 x 16 MFMA from the fp32 block matrix:
        // A operand = rows of block (I, J); B operand = columns of block (I, J).
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

        // The off-diagonal blocks of A are read (as bf16 MFMA row operands)
        // before any of them is overwritten by the matching block of T.
        const s16x4 a10 = rowop(1, 0), a21 = rowop(2, 1), a32 = rowop(3, 2);
        const s16x4 a20 = rowop(2, 0), a30 = rowop(3, 0), a31 = rowop(3, 1);

        // Blocks one below the diagonal: T_{I,I-1} = -T_II A_{I,I-1} T_{I-1,I-1}
        f32x4 t10, t21, t32;
        {
            const f32x4 y1 = mfma16(a10, colop(0, 0), z4);
            const f32x4 y2 = mfma16(a21, colop(1, 1), z4);
            const f32x4 y3 = mfma16(a32, colop(2, 2), z4);
            t10 = -mfma16(rowop(1, 1), accop(y1), z4);
            t21 = -mfma16(rowop(2, 2), accop(y2), z4);
            t32 = -mfma16(rowop(3, 3), accop(y3), z4);
        }
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            A[(16 + 4 * g4 + j) * kAP + c] = t10[j];
            A[(32 + 4 * g4 + j) * kAP + 16 + c] = t21[j];
            A[(48 + 4 * g4 + j) * kAP + 32 + c] = t32[j];
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

        // T' = T diag(b) and P = lower-incl(exp(G_r - G_i) scale QK^T), bf16, row-major
        uint16_t *out_t = ws_tp + ((size_t)gc * H_v + h) * (2 * kTileElems);
        uint16_t *out_p = out_t + kTileElems;
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
            const int idx = qq * 64 + lane;
            const int row = idx >> 3, col0 = (idx & 7) * 8;
            const float Gr = sG[wave][row];
            float tv[8], pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = col0 + e;
                const bool lower_block = (col >> 4) <= (row >> 4);
                tv[e] = lower_block ? A[row * kAP + col] * sB[wave][col] : 0.f;
                pv[e] = col <= row ? scale * __expf(Gr - sG[wave][col]) * sQK[row * kAP + col] : 0.f;
            }
            uint4 ot, op;
            ot.x = pack_bf2(tv[0], tv[1]); ot.y = pack_bf2(tv[2], tv[3]);
            ot.z = pack_bf2(tv[4], tv[5]); ot.w = pack_bf2(tv[6], tv[7]);
            op.x = pack_bf2(pv[0], pv[1]); op.y = pack_bf2(pv[2], pv[3]);
            op.z = pack_bf2(pv[4], pv[5]); op.w = pack_bf2(pv[6], pv[7]);
            *reinterpret_cast<uint4 *>(out_t + row * kChunk + col0) = ot;
            *reinterpret_cast<uint4 *>(out_p + row * kChunk + col0) = op;
        }
        wave_lds_sync();
    }
}

// ------------------------------------------------------------------- scan
struct ChunkRegs {
    uint4 kA[4], qA[4], tA[2], pA[2];
    float v[4];
    float gl;
};

__global__ __launch_bounds__(256) void scan_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *initial_state, float *final_state,
    const int32_t *__restrict__ cu, const int32_t *__restrict__ chunk_base, int N, int T,
    int H_qk, int H_v, float scale, const uint16_t *__restrict__ ws_tp,
    uint16_t *__restrict__ o) {
    __shared__ __attribute__((aligned(16))) uint16_t sS[kSlab * kKP];
    __shared__ __attribute__((aligned(16))) uint16_t sR[kSlab * kRP];
    __shared__ __attribute__((aligned(16))) uint16_t sU[kSlab * kRP];
    __shared__ __attribute__((aligned(16))) uint16_t sUs[kSlab * kRP];
    __shared__ __attribute__((aligned(16))) uint16_t sKt[kD * kRP];

    // Workgroup -> (sequence, V-head, slab).  Workgroups are handed to the 8
    // XCDs round-robin; consecutive units (all slabs of a head, neighbouring
    // heads of one QK group) are kept on one XCD so that they share its L2.
    const int per_xcd = gridDim.x >> 3;
    const int u = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    const int slab = u % kSlabs;
    const int nh = u / kSlabs;
    const int h = nh % H_v, n = nh / H_v;
    const int hq = h / (H_v / H_qk);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g4 = lane >> 4, c = lane & 15;
    const int s0 = cu ? cu[n] : 0, s1 = cu ? cu[n + 1] : T;
    const int nchunks = (s1 - s0 + kChunk - 1) / kChunk;
    const int cbase = chunk_base[n];

    // fp32 state: this lane holds S[16 slab + c][32 wave + 16 t + 4 g4 + j]
    const size_t st_off = ((size_t)n * H_v + h) * (kD * kD) + (size_t)(kSlab * slab + c) * kD;
    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (initial_state) {
            const float4 x = *reinterpret_cast<const float4 *>(initial_state + st_off + 32 * wave + 16 * t + 4 * g4);
            st[t] = f32x4{x.x, x.y, x.z, x.w};
        } else {
            st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    auto write_state_lds = [&]() {
#pragma unroll
        for (int t = 0; t < 2; ++t)
            *reinterpret_cast<uint2 *>(sS + c * kKP + 32 * wave + 16 * t + 4 * g4) =
                pack4(st[t][0], st[t][1], st[t][2], st[t][3]);
    };
    write_state_lds();

    auto fetch = [&](int ci, ChunkRegs &R) {
        const int c0 = s0 + kChunk * ci;
        const int L = min(kChunk, s1 - c0);
        const int row = 16 * wave + c;
        const uint4 z = make_uint4(0, 0, 0, 0);
        const size_t qk_off = ((size_t)(c0 + row) * H_qk + hq) * kD + 8 * g4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            R.kA[s] = row < L ? *reinterpret_cast<const uint4 *>(k + qk_off + 32 * s) : z;
            R.qA[s] = row < L ? *reinterpret_cast<const uint4 *>(q + qk_off + 32 * s) : z;
        }
        const uint16_t *tp = ws_tp + ((size_t)(cbase + ci) * H_v + h) * (2 * kTileElems) + row * kChunk + 8 * g4;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            R.tA[s] = *reinterpret_cast<const uint4 *>(tp + 32 * s);
            R.pA[s] = *reinterpret_cast<const uint4 *>(tp + kTileElems + 32 * s);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 16 * wave + 4 * g4 + j;
            R.v[j] = rr < L ? bf2f(v[((size_t)(c0 + rr) * H_v + h) * kD + kSlab * slab + c]) : 0.f;
        }
        R.gl = lane < L ? g[(size_t)(c0 + lane) * H_v + h] : 0.f;
    };

    ChunkRegs cur;
    if (nchunks > 0) fetch(0, cur);
    __syncthreads();

    for (int ci = 0; ci < nchunks; ++ci) {
        const int c0 = s0 + kChunk * ci;
        const int L = min(kChunk, s1 - c0);

        // K^T for the state update (column m = d_k, row = chunk row)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                sKt[(32 * s + 8 * g4 + i) * kRP + 16 * wave + c] = elem(cur.kA[s], i);

        // cumulative log decay of the chunk and the per-row factors
        const float G = wave_scan(cur.gl);
        const float GL = __shfl(G, 63, 64);
        float gam[4], dec[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float Gr = __shfl(G, 16 * wave + 4 * g4 + j, 64);
            gam[j] = __expf(Gr);
            dec[j] = __expf(GL - Gr);
        }
        const float gamL = __expf(GL);

        ChunkRegs nxt;
        if (ci + 1 < nchunks) fetch(ci + 1, nxt);

        // X = K S^T and Q S^T for chunk rows 16 wave .. +15
        f32x4 ax = {0.f, 0.f, 0.f, 0.f}, aq = ax;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 sb = *reinterpret_cast<const uint4 *>(sS + c * kKP + 32 * s + 8 * g4);
            ax = mfma32(cur.kA[s], sb, ax);
            aq = mfma32(cur.qA[s], sb, aq);
        }
        // R = V - diag(gamma) X   (stored transposed: [d_v col][chunk row])
        *reinterpret_cast<uint2 *>(sR + c * kRP + 16 * wave + 4 * g4) =
            pack4(cur.v[0] - gam[0] * ax[0], cur.v[1] - gam[1] * ax[1],
                  cur.v[2] - gam[2] * ax[2], cur.v[3] - gam[3] * ax[3]);
        __syncthreads();

        // U = T' R (T' is lower triangular: k-steps up to this row block)
        f32x4 au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s)
            if (s <= (wave >> 1))
                au = mfma32(cur.tA[s], *reinterpret_cast<const uint4 *>(sR + c * kRP + 32 * s + 8 * g4), au);
        *reinterpret_cast<uint2 *>(sU + c * kRP + 16 * wave + 4 * g4) = pack4(au[0], au[1], au[2], au[3]);
        *reinterpret_cast<uint2 *>(sUs + c * kRP + 16 * wave + 4 * g4) =
            pack4(dec[0] * au[0], dec[1] * au[1], dec[2] * au[2], dec[3] * au[3]);
        __syncthreads();

        // O = diag(gamma) scale Q S^T + P U
        f32x4 ao;
#pragma unroll
        for (int j = 0; j < 4; ++j) ao[j] = scale * gam[j] * aq[j];
#pragma unroll
        for (int s = 0; s < 2; ++s)
            if (s <= (wave >> 1))
                ao = mfma32(cur.pA[s], *reinterpret_cast<const uint4 *>(sU + c * kRP + 32 * s + 8 * g4), ao);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 16 * wave + 4 * g4 + j;
            if (rr < L) o[((size_t)(c0 + rr) * H_v + h) * kD + kSlab * slab + c] = f2bf(ao[j]);
        }

        // S' = gamma_L S + (diag(exp(G_L - G)) U)^T K  (this wave: d_k 32 wave .. +31)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 as = gamL * st[t];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint4 ka = *reinterpret_cast<const uint4 *>(sKt + (32 * wave + 16 * t + c) * kRP + 32 * s + 8 * g4);
                const uint4 ub = *reinterpret_cast<const uint4 *>(sUs + c * kRP + 32 * s + 8 * g4);
                as = mfma32(ka, ub, as);
            }
            st[t] = as;
        }
        write_state_lds();
        __syncthreads();
        if (ci + 1 < nchunks) cur = nxt;
    }

    if (final_state) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
            *reinterpret_cast<float4 *>(final_state + st_off + 32 * wave + 16 * t + 4 * g4) =
                make_float4(st[t][0], st[t][1], st[t][2], st[t][3]);
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

size_t chunked_workspace_bytes(int N, int T, int H_qk, int H_v) {
    (void)H_qk;
    const size_t max_chunks = (size_t)(T + kChunk - 1) / kChunk + (size_t)N;
    return align256((size_t)(N + 1) * sizeof(int32_t)) +
           max_chunks * (size_t)H_v * 2 * kTileElems * sizeof(uint16_t);
}

hipError_t launch_chunked_prefill(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, const float *S0, float *S_final,
                                  const int32_t *cu_seqlens, int N, int T, int H_qk, int H_v,
                                  float scale, void *o, void *workspace, hipStream_t stream) {
    int32_t *chunk_base = static_cast<int32_t *>(workspace);
    uint16_t *ws_tp = reinterpret_cast<uint16_t *>(static_cast<char *>(workspace) +
                                                   align256((size_t)(N + 1) * sizeof(int32_t)));
    const int max_chunks = (T + kChunk - 1) / kChunk + N;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu_seqlens, N, T, chunk_base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_kernel, dim3(max_chunks, H_qk), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k), g, beta,
                       cu_seqlens, chunk_base, N, T, H_qk, H_v, scale, ws_tp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan_kernel, dim3(N * H_v * kSlabs), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), g, S0, S_final, cu_seqlens, chunk_base, N,
                       T, H_qk, H_v, scale, ws_tp, static_cast<uint16_t *>(o));
    return hipGetLastError();
}

}  // namespace gdn
