/*
 * gdn_oracle.c -- plain fp64 CPU oracle of the Gated DeltaNet layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with the
 * HIP library.  It is deliberately slow and literal: every loop below is one
 * line of the method's definition, evaluated in double precision with no
 * blocking, fusion or reordering beyond what the definition states.
 *
 * Pages cited (title, site):
 *   [Dissect] "从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力"
 *             (www.2kiu.com) -- sec. 2.1 (layer config: 16 QK heads, 48 V heads,
 *             head dims 128, short conv of width 4, weights conv1d.weight /
 *             A_log / dt_bias, fp32 state dtype) and sec. 2.2 (the delta-rule
 *             state update and its erase-then-write meaning).
 *   [OOM]     "Qwen3.8-27B 混合线性注意力到底解决了什么" (www.mhpn.cn) -- sec. 1.2
 *             (a per-token step function taking q, k, v, the previous state and
 *             two gates, returning the output and the new state; its argument
 *             set is kept; its update body, which has no erase term and swaps the
 *             gate roles, is not followed).
 * The gated form S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T with
 * o_t = S_t q_t generalises the [Dissect sec. 2.2] rule (which is the a_t = 1
 * case) by the decay gate a_t = exp(g_t).
 *
 * Conventions (the readings of the pages taken here):
 *   - state S of one (sequence, V-head) is d_v x d_k, row-major, d_k contiguous
 *     (the v k^T orientation of [Dissect sec. 2.2]);
 *   - V-head h reads QK head h / (H_v / H_qk) (contiguous groups);
 *   - the decay gate is passed as its logarithm g (a = exp(g));
 *   - raw projection channels are ordered [q heads | k heads | v heads];
 *   - conv taps: w[c][3] multiplies the current token, w[c][0] the token three
 *     steps back, taps before a sequence's first token read zero, no bias;
 *   - L2 normalisation is y / sqrt(sum y^2 + eps).
 *
 * Parity pins: every function here is checked by the CPU tests against things
 * other than itself (brute-force products, closed forms, torch conv1d, the
 * erase-then-write invariant, orthonormal-key retrieval, split invariance).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL -1
#define ORC_ENOMEM -2

static int seq_bounds(const int32_t *cu, int N, int T, int n, int *s0, int *s1)
{
    if (cu == NULL) {
        if (N != 1)
            return ORC_EINVAL;
        *s0 = 0;
        *s1 = T;
        return ORC_OK;
    }
    *s0 = cu[n];
    *s1 = cu[n + 1];
    if (*s0 < 0 || *s1 < *s0 || *s1 > T)
        return ORC_EINVAL;
    return ORC_OK;
}

/*
 * Prelude: short causal depthwise conv (width 4) -> SiLU -> split into q, k, v
 * -> L2-normalise every q and k head.  [Dissect sec. 2.1]: conv kernel width 4
 * and the conv1d weight of each linear-attention layer.
 *
 * x  [T][C_raw]     raw projections (C_raw = 2*H_qk*dk + H_v*dv)
 * w  [C_raw][4]     conv weights
 * cu [N+1] or NULL  packed sequence offsets
 * q, k [T][H_qk][dk], v [T][H_v][dv]  outputs
 */
int orc_prelude(const double *x, const double *w, const int32_t *cu, int N, int T,
                int H_qk, int H_v, int dk, int dv, double eps,
                double *q, double *k, double *v)
{
    const int Cq = H_qk * dk;
    const int Craw = 2 * Cq + H_v * dv;
    if (T < 0 || N < 1 || H_qk < 1 || H_v < 1 || dk < 1 || dv < 1)
        return ORC_EINVAL;
    for (int n = 0; n < N; ++n) {
        int s0 = 0, s1 = 0;
        if (seq_bounds(cu, N, T, n, &s0, &s1))
            return ORC_EINVAL;
    }
    int status = ORC_OK;
    /* tokens are independent: threads take tokens, each with its own row y */
#pragma omp parallel
    {
        double *y = (double *)malloc(sizeof(double) * (size_t)(Craw > 0 ? Craw : 1));
        if (!y) {
#pragma omp atomic write
            status = ORC_ENOMEM;
        }
        for (int n = 0; n < N; ++n) {
            int s0 = 0, s1 = 0;
            seq_bounds(cu, N, T, n, &s0, &s1);
#pragma omp for schedule(static)
            for (int t = s0; t < s1; ++t) {
                if (!y)
                    continue;
                /* conv + SiLU on every channel */
                for (int c = 0; c < Craw; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < 4; ++j) {
                        int src = t - 3 + j;
                        if (src >= s0)
                            acc += w[(size_t)c * 4 + j] * x[(size_t)src * Craw + c];
                    }
                    y[c] = acc / (1.0 + exp(-acc));
                }
                /* L2 normalisation of each q head and each k head */
                for (int h = 0; h < H_qk; ++h) {
                    const double *yq = y + (size_t)h * dk;
                    const double *yk = y + Cq + (size_t)h * dk;
                    double sq = 0.0, sk = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        sq += yq[i] * yq[i];
                        sk += yk[i] * yk[i];
                    }
                    double rq = 1.0 / sqrt(sq + eps), rk = 1.0 / sqrt(sk + eps);
                    for (int i = 0; i < dk; ++i) {
                        q[((size_t)t * H_qk + h) * dk + i] = yq[i] * rq;
                        k[((size_t)t * H_qk + h) * dk + i] = yk[i] * rk;
                    }
                }
                for (int c = 0; c < H_v * dv; ++c)
                    v[(size_t)t * H_v * dv + c] = y[2 * Cq + c];
            }
        }
        free(y);
    }
    return status;
}

/*
 * One token of the gated delta rule on one state, in place:
 *   S <- a * S (I - b k k^T) + b v k^T,   o = S (scale * q)   (new S)
 * [Dissect sec. 2.2] gives the a = 1 form and its meaning: the value stored
 * under key k is erased with strength b before v is written under k.
 * The product S (I - b k k^T) is evaluated as S - b (S k) k^T, the same
 * matrix by associativity, so no d_k x d_k matrix is formed.
 */
static void delta_step(double *S, int dk, int dv, const double *qv, const double *kv,
                       const double *vv, double g, double beta, double scale, double *o,
                       double *Sk /* scratch [dv] */)
{
    const double alpha = exp(g);
    for (int i = 0; i < dv; ++i) {
        double acc = 0.0;
        for (int j = 0; j < dk; ++j)
            acc += S[(size_t)i * dk + j] * kv[j];
        Sk[i] = acc;
    }
    for (int i = 0; i < dv; ++i)
        for (int j = 0; j < dk; ++j) {
            double erased = S[(size_t)i * dk + j] - beta * Sk[i] * kv[j];
            S[(size_t)i * dk + j] = alpha * erased + beta * vv[i] * kv[j];
        }
    if (o)
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j)
                acc += S[(size_t)i * dk + j] * (scale * qv[j]);
            o[i] = acc;
        }
}

/*
 * Token-by-token recurrence over packed sequences (the authoritative form).
 * q, k [T][H_qk][dk]; v [T][H_v][dv]; g, beta [T][H_v]; S0 [N][H_v][dv][dk]
 * or NULL (zero); o [T][H_v][dv]; S_final [N][H_v][dv][dk] or NULL.
 * Only V-heads in [h_lo, h_hi) are computed (their o rows and final states);
 * other entries of o and S_final are left untouched.
 */
int orc_recurrent(const double *q, const double *k, const double *v, const double *g,
                  const double *beta, const double *S0, const int32_t *cu, int N, int T,
                  int H_qk, int H_v, int dk, int dv, double scale, double *o,
                  double *S_final, int h_lo, int h_hi)
{
    if (N < 1 || T < 0 || H_qk < 1 || H_v < 1 || H_v % H_qk != 0 || dk < 1 || dv < 1)
        return ORC_EINVAL;
    if (h_lo < 0 || h_hi > H_v || h_lo > h_hi)
        return ORC_EINVAL;
    for (int n = 0; n < N; ++n) {
        int s0 = 0, s1 = 0;
        if (seq_bounds(cu, N, T, n, &s0, &s1))
            return ORC_EINVAL;
    }
    const int group = H_v / H_qk;
    const int units = N * (h_hi - h_lo);
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        const int n = u / (h_hi - h_lo);
        const int h = h_lo + u % (h_hi - h_lo);
        const int hq = h / group;
        int s0 = 0, s1 = 0;
        seq_bounds(cu, N, T, n, &s0, &s1);
        double *S = (double *)malloc(sizeof(double) * (size_t)dv * dk);
        double *Sk = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !Sk) {
            free(S);
            free(Sk);
#pragma omp atomic write
            status = ORC_ENOMEM;
            continue;
        }
        const size_t ssz = (size_t)dv * dk;
        if (S0)
            memcpy(S, S0 + ((size_t)n * H_v + h) * ssz, sizeof(double) * ssz);
        else
            memset(S, 0, sizeof(double) * ssz);
        for (int t = s0; t < s1; ++t) {
            const double *qt = q + ((size_t)t * H_qk + hq) * dk;
            const double *kt = k + ((size_t)t * H_qk + hq) * dk;
            const double *vt = v + ((size_t)t * H_v + h) * dv;
            double *ot = o + ((size_t)t * H_v + h) * dv;
            delta_step(S, dk, dv, qt, kt, vt, g[(size_t)t * H_v + h], beta[(size_t)t * H_v + h],
                       scale, ot, Sk);
        }
        if (S_final)
            memcpy(S_final + ((size_t)n * H_v + h) * ssz, S, sizeof(double) * ssz);
        free(S);
        free(Sk);
    }
    return status;
}

/*
 * Decode step: the recurrence applied to one token per sequence, reading and
 * writing the state held in pool slot slot_idx[b].  ([OOM sec. 1.2]: the step
 * takes q, k, v, the previous state and the gates and returns the output and
 * the new state.)
 * q, k [B][H_qk][dk]; v [B][H_v][dv]; g, beta [B][H_v];
 * pool [P][H_v][dv][dk] (updated in place); o [B][H_v][dv].
 */
int orc_decode_step(const double *q, const double *k, const double *v, const double *g,
                    const double *beta, double *pool, const int32_t *slot_idx, int B, int P,
                    int H_qk, int H_v, int dk, int dv, double scale, double *o)
{
    if (B < 0 || P < 1 || H_qk < 1 || H_v < 1 || H_v % H_qk != 0 || dk < 1 || dv < 1)
        return ORC_EINVAL;
    for (int b = 0; b < B; ++b)
        if (slot_idx[b] < 0 || slot_idx[b] >= P)
            return ORC_EINVAL;
    const int group = H_v / H_qk;
    const size_t ssz = (size_t)dv * dk;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < B * H_v; ++u) {
        const int b = u / H_v, h = u % H_v, hq = h / group;
        double *Sk = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!Sk) {
#pragma omp atomic write
            status = ORC_ENOMEM;
            continue;
        }
        double *S = pool + ((size_t)slot_idx[b] * H_v + h) * ssz;
        delta_step(S, dk, dv, q + ((size_t)b * H_qk + hq) * dk, k + ((size_t)b * H_qk + hq) * dk,
                   v + ((size_t)b * H_v + h) * dv, g[(size_t)b * H_v + h],
                   beta[(size_t)b * H_v + h], scale, o + ((size_t)b * H_v + h) * dv, Sk);
        free(Sk);
    }
    return status;
}

/*
 * Chunked (WY / UT) form of the same recurrence, chunk length C.  This is an
 * exact algebraic rewrite of orc_recurrent used only as a cross-check of the
 * chunk equations.  Unrolling the recurrence inside a chunk gives
 * S_r = exp(G_r) (S + sum_{i<=r} exp(-G_i) u_i k_i^T) with
 * u_r = b_r (v_r - exp(G_r) S k_r - sum_{i<r} exp(G_r - G_i) (k_r . k_i) u_i),
 * a unit lower-triangular system in the rows u_r.  For one chunk with start
 * state S (dv x dk), tokens r = 0..L-1, cumulative log decay G_r = sum_{i<=r} g_i:
 *   A[r][i] = b_r exp(G_r - G_i) (k_r . k_i)            for i < r, else 0
 *   Tm      = (I + A)^{-1}                              (forward substitution)
 *   W       = Tm diag(b exp(G)) K,   U' = Tm diag(b) V,   U = U' - W S^T
 *   O       = diag(exp(G)) (scale Q) S^T + P U,
 *             P[r][i] = exp(G_r - G_i) (scale q_r . k_i) for i <= r, else 0
 *   S_next  = exp(G_{L-1}) S + U^T diag(exp(G_{L-1} - G)) K
 * Arguments as orc_recurrent, plus the chunk length C >= 1.
 */
int orc_chunked(const double *q, const double *k, const double *v, const double *g,
                const double *beta, const double *S0, const int32_t *cu, int N, int T, int H_qk,
                int H_v, int dk, int dv, double scale, int C, double *o, double *S_final,
                int h_lo, int h_hi)
{
    if (N < 1 || T < 0 || C < 1 || H_qk < 1 || H_v < 1 || H_v % H_qk != 0 || dk < 1 || dv < 1)
        return ORC_EINVAL;
    if (h_lo < 0 || h_hi > H_v || h_lo > h_hi)
        return ORC_EINVAL;
    for (int n = 0; n < N; ++n) {
        int s0 = 0, s1 = 0;
        if (seq_bounds(cu, N, T, n, &s0, &s1))
            return ORC_EINVAL;
    }
    const int group = H_v / H_qk;
    const int units = N * (h_hi - h_lo);
    const size_t ssz = (size_t)dv * dk;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        const int n = u / (h_hi - h_lo);
        const int h = h_lo + u % (h_hi - h_lo);
        const int hq = h / group;
        int s0 = 0, s1 = 0;
        seq_bounds(cu, N, T, n, &s0, &s1);
        double *S = (double *)malloc(sizeof(double) * ssz);
        double *Sn = (double *)malloc(sizeof(double) * ssz);
        double *G = (double *)malloc(sizeof(double) * C);
        double *A = (double *)malloc(sizeof(double) * C * C);
        double *Tm = (double *)malloc(sizeof(double) * C * C);
        double *W = (double *)malloc(sizeof(double) * (size_t)C * dk);
        double *U = (double *)malloc(sizeof(double) * (size_t)C * dv);
        if (!S || !Sn || !G || !A || !Tm || !W || !U) {
            free(S); free(Sn); free(G); free(A); free(Tm); free(W); free(U);
#pragma omp atomic write
            status = ORC_ENOMEM;
            continue;
        }
        if (S0)
            memcpy(S, S0 + ((size_t)n * H_v + h) * ssz, sizeof(double) * ssz);
        else
            memset(S, 0, sizeof(double) * ssz);
        for (int c0 = s0; c0 < s1; c0 += C) {
            const int L = (s1 - c0 < C) ? (s1 - c0) : C;
#define KV(r) (k + ((size_t)(c0 + (r)) * H_qk + hq) * dk)
#define QV(r) (q + ((size_t)(c0 + (r)) * H_qk + hq) * dk)
#define VV(r) (v + ((size_t)(c0 + (r)) * H_v + h) * dv)
#define GT(r) (g[(size_t)(c0 + (r)) * H_v + h])
#define BT(r) (beta[(size_t)(c0 + (r)) * H_v + h])
            /* cumulative log decay inside the chunk */
            double run = 0.0;
            for (int r = 0; r < L; ++r) {
                run += GT(r);
                G[r] = run;
            }
            /* A = strictly lower part of diag(b) Gamma (K K^T) */
            for (int r = 0; r < L; ++r)
                for (int i = 0; i < L; ++i) {
                    double val = 0.0;
                    if (i < r) {
                        double dot = 0.0;
                        for (int j = 0; j < dk; ++j)
                            dot += KV(r)[j] * KV(i)[j];
                        val = BT(r) * exp(G[r] - G[i]) * dot;
                    }
                    A[r * L + i] = val;
                }
            /* Tm = (I + A)^{-1}: solve (I + A) Tm = I column by column */
            for (int col = 0; col < L; ++col)
                for (int r = 0; r < L; ++r) {
                    double rhs = (r == col) ? 1.0 : 0.0;
                    for (int i = 0; i < r; ++i)
                        rhs -= A[r * L + i] * Tm[i * L + col];
                    Tm[r * L + col] = rhs;
                }
            /* W = Tm diag(b e^G) K ;  U = Tm diag(b) V - W S^T */
            for (int r = 0; r < L; ++r) {
                for (int j = 0; j < dk; ++j) {
                    double acc = 0.0;
                    for (int i = 0; i < L; ++i)
                        acc += Tm[r * L + i] * BT(i) * exp(G[i]) * KV(i)[j];
                    W[(size_t)r * dk + j] = acc;
                }
                for (int e = 0; e < dv; ++e) {
                    double up = 0.0;
                    for (int i = 0; i < L; ++i)
                        up += Tm[r * L + i] * BT(i) * VV(i)[e];
                    double ws = 0.0;
                    for (int j = 0; j < dk; ++j)
                        ws += W[(size_t)r * dk + j] * S[(size_t)e * dk + j];
                    U[(size_t)r * dv + e] = up - ws;
                }
            }
            /* P = lower part (incl. diagonal) of Gamma (scale Q K^T); reuses A */
            for (int r = 0; r < L; ++r)
                for (int i = 0; i < L; ++i) {
                    double val = 0.0;
                    if (i <= r) {
                        double dot = 0.0;
                        for (int j = 0; j < dk; ++j)
                            dot += scale * QV(r)[j] * KV(i)[j];
                        val = exp(G[r] - G[i]) * dot;
                    }
                    A[r * L + i] = val;
                }
            /* O = diag(e^G) (scale Q) S^T + P U */
            for (int r = 0; r < L; ++r) {
                double *orow = o + ((size_t)(c0 + r) * H_v + h) * dv;
                for (int e = 0; e < dv; ++e) {
                    double inter = 0.0;
                    for (int j = 0; j < dk; ++j)
                        inter += scale * QV(r)[j] * S[(size_t)e * dk + j];
                    double intra = 0.0;
                    for (int i = 0; i <= r; ++i)
                        intra += A[r * L + i] * U[(size_t)i * dv + e];
                    orow[e] = exp(G[r]) * inter + intra;
                }
            }
            /* S_next = e^{G_last} S + U^T diag(e^{G_last - G}) K */
            const double Gl = G[L - 1];
            for (int e = 0; e < dv; ++e)
                for (int j = 0; j < dk; ++j) {
                    double acc = exp(Gl) * S[(size_t)e * dk + j];
                    for (int i = 0; i < L; ++i)
                        acc += U[(size_t)i * dv + e] * exp(Gl - G[i]) * KV(i)[j];
                    Sn[(size_t)e * dk + j] = acc;
                }
            memcpy(S, Sn, sizeof(double) * ssz);
#undef KV
#undef QV
#undef VV
#undef GT
#undef BT
        }
        if (S_final)
            memcpy(S_final + ((size_t)n * H_v + h) * ssz, S, sizeof(double) * ssz);
        free(S); free(Sn); free(G); free(A); free(Tm); free(W); free(U);
    }
    return status;
}

/*
 * Gates from the raw per-token projections a, b of each V-head:
 *   g    = -softplus(a + dt_bias[h]) * exp(A_log[h])   (log of the decay a_t)
 *   beta = sigmoid(b) = 1 / (1 + exp(-b))
 * [Dissect sec. 2.1] names the layer's A_log and dt_bias weights; the formula
 * is the layer's gate parameterisation as the workloads state it.  softplus is
 * log(1 + exp(x)), written as max(x, 0) + log1p(exp(-|x|)), the same value
 * without overflow.
 * a, b [T][H_v]; A_log, dt_bias [H_v]; g, beta [T][H_v] outputs.
 */
int orc_gates(const double *a, const double *b, const double *A_log, const double *dt_bias,
              int T, int H_v, double *g, double *beta)
{
    if (T < 0 || H_v < 1)
        return ORC_EINVAL;
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H_v; ++h) {
            const size_t i = (size_t)t * H_v + h;
            const double x = a[i] + dt_bias[h];
            const double softplus = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
            g[i] = -softplus * exp(A_log[h]);
            beta[i] = 1.0 / (1.0 + exp(-b[i]));
        }
    }
    return ORC_OK;
}

/*
 * Output gate of the layer, per token and V-head: the d_v outputs o are
 * divided by their root mean square, scaled per channel by the norm weight w
 * and multiplied by SiLU(z):
 *   y[c] = o[c] / sqrt(mean_c(o^2) + eps) * w[c] * z[c] * sigmoid(z[c])
 * [Dissect sec. 2.1] lists the layer's norm and in_proj_z weights; the form
 * above is this oracle's reading of how they apply (the pages print no
 * formula).  o, z [R][dv]; w [dv]; y [R][dv]; R = rows (tokens x V-heads).
 */
int orc_gated_norm(const double *o, const double *z, const double *w, int R, int dv, double eps,
                   double *y)
{
    if (R < 0 || dv < 1)
        return ORC_EINVAL;
    for (int r = 0; r < R; ++r) {
        const double *orow = o + (size_t)r * dv;
        const double *zrow = z + (size_t)r * dv;
        double ss = 0.0;
        for (int c = 0; c < dv; ++c)
            ss += orow[c] * orow[c];
        const double inv = 1.0 / sqrt(ss / dv + eps);
        for (int c = 0; c < dv; ++c) {
            const double silu = zrow[c] / (1.0 + exp(-zrow[c]));
            y[(size_t)r * dv + c] = orow[c] * inv * w[c] * silu;
        }
    }
    return ORC_OK;
}

/*
 * Gradients of the token recurrence (reverse mode, the chain rule applied to
 * each step of orc_recurrent in reverse order).  [Local sec. 2.1] names a fused
 * forward and backward kernel for the GDN layer; the layer is trained, so its
 * gradients are part of what it computes.  Nothing about the method is new
 * here: for one step, with S = S_{t-1}, a = exp(g_t), u = S k_t and G the
 * gradient of the loss with respect to S_t (the later tokens' share plus
 * do_t (scale q_t)^T from o_t = S_t scale q_t):
 *     S_t   = a S + b (v_t - a u) k_t^T
 *     dq_t += scale S_t^T do_t           (summed over the V-heads of a QK head)
 *     w     = G k_t
 *     dv_t  = b w
 *     db_t  = (v_t - a u) . w
 *     dg_t  = a (<G, S> - b u . w)       (d/dg = a d/da)
 *     dk_t += b G^T (v_t - a u) - a b S^T w
 *     dS    = a (G - b w k_t^T)          (the gradient with respect to S_{t-1})
 * The states S_{t-1} are recomputed forward and kept for the whole sequence.
 *
 * Inputs as orc_recurrent, plus d_o [T][H_v][dv] (gradient of the loss with
 * respect to o) and dS_final [N][H_v][dv][dk] or NULL (with respect to the
 * final states; NULL = zero).  Outputs: dq, dk [T][H_qk][dk]; dv [T][H_v][dv];
 * dg, dbeta [T][H_v]; dS0 [N][H_v][dv][dk] or NULL (with respect to the
 * initial states).  Outputs are overwritten, not accumulated.  Work is split
 * over (sequence, QK head) so that the V-heads of a group, which add into the
 * same dq and dk, run in one thread.  Only QK heads in [hq_lo, hq_hi) and their
 * V-heads are computed; the other entries of every output are zero.
 */
int orc_recurrent_backward(const double *q, const double *k, const double *v, const double *g,
                           const double *beta, const double *S0, const int32_t *cu, int N,
                           int T, int H_qk, int H_v, int dk, int dv, double scale,
                           const double *d_o, const double *dS_final, double *dq, double *dkk,
                           double *dvv, double *dg, double *dbeta, double *dS0, int hq_lo,
                           int hq_hi)
{
    if (N < 1 || T < 0 || H_qk < 1 || H_v < 1 || H_v % H_qk != 0 || dk < 1 || dv < 1)
        return ORC_EINVAL;
    if (hq_lo < 0 || hq_hi > H_qk || hq_lo > hq_hi)
        return ORC_EINVAL;
    for (int n = 0; n < N; ++n) {
        int s0 = 0, s1 = 0;
        if (seq_bounds(cu, N, T, n, &s0, &s1))
            return ORC_EINVAL;
    }
    const int group = H_v / H_qk;
    const size_t ssz = (size_t)dv * dk;
    memset(dq, 0, sizeof(double) * (size_t)T * H_qk * dk);
    memset(dkk, 0, sizeof(double) * (size_t)T * H_qk * dk);
    memset(dvv, 0, sizeof(double) * (size_t)T * H_v * dv);
    memset(dg, 0, sizeof(double) * (size_t)T * H_v);
    memset(dbeta, 0, sizeof(double) * (size_t)T * H_v);
    if (dS0)
        memset(dS0, 0, sizeof(double) * (size_t)N * H_v * ssz);
    const int nq = hq_hi - hq_lo;
    int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < N * nq; ++u) {
        const int n = u / nq, hq = hq_lo + u % nq;
        int s0 = 0, s1 = 0;
        seq_bounds(cu, N, T, n, &s0, &s1);
        const int len = s1 - s0;
        double *St = (double *)malloc(sizeof(double) * ssz * ((size_t)len + 1));  /* S_{s0-1} .. S_{s1-1} */
        double *G = (double *)malloc(sizeof(double) * ssz);
        double *Sk = (double *)malloc(sizeof(double) * dv);
        double *w = (double *)malloc(sizeof(double) * dv);
        double *r = (double *)malloc(sizeof(double) * dv);
        if (!St || !G || !Sk || !w || !r) {
            free(St);
            free(G);
            free(Sk);
            free(w);
            free(r);
#pragma omp atomic write
            status = ORC_ENOMEM;
            continue;
        }
        for (int h = hq * group; h < (hq + 1) * group; ++h) {
            const size_t st_off = ((size_t)n * H_v + h) * ssz;
            if (S0)
                memcpy(St, S0 + st_off, sizeof(double) * ssz);
            else
                memset(St, 0, sizeof(double) * ssz);
            for (int t = s0; t < s1; ++t) {
                double *S = St + (size_t)(t - s0 + 1) * ssz;
                memcpy(S, S - ssz, sizeof(double) * ssz);
                delta_step(S, dk, dv, q + ((size_t)t * H_qk + hq) * dk,
                           k + ((size_t)t * H_qk + hq) * dk, v + ((size_t)t * H_v + h) * dv,
                           g[(size_t)t * H_v + h], beta[(size_t)t * H_v + h], scale, NULL, Sk);
            }
            if (dS_final)
                memcpy(G, dS_final + st_off, sizeof(double) * ssz);
            else
                memset(G, 0, sizeof(double) * ssz);
            for (int t = s1 - 1; t >= s0; --t) {
                const double *S = St + (size_t)(t - s0) * ssz;      /* S_{t-1} */
                const double *Snew = S + ssz;                      /* S_t */
                const double *qt = q + ((size_t)t * H_qk + hq) * dk;
                const double *kt = k + ((size_t)t * H_qk + hq) * dk;
                const double *vt = v + ((size_t)t * H_v + h) * dv;
                const double *dot = d_o + ((size_t)t * H_v + h) * dv;
                double *dqt = dq + ((size_t)t * H_qk + hq) * dk;
                double *dkt = dkk + ((size_t)t * H_qk + hq) * dk;
                const double a = exp(g[(size_t)t * H_v + h]), b = beta[(size_t)t * H_v + h];
                /* o_t = S_t (scale q_t) */
                for (int i = 0; i < dv; ++i)
                    for (int j = 0; j < dk; ++j) {
                        G[(size_t)i * dk + j] += dot[i] * scale * qt[j];
                        dqt[j] += scale * Snew[(size_t)i * dk + j] * dot[i];
                    }
                double gs = 0.0, uw = 0.0, rw = 0.0;
                for (int i = 0; i < dv; ++i) {
                    double su = 0.0, gw = 0.0;
                    for (int j = 0; j < dk; ++j) {
                        su += S[(size_t)i * dk + j] * kt[j];
                        gw += G[(size_t)i * dk + j] * kt[j];
                        gs += G[(size_t)i * dk + j] * S[(size_t)i * dk + j];
                    }
                    Sk[i] = su;
                    w[i] = gw;
                    r[i] = vt[i] - a * su;
                    uw += su * gw;
                    rw += r[i] * gw;
                }
                for (int i = 0; i < dv; ++i)
                    dvv[((size_t)t * H_v + h) * dv + i] = b * w[i];
                dbeta[(size_t)t * H_v + h] = rw;
                dg[(size_t)t * H_v + h] = a * (gs - b * uw);
                for (int j = 0; j < dk; ++j) {
                    double gr = 0.0, sw = 0.0;
                    for (int i = 0; i < dv; ++i) {
                        gr += G[(size_t)i * dk + j] * r[i];
                        sw += S[(size_t)i * dk + j] * w[i];
                    }
                    dkt[j] += b * gr - a * b * sw;
                }
                for (int i = 0; i < dv; ++i)
                    for (int j = 0; j < dk; ++j)
                        G[(size_t)i * dk + j] = a * (G[(size_t)i * dk + j] - b * w[i] * kt[j]);
            }
            if (dS0)
                memcpy(dS0 + st_off, G, sizeof(double) * ssz);
        }
        free(St);
        free(G);
        free(Sk);
        free(w);
        free(r);
    }
    return status;
}

/*
 * Gradients of orc_prelude (the chain rule through each of its steps, in
 * reverse): given dq, dk [T][H_qk][dk] and dv [T][H_v][dv] (gradients of the
 * loss with respect to the prelude's outputs), the gradients with respect to
 * the raw projections dx [T][C_raw] and the conv taps dw [C_raw][4] (both
 * overwritten).  For each token, with y the conv output of a channel,
 * a = SiLU(y), and for a q or k head n = a r, r = (sum a^2 + eps)^(-1/2):
 *     da = r (dn - n (n . dn))              (L2 norm; v channels: da = dv)
 *     dy = da sigmoid(y) (1 + y (1 - sigmoid(y)))      (SiLU)
 *     dx[t - 3 + j] += w[j] dy[t],  dw[j] += x[t - 3 + j] dy[t]
 * over the taps j whose source token t - 3 + j lies in the sequence
 * ([Dissect sec. 2.1]: conv of width 4 with the per-layer conv1d weight).
 */
int orc_prelude_backward(const double *x, const double *w, const int32_t *cu, int N, int T,
                         int H_qk, int H_v, int dk, int dv, double eps, const double *dq,
                         const double *dkk, const double *dvv, double *dx, double *dw)
{
    const int Cq = H_qk * dk;
    const int Craw = 2 * Cq + H_v * dv;
    if (T < 0 || N < 1 || H_qk < 1 || H_v < 1 || dk < 1 || dv < 1)
        return ORC_EINVAL;
    double *y = (double *)malloc(sizeof(double) * (size_t)Craw);
    double *dy = (double *)malloc(sizeof(double) * (size_t)Craw);
    if (!y || !dy) {
        free(y);
        free(dy);
        return ORC_ENOMEM;
    }
    memset(dx, 0, sizeof(double) * (size_t)T * Craw);
    memset(dw, 0, sizeof(double) * (size_t)Craw * 4);
    for (int n = 0; n < N; ++n) {
        int s0 = 0, s1 = 0;
        if (seq_bounds(cu, N, T, n, &s0, &s1)) {
            free(y);
            free(dy);
            return ORC_EINVAL;
        }
        for (int t = s0; t < s1; ++t) {
            for (int c = 0; c < Craw; ++c) {
                double acc = 0.0;
                for (int j = 0; j < 4; ++j) {
                    const int src = t - 3 + j;
                    if (src >= s0)
                        acc += w[(size_t)c * 4 + j] * x[(size_t)src * Craw + c];
                }
                y[c] = acc;
            }
            /* da into dy[], per channel */
            for (int part = 0; part < 2; ++part) {          /* q heads, then k heads */
                const double *dn_all = part == 0 ? dq : dkk;
                for (int h = 0; h < H_qk; ++h) {
                    const int c0 = part * Cq + h * dk;
                    const double *dn = dn_all + ((size_t)t * H_qk + h) * dk;
                    double ss = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        const double a = y[c0 + i] / (1.0 + exp(-y[c0 + i]));
                        ss += a * a;
                    }
                    const double r = 1.0 / sqrt(ss + eps);
                    double ndn = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        const double a = y[c0 + i] / (1.0 + exp(-y[c0 + i]));
                        ndn += a * r * dn[i];
                    }
                    for (int i = 0; i < dk; ++i) {
                        const double a = y[c0 + i] / (1.0 + exp(-y[c0 + i]));
                        dy[c0 + i] = r * (dn[i] - a * r * ndn);
                    }
                }
            }
            for (int c = 0; c < H_v * dv; ++c)
                dy[2 * Cq + c] = dvv[(size_t)t * H_v * dv + c];
            /* through SiLU, then the conv */
            for (int c = 0; c < Craw; ++c) {
                const double sg = 1.0 / (1.0 + exp(-y[c]));
                const double d = dy[c] * sg * (1.0 + y[c] * (1.0 - sg));
                for (int j = 0; j < 4; ++j) {
                    const int src = t - 3 + j;
                    if (src >= s0) {
                        dx[(size_t)src * Craw + c] += w[(size_t)c * 4 + j] * d;
                        dw[(size_t)c * 4 + j] += x[(size_t)src * Craw + c] * d;
                    }
                }
            }
        }
    }
    free(y);
    free(dy);
    return ORC_OK;
}

/*
 * Gradients of orc_gates: given dg, dbeta [T][H_v], the gradients with respect
 * to a, b [T][H_v] and A_log, dt_bias [H_v] (all overwritten).  With
 * g = -softplus(a + dt_bias) exp(A_log) and beta = sigmoid(b):
 *     da = -dg exp(A_log) sigmoid(a + dt_bias),   ddt_bias = sum over t of da,
 *     dA_log = sum over t of dg g,                db = dbeta beta (1 - beta).
 */
int orc_gates_backward(const double *a, const double *b, const double *A_log,
                       const double *dt_bias, int T, int H_v, const double *dg,
                       const double *dbeta, double *da, double *db, double *dA_log,
                       double *ddt_bias)
{
    if (T < 0 || H_v < 1)
        return ORC_EINVAL;
    for (int h = 0; h < H_v; ++h) {
        dA_log[h] = 0.0;
        ddt_bias[h] = 0.0;
    }
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H_v; ++h) {
            const size_t i = (size_t)t * H_v + h;
            const double xx = a[i] + dt_bias[h];
            const double softplus = (xx > 0.0 ? xx : 0.0) + log1p(exp(-fabs(xx)));
            const double g = -softplus * exp(A_log[h]);
            const double sg = 1.0 / (1.0 + exp(-xx));
            da[i] = -dg[i] * exp(A_log[h]) * sg;
            ddt_bias[h] += da[i];
            dA_log[h] += dg[i] * g;
            const double be = 1.0 / (1.0 + exp(-b[i]));
            db[i] = dbeta[i] * be * (1.0 - be);
        }
    }
    return ORC_OK;
}

/*
 * Gradients of orc_gated_norm: given dy [R][dv], the gradients with respect
 * to o, z [R][dv] and w [dv] (all overwritten).  Per row, with
 * r = (mean(o^2) + eps)^(-1/2), n = o r, s = SiLU(z) and u = dy w s:
 *     do = r (u - n mean(u n)),   dz = dy n w SiLU'(z),   dw += dy n s.
 */
int orc_gated_norm_backward(const double *o, const double *z, const double *w, int R, int dv,
                            double eps, const double *dy, double *d_o, double *dz, double *dw)
{
    if (R < 0 || dv < 1)
        return ORC_EINVAL;
    for (int c = 0; c < dv; ++c)
        dw[c] = 0.0;
    for (int r = 0; r < R; ++r) {
        const double *orow = o + (size_t)r * dv, *zrow = z + (size_t)r * dv;
        const double *dyr = dy + (size_t)r * dv;
        double ss = 0.0;
        for (int c = 0; c < dv; ++c)
            ss += orow[c] * orow[c];
        const double inv = 1.0 / sqrt(ss / dv + eps);
        double un = 0.0;
        for (int c = 0; c < dv; ++c) {
            const double sg = 1.0 / (1.0 + exp(-zrow[c]));
            un += dyr[c] * w[c] * zrow[c] * sg * orow[c] * inv;
        }
        for (int c = 0; c < dv; ++c) {
            const double sg = 1.0 / (1.0 + exp(-zrow[c]));
            const double n = orow[c] * inv, s = zrow[c] * sg;
            d_o[(size_t)r * dv + c] = inv * (dyr[c] * w[c] * s - n * un / dv);
            dz[(size_t)r * dv + c] = dyr[c] * n * w[c] * sg * (1.0 + zrow[c] * (1.0 - sg));
            dw[c] += dyr[c] * n * s;
        }
    }
    return ORC_OK;
}

int orc_version(void) { return 1; }
