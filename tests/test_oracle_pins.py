"""Pins of the fp64 oracle against things other than itself (CPU only).

Page keys used below:
  [Dissect] "从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力" (www.2kiu.com)
  [Local]   "Qwen3.8-27B：27B 如何打出千亿级效果，且塞进单张消费级显卡" (www.nzsm.cn)
"""
import json
import os

import numpy as np
import pytest
import torch

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand_case(rng, T, H_qk, H_v, dk, dv, unit_k=False, g_lo=0.01, g_hi=0.6):
    q = rng.standard_normal((T, H_qk, dk))
    k = rng.standard_normal((T, H_qk, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H_v, dv))
    g = -rng.uniform(g_lo, g_hi, (T, H_v))
    beta = rng.uniform(0.0, 1.0, (T, H_v))
    return q, k, v, g, beta


# --------------------------------------------------------------- recurrence
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_recurrent_equals_bruteforce_product(orc, T):
    """Brute force: S_T = S_0 prod_t M_t + sum_t b_t v_t k_t^T prod_{s>t} M_s with
    M_t = a_t (I - b_t k_t k_t^T), and o_t = S_t q_t, built from explicit dk x dk
    matrices.  dk != dv and two QK groups catch transposes and head mix-ups."""
    rng = np.random.default_rng(10 + T)
    H_qk, H_v, dk, dv = 2, 4, 5, 3
    q, k, v, g, beta = _rand_case(rng, T, H_qk, H_v, dk, dv)
    S0 = rng.standard_normal((1, H_v, dv, dk))
    o, S = orc.recurrent(q, k, v, g, beta, initial_state=S0)
    grp = H_v // H_qk
    for h in range(H_v):
        hq = h // grp
        M = [np.exp(g[t, h]) * (np.eye(dk) - beta[t, h] * np.outer(k[t, hq], k[t, hq]))
             for t in range(T)]
        for tt in range(1, T + 1):          # state after tt tokens
            prod = np.eye(dk)
            for t in range(tt):
                prod = prod @ M[t]
            St = S0[0, h] @ prod
            for t in range(tt):
                tail = np.eye(dk)
                for s in range(t + 1, tt):
                    tail = tail @ M[s]
                St = St + beta[t, h] * np.outer(v[t, h], k[t, hq]) @ tail
            np.testing.assert_allclose(o[tt - 1, h], St @ q[tt - 1, hq], rtol=1e-12, atol=1e-12)
            if tt == T:
                np.testing.assert_allclose(S[0, h], St, rtol=1e-12, atol=1e-12)


def test_beta_zero_alpha_one_keeps_state(orc):
    """b = 0 and a = 1: nothing is erased or written, S stays S_0, o_t = S_0 q_t."""
    rng = np.random.default_rng(1)
    q, k, v, g, beta = _rand_case(rng, 9, 1, 2, 6, 4)
    g[:] = 0.0
    beta[:] = 0.0
    S0 = rng.standard_normal((1, 2, 4, 6))
    o, S = orc.recurrent(q, k, v, g, beta, initial_state=S0)
    np.testing.assert_array_equal(S, S0)
    for h in range(2):
        np.testing.assert_allclose(o[:, h], q[:, 0] @ S0[0, h].T, rtol=1e-13, atol=1e-13)


def test_beta_zero_pure_decay(orc):
    """b = 0: S_t = exp(G_t) S_0 with G_t the running sum of g."""
    rng = np.random.default_rng(2)
    q, k, v, g, beta = _rand_case(rng, 11, 1, 3, 5, 5)
    beta[:] = 0.0
    S0 = rng.standard_normal((1, 3, 5, 5))
    o, S = orc.recurrent(q, k, v, g, beta, initial_state=S0)
    G = np.cumsum(g, axis=0)
    for h in range(3):
        np.testing.assert_allclose(S[0, h], np.exp(G[-1, h]) * S0[0, h], rtol=1e-12)
        np.testing.assert_allclose(o[:, h], np.exp(G[:, h])[:, None] * (q[:, 0] @ S0[0, h].T),
                                   rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("g_val", [0.0, -0.3, -4.0])
def test_full_strength_write_overwrites(orc, g_val):
    """[Dissect sec. 2.2] erase-then-write: with b = 1 and |k| = 1 the state maps
    k_t exactly to v_t after step t, whatever the decay.  With q_t = k_t the
    output o_t = S_t k_t must equal v_t."""
    rng = np.random.default_rng(3)
    q, k, v, g, beta = _rand_case(rng, 13, 1, 2, 7, 5, unit_k=True)
    g[:] = g_val
    beta[:] = 1.0
    S0 = rng.standard_normal((1, 2, 5, 7))
    o, _ = orc.recurrent(k, k, v, g, beta, initial_state=S0)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


def test_scalar_case_is_ema(orc):
    """dk = dv = 1, k = 1, a = 1: s_t = (1 - b_t) s_{t-1} + b_t v_t (an exponential
    moving average), o_t = s_t q_t."""
    rng = np.random.default_rng(4)
    T = 20
    q = rng.standard_normal((T, 1, 1))
    k = np.ones((T, 1, 1))
    v = rng.standard_normal((T, 1, 1))
    g = np.zeros((T, 1))
    beta = rng.uniform(0, 1, (T, 1))
    o, S = orc.recurrent(q, k, v, g, beta, initial_state=np.array([[[[0.7]]]]))
    s = 0.7
    for t in range(T):
        s = (1 - beta[t, 0]) * s + beta[t, 0] * v[t, 0, 0]
        assert abs(o[t, 0, 0] - s * q[t, 0, 0]) < 1e-13
    assert abs(S[0, 0, 0, 0] - s) < 1e-13


def test_orthonormal_keys_store_columns(orc):
    """k_t = e_t, S_0 = 0, a = b = 1: column t of S is v_t, and a query e_s
    returns v_s once it has been written."""
    dk, dv, T = 8, 3, 8
    rng = np.random.default_rng(5)
    k = np.eye(dk)[:T].reshape(T, 1, dk)
    v = rng.standard_normal((T, 1, dv))
    g = np.zeros((T, 1))
    beta = np.ones((T, 1))
    o, S = orc.recurrent(np.zeros_like(k), k, v, g, beta)
    np.testing.assert_array_equal(S[0, 0], v[:, 0, :].T)
    for s in range(T):
        qs = np.zeros((T, 1, dk))
        qs[:, 0, s] = 1.0
        o, _ = orc.recurrent(qs, k, v, g, beta)
        np.testing.assert_array_equal(o[s:, 0], np.repeat(v[s:s + 1, 0], T - s, axis=0))
        np.testing.assert_array_equal(o[:s, 0], 0.0)


def test_linear_in_state_and_values(orc):
    """For fixed q, k, g, b the layer is linear in (S_0, V) jointly."""
    rng = np.random.default_rng(6)
    q, k, v1, g, beta = _rand_case(rng, 17, 1, 3, 6, 4)
    v2 = rng.standard_normal(v1.shape)
    A = rng.standard_normal((1, 3, 4, 6))
    B = rng.standard_normal((1, 3, 4, 6))
    o1, S1 = orc.recurrent(q, k, v1, g, beta, initial_state=A)
    o2, S2 = orc.recurrent(q, k, v2, g, beta, initial_state=B)
    o3, S3 = orc.recurrent(q, k, 2 * v1 - 3 * v2, g, beta, initial_state=2 * A - 3 * B)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(S3, 2 * S1 - 3 * S2, rtol=1e-11, atol=1e-11)


def test_state_stays_bounded(orc):
    """|a (I - b k k^T)|_2 <= 1 for unit k and b in [0, 1], so |S_t|_F <= |S_{t-1}|_F
    + b_t |v_t| ; check the running bound along a long sequence."""
    rng = np.random.default_rng(7)
    T = 200
    q, k, v, g, beta = _rand_case(rng, T, 1, 1, 6, 6, unit_k=True, g_lo=0.0, g_hi=0.05)
    bound = 0.0
    for t in range(1, T + 1, 37):
        _, S = orc.recurrent(q[:t], k[:t], v[:t], g[:t], beta[:t])
        bound_t = np.sum(beta[:t, 0] * np.linalg.norm(v[:t, 0], axis=-1))
        assert np.linalg.norm(S[0, 0]) <= bound_t + 1e-12
        bound = max(bound, bound_t)


def test_varlen_equals_separate_runs(orc):
    rng = np.random.default_rng(8)
    lens = [5, 1, 12, 7]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta = _rand_case(rng, T, 2, 4, 6, 5)
    S0 = rng.standard_normal((4, 4, 5, 6))
    o, S = orc.recurrent(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu)
    for n in range(4):
        sl = slice(cu[n], cu[n + 1])
        on, Sn = orc.recurrent(q[sl], k[sl], v[sl], g[sl], beta[sl], initial_state=S0[n:n + 1])
        np.testing.assert_array_equal(o[sl], on)
        np.testing.assert_array_equal(S[n], Sn[0])


@pytest.mark.parametrize("split", [1, 7, 16, 29])
def test_split_with_state_handoff(orc, split):
    """The final state is a checkpoint: running [0, s) then [s, T) from the
    handed-over state equals the unsplit run."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta = _rand_case(rng, 30, 1, 3, 6, 5)
    o, S = orc.recurrent(q, k, v, g, beta)
    oa, Sa = orc.recurrent(q[:split], k[:split], v[:split], g[:split], beta[:split])
    ob, Sb = orc.recurrent(q[split:], k[split:], v[split:], g[split:], beta[split:],
                           initial_state=Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(Sb, S, rtol=1e-13, atol=1e-13)


def test_heads_subset_matches_full(orc):
    rng = np.random.default_rng(11)
    q, k, v, g, beta = _rand_case(rng, 10, 2, 6, 4, 4)
    o, S = orc.recurrent(q, k, v, g, beta)
    o2, S2 = orc.recurrent(q, k, v, g, beta, heads=(2, 5))
    np.testing.assert_array_equal(o2[:, 2:5], o[:, 2:5])
    np.testing.assert_array_equal(S2[:, 2:5], S[:, 2:5])
    assert not o2[:, :2].any() and not o2[:, 5:].any()


# ------------------------------------------------------------- chunked form
@pytest.mark.parametrize("C", [1, 2, 16, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_chunked_equals_recurrent(orc, C, T):
    rng = np.random.default_rng(100 * C + T)
    q, k, v, g, beta = _rand_case(rng, T, 1, 3, 16, 12, unit_k=True)
    S0 = rng.standard_normal((1, 3, 12, 16))
    o, S = orc.recurrent(q, k, v, g, beta, initial_state=S0, scale=0.5)
    oc, Sc = orc.chunked(q, k, v, g, beta, initial_state=S0, scale=0.5, chunk=C)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-10)


def test_chunked_strong_decay_and_varlen(orc):
    """Cumulative log decay inside a chunk far below the fp32 exp range
    (about -270) and sequence boundaries that fall inside chunks."""
    rng = np.random.default_rng(12)
    lens = [70, 3, 130]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta = _rand_case(rng, T, 1, 3, 16, 8, unit_k=True, g_lo=3.0, g_hi=5.5)
    S0 = rng.standard_normal((3, 3, 8, 16))
    o, S = orc.recurrent(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu)
    oc, Sc = orc.chunked(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu, chunk=64)
    G = np.cumsum(g[:64, 0])
    assert G[-1] < -190
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(Sc, S, rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------- prelude
def _prelude_reference_torch(x, w, cu, H_qk, H_v, dk, dv):
    """torch.nn.functional.conv1d (fp64, groups = channels, left padding 3 via
    symmetric padding then keeping the first T outputs) + silu + normalize."""
    F = torch.nn.functional
    outs = []
    for n in range(len(cu) - 1):
        xs = torch.from_numpy(x[cu[n]:cu[n + 1]]).T[None]          # [1, C, Tn]
        Tn = xs.shape[-1]
        y = F.conv1d(xs, torch.from_numpy(w)[:, None, :], padding=3, groups=w.shape[0])
        outs.append(F.silu(y[0, :, :Tn]).T)
    y = torch.cat(outs)
    Cq = H_qk * dk
    q = F.normalize(y[:, :Cq].reshape(-1, H_qk, dk), dim=-1, eps=0.0)
    k = F.normalize(y[:, Cq:2 * Cq].reshape(-1, H_qk, dk), dim=-1, eps=0.0)
    v = y[:, 2 * Cq:].reshape(-1, H_v, dv)
    return q.numpy(), k.numpy(), v.numpy()


def test_prelude_equals_torch_conv1d(orc):
    rng = np.random.default_rng(13)
    H_qk, H_v, dk, dv = 2, 6, 8, 4
    lens = [9, 2, 17, 1]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    C = 2 * H_qk * dk + H_v * dv
    x = rng.standard_normal((T, C))
    w = rng.normal(0, 0.5, (C, 4))
    q, k, v = orc.prelude(x, w, cu, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, eps=0.0)
    qr, kr, vr = _prelude_reference_torch(x, w, cu, H_qk, H_v, dk, dv)
    np.testing.assert_allclose(q, qr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(k, kr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v, vr, rtol=1e-12, atol=1e-12)


def test_prelude_identity_taps_and_eps(orc):
    """Taps (0, 0, 0, 1) pass the current token through; a constant head of value
    c gives q_i = silu(c) / sqrt(dk silu(c)^2 + eps)."""
    H_qk, H_v, dk, dv = 1, 1, 4, 2
    C = 2 * dk + dv
    w = np.zeros((C, 4))
    w[:, 3] = 1.0
    x = np.full((3, C), 0.25)
    x[:, dk:] = np.linspace(-1, 1, C - dk)
    eps = 1e-6
    q, k, v = orc.prelude(x, w, None, H_qk=1, H_v=1, dk=dk, dv=dv, eps=eps)
    s = 0.25 / (1 + np.exp(-0.25))
    np.testing.assert_allclose(q[:, 0, :], s / np.sqrt(dk * s * s + eps), rtol=1e-14)
    xs = x[:, 2 * dk:]
    np.testing.assert_allclose(v[:, 0, :], xs / (1 + np.exp(-xs)), rtol=1e-14)
    norms = np.linalg.norm(k[:, 0, :], axis=-1)
    assert np.all(norms < 1.0) and np.all(norms > 0.99)


def test_prelude_conv_resets_at_sequence_start(orc):
    """A sequence's first outputs must not see the previous sequence's tokens."""
    rng = np.random.default_rng(14)
    dk, dv = 4, 4
    C = 2 * dk + dv
    x = rng.standard_normal((10, C))
    w = rng.standard_normal((C, 4))
    cu = np.array([0, 6, 10], dtype=np.int32)
    q, k, v = orc.prelude(x, w, cu, H_qk=1, H_v=1, dk=dk, dv=dv)
    q2, k2, v2 = orc.prelude(x[6:], w, None, H_qk=1, H_v=1, dk=dk, dv=dv)
    np.testing.assert_array_equal(v[6:], v2)
    np.testing.assert_array_equal(q[6:], q2)


def test_prelude_history_equals_conv1d_over_the_joined_sequence(orc):
    """A prelude resumed with conv_state_in: each sequence's outputs are the
    last rows of torch's conv1d prelude over its history rows followed by its
    own rows (the history is the raw rows before its start)."""
    rng = np.random.default_rng(15)
    H_qk, H_v, dk, dv = 1, 3, 8, 4
    lens = [7, 1, 0, 2, 12]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    C = 2 * H_qk * dk + H_v * dv
    x = rng.standard_normal((T, C))
    w = rng.normal(0, 0.5, (C, 4))
    hist = rng.standard_normal((len(lens), 3, C))
    q, k, v = orc.prelude(x, w, cu, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, eps=0.0,
                          conv_state_in=hist)
    for n, (s0, s1) in enumerate(zip(cu[:-1], cu[1:])):
        joined = np.concatenate([hist[n], x[s0:s1]])
        qr, kr, vr = _prelude_reference_torch(joined, w, np.array([0, len(joined)], np.int32),
                                              H_qk, H_v, dk, dv)
        np.testing.assert_allclose(q[s0:s1], qr[3:], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(k[s0:s1], kr[3:], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(v[s0:s1], vr[3:], rtol=1e-12, atol=1e-12)
    # zero history is no history
    z = orc.prelude(x, w, cu, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv,
                    conv_state_in=np.zeros_like(hist))
    for a, b in zip(z, orc.prelude(x, w, cu, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv)):
        np.testing.assert_array_equal(a, b)


def test_prelude_split_at_any_row_with_carried_history(orc):
    """Cutting a sequence anywhere and passing the first part's conv_state as
    the second part's conv_state_in reproduces the whole sequence's prelude."""
    rng = np.random.default_rng(16)
    dk, dv = 4, 4
    C = 2 * dk + dv
    x = rng.standard_normal((11, C))
    w = rng.standard_normal((C, 4))
    whole = orc.prelude(x, w, None, H_qk=1, H_v=1, dk=dk, dv=dv)
    for cut in (0, 1, 2, 3, 4, 10, 11):
        hist = orc.conv_state(x[:cut])
        part = orc.prelude(x[cut:], w, None, H_qk=1, H_v=1, dk=dk, dv=dv, conv_state_in=hist)
        for a, b in zip(part, whole):
            np.testing.assert_allclose(a, b[cut:], rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------------ decode
def test_decode_step_matches_one_token_prefill_and_spares_other_slots(orc):
    d = synth.decode_inputs(21, B=5, P=9, H_qk=2, H_v=6, dk=16, dv=8)
    o, pool = orc.decode_step(d.q, d.k, d.v, d.g, d.beta, d.pool, d.slot_idx)
    for b in range(d.B):
        s = d.slot_idx[b]
        ob, Sb = orc.recurrent(d.q[b:b + 1], d.k[b:b + 1], d.v[b:b + 1], d.g[b:b + 1],
                               d.beta[b:b + 1], initial_state=d.pool[s:s + 1])
        np.testing.assert_array_equal(o[b], ob[0])
        np.testing.assert_array_equal(pool[s], Sb[0])
    untouched = np.setdiff1d(np.arange(d.P), d.slot_idx)
    assert np.isnan(pool[untouched]).all()
    assert (pool[untouched].astype(np.float32).view(np.uint32) == synth.CANARY_BITS).all()


# ------------------------------------------------------------------- gates
def test_gates_against_library_forms_and_identities(orc):
    """g = -softplus(a + dt_bias) exp(A_log), beta = sigmoid(b): against numpy's
    logaddexp (softplus(x) = log(e^0 + e^x)) and the logistic function, the
    closed values at zero, and softplus(x) - softplus(-x) = x."""
    rng = np.random.default_rng(31)
    T, H = 50, 6
    a = rng.normal(0.0, 4.0, (T, H))
    b = rng.normal(0.0, 4.0, (T, H))
    A_log = rng.uniform(-1, 1, H)
    dt = rng.uniform(-1, 1, H)
    g, beta = orc.gates(a, b, A_log, dt)
    np.testing.assert_allclose(g, -np.logaddexp(0.0, a + dt) * np.exp(A_log), rtol=1e-13)
    np.testing.assert_allclose(beta, 1.0 / (1.0 + np.exp(-b)), rtol=1e-13)
    np.testing.assert_allclose(beta + orc.gates(a, -b, A_log, dt)[1], 1.0, rtol=1e-14)
    g_neg, _ = orc.gates(-a - 2 * dt, b, A_log, dt)          # softplus(-(a + dt))
    np.testing.assert_allclose((-g + g_neg) / np.exp(A_log), a + dt, atol=1e-12)
    z = np.zeros((1, 2))
    g0, b0 = orc.gates(z, z, np.array([0.0, np.log(2.0)]), np.zeros(2))
    np.testing.assert_allclose(g0, [[-np.log(2.0), -2 * np.log(2.0)]], rtol=1e-15)
    np.testing.assert_allclose(b0, 0.5, rtol=0)
    big = orc.gates(np.array([[-800.0, 800.0]]), z, np.zeros(2), np.zeros(2))[0]
    assert big[0, 0] == -0.0 or abs(big[0, 0]) < 1e-300
    assert big[0, 1] == -800.0                               # no overflow for large a


def test_gates_match_the_workload_recipe(orc):
    """The oracle's gates reproduce the g, beta the input recipe stores (an
    independent numpy evaluation, rounded to fp32)."""
    p = synth.raw_prefill(41, T=100, H_qk=2, H_v=6, dk=8, dv=8)
    g, beta = orc.gates(p.meta["a"].astype(np.float64), p.meta["b"].astype(np.float64),
                        p.meta["A_log"], p.meta["dt_bias"])
    np.testing.assert_allclose(g, p.g, rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(beta, p.beta, rtol=2e-6, atol=1e-7)


# --------------------------------------------------- decode from raw rows
def test_conv_state_is_last_three_rows(orc):
    x = np.arange(10 * 3, dtype=np.float64).reshape(10, 3)
    cs = orc.conv_state(x, np.array([0, 5, 7, 7, 10], dtype=np.int32))
    np.testing.assert_array_equal(cs[0], x[2:5])
    np.testing.assert_array_equal(cs[1], np.vstack([np.zeros((1, 3)), x[5:7]]))
    np.testing.assert_array_equal(cs[2], np.zeros((3, 3)))       # empty sequence
    np.testing.assert_array_equal(cs[3], x[7:10])
    # rows missing before a short sequence's start come from the end of its history
    hist = -np.arange(4 * 9, dtype=np.float64).reshape(4, 3, 3) - 1
    ch = orc.conv_state(x, np.array([0, 5, 7, 7, 10], dtype=np.int32), conv_state_in=hist)
    np.testing.assert_array_equal(ch[0], x[2:5])
    np.testing.assert_array_equal(ch[1], np.vstack([hist[1, 2:], x[5:7]]))
    np.testing.assert_array_equal(ch[2], hist[2])
    np.testing.assert_array_equal(ch[3], x[7:10])


def test_raw_decode_chain_equals_prefill(orc):
    """T decode steps from raw rows, each conv window being the slot's three
    previous raw rows plus the new row, starting from zero history, give the
    outputs, final states and final conv history of one prelude + gates +
    recurrence over the T-token sequences (rolling conv state = causal conv)."""
    rng = np.random.default_rng(51)
    B, T, H_qk, H_v, dk, dv = 3, 7, 2, 4, 8, 6
    C = 2 * H_qk * dk + H_v * dv
    x = synth.bf16_bits(rng.standard_normal((B, T, C)).astype(np.float32))
    w = synth.bf16_bits(rng.normal(0, 0.5, (C, 4)).astype(np.float32))
    a = rng.standard_normal((B, T, H_v))
    b = rng.standard_normal((B, T, H_v))
    A_log, dt = rng.uniform(-1, 1, H_v), rng.uniform(-1, 1, H_v)
    S0 = rng.normal(0, 0.1, (B, H_v, dv, dk))
    P = 5
    slots = np.array([4, 0, 2], dtype=np.int32)
    pool = np.full((P, H_v, dv, dk), np.nan)
    pool[slots] = S0
    cs = np.zeros((P, 3, C), dtype=np.uint16)
    outs = []
    for t in range(T):
        o, cs, pool = orc.decode_step_raw(x[:, t], w, cs, a[:, t], b[:, t], A_log, dt, pool,
                                          slots, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv)
        outs.append(o)
    xs = x.reshape(B * T, C)
    cu = np.arange(0, B * T + 1, T, dtype=np.int32)
    q, k, v = orc.prelude(xs, w, cu, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv)
    g, beta = orc.gates(a.reshape(B * T, H_v), b.reshape(B * T, H_v), A_log, dt)
    o_ref, S_ref = orc.recurrent(q, k, v, g, beta, S0, cu)
    np.testing.assert_allclose(np.stack(outs, axis=1).reshape(B * T, H_v, dv), o_ref,
                               rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(pool[slots], S_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(cs[slots], orc.conv_state(xs, cu))
    assert np.isnan(pool[[1, 3]]).all() and (cs[[1, 3]] == 0).all()


# ----------------------------------------------- multi-token verification
def test_decode_multi_step_equals_prefill_and_rollback(orc):
    """n tokens per sequence through decode_multi_step equal a prefill of those
    n tokens from each slot's state (outputs and final state); every snapshot j
    equals the prefill of the first j tokens; rolling back to n_keep gives the
    state after n_keep tokens."""
    rng = np.random.default_rng(61)
    B, n, H_qk, H_v, dk, dv, P = 3, 4, 2, 4, 8, 6, 5
    q = rng.standard_normal((B, n, H_qk, dk))
    k = rng.standard_normal((B, n, H_qk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, n, H_v, dv))
    g = -rng.uniform(0.01, 0.5, (B, n, H_v))
    beta = rng.uniform(0, 1, (B, n, H_v))
    slots = np.array([2, 4, 0], dtype=np.int32)
    pool = rng.normal(0, 0.1, (P, H_v, dv, dk))
    o, snaps, new_pool = orc.decode_multi_step(q, k, v, g, beta, pool, slots)
    for b in range(B):
        s = slots[b]
        o_ref, S_ref = orc.recurrent(q[b], k[b], v[b], g[b], beta[b], pool[s:s + 1])
        np.testing.assert_allclose(o[b], o_ref, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(new_pool[s], S_ref[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(snaps[b, 0], pool[s])
        for j in range(1, n):
            _, S_j = orc.recurrent(q[b, :j], k[b, :j], v[b, :j], g[b, :j], beta[b, :j],
                                   pool[s:s + 1])
            np.testing.assert_allclose(snaps[b, j], S_j[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(new_pool[[1, 3]], pool[[1, 3]])
    keep = np.array([0, 4, 2])
    rolled = orc.state_rollback(snaps, keep, new_pool, slots)
    np.testing.assert_array_equal(rolled[2], pool[2])           # nothing kept
    np.testing.assert_array_equal(rolled[4], new_pool[4])       # everything kept
    np.testing.assert_array_equal(rolled[0], snaps[2, 2])


# ------------------------------------------------------------ output gate
def test_gated_norm_against_torch_and_invariants(orc):
    """Against torch's rms_norm and silu (library routines the oracle does not
    use), scale invariance of the norm, and zero output where z = 0."""
    rng = np.random.default_rng(71)
    o = rng.normal(0, 3, (5, 7, 16))
    z = rng.normal(0, 2, (5, 7, 16))
    w = rng.uniform(0.5, 1.5, 16)
    y = orc.gated_norm(o, z, w, eps=1e-6)
    ref = (torch.nn.functional.rms_norm(torch.from_numpy(o), (16,), torch.from_numpy(w), eps=1e-6)
           * torch.nn.functional.silu(torch.from_numpy(z))).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(orc.gated_norm(37.5 * o, z, w, eps=0.0),
                               orc.gated_norm(o, z, w, eps=0.0), rtol=1e-13)
    z0 = z.copy()
    z0[:, :, 3] = 0.0
    assert (orc.gated_norm(o, z0, w)[:, :, 3] == 0).all()
    # one-hot rows: the norm maps e_c to sqrt(d_v) e_c
    oh = np.zeros((1, 16))
    oh[0, 5] = 2.0
    big = np.full((1, 16), 60.0)                    # SiLU(60) = 60 to double precision
    np.testing.assert_allclose(orc.gated_norm(oh, big, np.ones(16), eps=0.0)[0, 5], 4.0 * 60.0,
                               rtol=1e-13)


# ------------------------------------------------------------- backward
def _loss_weights(rng, o_shape, S_shape):
    return rng.standard_normal(o_shape), rng.standard_normal(S_shape)


@pytest.mark.parametrize("with_state", [True, False])
def test_backward_equals_finite_differences(orc, with_state):
    """Every gradient of the recurrence against central differences of the
    forward oracle (L = <W_o, o> + <W_S, S_final>, step 1e-6): two QK groups
    of two V-heads, d_k != d_v, packed sequences of lengths 4, 1, 0, 3, and
    with and without an initial state and a final-state gradient."""
    rng = np.random.default_rng(80 + with_state)
    H_qk, H_v, dk, dv = 2, 4, 3, 2
    cu = np.array([0, 4, 5, 5, 8], dtype=np.int32)
    T, N = 8, 4
    q, k, v, g, beta = _rand_case(rng, T, H_qk, H_v, dk, dv, unit_k=True)
    S0 = rng.standard_normal((N, H_v, dv, dk)) if with_state else None
    Wo, WS = _loss_weights(rng, (T, H_v, dv), (N, H_v, dv, dk))
    if not with_state:
        WS = None
    scale = 0.7

    def loss(q, k, v, g, beta, S0):
        o, S = orc.recurrent(q, k, v, g, beta, S0, cu, scale=scale)
        return (o * Wo).sum() + (0.0 if WS is None else (S * WS).sum())

    grads = orc.recurrent_backward(q, k, v, g, beta, Wo, S0, WS, cu, scale=scale)
    args = [q, k, v, g, beta] + ([S0] if with_state else [])
    names = ["dq", "dk", "dv", "dg", "dbeta", "dS0"]
    for ai, a in enumerate(args):
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            ap = [x.copy() for x in args]
            am = [x.copy() for x in args]
            ap[ai][idx] += 1e-6
            am[ai][idx] -= 1e-6
            if not with_state:
                ap.append(None)
                am.append(None)
            fd[idx] = (loss(*ap) - loss(*am)) / 2e-6
        np.testing.assert_allclose(grads[ai], fd, rtol=0, atol=1e-7 * max(1.0, np.abs(fd).max()),
                                   err_msg=names[ai])
    if not with_state:
        # no initial state is a zero initial state; its gradient is still defined
        S0z = np.zeros((N, H_v, dv, dk))
        gz = orc.recurrent_backward(q, k, v, g, beta, Wo, S0z, None, cu, scale=scale)
        for a, b in zip(grads[:5], gz[:5]):
            np.testing.assert_array_equal(a, b)


def test_backward_against_torch_autograd(orc):
    """Against torch autograd (fp64) through a plain step loop written with
    torch ops, an implementation that shares nothing with the oracle's."""
    rng = np.random.default_rng(83)
    T, H_qk, H_v, dk, dv = 12, 1, 3, 5, 4
    q, k, v, g, beta = _rand_case(rng, T, H_qk, H_v, dk, dv, unit_k=True, g_hi=1.5)
    S0 = rng.standard_normal((1, H_v, dv, dk))
    Wo, WS = _loss_weights(rng, (T, H_v, dv), (1, H_v, dv, dk))
    ts = [torch.tensor(a, requires_grad=True) for a in (q, k, v, g, beta, S0)]
    tq, tk, tv, tg, tb, tS0 = ts
    loss = 0.0
    for h in range(H_v):
        S = tS0[0, h]
        for t in range(T):
            kt = tk[t, 0]
            S = torch.exp(tg[t, h]) * (S - tb[t, h] * torch.outer(S @ kt, kt)) \
                + tb[t, h] * torch.outer(tv[t, h], kt)
            loss = loss + (S @ (0.5 * tq[t, 0])) @ torch.from_numpy(Wo[t, h])
        loss = loss + (S * torch.from_numpy(WS[0, h])).sum()
    loss.backward()
    grads = orc.recurrent_backward(q, k, v, g, beta, Wo, S0, WS, scale=0.5)
    for got, t in zip(grads, ts):
        np.testing.assert_allclose(got, t.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_adjoint_identities(orc):
    """(o, S_final) is linear in (v, S_0) jointly and o is linear in q, so for
    any output gradients <dv, v> + <dS0, S_0> = <d_o, o> + <dS_T, S_T> and
    <dq, q> = <d_o, o> (Euler's identity for degree-1 homogeneous maps); at the
    real head size, several V-heads per QK head, ragged sequences."""
    rng = np.random.default_rng(84)
    cu = np.array([0, 70, 71, 200], dtype=np.int32)
    T, N, H_qk, H_v, d = 200, 3, 1, 3, 128
    q, k, v, g, beta = _rand_case(rng, T, H_qk, H_v, d, d, unit_k=True)
    S0 = rng.standard_normal((N, H_v, d, d))
    Wo, WS = _loss_weights(rng, (T, H_v, d), (N, H_v, d, d))
    o, S = orc.recurrent(q, k, v, g, beta, S0, cu)
    dq, dk_, dv, dg, db, dS0 = orc.recurrent_backward(q, k, v, g, beta, Wo, S0, WS, cu)
    lhs = (dv * v).sum() + (dS0 * S0).sum()
    rhs = (Wo * o).sum() + (WS * S).sum()
    assert abs(lhs - rhs) <= 1e-10 * (abs(rhs) + np.abs(Wo * o).sum())
    assert abs((dq * q).sum() - (Wo * o).sum()) <= 1e-10 * np.abs(Wo * o).sum()


def _fd(loss, args, ai, h=1e-6):
    """Central differences of loss(*args) with respect to every element of args[ai]."""
    a = args[ai]
    fd = np.zeros_like(a)
    for idx in np.ndindex(a.shape):
        a[idx] += h
        lp = loss(*args)
        a[idx] -= 2 * h
        lm = loss(*args)
        a[idx] += h
        fd[idx] = (lp - lm) / (2 * h)
    return fd


def test_prelude_backward_equals_finite_differences(orc):
    """dx and dw of the prelude (conv, SiLU, L2 norm of q and k) against
    central differences of orc.prelude: packed sequences of lengths 3, 1, 5
    (conv windows cut at sequence starts), two QK heads, d_k != d_v."""
    rng = np.random.default_rng(90)
    H_qk, H_v, dk, dv = 2, 2, 3, 2
    C = 2 * H_qk * dk + H_v * dv
    cu = np.array([0, 3, 4, 9], dtype=np.int32)
    x = rng.standard_normal((9, C))
    w = rng.standard_normal((C, 4))
    Wq, Wk = rng.standard_normal((9, H_qk, dk)), rng.standard_normal((9, H_qk, dk))
    Wv = rng.standard_normal((9, H_v, dv))

    def loss(x, w):
        q, k, v = orc.prelude(x, w, cu, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, eps=1e-3)
        return (q * Wq).sum() + (k * Wk).sum() + (v * Wv).sum()

    dx, dw = orc.prelude_backward(x, w, Wq, Wk, Wv, cu, H_qk=H_qk, H_v=H_v, eps=1e-3)
    for got, ai in ((dx, 0), (dw, 1)):
        fd = _fd(loss, [x, w], ai)
        np.testing.assert_allclose(got, fd, rtol=0, atol=1e-7 * max(1.0, np.abs(fd).max()))


def test_gates_backward_equals_finite_differences(orc):
    rng = np.random.default_rng(91)
    T, H = 5, 3
    a, b = rng.normal(0, 3, (T, H)), rng.normal(0, 3, (T, H))
    A_log, dt = rng.uniform(-1, 1, H), rng.uniform(-1, 1, H)
    Wg, Wb = rng.standard_normal((T, H)), rng.standard_normal((T, H))

    def loss(a, b, A_log, dt):
        g, beta = orc.gates(a, b, A_log, dt)
        return (g * Wg).sum() + (beta * Wb).sum()

    got = orc.gates_backward(a, b, A_log, dt, Wg, Wb)
    for ai in range(4):
        fd = _fd(loss, [a, b, A_log, dt], ai)
        np.testing.assert_allclose(got[ai], fd, rtol=0, atol=1e-7 * max(1.0, np.abs(fd).max()))


def test_layer_backward_composition_equals_finite_differences(orc):
    """The layer from raw projections (gates, prelude, recurrence): the
    gradients composed from the three backward functions against central
    differences of the composed forward, for every input including the
    initial state."""
    rng = np.random.default_rng(92)
    H_qk, H_v, d = 1, 2, 3
    C = 2 * H_qk * d + H_v * d
    cu = np.array([0, 4, 7], dtype=np.int32)
    T, N = 7, 2
    x, w = rng.standard_normal((T, C)), rng.standard_normal((C, 4))
    a, b = rng.standard_normal((T, H_v)), rng.standard_normal((T, H_v))
    A_log, dt = rng.uniform(-1, 1, H_v), rng.uniform(-1, 1, H_v)
    S0 = rng.standard_normal((N, H_v, d, d))
    Wo, WS = rng.standard_normal((T, H_v, d)), rng.standard_normal((N, H_v, d, d))

    def fwd(x, w, a, b, A_log, dt, S0):
        q, k, v = orc.prelude(x, w, cu, H_qk=H_qk, H_v=H_v, dk=d, dv=d, eps=1e-3)
        g, beta = orc.gates(a, b, A_log, dt)
        return q, k, v, g, beta

    def loss(x, w, a, b, A_log, dt, S0):
        q, k, v, g, beta = fwd(x, w, a, b, A_log, dt, S0)
        o, S = orc.recurrent(q, k, v, g, beta, S0, cu, scale=0.8)
        return (o * Wo).sum() + (S * WS).sum()

    q, k, v, g, beta = fwd(x, w, a, b, A_log, dt, S0)
    dq, dk, dv, dg, db, dS0 = orc.recurrent_backward(q, k, v, g, beta, Wo, S0, WS, cu, scale=0.8)
    dx, dw = orc.prelude_backward(x, w, dq, dk, dv, cu, H_qk=H_qk, H_v=H_v, eps=1e-3)
    da, dbr, dA, ddt = orc.gates_backward(a, b, A_log, dt, dg, db)
    args = [x, w, a, b, A_log, dt, S0]
    for got, ai in zip((dx, dw, da, dbr, dA, ddt, dS0), range(7)):
        fd = _fd(loss, args, ai)
        np.testing.assert_allclose(got, fd, rtol=0, atol=1e-7 * max(1.0, np.abs(fd).max()))


def test_gated_norm_backward_equals_finite_differences(orc):
    rng = np.random.default_rng(93)
    o, z = rng.normal(0, 2, (4, 6)), rng.normal(0, 2, (4, 6))
    w = rng.uniform(0.5, 1.5, 6)
    Wy = rng.standard_normal((4, 6))

    def loss(o, z, w):
        return (orc.gated_norm(o, z, w, eps=1e-3) * Wy).sum()

    got = orc.gated_norm_backward(o, z, w, Wy, eps=1e-3)
    for ai in range(3):
        fd = _fd(loss, [o, z, w], ai)
        np.testing.assert_allclose(got[ai], fd, rtol=0, atol=1e-7 * max(1.0, np.abs(fd).max()))


# ------------------------------------------------------------- size pins
def test_sizes_printed_on_pages():
    """The layer shape and the fp32 state dtype reproduce the state and KV-cache
    totals the pages print ([Dissect sec. 2.1, 2.2]; [Local sec. 2.1])."""
    gold = json.load(open(os.path.join(HERE, "golden", "state_sizes.json")))
    n_lin = gold["layer_counts"]["linear"]
    state_elems = synth.H_V * synth.D_V * synth.D_K           # one layer, one sequence
    fp32_MB = n_lin * state_elems * 4 / 1e6
    b16_MB = n_lin * state_elems * 2 / 1e6
    assert abs(fp32_MB - gold["gdn_state_total_fp32"]["value_MB"]) / 150 < 0.02   # 151.0 MB
    assert abs(b16_MB - gold["gdn_state_total_16bit"]["value_MB"]) / 75 < 0.02    # 75.5 MB
    fa = gold["full_attn_shape"]
    kv16 = gold["layer_counts"]["full"] * 2 * fa["kv_heads"] * fa["head_dim"] * fa["context"] * 2
    assert abs(kv16 / 2**30 - gold["full_attn_kv_16_layers"]["value_GB"]) < 0.5
    kv64 = kv16 * gold["layer_counts"]["total"] / gold["layer_counts"]["full"]
    assert abs(kv64 / 2**30 - gold["full_attn_kv_64_layers"]["value_GB"]) < 1.0


# ------------------------------------------------------ synthetic recipes
def test_synth_recipes_are_seeded_and_shaped():
    a = synth.tiny_recurrence(1001)
    b = synth.tiny_recurrence(1001)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.g, b.g)
    assert a.q.shape == (128, 1, 128) and a.v.shape == (128, 3, 128)
    assert np.all(a.g <= -0.01) and np.all(a.g >= -0.5)
    np.testing.assert_allclose(np.linalg.norm(a.k, axis=-1), 1.0, rtol=1e-6)
    L = synth.varlen_lengths(1004)
    assert len(L) == 8 and L.sum() <= 65536 and L.min() >= 512 and L.max() <= 16384
    assert np.any(L % 64 != 0)
    # ties go to the even mantissa; bf16 spacing at 1.0 is 2^-7
    x = np.array([1.0, 1.00390625, 1.01171875, 1.005], dtype=np.float32)
    assert np.array_equal(synth.bf16_value(synth.bf16_bits(x)), [1.0, 1.0, 1.015625, 1.0078125])
