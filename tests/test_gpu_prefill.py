"""Prefill on the GPU against the fp64 oracle: fp32 token path and bf16
chunked path, ragged tails, packed varlen, state hand-off, full sizes."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, TOL_F32, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _prefill(p, S0=None, scale=1.0):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    S0 = p.S0 if S0 is None else S0
    o, S = gdn.gdn_prefill(dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta),
                           None if S0 is None else dev(S0), cu, scale=scale)
    torch.cuda.synchronize()
    return host(o), S.cpu().numpy().astype(np.float64)


def test_tiny_fp32_recurrence():
    """B=1, T=128, 1 QK head / 3 V heads, fp32 io: bar 1e-4."""
    p = synth.workload_tiny()
    o, S = _prefill(p)
    o_ref, S_ref = oracle.recurrent(p.q, p.k, p.v, p.g, p.beta)
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "S")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 517])
def test_bf16_ragged_lengths(T):
    p = synth.direct_prefill(4000 + T, T=T, init_state=True)
    print("bf16 prefill T", T, flush=True)
    o, S = _prefill(p, scale=0.9)
    o_ref, S_ref = oracle.recurrent(p.q, p.k, p.v, p.g, p.beta, p.S0, scale=0.9)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "S")


def test_fp32_varlen_with_states():
    p = synth.direct_prefill(4100, lengths=[5, 64, 130, 1, 77], io="f32", init_state=True,
                             H_qk=4, H_v=12)
    o, S = _prefill(p)
    o_ref, S_ref = oracle.recurrent(p.q, p.k, p.v, p.g, p.beta, p.S0, p.cu_seqlens)
    assert_close(o, o_ref, TOL_F32, "o")
    assert_close(S, S_ref, TOL_F32, "S")


def test_bf16_varlen_mid_chunk_boundaries():
    p = synth.direct_prefill(4200, lengths=[70, 3, 128, 1, 191, 64], init_state=True)
    print("bf16 varlen", p.T, flush=True)
    o, S = _prefill(p)
    o_ref, S_ref = oracle.recurrent(p.q, p.k, p.v, p.g, p.beta, p.S0, p.cu_seqlens)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "S")
    # one sequence of the pack, run alone, gives the same result to the bar
    c = p.cu_seqlens
    sl = slice(c[2], c[3])
    q = synth.Prefill(T=c[3] - c[2], N=1, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv, io="bf16",
                      g=p.g[sl], beta=p.beta[sl], q=p.q[sl], k=p.k[sl], v=p.v[sl],
                      S0=p.S0[2:3])
    o1, S1 = _prefill(q)
    assert_close(o1, o[sl], TOL_BF16, "o alone")
    assert_close(S1[0], S[2], TOL_BF16, "S alone")


def test_bf16_split_handoff():
    """A prefill split at token s with the final state handed over equals the
    unsplit run: bit for bit at a chunk boundary (the fp32 state passes
    through memory unchanged), to the bf16 bar inside a chunk (the chunking of
    the rest moves)."""
    p = synth.direct_prefill(4300, T=700, init_state=True)
    o, S = _prefill(p)
    for s in (512, 333):
        a = synth.Prefill(T=s, N=1, H_qk=16, H_v=48, dk=128, dv=128, io="bf16", g=p.g[:s],
                          beta=p.beta[:s], q=p.q[:s], k=p.k[:s], v=p.v[:s], S0=p.S0)
        oa, Sa = _prefill(a)
        b = synth.Prefill(T=p.T - s, N=1, H_qk=16, H_v=48, dk=128, dv=128, io="bf16",
                          g=p.g[s:], beta=p.beta[s:], q=p.q[s:], k=p.k[s:], v=p.v[s:],
                          S0=Sa.astype(np.float32))
        ob, Sb = _prefill(b)
        assert_close(np.concatenate([oa, ob]), o, TOL_BF16, f"o split at {s}")
        assert_close(Sb, S, TOL_BF16, f"S split at {s}")
        if s % 64 == 0:
            assert np.array_equal(np.concatenate([oa, ob]), o) and np.array_equal(Sb, S)


def test_bf16_deterministic_and_inplace_state():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.direct_prefill(4400, T=300, init_state=True)
    o1, S1 = _prefill(p)
    o2, S2 = _prefill(p)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    st = dev(p.S0)
    o3, S3 = gdn.gdn_prefill(dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), st,
                             final_state=st)
    torch.cuda.synchronize()
    assert S3 is st
    assert np.array_equal(host(o3), o1) and np.array_equal(st.cpu().numpy(), S1.astype(np.float32))


def test_prefill_equals_decode_steps():
    """T decode steps from the same start state reproduce the prefill."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.direct_prefill(4500, T=70, init_state=True)
    o, S = _prefill(p)
    pool = dev(p.S0)
    slot = dev(np.zeros(1, dtype=np.int32))
    outs = []
    for t in range(p.T):
        ot = gdn.gdn_decode_step(dev(p.q[t:t + 1]), dev(p.k[t:t + 1]), dev(p.v[t:t + 1]),
                                 dev(p.g[t:t + 1]), dev(p.beta[t:t + 1]), pool, slot)
        outs.append(host(ot))
    torch.cuda.synchronize()
    assert_close(np.concatenate(outs), o, TOL_BF16, "o")
    assert_close(pool.cpu().numpy(), S, TOL_BF16, "S")


def test_bf16_long_sequence_segments():
    """One sequence of 65 chunks (ragged tail) is prepared and scanned in
    segments, the prep of each segment overlapping the scan of the one before.
    Checked against the oracle on every head and token; bit-identical to the
    same sequence run as chained calls split at chunk boundaries (each too
    short to be segmented: the state hand-off at a chunk boundary is exact),
    with no final state asked for, and with the state updated in place."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    nch = 65
    p = synth.direct_prefill(4600, T=64 * (nch - 1) + 37, init_state=True)
    print("segmented prefill T", p.T, flush=True)
    o, S = _prefill(p)
    o_ref, S_ref = oracle.recurrent(p.q, p.k, p.v, p.g, p.beta, p.S0)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "S")

    bounds = [0, 64 * 20, 64 * 41, 64 * 50, p.T]   # chunk-aligned, unlike the segments
    St, outs = p.S0, []
    for a, b in zip(bounds[:-1], bounds[1:]):
        part = synth.Prefill(T=b - a, N=1, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv, io="bf16",
                             g=p.g[a:b], beta=p.beta[a:b], q=p.q[a:b], k=p.k[a:b], v=p.v[a:b],
                             S0=St)
        oi, Si = _prefill(part)
        outs.append(oi)
        St = Si.astype(np.float32)
    assert np.array_equal(np.concatenate(outs), o)
    assert np.array_equal(St, S.astype(np.float32))

    args = (dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta))
    o2, none = gdn.gdn_prefill(*args, dev(p.S0), final_state=None)
    st = dev(p.S0)
    o3, S3 = gdn.gdn_prefill(*args, st, final_state=st)
    torch.cuda.synchronize()
    assert none is None and S3 is st
    assert np.array_equal(host(o2), o) and np.array_equal(host(o3), o)
    assert np.array_equal(st.cpu().numpy(), S.astype(np.float32))


def _all_heads_end_to_end(p, what):
    """The raw-projection workload through prelude + prefill on the GPU, as two
    calls and fused in one, each into outputs pre-filled with NaN (a unit the
    kernels never write fails the finiteness check).  The oracle runs the
    prelude and the recurrence once, for every head; every V-head's outputs at
    every token and every sequence's final state are compared with it, and the
    two GPU paths must agree bit for bit."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    S0 = None if p.S0 is None else dev(p.S0)
    xd = dev(p.x)
    nan_o = lambda: torch.full((p.T, p.H_v, p.dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    nan_s = lambda: torch.full((p.N, p.H_v, p.dv, p.dk), float("nan"), dtype=torch.float32, device="cuda")
    q, k, v = gdn.gdn_conv_prelude(xd, dev(p.w), cu, H_qk=p.H_qk, H_v=p.H_v)
    o2, S2 = gdn.gdn_prefill(q, k, v, dev(p.g), dev(p.beta), S0, cu, o=nan_o(), final_state=nan_s())
    del q, k, v
    of, Sf = gdn.gdn_prefill_raw(xd, dev(p.w), dev(p.g), dev(p.beta), S0, cu, H_qk=p.H_qk,
                                 H_v=p.H_v, o=nan_o(), final_state=nan_s())
    torch.cuda.synchronize()
    del xd
    assert torch.equal(of, o2) and torch.equal(Sf, S2), f"{what}: fused and two-call paths differ"
    o, S = host(o2), S2.cpu().numpy().astype(np.float64)
    del o2, S2, of, Sf
    print(what, "GPU done", flush=True)
    qr, kr, vr = oracle.prelude(p.x, p.w, p.cu_seqlens, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv)
    o_ref, S_ref = oracle.recurrent(qr, kr, vr, p.g, p.beta, p.S0, p.cu_seqlens)
    del qr, kr, vr
    print(what, "oracle done", flush=True)
    for h in range(p.H_v):
        assert_close(o[:, h], o_ref[:, h], TOL_BF16, f"{what} o head {h}")
        assert_close(S[:, h], S_ref[:, h], TOL_BF16, f"{what} S head {h}")


def test_prefill_32k_all_heads():
    """B=1, T=32768 from raw projections (prelude + chunked prefill): every
    V-head at every token against the oracle, two-call and fused paths."""
    _all_heads_end_to_end(synth.workload_prefill_32k(), "T32768")


def test_prefill_varlen_8seq_all_heads():
    """8 packed sequences (lengths U{512..16384}) with nonzero initial states:
    every V-head, every token, every sequence's final state; two-call and
    fused paths."""
    _all_heads_end_to_end(synth.workload_varlen(), "varlen")


def _special(T, g, beta, q, k, v, S0, H_qk=16, H_v=48):
    return synth.Prefill(T=T, N=1, H_qk=H_qk, H_v=H_v, dk=128, dv=128, io="bf16",
                         g=np.ascontiguousarray(g, dtype=np.float32),
                         beta=np.ascontiguousarray(beta, dtype=np.float32),
                         q=q, k=k, v=v, S0=S0)


@pytest.mark.parametrize("T", [517, 4133])
def test_chunked_no_write_no_decay_keeps_state(T):
    """beta = 0 and g = 0 (no erase, no write, no decay): the state never
    changes, so the final state is the initial state bit for bit and o_t = S_0 q_t
    ("从参数竞赛到效率革命：拆解 Qwen3.8-27B ...", sec. 2.2: the update with
    strength 0 leaves the state as it is).  T = 4133 runs in segments."""
    p = synth.direct_prefill(4700 + T, T=T, init_state=True)
    z = np.zeros((T, p.H_v), dtype=np.float32)
    s = _special(T, z, z, p.q, p.k, p.v, p.S0)
    o, S = _prefill(s)
    assert np.array_equal(S.astype(np.float32), p.S0), "state changed"
    o_ref, S_ref = oracle.recurrent(s.q, s.k, s.v, s.g, s.beta, s.S0)
    grp = s.H_v // s.H_qk
    qf = synth.bf16_value(s.q).astype(np.float64)
    o_closed = np.einsum("hij,thj->thi", s.S0[0].astype(np.float64), np.repeat(qf, grp, axis=1))
    assert_close(o_ref, o_closed, 1e-12, "oracle o = S0 q")
    assert_close(o, o_closed, TOL_BF16, "o = S0 q")


def _unit_bf16_keys(rng, T, H):
    """Rows with +-1/8 on 64 random coordinates: exactly unit length in bf16."""
    k = np.zeros((T, H, 128), dtype=np.float32)
    for t in range(T):
        for h in range(H):
            idx = rng.choice(128, 64, replace=False)
            k[t, h, idx] = rng.choice([-0.125, 0.125], 64)
    return synth.bf16_bits(k)


@pytest.mark.parametrize("T", [130, 4133])
def test_chunked_full_write_unit_keys_retrieves_value(T):
    """beta = 1 with exactly unit keys: after token t the state maps k_t to v_t
    whatever the decay (erase-then-write, sec. 2.2 of the page above), so with
    q = k every output equals its token's value: o_t = S_t k_t = v_t."""
    rng = np.random.default_rng(4800 + T)
    p = synth.direct_prefill(4800 + T, T=T, init_state=True)
    k = _unit_bf16_keys(rng, T, p.H_qk)
    one = np.ones((T, p.H_v), dtype=np.float32)
    s = _special(T, p.g, one, k, k, p.v, p.S0)
    o, _ = _prefill(s)
    vf = synth.bf16_value(s.v).astype(np.float64)
    o_ref, _ = oracle.recurrent(s.q, s.k, s.v, s.g, s.beta, s.S0)
    assert_close(o_ref, vf, 1e-12, "oracle o = v")
    assert_close(o, vf, TOL_BF16, "o = v")


def test_chunked_orthonormal_keys_exact():
    """Keys k_t = e_t (orthonormal), q = k, beta = 1, g = 0, zero initial state:
    the state after T <= 128 tokens holds v_t in column t and o_t = v_t.  Every
    product then adds exact zeros and ones, so the bf16 chunked path must give
    both bit for bit."""
    T = 128
    p = synth.direct_prefill(4900, T=T)
    e = np.zeros((T, p.H_qk, 128), dtype=np.float32)
    e[np.arange(T), :, np.arange(T)] = 1.0
    k = synth.bf16_bits(e)
    s = _special(T, np.zeros((T, p.H_v)), np.ones((T, p.H_v)), k, k, p.v, None)
    o, S = _prefill(s)
    vf = synth.bf16_value(s.v).astype(np.float64)            # [T, H_v, 128]
    assert np.array_equal(o, vf), "o != v"
    assert np.array_equal(S[0], np.transpose(vf, (1, 2, 0))), "state columns != v"


def test_nan_workspace_does_not_leak():
    """The workspace's contents on entry are ignored: a workspace filled with
    NaN gives the same bits as a zeroed one (one segmented sequence and a
    packed batch, two-call and fused paths)."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    for p in (synth.raw_prefill(5000, T=4133, init_state=True),
              synth.raw_prefill(5001, lengths=[700, 3, 1500, 64], init_state=True)):
        cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
        xd, wd, gd, bd, S0 = dev(p.x), dev(p.w), dev(p.g), dev(p.beta), dev(p.S0)
        q, k, v = gdn.gdn_conv_prelude(xd, wd, cu, H_qk=p.H_qk, H_v=p.H_v)
        outs = []
        for fill in (0, 0xFF):
            n1 = gdn.gdn_prefill_workspace_size(gdn.GDN_BF16, p.N, p.T, p.H_qk, p.H_v)
            n2 = gdn.gdn_prefill_raw_workspace_size(p.N, p.T, p.H_qk, p.H_v)
            w1 = torch.full((n1,), fill, dtype=torch.uint8, device="cuda")
            w2 = torch.full((n2,), fill, dtype=torch.uint8, device="cuda")
            outs.append(gdn.gdn_prefill(q, k, v, gd, bd, S0, cu, workspace=w1) +
                        gdn.gdn_prefill_raw(xd, wd, gd, bd, S0, cu, H_qk=p.H_qk, H_v=p.H_v,
                                            workspace=w2))
        torch.cuda.synchronize()
        for a, b in zip(*outs):
            assert torch.equal(a, b)
