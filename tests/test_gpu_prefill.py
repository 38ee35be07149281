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


def _sampled_heads_end_to_end(p, heads, what, fused=False):
    """prelude + prefill on the GPU (two calls, or fused in one); the oracle runs
    prelude + recurrence for the sampled V-heads only (their QK head's channels
    and their own v channels)."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    xd = dev(p.x)
    S0 = None if p.S0 is None else dev(p.S0)
    if fused:
        o, S = gdn.gdn_prefill_raw(xd, dev(p.w), dev(p.g), dev(p.beta), S0, cu, H_qk=p.H_qk,
                                   H_v=p.H_v)
        del xd
    else:
        q, k, v = gdn.gdn_conv_prelude(xd, dev(p.w), cu, H_qk=p.H_qk, H_v=p.H_v)
        del xd
        o, S = gdn.gdn_prefill(q, k, v, dev(p.g), dev(p.beta), S0, cu)
    torch.cuda.synchronize()
    grp = p.H_v // p.H_qk
    D = p.dk
    for h in heads:
        hq = h // grp
        chans = np.concatenate([np.arange(hq * D, (hq + 1) * D),
                                np.arange((p.H_qk + hq) * D, (p.H_qk + hq + 1) * D),
                                np.arange((2 * p.H_qk + h) * D, (2 * p.H_qk + h + 1) * D)])
        qr, kr, vr = oracle.prelude(p.x[:, chans], p.w[chans], p.cu_seqlens, H_qk=1, H_v=1,
                                    dk=D, dv=D)
        S0 = None if p.S0 is None else p.S0[:, h:h + 1]
        o_ref, S_ref = oracle.recurrent(qr, kr, vr, p.g[:, h:h + 1], p.beta[:, h:h + 1], S0,
                                        p.cu_seqlens)
        print(what, "head", h, flush=True)
        assert_close(host(o[:, h]), o_ref[:, 0], TOL_BF16, f"{what} o head {h}")
        assert_close(S[:, h].cpu().numpy(), S_ref[:, 0], TOL_BF16, f"{what} S head {h}")


def test_prefill_32k_sampled_heads():
    """B=1, T=32768 from raw projections: prelude + chunked prefill, V-heads
    sampled across QK groups, every token of those heads."""
    p = synth.workload_prefill_32k()
    _sampled_heads_end_to_end(p, [0, 25, 47], "T32768")


def test_prefill_varlen_8seq_sampled_heads():
    """8 packed sequences (lengths U{512..16384}), nonzero initial states."""
    p = synth.workload_varlen()
    _sampled_heads_end_to_end(p, [4, 38], "varlen")


def test_prefill_raw_32k_sampled_heads():
    """The 32768-token workload through the fused prelude + prefill."""
    p = synth.workload_prefill_32k()
    _sampled_heads_end_to_end(p, [2, 30, 46], "T32768 fused", fused=True)


def test_prefill_raw_varlen_8seq_sampled_heads():
    """The packed varlen workload through the fused prelude + prefill."""
    p = synth.workload_varlen()
    _sampled_heads_end_to_end(p, [7, 41], "varlen fused", fused=True)
