"""Gradients of the bf16 chunked prefill (gdn_prefill_backward) on the GPU
against the fp64 oracle's reverse-mode gradients of the token recurrence:
ragged lengths, packed varlen, initial state and final-state gradient present
or not, an odd head grid, T = 0, and the 32768-token and packed 8-sequence
workloads (four QK groups against the oracle element by element, every head
through the adjoint identities)."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def _gpu_backward(p, d_o, dSf, scale):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    out = gdn.gdn_prefill_backward(dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), dev(d_o),
                                   None if p.S0 is None else dev(p.S0),
                                   None if dSf is None else dev(dSf), cu, scale=scale)
    torch.cuda.synchronize()
    return [host(t) for t in out]


def _check(p, d_o, dSf, scale, qk_heads=None):
    got = _gpu_backward(p, d_o, dSf, scale)
    ref = oracle.recurrent_backward(p.q, p.k, p.v, p.g, p.beta, d_o, p.S0, dSf, p.cu_seqlens,
                                    scale=scale, qk_heads=qk_heads)
    if qk_heads is not None:
        lo, hi = qk_heads
        grp = p.H_v // p.H_qk
        sel_qk = slice(lo, hi)
        sel_v = slice(lo * grp, hi * grp)
        got = [got[0][:, sel_qk], got[1][:, sel_qk], got[2][:, sel_v], got[3][:, sel_v],
               got[4][:, sel_v], got[5][:, sel_v]]
        ref = [ref[0][:, sel_qk], ref[1][:, sel_qk], ref[2][:, sel_v], ref[3][:, sel_v],
               ref[4][:, sel_v], ref[5][:, sel_v]]
    for name, x, r in zip(NAMES, got, ref):
        assert_close(x, r, TOL_BF16, name)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 300])
def test_backward_ragged_lengths(T):
    p = synth.direct_prefill(7000 + T, T=T, init_state=True)
    d_o, dSf = synth.output_grads(7000 + T, T, 1)
    print("backward T", T, flush=True)
    _check(p, d_o, dSf, 0.9)


def test_backward_varlen():
    """Sequences that start mid-chunk, lengths 1..191, each with its own state."""
    p = synth.direct_prefill(7100, lengths=[70, 3, 128, 1, 191, 64, 2], init_state=True)
    d_o, dSf = synth.output_grads(7100, p.T, p.N)
    _check(p, d_o, dSf, 1.0)


def test_backward_no_state_no_final_gradient():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.direct_prefill(7200, T=200)
    d_o, _ = synth.output_grads(7200, p.T, 1)
    _check(p, d_o, None, 1.0)
    # skipping the initial-state gradient changes nothing else
    a = gdn.gdn_prefill_backward(dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), dev(d_o))
    b = gdn.gdn_prefill_backward(dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), dev(d_o),
                                 d_initial_state=None)
    torch.cuda.synchronize()
    assert b[5] is None
    for x, y in zip(a[:5], b[:5]):
        assert torch.equal(x, y)


def test_backward_odd_head_grid():
    """1 QK head, 3 V-heads: a reverse-scan grid of 12 workgroups."""
    p = synth.direct_prefill(7300, T=300, H_qk=1, H_v=3, init_state=True)
    d_o, dSf = synth.output_grads(7300, p.T, 1, H_v=3)
    _check(p, d_o, dSf, 1.0)


def test_backward_zero_length():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.direct_prefill(7400, T=4, init_state=True)
    _, dSf = synth.output_grads(7400, 4, 1)
    q = dev(p.q)[:0]
    v = dev(p.v)[:0]
    g = dev(p.g)[:0]
    out = gdn.gdn_prefill_backward(q, q, v, g, g, v, dev(p.S0), dev(dSf))
    torch.cuda.synchronize()
    assert np.array_equal(out[5].cpu().numpy(), dSf)
    out = gdn.gdn_prefill_backward(q, q, v, g, g, v)
    torch.cuda.synchronize()
    assert not out[5].any()


def test_backward_full_size_one_group_and_adjoint():
    """The 32768-token workload (16 QK / 48 V heads, initial state, final-state
    gradient): QK heads 6-9 and their twelve V-heads (workgroup placements on
    four different XCDs) against the oracle element by element; every head
    through <dv, v> + <dS0, S0> = <d_o, o> + <dS_T, S_T> and <dq, q> = <d_o, o>,
    which hold because (o, S_T) is linear in (v, S0) and o is linear in q."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    T = 32768
    p = synth.direct_prefill(7500, T=T, init_state=True)
    d_o, dSf = synth.output_grads(7500, T, 1)
    print("backward T", T, flush=True)
    _check(p, d_o, dSf, 1.0, qk_heads=(6, 10))
    dq, dk, dv, dg, db, dS0 = gdn.gdn_prefill_backward(dev(p.q), dev(p.k), dev(p.v), dev(p.g),
                                                       dev(p.beta), dev(d_o), dev(p.S0), dev(dSf))
    o, S = gdn.gdn_prefill(dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), dev(p.S0))
    f64 = lambda t: t.double()
    lhs = (f64(dv) * f64(dev(p.v))).sum() + (f64(dS0) * f64(dev(p.S0))).sum()
    rhs = (f64(dev(d_o)) * f64(o)).sum() + (f64(dev(dSf)) * f64(S)).sum()
    scale = (f64(dev(d_o)) * f64(o)).abs().sum()
    assert abs(float(lhs - rhs)) <= 2e-2 * float(scale), (float(lhs), float(rhs), float(scale))
    qq = (f64(dq) * f64(dev(p.q))).sum()
    oo = (f64(dev(d_o)) * f64(o)).sum()
    assert abs(float(qq - oo)) <= 2e-2 * float(scale), (float(qq), float(oo))
    for t in (dq, dk, dv, dg, db, dS0):
        assert torch.isfinite(t.float()).all()


def test_backward_varlen_8seq_one_group_and_adjoint():
    """The packed varlen workload (8 sequences, lengths U{512..16384}, each
    with its own initial state and final-state gradient): QK heads 10-13 and
    their V-heads against the oracle, every head through the adjoint identities of
    the test above (summed over the sequences)."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    lengths = synth.varlen_lengths(1004)
    p = synth.direct_prefill(7600, lengths=lengths, init_state=True)
    d_o, dSf = synth.output_grads(7600, p.T, p.N)
    print("backward varlen", list(lengths), flush=True)
    _check(p, d_o, dSf, 1.0, qk_heads=(10, 14))
    cu = dev(p.cu_seqlens)
    dq, dk, dv, dg, db, dS0 = gdn.gdn_prefill_backward(dev(p.q), dev(p.k), dev(p.v), dev(p.g),
                                                       dev(p.beta), dev(d_o), dev(p.S0), dev(dSf), cu)
    o, S = gdn.gdn_prefill(dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), dev(p.S0), cu)
    f64 = lambda t: t.double()
    lhs = (f64(dv) * f64(dev(p.v))).sum() + (f64(dS0) * f64(dev(p.S0))).sum()
    rhs = (f64(dev(d_o)) * f64(o)).sum() + (f64(dev(dSf)) * f64(S)).sum()
    scale = (f64(dev(d_o)) * f64(o)).abs().sum()
    assert abs(float(lhs - rhs)) <= 2e-2 * float(scale), (float(lhs), float(rhs), float(scale))
    qq = (f64(dq) * f64(dev(p.q))).sum()
    oo = (f64(dev(d_o)) * f64(o)).sum()
    assert abs(float(qq - oo)) <= 2e-2 * float(scale), (float(qq), float(oo))
    for t in (dq, dk, dv, dg, db, dS0):
        assert torch.isfinite(t.float()).all()
