"""The conv prelude fused into the chunked prefill (gdn_prefill_raw): bit for bit
equal to gdn_conv_prelude followed by gdn_prefill (the fused kernels apply the
prelude's arithmetic in the prelude's order), and within the bf16 bar of the
fp64 oracle (prelude + token recurrence)."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _fused_and_unfused(p, final_state=True):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    x, w, g, b = dev(p.x), dev(p.w), dev(p.g), dev(p.beta)
    S0 = None if p.S0 is None else dev(p.S0)
    q, k, v = gdn.gdn_conv_prelude(x, w, cu, H_qk=p.H_qk, H_v=p.H_v)
    o1, S1 = gdn.gdn_prefill(q, k, v, g, b, S0, cu)
    o2, S2 = gdn.gdn_prefill_raw(x, w, g, b, S0, cu, H_qk=p.H_qk, H_v=p.H_v,
                                 final_state=final_state)
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16).cpu().numpy()
    return (bits(o1), S1.cpu().numpy(), bits(o2), None if S2 is None else S2.cpu().numpy(),
            host(o2))


CASES = {
    "T1": dict(T=1),
    "T3": dict(T=3),
    "T63": dict(T=63),
    "T64": dict(T=64),
    "T65": dict(T=65),
    "T517": dict(T=517),
    # sequence starts mid-chunk and inside a conv window (lengths 1, 2, 3 < 4)
    "varlen": dict(lengths=[70, 3, 128, 1, 191, 64, 2]),
    # long enough to be split into segments with prep on the idle CUs
    "segmented": dict(T=64 * 64 + 37),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_bit_identical_to_prelude_then_prefill(name):
    p = synth.raw_prefill(5100 + len(name) * 7 + sum(map(ord, name)), init_state=True,
                          **CASES[name])
    print("fused prefill", name, "T", p.T, flush=True)
    o1, S1, o2, S2, _ = _fused_and_unfused(p)
    assert np.array_equal(o1, o2), "o differs"
    assert np.array_equal(S1, S2), "final state differs"


@pytest.mark.parametrize("name", ["T517", "varlen"])
def test_fused_against_oracle(name):
    p = synth.raw_prefill(5200 + len(name), init_state=True, **CASES[name])
    _, _, _, S, o = _fused_and_unfused(p)
    q, k, v = oracle.prelude(p.x, p.w, p.cu_seqlens, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv)
    o_ref, S_ref = oracle.recurrent(q, k, v, p.g, p.beta, p.S0, p.cu_seqlens)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S, S_ref, TOL_BF16, "S")


def test_fused_no_final_state_and_in_place():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.raw_prefill(5300, T=64 * 64 + 37, init_state=True)
    o1, S1, _, _, _ = _fused_and_unfused(p)
    x, w, g, b = dev(p.x), dev(p.w), dev(p.g), dev(p.beta)
    o2, none = gdn.gdn_prefill_raw(x, w, g, b, dev(p.S0), final_state=None)
    st = dev(p.S0)
    o3, S3 = gdn.gdn_prefill_raw(x, w, g, b, st, final_state=st)
    torch.cuda.synchronize()
    assert none is None and S3 is st
    bits = lambda t: t.view(torch.int16).cpu().numpy()
    assert np.array_equal(bits(o2), o1) and np.array_equal(bits(o3), o1)
    assert np.array_equal(st.cpu().numpy(), S1)


def test_odd_head_count_grid():
    """1 QK head, 3 V-heads: a scan grid (12 workgroups) that is not a multiple
    of the 8 XCDs; every (head, slab) must be computed exactly once."""
    p = synth.raw_prefill(5400, T=300, H_qk=1, H_v=3, init_state=True)
    o1, S1, o2, S2, o = _fused_and_unfused(p)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    q, k, v = oracle.prelude(p.x, p.w, None, H_qk=1, H_v=3, dk=p.dk, dv=p.dv)
    o_ref, S_ref = oracle.recurrent(q, k, v, p.g, p.beta, p.S0)
    assert_close(o, o_ref, TOL_BF16, "o")
    assert_close(S2, S_ref, TOL_BF16, "S")


def test_zero_length():
    """T = 0: no workspace; the final state is the initial state."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.raw_prefill(5500, T=8, init_state=True)
    x = dev(p.x)[:0]
    g = dev(p.g)[:0]
    b = dev(p.beta)[:0]
    o, S = gdn.gdn_prefill_raw(x, dev(p.w), g, b, dev(p.S0))
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and np.array_equal(S.cpu().numpy(), p.S0)
    q = torch.empty((0, 16, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((0, 48, 128), dtype=torch.bfloat16, device="cuda")
    o, S = gdn.gdn_prefill(q, q, v, g, b, dev(p.S0))
    torch.cuda.synchronize()
    assert np.array_equal(S.cpu().numpy(), p.S0)
