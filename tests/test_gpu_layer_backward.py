"""Gradients of the layer's prefill from raw projections
(gdn_layer_prefill_backward) on the GPU: against the fp64 oracle's composition
(prelude and gates, recurrence gradients, prelude and gates gradients), and
its recurrence part bit for bit against gdn_prefill_backward on the
prelude's and gates' outputs."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu

CASES = {
    "T517": dict(T=517),
    # sequences start inside a 128-token run and inside a conv window
    "varlen": dict(lengths=[70, 3, 128, 1, 191, 64, 2]),
}


def _inputs(seed, **kw):
    p = synth.raw_prefill(seed, init_state=True, **kw)
    d_o, dSf = synth.output_grads(seed, p.T, p.N)
    A_log = p.meta["A_log"].astype(np.float32)
    dt = p.meta["dt_bias"].astype(np.float32)
    return p, d_o, dSf, A_log, dt


def _gpu(p, d_o, dSf, A_log, dt, scale=1.0):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    out = gdn.gdn_layer_prefill_backward(dev(p.x), dev(p.w), dev(p.meta["a"]), dev(p.meta["b"]),
                                         dev(A_log), dev(dt), dev(d_o), dev(p.S0), dev(dSf), cu,
                                         H_qk=p.H_qk, H_v=p.H_v, scale=scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_layer_backward_against_oracle(name):
    p, d_o, dSf, A_log, dt = _inputs(7600 + len(name), **CASES[name])
    print("layer backward", name, "T", p.T, flush=True)
    got = [host(t) for t in _gpu(p, d_o, dSf, A_log, dt, scale=0.9)]
    a, b = p.meta["a"], p.meta["b"]
    q, k, v = oracle.prelude(p.x, p.w, p.cu_seqlens, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv)
    g, beta = oracle.gates(a, b, A_log, dt)
    dq, dk, dv, dg, db, dS0 = oracle.recurrent_backward(q, k, v, g, beta, d_o, p.S0, dSf,
                                                        p.cu_seqlens, scale=0.9)
    dx, dw = oracle.prelude_backward(p.x, p.w, dq, dk, dv, p.cu_seqlens, H_qk=p.H_qk, H_v=p.H_v)
    da, dbb, dA, ddt = oracle.gates_backward(a, b, A_log, dt, dg, db)
    for nm, x, r in zip(("dx", "dconv_w", "da", "db", "dA_log", "ddt_bias", "dS0"), got,
                        (dx, dw, da, dbb, dA, ddt, dS0)):
        assert_close(x, r, TOL_BF16, nm)


def test_layer_backward_matches_its_parts():
    """Its state gradient equals gdn_prefill_backward's on gdn_conv_prelude's and
    gdn_gates' outputs, bit for bit (same kernels, same inputs)."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p, d_o, dSf, A_log, dt = _inputs(7700, T=300)
    out = _gpu(p, d_o, dSf, A_log, dt)
    q, k, v = gdn.gdn_conv_prelude(dev(p.x), dev(p.w), None, H_qk=p.H_qk, H_v=p.H_v)
    g, beta = gdn.gdn_gates(dev(p.meta["a"]), dev(p.meta["b"]), dev(A_log), dev(dt))
    ref = gdn.gdn_prefill_backward(q, k, v, g, beta, dev(d_o), dev(p.S0), dev(dSf))
    torch.cuda.synchronize()
    assert torch.equal(out[6], ref[5])


def test_layer_backward_zero_length():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p, d_o, dSf, A_log, dt = _inputs(7800, T=4)
    x = dev(p.x)[:0]
    a = dev(p.meta["a"])[:0]
    do0 = dev(d_o)[:0]
    out = gdn.gdn_layer_prefill_backward(x, dev(p.w), a, a, dev(A_log), dev(dt), do0, dev(p.S0),
                                         dev(dSf), H_qk=p.H_qk, H_v=p.H_v)
    torch.cuda.synchronize()
    assert not out[1].any() and not out[4].any() and not out[5].any()
    assert np.array_equal(out[6].cpu().numpy(), dSf)


@pytest.mark.parametrize("rows", [1, 17, 48 * 700, 48 * 4000])
def test_gated_norm_backward_against_oracle(rows):
    """The output gate's gradients on bf16 rows of 128 (48 * 4000 rows take the
    grid-stride loop several times)."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    rng = np.random.default_rng(rows + 5)
    o = synth.bf16_bits(rng.normal(0, 2, (rows, 128)).astype(np.float32))
    z = synth.bf16_bits(rng.normal(0, 2, (rows, 128)).astype(np.float32))
    dy = synth.bf16_bits(rng.normal(0, 1, (rows, 128)).astype(np.float32))
    w = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    d_o, dz, dw = gdn.gdn_gated_norm_backward(dev(o), dev(z), dev(w), dev(dy))
    torch.cuda.synchronize()
    r_o, r_z, r_w = oracle.gated_norm_backward(o, z, w, dy)
    assert_close(host(d_o), r_o, TOL_BF16, "d_o")
    assert_close(host(dz), r_z, TOL_BF16, "dz")
    assert_close(host(dw), r_w, TOL_BF16, "dw")
