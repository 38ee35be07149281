"""The layer's forward from raw projections on the GPU: gates from a, b
(gdn_gates), the whole prefill (gdn_layer_prefill) with its conv history out,
and the decode step with a rolling conv state (gdn_layer_decode_step).  Each
is checked bit for bit against the separate calls it is made of, and against
the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, TOL_F32, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _bits(t):
    """Raw bit patterns (so NaN canaries compare equal to themselves)."""
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _weights(p):
    return p.meta["A_log"].astype(np.float32), p.meta["dt_bias"].astype(np.float32)


def test_gates_against_oracle():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    rng = np.random.default_rng(7)
    T, H = 1000, 48
    a = rng.normal(0, 3, (T, H)).astype(np.float32)
    b = rng.normal(0, 3, (T, H)).astype(np.float32)
    A_log = rng.uniform(-1, 1, H).astype(np.float32)
    dt = rng.uniform(-1, 1, H).astype(np.float32)
    g, beta = gdn.gdn_gates(dev(a), dev(b), dev(A_log), dev(dt))
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gates(a, b, A_log, dt)
    assert_close(host(g), g_ref, TOL_F32, "g")
    assert_close(host(beta), b_ref, TOL_F32, "beta")


CASES = {
    "T517": dict(T=517),
    "varlen": dict(lengths=[70, 3, 128, 1, 191, 64, 2]),
    "segmented": dict(T=64 * 64 + 37),
}


def _layer_prefill(p, **kw):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    A_log, dt = _weights(p)
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    S0 = None if p.S0 is None else dev(p.S0)
    out = gdn.gdn_layer_prefill(dev(p.x), dev(p.w), dev(p.meta["a"]), dev(p.meta["b"]),
                                dev(A_log), dev(dt), S0, cu, H_qk=p.H_qk, H_v=p.H_v, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_layer_prefill_bit_identical_to_its_parts(name):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.raw_prefill(5600 + len(name), init_state=True, **CASES[name])
    print("layer prefill", name, "T", p.T, flush=True)
    o, S, cs = _layer_prefill(p)
    A_log, dt = _weights(p)
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    g, beta = gdn.gdn_gates(dev(p.meta["a"]), dev(p.meta["b"]), dev(A_log), dev(dt))
    o2, S2 = gdn.gdn_prefill_raw(dev(p.x), dev(p.w), g, beta, dev(p.S0), cu, H_qk=p.H_qk,
                                 H_v=p.H_v)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(o), _bits(o2)) and np.array_equal(_bits(S), _bits(S2))
    assert np.array_equal(_bits(cs), oracle.conv_state(p.x, p.cu_seqlens).view(np.int16))


@pytest.mark.parametrize("name", ["T517", "varlen"])
def test_layer_prefill_against_oracle(name):
    p = synth.raw_prefill(5700 + len(name), init_state=True, **CASES[name])
    o, S, _ = _layer_prefill(p)
    A_log, dt = _weights(p)
    q, k, v = oracle.prelude(p.x, p.w, p.cu_seqlens, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv)
    g, beta = oracle.gates(p.meta["a"], p.meta["b"], A_log, dt)
    o_ref, S_ref = oracle.recurrent(q, k, v, g, beta, p.S0, p.cu_seqlens)
    assert_close(host(o), o_ref, TOL_BF16, "o")
    assert_close(S.cpu().numpy(), S_ref, TOL_BF16, "S")


def test_layer_decode_bit_identical_to_its_parts():
    """gdn_layer_decode_step against gdn_conv_prelude on each slot's 4-row
    window, gdn_gates and gdn_decode_step; the conv pool shifted in place and
    the slots not addressed untouched."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    d = synth.layer_decode_inputs(5800, B=40, P=64)
    cpool, pool = dev(d.conv_pool), dev(d.pool)
    o = gdn.gdn_layer_decode_step(dev(d.x), dev(d.w), dev(d.a), dev(d.b), dev(d.A_log),
                                  dev(d.dt_bias), cpool, pool, dev(d.slot_idx))
    torch.cuda.synchronize()
    C = d.x.shape[1]
    win = np.concatenate([d.conv_pool[d.slot_idx], d.x[:, None, :]], axis=1).reshape(4 * d.B, C)
    cu = dev(np.arange(0, 4 * d.B + 1, 4, dtype=np.int32))
    q, k, v = gdn.gdn_conv_prelude(dev(win), dev(d.w), cu)
    g, beta = gdn.gdn_gates(dev(d.a), dev(d.b), dev(d.A_log), dev(d.dt_bias))
    pool2 = dev(d.pool)
    o2 = gdn.gdn_decode_step(q[3::4].contiguous(), k[3::4].contiguous(), v[3::4].contiguous(), g,
                             beta, pool2, dev(d.slot_idx))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(o), _bits(o2))
    assert np.array_equal(_bits(pool), _bits(pool2))
    cp = _bits(cpool)
    shifted = np.concatenate([d.conv_pool[d.slot_idx][:, 1:], d.x[:, None, :]], axis=1)
    assert np.array_equal(cp[d.slot_idx], shifted.view(np.int16))
    rest = np.setdiff1d(np.arange(d.P), d.slot_idx)
    assert (cp[rest].view(np.uint16) == synth.CONV_CANARY_BITS).all()
    assert (pool.cpu().numpy()[rest].view(np.uint32) == synth.CANARY_BITS).all()


def test_layer_decode_against_oracle():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    d = synth.layer_decode_inputs(5900, B=64, P=128)
    cpool, pool = dev(d.conv_pool), dev(d.pool)
    o = gdn.gdn_layer_decode_step(dev(d.x), dev(d.w), dev(d.a), dev(d.b), dev(d.A_log),
                                  dev(d.dt_bias), cpool, pool, dev(d.slot_idx))
    torch.cuda.synchronize()
    o_ref, _, pool_ref = oracle.decode_step_raw(d.x, d.w, d.conv_pool, d.a, d.b, d.A_log,
                                                d.dt_bias, d.pool, d.slot_idx, H_qk=d.H_qk,
                                                H_v=d.H_v, dk=d.dk, dv=d.dv)
    assert_close(host(o), o_ref, TOL_BF16, "o")
    assert_close(pool.cpu().numpy()[d.slot_idx], pool_ref[d.slot_idx], TOL_BF16, "states")


def test_layer_prefill_then_decode_chain_against_oracle():
    """Two packed sequences prefilled from raw projections, their final states
    and conv histories moved into pool slots, then 6 decode steps of new raw
    rows: every decode output and the final states against one oracle run of
    prelude + gates + recurrence over the longer sequences."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    lens, D = [150, 2], 6
    full = synth.raw_prefill(6000, lengths=[l + D for l in lens], init_state=True)
    H_qk, H_v, C = full.H_qk, full.H_v, full.x.shape[1]
    A_log, dt = _weights(full)
    starts = np.concatenate([[0], np.cumsum([l + D for l in lens])])
    pre = np.concatenate([np.arange(s, s + l) for s, l in zip(starts, lens)])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    a, b = full.meta["a"], full.meta["b"]
    o, S, cs = gdn.gdn_layer_prefill(dev(full.x[pre]), dev(full.w), dev(a[pre]), dev(b[pre]),
                                     dev(A_log), dev(dt), dev(full.S0), dev(cu), H_qk=H_qk, H_v=H_v)
    slots = np.array([3, 1], dtype=np.int32)
    P = 4
    pool = torch.zeros((P, H_v, 128, 128), dtype=torch.float32, device="cuda")
    cpool = torch.zeros((P, 3, C), dtype=torch.bfloat16, device="cuda")
    pool[dev(slots).long()] = S
    cpool[dev(slots).long()] = cs
    outs = []
    for t in range(D):
        rows = starts[:-1] + np.array(lens) + t
        outs.append(host(gdn.gdn_layer_decode_step(dev(full.x[rows]), dev(full.w), dev(a[rows]),
                                                   dev(b[rows]), dev(A_log), dev(dt), cpool, pool,
                                                   dev(slots), H_qk=H_qk, H_v=H_v)))
    torch.cuda.synchronize()
    q, k, v = oracle.prelude(full.x, full.w, full.cu_seqlens, H_qk=H_qk, H_v=H_v, dk=128, dv=128)
    g, beta = oracle.gates(a, b, A_log, dt)
    o_ref, S_ref = oracle.recurrent(q, k, v, g, beta, full.S0, full.cu_seqlens)
    assert_close(host(o), o_ref[pre], TOL_BF16, "prefill o")
    dec_rows = np.stack([starts[:-1] + np.array(lens) + t for t in range(D)])     # [D, 2]
    assert_close(np.stack(outs), o_ref[dec_rows], TOL_BF16, "decode o")
    assert_close(pool.cpu().numpy()[slots], S_ref, TOL_BF16, "final states")


@pytest.mark.parametrize("rows", [1, 17, 48 * 700])
def test_gated_norm_against_oracle(rows):
    """The output gate on bf16 rows of 128 (in place and out of place)."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    rng = np.random.default_rng(rows)
    o = synth.bf16_bits(rng.normal(0, 2, (rows, 128)).astype(np.float32))
    z = synth.bf16_bits(rng.normal(0, 2, (rows, 128)).astype(np.float32))
    w = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    y = gdn.gdn_gated_norm(dev(o), dev(z), dev(w))
    od = dev(o)
    gdn.gdn_gated_norm(od, dev(z), dev(w), out=od)
    torch.cuda.synchronize()
    ref = oracle.gated_norm(o, z, w)
    assert_close(host(y), ref, TOL_BF16, "y")
    assert np.array_equal(_bits(od), _bits(y))
