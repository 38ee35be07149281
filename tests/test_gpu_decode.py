"""Decode step on the GPU against the fp64 oracle (slot pool, in-place update)."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _run(d, scale=1.0):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    pool = dev(d.pool)
    o = gdn.gdn_decode_step(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), pool,
                            dev(d.slot_idx), scale=scale)
    torch.cuda.synchronize()
    return host(o), pool.cpu().numpy()


def _check(d, o, pool, scale=1.0):
    o_ref, pool_ref = oracle.decode_step(d.q, d.k, d.v, d.g, d.beta, d.pool, d.slot_idx, scale)
    assert_close(o, o_ref, TOL_BF16, "o")
    slots = d.slot_idx
    assert_close(pool[slots], pool_ref[slots], TOL_BF16, "state")
    untouched = np.setdiff1d(np.arange(d.P), slots)
    # slots not addressed keep their NaN canary bit for bit
    assert (pool[untouched].view(np.uint32) == d.pool[untouched].view(np.uint32)).all()


def test_decode_b64_pool128():
    """One decode step, B=64 sequences, 16 QK / 48 V heads, pool of 128 slots."""
    d = synth.workload_decode_b64()
    print("decode B=64 P=128 seed", d.meta["seed"], flush=True)
    o, pool = _run(d)
    _check(d, o, pool)


@pytest.mark.parametrize("B,P", [(1, 1), (3, 7), (256, 256)])
def test_decode_sizes(B, P):
    d = synth.decode_inputs(2000 + B, B=B, P=P)
    print("decode", B, P, flush=True)
    o, pool = _run(d, scale=0.75)
    _check(d, o, pool, scale=0.75)


def test_decode_special_cases_exact():
    """beta = 0 with g = 0 leaves the state bit-identical and o = S q; beta = 1
    with unit k maps k to v (S k = v) after the step."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    d = synth.decode_inputs(2100, B=4, P=4, H_qk=2, H_v=6)
    g0 = np.zeros_like(d.g)
    b0 = np.zeros_like(d.beta)
    pool = dev(d.pool)
    gdn.gdn_decode_step(dev(d.q), dev(d.k), dev(d.v), dev(g0), dev(b0), pool, dev(d.slot_idx))
    torch.cuda.synchronize()
    assert (pool.cpu().numpy().view(np.uint32) == d.pool.view(np.uint32)).all()
    # keys of 64 entries +-1/8 (exactly unit length in bf16), beta = 1
    rng = np.random.default_rng(7)
    kk = np.zeros((d.B, d.H_qk, 128), dtype=np.float32)
    for b in range(d.B):
        for hq in range(d.H_qk):
            idx = rng.permutation(128)[:64]
            kk[b, hq, idx] = rng.choice([-0.125, 0.125], 64)
    kbits = synth.bf16_bits(kk)
    b1 = np.ones_like(d.beta)
    pool = dev(d.pool)
    gdn.gdn_decode_step(dev(d.q), dev(kbits), dev(d.v), dev(d.g), dev(b1), pool, dev(d.slot_idx))
    S = pool.cpu().numpy().astype(np.float64)
    vf = synth.bf16_value(d.v).astype(np.float64)
    for b in range(d.B):
        for h in range(d.H_v):
            Sk = S[d.slot_idx[b], h] @ kk[b, h // 3].astype(np.float64)
            np.testing.assert_allclose(Sk, vf[b, h], rtol=0, atol=1e-5 * (1 + np.abs(vf[b, h]).max()))


def test_decode_deterministic_and_empty():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    d = synth.decode_inputs(2200, B=16, P=32)
    o1, p1 = _run(d)
    o2, p2 = _run(d)
    assert np.array_equal(o1, o2) and np.array_equal(p1.view(np.uint32), p2.view(np.uint32))
    e = synth.decode_inputs(2201, B=0, P=4)
    pool = dev(e.pool)
    o = gdn.gdn_decode_step(dev(e.q), dev(e.k), dev(e.v), dev(e.g), dev(e.beta), pool,
                            dev(e.slot_idx))
    torch.cuda.synchronize()
    assert o.shape == (0, 48, 128)
