"""Multi-token decode (speculative-decoding verification) on the GPU:
gdn_decode_multi_step against n successive gdn_decode_step calls (bit for
bit: the state stays fp32 either way), against the fp64 oracle, and
gdn_state_rollback against the states after each prefix of the tokens."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _tokens(seed, B, n, P):
    """n decode steps' inputs for the same B slots, stacked along axis 1."""
    d0 = synth.decode_inputs((seed, 0), B=B, P=P)
    steps = [d0] + [synth.decode_inputs((seed, j), B=B, pool=d0.pool, slot_idx=d0.slot_idx,
                                        A_log=d0.meta["A_log"], dt_bias=d0.meta["dt_bias"])
                    for j in range(1, n)]
    stack = {f: np.stack([getattr(d, f) for d in steps], axis=1)
             for f in ("q", "k", "v", "g", "beta")}
    return d0, stack


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("n", [1, 4])
def test_multi_step_bit_identical_to_single_steps(n):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    d0, x = _tokens(6100 + n, B=48, n=n, P=96)
    pool = dev(d0.pool)
    o, snaps = gdn.gdn_decode_multi_step(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]),
                                         dev(x["beta"]), pool, dev(d0.slot_idx), snapshots=True)
    pool1 = dev(d0.pool)
    slots = dev(d0.slot_idx)
    inter = []
    outs = []
    for j in range(n):
        inter.append(_bits(pool1)[d0.slot_idx])
        outs.append(_bits(gdn.gdn_decode_step(
            dev(x["q"][:, j]), dev(x["k"][:, j]), dev(x["v"][:, j]), dev(x["g"][:, j]),
            dev(x["beta"][:, j]), pool1, slots)))
    torch.cuda.synchronize()
    assert np.array_equal(_bits(o), np.stack(outs, axis=1))
    assert np.array_equal(_bits(pool), _bits(pool1))
    assert np.array_equal(_bits(snaps), np.stack(inter, axis=1))


def test_multi_step_against_oracle_and_rollback():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    n = 5
    d0, x = _tokens(6200, B=64, n=n, P=128)
    pool = dev(d0.pool)
    slots = dev(d0.slot_idx)
    o, snaps = gdn.gdn_decode_multi_step(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"]),
                                         dev(x["beta"]), pool, slots, snapshots=True)
    torch.cuda.synchronize()
    o_ref, s_ref, pool_ref = oracle.decode_multi_step(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                                      d0.pool, d0.slot_idx)
    assert_close(host(o), o_ref, TOL_BF16, "o")
    assert_close(snaps.cpu().numpy(), s_ref, TOL_BF16, "snapshots")
    assert_close(pool.cpu().numpy()[d0.slot_idx], pool_ref[d0.slot_idx], TOL_BF16, "final states")
    # keep a random prefix of each sequence's tokens (0 .. n)
    keep = np.random.default_rng(3).integers(0, n + 1, 64).astype(np.int32)
    after = _bits(pool)
    gdn.gdn_state_rollback(snaps, dev(keep), pool, slots)
    torch.cuda.synchronize()
    got = _bits(pool)
    sn = _bits(snaps)
    for b, s in enumerate(d0.slot_idx):
        want = after[s] if keep[b] == n else sn[b, keep[b]]
        assert np.array_equal(got[s], want), b
    rest = np.setdiff1d(np.arange(d0.P), d0.slot_idx)
    assert (got[rest].view(np.uint32) == synth.CANARY_BITS).all()
