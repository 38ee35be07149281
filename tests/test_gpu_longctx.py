"""Long-context hand-off at full size: a 262144-token prefill from raw
projections (the conv prelude fused into the chunked prefill), whose final
state seeds 256 decode sequences that then take 64 autoregressive steps.  One
V-head of every QK group (so every placement of a QK group's workgroups, and
all 128 columns of each checked head) is compared with the fp64 oracle at
every token of the prefill, at every decode step and in the final pool; every
output of the prefill must be finite.  The oracle runs only the checked heads
(their QK heads' q, k channels and their own v channels): every head's
computation is independent."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu

T_LONG = 262144
B_DEC = 256
STEPS = 64
H_QK, GRP = 16, 3
HEADS = [GRP * j + j % GRP for j in range(H_QK)]     # one V-head per QK group


def test_longctx_262144_prefill_then_decode_one_head_per_group():
    import torch
    import linear_attention_sequence_delta_amd as gdn

    p = synth.workload_longctx_prefill(T_LONG)
    print("inputs generated", flush=True)
    xd = dev(p.x)
    o = torch.full((p.T, p.H_v, p.dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    o, S = gdn.gdn_prefill_raw(xd, dev(p.w), dev(p.g), dev(p.beta), None, None, H_qk=p.H_qk,
                               H_v=p.H_v, o=o)
    torch.cuda.synchronize()
    del xd
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(S).all())
    o_h = host(o[:, HEADS])
    del o
    print("GPU prefill done", flush=True)

    D = p.dk
    hs = np.array(HEADS)
    chans = np.concatenate([np.arange(2 * H_QK * D),
                            ((2 * H_QK + hs)[:, None] * D + np.arange(D)[None, :]).ravel()])
    # the checked V-heads are V-heads 0..15 of a layer with one V-head per QK head
    qr, kr, vr = oracle.prelude(p.x[:, chans], p.w[chans], None, H_qk=H_QK, H_v=H_QK, dk=D, dv=D)
    o_ref, S_ref = oracle.recurrent(qr, kr, vr, p.g[:, HEADS], p.beta[:, HEADS])
    del qr, kr, vr
    print("oracle prefill done", flush=True)
    for j, h in enumerate(HEADS):
        assert_close(o_h[:, j], o_ref[:, j], TOL_BF16, f"prefill o head {h}")
        assert_close(S[0, h].cpu().numpy(), S_ref[0, j], TOL_BF16, f"prefill final state head {h}")

    # hand-off: every decode sequence continues from the prefill's final state
    pool = S[0].unsqueeze(0).expand(B_DEC, -1, -1, -1).contiguous()
    pool_ref = np.repeat(S_ref[:1], B_DEC, axis=0)            # [256, 16, 128, 128] fp64
    slot = None
    outs, outs_ref = [], []
    for step in range(STEPS):
        d = synth.workload_longctx_decode(step, B=B_DEC, pool=pool_ref[:1], slot_idx=slot,
                                          A_log=p.meta["A_log"], dt_bias=p.meta["dt_bias"])
        slot = d.slot_idx
        od = gdn.gdn_decode_step(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), pool,
                                 dev(slot))
        outs.append(host(od[:, HEADS]))
        o_st, pool_ref = oracle.decode_step(d.q, d.k, d.v[:, HEADS], d.g[:, HEADS],
                                            d.beta[:, HEADS], pool_ref, slot)
        outs_ref.append(o_st)
    torch.cuda.synchronize()
    print("decode steps done", flush=True)
    assert_close(np.stack(outs), np.stack(outs_ref), TOL_BF16, "decode o")
    assert_close(pool[:, HEADS].cpu().numpy(), pool_ref, TOL_BF16, "decode final pool")
