"""Long-context hand-off at full size: a 262144-token prefill from raw
projections (the conv prelude fused into the chunked prefill), whose final
state seeds 256 decode
sequences that then take 64 autoregressive steps.  A sampled V-head is checked
against the fp64 oracle at every token of the prefill, at every decode step and
in the final pool.  The oracle runs only the sampled head (its QK head's q, k
channels and its own v channels): every head's computation is independent."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu

T_LONG = 262144
B_DEC = 256
STEPS = 64
HEAD = 29          # V-head 29 reads QK head 9


def test_longctx_262144_prefill_then_decode_sampled_head():
    import torch
    import linear_attention_sequence_delta_amd as gdn

    p = synth.workload_longctx_prefill(T_LONG)
    print("inputs generated", flush=True)
    xd = dev(p.x)
    o, S = gdn.gdn_prefill_raw(xd, dev(p.w), dev(p.g), dev(p.beta), None, None, H_qk=p.H_qk,
                               H_v=p.H_v)
    torch.cuda.synchronize()
    del xd
    o_h = host(o[:, HEAD])
    del o
    print("GPU prefill done", flush=True)

    grp = p.H_v // p.H_qk
    hq, D = HEAD // grp, p.dk
    chans = np.concatenate([np.arange(hq * D, (hq + 1) * D),
                            np.arange((p.H_qk + hq) * D, (p.H_qk + hq + 1) * D),
                            np.arange((2 * p.H_qk + HEAD) * D, (2 * p.H_qk + HEAD + 1) * D)])
    qr, kr, vr = oracle.prelude(p.x[:, chans], p.w[chans], None, H_qk=1, H_v=1, dk=D, dv=D)
    o_ref, S_ref = oracle.recurrent(qr, kr, vr, p.g[:, HEAD:HEAD + 1], p.beta[:, HEAD:HEAD + 1])
    del qr, kr, vr
    print("oracle prefill done", flush=True)
    assert_close(o_h, o_ref[:, 0], TOL_BF16, "prefill o")
    assert_close(S[0, HEAD].cpu().numpy(), S_ref[0, 0], TOL_BF16, "prefill final state")

    # hand-off: every decode sequence continues from the prefill's final state
    pool = S[0].unsqueeze(0).expand(B_DEC, -1, -1, -1).contiguous()
    pool_ref = np.repeat(S_ref[:, 0:1], B_DEC, axis=0)            # [256, 1, 128, 128] fp64
    slot = None
    outs, outs_ref = [], []
    for step in range(STEPS):
        d = synth.workload_longctx_decode(step, B=B_DEC, pool=pool_ref[:1], slot_idx=slot,
                                          A_log=p.meta["A_log"], dt_bias=p.meta["dt_bias"])
        slot = d.slot_idx
        od = gdn.gdn_decode_step(dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), pool,
                                 dev(slot))
        outs.append(host(od[:, HEAD]))
        o_st, pool_ref = oracle.decode_step(d.q[:, hq:hq + 1], d.k[:, hq:hq + 1],
                                            d.v[:, HEAD:HEAD + 1], d.g[:, HEAD:HEAD + 1],
                                            d.beta[:, HEAD:HEAD + 1], pool_ref, slot)
        outs_ref.append(o_st[:, 0])
    torch.cuda.synchronize()
    print("decode steps done", flush=True)
    assert_close(np.stack(outs), np.stack(outs_ref), TOL_BF16, "decode o")
    assert_close(pool[:, HEAD].cpu().numpy(), pool_ref[:, 0], TOL_BF16, "decode final pool")
