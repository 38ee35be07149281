"""gdn_prefill_no_alloc (the workspace in the library's own scratch array)
against gdn_prefill (the same computation with a caller workspace), through
the C ABI: two calls in a row, the second on a smaller input, each compared
with the existing entry point's outputs to the bf16 bar (and, the kernels being
the same, bit for bit); a call whose workspace would exceed the scratch is
rejected before anything is enqueued."""
import numpy as np
import pytest

import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _both(p):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    args = (dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta))
    S0 = dev(p.S0)
    o_ref, S_ref = gdn.gdn_prefill(*args, S0, cu)
    o = torch.full_like(o_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    gdn.gdn_prefill_no_alloc(*args, o, S0, S, cu)
    torch.cuda.synchronize()
    assert_close(host(o), host(o_ref), TOL_BF16, "o")
    assert_close(S.cpu().numpy(), S_ref.cpu().numpy(), TOL_BF16, "final state")
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_no_alloc_prefill_matches_prefill_twice():
    _both(synth.direct_prefill(5400, T=3000, init_state=True))                       # 47 chunks
    _both(synth.direct_prefill(5401, lengths=[700, 1, 300], init_state=True))        # smaller


def test_no_alloc_prefill_rejects_oversize():
    import torch
    import linear_attention_sequence_delta_amd as gdn
    T = 8192                                     # 128 chunks x 48 V-heads: more than 64 MiB
    assert gdn.gdn_prefill_workspace_size(gdn.GDN_BF16, 1, T, 16, 48) > (64 << 20)
    q = torch.zeros((T, 16, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((T, 48, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((T, 48), dtype=torch.float32, device="cuda")
    o = torch.full((T, 48, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn.GDNError) as err:
        gdn.gdn_prefill_no_alloc(q, q, v, g, g, o)
    assert err.value.code == gdn.GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o.float() == 3.0).all())
