"""Conv/SiLU/L2 prelude on the GPU against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _run(p, eps=1e-6):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    q, k, v = gdn.gdn_conv_prelude(dev(p.x), dev(p.w), cu, H_qk=p.H_qk, H_v=p.H_v, l2_eps=eps)
    torch.cuda.synchronize()
    return host(q), host(k), host(v)


@pytest.mark.parametrize("lengths", [None, [37, 64, 1, 100, 3, 95]])
def test_prelude_matches_oracle(lengths):
    p = synth.raw_prefill(3001, T=300, lengths=lengths)
    print("prelude T", p.T, "lengths", lengths, flush=True)
    q, k, v = _run(p)
    qr, kr, vr = oracle.prelude(p.x, p.w, p.cu_seqlens, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv)
    # per-token, per-head comparison: bf16 outputs (relative 2^-9)
    for name, a, r in (("q", q, qr), ("k", k, kr), ("v", v, vr)):
        assert_close(a, r, TOL_BF16, name)
        np.testing.assert_allclose(a, r, rtol=8e-3, atol=8e-3 * np.abs(r).max())
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-2)


def test_prelude_full_length_sampled_tokens():
    """T = 32768 (the long-prompt workload): every output row of a token sample."""
    p = synth.workload_prefill_32k()
    q, k, v = _run(p)
    rng = np.random.default_rng(0)
    toks = np.unique(np.concatenate([[0, 1, 2, 3, p.T - 1], rng.integers(0, p.T, 60)]))
    for t in toks:
        lo = max(0, t - 3)
        qr, kr, vr = oracle.prelude(p.x[lo:t + 1], p.w, None, H_qk=p.H_qk, H_v=p.H_v,
                                    dk=p.dk, dv=p.dv)
        for a, r in ((q[t], qr[-1]), (k[t], kr[-1]), (v[t], vr[-1])):
            np.testing.assert_allclose(a, r, rtol=8e-3, atol=8e-3 * np.abs(r).max())
