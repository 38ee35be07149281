"""A training forward pass that keeps the chunk states (gdn_prefill_save_states,
gdn_prefill_raw_save_states) and the backward that reads them
(gdn_prefill_backward_saved), on the GPU:

* the forward's outputs are bit-identical with and without keeping the states;
* the kept states are the initial state (rounded to bf16) at each sequence's
  first chunk, and match the oracle's recurrence after the tokens before each
  later chunk;
* the fused prelude path keeps the same states, bit for bit, as the prelude
  followed by the bf16 prefill;
* the backward from the kept states is bit-identical to the backward that
  recomputes them (ragged, packed varlen, and a sequence long enough for the
  forward to run in segments)."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu

CASES = {
    "T65": dict(T=65),
    "T300": dict(T=300),
    "varlen": dict(lengths=[70, 3, 128, 1, 191, 64, 2]),
    "T8192": dict(T=8192),        # 128 chunks: the forward runs in segments
}


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(a, b, what):
    import torch
    assert torch.equal(_bits(a), _bits(b)), what


def _chunk_starts(p):
    """(global chunk index, sequence, first token) of every chunk, in the order
    the kept states use: sequence by sequence, chunk by chunk."""
    cu = [0, p.T] if p.cu_seqlens is None else list(p.cu_seqlens)
    out, gc = [], 0
    for n in range(len(cu) - 1):
        for t in range(cu[n], cu[n + 1], 64):
            out.append((gc, n, t))
            gc += 1
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_forward_unchanged_and_states_pinned(name):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.direct_prefill(8100, init_state=True, **CASES[name])
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    args = (dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), dev(p.S0), cu)
    print("save states", name, flush=True)
    o0, S0f = gdn.gdn_prefill(*args)
    o1, S1f, cs = gdn.gdn_prefill(*args, chunk_states=True)
    torch.cuda.synchronize()
    _same(o0, o1, "o")
    _same(S0f, S1f, "final state")
    cs = cs[: gdn.gdn_chunk_states_size(p.N, p.T, p.H_v) // 2].view(-1, p.H_v, 128, 128)
    starts = _chunk_starts(p)
    S0_bf16 = torch.from_numpy(p.S0).to(torch.bfloat16)
    cs_h = cs.cpu()
    seq_start = [0] if p.cu_seqlens is None else [int(x) for x in p.cu_seqlens[:-1]]
    for gc, n, t in starts:
        if t == seq_start[n]:
            # the first chunk of a sequence starts from its initial state
            _same(cs_h[gc], S0_bf16[n], f"chunk {gc}")
    # later chunks against the oracle's recurrence over the tokens before them
    checked = 0
    for gc, n, t in starts:
        s0 = seq_start[n]
        if t == s0 or checked >= 4:
            continue
        sl = slice(s0, t)
        _, S_ref = oracle.recurrent(p.q[sl], p.k[sl], p.v[sl], p.g[sl], p.beta[sl], p.S0[n:n + 1])
        assert_close(host(cs[gc]), S_ref[0], TOL_BF16, f"chunk {gc} state")
        checked += 1


@pytest.mark.parametrize("name", ["T300", "varlen", "T8192"])
def test_fused_prelude_keeps_the_same_states(name):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.raw_prefill(8200, init_state=True, **CASES[name])
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    x, w = dev(p.x), dev(p.w)
    g, beta, S0 = dev(p.g), dev(p.beta), dev(p.S0)
    print("fused save states", name, flush=True)
    o_raw, S_raw = gdn.gdn_prefill_raw(x, w, g, beta, S0, cu)
    o1, S1, cs1 = gdn.gdn_prefill_raw(x, w, g, beta, S0, cu, chunk_states=True)
    q, k, v = gdn.gdn_conv_prelude(x, w, cu)
    o2, S2, cs2 = gdn.gdn_prefill(q, k, v, g, beta, S0, cu, chunk_states=True)
    torch.cuda.synchronize()
    _same(o_raw, o1, "o")
    _same(S_raw, S1, "final state")
    n = gdn.gdn_chunk_states_size(p.N, p.T, p.H_v) // 2
    nch = len(_chunk_starts(p))
    per = p.H_v * 128 * 128
    _same(cs1[: nch * per], cs2[: nch * per], "chunk states")
    assert n >= nch * per


@pytest.mark.parametrize("name", list(CASES))
def test_backward_from_kept_states_is_bit_identical(name):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.direct_prefill(8300, init_state=True, **CASES[name])
    d_o, dSf = synth.output_grads(8300, p.T, p.N)
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    q, k, v, g, beta, S0 = (dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), dev(p.S0))
    print("backward from kept states", name, flush=True)
    _, _, cs = gdn.gdn_prefill(q, k, v, g, beta, S0, cu, chunk_states=True)
    ref = gdn.gdn_prefill_backward(q, k, v, g, beta, dev(d_o), S0, dev(dSf), cu)
    got = gdn.gdn_prefill_backward(q, k, v, g, beta, dev(d_o), None, dev(dSf), cu, chunk_states=cs)
    torch.cuda.synchronize()
    for nm, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), got, ref):
        _same(a, b, nm)


def test_backward_from_kept_states_against_oracle():
    """The whole training pair against the oracle's gradients (T = 517, ragged
    end, initial state and final-state gradient)."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.direct_prefill(8400, T=517, init_state=True)
    d_o, dSf = synth.output_grads(8400, p.T, 1)
    q, k, v, g, beta, S0 = (dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), dev(p.S0))
    _, _, cs = gdn.gdn_prefill(q, k, v, g, beta, S0, chunk_states=True)
    got = gdn.gdn_prefill_backward(q, k, v, g, beta, dev(d_o), None, dev(dSf), chunk_states=cs)
    torch.cuda.synchronize()
    ref = oracle.recurrent_backward(p.q, p.k, p.v, p.g, p.beta, d_o, p.S0, dSf, None)
    for nm, x, r in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), got, ref):
        assert_close(host(x), r, TOL_BF16, nm)


@pytest.mark.parametrize("name", ["T300", "varlen", "T8192"])
def test_layer_pair_from_kept_states_is_bit_identical(name):
    """gdn_layer_prefill keeping the chunk states, then
    gdn_layer_prefill_backward from them: outputs and gradients bit-identical
    to the plain layer calls."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.raw_prefill(8500, init_state=True, **CASES[name])
    d_o, dSf = synth.output_grads(8500, p.T, p.N)
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    x, w, S0 = dev(p.x), dev(p.w), dev(p.S0)
    a, b = dev(p.meta["a"]), dev(p.meta["b"])
    A_log = dev(p.meta["A_log"].astype(np.float32))
    dtb = dev(p.meta["dt_bias"].astype(np.float32))
    print("layer pair", name, flush=True)
    o0, S0f, c0 = gdn.gdn_layer_prefill(x, w, a, b, A_log, dtb, S0, cu)
    o1, S1f, c1, cs = gdn.gdn_layer_prefill(x, w, a, b, A_log, dtb, S0, cu, chunk_states=True)
    ref = gdn.gdn_layer_prefill_backward(x, w, a, b, A_log, dtb, dev(d_o), S0, dev(dSf), cu)
    got = gdn.gdn_layer_prefill_backward(x, w, a, b, A_log, dtb, dev(d_o), None, dev(dSf), cu,
                                         chunk_states=cs)
    torch.cuda.synchronize()
    for nm, u, t in (("o", o0, o1), ("final state", S0f, S1f), ("conv state", c0, c1)):
        _same(u, t, nm)
    for nm, u, t in zip(("dx", "dconv_w", "da", "db", "dA_log", "ddt_bias", "dS0"), got, ref):
        _same(u, t, nm)
