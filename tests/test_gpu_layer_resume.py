"""A prefill resumed from a previous one (gdn_layer_prefill and
gdn_layer_prefill_gated with conv_state_in): the conv window of a sequence's
first rows reaches into the three raw rows it carries over, and the state
recurrence starts from the carried state (Gated DeltaNet's short convolution
before q, k, v, "从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合
注意力", sec. 2.1; the delta rule's recurrence, sec. 2.2).

* against the fp64 oracle's prelude with the same history, gates and
  recurrence, and the conv history out against the oracle's bit for bit;
* a sequence cut at a multiple of the 64-token chunk from its start, run as two
  calls (the second given the first's final state and conv history), is bit
  for bit one call over the whole sequence: every chunk sees the same rows;
* cut anywhere else, the second call matches the oracle over the whole
  sequence; conv_state_in and conv_state may be one tensor (updated in place);
* the gated call with a history is bit for bit the ungated one followed by the
  gate, and splits the same way."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu

CASES = {
    "T517": dict(T=517),
    "varlen": dict(lengths=[70, 3, 128, 1, 191, 64, 2, 0]),
}


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _history(seed, N, C):
    rng = np.random.default_rng(seed)
    return synth.bf16_bits(rng.standard_normal((N, 3, C)).astype(np.float32))


def _weights(p):
    return dev(p.meta["A_log"].astype(np.float32)), dev(p.meta["dt_bias"].astype(np.float32))


def _call(x, w, a, b, S0, cu, p, **kw):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    A_log, dt = _weights(p)
    out = gdn.gdn_layer_prefill(dev(x), dev(w), dev(a), dev(b), A_log, dt,
                                None if S0 is None else dev(S0),
                                None if cu is None else dev(cu), H_qk=p.H_qk, H_v=p.H_v, **kw)
    torch.cuda.synchronize()
    return out


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _rows(cu, lo, hi):
    """Row indices of [lo[n], hi[n]) within each sequence n of offsets cu."""
    return np.concatenate([np.arange(cu[n] + lo[n], cu[n] + hi[n]) for n in range(len(cu) - 1)]
                          + [np.zeros(0, np.int64)]).astype(np.int64)


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_with_history_against_oracle(name):
    p = synth.raw_prefill(7100 + len(name), init_state=True, **CASES[name])
    C = p.x.shape[1]
    hist = _history(7150 + len(name), p.N, C)
    print("resumed prefill", name, "T", p.T, flush=True)
    o, S, cs = _call(p.x, p.w, p.meta["a"], p.meta["b"], p.S0, p.cu_seqlens, p,
                     conv_state_in=dev(hist))
    q, k, v = oracle.prelude(p.x, p.w, p.cu_seqlens, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv,
                             conv_state_in=hist)
    g, beta = oracle.gates(p.meta["a"], p.meta["b"], p.meta["A_log"], p.meta["dt_bias"])
    o_ref, S_ref = oracle.recurrent(q, k, v, g, beta, p.S0, p.cu_seqlens)
    assert_close(host(o), o_ref, TOL_BF16, "o")
    assert_close(S.cpu().numpy(), S_ref, TOL_BF16, "S")
    cs_ref = oracle.conv_state(p.x, p.cu_seqlens, conv_state_in=hist)
    assert np.array_equal(_bits(cs), cs_ref.view(np.int16))
    # the history changes the outputs of exactly the first three rows of each sequence
    o0, _, _ = _call(p.x, p.w, p.meta["a"], p.meta["b"], p.S0, p.cu_seqlens, p)
    assert not np.array_equal(_bits(o), _bits(o0))


SPLITS = {
    # (lengths, first-part lengths): cuts at multiples of 64 from each start
    "single": ([517], [128]),
    "segmented": ([64 * 64 + 37], [64 * 33]),
    "varlen": ([200, 70, 3, 130, 64], [128, 64, 0, 64, 64]),
}


@pytest.mark.parametrize("name", list(SPLITS))
def test_split_at_chunk_boundary_is_bit_identical(name):
    lengths, first = SPLITS[name]
    full = synth.raw_prefill(7200 + len(name), lengths=lengths, init_state=True)
    a, b = full.meta["a"], full.meta["b"]
    cu = _cu(lengths)
    i1 = _rows(cu, [0] * len(lengths), first)
    i2 = _rows(cu, first, lengths)
    cu1 = _cu(first)
    cu2 = _cu(np.subtract(lengths, first))
    print("split prefill", name, lengths, first, flush=True)
    o, S, cs = _call(full.x, full.w, a, b, full.S0, cu, full)
    o1, S1, cs1 = _call(full.x[i1], full.w, a[i1], b[i1], full.S0, cu1, full)
    o2, S2, cs2 = _call(full.x[i2], full.w, a[i2], b[i2], S1.cpu().numpy(), cu2, full,
                        conv_state_in=cs1)
    ob = _bits(o)
    assert np.array_equal(_bits(o1), ob[i1]), "first part"
    assert np.array_equal(_bits(o2), ob[i2]), "second part"
    assert np.array_equal(_bits(S2), _bits(S)), "final state"
    assert np.array_equal(_bits(cs2), _bits(cs)), "conv history"


def test_split_anywhere_against_oracle_and_in_place_history():
    """Cut at row 203 of 517 (mid-chunk) and, in a packed batch, at rows 1, 2
    and 65; the second call's conv history is updated in place (conv_state_in
    is the conv_state tensor)."""
    lengths, first = [517, 9, 4, 150], [203, 1, 2, 65]
    full = synth.raw_prefill(7300, lengths=lengths, init_state=True)
    a, b = full.meta["a"], full.meta["b"]
    cu = _cu(lengths)
    i2 = _rows(cu, first, lengths)
    i1 = _rows(cu, [0] * len(lengths), first)
    print("split prefill mid-chunk", lengths, first, flush=True)
    _, S1, cs1 = _call(full.x[i1], full.w, a[i1], b[i1], full.S0, _cu(first), full)
    o2, S2, cs_same = _call(full.x[i2], full.w, a[i2], b[i2], S1.cpu().numpy(),
                            _cu(np.subtract(lengths, first)), full, conv_state_in=cs1,
                            conv_state=cs1)
    assert cs_same is cs1
    q, k, v = oracle.prelude(full.x, full.w, cu, H_qk=full.H_qk, H_v=full.H_v, dk=full.dk,
                             dv=full.dv)
    g, beta = oracle.gates(a, b, full.meta["A_log"], full.meta["dt_bias"])
    o_ref, S_ref = oracle.recurrent(q, k, v, g, beta, full.S0, cu)
    assert_close(host(o2), o_ref[i2], TOL_BF16, "o (second part)")
    assert_close(S2.cpu().numpy(), S_ref, TOL_BF16, "S")
    assert np.array_equal(_bits(cs1), oracle.conv_state(full.x, cu).view(np.int16))


def _gated(x, w, a, b, z, nw, S0, cu, p, **kw):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    A_log, dt = _weights(p)
    out = gdn.gdn_layer_prefill_gated(dev(x), dev(w), dev(a), dev(b), A_log, dt, dev(z), dev(nw),
                                      None if S0 is None else dev(S0),
                                      None if cu is None else dev(cu), H_qk=p.H_qk, H_v=p.H_v,
                                      **kw)
    torch.cuda.synchronize()
    return out


GATED_SPLITS = {
    # one sequence: the gate fused into the scan (its grid fits the device);
    # 8192 tokens also run in segments
    "single": ([600], [192]),
    "segmented": ([8192], [4096]),
    # three sequences: the scan's grid is too large to fuse, the gate runs after it
    "packed": ([300, 70, 2], [192, 64, 0]),
}


@pytest.mark.parametrize("name", list(GATED_SPLITS))
def test_gated_with_history_equals_prefill_then_gate_and_splits(name):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    lengths, first = GATED_SPLITS[name]
    p = synth.raw_prefill(7400 + len(name), lengths=lengths, init_state=True)
    rng = np.random.default_rng(7401)
    z = synth.bf16_bits(rng.normal(0.0, 1.0, (p.T, p.H_v, p.dv)).astype(np.float32))
    nw = rng.uniform(0.5, 1.5, p.dv).astype(np.float32)
    hist = _history(7402, p.N, p.x.shape[1])
    a, b = p.meta["a"], p.meta["b"]
    print("gated resumed prefill", name, lengths, flush=True)
    y, o, S, cs = _gated(p.x, p.w, a, b, z, nw, p.S0, p.cu_seqlens, p, conv_state_in=dev(hist))
    o2, S2, cs2 = _call(p.x, p.w, a, b, p.S0, p.cu_seqlens, p, conv_state_in=dev(hist))
    y2 = gdn.gdn_gated_norm(o2, dev(z), dev(nw))
    torch.cuda.synchronize()
    for u, w_, what in ((y, y2, "y"), (o, o2, "o"), (S, S2, "S"), (cs, cs2, "conv history")):
        assert np.array_equal(_bits(u), _bits(w_)), what
    # the same call cut at chunk boundaries: two gated calls give the same y
    cu = p.cu_seqlens
    i1 = _rows(cu, [0] * len(lengths), first)
    i2 = _rows(cu, first, lengths)
    ya, _, Sa, csa = _gated(p.x[i1], p.w, a[i1], b[i1], z[i1], nw, p.S0, _cu(first), p,
                            conv_state_in=dev(hist))
    yb, _, Sb, csb = _gated(p.x[i2], p.w, a[i2], b[i2], z[i2], nw, Sa.cpu().numpy(),
                            _cu(np.subtract(lengths, first)), p, conv_state_in=csa)
    yb_ = _bits(y)
    assert np.array_equal(_bits(ya), yb_[i1]) and np.array_equal(_bits(yb), yb_[i2])
    assert np.array_equal(_bits(Sb), _bits(S)) and np.array_equal(_bits(csb), _bits(cs))
