"""Failure modes that other implementations of this layer are reported to have
("Qwen3.8-27B：27B 如何打出千亿级效果，且塞进单张消费级显卡", sec. 5: whole-graph
capture garbling the output, a slot finder looping forever), turned into checks:

* a prefill and a backward of one long sequence (which, run eagerly, fork part
  of their work onto an auxiliary stream) and a decode step, captured into a HIP graph and
  replayed several times with eager work and synchronisations in between, give
  the eager results bit for bit at every replay;
* with GDN_DEBUG=1 (read at every call) duplicate and out-of-range slot ids and
  a decreasing cu_seqlens are rejected on the device before any layer kernel
  runs, and valid inputs pass and give the same results as without it.

The invalid inputs are chosen so that no kernel could fault even unchecked:
the out-of-range slot id addresses a slot that exists in the allocation
(only the P passed in excludes it), and the duplicate-id check runs first, so
the later cases run only once the checks are known to be live."""
import os

import numpy as np
import pytest

import synth
from _util import dev

pytestmark = pytest.mark.gpu


def _replays_match(graph, outs, eager, other_work, n=3):
    import torch
    for i in range(n):
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {i} differs from the eager call"
        other_work()
        torch.cuda.synchronize()


def test_graph_capture_segmented_prefill_raw():
    """T = 8192 from raw projections: eagerly this runs in segments with the prep
    of later segments on the auxiliary stream; captured, it stays on the
    capturing stream, with the same bits."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.raw_prefill(5100, T=8192, init_state=True)
    x, w, g, b, S0 = dev(p.x), dev(p.w), dev(p.g), dev(p.beta), dev(p.S0)
    ws = torch.empty(gdn.gdn_prefill_raw_workspace_size(1, p.T, p.H_qk, p.H_v), dtype=torch.uint8,
                     device="cuda")
    o_e, S_e = gdn.gdn_prefill_raw(x, w, g, b, S0, H_qk=p.H_qk, H_v=p.H_v, workspace=ws)
    torch.cuda.synchronize()
    o_g = torch.empty_like(o_e)
    S_g = torch.empty_like(S_e)
    ws_g = torch.empty_like(ws)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            gdn.gdn_prefill_raw(x, w, g, b, S0, H_qk=p.H_qk, H_v=p.H_v, o=o_g, final_state=S_g,
                                workspace=ws_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def other():      # eager work between replays, on the same buffers' neighbours
        gdn.gdn_prefill_raw(x, w, g, b, S0, H_qk=p.H_qk, H_v=p.H_v, workspace=ws)
        (o_e.float() * 2).sum()

    _replays_match(graph, (o_g, S_g), (o_e, S_e), other)


@pytest.mark.parametrize("kept", [False, True])
def test_graph_capture_segmented_backward(kept):
    """T = 8192 backward (recomputing the forward, or from kept chunk states):
    eagerly the reverse scan runs in segments, with the backward records and the
    last segment's chunk gradients on the auxiliary stream; captured, everything
    runs unsegmented on the capturing stream.  Every replay gives the eager
    gradients bit for bit."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.direct_prefill(5150 + kept, T=8192, init_state=True)
    d_o, dSf = synth.output_grads(5150 + kept, p.T, p.N)
    q, k, v, g, b, S0 = dev(p.q), dev(p.k), dev(p.v), dev(p.g), dev(p.beta), dev(p.S0)
    do, dsf = dev(d_o), dev(dSf)
    cs = gdn.gdn_prefill(q, k, v, g, b, S0, chunk_states=True)[2] if kept else None
    size = gdn.gdn_prefill_backward_saved_workspace_size if kept else gdn.gdn_prefill_backward_workspace_size
    ws = torch.empty(size(1, p.T, p.H_qk, p.H_v), dtype=torch.uint8, device="cuda")
    print("backward capture, kept states", kept, flush=True)
    eager = gdn.gdn_prefill_backward(q, k, v, g, b, do, S0, dsf, scale=1.0, workspace=ws,
                                     chunk_states=cs)
    torch.cuda.synchronize()
    ws_g = torch.empty_like(ws)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            outs = gdn.gdn_prefill_backward(q, k, v, g, b, do, S0, dsf, scale=1.0, workspace=ws_g,
                                            chunk_states=cs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def other():
        gdn.gdn_prefill_backward(q, k, v, g, b, do, S0, dsf, scale=1.0, workspace=ws,
                                 chunk_states=cs)

    _replays_match(graph, outs, eager, other)


def test_graph_capture_decode_step():
    """A decode step updates its slots in place: each replay advances the
    captured pool by one token, exactly as an eager step advances a copy."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    d = synth.decode_inputs(5200, B=64, P=128)
    q, k, v, g, b, slot = dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta), dev(d.slot_idx)
    pool_e = dev(d.pool)
    pool_g = pool_e.clone()
    o_g = torch.empty((d.B, d.H_v, d.dv), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_decode_step(q, k, v, g, b, pool_g.clone(), slot)      # first use before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            gdn.gdn_decode_step(q, k, v, g, b, pool_g, slot, o=o_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(3):
        graph.replay()
        o_e = gdn.gdn_decode_step(q, k, v, g, b, pool_e, slot)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {i}: o differs"
        assert torch.equal(pool_g.view(torch.int32), pool_e.view(torch.int32)), f"replay {i}: pool differs"
        (pool_e[:1] * 0.5).sum()                                   # eager work in between
        torch.cuda.synchronize()


@pytest.fixture
def debug_on():
    old = os.environ.get("GDN_DEBUG")
    os.environ["GDN_DEBUG"] = "1"
    yield
    if old is None:
        del os.environ["GDN_DEBUG"]
    else:
        os.environ["GDN_DEBUG"] = old


def test_debug_mode_rejects_bad_slots_and_cu_seqlens(debug_on):
    import torch
    import linear_attention_sequence_delta_amd as gdn
    P = 16
    d = synth.decode_inputs(5300, B=8, P=P + 1)        # one slot more than the P passed below
    q, k, v, g, b = dev(d.q), dev(d.k), dev(d.v), dev(d.g), dev(d.beta)
    gen = torch.Generator(device="cuda").manual_seed(5300)
    pool = torch.randn((P + 1, d.H_v, d.dv, d.dk), generator=gen, device="cuda") * 0.02
    before = pool.clone()

    def step(slots):
        return gdn.gdn_decode_step(q, k, v, g, b, pool[:P], dev(np.asarray(slots, dtype=np.int32)))

    ok = [2, 9, 0, 15, 4, 11, 7, 13]
    # duplicate ids (harmless unchecked: a race on valid slots)
    dup = list(ok)
    dup[3] = dup[1]
    with pytest.raises(gdn.GDNError) as err:
        step(dup)
    assert err.value.code == gdn.GDN_ERR_DEVICE_CHECK
    torch.cuda.synchronize()
    assert torch.equal(pool.view(torch.int32), before.view(torch.int32)), "a rejected call changed the pool"
    # an id outside [0, P) (slot P exists in the allocation)
    bad = list(ok)
    bad[5] = P
    with pytest.raises(gdn.GDNError) as err:
        step(bad)
    assert err.value.code == gdn.GDN_ERR_DEVICE_CHECK
    torch.cuda.synchronize()
    assert torch.equal(pool.view(torch.int32), before.view(torch.int32)), "a rejected call changed the pool"
    # valid ids pass, with the same results as without debug mode
    o1 = step(ok)
    after_debug = pool.clone()
    pool.copy_(before)
    os.environ["GDN_DEBUG"] = "0"
    o2 = step(ok)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(pool.view(torch.int32), after_debug.view(torch.int32))
    os.environ["GDN_DEBUG"] = "1"

    # a decreasing cu_seqlens is rejected before the prefill's kernels run
    pf = synth.direct_prefill(5301, lengths=[120, 30, 50], init_state=True)
    cu = dev(np.array([0, 120, 100, 200], dtype=np.int32))
    o = torch.full((pf.T, pf.H_v, pf.dv), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn.GDNError) as err:
        gdn.gdn_prefill(dev(pf.q), dev(pf.k), dev(pf.v), dev(pf.g), dev(pf.beta), dev(pf.S0), cu, o=o)
    assert err.value.code == gdn.GDN_ERR_DEVICE_CHECK
    torch.cuda.synchronize()
    assert bool((o.float() == 7.0).all()), "a rejected prefill wrote outputs"
    # the valid packing passes in debug mode
    cu_ok = dev(pf.cu_seqlens)
    gdn.gdn_prefill(dev(pf.q), dev(pf.k), dev(pf.v), dev(pf.g), dev(pf.beta), dev(pf.S0), cu_ok, o=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
