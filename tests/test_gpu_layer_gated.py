"""The layer's prefill with its output gate in the same call
(gdn_layer_prefill_gated): the gate y = o / sqrt(mean(o^2) + eps) * w * SiLU(z)
(the layer's norm and in_proj_z weights, "从参数竞赛到效率革命：拆解 Qwen3.8-27B
的稠密架构与长上下文混合注意力", sec. 2.1) is applied inside the chunked prefill as
rows of o are completed.  y and o must be bit-identical to gdn_layer_prefill
followed by gdn_gated_norm, and y must match the fp64 oracle's gates, prelude,
recurrence and gate composed (within the bound that o's parity bar implies
through the gate's per-row normalisation); every row of y is written
(NaN-filled outputs and workspace beforehand), also under graph capture with
replays."""
import numpy as np
import pytest

import oracle
import synth
from _util import TOL_BF16, assert_close, dev, errors, host

pytestmark = pytest.mark.gpu

CASES = {
    "T517": dict(T=517),
    "varlen": dict(lengths=[70, 3, 128, 1, 191, 64, 2]),
    "segmented": dict(T=64 * 64 + 37),
}


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _gate_inputs(seed, T, H_v, dv=128):
    rng = np.random.default_rng(seed)
    z = synth.bf16_bits(rng.normal(0.0, 1.0, (T, H_v, dv)).astype(np.float32))
    w = rng.uniform(0.5, 1.5, dv).astype(np.float32)
    return z, w


def _assert_gate_close(y, o_ref, z, w, what, eps=1e-6):
    """y against the fp64 gate of the oracle's o.  The gate divides each row by
    its own RMS, so o's parity bar (errors up to TOL_BF16 of max|o|) reaches y
    divided by that row's RMS: with n = o / rms and g = w SiLU(z), a change d
    in o (|d| <= D) moves y_e by at most D / rms * (1 + |n_e|) * |g_e| (the
    second term through rms itself, since mean|n| <= 1).  Each element is held
    to that bound plus y's bf16 rounding, and the whole output to the RMS-
    relative bar."""
    zf = synth.bf16_value(z).astype(np.float64)
    y_ref = oracle.gated_norm(o_ref, zf, w, eps)
    _, e_rms, _ = errors(y, y_ref)
    assert e_rms <= TOL_BF16, f"{what}: rms-rel {e_rms:.3e} > {TOL_BF16}"
    rms = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + eps)
    n = o_ref / rms
    gain = np.abs(w * zf / (1.0 + np.exp(-zf)))
    D = TOL_BF16 * np.max(np.abs(o_ref))
    bound = D / rms * (1.0 + np.abs(n)) * gain + 2.0 ** -8 * np.abs(y_ref) + 1e-6
    err = np.abs(y - y_ref)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (f"{what}: error {err[worst]:.3e} above its bound {bound[worst]:.3e} "
                                  f"at {worst}")


def _run_both(p, z, w, nan_fill=True):
    """gdn_layer_prefill_gated, and gdn_layer_prefill + gdn_gated_norm, on the
    same inputs; returns ((y, o, S, cs), (y2, o2, S2, cs2))."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    A_log = dev(p.meta["A_log"].astype(np.float32))
    dt = dev(p.meta["dt_bias"].astype(np.float32))
    x, cw, a, b = dev(p.x), dev(p.w), dev(p.meta["a"]), dev(p.meta["b"])
    cu = None if p.cu_seqlens is None else dev(p.cu_seqlens)
    S0 = None if p.S0 is None else dev(p.S0)
    zd, wd = dev(z), dev(w)
    shape = (p.T, p.H_v, p.dv)
    y = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    o = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(gdn.gdn_layer_prefill_gated_workspace_size(1 if cu is None else cu.numel() - 1,
                                                                p.T, p.H_qk, p.H_v),
                     dtype=torch.uint8, device="cuda")
    if nan_fill:
        ws.fill_(0xFF)
    y, o, S, cs = gdn.gdn_layer_prefill_gated(x, cw, a, b, A_log, dt, zd, wd, S0, cu, H_qk=p.H_qk,
                                              H_v=p.H_v, o=o, y=y, workspace=ws)
    o2, S2, cs2 = gdn.gdn_layer_prefill(x, cw, a, b, A_log, dt, S0, cu, H_qk=p.H_qk, H_v=p.H_v)
    y2 = gdn.gdn_gated_norm(o2, zd, wd)
    torch.cuda.synchronize()
    return (y, o, S, cs), (y2, o2, S2, cs2)


@pytest.mark.parametrize("name", list(CASES))
def test_gated_layer_prefill_bit_identical_to_prefill_then_gate(name):
    p = synth.raw_prefill(6100 + len(name), init_state=True, **CASES[name])
    z, w = _gate_inputs(6100 + len(name), p.T, p.H_v)
    print("gated layer prefill", name, "T", p.T, flush=True)
    (y, o, S, cs), (y2, o2, S2, cs2) = _run_both(p, z, w)
    for a_, b_, what in ((y, y2, "y"), (o, o2, "o"), (S, S2, "final state"), (cs, cs2, "conv state")):
        assert np.array_equal(_bits(a_), _bits(b_)), f"{what} differs from the separate calls"


@pytest.mark.parametrize("name", ["T517", "varlen"])
def test_gated_layer_prefill_against_oracle(name):
    p = synth.raw_prefill(6200 + len(name), init_state=True, **CASES[name])
    z, w = _gate_inputs(6200 + len(name), p.T, p.H_v)
    (y, o, S, _), _ = _run_both(p, z, w)
    A_log, dt = p.meta["A_log"], p.meta["dt_bias"]
    q, k, v = oracle.prelude(p.x, p.w, p.cu_seqlens, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv)
    g, beta = oracle.gates(p.meta["a"], p.meta["b"], A_log, dt)
    o_ref, S_ref = oracle.recurrent(q, k, v, g, beta, p.S0, p.cu_seqlens)
    assert_close(host(o), o_ref, TOL_BF16, "o")
    _assert_gate_close(host(y), o_ref, z, w, "y")
    assert_close(S.cpu().numpy(), S_ref, TOL_BF16, "S")


def test_gated_layer_prefill_32k_all_heads():
    """The 32768-token workload from raw projections, all 48 V-heads: y against
    the oracle composition element by element, and bit-identical to the
    separate calls."""
    p = synth.workload_prefill_32k()
    z, w = _gate_inputs(6300, p.T, p.H_v)
    print("gated layer prefill 32768", flush=True)
    (y, o, S, _), (y2, o2, S2, _) = _run_both(p, z, w, nan_fill=False)
    assert np.array_equal(_bits(y), _bits(y2)) and np.array_equal(_bits(o), _bits(o2))
    yh = host(y)
    del y, o, y2, o2
    A_log, dt = p.meta["A_log"], p.meta["dt_bias"]
    q, k, v = oracle.prelude(p.x, p.w, None, H_qk=p.H_qk, H_v=p.H_v, dk=p.dk, dv=p.dv)
    g, beta = oracle.gates(p.meta["a"], p.meta["b"], A_log, dt)
    o_ref, _ = oracle.recurrent(q, k, v, g, beta)
    del q, k, v
    _assert_gate_close(yh, o_ref, z, w, "y")


def test_gated_layer_prefill_graph_replays():
    """Captured into a HIP graph (one long sequence: eagerly it runs in
    segments) and replayed three times with eager work in between: every
    replay gives the eager call's bits (the arrival counts are cleared by the
    call itself)."""
    import torch
    import linear_attention_sequence_delta_amd as gdn
    p = synth.raw_prefill(6400, T=8192, init_state=True)
    z, w = _gate_inputs(6400, p.T, p.H_v)
    A_log = dev(p.meta["A_log"].astype(np.float32))
    dt = dev(p.meta["dt_bias"].astype(np.float32))
    x, cw, a, b, S0, zd, wd = (dev(t) for t in (p.x, p.w, p.meta["a"], p.meta["b"], p.S0, z, w))
    y_e, o_e, S_e, _ = gdn.gdn_layer_prefill_gated(x, cw, a, b, A_log, dt, zd, wd, S0, H_qk=p.H_qk,
                                                   H_v=p.H_v, conv_state=False)
    torch.cuda.synchronize()
    y_g, o_g, S_g = torch.empty_like(y_e), torch.empty_like(o_e), torch.empty_like(S_e)
    ws = torch.empty(gdn.gdn_layer_prefill_gated_workspace_size(1, p.T, p.H_qk, p.H_v),
                     dtype=torch.uint8, device="cuda")
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            gdn.gdn_layer_prefill_gated(x, cw, a, b, A_log, dt, zd, wd, S0, H_qk=p.H_qk, H_v=p.H_v,
                                        final_state=S_g, conv_state=False, o=o_g, y=y_g,
                                        workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(3):
        y_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a_, b_, what in ((y_g, y_e, "y"), (o_g, o_e, "o"), (S_g, S_e, "final state")):
            assert torch.equal(a_.view(torch.int16 if a_.dtype == torch.bfloat16 else torch.int32),
                               b_.view(torch.int16 if b_.dtype == torch.bfloat16 else torch.int32)), \
                f"replay {i}: {what} differs"
        (o_e.float() * 2).sum()                      # eager work in between
        torch.cuda.synchronize()
