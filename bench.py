"""Benchmark of the Gated DeltaNet layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the layer's prefill path over one batch of synthetic
input: the conv/SiLU/L2 prelude on raw bf16 projections and the chunked
prefill, for one sequence of 32768 tokens with 16 QK heads, 48 V heads and
d_k = d_v = 128, as one gdn_prefill_raw call (prelude fused into the prefill's
plan, prep and scan kernels).  `value` is prefill tokens/s over the K timed
steps.  The same step as two calls (gdn_conv_prelude, then gdn_prefill) is
timed beside it and reported under "phases_us".  `--path fused|unfused`
times one of the two only (for profiling runs).  The decode side of the metric (one decode
step for 256 sequences over a 256-slot state pool) is timed in the same run
and reported under "decode".  Every input is generated and resident in HBM
before the timed regions start; timing uses HIP events on the stream the
kernels run on.  The fp64 oracle is timed on the host's cores over a bounded
sample of the same workload and reported as "cpu_baseline".

The long-context hand-off is timed in the same run and reported under
"longctx": a 262144-token prelude + prefill, then 64 decode steps of 256
sequences that continue from its final state, and a stack of 48 independently
seeded layers (one decode step each, B = 256) per decode token.
`--no-longctx` skips it.

`--copy-calibration BYTES` runs a plain device copy of BYTES bytes instead: the
reference run for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0

T_PREFILL = 32768
B_DECODE = 256
H_QK, H_V, D = 16, 48, 128
CHUNK = 64

# Algorithmic work (no materialised per-chunk state counted):
# prefill flops per token per V-head: three dense C x d x d products (K S^T,
# Q S^T, the state update: 6 d^2) plus five C x C x d triangular products
# counted at their useful half (K K^T, Q K^T, T applied to K and V, P U: 5 C d).
PREFILL_FLOP_PER_TOKEN = H_V * (6 * D * D + 5 * CHUNK * D)
# prelude bytes per token: raw projections in + q, k, v out (bf16)
PRELUDE_BYTES_PER_TOKEN = 2 * 2 * (2 * H_QK * D + H_V * D)
# decode bytes per sequence: each (sequence, V-head) state read and written
# once in fp32, plus q, k, v, o in bf16 and g, beta in fp32
DECODE_BYTES_PER_SEQ = (H_V * (2 * D * D * 4 + 2 * D * 2 + 2 * 4) + 2 * H_QK * D * 2)

# backward (gdn_prefill_backward) flops per token per V-head, as executed and
# counted at the useful half of triangular products: d x d products 18 d^2
# (forward states again: K S^T and the update, 4 d^2; reverse scan: K dS'^T and
# the two-term state-gradient update, 6 d^2; per chunk: K S^T, dO S, dR S,
# U dS', 8 d^2) and C x C x d products 10 C d (P^T dO, T'^T dU, T' R, dO U^T,
# dU R^T, M_P K, M_P^T Q, the two M_A' K, K K^T with Q K^T).
BACKWARD_FLOP_PER_TOKEN = H_V * (18 * D * D + 10 * CHUNK * D)

T_LONG, LONG_STEPS, STACK_LAYERS = 262144, 64, 48
MULTI_TOKENS = 4

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_T32768.txt")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_B256.txt")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_ops_prefill_T32768.txt")
CSRC = os.path.join(ROOT, "linear_attention_sequence_delta_amd", "csrc")
CHUNKED_SRC = os.path.join(CSRC, "gdn_chunked.hip")
RECURRENT_SRC = os.path.join(CSRC, "gdn_recurrent.hip")


def _sha(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _profile_value(path, key, src=CHUNKED_SRC):
    """A per-launch figure from a committed counter summary, or None when it is
    missing or the kernels changed since the counters were taken."""
    try:
        kv = {}
        for line in open(path):
            if "=" in line and not line.startswith("#"):
                k, val = line.split("=", 1)
                kv[k.strip()] = val.strip()
        if kv.get("source_sha256_16") != _sha(src):
            return None
        return float(kv[key])
    except (OSError, KeyError, ValueError):
        return None


def _traffic_bytes():
    return _profile_value(TRAFFIC_FILE, "hbm_bytes_per_prefill")


def _decode_traffic_bytes():
    return _profile_value(DECODE_TRAFFIC_FILE, "hbm_bytes_per_decode_step", RECURRENT_SRC)


def _issued_mfma_flops():
    return _profile_value(MFMA_FILE, "bf16_mfma_flop_per_prefill")


def _digests(**arrays):
    """SHA-256 (first 16 hex digits) of each host input array's bytes."""
    import numpy as np
    return {k: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
            for k, a in arrays.items()}


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def run_gpu(steps, warmup, path="both"):
    import numpy as np
    import torch
    import linear_attention_sequence_delta_amd as gdn
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a):
        import numpy as np
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    # ---------------- prefill workload (inputs resident before timing)
    p = synth.workload_prefill_32k(T_PREFILL)
    x, w = to_dev(p.x), to_dev(p.w)
    g, beta = to_dev(p.g), to_dev(p.beta)
    o = torch.empty((p.T, H_V, D), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((1, H_V, D, D), dtype=torch.float32, device=dev)
    res = {"numpy": np.__version__,
           "digests": {"prefill_T32768": _digests(x=p.x, w=p.w, g=p.g, beta=p.beta)}}

    if path in ("both", "fused"):
        wsr = torch.empty(gdn.gdn_prefill_raw_workspace_size(1, p.T, H_QK, H_V),
                          dtype=torch.uint8, device=dev)

        def fused():
            gdn.gdn_prefill_raw(x, w, g, beta, None, None, H_qk=H_QK, H_v=H_V,
                                final_state=fs, o=o, workspace=wsr)

        for _ in range(warmup):
            fused()
        torch.cuda.synchronize()
        ev = [_events(torch) for _ in range(steps)]
        t0 = time.perf_counter()
        for a0, a1 in ev:
            a0.record()
            fused()
            a1.record()
        torch.cuda.synchronize()
        res["wall_fused"] = (time.perf_counter() - t0) / steps * 1e6
        res["fused_us"] = sum(a0.elapsed_time(a1) for a0, a1 in ev) / steps * 1e3
        del wsr

    if path in ("both", "unfused"):
        q = torch.empty((p.T, H_QK, D), dtype=torch.bfloat16, device=dev)
        k = torch.empty_like(q)
        v = torch.empty((p.T, H_V, D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(gdn.gdn_prefill_workspace_size(gdn.GDN_BF16, 1, p.T, H_QK, H_V),
                         dtype=torch.uint8, device=dev)

        def prelude():
            gdn.gdn_conv_prelude(x, w, None, H_qk=H_QK, H_v=H_V, out=(q, k, v))

        def prefill():
            gdn.gdn_prefill(q, k, v, g, beta, None, None, final_state=fs, o=o, workspace=ws)

        for _ in range(warmup):
            prelude()
            prefill()
        torch.cuda.synchronize()
        ev = [(_events(torch), _events(torch)) for _ in range(steps)]
        for (a0, a1), (b0, b1) in ev:
            a0.record()
            prelude()
            a1.record()
            b0.record()
            prefill()
            b1.record()
        torch.cuda.synchronize()
        res["pre_us"] = sum(a0.elapsed_time(a1) for (a0, a1), _ in ev) / steps * 1e3
        res["pf_us"] = sum(b0.elapsed_time(b1) for _, (b0, b1) in ev) / steps * 1e3
        del q, k, v, ws

    # the backward of the prefill (training step's layer gradient), on the same
    # workload's q, k, v (from the prelude, untimed), d_o ~ N(0, 1) bf16, no
    # initial state and no final-state gradient
    if path == "both":
        q = torch.empty((p.T, H_QK, D), dtype=torch.bfloat16, device=dev)
        k = torch.empty_like(q)
        v = torch.empty((p.T, H_V, D), dtype=torch.bfloat16, device=dev)
        gdn.gdn_conv_prelude(x, w, None, H_qk=H_QK, H_v=H_V, out=(q, k, v))
        genb = torch.Generator(device=dev)
        genb.manual_seed(1003002)
        d_o = torch.randn(v.shape, generator=genb, device=dev).to(torch.bfloat16)
        wsb = torch.empty(gdn.gdn_prefill_backward_workspace_size(1, p.T, H_QK, H_V),
                          dtype=torch.uint8, device=dev)

        def backward():
            gdn.gdn_prefill_backward(q, k, v, g, beta, d_o, workspace=wsb)

        for _ in range(max(warmup, 1)):
            backward()
        torch.cuda.synchronize()
        bsteps = max(steps // 2, 3)
        b0, b1 = _events(torch)
        b0.record()
        for _ in range(bsteps):
            backward()
        b1.record()
        torch.cuda.synchronize()
        res["bwd_us"] = b0.elapsed_time(b1) / bsteps * 1e3
        # a training pair: the forward keeps the chunk states (from the raw
        # projections, prelude fused), the backward reads them
        del wsb
        cs = torch.empty(gdn.gdn_chunk_states_size(1, p.T, H_V) // 2, dtype=torch.bfloat16, device=dev)
        wsf = torch.empty(gdn.gdn_prefill_raw_workspace_size(1, p.T, H_QK, H_V), dtype=torch.uint8,
                          device=dev)
        wss = torch.empty(gdn.gdn_prefill_backward_saved_workspace_size(1, p.T, H_QK, H_V),
                          dtype=torch.uint8, device=dev)

        def fwd_keep():
            gdn.gdn_prefill_raw(x, w, g, beta, None, None, H_qk=H_QK, H_v=H_V, final_state=fs, o=o,
                                workspace=wsf, chunk_states=cs)

        def bwd_saved():
            gdn.gdn_prefill_backward(q, k, v, g, beta, d_o, workspace=wss, chunk_states=cs)

        for _ in range(max(warmup, 1)):
            fwd_keep()
            bwd_saved()
        torch.cuda.synchronize()
        ev = [(_events(torch), _events(torch)) for _ in range(bsteps)]
        for (a0, a1), (c0, c1) in ev:
            a0.record()
            fwd_keep()
            a1.record()
            c0.record()
            bwd_saved()
            c1.record()
        torch.cuda.synchronize()
        res["fwd_keep_us"] = sum(a0.elapsed_time(a1) for (a0, a1), _ in ev) / bsteps * 1e3
        res["bwd_saved_us"] = sum(c0.elapsed_time(c1) for _, (c0, c1) in ev) / bsteps * 1e3
        del q, k, v, cs, wsf, wss
        # the whole layer's backward from the raw projections
        A_log = to_dev(p.meta["A_log"].astype(np.float32))
        dtb = to_dev(p.meta["dt_bias"].astype(np.float32))
        ra, rb = to_dev(p.meta["a"]), to_dev(p.meta["b"])
        wsl = torch.empty(gdn.gdn_layer_prefill_backward_workspace_size(1, p.T, H_QK, H_V),
                          dtype=torch.uint8, device=dev)

        def layer_backward():
            gdn.gdn_layer_prefill_backward(x, w, ra, rb, A_log, dtb, d_o, H_qk=H_QK, H_v=H_V,
                                           workspace=wsl)

        layer_backward()
        torch.cuda.synchronize()
        b0.record()
        for _ in range(bsteps):
            layer_backward()
        b1.record()
        torch.cuda.synchronize()
        res["layer_bwd_us"] = b0.elapsed_time(b1) / bsteps * 1e3
        del d_o, wsl

    # the output gate on the prefill's o (z ~ N(0, 1), norm weight ~ U(0.5, 1.5))
    gen = torch.Generator(device=dev)
    gen.manual_seed(1003001)
    z = torch.randn(o.shape, generator=gen, device=dev).to(torch.bfloat16)
    wn = torch.rand((D,), generator=gen, device=dev) + 0.5
    y = torch.empty_like(o)
    for _ in range(2):
        gdn.gdn_gated_norm(o, z, wn, out=y)
    torch.cuda.synchronize()
    g0, g1 = _events(torch)
    g0.record()
    for _ in range(steps):
        gdn.gdn_gated_norm(o, z, wn, out=y)
    g1.record()
    torch.cuda.synchronize()
    res["gate_us"] = g0.elapsed_time(g1) / steps * 1e3
    # its backward (dy ~ N(0, 1))
    gy = torch.randn(o.shape, generator=gen, device=dev).to(torch.bfloat16)
    gws = torch.empty(max(int(gdn.lib().gdn_gated_norm_backward_workspace_size(o.numel() // D, D)), 1),
                      dtype=torch.uint8, device=dev)
    for _ in range(2):
        gdn.gdn_gated_norm_backward(o, z, wn, gy, workspace=gws)
    torch.cuda.synchronize()
    g0.record()
    for _ in range(steps):
        gdn.gdn_gated_norm_backward(o, z, wn, gy, workspace=gws)
    g1.record()
    torch.cuda.synchronize()
    res["gate_bwd_us"] = g0.elapsed_time(g1) / steps * 1e3
    del y, gy, gws

    # the layer's prefill with the output gate: one gdn_layer_prefill_gated
    # call (gates, fused prelude + prefill, gate applied in the scan's
    # stores) against gdn_layer_prefill followed by gdn_gated_norm
    if path in ("both", "fused"):
        la, lb = to_dev(p.meta["a"]), to_dev(p.meta["b"])
        lA = to_dev(p.meta["A_log"].astype(np.float32))
        ldt = to_dev(p.meta["dt_bias"].astype(np.float32))
        yg = torch.empty_like(o)
        wsg = torch.empty(gdn.gdn_layer_prefill_gated_workspace_size(1, p.T, H_QK, H_V),
                          dtype=torch.uint8, device=dev)
        wsl = torch.empty(gdn.gdn_layer_prefill_workspace_size(1, p.T, H_QK, H_V),
                          dtype=torch.uint8, device=dev)

        def gated():
            gdn.gdn_layer_prefill_gated(x, w, la, lb, lA, ldt, z, wn, None, None, H_qk=H_QK,
                                        H_v=H_V, final_state=fs, conv_state=False, o=o, y=yg,
                                        workspace=wsg)

        def separate():
            gdn.gdn_layer_prefill(x, w, la, lb, lA, ldt, None, None, H_qk=H_QK, H_v=H_V,
                                  final_state=fs, conv_state=False, o=o, workspace=wsl)
            gdn.gdn_gated_norm(o, z, wn, out=yg)

        for key, fn in (("layer_gated_us", gated), ("layer_separate_us", separate)):
            for _ in range(max(warmup // 4, 2)):
                fn()
            torch.cuda.synchronize()
            g0.record()
            for _ in range(steps):
                fn()
            g1.record()
            torch.cuda.synchronize()
            res[key] = g0.elapsed_time(g1) / steps * 1e3
        del yg, wsg, wsl
    del z

    # the packed varlen workload (8 sequences, lengths U{512..16384}, initial
    # states): the same fused call over several independent sequences
    if path == "both":
        pv = synth.workload_varlen()
        xv, wv = to_dev(pv.x), to_dev(pv.w)
        gv, bv, S0v, cuv = to_dev(pv.g), to_dev(pv.beta), to_dev(pv.S0), to_dev(pv.cu_seqlens)
        ov = torch.empty((pv.T, H_V, D), dtype=torch.bfloat16, device=dev)
        fsv = torch.empty((pv.N, H_V, D, D), dtype=torch.float32, device=dev)
        wsv = torch.empty(gdn.gdn_prefill_raw_workspace_size(pv.N, pv.T, H_QK, H_V),
                          dtype=torch.uint8, device=dev)

        def varlen():
            gdn.gdn_prefill_raw(xv, wv, gv, bv, S0v, cuv, H_qk=H_QK, H_v=H_V, final_state=fsv,
                                o=ov, workspace=wsv)

        for _ in range(max(warmup, 1)):
            varlen()
        torch.cuda.synchronize()
        g0.record()
        for _ in range(steps):
            varlen()
        g1.record()
        torch.cuda.synchronize()
        res["varlen_us"] = g0.elapsed_time(g1) / steps * 1e3
        res["varlen_T"] = pv.T
        res["varlen_lengths"] = [int(x) for x in np.diff(pv.cu_seqlens)]
        res["digests"]["prefill_varlen_8seq"] = _digests(x=pv.x, w=pv.w, g=pv.g, beta=pv.beta,
                                                         S0=pv.S0, cu_seqlens=pv.cu_seqlens)
        del xv, wv, gv, bv, S0v, cuv, ov, fsv, wsv

    # ---------------- decode workload: B = 256 over rotating 256-slot pools
    d = synth.decode_inputs(1005, B=B_DECODE, P=B_DECODE)
    res["digests"]["decode_B256"] = _digests(q=d.q, k=d.k, v=d.v, g=d.g, beta=d.beta,
                                             pool=d.pool, slot_idx=d.slot_idx)
    pools = [to_dev(d.pool) for _ in range(2)]     # 768 MiB each, larger than the on-die cache
    dq, dk, dv_, dg, db = (to_dev(a) for a in (d.q, d.k, d.v, d.g, d.beta))
    slots = to_dev(d.slot_idx)
    od = torch.empty((B_DECODE, H_V, D), dtype=torch.bfloat16, device=dev)
    del x, o
    dsteps = max(steps * 4, 8)
    for i in range(max(warmup, 2)):
        gdn.gdn_decode_step(dq, dk, dv_, dg, db, pools[i % 2], slots, o=od)
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record()
    for i in range(dsteps):
        gdn.gdn_decode_step(dq, dk, dv_, dg, db, pools[i % 2], slots, o=od)
    e1.record()
    torch.cuda.synchronize()
    dec_us = e0.elapsed_time(e1) / dsteps * 1e3

    res["dec_us"] = dec_us
    del pools

    # the same step from raw projections (conv history in a slot pool, gates
    # from raw a, b): gdn_layer_decode_step, pools rotated the same way
    ld = synth.layer_decode_inputs(1005, B=B_DECODE, P=B_DECODE)
    lpools = [to_dev(ld.pool) for _ in range(2)]
    cpools = [to_dev(ld.conv_pool) for _ in range(2)]
    lx, lw, la, lb, lA, ldt, lsl = (to_dev(a) for a in (ld.x, ld.w, ld.a, ld.b, ld.A_log,
                                                         ld.dt_bias, ld.slot_idx))
    for i in range(max(warmup, 2)):
        gdn.gdn_layer_decode_step(lx, lw, la, lb, lA, ldt, cpools[i % 2], lpools[i % 2], lsl, o=od)
    torch.cuda.synchronize()
    e0.record()
    for i in range(dsteps):
        gdn.gdn_layer_decode_step(lx, lw, la, lb, lA, ldt, cpools[i % 2], lpools[i % 2], lsl, o=od)
    e1.record()
    torch.cuda.synchronize()
    res["layer_dec_us"] = e0.elapsed_time(e1) / dsteps * 1e3
    del lpools, cpools

    # 4 tokens per sequence in one call (speculative verification), B = 256,
    # with and without the per-token state snapshots
    n_mt = MULTI_TOKENS
    mq, mk, mv, mg, mb = (to_dev(np.repeat(a[:, None], n_mt, axis=1))
                          for a in (d.q, d.k, d.v, d.g, d.beta))
    mo = torch.empty((B_DECODE, n_mt, H_V, D), dtype=torch.bfloat16, device=dev)
    mpools = [to_dev(d.pool) for _ in range(2)]
    snaps = torch.empty((B_DECODE, n_mt, H_V, D, D), dtype=torch.float32, device=dev)
    for key, sn in (("multi_us", None), ("multi_snap_us", snaps)):
        for i in range(2):
            gdn.gdn_decode_multi_step(mq, mk, mv, mg, mb, mpools[i % 2], slots, o=mo, snapshots=sn)
        torch.cuda.synchronize()
        e0.record()
        for i in range(dsteps):
            gdn.gdn_decode_multi_step(mq, mk, mv, mg, mb, mpools[i % 2], slots, o=mo, snapshots=sn)
        e1.record()
        torch.cuda.synchronize()
        res[key] = e0.elapsed_time(e1) / dsteps * 1e3
    return res


def run_longctx():
    """T = 262144 prelude + prefill, then 64 decode steps of 256 sequences that
    all continue from its final state, then a 48-layer decode stack."""
    import numpy as np
    import torch
    import linear_attention_sequence_delta_amd as gdn
    import synth

    dev = torch.device("cuda:0")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    p = synth.workload_longctx_prefill(T_LONG)
    x, w, g, beta = to_dev(p.x), to_dev(p.w), to_dev(p.g), to_dev(p.beta)
    del p.x
    o = torch.empty((T_LONG, H_V, D), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((1, H_V, D, D), dtype=torch.float32, device=dev)
    e0, e1 = _events(torch)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3

    q = torch.empty((T_LONG, H_QK, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((T_LONG, H_V, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(gdn.gdn_prefill_workspace_size(gdn.GDN_BF16, 1, T_LONG, H_QK, H_V),
                     dtype=torch.uint8, device=dev)

    def two_calls():
        gdn.gdn_conv_prelude(x, w, None, H_qk=H_QK, H_v=H_V, out=(q, k, v))
        gdn.gdn_prefill(q, k, v, g, beta, None, None, final_state=fs, o=o, workspace=ws)

    unfused_us = timed(two_calls)
    del q, k, v, ws
    wsr = torch.empty(gdn.gdn_prefill_raw_workspace_size(1, T_LONG, H_QK, H_V),
                      dtype=torch.uint8, device=dev)
    pre_us = timed(lambda: gdn.gdn_prefill_raw(x, w, g, beta, None, None, H_qk=H_QK, H_v=H_V,
                                               final_state=fs, o=o, workspace=wsr))
    del x, o, wsr

    # hand-off: 256 sequences continue from the prefill's final state
    pool = fs[0].unsqueeze(0).expand(B_DECODE, -1, -1, -1).contiguous()
    steps = []
    slot = None
    for st in range(LONG_STEPS):
        d = synth.workload_longctx_decode(st, B=B_DECODE, pool=np.zeros((1,), np.float32),
                                          slot_idx=slot, A_log=p.meta["A_log"],
                                          dt_bias=p.meta["dt_bias"])
        slot = d.slot_idx
        steps.append(tuple(to_dev(a) for a in (d.q, d.k, d.v, d.g, d.beta)))
    slot_d = to_dev(slot)
    od = torch.empty((B_DECODE, H_V, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    e0.record()
    for (dq, dk, dv_, dg, db) in steps:
        gdn.gdn_decode_step(dq, dk, dv_, dg, db, pool, slot_d, o=od)
    e1.record()
    torch.cuda.synchronize()
    dec_us = e0.elapsed_time(e1) * 1e3 / LONG_STEPS
    del pool, steps

    # 48 independently seeded layers, one decode step each per token.  Pools
    # (768 MiB each) and per-layer inputs are drawn on the GPU from seeded
    # generators (layer l: seed 1005000 + l); rows of q and k are normalised.
    gen = torch.Generator(device=dev)
    layers = []
    for l in range(STACK_LAYERS):
        gen.manual_seed(1005000 + l)
        lp = torch.randn((B_DECODE, H_V, D, D), generator=gen, device=dev) * 0.02
        lq = torch.nn.functional.normalize(
            torch.randn((B_DECODE, H_QK, D), generator=gen, device=dev), dim=-1).to(torch.bfloat16)
        lk = torch.nn.functional.normalize(
            torch.randn((B_DECODE, H_QK, D), generator=gen, device=dev), dim=-1).to(torch.bfloat16)
        lv = torch.randn((B_DECODE, H_V, D), generator=gen, device=dev).to(torch.bfloat16)
        lg = -torch.rand((B_DECODE, H_V), generator=gen, device=dev) * 0.5
        lb = torch.sigmoid(torch.randn((B_DECODE, H_V), generator=gen, device=dev))
        layers.append((lq, lk, lv, lg, lb, lp))
    slots = torch.arange(B_DECODE, dtype=torch.int32, device=dev)
    for (lq, lk, lv, lg, lb, lp) in layers:
        gdn.gdn_decode_step(lq, lk, lv, lg, lb, lp, slots, o=od)
    torch.cuda.synchronize()
    tokens = 3
    e0.record()
    for _ in range(tokens):
        for (lq, lk, lv, lg, lb, lp) in layers:
            gdn.gdn_decode_step(lq, lk, lv, lg, lb, lp, slots, o=od)
    e1.record()
    torch.cuda.synchronize()
    stack_ms = e0.elapsed_time(e1) / tokens
    return {"prefill": {"T": T_LONG, "us": pre_us, "tokens_per_s": T_LONG / (pre_us * 1e-6),
                        "what": "conv prelude fused into the chunked prefill (gdn_prefill_raw), "
                                "one 262144-token sequence",
                        "two_calls_us": unfused_us},
            "decode": {"B": B_DECODE, "steps": LONG_STEPS, "us_per_step": dec_us,
                       "tokens_per_s": B_DECODE / (dec_us * 1e-6),
                       "what": "256 sequences continuing from the prefill's final state"},
            "stack48": {"layers": STACK_LAYERS, "ms_per_token": stack_ms,
                        "tokens_per_s": B_DECODE / (stack_ms * 1e-3),
                        "what": "48 independently seeded layers, one B = 256 decode step each",
                        "inputs": "timing only: each layer's pool, q, k, v and gates drawn on the "
                                  "GPU by torch.Generator (seed 1005000 + layer), outside the "
                                  "host-side seeded recipe; results are not compared"}}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline():
    """The fp64 oracle on the host's cores, on the same synthetic workloads:
    the 32768-token prefill (prelude + token recurrence, all 48 V-heads), the
    packed 8-sequence prefill, and one decode step at B = 64 (128-slot pool)
    and at B = 256 (256-slot pool).  The headline value is the first; every
    figure is whole-workload (no sampling beyond what "sample" says)."""
    import numpy as np
    import oracle
    import synth
    oracle._load()
    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or len(os.sched_getaffinity(0))

    def prefill_rate(p):
        t0 = time.perf_counter()
        qo, ko, vo = oracle.prelude(p.x, p.w, p.cu_seqlens, H_qk=H_QK, H_v=H_V, dk=D, dv=D)
        oracle.recurrent(qo, ko, vo, p.g, p.beta, p.S0, p.cu_seqlens)
        dt = time.perf_counter() - t0
        return p.T / dt, dt

    def decode_rate(d):
        t0 = time.perf_counter()
        oracle.decode_step(d.q, d.k, d.v, d.g, d.beta, d.pool, d.slot_idx)
        dt = time.perf_counter() - t0
        return d.B / dt, dt

    p3 = synth.workload_prefill_32k(T_PREFILL)
    v3, t3 = prefill_rate(p3)
    del p3
    p4 = synth.workload_varlen()
    v4, t4 = prefill_rate(p4)
    T4 = p4.T
    del p4
    d2 = synth.workload_decode_b64()
    v2, t2 = decode_rate(d2)
    del d2
    d5 = synth.decode_inputs(1005, B=B_DECODE, P=B_DECODE)
    v5, t5 = decode_rate(d5)
    del d5
    return {"value": v3, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"fp64 oracle, whole workloads: prelude + token-by-token recurrence over "
                      f"all {T_PREFILL} prefill tokens and all {H_V} V-heads ({t3:.1f} s; "
                      f"prelude OpenMP over tokens, recurrence OpenMP over heads)",
            "configs": {
                "prefill_T32768": {"tokens_per_s": v3, "s": t3},
                "prefill_varlen_8seq": {"tokens_per_s": v4, "s": t4, "tokens": T4,
                                        "what": "packed 8-sequence prefill with initial states"},
                "decode_B64": {"tokens_per_s": v2, "s": t2,
                               "what": "one decode step, 64 sequences, 128-slot pool"},
                "decode_B256": {"tokens_per_s": v5, "s": t5,
                                "what": "one decode step, 256 sequences, 256-slot pool (the "
                                        "long-context hand-off's decode shape; its 262144-token "
                                        "prefill runs at the 32768-token prefill's per-token "
                                        "rate, the oracle's cost being linear in tokens)"}}}


def copy_rate_gbps(nbytes=1 << 30, reps=20):
    """HBM rate of a plain device copy (torch copy_, nbytes read and nbytes
    written per copy), timed with HIP events after warm-up copies."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / t / 1e9


def copy_calibration(nbytes):
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "note": "each copy reads and writes copy_bytes"}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-longctx", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--path", choices=("both", "fused", "unfused"), default="both")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the layer shards by "
              "sequence and head with no exchange, so the per-GPU figure is the one-GPU run.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import linear_attention_sequence_delta_amd as gdn
    if not os.path.exists(gdn.LIB_PATH):
        from linear_attention_sequence_delta_amd import build as _b
        _b.build()

    r = run_gpu(args.steps, args.warmup, args.path)
    T = T_PREFILL
    fused = "fused_us" in r
    # the timed step and the call the roofline is for
    step_us = r["fused_us"] if fused else r["pre_us"] + r["pf_us"]
    call_us = r["fused_us"] if fused else r["pf_us"]
    flops = PREFILL_FLOP_PER_TOKEN * T
    achieved_tflops = flops / (call_us * 1e-6) / 1e12
    traffic = _traffic_bytes() if fused else None
    issued = _issued_mfma_flops() if fused else None
    pre_bytes = PRELUDE_BYTES_PER_TOKEN * T
    dec_bytes = DECODE_BYTES_PER_SEQ * B_DECODE
    dec_traffic = _decode_traffic_bytes()
    phases = {}
    if fused:
        phases["fused_call"] = r["fused_us"]
        phases["fused_wall_per_call"] = r["wall_fused"]
    if "pre_us" in r:
        phases.update({"prelude": r["pre_us"], "prefill": r["pf_us"],
                       "two_calls": r["pre_us"] + r["pf_us"]})
    out = {
        "metric": "GDN layer tokens/s (prefill T=32K; decode B=256) + % of MFMA/HBM roofline",
        "value": T / (step_us * 1e-6),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_us / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic, seeded: raw projections N(0,1) bf16, conv weights N(0,0.5) bf16, "
                "gates from A_log, dt_bias ~ U(-1,1) and a, b ~ N(0,1)",
        "data_digests": r["digests"],
        "numpy": r["numpy"],
        "config": {"workload": "prefill of one 32768-token sequence from raw bf16 projections "
                               "(conv prelude + chunked prefill), 16 QK / 48 V heads, d=128, "
                               "chunk 64, fp32 state",
                   "T": T, "H_qk": H_QK, "H_v": H_V, "d_k": D, "d_v": D, "chunk": CHUNK,
                   "entry": "gdn_prefill_raw" if fused else "gdn_conv_prelude + gdn_prefill"},
        "roofline": {"bound": "mfma", "achieved": achieved_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved_tflops / PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "kernel": ("gdn_prefill_raw (plan + prep + scan kernels, prelude fused)"
                                if fused else "gdn_prefill (plan + prep + scan kernels)"),
                     "algorithmic_flop_per_launch": flops,
                     "issued_mfma_flop_per_launch": issued,
                     "issued_frac": (None if issued is None else
                                     issued / (call_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS)},
        "phases_us": phases,
        "decode": {"value": B_DECODE / (r["dec_us"] * 1e-6), "unit": "tokens/s",
                   "us_per_step": r["dec_us"],
                   "workload": "one decode step of 256 sequences, 16 QK / 48 V heads, fp32 "
                               "states in a 256-slot pool (pools rotated, 768 MiB each)",
                   "roofline": {"bound": "hbm",
                                "achieved": dec_bytes / (r["dec_us"] * 1e-6) / 1e9,
                                "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                "frac": dec_bytes / (r["dec_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                                "algorithmic_bytes_per_step": dec_bytes,
                                "traffic": dec_traffic,
                                "traffic_frac": (None if dec_traffic is None else
                                                 dec_traffic / (r["dec_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS)},
                   "multi_token": {
                       "tokens_per_call": MULTI_TOKENS,
                       "us_per_call": r["multi_us"],
                       "tokens_per_s": B_DECODE * MULTI_TOKENS / (r["multi_us"] * 1e-6),
                       "us_per_call_with_snapshots": r["multi_snap_us"],
                       "what": "gdn_decode_multi_step: 4 tokens per sequence in one pass over "
                               "the state (speculative verification); with snapshots it also "
                               "writes the state before each token for rollback"},
                   "from_raw_projections": {
                       "us_per_step": r["layer_dec_us"],
                       "tokens_per_s": B_DECODE / (r["layer_dec_us"] * 1e-6),
                       "what": "gdn_layer_decode_step: conv from each slot's 3-row history + the "
                               "new raw row, gates from raw a, b, the update, history shift"}},
    }
    cps = copy_rate_gbps()
    out["hbm_copy"] = {"GB/s": cps, "frac": cps / PEAK_HBM_GBPS,
                       "what": "torch copy_ of a 1 GiB device buffer (reads and writes in equal "
                               "parts, the mix of the decode step and the prelude): context for "
                               "their HBM fractions, not a step"}
    gate_bytes = 3 * T * H_V * D * 2
    gate_bwd_bytes = 5 * T * H_V * D * 2     # o, z, dy in; d_o, dz out
    out["output_gate"] = {"us": r["gate_us"], "what": "gdn_gated_norm on the prefill's o "
                          "(RMS norm per head, norm weight, SiLU(z)); not part of the step",
                          "roofline": {"bound": "hbm", "achieved": gate_bytes / (r["gate_us"] * 1e-6) / 1e9,
                                       "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                       "frac": gate_bytes / (r["gate_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS},
                          "backward": {"us": r["gate_bwd_us"],
                                       "what": "gdn_gated_norm_backward (d_o, dz, dw)",
                                       "roofline": {"bound": "hbm",
                                                    "achieved": gate_bwd_bytes / (r["gate_bwd_us"] * 1e-6) / 1e9,
                                                    "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                                    "frac": gate_bwd_bytes / (r["gate_bwd_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS}}}
    if "layer_gated_us" in r:
        out["layer_step_gated"] = {
            "us": r["layer_gated_us"], "tokens_per_s": T / (r["layer_gated_us"] * 1e-6),
            "separate_us": r["layer_separate_us"],
            "mfma_frac": PREFILL_FLOP_PER_TOKEN * T / (r["layer_gated_us"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
            "what": "gdn_layer_prefill_gated: gates from raw a, b, the prelude fused into the chunked "
                    "prefill, and the output gate (RMS norm x weight x SiLU(z)) applied inside the "
                    "scan as rows of o complete, one call; separate_us: gdn_layer_prefill then "
                    "gdn_gated_norm"}
    if "bwd_us" in r:
        bflops = BACKWARD_FLOP_PER_TOKEN * T
        btf = bflops / (r["bwd_us"] * 1e-6) / 1e12
        out["backward"] = {"us": r["bwd_us"], "tokens_per_s": T / (r["bwd_us"] * 1e-6),
                           "what": "gdn_prefill_backward on the prefill workload's q, k, v "
                                   "(d_o ~ N(0,1), no initial state): dq, dk, dv, dg, dbeta; "
                                   "not part of the step",
                           "roofline": {"bound": "mfma", "achieved": btf,
                                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                        "frac": btf / PEAK_BF16_TFLOPS,
                                        "algorithmic_flop_per_launch": bflops},
                           "layer": {"us": r["layer_bwd_us"],
                                     "tokens_per_s": T / (r["layer_bwd_us"] * 1e-6),
                                     "what": "gdn_layer_prefill_backward from the raw projections "
                                             "(gates and prelude recomputed, the recurrence's "
                                             "gradients, then through the prelude and gates): "
                                             "dx, dconv_w, da, db, dA_log, ddt_bias"},
                           "from_kept_states": {
                               "forward_us": r["fwd_keep_us"], "backward_us": r["bwd_saved_us"],
                               "pair_us": r["fwd_keep_us"] + r["bwd_saved_us"],
                               "pair_tokens_per_s": T / ((r["fwd_keep_us"] + r["bwd_saved_us"]) * 1e-6),
                               "what": "a training pair: gdn_prefill_raw keeping the chunk states, "
                                       "then gdn_prefill_backward reading them (the forward scan "
                                       "is not repeated)"}}
    if "varlen_us" in r:
        vf = PREFILL_FLOP_PER_TOKEN * r["varlen_T"]
        out["varlen_8seq"] = {"us": r["varlen_us"], "tokens": r["varlen_T"],
                              "lengths": r["varlen_lengths"],
                              "tokens_per_s": r["varlen_T"] / (r["varlen_us"] * 1e-6),
                              "mfma_frac": vf / (r["varlen_us"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                              "what": "gdn_prefill_raw on the packed 8-sequence workload (initial "
                                      "states); not part of the step"}
    if "pre_us" in r:
        out["prelude_roofline"] = {"bound": "hbm", "kernel": "gdn_conv_prelude (two-call path)",
                                   "achieved": pre_bytes / (r["pre_us"] * 1e-6) / 1e9,
                                   "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                   "frac": pre_bytes / (r["pre_us"] * 1e-6) / 1e9 / PEAK_HBM_GBPS}
    if not args.no_longctx:
        out["longctx"] = run_longctx()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
