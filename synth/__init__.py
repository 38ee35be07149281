"""Seeded synthetic inputs for the Gated DeltaNet layer workloads.

This module only draws random numbers and shapes them into inputs; it holds
none of the layer's arithmetic (no conv, no recurrence, no normalisation of
layer outputs).  Both the HIP path's tests/benchmark and the fp64 oracle take
their inputs from here, and nothing else is shared between them.

Recipe (the same for every workload):
  * ``numpy.random.SeedSequence(seed).spawn(n)`` gives one PCG64 generator per
    tensor, in the order each generator lists them;
  * ``N(0, s)`` means a normal with standard deviation ``s``;
  * bf16 tensors are float32 draws rounded to nearest-even and returned as
    ``numpy.uint16`` bit patterns; float32 tensors are returned as float32;
  * raw projections [T, C] are drawn one stream per 128-channel block: block b
    (channels 128 b .. 128 b + 127) takes child b of the tensor's seed and is
    filled with float32 normals in row-major order (blocks drawn in parallel).

Gate recipe of the gated workloads (the decay gate is handed to the layer as
its logarithm g, the write strength as beta):
    g    = -softplus(a + dt_bias[h]) * exp(A_log[h]),   a ~ N(0, 1)
    beta = sigmoid(b),                                   b ~ N(0, 1)
with A_log, dt_bias ~ U(-1, 1) per V-head -- evaluated in float64 and rounded
to float32.  The names A_log and dt_bias are the layer's weight names on the
page "从参数竞赛到效率革命：拆解 Qwen3.8-27B 的稠密架构与长上下文混合注意力", sec. 2.1.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Layer shape of the linear-attention layers ("拆解 Qwen3.8-27B ..." sec. 2.1):
H_QK = 16
H_V = 48
D_K = 128
D_V = 128
CONV_W = 4


def c_raw(H_qk: int = H_QK, H_v: int = H_V, dk: int = D_K, dv: int = D_V) -> int:
    """Raw projection width: [q heads | k heads | v heads]."""
    return 2 * H_qk * dk + H_v * dv


# ---------------------------------------------------------------- bf16 bits
def bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bit patterns (round to nearest even; inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rngs(seed, n):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _unit_rows(z):
    """Rows of z scaled to unit length (input recipe: 'then L2-normalised per token')."""
    z = np.asarray(z, dtype=np.float64)
    return z / np.sqrt(np.sum(z * z, axis=-1, keepdims=True))


def _gates(rng_a, rng_b, A_log, dt_bias, T):
    """The workloads' gate recipe: raw a, b ~ N(0, 1) per token and V-head, then
    g = -softplus(a + dt_bias) exp(A_log), beta = sigmoid(b) in fp64, stored
    fp32.  Returns (g, beta, a, b); a, b as fp32 (what a layer kernel that
    forms the gates itself is given)."""
    a = rng_a.standard_normal((T, A_log.size))
    b = rng_b.standard_normal((T, A_log.size))
    sp = np.log1p(np.exp(a + dt_bias[None, :]))
    g = -sp * np.exp(A_log[None, :])
    beta = 1.0 / (1.0 + np.exp(-b))
    return g.astype(np.float32), beta.astype(np.float32), a.astype(np.float32), b.astype(np.float32)


def _raw_bf16(seq, T, C, block: int = 128):
    """[T, C] bf16 bits ~ N(0, 1): channel block b (``block`` channels) is drawn
    from its own PCG64 stream, child b of ``seq``, as float32 normals in
    row-major order.  Blocks are independent, so they are drawn in parallel."""
    out = np.empty((T, C), dtype=np.uint16)
    nb = (C + block - 1) // block
    kids = seq.spawn(nb)

    def fill(b):
        c0, c1 = b * block, min(C, (b + 1) * block)
        r = np.random.Generator(np.random.PCG64(kids[b]))
        out[:, c0:c1] = bf16_bits(r.standard_normal((T, c1 - c0), dtype=np.float32))

    with ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        list(ex.map(fill, range(nb)))
    return out


# ---------------------------------------------------------------- workloads
@dataclass
class Prefill:
    """Host inputs of one prefill call (all numpy)."""
    T: int
    N: int
    H_qk: int
    H_v: int
    dk: int
    dv: int
    io: str                      # "f32" or "bf16"
    g: np.ndarray                # [T, H_v] f32 log-decay
    beta: np.ndarray             # [T, H_v] f32
    q: Optional[np.ndarray] = None   # [T, H_qk, dk]  (bf16 bits or f32)
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None   # [T, H_v, dv]
    x: Optional[np.ndarray] = None   # [T, C_raw] bf16 bits (raw projections)
    w: Optional[np.ndarray] = None   # [C_raw, 4] bf16 bits (conv weights)
    S0: Optional[np.ndarray] = None  # [N, H_v, dv, dk] f32
    cu_seqlens: Optional[np.ndarray] = None  # [N+1] int32
    meta: dict = field(default_factory=dict)


@dataclass
class Decode:
    """Host inputs of one decode step over a state-slot pool."""
    B: int
    P: int
    H_qk: int
    H_v: int
    dk: int
    dv: int
    q: np.ndarray                # [B, H_qk, dk] bf16 bits
    k: np.ndarray
    v: np.ndarray                # [B, H_v, dv] bf16 bits
    g: np.ndarray                # [B, H_v] f32
    beta: np.ndarray             # [B, H_v] f32
    pool: np.ndarray             # [P, H_v, dv, dk] f32 (unused slots: NaN canary)
    slot_idx: np.ndarray         # [B] int32, distinct
    meta: dict = field(default_factory=dict)


CANARY_BITS = np.uint32(0x7FC0DEAD)  # a quiet NaN with a recognisable payload


def tiny_recurrence(seed: int = 1001, T: int = 128, H_qk: int = 1, H_v: int = 3,
                    dk: int = D_K, dv: int = D_V) -> Prefill:
    """Tiny fp32 recurrence: unit q, k; v ~ N(0,1); beta = sigmoid(N(0,1));
    g = -U(0.01, 0.5); zero initial state.  Generators: q, k, v, b, g."""
    rq, rk, rv, rb, rg = _rngs(seed, 5)
    q = _unit_rows(rq.standard_normal((T, H_qk, dk))).astype(np.float32)
    k = _unit_rows(rk.standard_normal((T, H_qk, dk))).astype(np.float32)
    v = rv.standard_normal((T, H_v, dv)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rb.standard_normal((T, H_v))))).astype(np.float32)
    g = (-rg.uniform(0.01, 0.5, (T, H_v))).astype(np.float32)
    return Prefill(T=T, N=1, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, io="f32", g=g, beta=beta,
                   q=q, k=k, v=v, meta={"seed": seed, "recipe": "tiny_recurrence"})


def varlen_lengths(seed: int = 1004, n: int = 8, lo: int = 512, hi: int = 16384,
                   total_max: int = 65536, chunk: int = 64) -> np.ndarray:
    """n lengths ~ U{lo..hi}, all redrawn until the sum is <= total_max and at
    least one length is not a multiple of the chunk."""
    rng = _rngs((seed, 0xC0), 1)[0]
    while True:
        L = rng.integers(lo, hi + 1, size=n)
        if L.sum() <= total_max and np.any(L % chunk != 0):
            return L.astype(np.int64)


def raw_prefill(seed: int, T: Optional[int] = None, lengths=None, H_qk: int = H_QK,
                H_v: int = H_V, dk: int = D_K, dv: int = D_V, init_state: bool = False,
                state_std: float = 0.02) -> Prefill:
    """Prefill from raw projections: x ~ N(0,1) bf16 [T, C_raw]; conv weights
    ~ N(0, 0.5) bf16; gates per the module recipe; optional initial states
    ~ N(0, state_std).  Streams: x (one child stream per 128-channel block), w,
    a, b, A_log, dt_bias, S0."""
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        T = int(lengths.sum())
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        N = len(lengths)
    else:
        cu, N = None, 1
    seqs = np.random.SeedSequence(seed).spawn(7)
    rw, ra, rb, rA, rd, rs = [np.random.Generator(np.random.PCG64(q)) for q in seqs[1:]]
    C = c_raw(H_qk, H_v, dk, dv)
    x = _raw_bf16(seqs[0], T, C)
    w = bf16_bits(rw.normal(0.0, 0.5, (C, CONV_W)).astype(np.float32))
    A_log = rA.uniform(-1.0, 1.0, H_v)
    dt_bias = rd.uniform(-1.0, 1.0, H_v)
    g, beta, a, b = _gates(ra, rb, A_log, dt_bias, T)
    S0 = None
    if init_state:
        S0 = rs.normal(0.0, state_std, (N, H_v, dv, dk)).astype(np.float32)
    return Prefill(T=T, N=N, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, io="bf16", g=g, beta=beta,
                   x=x, w=w, S0=S0, cu_seqlens=cu,
                   meta={"seed": seed, "recipe": "raw_prefill", "A_log": A_log,
                         "dt_bias": dt_bias, "a": a, "b": b})


def direct_prefill(seed: int, T: Optional[int] = None, lengths=None, H_qk: int = H_QK,
                   H_v: int = H_V, dk: int = D_K, dv: int = D_V, io: str = "bf16",
                   init_state: bool = False, state_std: float = 0.02,
                   g_range: Optional[tuple] = None) -> Prefill:
    """Prefill from post-prelude inputs: unit q, k and v ~ N(0,1) (bf16 bits or
    f32); gates per the module recipe, or g = -U(g_range) when given.
    Generators: q, k, v, a, b, A_log, dt_bias, S0."""
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        T = int(lengths.sum())
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        N = len(lengths)
    else:
        cu, N = None, 1
    rq, rk, rv, ra, rb, rA, rd, rs = _rngs(seed, 8)
    q = _unit_rows(rq.standard_normal((T, H_qk, dk))).astype(np.float32)
    k = _unit_rows(rk.standard_normal((T, H_qk, dk))).astype(np.float32)
    v = rv.standard_normal((T, H_v, dv), dtype=np.float32)
    if io == "bf16":
        q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    A_log = rA.uniform(-1.0, 1.0, H_v)
    dt_bias = rd.uniform(-1.0, 1.0, H_v)
    g, beta, _, _ = _gates(ra, rb, A_log, dt_bias, T)
    if g_range is not None:
        g = (-ra.uniform(g_range[0], g_range[1], (T, H_v))).astype(np.float32)
    S0 = None
    if init_state:
        S0 = rs.normal(0.0, state_std, (N, H_v, dv, dk)).astype(np.float32)
    return Prefill(T=T, N=N, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, io=io, g=g, beta=beta,
                   q=q, k=k, v=v, S0=S0, cu_seqlens=cu,
                   meta={"seed": seed, "recipe": "direct_prefill"})


def output_grads(seed: int, T: int, N: int, H_v: int = H_V, dk: int = D_K, dv: int = D_V,
                 state_std: float = 0.02):
    """Gradients handed to a prefill's backward: d_o ~ N(0, 1) as bf16 bits
    [T, H_v, dv] and d_final_state ~ N(0, state_std) fp32 [N, H_v, dv, dk].
    Generators: d_o, d_final_state."""
    ro, rs = _rngs((seed, 0xB0), 2)
    d_o = bf16_bits(ro.standard_normal((T, H_v, dv), dtype=np.float32))
    dSf = rs.normal(0.0, state_std, (N, H_v, dv, dk)).astype(np.float32)
    return d_o, dSf


def decode_inputs(seed: int, B: int, P: Optional[int] = None, H_qk: int = H_QK,
                  H_v: int = H_V, dk: int = D_K, dv: int = D_V, state_std: float = 0.02,
                  pool: Optional[np.ndarray] = None, slot_idx=None, A_log=None,
                  dt_bias=None) -> Decode:
    """One decode step: unit q, k (bf16), v ~ N(0,1) (bf16), gates per the module
    recipe, a pool of P slots whose B addressed slots hold N(0, state_std) states
    and whose other slots hold a NaN canary; slot_idx = the first B entries of a
    seeded permutation of 0..P-1.  A given ``pool``/``slot_idx`` is used as is,
    and a given ``A_log``/``dt_bias`` (the layer's weights) replaces the drawn ones.
    Generators: q, k, v, a, b, A_log, dt_bias, perm, states."""
    P = P if P is not None else (pool.shape[0] if pool is not None else 2 * B)
    rq, rk, rv, ra, rb, rA, rd, rp, rs = _rngs(seed, 9)
    q = bf16_bits(_unit_rows(rq.standard_normal((B, H_qk, dk))).astype(np.float32))
    k = bf16_bits(_unit_rows(rk.standard_normal((B, H_qk, dk))).astype(np.float32))
    v = bf16_bits(rv.standard_normal((B, H_v, dv), dtype=np.float32))
    A_draw = rA.uniform(-1.0, 1.0, H_v)
    dt_draw = rd.uniform(-1.0, 1.0, H_v)
    A_log = A_draw if A_log is None else np.asarray(A_log, dtype=np.float64)
    dt_bias = dt_draw if dt_bias is None else np.asarray(dt_bias, dtype=np.float64)
    g, beta, a, b = _gates(ra, rb, A_log, dt_bias, B)
    if slot_idx is None:
        slot_idx = rp.permutation(P)[:B].astype(np.int32)
    slot_idx = np.ascontiguousarray(slot_idx, dtype=np.int32)
    if pool is None:
        pool = np.empty((P, H_v, dv, dk), dtype=np.float32)
        pool.view(np.uint32)[...] = CANARY_BITS
        for b in range(B):
            pool[slot_idx[b]] = rs.normal(0.0, state_std, (H_v, dv, dk)).astype(np.float32)
    return Decode(B=B, P=P, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, q=q, k=k, v=v, g=g, beta=beta,
                  pool=pool, slot_idx=slot_idx,
                  meta={"seed": seed, "recipe": "decode_inputs", "A_log": A_log,
                        "dt_bias": dt_bias, "a": a, "b": b})


# bf16 canary (a quiet NaN) for conv-state slots a call must not touch
CONV_CANARY_BITS = 0x7FC1


@dataclass
class LayerDecode:
    """Host inputs of one decode step from raw projections (all numpy)."""
    B: int
    P: int
    H_qk: int
    H_v: int
    dk: int
    dv: int
    x: np.ndarray          # [B, C_raw] bf16 bits, the new token's raw projections
    w: np.ndarray          # [C_raw, 4] bf16 bits, conv taps
    a: np.ndarray          # [B, H_v] fp32 raw gate projections
    b: np.ndarray          # [B, H_v] fp32
    A_log: np.ndarray      # [H_v] fp32
    dt_bias: np.ndarray    # [H_v] fp32
    conv_pool: np.ndarray  # [P, 3, C_raw] bf16 bits, the last three raw rows of each slot
    pool: np.ndarray       # [P, H_v, dv, dk] fp32 states
    slot_idx: np.ndarray   # [B] int32
    meta: dict = field(default_factory=dict)


def layer_decode_inputs(seed, B: int, P: Optional[int] = None, H_qk: int = H_QK, H_v: int = H_V,
                        dk: int = D_K, dv: int = D_V, state_std: float = 0.02, w=None,
                        A_log=None, dt_bias=None, conv_pool=None, pool=None,
                        slot_idx=None) -> LayerDecode:
    """One decode step from raw projections: x ~ N(0, 1) bf16; a, b ~ N(0, 1);
    conv taps ~ N(0, 0.5) bf16 and A_log, dt_bias ~ U(-1, 1) unless the layer's
    weights are given; the addressed slots of a fresh conv-state pool hold
    N(0, 1) bf16 rows and of a fresh state pool N(0, state_std) states, the
    other slots a NaN canary; slot_idx = the first B entries of a seeded
    permutation.  Given pools / slot_idx are used as they are.
    Generators: x, w, a, b, A_log, dt_bias, perm, conv rows, states."""
    rx, rw, ra, rb, rA, rd, rp, rc, rs = _rngs(seed, 9)
    C = c_raw(H_qk, H_v, dk, dv)
    P = P if P is not None else (pool.shape[0] if pool is not None else 2 * B)
    x = bf16_bits(rx.standard_normal((B, C), dtype=np.float32))
    w_draw = bf16_bits(rw.normal(0.0, 0.5, (C, CONV_W)).astype(np.float32))
    w = w_draw if w is None else w
    A_draw = rA.uniform(-1.0, 1.0, H_v)
    dt_draw = rd.uniform(-1.0, 1.0, H_v)
    A_log = (A_draw if A_log is None else np.asarray(A_log, dtype=np.float64)).astype(np.float32)
    dt_bias = (dt_draw if dt_bias is None else np.asarray(dt_bias, dtype=np.float64)).astype(np.float32)
    a = ra.standard_normal((B, H_v)).astype(np.float32)
    b = rb.standard_normal((B, H_v)).astype(np.float32)
    if slot_idx is None:
        slot_idx = rp.permutation(P)[:B].astype(np.int32)
    slot_idx = np.ascontiguousarray(slot_idx, dtype=np.int32)
    if conv_pool is None:
        conv_pool = np.full((P, 3, C), CONV_CANARY_BITS, dtype=np.uint16)
        for i in range(B):
            conv_pool[slot_idx[i]] = bf16_bits(rc.standard_normal((3, C), dtype=np.float32))
    if pool is None:
        pool = np.empty((P, H_v, dv, dk), dtype=np.float32)
        pool.view(np.uint32)[...] = CANARY_BITS
        for i in range(B):
            pool[slot_idx[i]] = rs.normal(0.0, state_std, (H_v, dv, dk)).astype(np.float32)
    return LayerDecode(B=B, P=P, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, x=x, w=w, a=a, b=b,
                       A_log=A_log, dt_bias=dt_bias, conv_pool=conv_pool, pool=pool,
                       slot_idx=slot_idx, meta={"seed": seed, "recipe": "layer_decode_inputs"})


# ------------------------------------------------- the five named workloads
WORKLOADS = {
    "tiny_recurrence_T128": "B=1, T=128, 1 QK head / 3 V heads, d=128, all fp32",
    "decode_B64": "one decode step, B=64, 16 QK / 48 V heads, pool of 128 slots",
    "prefill_T32768": "B=1, T=32768 from raw bf16 projections, 16 QK / 48 V heads",
    "varlen_8seq": "8 packed sequences, lengths U{512..16384} (sum <= 65536), initial states",
    "longctx_T262144": "B=1, T=262144 prefill, then 256 sequences x 64 decode steps",
}


def workload_tiny():
    return tiny_recurrence(1001)


def workload_decode_b64():
    return decode_inputs(1002, B=64, P=128)


def workload_prefill_32k(T: int = 32768):
    return raw_prefill(1003, T=T)


def workload_varlen():
    return raw_prefill(1004, lengths=varlen_lengths(1004), init_state=True)


def workload_longctx_prefill(T: int = 262144):
    return raw_prefill(1005, T=T)


def workload_longctx_decode(step: int, B: int = 256, pool=None, slot_idx=None, A_log=None,
                            dt_bias=None):
    """Per-step decode inputs of the long-context hand-off: fresh q, k, v and gate
    draws per step; pass the prefill's A_log / dt_bias (its ``meta``) so that the
    steps use the same layer's gate weights."""
    return decode_inputs((1005, 1, step), B=B, P=B, pool=pool, slot_idx=slot_idx, A_log=A_log,
                         dt_bias=dt_bias)
