"""fp64 CPU oracle of the Gated DeltaNet layer (ctypes wrapper over gdn_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does, and
this package imports nothing from it.  It shares no code with the HIP path.

Every array handed to the C oracle is converted here to float64.  bf16 inputs
arrive as ``numpy.uint16`` bit patterns and are widened exactly (a bf16 value
is the top half of an IEEE float32).

What each function computes, and the page passages it follows, is documented
in ``gdn_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
             "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.orc_prelude.argtypes = [P, P, P, I, I, I, I, I, I, D, P, P, P]
    lib.orc_recurrent.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, D, P, P, I, I]
    lib.orc_chunked.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, D, I, P, P, I, I]
    lib.orc_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, D, P]
    lib.orc_gates.argtypes = [P, P, P, P, I, I, P, P]
    lib.orc_gated_norm.argtypes = [P, P, P, I, I, D, P]
    lib.orc_recurrent_backward.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, D, P, P, P, P,
                                           P, P, P, P, I, I]
    lib.orc_prelude_backward.argtypes = [P, P, P, I, I, I, I, I, I, D, P, P, P, P, P]
    lib.orc_gates_backward.argtypes = [P, P, P, P, I, I, P, P, P, P, P, P]
    lib.orc_gated_norm_backward.argtypes = [P, P, P, I, I, D, P, P, P, P]
    for f in (lib.orc_prelude, lib.orc_recurrent, lib.orc_chunked, lib.orc_decode_step,
              lib.orc_gates, lib.orc_gated_norm, lib.orc_recurrent_backward,
              lib.orc_prelude_backward, lib.orc_gates_backward, lib.orc_gated_norm_backward):
        f.restype = I
    _lib = lib
    return lib


def f64(a) -> np.ndarray:
    """Widen an input array to contiguous float64 (uint16 arrays are bf16 bits)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        a = (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _cu(cu_seqlens, T):
    if cu_seqlens is None:
        return None, 1
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    if cu.ndim != 1 or cu.size < 2 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must be a non-decreasing int32 vector from 0 to T")
    return cu, cu.size - 1


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed with code {rc}")


def _with_history(x, cu_seqlens, conv_state_in):
    """Each sequence's three history rows placed before its first row: the
    extended rows, their sequence offsets, and the indices of the original rows
    in the extended layout."""
    T, C = x.shape
    cu, N = _cu(cu_seqlens, T)
    hist = f64(conv_state_in)
    if hist.shape != (N, 3, C):
        raise ValueError("conv_state_in must be [N, 3, C_raw]")
    bounds = [(0, T)] if cu is None else [(int(cu[n]), int(cu[n + 1])) for n in range(N)]
    rows, keep, cu_ext = [], [], [0]
    for n, (s0, s1) in enumerate(bounds):
        keep.append(np.arange(cu_ext[-1] + 3, cu_ext[-1] + 3 + s1 - s0))
        rows += [hist[n], x[s0:s1]]
        cu_ext.append(cu_ext[-1] + 3 + s1 - s0)
    return np.concatenate(rows), np.asarray(cu_ext, dtype=np.int32), np.concatenate(keep)


def prelude(x, w, cu_seqlens=None, *, H_qk, H_v, dk, dv, eps=1e-6, conv_state_in=None):
    """Causal conv (width 4) -> SiLU -> L2 norm of q, k.  Returns fp64 (q, k, v).

    The conv window of a sequence's first rows reaches back three rows before
    its start: zeros, or the rows conv_state_in [N, 3, C_raw] (oldest first)
    holds for it, as the raw rows a previous part of the same sequence ended
    with.  Those rows are placed before the sequence and their outputs dropped."""
    x = f64(x)
    w = f64(w)
    T, Craw = x.shape
    if Craw != 2 * H_qk * dk + H_v * dv or w.shape != (Craw, 4):
        raise ValueError("prelude shape mismatch")
    if conv_state_in is not None:
        xe, cue, keep = _with_history(x, cu_seqlens, conv_state_in)
        q, k, v = prelude(xe, w, cue, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, eps=eps)
        return q[keep], k[keep], v[keep]
    cu, N = _cu(cu_seqlens, T)
    q = np.zeros((T, H_qk, dk))
    k = np.zeros((T, H_qk, dk))
    v = np.zeros((T, H_v, dv))
    rc = _load().orc_prelude(_ptr(x), _ptr(w), _ptr(cu), N, T, H_qk, H_v, dk, dv, eps,
                             _ptr(q), _ptr(k), _ptr(v))
    _check(rc, "prelude")
    return q, k, v


def prelude_backward(x, w, dq, dk, dv, cu_seqlens=None, *, H_qk, H_v, eps=1e-6):
    """Gradients of ``prelude`` with respect to x [T, C_raw] and w [C_raw, 4],
    given dq, dk [T, H_qk, dk] and dv [T, H_v, dv].  Returns fp64 (dx, dw)."""
    x, w, dq, dk, dv = (f64(a) for a in (x, w, dq, dk, dv))
    T, Craw = x.shape
    d_k, d_v = dq.shape[2], dv.shape[2]
    if Craw != 2 * H_qk * d_k + H_v * d_v or w.shape != (Craw, 4) or dk.shape != dq.shape:
        raise ValueError("prelude_backward shape mismatch")
    cu, N = _cu(cu_seqlens, T)
    dx = np.zeros((T, Craw))
    dw = np.zeros((Craw, 4))
    _check(_load().orc_prelude_backward(_ptr(x), _ptr(w), _ptr(cu), N, T, H_qk, H_v, d_k, d_v,
                                        float(eps), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dx),
                                        _ptr(dw)), "prelude_backward")
    return dx, dw


def gates_backward(a, b, A_log, dt_bias, dg, dbeta):
    """Gradients of ``gates`` with respect to a, b [T, H_v] and A_log, dt_bias
    [H_v], given dg, dbeta [T, H_v].  Returns fp64 (da, db, dA_log, ddt_bias)."""
    a, b, A_log, dt_bias, dg, dbeta = (f64(x) for x in (a, b, A_log, dt_bias, dg, dbeta))
    T, H_v = a.shape
    if b.shape != (T, H_v) or dg.shape != (T, H_v) or dbeta.shape != (T, H_v):
        raise ValueError("gates_backward shape mismatch")
    da, db = np.zeros((T, H_v)), np.zeros((T, H_v))
    dA, ddt = np.zeros(H_v), np.zeros(H_v)
    _check(_load().orc_gates_backward(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), T, H_v,
                                      _ptr(dg), _ptr(dbeta), _ptr(da), _ptr(db), _ptr(dA),
                                      _ptr(ddt)), "gates_backward")
    return da, db, dA, ddt


def _prefill_args(q, k, v, g, beta, initial_state, cu_seqlens):
    q, k, v, g, beta = (f64(a) for a in (q, k, v, g, beta))
    T, H_qk, dk = q.shape
    _, H_v, dv = v.shape
    if k.shape != q.shape or v.shape[0] != T or g.shape != (T, H_v) or beta.shape != (T, H_v):
        raise ValueError("prefill shape mismatch")
    cu, N = _cu(cu_seqlens, T)
    S0 = None if initial_state is None else f64(initial_state)
    if S0 is not None and S0.shape != (N, H_v, dv, dk):
        raise ValueError("initial_state shape mismatch")
    return q, k, v, g, beta, S0, cu, N, T, H_qk, H_v, dk, dv


def recurrent(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0, heads=None):
    """Token-by-token gated delta rule.  Returns fp64 (o [T,H_v,dv], S [N,H_v,dv,dk]).

    ``heads`` = (h_lo, h_hi) restricts the work to those V-heads; the other
    entries of the results are zero.
    """
    q, k, v, g, beta, S0, cu, N, T, H_qk, H_v, dk, dv = _prefill_args(
        q, k, v, g, beta, initial_state, cu_seqlens)
    h_lo, h_hi = (0, H_v) if heads is None else heads
    o = np.zeros((T, H_v, dv))
    S = np.zeros((N, H_v, dv, dk))
    rc = _load().orc_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                               _ptr(cu), N, T, H_qk, H_v, dk, dv, float(scale), _ptr(o),
                               _ptr(S), h_lo, h_hi)
    _check(rc, "recurrent")
    return o, S


def recurrent_backward(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None,
                       cu_seqlens=None, scale=1.0, qk_heads=None):
    """Gradients of ``recurrent`` by reverse mode through the token steps.

    d_o [T, H_v, dv] is the gradient with respect to o, d_final_state
    [N, H_v, dv, dk] (or None = zero) the one with respect to the final states.
    Returns fp64 (dq, dk, dv, dg, dbeta, dS0) with the shapes of q, k, v, g,
    beta and the initial states [N, H_v, dv, dk].  ``qk_heads`` = (lo, hi)
    restricts the work to those QK heads and their V-heads (other entries
    zero)."""
    q, k, v, g, beta, S0, cu, N, T, H_qk, H_v, dk, dv = _prefill_args(
        q, k, v, g, beta, initial_state, cu_seqlens)
    d_o = f64(d_o)
    if d_o.shape != v.shape:
        raise ValueError("d_o shape mismatch")
    dSf = None if d_final_state is None else f64(d_final_state)
    if dSf is not None and dSf.shape != (N, H_v, dv, dk):
        raise ValueError("d_final_state shape mismatch")
    dq, dkk = np.zeros(q.shape), np.zeros(k.shape)
    dvv = np.zeros(v.shape)
    dg, db = np.zeros(g.shape), np.zeros(beta.shape)
    dS0 = np.zeros((N, H_v, dv, dk))
    lo, hi = (0, H_qk) if qk_heads is None else qk_heads
    rc = _load().orc_recurrent_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(S0), _ptr(cu), N, T, H_qk, H_v, dk, dv,
                                        float(scale), _ptr(d_o), _ptr(dSf), _ptr(dq), _ptr(dkk),
                                        _ptr(dvv), _ptr(dg), _ptr(db), _ptr(dS0), int(lo),
                                        int(hi))
    _check(rc, "recurrent_backward")
    return dq, dkk, dvv, dg, db, dS0


def chunked(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0, chunk=64,
            heads=None):
    """Chunked (WY/UT) form of the same recurrence; same results up to rounding."""
    q, k, v, g, beta, S0, cu, N, T, H_qk, H_v, dk, dv = _prefill_args(
        q, k, v, g, beta, initial_state, cu_seqlens)
    h_lo, h_hi = (0, H_v) if heads is None else heads
    o = np.zeros((T, H_v, dv))
    S = np.zeros((N, H_v, dv, dk))
    rc = _load().orc_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                             _ptr(cu), N, T, H_qk, H_v, dk, dv, float(scale), int(chunk),
                             _ptr(o), _ptr(S), h_lo, h_hi)
    _check(rc, "chunked")
    return o, S


def decode_step(q, k, v, g, beta, pool, slot_idx, scale=1.0):
    """One token per sequence on pool[slot_idx[b]].  Returns (o, new pool) in fp64.

    The input pool is not modified; the returned pool is a float64 copy with the
    addressed slots advanced by one token.
    """
    q, k, v, g, beta = (f64(a) for a in (q, k, v, g, beta))
    B, H_qk, dk = q.shape
    _, H_v, dv = v.shape
    pool = f64(pool).copy()
    P = pool.shape[0]
    if pool.shape != (P, H_v, dv, dk) or g.shape != (B, H_v) or beta.shape != (B, H_v):
        raise ValueError("decode shape mismatch")
    slots = np.ascontiguousarray(slot_idx, dtype=np.int32)
    if slots.shape != (B,):
        raise ValueError("slot_idx shape mismatch")
    o = np.zeros((B, H_v, dv))
    rc = _load().orc_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(pool),
                                 _ptr(slots), B, P, H_qk, H_v, dk, dv, float(scale), _ptr(o))
    _check(rc, "decode_step")
    return o, pool


def gates(a, b, A_log, dt_bias):
    """g = -softplus(a + dt_bias) * exp(A_log), beta = sigmoid(b), per token and
    V-head.  a, b [T, H_v]; A_log, dt_bias [H_v].  Returns fp64 (g, beta)."""
    a, b, A_log, dt_bias = (f64(x) for x in (a, b, A_log, dt_bias))
    T, H_v = a.shape
    if b.shape != (T, H_v) or A_log.shape != (H_v,) or dt_bias.shape != (H_v,):
        raise ValueError("gates shape mismatch")
    g = np.zeros((T, H_v))
    beta = np.zeros((T, H_v))
    _check(_load().orc_gates(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), T, H_v, _ptr(g),
                             _ptr(beta)), "gates")
    return g, beta


def conv_state(x, cu_seqlens=None, conv_state_in=None):
    """The conv history a sequence leaves for its next token: its last three raw
    rows, oldest first ([N, 3, C_raw], same dtype as x).  Where the sequence has
    fewer than three rows the rest comes from the rows before its start: zeros,
    or the end of its conv_state_in history [N, 3, C_raw]."""
    x = np.asarray(x)
    T = x.shape[0]
    cu, N = _cu(cu_seqlens, T)
    bounds = [(0, T)] if cu is None else [(int(cu[n]), int(cu[n + 1])) for n in range(N)]
    out = np.zeros((N, 3, x.shape[1]), dtype=x.dtype)
    for n, (s0, s1) in enumerate(bounds):
        for j in range(3):
            t = s1 - 3 + j
            if t >= s0:
                out[n, j] = x[t]
            elif conv_state_in is not None:
                out[n, j] = np.asarray(conv_state_in)[n, 3 + t - s0]
    return out


def decode_step_raw(x, w, conv_state_pool, a, b, A_log, dt_bias, pool, slot_idx, *, H_qk, H_v,
                    dk, dv, eps=1e-6, scale=1.0):
    """One token per sequence from the raw projections x [B, C_raw]: the conv
    window of sequence b is the three raw rows kept in conv_state_pool[slot]
    followed by x[b]; conv, SiLU and L2 norm as in ``prelude``; gates as in
    ``gates``; then ``decode_step``.  Returns (o, new conv-state pool, new
    state pool); the new conv state of an addressed slot is its rows 1, 2 and
    x[b] (same dtype as the pool given), the inputs are not modified."""
    slots = np.ascontiguousarray(slot_idx, dtype=np.int32)
    cs = np.asarray(conv_state_pool)
    x = np.asarray(x)
    B, C = x.shape
    if cs.shape[1:] != (3, C) or slots.shape != (B,):
        raise ValueError("decode_step_raw shape mismatch")
    # each window is its own 4-row sequence; only its last row's outputs are used
    win = np.concatenate([f64(cs[slots]), f64(x)[:, None, :]], axis=1).reshape(4 * B, C)
    cu = np.arange(0, 4 * B + 1, 4, dtype=np.int32)
    q, k, v = prelude(win, w, cu, H_qk=H_qk, H_v=H_v, dk=dk, dv=dv, eps=eps)
    g, beta = gates(a, b, A_log, dt_bias)
    o, new_pool = decode_step(q[3::4], k[3::4], v[3::4], g, beta, pool, slots, scale)
    new_cs = cs.copy()
    new_cs[slots] = np.concatenate([cs[slots][:, 1:], x[:, None, :]], axis=1)
    return o, new_cs, new_pool


def decode_multi_step(q, k, v, g, beta, pool, slot_idx, scale=1.0):
    """n tokens per sequence in order (speculative-decoding verification):
    q, k [B, n, H_qk, dk]; v [B, n, H_v, dv]; g, beta [B, n, H_v].  Token j of
    sequence b is ``decode_step`` applied to slot slot_idx[b] after tokens
    0..j-1.  Returns (o [B, n, H_v, dv], snapshots [B, n, H_v, dv, dk] with
    snapshots[b, j] the slot's state before token j, new pool) in fp64."""
    q, k, v, g, beta = (f64(a) for a in (q, k, v, g, beta))
    B, n = q.shape[:2]
    pool = f64(pool).copy()
    slots = np.ascontiguousarray(slot_idx, dtype=np.int32)
    o = np.zeros((B, n) + v.shape[2:])
    snaps = np.zeros((B, n) + pool.shape[1:])
    for j in range(n):
        snaps[:, j] = pool[slots]
        o[:, j], pool = decode_step(q[:, j], k[:, j], v[:, j], g[:, j], beta[:, j], pool, slots,
                                    scale)
    return o, snaps, pool


def state_rollback(snapshots, n_keep, pool, slot_idx):
    """Keep the first n_keep[b] of sequence b's n verified tokens: its slot
    takes snapshots[b, n_keep[b]] (the state after n_keep[b] tokens) when
    n_keep[b] < n, and is left as it is when n_keep[b] == n.  Returns the new
    pool (a copy, same dtype)."""
    pool = np.array(pool, copy=True)
    snaps = np.asarray(snapshots)
    n = snaps.shape[1]
    for b, s in enumerate(np.asarray(slot_idx)):
        if n_keep[b] < n:
            pool[s] = snaps[b, n_keep[b]]
    return pool


def gated_norm(o, z, w, eps=1e-6):
    """Output gate: o / sqrt(mean(o^2) + eps) * w * SiLU(z) over the last axis
    (d_v) of o and z; w [d_v].  Returns fp64 with o's shape."""
    o, z, w = f64(o), f64(z), f64(w)
    if o.shape != z.shape or w.shape != (o.shape[-1],):
        raise ValueError("gated_norm shape mismatch")
    dv = o.shape[-1]
    R = o.size // dv
    y = np.zeros(o.shape)
    _check(_load().orc_gated_norm(_ptr(np.ascontiguousarray(o)), _ptr(np.ascontiguousarray(z)),
                                  _ptr(w), R, dv, float(eps), _ptr(y)), "gated_norm")
    return y


def gated_norm_backward(o, z, w, dy, eps=1e-6):
    """Gradients of ``gated_norm`` with respect to o, z (shape of o) and w [d_v],
    given dy (shape of o).  Returns fp64 (d_o, dz, dw)."""
    o, z, w, dy = f64(o), f64(z), f64(w), f64(dy)
    if o.shape != z.shape or dy.shape != o.shape or w.shape != (o.shape[-1],):
        raise ValueError("gated_norm_backward shape mismatch")
    dv = o.shape[-1]
    R = o.size // dv
    d_o, dz, dw = np.zeros(o.shape), np.zeros(o.shape), np.zeros(dv)
    _check(_load().orc_gated_norm_backward(
        _ptr(np.ascontiguousarray(o)), _ptr(np.ascontiguousarray(z)), _ptr(w), R, dv, float(eps),
        _ptr(np.ascontiguousarray(dy)), _ptr(d_o), _ptr(dz), _ptr(dw)), "gated_norm_backward")
    return d_o, dz, dw
