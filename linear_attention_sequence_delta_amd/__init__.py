"""MI355X (gfx950) Gated DeltaNet layer: thin Python binding over libgdn.so.

The functions here carry the names of the C entry points in include/gdn.h and
only marshal arguments: they check devices, dtypes and shapes of torch tensors,
allocate outputs with torch, and pass raw device pointers plus the current HIP
stream to the library.  Every step of the layer runs in the library's kernels;
there is no Python or CPU fallback -- if libgdn.so is missing or cannot be
loaded, every call raises.

Build the library with ``python -m linear_attention_sequence_delta_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARG = -1
GDN_ERR_UNSUPPORTED = -2
GDN_ERR_WORKSPACE = -3
GDN_ERR_HIP = -4
GDN_ERR_DEVICE_CHECK = -5
GDN_F32 = 0
GDN_BF16 = 1

EXPORTS = ("gdn_abi_version", "gdn_last_error", "gdn_conv_prelude",
           "gdn_prefill_workspace_size", "gdn_prefill", "gdn_prefill_raw_workspace_size",
           "gdn_prefill_raw", "gdn_prefill_backward_workspace_size", "gdn_prefill_backward",
           "gdn_layer_prefill_backward_workspace_size", "gdn_layer_prefill_backward",
           "gdn_gates", "gdn_layer_prefill_workspace_size",
           "gdn_layer_prefill", "gdn_layer_decode_step", "gdn_decode_multi_step",
           "gdn_state_rollback", "gdn_gated_norm", "gdn_gated_norm_backward_workspace_size",
           "gdn_gated_norm_backward", "gdn_decode_step", "gdn_chunk_states_size",
           "gdn_prefill_save_states", "gdn_prefill_raw_save_states",
           "gdn_prefill_backward_saved_workspace_size", "gdn_prefill_backward_saved",
           "gdn_layer_prefill_save_states", "gdn_layer_prefill_backward_saved_workspace_size",
           "gdn_layer_prefill_backward_saved", "gdn_prefill_no_alloc",
           "gdn_layer_prefill_gated_workspace_size", "gdn_layer_prefill_gated")

_lib = None


class GDNError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded libgdn.so with argument types set (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m linear_attention_sequence_delta_amd.build`")
    # torch first: its HIP runtime is then the one the process has loaded when
    # libgdn.so's dependencies are resolved (loading the library first would
    # bring in the system runtime ahead of torch's)
    _torch()
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.gdn_abi_version.argtypes = []
    L.gdn_abi_version.restype = I
    L.gdn_last_error.argtypes = []
    L.gdn_last_error.restype = ctypes.c_char_p
    L.gdn_conv_prelude.argtypes = [P, P, P, I, I, I, I, I, I, F, P, P, P, P]
    L.gdn_conv_prelude.restype = I
    L.gdn_prefill_workspace_size.argtypes = [I, I, I, I, I, I, I]
    L.gdn_prefill_workspace_size.restype = Z
    L.gdn_prefill.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, P, Z, P]
    L.gdn_prefill.restype = I
    L.gdn_prefill_no_alloc.argtypes = [I, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, P]
    L.gdn_prefill_no_alloc.restype = I
    L.gdn_prefill_raw_workspace_size.argtypes = [I, I, I, I, I, I]
    L.gdn_prefill_raw_workspace_size.restype = Z
    L.gdn_prefill_raw.argtypes = [P, P, F, P, P, P, P, P, I, I, I, I, I, I, F, P, P, Z, P]
    L.gdn_prefill_raw.restype = I
    L.gdn_prefill_backward_workspace_size.argtypes = [I, I, I, I, I, I]
    L.gdn_prefill_backward_workspace_size.restype = Z
    L.gdn_prefill_backward.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, P, P, P,
                                       P, P, P, Z, P]
    L.gdn_prefill_backward.restype = I
    L.gdn_layer_prefill_backward_workspace_size.argtypes = [I, I, I, I, I, I]
    L.gdn_layer_prefill_backward_workspace_size.restype = Z
    L.gdn_layer_prefill_backward.argtypes = [P, P, P, P, P, P, F, P, P, P, P, I, I, I, I, I, I, F,
                                             P, P, P, P, P, P, P, P, Z, P]
    L.gdn_layer_prefill_backward.restype = I
    L.gdn_gates.argtypes = [P, P, P, P, I, I, P, P, P]
    L.gdn_gates.restype = I
    L.gdn_layer_prefill_workspace_size.argtypes = [I, I, I, I, I, I]
    L.gdn_layer_prefill_workspace_size.restype = Z
    L.gdn_layer_prefill.argtypes = [P, P, P, P, P, P, F, P, P, P, P, P, I, I, I, I, I, I, F, P,
                                    P, Z, P]
    L.gdn_layer_prefill.restype = I
    L.gdn_layer_prefill_gated_workspace_size.argtypes = [I, I, I, I, I, I]
    L.gdn_layer_prefill_gated_workspace_size.restype = Z
    L.gdn_layer_prefill_gated.argtypes = [P, P, P, P, P, P, F, P, P, F, P, P, P, P, P, I, I, I, I, I,
                                          I, F, P, P, P, Z, P]
    L.gdn_layer_prefill_gated.restype = I
    L.gdn_layer_decode_step.argtypes = [P, P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, F, P, P]
    L.gdn_layer_decode_step.restype = I
    L.gdn_decode_multi_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, P]
    L.gdn_decode_multi_step.restype = I
    L.gdn_state_rollback.argtypes = [P, P, I, P, P, I, I, I, I, I, P]
    L.gdn_state_rollback.restype = I
    L.gdn_gated_norm.argtypes = [P, P, P, I, I, F, P, P]
    L.gdn_gated_norm.restype = I
    L.gdn_gated_norm_backward_workspace_size.argtypes = [I, I]
    L.gdn_gated_norm_backward_workspace_size.restype = Z
    L.gdn_gated_norm_backward.argtypes = [P, P, P, P, I, I, F, P, P, P, P, Z, P]
    L.gdn_gated_norm_backward.restype = I
    L.gdn_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, P]
    L.gdn_decode_step.restype = I
    L.gdn_chunk_states_size.argtypes = [I, I, I, I, I]
    L.gdn_chunk_states_size.restype = Z
    L.gdn_prefill_save_states.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, P, Z, P,
                                          Z, P]
    L.gdn_prefill_save_states.restype = I
    L.gdn_prefill_raw_save_states.argtypes = [P, P, F, P, P, P, P, P, I, I, I, I, I, I, F, P, P, Z,
                                              P, Z, P]
    L.gdn_prefill_raw_save_states.restype = I
    L.gdn_prefill_backward_saved_workspace_size.argtypes = [I, I, I, I, I, I]
    L.gdn_prefill_backward_saved_workspace_size.restype = Z
    L.gdn_prefill_backward_saved.argtypes = [P, P, P, P, P, P, Z, P, P, P, I, I, I, I, I, I, F, P,
                                             P, P, P, P, P, P, Z, P]
    L.gdn_prefill_backward_saved.restype = I
    L.gdn_layer_prefill_save_states.argtypes = [P, P, P, P, P, P, F, P, P, P, P, I, I, I, I, I, I,
                                                F, P, P, Z, P, Z, P]
    L.gdn_layer_prefill_save_states.restype = I
    L.gdn_layer_prefill_backward_saved_workspace_size.argtypes = [I, I, I, I, I, I]
    L.gdn_layer_prefill_backward_saved_workspace_size.restype = Z
    L.gdn_layer_prefill_backward_saved.argtypes = [P, P, P, P, P, P, F, P, Z, P, P, P, I, I, I, I,
                                                   I, I, F, P, P, P, P, P, P, P, P, Z, P]
    L.gdn_layer_prefill_backward_saved.restype = I
    _lib = L
    return L


def _check(rc: int, fn: str):
    if rc != GDN_OK:
        raise GDNError(rc, fn, lib().gdn_last_error().decode(errors="replace"))


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, device, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _device_of(t):
    if t.device.type != "cuda":
        raise ValueError("tensors must be on a HIP device (torch 'cuda')")
    return t.device


def gdn_abi_version() -> int:
    return lib().gdn_abi_version()


def gdn_conv_prelude(x, conv_w, cu_seqlens=None, *, H_qk: int = 16, H_v: int = 48,
                     d_k: int = 128, d_v: int = 128, l2_eps: float = 1e-6,
                     out: Optional[Tuple] = None):
    """Causal conv (width 4) + SiLU + q/k L2 norm.  x: bf16 [T, C_raw]; conv_w:
    bf16 [C_raw, 4]; cu_seqlens: int32 [N+1] or None.  Returns bf16 (q, k, v)."""
    torch = _torch()
    dev = _device_of(x)
    _need(x, "x", torch.bfloat16, dev, 2)
    _need(conv_w, "conv_w", torch.bfloat16, dev, 2)
    T = x.shape[0]
    N = 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.numel() - 1
    if out is None:
        q = torch.empty((T, H_qk, d_k), dtype=torch.bfloat16, device=dev)
        k = torch.empty((T, H_qk, d_k), dtype=torch.bfloat16, device=dev)
        v = torch.empty((T, H_v, d_v), dtype=torch.bfloat16, device=dev)
    else:
        q, k, v = out
        for name, t, shp in (("q", q, (T, H_qk, d_k)), ("k", k, (T, H_qk, d_k)),
                             ("v", v, (T, H_v, d_v))):
            _need(t, name, torch.bfloat16, dev)
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} must have shape {shp}")
    if x.shape[1] != 2 * H_qk * d_k + H_v * d_v or tuple(conv_w.shape) != (x.shape[1], 4):
        raise ValueError("x / conv_w shapes do not match the head configuration")
    rc = lib().gdn_conv_prelude(_ptr(x), _ptr(conv_w), _ptr(cu_seqlens), N, T, H_qk, H_v, d_k,
                                d_v, float(l2_eps), _ptr(q), _ptr(k), _ptr(v), _stream(dev))
    _check(rc, "gdn_conv_prelude")
    return q, k, v


def gdn_prefill_workspace_size(io_dtype: int, N: int, T: int, H_qk: int, H_v: int,
                               d_k: int = 128, d_v: int = 128) -> int:
    return int(lib().gdn_prefill_workspace_size(io_dtype, N, T, H_qk, H_v, d_k, d_v))


def gdn_chunk_states_size(N: int, T: int, H_v: int, d_k: int = 128, d_v: int = 128) -> int:
    """Bytes of the chunk-states buffer a training forward pass keeps."""
    return int(lib().gdn_chunk_states_size(N, T, H_v, d_k, d_v))


def _chunk_states_arg(chunk_states, N, T, H_v, d_k, d_v, dev):
    torch = _torch()
    need = gdn_chunk_states_size(N, T, H_v, d_k, d_v)
    if chunk_states is True:
        chunk_states = torch.empty(max(need, 2) // 2, dtype=torch.bfloat16, device=dev)
    _need(chunk_states, "chunk_states", torch.bfloat16, dev)
    nbytes = chunk_states.numel() * chunk_states.element_size()
    if nbytes < need:
        raise ValueError(f"chunk_states holds {nbytes} bytes, {need} needed")
    return chunk_states, nbytes


def gdn_prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *, scale: float = 1.0,
                final_state=True, o=None, workspace=None, chunk_states=None):
    """Prefill over packed sequences.  q, k: [T, H_qk, 128]; v: [T, H_v, 128], all
    bf16 (chunked matrix-core path) or all fp32 (token-by-token fp32 path); g,
    beta: fp32 [T, H_v]; initial_state: fp32 [N, H_v, 128, 128] or None.

    final_state: True (allocate and return it), False/None (skip it), or an fp32
    tensor to write (may be ``initial_state`` itself for an in-place hand-off).
    chunk_states (bf16 only): None, True (allocate) or a bf16 tensor of at least
    gdn_chunk_states_size bytes: the states at chunk starts are kept there for
    gdn_prefill_backward.  Returns (o, final_state or None), plus chunk_states
    when it is given."""
    torch = _torch()
    dev = _device_of(q)
    if q.dtype == torch.bfloat16:
        io, io_t = GDN_BF16, torch.bfloat16
    elif q.dtype == torch.float32:
        io, io_t = GDN_F32, torch.float32
    else:
        raise ValueError("q must be bfloat16 or float32")
    _need(q, "q", io_t, dev, 3)
    _need(k, "k", io_t, dev, 3)
    _need(v, "v", io_t, dev, 3)
    T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if tuple(k.shape) != (T, H_qk, d_k) or v.shape[0] != T:
        raise ValueError("q, k, v shapes disagree")
    _need(g, "g", torch.float32, dev, 2)
    _need(beta, "beta", torch.float32, dev, 2)
    if tuple(g.shape) != (T, H_v) or tuple(beta.shape) != (T, H_v):
        raise ValueError("g and beta must be [T, H_v]")
    N = 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.numel() - 1
    sshape = (N, H_v, d_v, d_k)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev, 4)
        if tuple(initial_state.shape) != sshape:
            raise ValueError(f"initial_state must be {sshape}")
    if final_state is True:
        fs = torch.empty(sshape, dtype=torch.float32, device=dev)
    elif final_state is None or final_state is False:
        fs = None
    else:
        fs = final_state
        _need(fs, "final_state", torch.float32, dev, 4)
        if tuple(fs.shape) != sshape:
            raise ValueError(f"final_state must be {sshape}")
    if o is None:
        o = torch.empty((T, H_v, d_v), dtype=io_t, device=dev)
    else:
        _need(o, "o", io_t, dev, 3)
        if tuple(o.shape) != (T, H_v, d_v):
            raise ValueError("o must be [T, H_v, d_v]")
    ws_need = gdn_prefill_workspace_size(io, N, T, H_qk, H_v, d_k, d_v)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if chunk_states is not None:
        if io != GDN_BF16:
            raise ValueError("chunk_states are kept by the bf16 prefill only")
        cs, cs_bytes = _chunk_states_arg(chunk_states, N, T, H_v, d_k, d_v, dev)
        rc = lib().gdn_prefill_save_states(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                           _ptr(initial_state), _ptr(fs), _ptr(cu_seqlens), N, T,
                                           H_qk, H_v, d_k, d_v, float(scale), _ptr(o), _ptr(cs),
                                           cs_bytes, _ptr(workspace), ws_bytes, _stream(dev))
        _check(rc, "gdn_prefill_save_states")
        return o, fs, cs
    rc = lib().gdn_prefill(io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(initial_state), _ptr(fs), _ptr(cu_seqlens), N, T, H_qk, H_v,
                           d_k, d_v, float(scale), _ptr(o), _ptr(workspace), ws_bytes,
                           _stream(dev))
    _check(rc, "gdn_prefill")
    return o, fs


def gdn_prefill_no_alloc(q, k, v, g, beta, o, initial_state=None, final_state=None,
                         cu_seqlens=None, *, scale: float = 1.0):
    """gdn_prefill with the workspace in the library's own scratch: allocates
    nothing (the caller passes o and, if wanted, final_state).  Same tensors as
    gdn_prefill; the bf16 path is limited to a workspace of 64 MiB."""
    torch = _torch()
    dev = _device_of(q)
    io = GDN_BF16 if q.dtype == torch.bfloat16 else GDN_F32
    io_t = torch.bfloat16 if io == GDN_BF16 else torch.float32
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _need(t, name, io_t, dev, 3)
    _need(g, "g", torch.float32, dev, 2)
    _need(beta, "beta", torch.float32, dev, 2)
    T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    for t, name in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _need(t, name, torch.float32, dev, 4)
    rc = lib().gdn_prefill_no_alloc(io, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(initial_state), _ptr(final_state), _ptr(cu_seqlens), N,
                                    T, H_qk, H_v, d_k, d_v, float(scale), _ptr(o), _stream(dev))
    _check(rc, "gdn_prefill_no_alloc")
    return o, final_state


def gdn_prefill_backward_workspace_size(N: int, T: int, H_qk: int, H_v: int, d_k: int = 128,
                                        d_v: int = 128) -> int:
    return int(lib().gdn_prefill_backward_workspace_size(N, T, H_qk, H_v, d_k, d_v))


def gdn_prefill_backward_saved_workspace_size(N: int, T: int, H_qk: int, H_v: int,
                                              d_k: int = 128, d_v: int = 128) -> int:
    return int(lib().gdn_prefill_backward_saved_workspace_size(N, T, H_qk, H_v, d_k, d_v))


def gdn_prefill_backward(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None,
                         cu_seqlens=None, *, scale: float = 1.0, d_initial_state=True,
                         workspace=None, chunk_states=None):
    """Gradients of the bf16 gdn_prefill.  q, k: bf16 [T, H_qk, 128]; v, d_o:
    bf16 [T, H_v, 128]; g, beta: fp32 [T, H_v]; initial_state, d_final_state:
    fp32 [N, H_v, 128, 128] or None.  d_initial_state: True (allocate and
    return it), False/None (skip it) or an fp32 tensor to write.
    chunk_states: the bf16 buffer a gdn_prefill / gdn_prefill_raw with
    chunk_states filled on the same inputs (then initial_state is not read and
    the forward states are not recomputed).  Returns (dq, dk, dv, dg, dbeta,
    d_initial_state or None)."""
    torch = _torch()
    dev = _device_of(q)
    for t, name in ((q, "q"), (k, "k"), (v, "v"), (d_o, "d_o")):
        _need(t, name, torch.bfloat16, dev, 3)
    T, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if tuple(k.shape) != (T, H_qk, d_k) or v.shape[0] != T or tuple(d_o.shape) != tuple(v.shape):
        raise ValueError("q, k, v, d_o shapes disagree")
    _need(g, "g", torch.float32, dev, 2)
    _need(beta, "beta", torch.float32, dev, 2)
    if tuple(g.shape) != (T, H_v) or tuple(beta.shape) != (T, H_v):
        raise ValueError("g and beta must be [T, H_v]")
    N = 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.numel() - 1
    sshape = (N, H_v, d_v, d_k)
    for t, name in ((initial_state, "initial_state"), (d_final_state, "d_final_state")):
        if t is not None:
            _need(t, name, torch.float32, dev, 4)
            if tuple(t.shape) != sshape:
                raise ValueError(f"{name} must be {sshape}")
    if d_initial_state is True:
        dS0 = torch.empty(sshape, dtype=torch.float32, device=dev)
    elif d_initial_state is None or d_initial_state is False:
        dS0 = None
    else:
        dS0 = d_initial_state
        _need(dS0, "d_initial_state", torch.float32, dev, 4)
        if tuple(dS0.shape) != sshape:
            raise ValueError(f"d_initial_state must be {sshape}")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = torch.empty_like(g)
    db = torch.empty_like(beta)
    if chunk_states is not None:
        if chunk_states is True:
            raise ValueError("chunk_states must be the buffer the forward pass filled")
        cs, cs_bytes = _chunk_states_arg(chunk_states, N, T, H_v, d_k, d_v, dev)
        ws_need = gdn_prefill_backward_saved_workspace_size(N, T, H_qk, H_v, d_k, d_v)
        if workspace is None:
            workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
        rc = lib().gdn_prefill_backward_saved(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cs), cs_bytes, _ptr(cu_seqlens),
            _ptr(d_o), _ptr(d_final_state), N, T, H_qk, H_v, d_k, d_v, float(scale), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dS0), _ptr(workspace), ws_bytes,
            _stream(dev))
        _check(rc, "gdn_prefill_backward_saved")
        return dq, dk, dv, dg, db, dS0
    ws_need = gdn_prefill_backward_workspace_size(N, T, H_qk, H_v, d_k, d_v)
    if workspace is None:
        workspace = torch.empty(max(ws_need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().gdn_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(initial_state), _ptr(cu_seqlens), _ptr(d_o),
                                    _ptr(d_final_state), N, T, H_qk, H_v, d_k, d_v, float(scale),
                                    _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(db), _ptr(dS0),
                                    _ptr(workspace), ws_bytes, _stream(dev))
    _check(rc, "gdn_prefill_backward")
    return dq, dk, dv, dg, db, dS0


def gdn_layer_prefill_backward_workspace_size(N: int, T: int, H_qk: int, H_v: int,
                                              d_k: int = 128, d_v: int = 128) -> int:
    return int(lib().gdn_layer_prefill_backward_workspace_size(N, T, H_qk, H_v, d_k, d_v))


def gdn_layer_prefill_backward(x, conv_w, a, b, A_log, dt_bias, d_o, initial_state=None,
                               d_final_state=None, cu_seqlens=None, *, H_qk: int = 16,
                               H_v: int = 48, d_k: int = 128, d_v: int = 128,
                               l2_eps: float = 1e-6, scale: float = 1.0, d_initial_state=True,
                               workspace=None, chunk_states=None):
    """Gradients of gdn_layer_prefill (chunk_states: the buffer a
    gdn_layer_prefill with chunk_states filled on the same inputs; then
    initial_state is not read).  x: bf16 [T, C_raw]; conv_w: bf16
    [C_raw, 4]; a, b: fp32 [T, H_v]; A_log, dt_bias: fp32 [H_v]; d_o: bf16
    [T, H_v, d_v]; initial_state, d_final_state: fp32 [N, H_v, 128, 128] or None.
    Returns (dx bf16, dconv_w fp32 [C_raw, 4], da, db, dA_log, ddt_bias,
    d_initial_state or None)."""
    torch = _torch()
    dev = _device_of(x)
    _need(x, "x", torch.bfloat16, dev, 2)
    _need(conv_w, "conv_w", torch.bfloat16, dev, 2)
    _need(d_o, "d_o", torch.bfloat16, dev, 3)
    T, C = x.shape
    if C != (2 * H_qk + H_v) * d_k or tuple(conv_w.shape) != (C, 4):
        raise ValueError("x / conv_w shapes do not match H_qk, H_v")
    if tuple(d_o.shape) != (T, H_v, d_v):
        raise ValueError("d_o must be [T, H_v, d_v]")
    for t, name in ((a, "a"), (b, "b")):
        _need(t, name, torch.float32, dev, 2)
        if tuple(t.shape) != (T, H_v):
            raise ValueError(f"{name} must be [T, H_v]")
    for t, name in ((A_log, "A_log"), (dt_bias, "dt_bias")):
        _need(t, name, torch.float32, dev, 1)
        if tuple(t.shape) != (H_v,):
            raise ValueError(f"{name} must be [H_v]")
    N = 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.numel() - 1
    sshape = (N, H_v, d_v, d_k)
    for t, name in ((initial_state, "initial_state"), (d_final_state, "d_final_state")):
        if t is not None:
            _need(t, name, torch.float32, dev, 4)
            if tuple(t.shape) != sshape:
                raise ValueError(f"{name} must be {sshape}")
    if d_initial_state is True:
        dS0 = torch.empty(sshape, dtype=torch.float32, device=dev)
    elif d_initial_state is None or d_initial_state is False:
        dS0 = None
    else:
        dS0 = d_initial_state
        _need(dS0, "d_initial_state", torch.float32, dev, 4)
        if tuple(dS0.shape) != sshape:
            raise ValueError(f"d_initial_state must be {sshape}")
    dx = torch.empty_like(x)
    dw = torch.empty((C, 4), dtype=torch.float32, device=dev)
    da, db = torch.empty_like(a), torch.empty_like(b)
    dA, ddt = torch.empty_like(A_log), torch.empty_like(dt_bias)
    if chunk_states is not None:
        if chunk_states is True:
            raise ValueError("chunk_states must be the buffer the forward pass filled")
        kst, k_bytes = _chunk_states_arg(chunk_states, N, T, H_v, d_k, d_v, dev)
        need = int(lib().gdn_layer_prefill_backward_saved_workspace_size(N, T, H_qk, H_v, d_k, d_v))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
        rc = lib().gdn_layer_prefill_backward_saved(
            _ptr(x), _ptr(conv_w), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), float(l2_eps),
            _ptr(kst), k_bytes, _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final_state), N, T, H_qk, H_v,
            d_k, d_v, float(scale), _ptr(dx), _ptr(dw), _ptr(da), _ptr(db), _ptr(dA), _ptr(ddt),
            _ptr(dS0), _ptr(workspace), ws_bytes, _stream(dev))
        _check(rc, "gdn_layer_prefill_backward_saved")
        return dx, dw, da, db, dA, ddt, dS0
    need = gdn_layer_prefill_backward_workspace_size(N, T, H_qk, H_v, d_k, d_v)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().gdn_layer_prefill_backward(
        _ptr(x), _ptr(conv_w), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), float(l2_eps),
        _ptr(initial_state), _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final_state), N, T, H_qk, H_v,
        d_k, d_v, float(scale), _ptr(dx), _ptr(dw), _ptr(da), _ptr(db), _ptr(dA), _ptr(ddt),
        _ptr(dS0), _ptr(workspace), ws_bytes, _stream(dev))
    _check(rc, "gdn_layer_prefill_backward")
    return dx, dw, da, db, dA, ddt, dS0


def gdn_prefill_raw_workspace_size(N: int, T: int, H_qk: int, H_v: int, d_k: int = 128,
                                   d_v: int = 128) -> int:
    return int(lib().gdn_prefill_raw_workspace_size(N, T, H_qk, H_v, d_k, d_v))


def gdn_prefill_raw(x, conv_w, g, beta, initial_state=None, cu_seqlens=None, *, H_qk: int = 16,
                    H_v: int = 48, d_k: int = 128, d_v: int = 128, l2_eps: float = 1e-6,
                    scale: float = 1.0, final_state=True, o=None, workspace=None,
                    chunk_states=None):
    """Prefill from the raw projections, conv prelude fused.  x: bf16 [T, C_raw];
    conv_w: bf16 [C_raw, 4]; g, beta: fp32 [T, H_v]; initial_state: fp32
    [N, H_v, 128, 128] or None; final_state and chunk_states as for gdn_prefill.
    Returns (o bf16 [T, H_v, d_v], final_state or None), plus chunk_states when
    it is given."""
    torch = _torch()
    dev = _device_of(x)
    _need(x, "x", torch.bfloat16, dev, 2)
    _need(conv_w, "conv_w", torch.bfloat16, dev, 2)
    T = x.shape[0]
    if x.shape[1] != 2 * H_qk * d_k + H_v * d_v or tuple(conv_w.shape) != (x.shape[1], 4):
        raise ValueError("x / conv_w shapes do not match the head configuration")
    _need(g, "g", torch.float32, dev, 2)
    _need(beta, "beta", torch.float32, dev, 2)
    if tuple(g.shape) != (T, H_v) or tuple(beta.shape) != (T, H_v):
        raise ValueError("g and beta must be [T, H_v]")
    N = 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.numel() - 1
    sshape = (N, H_v, d_v, d_k)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev, 4)
        if tuple(initial_state.shape) != sshape:
            raise ValueError(f"initial_state must be {sshape}")
    if final_state is True:
        fs = torch.empty(sshape, dtype=torch.float32, device=dev)
    elif final_state is None or final_state is False:
        fs = None
    else:
        fs = final_state
        _need(fs, "final_state", torch.float32, dev, 4)
        if tuple(fs.shape) != sshape:
            raise ValueError(f"final_state must be {sshape}")
    if o is None:
        o = torch.empty((T, H_v, d_v), dtype=torch.bfloat16, device=dev)
    else:
        _need(o, "o", torch.bfloat16, dev, 3)
        if tuple(o.shape) != (T, H_v, d_v):
            raise ValueError("o must be [T, H_v, d_v]")
    ws_need = gdn_prefill_raw_workspace_size(N, T, H_qk, H_v, d_k, d_v)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if chunk_states is not None:
        cs, cs_bytes = _chunk_states_arg(chunk_states, N, T, H_v, d_k, d_v, dev)
        rc = lib().gdn_prefill_raw_save_states(
            _ptr(x), _ptr(conv_w), float(l2_eps), _ptr(g), _ptr(beta), _ptr(initial_state),
            _ptr(fs), _ptr(cu_seqlens), N, T, H_qk, H_v, d_k, d_v, float(scale), _ptr(o), _ptr(cs),
            cs_bytes, _ptr(workspace), ws_bytes, _stream(dev))
        _check(rc, "gdn_prefill_raw_save_states")
        return o, fs, cs
    rc = lib().gdn_prefill_raw(_ptr(x), _ptr(conv_w), float(l2_eps), _ptr(g), _ptr(beta),
                               _ptr(initial_state), _ptr(fs), _ptr(cu_seqlens), N, T, H_qk, H_v,
                               d_k, d_v, float(scale), _ptr(o), _ptr(workspace), ws_bytes,
                               _stream(dev))
    _check(rc, "gdn_prefill_raw")
    return o, fs


def gdn_gates(a, b, A_log, dt_bias, *, out=None):
    """g = -softplus(a + dt_bias) exp(A_log), beta = sigmoid(b).  a, b: fp32
    [T, H_v]; A_log, dt_bias: fp32 [H_v].  Returns fp32 (g, beta)."""
    torch = _torch()
    dev = _device_of(a)
    _need(a, "a", torch.float32, dev, 2)
    _need(b, "b", torch.float32, dev, 2)
    T, H_v = a.shape
    if tuple(b.shape) != (T, H_v):
        raise ValueError("a and b must have the same shape")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        _need(t, name, torch.float32, dev, 1)
        if t.numel() != H_v:
            raise ValueError(f"{name} must have H_v = {H_v} entries")
    if out is None:
        g, beta = torch.empty_like(a), torch.empty_like(a)
    else:
        g, beta = out
        for name, t in (("g", g), ("beta", beta)):
            _need(t, name, torch.float32, dev, 2)
            if tuple(t.shape) != (T, H_v):
                raise ValueError(f"{name} must be [T, H_v]")
    _check(lib().gdn_gates(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), T, H_v, _ptr(g),
                           _ptr(beta), _stream(dev)), "gdn_gates")
    return g, beta


def _conv_state_in_arg(t, N, C, dev):
    if t is None:
        return None
    torch = _torch()
    _need(t, "conv_state_in", torch.bfloat16, dev, 3)
    if tuple(t.shape) != (N, 3, C):
        raise ValueError(f"conv_state_in must be {(N, 3, C)}")
    return t


def gdn_layer_prefill_workspace_size(N: int, T: int, H_qk: int, H_v: int, d_k: int = 128,
                                     d_v: int = 128) -> int:
    return int(lib().gdn_layer_prefill_workspace_size(N, T, H_qk, H_v, d_k, d_v))


def gdn_layer_prefill(x, conv_w, a, b, A_log, dt_bias, initial_state=None, cu_seqlens=None, *,
                      H_qk: int = 16, H_v: int = 48, d_k: int = 128, d_v: int = 128,
                      l2_eps: float = 1e-6, scale: float = 1.0, final_state=True,
                      conv_state=True, o=None, workspace=None, chunk_states=None,
                      conv_state_in=None):
    """The layer's prefill from raw projections: gates from a, b, then the fused
    prelude + chunked prefill, then each sequence's conv history.  x: bf16
    [T, C_raw]; a, b: fp32 [T, H_v]; A_log, dt_bias: fp32 [H_v].  final_state /
    conv_state: True (allocate), False/None (skip) or a tensor to write
    (conv_state: bf16 [N, 3, C_raw]); chunk_states as for gdn_prefill (not
    with conv_state_in).  conv_state_in: bf16 [N, 3, C_raw], the conv history
    each sequence resumes from (a previous call's conv_state; may be the
    conv_state tensor itself), or None for zeros.  Returns (o, final_state,
    conv_state), plus chunk_states when it is given."""
    torch = _torch()
    dev = _device_of(x)
    _need(x, "x", torch.bfloat16, dev, 2)
    _need(conv_w, "conv_w", torch.bfloat16, dev, 2)
    T, C = x.shape
    if C != 2 * H_qk * d_k + H_v * d_v or tuple(conv_w.shape) != (C, 4):
        raise ValueError("x / conv_w shapes do not match the head configuration")
    for name, t in (("a", a), ("b", b)):
        _need(t, name, torch.float32, dev, 2)
        if tuple(t.shape) != (T, H_v):
            raise ValueError(f"{name} must be [T, H_v]")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        _need(t, name, torch.float32, dev, 1)
        if t.numel() != H_v:
            raise ValueError(f"{name} must have H_v = {H_v} entries")
    N = 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.numel() - 1
    sshape = (N, H_v, d_v, d_k)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev, 4)
        if tuple(initial_state.shape) != sshape:
            raise ValueError(f"initial_state must be {sshape}")

    def out_arg(val, shape, dtype, name):
        if val is True:
            return torch.empty(shape, dtype=dtype, device=dev)
        if val is None or val is False:
            return None
        _need(val, name, dtype, dev, len(shape))
        if tuple(val.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
        return val

    fs = out_arg(final_state, sshape, torch.float32, "final_state")
    cs = out_arg(conv_state, (N, 3, C), torch.bfloat16, "conv_state")
    ci = _conv_state_in_arg(conv_state_in, N, C, dev)
    o = out_arg(True if o is None else o, (T, H_v, d_v), torch.bfloat16, "o")
    ws_need = gdn_layer_prefill_workspace_size(N, T, H_qk, H_v, d_k, d_v)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if chunk_states is not None:
        if ci is not None:
            raise ValueError("chunk_states (training) takes no conv_state_in")
        kst, k_bytes = _chunk_states_arg(chunk_states, N, T, H_v, d_k, d_v, dev)
        rc = lib().gdn_layer_prefill_save_states(
            _ptr(x), _ptr(conv_w), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), float(l2_eps),
            _ptr(initial_state), _ptr(fs), _ptr(cs), _ptr(cu_seqlens), N, T, H_qk, H_v, d_k, d_v,
            float(scale), _ptr(o), _ptr(kst), k_bytes, _ptr(workspace), ws_bytes, _stream(dev))
        _check(rc, "gdn_layer_prefill_save_states")
        return o, fs, cs, kst
    rc = lib().gdn_layer_prefill(_ptr(x), _ptr(conv_w), _ptr(a), _ptr(b), _ptr(A_log),
                                 _ptr(dt_bias), float(l2_eps), _ptr(initial_state), _ptr(fs),
                                 _ptr(ci), _ptr(cs), _ptr(cu_seqlens), N, T, H_qk, H_v, d_k, d_v,
                                 float(scale), _ptr(o), _ptr(workspace), ws_bytes, _stream(dev))
    _check(rc, "gdn_layer_prefill")
    return o, fs, cs


def gdn_layer_prefill_gated_workspace_size(N, T, H_qk=16, H_v=48, d_k=128, d_v=128):
    return int(lib().gdn_layer_prefill_gated_workspace_size(N, T, H_qk, H_v, d_k, d_v))


def gdn_layer_prefill_gated(x, conv_w, a, b, A_log, dt_bias, z, norm_w, initial_state=None,
                            cu_seqlens=None, *, H_qk: int = 16, H_v: int = 48, d_k: int = 128,
                            d_v: int = 128, l2_eps: float = 1e-6, norm_eps: float = 1e-6,
                            scale: float = 1.0, final_state=True, conv_state=True, o=None, y=None,
                            workspace=None, conv_state_in=None):
    """gdn_layer_prefill with the output gate applied in the same call: z bf16
    [T, H_v, d_v], norm_w fp32 [d_v]; conv_state_in as for gdn_layer_prefill.
    Returns (y, o, final_state, conv_state), y the gated outputs."""
    torch = _torch()
    dev = _device_of(x)
    _need(x, "x", torch.bfloat16, dev, 2)
    _need(conv_w, "conv_w", torch.bfloat16, dev, 2)
    T, C = x.shape
    if C != 2 * H_qk * d_k + H_v * d_v or tuple(conv_w.shape) != (C, 4):
        raise ValueError("x / conv_w shapes do not match the head configuration")
    for name, t in (("a", a), ("b", b)):
        _need(t, name, torch.float32, dev, 2)
        if tuple(t.shape) != (T, H_v):
            raise ValueError(f"{name} must be [T, H_v]")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        _need(t, name, torch.float32, dev, 1)
        if t.numel() != H_v:
            raise ValueError(f"{name} must have H_v = {H_v} entries")
    _need(z, "z", torch.bfloat16, dev, 3)
    if tuple(z.shape) != (T, H_v, d_v):
        raise ValueError("z must be [T, H_v, d_v]")
    _need(norm_w, "norm_w", torch.float32, dev, 1)
    if norm_w.numel() != d_v:
        raise ValueError("norm_w must have d_v entries")
    N = 1
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev, 1)
        N = cu_seqlens.numel() - 1
    sshape = (N, H_v, d_v, d_k)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev, 4)
        if tuple(initial_state.shape) != sshape:
            raise ValueError(f"initial_state must be {sshape}")

    def out_arg(val, shape, dtype, name):
        if val is True:
            return torch.empty(shape, dtype=dtype, device=dev)
        if val is None or val is False:
            return None
        _need(val, name, dtype, dev, len(shape))
        if tuple(val.shape) != shape:
            raise ValueError(f"{name} must be {shape}")
        return val

    fs = out_arg(final_state, sshape, torch.float32, "final_state")
    cs = out_arg(conv_state, (N, 3, C), torch.bfloat16, "conv_state")
    o = out_arg(True if o is None else o, (T, H_v, d_v), torch.bfloat16, "o")
    y = out_arg(True if y is None else y, (T, H_v, d_v), torch.bfloat16, "y")
    ci = _conv_state_in_arg(conv_state_in, N, C, dev)
    ws_need = gdn_layer_prefill_gated_workspace_size(N, T, H_qk, H_v, d_k, d_v)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = lib().gdn_layer_prefill_gated(
        _ptr(x), _ptr(conv_w), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), float(l2_eps),
        _ptr(z), _ptr(norm_w), float(norm_eps), _ptr(initial_state), _ptr(fs), _ptr(ci), _ptr(cs),
        _ptr(cu_seqlens), N, T, H_qk, H_v, d_k, d_v, float(scale), _ptr(o), _ptr(y),
        _ptr(workspace), ws_bytes, _stream(dev))
    _check(rc, "gdn_layer_prefill_gated")
    return y, o, fs, cs


def gdn_layer_decode_step(x, conv_w, a, b, A_log, dt_bias, conv_state_pool, state_pool,
                          slot_idx, *, H_qk: int = 16, H_v: int = 48, d_k: int = 128,
                          d_v: int = 128, l2_eps: float = 1e-6, scale: float = 1.0, o=None):
    """One token per sequence from raw projections x: bf16 [B, C_raw]; a, b:
    fp32 [B, H_v]; conv_state_pool: bf16 [P, 3, C_raw] and state_pool: fp32
    [P, H_v, 128, 128], both advanced in place at slot_idx.  Returns o (bf16)."""
    torch = _torch()
    dev = _device_of(x)
    _need(x, "x", torch.bfloat16, dev, 2)
    _need(conv_w, "conv_w", torch.bfloat16, dev, 2)
    B, C = x.shape
    if C != 2 * H_qk * d_k + H_v * d_v or tuple(conv_w.shape) != (C, 4):
        raise ValueError("x / conv_w shapes do not match the head configuration")
    for name, t in (("a", a), ("b", b)):
        _need(t, name, torch.float32, dev, 2)
        if tuple(t.shape) != (B, H_v):
            raise ValueError(f"{name} must be [B, H_v]")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        _need(t, name, torch.float32, dev, 1)
        if t.numel() != H_v:
            raise ValueError(f"{name} must have H_v = {H_v} entries")
    _need(conv_state_pool, "conv_state_pool", torch.bfloat16, dev, 3)
    _need(state_pool, "state_pool", torch.float32, dev, 4)
    _need(slot_idx, "slot_idx", torch.int32, dev, 1)
    P = state_pool.shape[0]
    if (tuple(conv_state_pool.shape) != (P, 3, C) or tuple(state_pool.shape[1:]) != (H_v, d_v, d_k)
            or slot_idx.numel() != B):
        raise ValueError("decode shapes disagree")
    if o is None:
        o = torch.empty((B, H_v, d_v), dtype=torch.bfloat16, device=dev)
    else:
        _need(o, "o", torch.bfloat16, dev, 3)
    rc = lib().gdn_layer_decode_step(_ptr(x), _ptr(conv_w), _ptr(a), _ptr(b), _ptr(A_log),
                                     _ptr(dt_bias), float(l2_eps), _ptr(conv_state_pool),
                                     _ptr(state_pool), _ptr(slot_idx), B, P, H_qk, H_v, d_k, d_v,
                                     float(scale), _ptr(o), _stream(dev))
    _check(rc, "gdn_layer_decode_step")
    return o


def gdn_decode_multi_step(q, k, v, g, beta, state_pool, slot_idx, *, scale: float = 1.0, o=None,
                          snapshots=False):
    """n tokens per sequence in order.  q, k: bf16 [B, n, H_qk, 128]; v: bf16
    [B, n, H_v, 128]; g, beta: fp32 [B, n, H_v]; the pool advances in place.
    snapshots: True (allocate), False/None (skip) or an fp32
    [B, n, H_v, 128, 128] tensor that receives the state before each token.
    Returns (o bf16 [B, n, H_v, 128], snapshots or None)."""
    torch = _torch()
    dev = _device_of(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, dev, 4)
    B, n, H_qk, d_k = q.shape
    H_v, d_v = v.shape[2], v.shape[3]
    _need(g, "g", torch.float32, dev, 3)
    _need(beta, "beta", torch.float32, dev, 3)
    _need(state_pool, "state_pool", torch.float32, dev, 4)
    _need(slot_idx, "slot_idx", torch.int32, dev, 1)
    P = state_pool.shape[0]
    if (tuple(k.shape) != (B, n, H_qk, d_k) or tuple(v.shape[:2]) != (B, n)
            or tuple(g.shape) != (B, n, H_v) or tuple(beta.shape) != (B, n, H_v)
            or tuple(state_pool.shape[1:]) != (H_v, d_v, d_k) or slot_idx.numel() != B):
        raise ValueError("multi-token decode shapes disagree")
    if o is None:
        o = torch.empty((B, n, H_v, d_v), dtype=torch.bfloat16, device=dev)
    else:
        _need(o, "o", torch.bfloat16, dev, 4)
    if snapshots is True:
        snapshots = torch.empty((B, n, H_v, d_v, d_k), dtype=torch.float32, device=dev)
    elif snapshots is False:
        snapshots = None
    elif snapshots is not None:
        _need(snapshots, "snapshots", torch.float32, dev, 5)
    rc = lib().gdn_decode_multi_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(state_pool), _ptr(slot_idx), B, P, n, H_qk, H_v, d_k,
                                     d_v, float(scale), _ptr(o), _ptr(snapshots), _stream(dev))
    _check(rc, "gdn_decode_multi_step")
    return o, snapshots


def gdn_state_rollback(snapshots, n_keep, state_pool, slot_idx):
    """Slot slot_idx[b] takes snapshots[b, n_keep[b]] when n_keep[b] < n (kept
    otherwise).  snapshots: fp32 [B, n, H_v, 128, 128]; n_keep: int32 [B]."""
    torch = _torch()
    dev = _device_of(snapshots)
    _need(snapshots, "snapshots", torch.float32, dev, 5)
    _need(n_keep, "n_keep", torch.int32, dev, 1)
    _need(state_pool, "state_pool", torch.float32, dev, 4)
    _need(slot_idx, "slot_idx", torch.int32, dev, 1)
    B, n, H_v, d_v, d_k = snapshots.shape
    if n_keep.numel() != B or slot_idx.numel() != B or tuple(state_pool.shape[1:]) != (H_v, d_v, d_k):
        raise ValueError("rollback shapes disagree")
    rc = lib().gdn_state_rollback(_ptr(snapshots), _ptr(n_keep), n, _ptr(state_pool),
                                  _ptr(slot_idx), B, state_pool.shape[0], H_v, d_k, d_v,
                                  _stream(dev))
    _check(rc, "gdn_state_rollback")


def gdn_gated_norm(o, z, w, *, eps: float = 1e-6, out=None):
    """Output gate: o / sqrt(mean(o^2) + eps) * w * SiLU(z) over the last axis.
    o, z: bf16 [..., 128]; w: fp32 [128]; out: bf16 like o (may be o).
    Returns out."""
    torch = _torch()
    dev = _device_of(o)
    _need(o, "o", torch.bfloat16, dev)
    _need(z, "z", torch.bfloat16, dev)
    _need(w, "w", torch.float32, dev, 1)
    d_v = o.shape[-1]
    if tuple(z.shape) != tuple(o.shape) or w.numel() != d_v:
        raise ValueError("o and z must have the same shape and w d_v entries")
    if out is None:
        out = torch.empty_like(o)
    else:
        _need(out, "out", torch.bfloat16, dev)
        if tuple(out.shape) != tuple(o.shape):
            raise ValueError("out must have o's shape")
    rows = o.numel() // d_v
    _check(lib().gdn_gated_norm(_ptr(o), _ptr(z), _ptr(w), rows, d_v, float(eps), _ptr(out),
                                _stream(dev)), "gdn_gated_norm")
    return out


def gdn_decode_step(q, k, v, g, beta, state_pool, slot_idx, *, scale: float = 1.0, o=None):
    """One token per sequence; states in state_pool[slot_idx[b]] advance in place.
    q, k: bf16 [B, H_qk, 128]; v: bf16 [B, H_v, 128]; g, beta: fp32 [B, H_v];
    state_pool: fp32 [P, H_v, 128, 128]; slot_idx: int32 [B].  Returns o (bf16)."""
    torch = _torch()
    dev = _device_of(q)
    for name, t, nd in (("q", q, 3), ("k", k, 3), ("v", v, 3)):
        _need(t, name, torch.bfloat16, dev, nd)
    B, H_qk, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    _need(g, "g", torch.float32, dev, 2)
    _need(beta, "beta", torch.float32, dev, 2)
    _need(state_pool, "state_pool", torch.float32, dev, 4)
    _need(slot_idx, "slot_idx", torch.int32, dev, 1)
    P = state_pool.shape[0]
    if (tuple(k.shape) != (B, H_qk, d_k) or v.shape[0] != B or tuple(g.shape) != (B, H_v)
            or tuple(beta.shape) != (B, H_v) or tuple(state_pool.shape[1:]) != (H_v, d_v, d_k)
            or slot_idx.numel() != B):
        raise ValueError("decode shapes disagree")
    if o is None:
        o = torch.empty((B, H_v, d_v), dtype=torch.bfloat16, device=dev)
    else:
        _need(o, "o", torch.bfloat16, dev, 3)
    rc = lib().gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
                               _ptr(slot_idx), B, P, H_qk, H_v, d_k, d_v, float(scale), _ptr(o),
                               _stream(dev))
    _check(rc, "gdn_decode_step")
    return o


def gdn_gated_norm_backward(o, z, w, dy, *, eps: float = 1e-6, workspace=None):
    """Gradients of gdn_gated_norm: o, z, dy bf16 [..., 128]; w fp32 [128].
    Returns (d_o bf16, dz bf16, dw fp32 [128])."""
    torch = _torch()
    dev = _device_of(o)
    for t, name in ((o, "o"), (z, "z"), (dy, "dy")):
        if t.dtype != torch.bfloat16 or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bf16 tensor on {dev}")
    if tuple(z.shape) != tuple(o.shape) or tuple(dy.shape) != tuple(o.shape) or o.shape[-1] != 128:
        raise ValueError("o, z and dy must share a shape [..., 128]")
    _need(w, "w", torch.float32, dev, 1)
    rows = o.numel() // 128
    d_o, dz = torch.empty_like(o), torch.empty_like(z)
    dw = torch.empty((128,), dtype=torch.float32, device=dev)
    need = int(lib().gdn_gated_norm_backward_workspace_size(rows, 128))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib().gdn_gated_norm_backward(_ptr(o), _ptr(z), _ptr(w), _ptr(dy), rows, 128, float(eps),
                                       _ptr(d_o), _ptr(dz), _ptr(dw), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc, "gdn_gated_norm_backward")
    return d_o, dz, dw


__all__ = ["lib", "GDNError", "gdn_abi_version", "gdn_conv_prelude", "gdn_prefill",
           "gdn_prefill_no_alloc",
           "gdn_chunk_states_size", "gdn_prefill_backward_saved_workspace_size",
           "gdn_prefill_workspace_size", "gdn_prefill_raw", "gdn_prefill_raw_workspace_size",
           "gdn_prefill_backward", "gdn_prefill_backward_workspace_size",
           "gdn_layer_prefill_backward", "gdn_layer_prefill_backward_workspace_size",
           "gdn_gates", "gdn_layer_prefill", "gdn_layer_prefill_workspace_size",
           "gdn_layer_prefill_gated", "gdn_layer_prefill_gated_workspace_size",
           "gdn_layer_decode_step", "gdn_decode_multi_step", "gdn_state_rollback",
           "gdn_gated_norm", "gdn_gated_norm_backward", "gdn_decode_step", "GDN_F32", "GDN_BF16",
           "EXPORTS"]
