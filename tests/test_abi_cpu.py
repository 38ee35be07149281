"""The C-ABI library loads, exports every entry point include/gdn.h declares,
and rejects bad arguments on the host before any device call (CPU only)."""
import ctypes
import os
import re

import pytest

import linear_attention_sequence_delta_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


def test_exports_match_header():
    L = gdn.lib()
    decl = _declared()
    assert decl == sorted(gdn.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name
    assert gdn.gdn_abi_version() == 5


def _prefill(L, **kw):
    a = dict(io=1, q=1, k=2, v=3, g=4, beta=5, S0=None, Sf=None, cu=None, N=1, T=64, H_qk=16,
             H_v=48, d_k=128, d_v=128, scale=1.0, o=0x100000, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.gdn_prefill(a["io"], a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["Sf"],
                         a["cu"], a["N"], a["T"], a["H_qk"], a["H_v"], a["d_k"], a["d_v"],
                         a["scale"], a["o"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d_k=64), gdn.GDN_ERR_UNSUPPORTED),
    (dict(d_v=256), gdn.GDN_ERR_UNSUPPORTED),
    (dict(io=7), gdn.GDN_ERR_UNSUPPORTED),
    (dict(H_v=47), gdn.GDN_ERR_INVALID_ARG),
    (dict(H_qk=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(N=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(N=0), gdn.GDN_ERR_INVALID_ARG),
    (dict(T=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(q=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=1), gdn.GDN_ERR_INVALID_ARG),                    # o overlaps q
])
def test_prefill_rejects_bad_arguments(kw, code):
    L = gdn.lib()
    assert _prefill(L, **kw) == code
    assert L.gdn_last_error().decode()


def test_prefill_workspace_checked():
    L = gdn.lib()
    need = gdn.gdn_prefill_workspace_size(gdn.GDN_BF16, 1, 4096, 16, 48)
    if need == 0:
        pytest.skip("bf16 prefill needs no workspace in this build")
    big = 1 << 40
    assert _prefill(L, T=4096, o=big, ws=None, ws_bytes=0) == gdn.GDN_ERR_WORKSPACE
    assert _prefill(L, T=4096, o=big, ws=2 * big, ws_bytes=need - 1) == gdn.GDN_ERR_WORKSPACE
    assert "workspace" in L.gdn_last_error().decode()


def test_final_state_partial_alias_rejected():
    L = gdn.lib()
    big = 1 << 40
    ns = 48 * 128 * 128 * 4
    ws = gdn.gdn_prefill_workspace_size(gdn.GDN_BF16, 1, 64, 16, 48)
    rc = _prefill(L, o=big, S0=2 * big, Sf=2 * big + 4096, ws=3 * big, ws_bytes=ws)
    assert rc == gdn.GDN_ERR_INVALID_ARG
    assert ns > 4096


def test_decode_rejects_bad_arguments():
    L = gdn.lib()
    args = [1, 2, 3, 4, 5, 0x100000000, 6, 4, 8, 16, 48, 128, 128, 1.0, 0x10000000000, None]
    assert L.gdn_decode_step(*args[:11], 64, 128, 1.0, args[14], None) == gdn.GDN_ERR_UNSUPPORTED
    assert L.gdn_decode_step(*args[:7], 9, 8, *args[9:]) == gdn.GDN_ERR_INVALID_ARG   # B > P
    assert L.gdn_decode_step(*args[:7], 4, 0, *args[9:]) == gdn.GDN_ERR_INVALID_ARG   # P = 0
    bad = list(args)
    bad[6] = None
    assert L.gdn_decode_step(*bad) == gdn.GDN_ERR_INVALID_ARG                      # slot_idx NULL
    zero = list(args)
    zero[7] = 0
    assert L.gdn_decode_step(*zero) == gdn.GDN_OK                                  # B = 0: no-op


def test_prelude_rejects_bad_arguments():
    L = gdn.lib()
    base = [1, 2, None, 1, 10, 16, 48, 128, 128, 1e-6, 0x100000000, 0x200000000, 0x300000000, None]
    a = list(base); a[4] = 0
    assert L.gdn_conv_prelude(*a) == gdn.GDN_OK                                     # T = 0: no-op
    a = list(base); a[3] = 3
    assert L.gdn_conv_prelude(*a) == gdn.GDN_ERR_INVALID_ARG                        # N != 1, no cu
    a = list(base); a[9] = -1.0
    assert L.gdn_conv_prelude(*a) == gdn.GDN_ERR_INVALID_ARG
    a = list(base); a[7] = 96
    assert L.gdn_conv_prelude(*a) == gdn.GDN_ERR_UNSUPPORTED
    a = list(base); a[0] = None
    assert L.gdn_conv_prelude(*a) == gdn.GDN_ERR_INVALID_ARG


def _prefill_raw(L, **kw):
    a = dict(x=1, w=2, eps=1e-6, g=4, beta=5, S0=None, Sf=None, cu=None, N=1, T=64, H_qk=16,
             H_v=48, d_k=128, d_v=128, scale=1.0, o=1 << 40, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.gdn_prefill_raw(a["x"], a["w"], a["eps"], a["g"], a["beta"], a["S0"], a["Sf"],
                             a["cu"], a["N"], a["T"], a["H_qk"], a["H_v"], a["d_k"], a["d_v"],
                             a["scale"], a["o"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d_k=64), gdn.GDN_ERR_UNSUPPORTED),
    (dict(H_qk=1, H_v=16), gdn.GDN_ERR_UNSUPPORTED),          # 16 V-heads per QK head
    (dict(H_v=47), gdn.GDN_ERR_INVALID_ARG),
    (dict(N=2), gdn.GDN_ERR_INVALID_ARG),
    (dict(T=-1), gdn.GDN_ERR_INVALID_ARG),
    (dict(x=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(eps=float("nan")), gdn.GDN_ERR_INVALID_ARG),
    (dict(eps=-1.0), gdn.GDN_ERR_INVALID_ARG),
    (dict(scale=float("inf")), gdn.GDN_ERR_INVALID_ARG),
    (dict(o=1), gdn.GDN_ERR_INVALID_ARG),                     # o overlaps x_raw
    (dict(), gdn.GDN_ERR_WORKSPACE),                          # no workspace
])
def test_prefill_raw_rejects_bad_arguments(kw, code):
    L = gdn.lib()
    assert _prefill_raw(L, **kw) == code
    assert L.gdn_last_error().decode()


def test_prefill_raw_workspace_size():
    """The fused path keeps the unfused records plus the normalised q and k rows."""
    for N, T in ((1, 1), (1, 4133), (8, 65536)):
        plain = gdn.gdn_prefill_workspace_size(gdn.GDN_BF16, N, T, 16, 48)
        fused = gdn.gdn_prefill_raw_workspace_size(N, T, 16, 48)
        chunks = (T + 63) // 64 + N
        assert fused == plain + 2 * chunks * 64 * 16 * 128 * 2
    assert gdn.gdn_prefill_raw_workspace_size(1, 0, 16, 48) == 0
    L = gdn.lib()
    need = gdn.gdn_prefill_raw_workspace_size(1, 64, 16, 48)
    assert _prefill_raw(L, ws=1 << 41, ws_bytes=need - 1) == gdn.GDN_ERR_WORKSPACE


def test_gates_rejects_bad_arguments():
    L = gdn.lib()
    big = 1 << 40
    assert L.gdn_gates(big, big + (1 << 30), 1 << 39, (1 << 39) + 4096, 64, 48, None, 2 * big,
                       None) == gdn.GDN_ERR_INVALID_ARG                       # g NULL
    assert L.gdn_gates(big, big + (1 << 30), 1 << 39, (1 << 39) + 4096, 64, 48, big, 2 * big,
                       None) == gdn.GDN_ERR_INVALID_ARG                       # g overlaps a
    assert L.gdn_gates(None, None, None, None, 0, 48, None, None, None) == gdn.GDN_OK   # T = 0
    assert L.gdn_gates(None, None, None, None, 4, 0, None, None, None) == gdn.GDN_ERR_INVALID_ARG


def _layer_prefill(L, **kw):
    big = 1 << 40
    a = dict(x=big, w=2 * big, a=3 * big, b=4 * big, A=5 * big, dt=6 * big, eps=1e-6, S0=None,
             Sf=None, ci=None, cs=None, cu=None, N=1, T=64, H_qk=16, H_v=48, d_k=128, d_v=128,
             scale=1.0, o=7 * big, ws=8 * big,
             ws_bytes=gdn.gdn_layer_prefill_workspace_size(1, 64, 16, 48), stream=None)
    a.update(kw)
    return L.gdn_layer_prefill(a["x"], a["w"], a["a"], a["b"], a["A"], a["dt"], a["eps"], a["S0"],
                               a["Sf"], a["ci"], a["cs"], a["cu"], a["N"], a["T"], a["H_qk"],
                               a["H_v"], a["d_k"], a["d_v"], a["scale"], a["o"], a["ws"],
                               a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(a=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(A=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(ws_bytes=1), gdn.GDN_ERR_WORKSPACE),
    (dict(cs=1 << 40), gdn.GDN_ERR_INVALID_ARG),        # conv history out overlaps x_raw
    (dict(o=3 * (1 << 40)), gdn.GDN_ERR_INVALID_ARG),    # o overlaps a
    (dict(eps=float("nan")), gdn.GDN_ERR_INVALID_ARG),
    (dict(d_v=64), gdn.GDN_ERR_UNSUPPORTED),
    (dict(ci=7 * (1 << 40)), gdn.GDN_ERR_INVALID_ARG),   # conv history in overlaps o
    (dict(ci=8 * (1 << 40)), gdn.GDN_ERR_INVALID_ARG),   # ... or the workspace
    (dict(cs=12 << 40, ci=(12 << 40) + 64), gdn.GDN_ERR_INVALID_ARG),   # a shifted view of the history out
])
def test_layer_prefill_rejects_bad_arguments(kw, code):
    L = gdn.lib()
    assert _layer_prefill(L, **kw) == code
    assert L.gdn_last_error().decode()


def test_layer_prefill_workspace_size():
    for N, T in ((1, 1), (1, 4133), (8, 65536)):
        gate = (T * 48 * 4 + 255) // 256 * 256
        assert (gdn.gdn_layer_prefill_workspace_size(N, T, 16, 48)
                == 2 * gate + gdn.gdn_prefill_raw_workspace_size(N, T, 16, 48))
    assert gdn.gdn_layer_prefill_workspace_size(1, 0, 16, 48) == 0


def _layer_prefill_gated(L, **kw):
    big = 1 << 40
    a = dict(x=big, w=2 * big, a=3 * big, b=4 * big, A=5 * big, dt=6 * big, eps=1e-6, z=9 * big,
             nw=10 * big, neps=1e-6, S0=None, Sf=None, ci=None, cs=None, cu=None, N=1, T=64,
             H_qk=16, H_v=48, d_k=128, d_v=128, scale=1.0, o=7 * big, y=11 * big, ws=8 * big,
             ws_bytes=gdn.gdn_layer_prefill_gated_workspace_size(1, 64, 16, 48), stream=None)
    a.update(kw)
    return L.gdn_layer_prefill_gated(a["x"], a["w"], a["a"], a["b"], a["A"], a["dt"], a["eps"],
                                     a["z"], a["nw"], a["neps"], a["S0"], a["Sf"], a["ci"], a["cs"],
                                     a["cu"], a["N"], a["T"], a["H_qk"], a["H_v"], a["d_k"],
                                     a["d_v"], a["scale"], a["o"], a["y"], a["ws"], a["ws_bytes"],
                                     a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(z=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(nw=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(y=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(neps=float("nan")), gdn.GDN_ERR_INVALID_ARG),
    (dict(neps=-1.0), gdn.GDN_ERR_INVALID_ARG),
    (dict(y=7 * (1 << 40)), gdn.GDN_ERR_INVALID_ARG),     # y overlaps o
    (dict(y=9 * (1 << 40)), gdn.GDN_ERR_INVALID_ARG),     # y overlaps z
    (dict(z=7 * (1 << 40)), gdn.GDN_ERR_INVALID_ARG),     # z overlaps o
    (dict(ws_bytes="plain"), gdn.GDN_ERR_WORKSPACE),     # gdn_layer_prefill's size: too small
    (dict(a=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(d_v=64), gdn.GDN_ERR_UNSUPPORTED),
])
def test_layer_prefill_gated_rejects_bad_arguments(kw, code):
    L = gdn.lib()
    if kw.get("ws_bytes") == "plain":
        kw = dict(kw, ws_bytes=gdn.gdn_layer_prefill_workspace_size(1, 64, 16, 48))
    assert _layer_prefill_gated(L, **kw) == code
    assert L.gdn_last_error().decode()


def test_layer_prefill_gated_workspace_size():
    for N, T in ((1, 1), (1, 4133), (8, 65536)):
        plain = gdn.gdn_layer_prefill_workspace_size(N, T, 16, 48)
        chunks = (T + 63) // 64 + N
        part = chunks * 48 * 64 * 4 * 8         # a tagged 8-byte sum per (chunk, V-head, row, slab)
        assert gdn.gdn_layer_prefill_gated_workspace_size(N, T, 16, 48) == plain + part
    assert gdn.gdn_layer_prefill_gated_workspace_size(1, 0, 16, 48) == 0


def test_layer_decode_rejects_bad_arguments():
    L = gdn.lib()
    big = 1 << 40

    def call(**kw):
        a = dict(x=big, w=2 * big, a=3 * big, b=4 * big, A=5 * big, dt=6 * big, eps=1e-6,
                 cs=7 * big, pool=8 * big, slots=9 * big, B=4, P=8, o=10 * big)
        a.update(kw)
        return L.gdn_layer_decode_step(a["x"], a["w"], a["a"], a["b"], a["A"], a["dt"], a["eps"],
                                       a["cs"], a["pool"], a["slots"], a["B"], a["P"], 16, 48, 128,
                                       128, 1.0, a["o"], None)
    assert call(cs=None) == gdn.GDN_ERR_INVALID_ARG
    assert call(B=9) == gdn.GDN_ERR_INVALID_ARG                 # more sequences than slots
    assert call(cs=8 * big) == gdn.GDN_ERR_INVALID_ARG          # the two pools overlap
    assert call(o=8 * big) == gdn.GDN_ERR_INVALID_ARG           # o overlaps the state pool
    assert call(B=0, x=None) == gdn.GDN_OK                      # B = 0: no-op


def test_multi_step_and_rollback_reject_bad_arguments():
    L = gdn.lib()
    big = 1 << 40

    def multi(**kw):
        a = dict(q=big, k=2 * big, v=3 * big, g=4 * big, beta=5 * big, pool=6 * big,
                 slots=7 * big, B=4, P=8, n=3, o=8 * big, snaps=9 * big)
        a.update(kw)
        return L.gdn_decode_multi_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"],
                                       a["slots"], a["B"], a["P"], a["n"], 16, 48, 128, 128, 1.0,
                                       a["o"], a["snaps"], None)
    assert multi(n=0) == gdn.GDN_ERR_INVALID_ARG
    assert multi(q=None) == gdn.GDN_ERR_INVALID_ARG
    assert multi(snaps=6 * big) == gdn.GDN_ERR_INVALID_ARG      # snapshots overlap the pool
    assert multi(o=6 * big) == gdn.GDN_ERR_INVALID_ARG          # o overlaps the pool
    assert multi(B=0, q=None) == gdn.GDN_OK
    assert L.gdn_state_rollback(None, big, 3, 2 * big, 3 * big, 4, 8, 48, 128, 128,
                                None) == gdn.GDN_ERR_INVALID_ARG
    assert L.gdn_state_rollback(big, 2 * big, 0, 3 * big, 4 * big, 4, 8, 48, 128, 128,
                                None) == gdn.GDN_ERR_INVALID_ARG
    assert L.gdn_state_rollback(big, 2 * big, 3, big, 4 * big, 4, 8, 48, 128, 128,
                                None) == gdn.GDN_ERR_INVALID_ARG    # snapshots overlap the pool


def test_gated_norm_rejects_bad_arguments():
    L = gdn.lib()
    big = 1 << 40
    assert L.gdn_gated_norm(big, 2 * big, 3 * big, 10, 64, 1e-6, 4 * big, None) == gdn.GDN_ERR_UNSUPPORTED
    assert L.gdn_gated_norm(big, 2 * big, 3 * big, 10, 128, float("nan"), 4 * big, None) == gdn.GDN_ERR_INVALID_ARG
    assert L.gdn_gated_norm(big, 2 * big, 3 * big, 10, 128, 1e-6, big + 64, None) == gdn.GDN_ERR_INVALID_ARG
    assert L.gdn_gated_norm(big, 2 * big, 3 * big, 10, 128, 1e-6, 2 * big, None) == gdn.GDN_ERR_INVALID_ARG
    assert L.gdn_gated_norm(None, None, None, 0, 128, 1e-6, None, None) == gdn.GDN_OK


def _backward(L, **kw):
    """gdn_prefill_backward with fake (never dereferenced) device pointers that
    do not overlap; the host checks reject before any device call."""
    a = dict(q=0x10000000, k=0x20000000, v=0x30000000, g=0x40000000, beta=0x50000000, S0=None,
             cu=None, d_o=0x60000000, dSf=None, N=1, T=64, H_qk=16, H_v=48, d_k=128, d_v=128,
             scale=1.0, dq=0x70000000, dk=0x80000000, dv=0x90000000, dg=0xA0000000,
             db=0xB0000000, dS0=None, ws=0xC0000000, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return L.gdn_prefill_backward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["cu"],
                                  a["d_o"], a["dSf"], a["N"], a["T"], a["H_qk"], a["H_v"],
                                  a["d_k"], a["d_v"], a["scale"], a["dq"], a["dk"], a["dv"],
                                  a["dg"], a["db"], a["dS0"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d_k=64), gdn.GDN_ERR_UNSUPPORTED),
    (dict(H_v=47), gdn.GDN_ERR_INVALID_ARG),
    (dict(H_qk=1, H_v=16), gdn.GDN_ERR_UNSUPPORTED),
    (dict(dq=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(d_o=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(scale=float("nan")), gdn.GDN_ERR_INVALID_ARG),
    (dict(ws_bytes=16), gdn.GDN_ERR_WORKSPACE),
    (dict(ws=None), gdn.GDN_ERR_WORKSPACE),
    (dict(dq=0x10000000), gdn.GDN_ERR_INVALID_ARG),            # dq overlaps q
    (dict(dv=0x80000000), gdn.GDN_ERR_INVALID_ARG),            # dv overlaps dk
    (dict(ws=0x60000000), gdn.GDN_ERR_INVALID_ARG),            # workspace overlaps d_o
    (dict(N=2), gdn.GDN_ERR_INVALID_ARG),                      # N > 1 needs cu_seqlens
])
def test_prefill_backward_rejects_bad_arguments(kw, code):
    assert _backward(gdn.lib(), **kw) == code


def test_backward_workspace_sizes():
    L = gdn.lib()
    assert gdn.gdn_prefill_backward_workspace_size(1, 0, 16, 48) > 0
    assert gdn.gdn_prefill_backward_workspace_size(0, 64, 16, 48) == 0
    a = gdn.gdn_prefill_backward_workspace_size(1, 32768, 16, 48)
    assert a > gdn.gdn_prefill_backward_workspace_size(1, 4096, 16, 48)
    assert gdn.gdn_layer_prefill_backward_workspace_size(1, 32768, 16, 48) > a
    assert L.gdn_layer_prefill_backward_workspace_size(1, -1, 16, 48, 128, 128) == 0


def _layer_backward(L, **kw):
    a = dict(x=0x10000000, w=0x18000000, a=0x20000000, b=0x28000000, A=0x30000000,
             dt=0x30100000, eps=1e-6, S0=None, cu=None, d_o=0x40000000, dSf=None, N=1, T=64,
             H_qk=16, H_v=48, d_k=128, d_v=128, scale=1.0, dx=0x50000000, dw=0x58000000,
             da=0x60000000, db=0x68000000, dA=0x70000000, ddt=0x70100000, dS0=None,
             ws=0x80000000, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return L.gdn_layer_prefill_backward(
        a["x"], a["w"], a["a"], a["b"], a["A"], a["dt"], a["eps"], a["S0"], a["cu"], a["d_o"],
        a["dSf"], a["N"], a["T"], a["H_qk"], a["H_v"], a["d_k"], a["d_v"], a["scale"], a["dx"],
        a["dw"], a["da"], a["db"], a["dA"], a["ddt"], a["dS0"], a["ws"], a["ws_bytes"],
        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d_v=64), gdn.GDN_ERR_UNSUPPORTED),
    (dict(eps=-1.0), gdn.GDN_ERR_INVALID_ARG),
    (dict(w=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(dA=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(dx=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(ws_bytes=1024), gdn.GDN_ERR_WORKSPACE),
    (dict(dx=0x10000000), gdn.GDN_ERR_INVALID_ARG),            # dx overlaps x
    (dict(db=0x60000000), gdn.GDN_ERR_INVALID_ARG),            # db overlaps da
])
def test_layer_backward_rejects_bad_arguments(kw, code):
    assert _layer_backward(gdn.lib(), **kw) == code


def test_gated_norm_backward_rejects_bad_arguments():
    L = gdn.lib()
    o, z, w, dy, d_o, dz, dw, ws = (0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000,
                                    0x60000000, 0x70000000, 0x80000000)

    def call(**kw):
        a = dict(o=o, z=z, w=w, dy=dy, rows=64, d_v=128, eps=1e-6, d_o=d_o, dz=dz, dw=dw, ws=ws,
                 ws_bytes=1 << 30)
        a.update(kw)
        return L.gdn_gated_norm_backward(a["o"], a["z"], a["w"], a["dy"], a["rows"], a["d_v"],
                                         a["eps"], a["d_o"], a["dz"], a["dw"], a["ws"],
                                         a["ws_bytes"], None)

    assert call(d_v=64) == gdn.GDN_ERR_UNSUPPORTED
    assert call(rows=-1) == gdn.GDN_ERR_INVALID_ARG
    assert call(eps=float("inf")) == gdn.GDN_ERR_INVALID_ARG
    assert call(dw=None) == gdn.GDN_ERR_INVALID_ARG
    assert call(dy=None) == gdn.GDN_ERR_INVALID_ARG
    assert call(ws_bytes=8) == gdn.GDN_ERR_WORKSPACE
    assert call(d_o=o) == gdn.GDN_ERR_INVALID_ARG              # d_o overlaps o
    assert call(dz=d_o) == gdn.GDN_ERR_INVALID_ARG             # dz overlaps d_o
    assert L.gdn_gated_norm_backward_workspace_size(64, 128) > 0
    assert L.gdn_gated_norm_backward_workspace_size(64, 64) == 0


def _prefill_save(L, **kw):
    """gdn_prefill_save_states with far-apart fake device addresses (rejected
    on the host before any device call)."""
    a = dict(q=0x10000000, k=0x20000000, v=0x30000000, g=0x40000000, beta=0x50000000, S0=None,
             Sf=None, cu=None, N=1, T=64, H_qk=16, H_v=48, d_k=128, d_v=128, scale=1.0,
             o=0x60000000, cs=0x1000000000, cs_bytes=1 << 40, ws=0x70000000, ws_bytes=1 << 28,
             stream=None)
    a.update(kw)
    return L.gdn_prefill_save_states(a["q"], a["k"], a["v"], a["g"], a["beta"], a["S0"], a["Sf"],
                                     a["cu"], a["N"], a["T"], a["H_qk"], a["H_v"], a["d_k"],
                                     a["d_v"], a["scale"], a["o"], a["cs"], a["cs_bytes"], a["ws"],
                                     a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cs=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(cs_bytes=1024), gdn.GDN_ERR_INVALID_ARG),
    (dict(cs=0x10000000), gdn.GDN_ERR_INVALID_ARG),            # chunk_states overlaps q
    (dict(cs=0x70000000), gdn.GDN_ERR_INVALID_ARG),            # chunk_states overlaps the workspace
    (dict(d_k=64), gdn.GDN_ERR_UNSUPPORTED),
    (dict(ws_bytes=16), gdn.GDN_ERR_WORKSPACE),
])
def test_prefill_save_states_rejects_bad_arguments(kw, code):
    L = gdn.lib()
    assert _prefill_save(L, **kw) == code
    assert L.gdn_last_error().decode()


def _prefill_raw_save(L, **kw):
    a = dict(x=0x10000000, w=0x20000000, eps=1e-6, g=0x40000000, beta=0x50000000, S0=None,
             Sf=None, cu=None, N=1, T=64, H_qk=16, H_v=48, d_k=128, d_v=128, scale=1.0,
             o=0x60000000, cs=0x1000000000, cs_bytes=1 << 40, ws=0x70000000, ws_bytes=1 << 28,
             stream=None)
    a.update(kw)
    return L.gdn_prefill_raw_save_states(a["x"], a["w"], a["eps"], a["g"], a["beta"], a["S0"],
                                         a["Sf"], a["cu"], a["N"], a["T"], a["H_qk"], a["H_v"],
                                         a["d_k"], a["d_v"], a["scale"], a["o"], a["cs"],
                                         a["cs_bytes"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cs=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(cs_bytes=1024), gdn.GDN_ERR_INVALID_ARG),
    (dict(cs=0x10000000), gdn.GDN_ERR_INVALID_ARG),            # chunk_states overlaps x
    (dict(eps=-1.0), gdn.GDN_ERR_INVALID_ARG),
])
def test_prefill_raw_save_states_rejects_bad_arguments(kw, code):
    assert _prefill_raw_save(gdn.lib(), **kw) == code


def _backward_saved(L, **kw):
    a = dict(q=0x10000000, k=0x20000000, v=0x30000000, g=0x40000000, beta=0x50000000,
             cs=0x1000000000, cs_bytes=1 << 40, cu=None, d_o=0x60000000, dSf=None, N=1, T=64,
             H_qk=16, H_v=48, d_k=128, d_v=128, scale=1.0, dq=0x70000000, dk=0x80000000,
             dv=0x90000000, dg=0xA0000000, db=0xB0000000, dS0=None, ws=0xC0000000,
             ws_bytes=1 << 34, stream=None)
    a.update(kw)
    return L.gdn_prefill_backward_saved(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cs"],
                                        a["cs_bytes"], a["cu"], a["d_o"], a["dSf"], a["N"], a["T"],
                                        a["H_qk"], a["H_v"], a["d_k"], a["d_v"], a["scale"],
                                        a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dS0"],
                                        a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cs=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(cs_bytes=1024), gdn.GDN_ERR_INVALID_ARG),
    (dict(dq=0x1000000000), gdn.GDN_ERR_INVALID_ARG),          # dq overlaps chunk_states
    (dict(ws=0x1000000000), gdn.GDN_ERR_INVALID_ARG),          # workspace overlaps chunk_states
    (dict(ws_bytes=1024), gdn.GDN_ERR_WORKSPACE),
    (dict(dq=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(H_v=47), gdn.GDN_ERR_INVALID_ARG),
])
def test_prefill_backward_saved_rejects_bad_arguments(kw, code):
    assert _backward_saved(gdn.lib(), **kw) == code


def test_chunk_states_and_saved_workspace_sizes():
    assert gdn.gdn_chunk_states_size(1, 32768, 48) == (512 + 1) * 48 * 128 * 128 * 2
    assert gdn.gdn_chunk_states_size(3, 100, 48) == (2 + 3) * 48 * 128 * 128 * 2
    assert gdn.gdn_chunk_states_size(1, 0, 48) == 48 * 128 * 128 * 2
    assert gdn.gdn_chunk_states_size(0, 64, 48) == 0
    assert gdn.gdn_chunk_states_size(1, 64, 48, 64, 128) == 0
    full = gdn.gdn_prefill_backward_workspace_size(1, 32768, 16, 48)
    saved = gdn.gdn_prefill_backward_saved_workspace_size(1, 32768, 16, 48)
    # the saved form drops the states and the forward records
    assert 0 < saved < full - gdn.gdn_chunk_states_size(1, 32768, 48)
    assert gdn.gdn_prefill_backward_saved_workspace_size(0, 64, 16, 48) == 0


def _layer_prefill_save(L, **kw):
    a = dict(x=0x10000000, w=0x18000000, a=0x20000000, b=0x28000000, A=0x30000000,
             dt=0x30100000, eps=1e-6, S0=None, Sf=None, conv=None, cu=None, N=1, T=64, H_qk=16,
             H_v=48, d_k=128, d_v=128, scale=1.0, o=0x40000000, cs=0x1000000000,
             cs_bytes=1 << 40, ws=0x80000000, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.gdn_layer_prefill_save_states(
        a["x"], a["w"], a["a"], a["b"], a["A"], a["dt"], a["eps"], a["S0"], a["Sf"], a["conv"],
        a["cu"], a["N"], a["T"], a["H_qk"], a["H_v"], a["d_k"], a["d_v"], a["scale"], a["o"],
        a["cs"], a["cs_bytes"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cs=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(cs_bytes=1024), gdn.GDN_ERR_INVALID_ARG),
    (dict(cs=0x20000000), gdn.GDN_ERR_INVALID_ARG),            # chunk_states overlaps a
    (dict(ws_bytes=16), gdn.GDN_ERR_WORKSPACE),
])
def test_layer_prefill_save_states_rejects_bad_arguments(kw, code):
    assert _layer_prefill_save(gdn.lib(), **kw) == code


def _layer_backward_saved(L, **kw):
    a = dict(x=0x10000000, w=0x18000000, a=0x20000000, b=0x28000000, A=0x30000000,
             dt=0x30100000, eps=1e-6, cs=0x1000000000, cs_bytes=1 << 40, cu=None,
             d_o=0x40000000, dSf=None, N=1, T=64, H_qk=16, H_v=48, d_k=128, d_v=128, scale=1.0,
             dx=0x50000000, dw=0x58000000, da=0x60000000, db=0x68000000, dA=0x70000000,
             ddt=0x70100000, dS0=None, ws=0x80000000, ws_bytes=1 << 36, stream=None)
    a.update(kw)
    return L.gdn_layer_prefill_backward_saved(
        a["x"], a["w"], a["a"], a["b"], a["A"], a["dt"], a["eps"], a["cs"], a["cs_bytes"], a["cu"],
        a["d_o"], a["dSf"], a["N"], a["T"], a["H_qk"], a["H_v"], a["d_k"], a["d_v"], a["scale"],
        a["dx"], a["dw"], a["da"], a["db"], a["dA"], a["ddt"], a["dS0"], a["ws"], a["ws_bytes"],
        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(cs=None), gdn.GDN_ERR_INVALID_ARG),
    (dict(cs_bytes=1024), gdn.GDN_ERR_INVALID_ARG),
    (dict(dx=0x1000000000), gdn.GDN_ERR_INVALID_ARG),          # dx overlaps chunk_states
    (dict(ws_bytes=1024), gdn.GDN_ERR_WORKSPACE),
    (dict(eps=-1.0), gdn.GDN_ERR_INVALID_ARG),
])
def test_layer_backward_saved_rejects_bad_arguments(kw, code):
    assert _layer_backward_saved(gdn.lib(), **kw) == code


def test_layer_saved_workspace_size():
    L = gdn.lib()
    full = gdn.gdn_layer_prefill_backward_workspace_size(1, 32768, 16, 48)
    saved = L.gdn_layer_prefill_backward_saved_workspace_size(1, 32768, 16, 48, 128, 128)
    assert 0 < saved < full
    assert L.gdn_layer_prefill_backward_saved_workspace_size(0, 64, 16, 48, 128, 128) == 0
