"""Shared test helpers: host<->device marshalling and the parity metrics."""
import numpy as np

# Parity bars: normalised max-abs and RMS-relative error, per output.
TOL_F32 = 1e-4     # fp32 io
TOL_BF16 = 2e-2    # bf16 io, fp32 state


def dev(a, device="cuda"):
    """numpy -> torch on the GPU; uint16 arrays are bf16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host(t):
    """torch -> numpy float64 (bf16 widened exactly)."""
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def errors(x, ref):
    """(normalised max-abs, RMS-relative, raw max-abs) of x against ref."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(x - ref)
    scale = np.max(np.abs(ref))
    e_max = float(d.max() / scale) if scale > 0 else float(d.max())
    nrm = np.linalg.norm(ref)
    e_rms = float(np.linalg.norm(x - ref) / nrm) if nrm > 0 else float(np.linalg.norm(x - ref))
    return e_max, e_rms, float(d.max())


def assert_close(x, ref, tol, what=""):
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    e_max, e_rms, raw = errors(x, ref)
    assert e_max <= tol and e_rms <= tol, (
        f"{what}: normalised max-abs {e_max:.3e}, rms-rel {e_rms:.3e} (raw {raw:.3e}) > {tol}")
    return e_max, e_rms
