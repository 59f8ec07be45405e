"""Helpers shared by the GPU parity tests (data movement and error metrics only)."""

import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def lib():
    import context_long_sequence_amd as ra

    ra.load()  # raises if the HIP library was not built: the GPU tests never run without it
    return ra


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device()).to(dtype)


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def rel_to_max(a, ref):
    ref = np.asarray(ref, np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    return max_abs(a, ref) / max(m, 1e-30)


def lse_close(got, ref, atol):
    """Finite entries within atol; +-inf entries must match exactly."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf_ref = ~np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), ~inf_ref), "LSE -inf pattern differs"
    assert np.all(got[inf_ref] == ref[inf_ref])
    fin = ~inf_ref
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= atol, f"LSE max-abs {err:.3e} > {atol:.1e}"
    return err


def report(name, **vals):
    print(f"[{name}] " + "  ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}" for k, v in vals.items()),
          flush=True)
