"""Shared helpers for the GPU parity tests (not a test module)."""
import sys

import numpy as np
import pytest

# Parity bar: bf16 inputs with fp32 accumulation -> max-abs 2e-2 and rel-L2 5e-3;
# fp32 inputs -> max-abs 1e-4.
TOL = {"bf16": (2e-2, 5e-3), "fp32": (1e-4, None)}


def device():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tdt(dtype):
    import torch
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]


def to_dev(x, dtype=None, dev=None):
    """NumPy array -> device tensor; q/k/v arrays already hold dtype-exact values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(tdt(dtype))
    return t.to(dev or "cuda:0").contiguous()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def metrics(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    max_abs = float(np.max(np.abs(d), initial=0.0))
    den = float(np.sqrt(np.sum(ref * ref)))
    rel = float(np.sqrt(np.sum(d * d)) / den) if den > 0 else float(np.sqrt(np.sum(d * d)))
    return max_abs, rel


def check(name, got, ref, dtype):
    max_abs, rel = metrics(got, ref)
    tol_abs, tol_rel = TOL[dtype]
    say(f"[parity] {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} ({dtype})")
    assert np.all(np.isfinite(np.asarray(got))), f"{name}: non-finite values"
    assert max_abs <= tol_abs, f"{name}: max_abs {max_abs:.3e} > {tol_abs}"
    if tol_rel is not None:
        assert rel <= tol_rel, f"{name}: rel_l2 {rel:.3e} > {tol_rel}"
    return max_abs, rel
