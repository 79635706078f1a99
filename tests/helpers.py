"""Shared test helpers: tensor conversion and the parity metric."""
import numpy as np
import torch


def np64(t):
    """Exact float64 copy of a (CPU or device) tensor."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def npw(d):
    return {k: (np64(v) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def cuda(d):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


TOL = {"f32": 1e-4, "bf16": 2e-2}


def assert_close(got, ref, dtype, what=""):
    e = rel_err(got, ref)
    assert e <= TOL[dtype], f"{what}: max rel err {e:.3e} > {TOL[dtype]:.0e}"
    return e
