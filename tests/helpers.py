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


def bf16_ulp(v):
    """Spacing of bfloat16 numbers at |v| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def assert_delta_close(got_out, ref_out, x_in, dtype, what=""):
    """Compare a residual update (out - x) at the delta's own scale.  Both sides
    round x + delta to the storage dtype; where their fp32/fp64 deltas straddle
    a rounding boundary the stored outputs differ by one unit in the last place
    of the output, so that much is forgiven element by element."""
    got_out = np.asarray(got_out, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    slack = bf16_ulp(ref_out) if dtype == "bf16" else 0.0
    diff = np.maximum(np.abs(got_out - ref_out) - slack, 0.0)
    den = np.max(np.abs(ref_out - np.asarray(x_in, np.float64)))
    e = float(np.max(diff) / (den if den > 0 else 1.0))
    assert e <= TOL[dtype], f"{what}: max rel err of the update {e:.3e} > {TOL[dtype]:.0e}"
    return e
