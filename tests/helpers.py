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


def top2(logits):
    """Per row: the largest value and its lead over the runner-up."""
    part = -np.partition(-np.asarray(logits, np.float64), 1, axis=1)[:, :2]
    return part[:, 0], part[:, 0] - part[:, 1]


def check_sampler_outputs(tokens, commit, ref, ref_logits, noise, tau, band_logit, band_h):
    """Sampler outputs of a step whose logits differ from the oracle's by up
    to band_logit / 2 (band_h / 2 for the entropies).

    Commit decisions are exact where the oracle's entropy is more than band_h
    from tau; inside that band either decision is valid.  A committed
    position holds the argmax: exact where the oracle's best logit leads by
    more than band_logit, else a token within band_logit of the oracle's best.
    A re-noised position holds exactly its Philox token.
    Returns the number of positions decided inside a band."""
    tokens = np.asarray(tokens).astype(np.int64)
    commit = np.asarray(commit).astype(bool)
    H = ref["entropy"]
    clear_h = np.abs(H - tau) > band_h
    np.testing.assert_array_equal(commit[clear_h], ref["commit"][clear_h])
    best, lead = top2(ref_logits)
    rows = np.arange(len(tokens))
    c = commit
    assert (tokens[~c] == np.asarray(noise)[~c]).all(), "re-noised positions must hold their Philox token"
    exact = c & (lead > band_logit)
    np.testing.assert_array_equal(tokens[exact], ref["argmax"][exact])
    near = c & ~exact
    if near.any():
        got = np.asarray(ref_logits, np.float64)[rows[near], tokens[near]]
        assert (got >= best[near] - band_logit).all(), "a committed token outside the argmax band"
    return int((~clear_h).sum() + near.sum())


def check_router_sets(idx, ref_idx, ref_logits, k, band=1e-3):
    """Top-k expert sets: equal to the oracle's (in order) where its k-th and
    (k+1)-th logits are more than `band` apart; elsewhere the two sets may
    differ only by experts within `band` of the oracle's k-th logit."""
    idx = np.asarray(idx)
    srt = -np.sort(-np.asarray(ref_logits, np.float64), axis=1)
    clear = (srt[:, k - 1] - srt[:, k]) > band
    np.testing.assert_array_equal(idx[clear], ref_idx[clear])
    for t in np.nonzero(~clear)[0]:
        diff = set(idx[t].tolist()) ^ set(ref_idx[t].tolist())
        kth = srt[t, k - 1]
        assert all(abs(ref_logits[t, e] - kth) <= band for e in diff), (t, diff)
    return clear
