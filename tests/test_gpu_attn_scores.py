"""bf16 attention with wide score ranges against the oracle.

The kernel's online softmax keeps a reference maximum per query that moves
only when a score exceeds it by more than a fixed slack, and masks scores
only in tiles cut by the key range, the causal diagonal or the window.  With
QK-norm gains of 2 the scores spread over hundreds of nats, so the running
maximum jumps by more than the slack many times along the keys and creeps
below it in between; the layer output must still match the oracle's plain
softmax.  Also run: a key range that starts and ends inside a tile on both
sides (decode with a sliding window that cuts mid-tile) and a causal encode.
"""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from oracle import dg_oracle as O
from tests.helpers import assert_delta_close, cuda, np64, npw

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    torch.manual_seed(0)
    yield


def run(cfg, w, ck, cv, P, x, causal):
    xd = x.clone().cuda()
    kd, vtd = ck.cuda(), cv.transpose(1, 2).contiguous().cuda()
    B.dg_attn_layer(cfg, cuda(w), kd, vtd, P, xd, causal)
    torch.cuda.synchronize()
    return xd


@pytest.mark.parametrize("kind,P,n_tok,causal", [
    ("global", 4096, 256, 0),     # the canvas step's global layer shape
    ("sliding", 1500, 200, 0),    # window 1024 cuts the key range mid-tile
    ("sliding", 100, 300, 1),     # causal encode: diagonal and window tiles
])
def test_wide_scores(kind, P, n_tok, causal):
    cfg = synth.global_cfg() if kind == "global" else synth.sliding_cfg()
    if causal:
        cfg = dict(cfg, window=128)
    g = synth.generator(91 + P)
    w = synth.attn_weights(cfg, g, gamma=(2.0, 2.0))
    cap = (P + n_tok + 31) // 32 * 32
    ck, cv = synth.kv_cache_random(cfg["n_kv_heads"], cap, cfg["head_dim"], g, "bf16")
    x = synth.hidden_states(n_tok, cfg["hidden"], g, "bf16")
    xo = run(cfg, w, ck, cv, P, x, causal)
    ref, _, _ = O.attn_layer(cfg, npw(w), np64(ck), np64(cv), P, np64(x), causal, "bf16")
    assert np.isfinite(np64(xo)).all()
    e = assert_delta_close(np64(xo), ref, np64(x), "bf16", f"{kind} P={P} causal={causal}")
    print(f"{kind} P={P} n={n_tok} causal={causal}: rel err of the update {e:.2e}")


def test_scores_rising_along_the_keys():
    """Committed keys scaled from 1x to 8x across the sliding window (QK-norm
    gains of 2): within every key slice the later tiles' scores pass the
    first tile's maximum by far more than 32 nats, which is where a kernel
    whose softmax keeps a fixed reference must re-run the slice against the
    exact maximum.  The layer output must match the oracle's plain softmax."""
    cfg = synth.sliding_cfg()
    P, n_tok = 2048, 256
    g = synth.generator(97)
    w = synth.attn_weights(cfg, g, gamma=(2.0, 2.0))
    cap = P + n_tok
    ck, cv = synth.kv_cache_random(cfg["n_kv_heads"], cap, cfg["head_dim"], g, "bf16")
    lo = P - cfg["window"]
    ramp = torch.ones(cap)
    ramp[lo:P] = torch.linspace(1.0, 8.0, P - lo)
    ck = (ck.float() * ramp[None, :, None]).to(torch.bfloat16)
    x = synth.hidden_states(n_tok, cfg["hidden"], g, "bf16")
    xo = run(cfg, w, ck, cv, P, x, 0)
    ref, _, _ = O.attn_layer(cfg, npw(w), np64(ck), np64(cv), P, np64(x), 0, "bf16")
    assert np.isfinite(np64(xo)).all()
    e = assert_delta_close(np64(xo), ref, np64(x), "bf16", "rising scores")
    print(f"rising key scale: rel err of the update {e:.2e}")
