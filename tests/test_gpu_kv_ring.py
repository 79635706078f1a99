"""Sliding-layer ring cache: position m at row m mod capacity.

The ring is a storage layout, not arithmetic: the same keys are read in the
same order and the split-KV plan depends only on key counts, so the ring
path must give bit-identical results to the plain cache.  The plain path is
itself checked against the oracle (test_gpu_parity.py); here the ring runs
are compared bit for bit with it, and the long-context case also with the
oracle at the bf16 bar.
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


def sync():
    torch.cuda.synchronize()


def run_layer_sequence(cfg, w, chunks, canvas, cap, ring):
    """Encode `chunks` one call each, then decode `canvas`; returns the outputs."""
    Hkv, dh = cfg["n_kv_heads"], cfg["head_dim"]
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    kd = torch.zeros(Hkv, cap, dh, dtype=dt, device="cuda")
    vd = torch.zeros(Hkv, dh, cap, dtype=dt, device="cuda")
    outs, P = [], 0
    for x in chunks:
        xd = x.clone().cuda()
        P = B.dg_attn_layer(cfg, cuda(w), kd, vd, P, xd, 1, ring=ring)
        outs.append(xd)
    xd = canvas.clone().cuda()
    B.dg_attn_layer(cfg, cuda(w), kd, vd, P, xd, 0, ring=ring)
    sync()
    return outs, xd, P


@pytest.mark.parametrize("dtype,window,chunk,n_chunks,canvas", [
    ("f32", 32, 16, 9, 16),      # tiny layer: the ring (64 rows) wraps twice
    ("bf16", 1024, 256, 6, 256),  # canvas shape: 1,536 committed positions through a 1,280-row ring
])
def test_ring_equals_plain_cache(dtype, window, chunk, n_chunks, canvas):
    if dtype == "f32":
        cfg = synth.tiny_attn_cfg(0, "f32")
        cfg["window"] = window
    else:
        cfg = dict(synth.sliding_cfg(), window=window)
    g = synth.generator(81)
    w = synth.attn_weights(cfg, g)
    chunks = [synth.hidden_states(chunk, cfg["hidden"], g, dtype) for _ in range(n_chunks)]
    xc = synth.hidden_states(canvas, cfg["hidden"], g, dtype)
    total = chunk * n_chunks + canvas
    plain_o, plain_c, P1 = run_layer_sequence(cfg, w, chunks, xc, (total + 31) // 32 * 32, False)
    ring_cap = B.ring_capacity(window, max(chunk, canvas))
    assert ring_cap < total
    ring_o, ring_c, P2 = run_layer_sequence(cfg, w, chunks, xc, ring_cap, True)
    assert P1 == P2 == chunk * n_chunks
    for a, b in zip(plain_o, ring_o):
        assert torch.equal(a, b)
    assert torch.equal(plain_c, ring_c)


def test_ring_long_context_against_oracle():
    """bf16 sliding layer: 2,048 committed positions through a 1,280-row ring,
    then the 256-token canvas; the oracle keeps the whole cache."""
    cfg = synth.sliding_cfg()
    g = synth.generator(83)
    w = synth.attn_weights(cfg, g)
    Hkv, dh = cfg["n_kv_heads"], cfg["head_dim"]
    chunks = [synth.hidden_states(256, cfg["hidden"], g, "bf16") for _ in range(8)]
    xc = synth.hidden_states(256, cfg["hidden"], g, "bf16")
    _, xo, P = run_layer_sequence(cfg, w, chunks, xc, B.ring_capacity(1024, 256), True)
    wn = npw(w)
    rk, rv = np.zeros((Hkv, P + 256, dh)), np.zeros((Hkv, P + 256, dh))
    p = 0
    for x in chunks:
        _, k, v = O.attn_layer(cfg, wn, rk, rv, p, np64(x), 1, "bf16")
        rk[:, p:p + 256], rv[:, p:p + 256] = k, v
        p += 256
    ref, _, _ = O.attn_layer(cfg, wn, rk, rv, P, np64(xc), 0, "bf16")
    assert_delta_close(np64(xo), ref, np64(xc), "bf16", "ring decode delta")


def test_tiny_model_ring_steps_equal_plain():
    """Whole tiny model: a chunked prompt commit and two denoising steps with
    ring caches on the sliding layers give the same logits and tokens as
    the plain caches."""
    from tests.test_gpu_parity import gpu_weights, tiny_model
    mcfg, w = tiny_model("f32")
    model = B.Model(mcfg, gpu_weights(w))
    V, C = mcfg["vocab"], 32
    prompt = synth.tokens(160, V, synth.generator(2)).cuda()
    res = []
    for ring_tokens in (0, 32):
        kv = B.KV(mcfg, 256, ring_tokens=ring_tokens)
        for p0 in range(0, 160, 32):
            B.dg_commit_canvas(model, kv, prompt[p0:p0 + 32])
        canvas = B.Canvas(C, mcfg["hidden"], "f32", keep_logits_vocab=V)
        canvas.tokens.copy_(B.dg_canvas_noise(C, V, 1, 0))
        out = []
        for step in range(2):
            s = synth.sampler_cfg(V, t_max=2.0, t_min=0.5, n_steps=4, step=step)
            B.dg_canvas_step(model, kv, canvas, s)
            sync()
            out.append((canvas.logits.clone(), canvas.tokens.clone()))
        res.append(out)
        if ring_tokens:
            assert kv.k[0].shape[1] == B.ring_capacity(mcfg["sliding"]["window"], 32) < 160
    for (la, ta), (lb, tb) in zip(*res):
        assert torch.equal(la, lb) and torch.equal(ta, tb)
