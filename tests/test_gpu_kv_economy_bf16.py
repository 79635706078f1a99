"""bf16 stack at the canvas head dimensions (sliding d_h 256, global d_h 512
with W_v = W_k and rotary 0.25) with the KV economies on: sliding layers in
a ring that wraps during the prompt commit, global layers keeping only V.

The ring is a storage layout: the same keys in the same order, so the steps
must equal the plain caches' bit for bit.  Value-only keys are rebuilt from
the stored bf16 values (K = RoPE_p(gamma_k * V)), which rounds differently
from the projection's own keys, so that run is compared with the plain one at
the bf16 bar.  Two canvases per forward with both economies are compared with
each canvas stepped alone.  The plain stack itself is checked against the
oracle by the whole-stack tests.
"""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from tests.helpers import assert_close, np64

pytestmark = pytest.mark.gpu

C, PROMPT, CHUNK = 256, 768, 256


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


def model():
    D = 1024
    mcfg = synth.model_cfg(synth.attn_cfg(D, 8, 4, 256, 0, window=256),
                           synth.attn_cfg(D, 8, 1, 512, 1, rope_base=1e6, rotary_factor=0.25),
                           synth.moe_cfg(D, 16, 4, 256, 256), n_layers=6, global_every=3, vocab=8192,
                           sc_ffn=256)
    # QK-norm gains in the stable range of the whole-stack tests
    w = synth.model_weights(mcfg, seed=5, device="cuda", gamma_range=(0.2, 0.3))
    return mcfg, B.Model(mcfg, w)


def run(mcfg, m, prompts, ring, v_only, batch):
    """Commit each prompt in 256-token chunks, then two steps of its canvas
    (all canvases in one forward when batch); returns per canvas the logits,
    tokens and u of both steps."""
    V = mcfg["vocab"]
    n = len(prompts)
    kvs = [B.KV(mcfg, PROMPT + C, ring_tokens=CHUNK if ring else 0, v_only_global=v_only) for _ in range(n)]
    for kv, p in zip(kvs, prompts):
        for p0 in range(0, PROMPT, CHUNK):
            B.dg_commit_canvas(m, kv, p[p0:p0 + CHUNK])
    if ring:
        assert kvs[0].k[0].shape[1] == B.ring_capacity(256, CHUNK) < PROMPT
    groups = [list(range(n))] if batch else [[b] for b in range(n)]
    out = {}
    for grp in groups:
        cv = B.Canvas(C, mcfg["hidden"], "bf16", keep_logits_vocab=V, n_canvas=len(grp))
        for i, b in enumerate(grp):
            cv.tokens[i * C:(i + 1) * C].copy_(B.dg_canvas_noise(C, V, 1, b))
        steps = []
        for step in range(2):
            scs = [synth.sampler_cfg(V, t_max=40.0, t_min=10.0, n_steps=4, step=step, canvas_idx=b) for b in grp]
            if len(grp) > 1:
                B.dg_canvas_step_batch(m, [kvs[b] for b in grp], cv, scs)
            else:
                B.dg_canvas_step(m, kvs[grp[0]], cv, scs[0])
            torch.cuda.synchronize()
            steps.append((cv.logits.cpu().clone(), cv.tokens.cpu().clone(), cv.u.float().cpu().clone()))
        for i, b in enumerate(grp):
            out[b] = [(lg[i * C:(i + 1) * C], tk[i * C:(i + 1) * C], u[i * C:(i + 1) * C]) for lg, tk, u in steps]
    return out


def test_ring_and_value_only_caches_bf16_stack():
    mcfg, m = model()
    V = mcfg["vocab"]
    prompts = [synth.tokens(PROMPT, V, synth.generator(20 + b)).cuda() for b in range(2)]
    plain = run(mcfg, m, prompts[:1], ring=False, v_only=False, batch=False)
    ring = run(mcfg, m, prompts[:1], ring=True, v_only=False, batch=False)
    for (lp, tp, up), (lr, tr, ur) in zip(plain[0], ring[0]):
        assert torch.equal(lp, lr) and torch.equal(tp, tr) and torch.equal(up, ur)
    econ = run(mcfg, m, prompts[:1], ring=True, v_only=True, batch=False)
    for s, ((lp, tp, up), (le, te, ue)) in enumerate(zip(plain[0], econ[0])):
        assert_close(np64(le), np64(lp), "bf16", f"logits step {s}, value-only + ring vs plain")
        assert_close(np64(ue), np64(up), "bf16", f"u step {s}, value-only + ring vs plain")
        agree = float((te == tp).float().mean())
        assert agree >= 0.98, f"step {s}: tokens agree at {agree:.3f}"
    # two canvases in one forward, both economies on, against each stepped alone
    alone = run(mcfg, m, prompts, ring=True, v_only=True, batch=False)
    both = run(mcfg, m, prompts, ring=True, v_only=True, batch=True)
    for b in range(2):
        for s, ((la, ta, ua), (lb, tb, ub)) in enumerate(zip(alone[b], both[b])):
            assert_close(np64(lb), np64(la), "bf16", f"canvas {b} step {s} logits, batched vs alone")
            assert_close(np64(ub), np64(ua), "bf16", f"canvas {b} step {s} u, batched vs alone")
            assert float((tb == ta).float().mean()) >= 0.98
