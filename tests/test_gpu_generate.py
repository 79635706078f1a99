"""The block-autoregressive host loop (generate.py) against the oracle's loop.

aibars.net news, block-autoregressive denoising: commit the prompt, denoise a
noise block, commit it, start the next.  DiffusionGemma Technical Report
review, section 1 (Adaptive Stopping): stop once no position is re-noised,
or once the proposals are stable.  The tiny fp32 model echoes its input
token, so the temperature schedule (45 -> 12 over 6 steps) is what moves
the entropies across the bound: canvases stop after 4-6 steps.  The seeded
case keeps every entropy at least 0.1 nats from the bound and every argmax
lead far above the fp32 error, so steps and tokens must match exactly.
"""
import math

import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from discrete_text_diffusion_step_amd.generate import generate
from oracle import dg_oracle as O
from tests.helpers import assert_close, np64, npw

pytestmark = pytest.mark.gpu

P, C, N_CANVAS, STEPS = 64, 32, 2, 6


@pytest.fixture(scope="module")
def tiny(gpu_lib):
    mcfg = synth.tiny_model_cfg(dtype="f32")
    w = synth.model_weights(mcfg, seed=0)
    wn = dict(embed=np64(w["embed"]), w_final_norm=np64(w["w_final_norm"]), sc=npw(w["sc"]),
              attn=[npw(a) for a in w["attn"]], moe=[npw(m) for m in w["moe"]], layer_scalar=w["layer_scalar"])
    gw = dict(embed=w["embed"].cuda(), w_final_norm=w["w_final_norm"].cuda(),
              sc={k: v.cuda() for k, v in w["sc"].items()},
              attn=[{k: (v.cuda() if v is not None else None) for k, v in a.items()} for a in w["attn"]],
              moe=[{k: (v.cuda() if v is not None else None) for k, v in m.items()} for m in w["moe"]],
              layer_scalar=w["layer_scalar"])
    return mcfg, B.Model(mcfg, gw), wn


@pytest.mark.parametrize("stop_rule,own_stream", [("renoised", False), ("stable", False), ("renoised", True)])
def test_generate_matches_oracle_loop(tiny, stop_rule, own_stream):
    mcfg, model, wn = tiny
    V = mcfg["vocab"]
    tau = 0.5 * math.log(V)
    cap = P + (N_CANVAS + 1) * C
    prompt = synth.tokens(P, V, synth.generator(2))
    kv = B.KV(mcfg, cap)
    stream = torch.cuda.Stream() if own_stream else None
    toks, used = generate(model, kv, prompt.cuda(), N_CANVAS, canvas_len=C, max_steps=STEPS, seed=1, t_max=45.0,
                          t_min=12.0, tau=tau, stream=stream, stop_rule=stop_rule)
    torch.cuda.synchronize()
    L = mcfg["n_layers"]
    kv0 = dict(k=[np.zeros((2, cap, 64)) for _ in range(L)], v=[np.zeros((2, cap, 64)) for _ in range(L)], kv_len=0)
    ref = O.generate(mcfg, wn, kv0, prompt.numpy(), N_CANVAS, C, STEPS, 1, 45.0, 12.0, tau, "f32",
                     stop_rule=stop_rule)
    # the seeded case decides nothing inside a floating-point band
    assert ref["min_entropy_gap"] > 1e-2 and ref["min_lead"] > 1.0
    assert used == ref["steps"], (used, ref["steps"])
    assert 1 < min(used) and max(used) <= STEPS
    np.testing.assert_array_equal(toks.cpu().numpy(), ref["tokens"])
    assert kv.kv_len == P + N_CANVAS * C
    n = kv.kv_len
    for l in range(L):
        assert_close(np64(kv.k[l])[:, :n], ref["kv"]["k"][l][:, :n], "f32", f"k[{l}]")
        assert_close(np64(kv.v[l].transpose(1, 2))[:, :n], ref["kv"]["v"][l][:, :n], "f32", f"v[{l}]")
