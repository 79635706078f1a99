"""Several canvases in one forward (dg_canvas_step_batch) against each canvas
stepped alone (dg_canvas_step, itself checked against the oracle), and one
batched canvas against the oracle directly.

The batched products run over more rows, so their tiling and split-K may
differ from the single-canvas run: logits and u are compared at the fp32
bar; tokens and commits bit for bit where the oracle-side entropy is more
than 1e-3 nats from the bound.
"""
import math

import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from oracle import dg_oracle as O
from tests.helpers import assert_close, np64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    torch.manual_seed(0)
    yield


def sync():
    torch.cuda.synchronize()


def test_batch_equals_single_canvases():
    from tests.test_gpu_parity import gpu_weights, oracle_weights, tiny_model
    mcfg, w = tiny_model("f32")
    model = B.Model(mcfg, gpu_weights(w))
    V, C, D = mcfg["vocab"], 32, mcfg["hidden"]
    prompts = [synth.tokens(n, V, synth.generator(10 + i)).cuda() for i, n in enumerate((64, 32, 96))]
    nb = len(prompts)

    def fresh_caches():
        kvs = []
        for p in prompts:
            kv = B.KV(mcfg, 160)
            B.dg_commit_canvas(model, kv, p)
            kvs.append(kv)
        return kvs

    def scfg(b, step):
        t = (2.0, 1.0, 0.7)[b]
        return synth.sampler_cfg(V, t_max=t, t_min=0.5, n_steps=4, step=step, canvas_idx=b)

    # batched
    kvs = fresh_caches()
    batch = B.Canvas(C, D, "f32", keep_logits_vocab=V, n_canvas=nb)
    for b in range(nb):
        batch.tokens[b * C:(b + 1) * C].copy_(B.dg_canvas_noise(C, V, 1, b))
    got = []
    for step in range(2):
        B.dg_canvas_step_batch(model, kvs, batch, [scfg(b, step) for b in range(nb)])
        sync()
        got.append(dict(logits=batch.logits.clone(), tokens=batch.tokens.clone(), u=batch.u.clone(),
                        entropy=batch.entropy.clone(), n_renoised=batch.n_renoised.clone()))
    assert [kv.kv_len for kv in kvs] == [64, 32, 96]     # decode leaves the caches as they were

    # each canvas alone
    kvs1 = fresh_caches()
    for b in range(nb):
        one = B.Canvas(C, D, "f32", keep_logits_vocab=V)
        one.tokens.copy_(B.dg_canvas_noise(C, V, 1, b))
        for step in range(2):
            B.dg_canvas_step(model, kvs1[b], one, scfg(b, step))
            sync()
            g = got[step]
            rows = slice(b * C, (b + 1) * C)
            assert_close(np64(g["logits"][rows]), np64(one.logits), "f32", f"canvas {b} step {step} logits")
            assert_close(np64(g["u"][rows]), np64(one.u), "f32", f"canvas {b} step {step} u")
            H = np64(one.entropy)
            clear = np.abs(H - scfg(b, step)["tau"]) > 1e-3
            np.testing.assert_array_equal(g["tokens"][rows].cpu().numpy()[clear], one.tokens.cpu().numpy()[clear])
            if clear.all():
                assert int(g["n_renoised"][b].item()) == int(one.n_renoised.item())
            # continue the single run from the batched tokens, so both see the same canvas
            one.tokens.copy_(g["tokens"][rows])
            one.u.copy_(g["u"][rows])

    # canvas 2 of the first batched step against the oracle
    wn = oracle_weights(w)
    rkv = dict(k=[np.zeros((2, 160, 64)) for _ in range(2)], v=[np.zeros((2, 160, 64)) for _ in range(2)],
               kv_len=0)
    kn, vn = O.commit_canvas(mcfg, wn, rkv, prompts[2].cpu().numpy(), "f32")
    for l in range(2):
        rkv["k"][l][:, :96], rkv["v"][l][:, :96] = kn[l], vn[l]
    rkv["kv_len"] = 96
    ref = O.canvas_step(mcfg, wn, rkv, dict(tokens=O.canvas_noise(C, V, 1, 2), u=None), scfg(2, 0), "f32")
    assert_close(np64(got[0]["logits"][2 * C:3 * C]), ref["logits"], "f32", "batched canvas 2 vs oracle")
    assert np.max(np.abs(np64(got[0]["entropy"][2 * C:3 * C]) - ref["entropy"])) < 1e-4 * math.log(V)


def test_batch_validation():
    from tests.test_gpu_parity import gpu_weights, tiny_model
    mcfg, w = tiny_model("f32")
    model = B.Model(mcfg, gpu_weights(w))
    V, C = mcfg["vocab"], 32
    kv = B.KV(mcfg, 64)
    batch = B.Canvas(C, mcfg["hidden"], "f32", n_canvas=2)
    full = B.KV(mcfg, 64)
    full.set_len(48)                       # 48 + 32 rows do not fit 64
    with pytest.raises(B.DGError) as e:
        B.dg_canvas_step_batch(model, [kv, full], batch, [synth.sampler_cfg(V)] * 2)
    assert e.value.status == -7


def test_batch_bf16_every_canvas_vs_oracle():
    """bf16 tiny stack, eight canvases of 32 in one forward (cache lengths
    64, 32, 96, 16, 48, 80, 8, 128; eight temperatures at step 0), two steps,
    every canvas against the oracle at the bf16 bar.  The 256 rows fill one
    head tile, so the head's epilogue takes the sampler's row statistics with
    a different temperature for every 32 rows.
    Router logits are injected (the same on both sides) and the QK-norm gains
    drawn from U[0.2, 0.3], so the comparison measures the kernels, not the
    conditioning of a random-init stack."""
    from tests.helpers import check_sampler_outputs
    from tests.test_gpu_parity import gpu_weights, oracle_weights
    mcfg = synth.tiny_model_cfg(dtype="bf16")
    w = synth.model_weights(mcfg, seed=0, gamma_range=(0.2, 0.3))
    model = B.Model(mcfg, gpu_weights(w))
    wn = oracle_weights(w)
    V, C, D, L = mcfg["vocab"], 32, mcfg["hidden"], mcfg["n_layers"]
    lens = (64, 32, 96, 16, 48, 80, 8, 128)
    nb = len(lens)
    prompts = [synth.tokens(n, V, synth.generator(10 + i)) for i, n in enumerate(lens)]
    kvs, rkvs = [], []
    for p in prompts:
        kv = B.KV(mcfg, 160)
        B.dg_commit_canvas(model, kv, p.cuda())
        kvs.append(kv)
        rkv = dict(k=[np.zeros((2, 160, 64)) for _ in range(L)], v=[np.zeros((2, 160, 64)) for _ in range(L)],
                   kv_len=0)
        # (each canvas's own cache; 128 + 32 rows fit 160)
        kn, vn = O.commit_canvas(mcfg, wn, rkv, p.numpy(), "bf16")
        for l in range(L):
            rkv["k"][l][:, :len(p)], rkv["v"][l][:, :len(p)] = kn[l], vn[l]
        rkv["kv_len"] = len(p)
        rkvs.append(rkv)

    def scfg(b, step):
        t = (2.0, 1.0, 0.7, 1.5, 3.0, 0.9, 1.2, 5.0)[b]
        return synth.sampler_cfg(V, t_max=t, t_min=0.5, n_steps=4, step=step, canvas_idx=b)

    batch = B.Canvas(C, D, "bf16", keep_logits_vocab=V, n_canvas=nb)
    tokens = [O.canvas_noise(C, V, 1, b) for b in range(nb)]
    for b in range(nb):
        batch.tokens[b * C:(b + 1) * C].copy_(torch.from_numpy(tokens[b].astype(np.int32)))
    us = [None] * nb
    g = synth.generator(321)
    for step in range(2):
        rl = [synth.router_logits(nb * C, mcfg["moe"]["n_experts"], g) for _ in range(L)]
        model.set_router_logits([t.cuda() for t in rl])
        B.dg_canvas_step_batch(model, kvs, batch, [scfg(b, step) for b in range(nb)])
        sync()
        for b in range(nb):
            rows = slice(b * C, (b + 1) * C)
            s = scfg(b, step)
            wb = dict(wn, router_logits=[t[rows].double().numpy() for t in rl])
            ref = O.canvas_step(mcfg, wb, rkvs[b], dict(tokens=tokens[b], u=us[b]), s, "bf16")
            lg = np64(batch.logits[rows])
            assert_close(lg, ref["logits"], "bf16", f"canvas {b} step {step} logits")
            assert_close(np64(batch.u[rows]), ref["u_next"], "bf16", f"canvas {b} step {step} u")
            dl = float(np.max(np.abs(lg - ref["logits"])))
            dh = float(np.max(np.abs(np64(batch.entropy[rows]) - ref["entropy"])))
            assert dh <= 2e-2 * math.log(V)
            noise = O.renoise_tokens(C, V, s["seed"], s["step"], s["canvas_idx"])
            check_sampler_outputs(batch.tokens[rows].cpu().numpy(), batch.commit[rows].cpu().numpy(), ref,
                                  ref["logits"], noise, s["tau"], band_logit=2 * dl, band_h=2 * dh + 1e-6)
            tokens[b], us[b] = ref["tokens"], ref["u_next"]
            batch.tokens[rows].copy_(torch.from_numpy(tokens[b].astype(np.int32)))
    model.set_router_logits(None)
    assert [kv.kv_len for kv in kvs] == list(lens)
