"""Value-only caches for global layers against the oracle.

In W_v = W_k layers the stored value is the unit-RMS raw key and the key is
its rotation, K = RoPE_p(k_norm * V) (aitrends attention paragraph: KV
saving / reconstruction; pinned in the oracle tests), so a global layer can
keep V alone and rebuild the committed keys on every call.  The rebuilt keys
are rounded once from the stored values, so they may differ from keys
stored at commit time by one bf16 ulp: results are compared with the oracle
at the bf16 bar (fp32 bar for the fp32 model), not bit for bit.
"""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from oracle import dg_oracle as O
from tests.helpers import assert_close, assert_delta_close, cuda, np64, npw

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("P", [32768, 1000])
def test_global_layer_value_only_cache(P):
    """Global layer at the canvas shape over P committed positions whose
    values are unit-RMS rows and whose keys are consistent with them
    (K = RoPE(gamma_k V), the synthetic 'consistent variant' of the cache):
    the device gets only V; the oracle gets K and V."""
    cfg = synth.global_cfg()
    Hkv, dh = cfg["n_kv_heads"], cfg["head_dim"]
    g = synth.generator(97)
    w = synth.attn_weights(cfg, g)
    raw = np64(synth.hidden_states(Hkv * P, dh, g, "bf16")).reshape(Hkv, P, dh)
    v = O.store(O.rms(raw, 1.0, cfg["rms_eps"]), "bf16")
    freqs = O.rope_freqs(dh, cfg["rope_base"], cfg["rotary_factor"])
    k = O.store(O.rope(np64(w["k_norm"]) * v, np.arange(P), freqs), "bf16")
    cap = P + 256
    ck, cv = np.zeros((Hkv, cap, dh)), np.zeros((Hkv, cap, dh))
    ck[:, :P], cv[:, :P] = k, v
    x = synth.hidden_states(256, cfg["hidden"], g, "bf16")
    xd = x.clone().cuda()
    kd = torch.full((Hkv, cap, dh), float("nan"), dtype=torch.bfloat16, device="cuda")   # scratch: never read stale
    vtd = torch.from_numpy(cv).to(torch.bfloat16).transpose(1, 2).contiguous().cuda()
    n = B.dg_attn_layer(cfg, cuda(w), kd, vtd, P, xd, 0, v_only=True)
    torch.cuda.synchronize()
    assert n == P
    # the rebuilt keys of the committed positions, against the oracle's rotation of the same values
    rebuilt = np64(kd[:, :P])
    assert_close(rebuilt, k, "bf16", "rebuilt keys")
    exact = float(np.mean(rebuilt == k))
    assert exact > 0.95, exact
    ref, _, _ = O.attn_layer(cfg, npw(w), ck, cv, P, np64(x), 0, "bf16")
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "value-only decode delta")


def test_value_only_stack_matches_plain_and_oracle():
    """Tiny fp32 stack of 4 layers (layers 1 and 3 global): the prompt commit
    runs layer 1's causal encode from V alone; then two steps.  Against the
    same stack with plain caches and against the oracle, at the fp32 bar."""
    from tests.test_gpu_parity import gpu_weights, oracle_weights
    mcfg = synth.tiny_model_cfg(n_layers=4, global_every=2, dtype="f32")
    w = synth.model_weights(mcfg, seed=0)
    model = B.Model(mcfg, gpu_weights(w))
    wn = oracle_weights(w)
    V, C, L = mcfg["vocab"], 32, 4
    prompt = synth.tokens(64, V, synth.generator(2))
    runs = {}
    for vo in (False, True):
        kv = B.KV(mcfg, 128, v_only_global=vo)
        B.dg_commit_canvas(model, kv, prompt.cuda())
        canvas = B.Canvas(C, mcfg["hidden"], "f32", keep_logits_vocab=V)
        canvas.tokens.copy_(B.dg_canvas_noise(C, V, 1, 0))
        out = []
        for step in range(2):
            s = synth.sampler_cfg(V, t_max=45.0, t_min=12.0, n_steps=4, step=step)
            B.dg_canvas_step(model, kv, canvas, s)
            torch.cuda.synchronize()
            out.append((canvas.logits.cpu().clone(), canvas.tokens.cpu().clone(), canvas.u.cpu().clone()))
        runs[vo] = (kv, out)
    kv_p, out_p = runs[False]
    kv_v, out_v = runs[True]
    assert kv_v.k[1].data_ptr() == kv_v.k[3].data_ptr()          # one key scratch for both global layers
    for l in (1, 3):   # the values stored by the commit are the same either way
        np.testing.assert_array_equal(kv_v.v[l][:, :, :64].cpu().numpy(), kv_p.v[l][:, :, :64].cpu().numpy())
    for (lp, tp, up), (lv, tv, uv) in zip(out_p, out_v):
        assert_close(np64(lv), np64(lp), "f32", "logits, value-only vs plain")
        assert_close(np64(uv), np64(up), "f32", "u, value-only vs plain")
    # and the oracle, from its own commit
    rkv = dict(k=[np.zeros((2, 128, 64)) for _ in range(L)], v=[np.zeros((2, 128, 64)) for _ in range(L)], kv_len=0)
    kn, vn = O.commit_canvas(mcfg, wn, rkv, prompt.numpy(), "f32")
    for l in range(L):
        rkv["k"][l][:, :64], rkv["v"][l][:, :64] = kn[l], vn[l]
    rkv["kv_len"] = 64
    s = synth.sampler_cfg(V, t_max=45.0, t_min=12.0, n_steps=4, step=0)
    ref = O.canvas_step(mcfg, wn, rkv, dict(tokens=O.canvas_noise(C, V, 1, 0), u=None), s, "f32")
    assert_close(np64(out_v[0][0]), ref["logits"], "f32", "value-only step 0 vs oracle")
