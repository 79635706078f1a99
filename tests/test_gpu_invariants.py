"""Black-box invariants of the device path that hold at any size.

- Attention rows are convex combinations of the visible values ([AIT]
  attention paragraph: softmax over the visible keys): with every value
  equal to 1, the attention output is 1 whatever the scores.
- Failure detection: logits rows holding NaN or +-inf are counted
  (n_nonfinite), re-noised, and never propose an out-of-range token.
"""
import math

import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from oracle import dg_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("layer_type,P", [(0, 2048), (1, 4096)])
def test_values_all_one_give_attention_output_one(layer_type, P):
    """Canvas shape (256 queries).  With eps = 0, x = 1 and a unit pre-norm
    weight, h = 1 exactly; one weight of 1 per value row makes every canvas
    value 1 (global layers: the shared raw key is 1, whose unit-RMS value is
    1), and the committed values are 1.  W_o is the identity on the first
    hidden columns, so x_out = 1 + o there: 2 up to the rounding of the
    probabilities."""
    cfg = dict(synth.sliding_cfg() if layer_type == 0 else synth.global_cfg(), rms_eps=0.0)
    D, Hq, Hkv, dh = cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    g = synth.generator(91 + layer_type)
    w = synth.attn_weights(cfg, g)
    w["w_in_norm"] = torch.ones(D, dtype=torch.bfloat16)
    wv = torch.zeros(Hkv * dh, D, dtype=torch.bfloat16)
    wv[:, 0] = 1.0
    if cfg["shared_kv"]:
        w["w_k"] = wv
    else:
        w["w_v"] = wv
    wo = torch.zeros(D, Hq * dh, dtype=torch.bfloat16)
    wo[torch.arange(D), torch.arange(D)] = 1.0
    w["w_o"] = wo
    cap = P + 256
    ck, _ = synth.kv_cache_random(Hkv, cap, dh, g, "bf16")
    vt = torch.ones(Hkv, dh, cap, dtype=torch.bfloat16)
    x = torch.ones(256, D, dtype=torch.bfloat16).cuda()
    B.dg_attn_layer(cfg, {k: (v.cuda() if v is not None else None) for k, v in w.items()}, ck.cuda(), vt.cuda(),
                    P, x, 0)
    torch.cuda.synchronize()
    out = x.float().cpu().numpy()
    # one bf16 ulp at 2 is 2^-6
    assert np.max(np.abs(out - 2.0)) <= 2.0 ** -6, np.max(np.abs(out - 2.0))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sampler_nonfinite_rows(dtype):
    V, n = 262144, 40
    g = synth.generator(93)
    lg = synth.sampler_logits(n, V, g)
    lg[5, 1000] = float("nan")          # one NaN: the argmax skips it
    lg[6] = float("nan")                # no number at all: token 0
    lg[7, 7] = float("inf")
    lg[8, 3] = float("-inf")
    if dtype == "bf16":
        lg = lg.to(torch.bfloat16)
    for final in (False, True):
        s = synth.sampler_cfg(V, step=2, canvas_idx=1, final_step=final)
        out = B.dg_sample_renoise(s, lg.cuda())
        torch.cuda.synchronize()
        with np.errstate(invalid="ignore", over="ignore"):
            ref = O.sample_renoise(lg.double().numpy(), s)
        assert int(out["n_nonfinite"].item()) == ref["n_nonfinite"] == 4
        tok = out["tokens"].cpu().numpy()
        assert (tok >= 0).all() and (tok < V).all()
        bad = np.array([5, 6, 7, 8])
        np.testing.assert_array_equal(tok[bad], ref["tokens"][bad])
        np.testing.assert_array_equal(out["commit"].cpu().numpy()[bad].astype(bool), ref["commit"][bad])
        assert np.isnan(out["entropy"].cpu().numpy()[bad]).all()
        # rows without a non-finite value are unaffected
        ok = np.setdiff1d(np.arange(n), bad)
        clear = np.abs(ref["entropy"][ok] - s["tau"]) > 1e-3
        np.testing.assert_array_equal(tok[ok][clear], ref["tokens"][ok][clear])
        H = out["entropy"].cpu().numpy()[ok]
        assert np.max(np.abs(H - ref["entropy"][ok])) < 1e-4 * math.log(V)
