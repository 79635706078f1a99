"""The benchmarked bf16 stack against the oracle, at the benchmark's width.

Every dimension is the benchmark's (hidden 2816; sliding layers 16/8 heads of
256 with window 1024; global layers 16/2 heads of 512 sharing W_k = W_v with
rotary factor 0.25; 128 experts top-8 + a shared expert, SwiGLU 704; tied
vocabulary 262,144; self-conditioning MLP 704), so every kernel runs in the
configuration the benchmark times: the wide split-K projections, the fused
O-proj partials + residual + pre-MoE norm pass, the fused MoE combine x layer
scalar + next pre-norm pass, the wide-tile expert products and the
vocabulary-wide head / sampler / P.E.  Only the depth is cut (6 layers, the
last one global; DG_STACK_LAYERS / DG_STACK_PROMPT select 30 and 4096, the
full configuration, as an opt-in run) so the float64 oracle finishes in about
a minute.  Layer scalars are drawn from U[0.8, 1.2] and the route scale is
1.3, so a device path that dropped s_l or scaled only the MoE output fails
(aitrends glossary "Layer Scalar", "MoE").

Sequence (aitrends attention paragraph: encode as a causal prefill, decode
over [committed | canvas]; velog Self-conditioning):
  commit a 1280-token prompt (the 1024-row window masks in both modes),
  step 0 at temperature 1 (every position commits its argmax),
  step 1 with self-conditioning at temperature 100 (near the transition: part
  of the canvas commits, the rest is re-noised; a spread-out P through P.E),
  commit the canvas (appends rows [1280, 1536)).
Each side continues from its own cache and self-conditioning vector; the
canvas tokens of step 1 are the oracle's (the device's equal them wherever
the oracle's argmax is clear of the logit band).

Conditioning.  Two things make a composed bf16 stack differ from a float64
one beyond rounding, and both are properties of the problem, not of the
device (the oracle against itself with 1-ulp input noise shows the same):
  - attention sharpness: scale-1 scores d_h * g_q * g_k * cos(theta) with the
    benchmark's gains g ~ U[0.5, 1.5] spread over about 16 nats, so a 1-ulp
    change of q or k moves competing softmax weights by tens of percent and
    the difference grows layer by layer (0.6% -> 22% in four layers).  The
    gains here are U[0.2, 0.3] (scores of about 1 nat), where it stays near
    1%.  Kernel cost does not depend on the gains.
  - routing: top-8 of 128 is a discrete decision; after one layer 28% of the
    attention outputs differ from the oracle's by one bf16 ulp, which moves
    router logits by up to 0.03, and about 1.3% of tokens per layer have an
    8th/9th gap below that and take another expert.
test_stack_injected_routing feeds both sides the same router logits (the
"same logits" contract) and holds every stage to the bar;
test_stack_computed_routing runs the router product on each side and bounds
the share of positions that left the bar.
"""
import math
import os
import time

import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from oracle import dg_oracle as O
from tests.helpers import TOL, assert_close, check_sampler_outputs, np64

pytestmark = pytest.mark.gpu

N_LAYERS = int(os.environ.get("DG_STACK_LAYERS", "6"))
# constant QK-norm gains: with the benchmark's U[0.5, 1.5] the attention
# scores have a spread of about 16 nats and the random-init stack is chaotic
# (the oracle against itself, with 1-ulp input noise, drifts 0.6% -> 22% in
# four layers); at U[0.2, 0.3] the same noise stays near 1% at every layer
GAMMA = (0.2, 0.3)
PROMPT = int(os.environ.get("DG_STACK_PROMPT", "1280"))
C = 256
# temperature of the second step: the self-logit of this random-init model is
# about 2800 against a spread of about 53; at t = 100 the entropies span about
# 2 to 9 nats around tau = 6.24, so part of the canvas commits and the rest is
# re-noised (t = 80: every position commits, t = 120: none)
T1 = 100.0


def say(*a):
    print(*a, flush=True)


class HostLayers:
    """Per-layer weights kept on the host in bf16; each access hands the
    oracle float32 arrays (bf16 values widen exactly), one layer at a time."""

    def __init__(self, layers):
        self.layers = layers

    def __len__(self):
        return len(self.layers)

    def __getitem__(self, l):
        say(f"[stack]   oracle reads layer {l}")   # a progress line per layer of the float64 oracle
        return {k: (v.float().numpy() if isinstance(v, torch.Tensor) else v) for k, v in self.layers[l].items()}


@pytest.fixture(scope="module")
def stack(gpu_lib):
    mcfg = synth.full_model_cfg()
    mcfg["n_layers"] = N_LAYERS
    mcfg["moe"]["route_scale"] = 1.3
    t0 = time.time()
    w = synth.model_weights(mcfg, seed=1, device="cuda", gamma_range=GAMMA)
    g = synth.generator(77)
    w["layer_scalar"] = [float(v) for v in (torch.rand(N_LAYERS, generator=g) * 0.4 + 0.8)]
    torch.cuda.synchronize()
    host = dict(embed=w["embed"].float().cpu().numpy(), w_final_norm=np64(w["w_final_norm"]),
                sc={k: np64(v) for k, v in w["sc"].items()},
                attn=HostLayers([{k: (v.cpu() if v is not None else None) for k, v in a.items()}
                                 for a in w["attn"]]),
                moe=HostLayers([{k: (v.cpu() if v is not None else None) for k, v in m.items()}
                                for m in w["moe"]]),
                layer_scalar=list(w["layer_scalar"]))
    model = B.Model(mcfg, w)
    say(f"[stack] {N_LAYERS} layers at full width, weights on device and host in {time.time() - t0:.1f}s; "
        f"layer scalars {np.round(w['layer_scalar'], 3).tolist()}")
    return mcfg, model, host


def oracle_kv(mcfg, cap):
    ks, vs = [], []
    for l in range(mcfg["n_layers"]):
        c = mcfg["global"] if O.layer_type(l, mcfg["global_every"]) else mcfg["sliding"]
        ks.append(np.zeros((c["n_kv_heads"], cap, c["head_dim"])))
        vs.append(np.zeros((c["n_kv_heads"], cap, c["head_dim"])))
    return dict(k=ks, v=vs, kv_len=0)


def token_errors(got, ref):
    """Per token: max |got - ref| over heads and dims / max |ref| of the tensor."""
    return np.abs(got - ref).max(axis=(0, 2)) / np.abs(ref).max()


def compare_appended(mcfg, kv, kn, vn, r0, r1, what, strict=True):
    """Every layer's appended K/V rows against the oracle's.  Returns, per
    layer, the fraction of tokens within the bar and the largest error."""
    out = []
    for l in range(mcfg["n_layers"]):
        gk, gv = np64(kv.k[l][:, r0:r1]), np64(kv.v[l].transpose(1, 2)[:, r0:r1])
        if strict:
            assert_close(gk, kn[l], "bf16", f"{what} k[{l}]")
            assert_close(gv, vn[l], "bf16", f"{what} v[{l}]")
        e = np.maximum(token_errors(gk, kn[l]), token_errors(gv, vn[l]))
        out.append((round(float((e <= TOL["bf16"]).mean()), 4), round(float(e.max()), 4)))
    say(f"[stack] {what} K/V per layer (fraction of tokens within the bar, max error): {out}")
    return out


def check_step(canvas, ref, s, V, what, strict=True):
    lg = canvas.logits.cpu().numpy()
    den = np.abs(ref["logits"]).max()
    row_err = np.abs(lg - ref["logits"]).max(axis=1) / den
    u_den = np.abs(ref["u_next"]).max()
    u_row = np.abs(np64(canvas.u) - ref["u_next"]).max(axis=1) / u_den
    H = canvas.entropy.cpu().numpy()
    t = ref["temperature"]
    stats = dict(rows_within=round(float((row_err <= TOL["bf16"]).mean()), 4),
                 logits_err=round(float(row_err.max()), 4), u_rows_within=round(float((u_row <= TOL["bf16"]).mean()), 4),
                 u_err=round(float(u_row.max()), 4))
    say(f"[stack] {what} (t={t}): {stats}")
    if not strict:
        return stats
    assert_close(lg, ref["logits"], "bf16", f"{what} logits")
    dl = float(np.max(np.abs(lg - ref["logits"])))
    # the entropy inherits the logits' error: the bf16 bar on its scale [0, ln V]
    dh = float(np.max(np.abs(H - ref["entropy"])))
    assert dh <= TOL["bf16"] * math.log(V), f"{what} entropy"
    noise = O.renoise_tokens(C, V, s["seed"], s["step"], s["canvas_idx"])
    tok = canvas.tokens.cpu().numpy()
    com = canvas.commit.cpu().numpy()
    n_band = check_sampler_outputs(tok, com, ref, ref["logits"], noise, s["tau"], band_logit=2 * dl,
                                   band_h=2 * dh + 1e-6)
    nre = int(canvas.n_renoised.item())
    assert nre == int((com == 0).sum())
    if n_band == 0:
        assert nre == ref["n_renoised"]
    assert int(canvas.n_nonfinite.item()) == 0
    assert_close(np64(canvas.u), ref["u_next"], "bf16", f"{what} u")
    say(f"[stack] {what}: n_renoised {nre}, positions decided inside a band {n_band}")
    return stats


def router_inputs(mcfg, n, seed):
    """Per-layer injected router logits N(0, 1) [n, n_experts] (the last
    layer's too: a step routes every layer)."""
    g = synth.generator(seed)
    return [synth.router_logits(n, mcfg["moe"]["n_experts"], g) for _ in range(mcfg["n_layers"])]


def inject(model, host, logits):
    model.set_router_logits(None if logits is None else [t.cuda() for t in logits])
    host["router_logits"] = None if logits is None else [t.double().numpy() for t in logits]


def run_sequence(stack, injected):
    """Commit the prompt, two steps, commit the canvas; compare each stage.
    injected: identical router logits on both sides (strict), else the
    router product on each side (the benchmark's path)."""
    mcfg, model, host = stack
    V = mcfg["vocab"]
    cap = PROMPT + 2 * C
    kv = B.KV(mcfg, cap)
    prompt = synth.tokens(PROMPT, V, synth.generator(2))
    t0 = time.time()
    inject(model, host, router_inputs(mcfg, PROMPT, 500) if injected else None)
    B.dg_commit_canvas(model, kv, prompt.cuda())
    torch.cuda.synchronize()
    assert kv.kv_len == PROMPT
    rkv = oracle_kv(mcfg, cap)
    kn, vn = O.commit_canvas(mcfg, host, rkv, prompt.numpy(), "bf16")
    stats = dict(prompt=compare_appended(mcfg, kv, kn, vn, 0, PROMPT, "prompt", strict=injected))
    for l in range(mcfg["n_layers"]):
        rkv["k"][l][:, :PROMPT], rkv["v"][l][:, :PROMPT] = kn[l], vn[l]
    rkv["kv_len"] = PROMPT
    say(f"[stack] prompt K/V of {mcfg['n_layers']} layers compared ({time.time() - t0:.0f}s)")

    canvas = B.Canvas(C, mcfg["hidden"], "bf16", keep_logits_vocab=V)
    canvas.tokens.copy_(B.dg_canvas_noise(C, V, 1, 0))
    tokens = O.canvas_noise(C, V, 1, 0)
    np.testing.assert_array_equal(canvas.tokens.cpu().numpy(), tokens)
    u = None
    for step in range(2):
        s = synth.sampler_cfg(V, t_max=1.0, t_min=T1, n_steps=2, step=step)
        inject(model, host, router_inputs(mcfg, C, 600 + step) if injected else None)
        B.dg_canvas_step(model, kv, canvas, s)
        torch.cuda.synchronize()
        assert kv.kv_len == PROMPT            # decode leaves the cache length alone
        ref = O.canvas_step(mcfg, host, rkv, dict(tokens=tokens, u=u), s, "bf16")
        stats[f"step{step}"] = check_step(canvas, ref, s, V, f"step {step}", strict=injected)
        if step == 0:
            assert ref["commit"].all()        # peaked random-init logits: every position commits
        else:
            # near the commit / re-noise transition: the step decides both ways
            assert 0 < ref["n_renoised"] < C, ref["n_renoised"]
        tokens, u = ref["tokens"], ref["u_next"]
        canvas.tokens.copy_(torch.from_numpy(tokens.astype(np.int32)))
    say(f"[stack] two steps compared ({time.time() - t0:.0f}s)")

    inject(model, host, router_inputs(mcfg, C, 700) if injected else None)
    B.dg_commit_canvas(model, kv, canvas.tokens)
    torch.cuda.synchronize()
    assert kv.kv_len == PROMPT + C
    kn, vn = O.commit_canvas(mcfg, host, rkv, tokens, "bf16")
    stats["canvas_commit"] = compare_appended(mcfg, kv, kn, vn, PROMPT, PROMPT + C, "canvas commit", strict=injected)
    say(f"[stack] canvas commit K/V compared ({time.time() - t0:.0f}s)")
    inject(model, host, None)
    return stats


def test_stack_injected_routing(stack):
    """Strict: with the same router logits on both sides, every stage of the
    stack (all fused kernels included) is within the bf16 bar."""
    run_sequence(stack, injected=True)


def test_stack_computed_routing(stack):
    """The benchmark's path, router product included, reported against the
    oracle.  Routing is a discrete decision downstream of bf16 rounding, so
    a token whose 8th/9th router logits are nearly tied may take another
    expert on each side and then differ by a few percent."""
    stats = run_sequence(stack, injected=False)
    say(f"[stack] computed routing: {stats}")
    # measured: at least 83% of prompt tokens per layer and 99.6% of canvas
    # rows stay within the bar; the first layer's K/V has no routing upstream
    for name in ("prompt", "canvas_commit"):
        assert stats[name][0][0] == 1.0
        assert min(f for f, _ in stats[name]) >= 0.75, (name, stats[name])
    for name in ("step0", "step1"):
        assert stats[name]["rows_within"] >= 0.9 and stats[name]["u_rows_within"] >= 0.9, (name, stats[name])


def test_stack_step_runs_twice_bit_identical(stack):
    """Race detector: the same step from the same state gives the same bits
    (no float atomics, no order that depends on scheduling)."""
    mcfg, model, _ = stack
    V = mcfg["vocab"]
    kv = B.KV(mcfg, 1024 + C)
    B.dg_commit_canvas(model, kv, synth.tokens(1024, V, synth.generator(3)).cuda())
    outs = []
    for _ in range(2):
        canvas = B.Canvas(C, mcfg["hidden"], "bf16", keep_logits_vocab=V)
        canvas.tokens.copy_(B.dg_canvas_noise(C, V, 1, 5))
        s = synth.sampler_cfg(V, t_max=30.0, t_min=30.0)
        B.dg_canvas_step(model, kv, canvas, s)
        B.dg_canvas_step(model, kv, canvas, dict(s, step=1))   # with self-conditioning
        torch.cuda.synchronize()
        outs.append((canvas.logits.cpu(), canvas.u.cpu(), canvas.tokens.cpu(), canvas.entropy.cpu(),
                     kv.k[0][:, 1024:].cpu(), kv.v[N_LAYERS - 1][:, :, 1024:].cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    assert outs[0][0].abs().max() > 0
