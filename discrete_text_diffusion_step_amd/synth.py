"""Seeded synthetic inputs for the canvas denoising step.

This module only draws random tensors and builds configuration records; it
holds none of the method's arithmetic.  Both the HIP path and the CPU oracle
consume what it produces: the tests hand the same tensors to each side.

Shapes and distributions follow the DiffusionGemma-26B-A4B description
(thakicloud "DiffusionGemma 26B-A4B" post, Architecture: 30 layers, 128
experts with 8 active + 1 shared, vocabulary 262,144, window 1,024, canvas
256) with random initialisation: weights N(0, 0.02), embeddings N(0, 1),
constant QK-norm vectors with gamma ~ U[0.5, 1.5] (aitrends.kr notebook
summary, glossary "Scalar QK Norm"), pre-norm weights U[0.5, 1.5].
Pages give no weights, so every tensor here is a stand-in of the right shape.
"""
import math

import torch

# ----------------------------------------------------------------------------
# configuration records (plain dicts; the binding turns them into C structs)
# ----------------------------------------------------------------------------


def attn_cfg(hidden, n_q_heads, n_kv_heads, head_dim, layer_type, window=1024,
             rope_base=10000.0, rotary_factor=1.0, rms_eps=1e-6, dtype="bf16"):
    glob = layer_type == 1
    return dict(hidden=hidden, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                head_dim=head_dim, layer_type=layer_type, window=window,
                shared_kv=1 if glob else 0, v_unit_rms=1 if glob else 0,
                rope_base=rope_base, rotary_factor=rotary_factor if glob else 1.0,
                rms_eps=rms_eps, dtype=dtype)


def moe_cfg(hidden, n_experts, top_k, ffn, shared_ffn, route_scale=1.0,
            rms_eps=1e-6, layer_scalar=1.0, dtype="bf16"):
    return dict(hidden=hidden, n_experts=n_experts, top_k=top_k, ffn=ffn,
                shared_ffn=shared_ffn, route_scale=route_scale, rms_eps=rms_eps,
                layer_scalar=layer_scalar, dtype=dtype)


def model_cfg(sliding, glob, moe, n_layers, global_every, vocab, sc_ffn, rms_eps=1e-6,
              dtype="bf16"):
    return dict(sliding=sliding, **{"global": glob}, moe=moe, n_layers=n_layers,
                global_every=global_every, vocab=vocab, sc_ffn=sc_ffn,
                hidden=sliding["hidden"], rms_eps=rms_eps, dtype=dtype)


def sampler_cfg(vocab, tau=None, t_max=1.0, t_min=1.0, n_steps=48, step=0,
                canvas_idx=0, seed=1, final_step=False):
    if tau is None:
        tau = 0.5 * math.log(vocab)   # half the uniform entropy, in nats
    return dict(vocab=vocab, tau=tau, t_max=t_max, t_min=t_min, n_steps=n_steps,
                step=step, canvas_idx=canvas_idx, seed=seed, final_step=final_step)


# The five workloads.  TINY: one decoder layer + sampler in fp32.  SLIDING /
# GLOBAL: one attention layer each at canvas shape.  MOE_HEAD: MoE block,
# tied head and sampler.  FULL: the 30-layer stack.
TINY = dict(hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, window=32,
            n_experts=8, top_k=2, ffn=128, shared_ffn=128, vocab=4096,
            prefix=64, canvas=32, sc_ffn=128)
SLIDING = dict(hidden=2816, n_q_heads=16, n_kv_heads=8, head_dim=256, window=1024,
               rope_base=10000.0, cache=2048, canvas=256)
GLOBAL = dict(hidden=2816, n_q_heads=16, n_kv_heads=2, head_dim=512,
              rope_base=1e6, rotary_factor=0.25, cache=32768, canvas=256)
MOE_HEAD = dict(hidden=2816, n_experts=128, top_k=8, ffn=704, shared_ffn=704,
                vocab=262144, canvas=256)
FULL = dict(n_layers=30, global_every=6, prompt=4096, n_canvases=8, n_steps=48,
            canvas=256, sc_ffn=704)


def tiny_attn_cfg(layer_type, dtype="f32"):
    t = TINY
    return attn_cfg(t["hidden"], t["n_q_heads"], t["n_kv_heads"], t["head_dim"],
                    layer_type, window=t["window"],
                    rope_base=10000.0 if layer_type == 0 else 1e6,
                    rotary_factor=0.25, dtype=dtype)


def tiny_moe_cfg(dtype="f32"):
    t = TINY
    return moe_cfg(t["hidden"], t["n_experts"], t["top_k"], t["ffn"], t["shared_ffn"],
                   dtype=dtype)


def tiny_model_cfg(n_layers=2, global_every=2, dtype="f32"):
    """Tiny stack: layer l is global iff l % global_every == global_every - 1."""
    t = TINY
    return model_cfg(tiny_attn_cfg(0, dtype), tiny_attn_cfg(1, dtype), tiny_moe_cfg(dtype),
                     n_layers, global_every, t["vocab"], t["sc_ffn"], dtype=dtype)


def sliding_cfg():
    s = SLIDING
    return attn_cfg(s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], 0,
                    window=s["window"], rope_base=s["rope_base"])


def global_cfg():
    g = GLOBAL
    return attn_cfg(g["hidden"], g["n_q_heads"], g["n_kv_heads"], g["head_dim"], 1,
                    rope_base=g["rope_base"], rotary_factor=g["rotary_factor"])


def full_model_cfg():
    m = MOE_HEAD
    return model_cfg(sliding_cfg(), global_cfg(),
                     moe_cfg(m["hidden"], m["n_experts"], m["top_k"], m["ffn"], m["shared_ffn"]),
                     FULL["n_layers"], FULL["global_every"], m["vocab"], FULL["sc_ffn"])


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name):
    return _TORCH_DTYPE[name]


def _normal(gen, shape, std, dtype, device):
    t = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(_TORCH_DTYPE[dtype])


def _uniform(gen, shape, lo, hi, dtype, device):
    t = torch.rand(*shape, generator=gen, device=device, dtype=torch.float32)
    return (t * (hi - lo) + lo).to(_TORCH_DTYPE[dtype])


def generator(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def attn_weights(cfg, gen, std=0.02, device="cpu", gamma=None):
    """One attention layer: pre-norm vector, projections, constant QK-norm vectors."""
    D, Hq, Hkv, dh = cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    dt = cfg["dtype"]
    w = dict(
        w_in_norm=_uniform(gen, (D,), 0.5, 1.5, dt, device),
        w_q=_normal(gen, (Hq * dh, D), std, dt, device),
        w_k=_normal(gen, (Hkv * dh, D), std, dt, device),
        w_v=None if cfg["shared_kv"] else _normal(gen, (Hkv * dh, D), std, dt, device),
        w_o=_normal(gen, (D, Hq * dh), std, dt, device),
    )
    if gamma is None:
        gq = float(_uniform(gen, (1,), 0.5, 1.5, "f32", "cpu" if device == "cpu" else device).item())
        gk = float(_uniform(gen, (1,), 0.5, 1.5, "f32", "cpu" if device == "cpu" else device).item())
    else:
        gq, gk = gamma
    w["q_norm"] = torch.full((dh,), gq, dtype=_TORCH_DTYPE[dt], device=device)
    w["k_norm"] = torch.full((dh,), gk, dtype=_TORCH_DTYPE[dt], device=device)
    return w


def moe_weights(cfg, gen, std=0.02, device="cpu", with_router=True):
    D, E, F, Fs = cfg["hidden"], cfg["n_experts"], cfg["ffn"], cfg["shared_ffn"]
    dt = cfg["dtype"]
    return dict(
        w_in_norm=_uniform(gen, (D,), 0.5, 1.5, dt, device),
        w_router=_normal(gen, (E, D), std, dt, device) if with_router else None,
        w_gate=_normal(gen, (E, F, D), std, dt, device),
        w_up=_normal(gen, (E, F, D), std, dt, device),
        w_down=_normal(gen, (E, D, F), std, dt, device),
        ws_gate=_normal(gen, (Fs, D), std, dt, device),
        ws_up=_normal(gen, (Fs, D), std, dt, device),
        ws_down=_normal(gen, (D, Fs), std, dt, device),
    )


def embed_table(vocab, hidden, gen, dtype, device="cpu"):
    return _normal(gen, (vocab, hidden), 1.0, dtype, device)


def selfcond_weights(hidden, sc_ffn, gen, dtype, std=0.02, device="cpu"):
    return dict(sc_gate=_normal(gen, (sc_ffn, hidden), std, dtype, device),
                sc_up=_normal(gen, (sc_ffn, hidden), std, dtype, device),
                sc_down=_normal(gen, (hidden, sc_ffn), std, dtype, device))


def hidden_states(n, hidden, gen, dtype, device="cpu"):
    return _normal(gen, (n, hidden), 1.0, dtype, device)


def kv_cache_random(n_kv_heads, capacity, head_dim, gen, dtype, device="cpu"):
    """Committed K/V rows drawn N(0, 1) (the single-layer workloads)."""
    k = _normal(gen, (n_kv_heads, capacity, head_dim), 1.0, dtype, device)
    v = _normal(gen, (n_kv_heads, capacity, head_dim), 1.0, dtype, device)
    return k, v


def tokens(n, vocab, gen, device="cpu"):
    return torch.randint(0, vocab, (n,), generator=gen, device=device, dtype=torch.int32)


def router_logits(n, n_experts, gen, device="cpu"):
    return torch.randn(n, n_experts, generator=gen, device=device, dtype=torch.float32)


def sampler_logits(n, vocab, gen, s_max=7.0, n_flat=4, n_peaked=4, device="cpu"):
    """Logits with controlled sharpness: row j is s_j * z_j, z ~ N(0,1),
    s_j ~ U[0, s_max] (so the entropy spans the commit threshold), plus
    n_flat all-equal rows and n_peaked rows with one dominant entry."""
    z = torch.randn(n, vocab, generator=gen, device=device, dtype=torch.float32)
    s = torch.rand(n, 1, generator=gen, device=device, dtype=torch.float32) * s_max
    out = z * s
    for j in range(min(n_flat, n)):
        out[j] = 0.25
    for j in range(n_flat, min(n_flat + n_peaked, n)):
        hot = int(torch.randint(0, vocab, (1,), generator=gen, device=device).item())
        out[j] = z[j] * 0.1
        out[j, hot] = 60.0
    return out


def model_weights(mcfg, seed, device="cpu", std=0.02, layer_seed_base=1000, gamma_range=None):
    """Weights for a whole stack; layer l draws from seed layer_seed_base + l.
    gamma_range=(lo, hi): the constant QK-norm gains of layer l are drawn
    from U[lo, hi] (seed 2000 + l) instead of U[0.5, 1.5]."""
    dt = mcfg["dtype"]
    D, V = mcfg["hidden"], mcfg["vocab"]
    g = generator(seed, device)
    w = dict(embed=embed_table(V, D, g, dt, device),
             w_final_norm=_uniform(g, (D,), 0.5, 1.5, dt, device))
    w["sc"] = selfcond_weights(D, mcfg["sc_ffn"], g, dt, std, device) if mcfg["sc_ffn"] else None
    w["attn"], w["moe"], w["layer_scalar"] = [], [], []
    for l in range(mcfg["n_layers"]):
        gl = generator(layer_seed_base + l, device)
        glob = (l % mcfg["global_every"]) == mcfg["global_every"] - 1
        acfg = mcfg["global"] if glob else mcfg["sliding"]
        gamma = None
        if gamma_range is not None:
            gg = generator(2000 + l)
            gamma = tuple(float(v) for v in torch.rand(2, generator=gg) * (gamma_range[1] - gamma_range[0])
                          + gamma_range[0])
        w["attn"].append(attn_weights(acfg, gl, std, device, gamma=gamma))
        w["moe"].append(moe_weights(mcfg["moe"], gl, std, device))
        w["layer_scalar"].append(1.0)
    return w
