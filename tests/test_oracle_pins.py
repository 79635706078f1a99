"""Pins for the CPU oracle: checks against facts the pages and mathematics fix.

None of these re-types an oracle formula; each compares the oracle with a
closed form, an invariant, a textbook/library routine or a published vector
so that a plausible slip (dropped term, wrong sign or index, transposed
operand, wrong scale) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from discrete_text_diffusion_step_amd import synth
from oracle import dg_oracle as O
from oracle.philox import philox4x32_10, uniform_token

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def np64(t):
    return t.detach().to(torch.float64).cpu().numpy() if t is not None else None


def npw(d):
    return {k: (np64(v) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


# ----------------------------------------------------------------------------
# Philox and the uniform re-noise token
# ----------------------------------------------------------------------------


def test_philox_known_answer_vectors():
    rows = []
    with open(os.path.join(GOLDEN, "philox_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v = [int(x, 16) for x in line.split()]
            rows.append(v)
    assert len(rows) == 3
    for v in rows:
        out = philox4x32_10(v[0:4], v[4:6])
        assert [int(x) for x in out] == v[6:10]


def test_uniform_token_is_uniform_chi2():
    n, V = 1_000_000, 256
    ctr = np.zeros((n, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n) % 4096
    ctr[:, 1] = np.arange(n) // 4096
    x = philox4x32_10(ctr, [1, 0])
    tok = uniform_token(x[:, 0], V)
    assert tok.min() >= 0 and tok.max() < V
    counts = np.bincount(tok, minlength=V)
    chi2, p = scipy.stats.chisquare(counts)
    assert p > 1e-4, (chi2, p)


def test_uniform_token_power_of_two_is_top_bits():
    # for V = 2**18 the map floor(x * V / 2**32) keeps the top 18 bits
    x = np.array([0, 1, 0x3FFF, 0x4000, 0xFFFFFFFF, 0x80000000], dtype=np.uint64)
    assert list(uniform_token(x, 1 << 18)) == [0, 0, 0, 1, (1 << 18) - 1, 1 << 17]


def test_renoise_counters_distinct_per_position_step_canvas():
    a = O.renoise_tokens(64, 1 << 18, 1, 0, 0)
    b = O.renoise_tokens(64, 1 << 18, 1, 1, 0)
    c = O.renoise_tokens(64, 1 << 18, 1, 0, 1)
    d = O.renoise_tokens(64, 1 << 18, 2, 0, 0)
    assert len(set(a.tolist())) > 60
    assert not np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------


def test_rms_constant_weight_gives_rms_gamma():
    rng = np.random.default_rng(0)
    x = rng.normal(size=(7, 96)) * rng.uniform(0.1, 10, size=(7, 1))
    g = 1.37
    y = O.rms(x, g, eps=0.0)
    rms_y = np.sqrt(np.mean(y * y, axis=-1))
    np.testing.assert_allclose(rms_y, g, rtol=1e-13)
    # direction preserved
    cos = np.sum(x * y, -1) / np.linalg.norm(x, axis=-1) / np.linalg.norm(y, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-13)
    # eps on the L2 norm: rms(y) = g * ||x|| / (||x|| + eps)
    eps = 0.5
    y = O.rms(x, g, eps=eps)
    nx = np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), g * nx / (nx + eps), rtol=1e-13)
    # zero row stays zero
    assert np.all(O.rms(np.zeros((1, 8)), 1.0, 1e-6) == 0)
    # per-element weight multiplies elementwise
    w = rng.uniform(0.5, 1.5, size=96)
    np.testing.assert_allclose(O.rms(x, w, 0.0), O.rms(x, 1.0, 0.0) * w, rtol=1e-14)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(size=5000) * 10 ** rng.uniform(-8, 8, size=5000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.005859375, 65504.0]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(x), ref)


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------


def test_rope_freqs_full_and_partial():
    f = O.rope_freqs(64, 10000.0)
    assert f[0] == 1.0
    np.testing.assert_allclose(f[1:] / f[:-1], 10000.0 ** (-2 / 64), rtol=1e-13)
    fp = O.rope_freqs(512, 1e6, 0.25)
    assert np.count_nonzero(fp) == 64          # first 25% of the 256 frequencies
    np.testing.assert_array_equal(fp[:64], O.rope_freqs(512, 1e6)[:64])


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(2)
    d = 64
    x = rng.normal(size=(10, d))
    pos = rng.integers(0, 40000, size=10)
    f = O.rope_freqs(d, 10000.0)
    y = O.rope(x, pos, f)
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, None] * f[None, :])
    np.testing.assert_allclose(y[:, : d // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, d // 2:], z.imag, atol=1e-12)


def test_rope_invariants():
    rng = np.random.default_rng(3)
    d = 128
    q = rng.normal(size=(6, d))
    k = rng.normal(size=(6, d))
    f = O.rope_freqs(d, 10000.0)
    pos = np.arange(6) * 17 + 5
    yq = O.rope(q, pos, f)
    # pair norms preserved
    h = d // 2
    np.testing.assert_allclose(yq[:, :h] ** 2 + yq[:, h:] ** 2, q[:, :h] ** 2 + q[:, h:] ** 2, rtol=1e-12)
    # position 0 is the identity
    np.testing.assert_array_equal(O.rope(q, np.zeros(6), f), q)
    # relative position: shifting both positions leaves the dot product unchanged
    for delta in (1, 1000, 33000):
        a = np.sum(O.rope(q, pos, f) * O.rope(k, pos + 3, f), -1)
        b = np.sum(O.rope(q, pos + delta, f) * O.rope(k, pos + 3 + delta, f), -1)
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


def test_partial_rope_leaves_zeroed_dims_bit_identical():
    rng = np.random.default_rng(4)
    d = 512
    x = rng.normal(size=(5, d))
    f = O.rope_freqs(d, 1e6, 0.25)
    y = O.rope(x, np.arange(32768, 32773), f)
    keep = 64
    np.testing.assert_array_equal(y[:, keep:d // 2], x[:, keep:d // 2])
    np.testing.assert_array_equal(y[:, d // 2 + keep:], x[:, d // 2 + keep:])
    assert not np.allclose(y[:, :keep], x[:, :keep])


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------


def tiny_layer(layer_type, seed=0, eps=None, dtype="f32"):
    cfg = synth.tiny_attn_cfg(layer_type, dtype)
    if eps is not None:
        cfg["rms_eps"] = eps
    g = synth.generator(seed)
    w = npw(synth.attn_weights(cfg, g))
    return cfg, w, g


def encode_prefix(cfg, w, g, P, dtype="f32"):
    """Fill a cache by encoding P random tokens' hidden states (oracle only)."""
    Hkv, dh = cfg["n_kv_heads"], cfg["head_dim"]
    xp = np64(synth.hidden_states(P, cfg["hidden"], g, dtype))
    ck = np.zeros((Hkv, P + 64, dh))
    cv = np.zeros((Hkv, P + 64, dh))
    _, k, v = O.attn_layer(cfg, w, ck, cv, 0, xp, 1, dtype)
    ck[:, :P] = k
    cv[:, :P] = v
    return ck, cv


@pytest.mark.parametrize("layer_type", [0, 1])
def test_scalar_qk_norm_fixes_logit_scale(layer_type):
    """[AIT] QK-norm paragraph: with constant q/k norm vectors the logit is
    d_h * gamma_q * gamma_k * cos(theta) (scale 1, no 1/sqrt(d_h))."""
    cfg, w, g = tiny_layer(layer_type, eps=0.0)
    ck, cv = encode_prefix(cfg, w, g, 64)
    x = np64(synth.hidden_states(32, cfg["hidden"], g, "f32"))
    _, _, _, ex = O.attn_layer(cfg, w, ck, cv, 64, x, 0, "f32", want_probs=True)
    q, K, s = ex["q"], ex["K"], ex["scores"]
    dh = cfg["head_dim"]
    gq, gk = w["q_norm"][0], w["k_norm"][0]
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), gq * math.sqrt(dh), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(K, axis=-1), gk * math.sqrt(dh), rtol=1e-12)
    n_rep = cfg["n_q_heads"] // cfg["n_kv_heads"]
    for hq in range(cfg["n_q_heads"]):
        kk = K[hq // n_rep]
        cos = (q[hq] / np.linalg.norm(q[hq], axis=-1, keepdims=True)) @ \
              (kk / np.linalg.norm(kk, axis=-1, keepdims=True)).T
        cols = ex["vis"].any(0)             # scores exist for keys some query can see
        np.testing.assert_allclose(s[hq][:, cols], (dh * gq * gk * cos)[:, cols], rtol=1e-10, atol=1e-10)


def test_attention_rows_sum_to_one_and_window_masks():
    cfg, w, g = tiny_layer(0)
    P, C, W = 64, 32, cfg["window"]
    ck, cv = encode_prefix(cfg, w, g, P)
    x = np64(synth.hidden_states(C, cfg["hidden"], g, "f32"))
    out, _, _, ex = O.attn_layer(cfg, w, ck, cv, P, x, 0, "f32", want_probs=True)
    a = ex["probs"]
    np.testing.assert_allclose(a.sum(-1), 1.0, rtol=1e-12)
    assert np.all(a[:, :, : P - W] == 0.0)           # committed rows out of the window
    assert np.all(a[:, :, P - W:] > 0.0)
    # NaN-poisoned out-of-window rows change nothing
    ck2, cv2 = ck.copy(), cv.copy()
    ck2[:, : P - W] = np.nan
    cv2[:, : P - W] = np.nan
    out2, _, _ = O.attn_layer(cfg, w, ck2, cv2, P, x, 0, "f32")
    np.testing.assert_array_equal(out, out2)


def test_global_layer_sees_whole_prefix():
    cfg, w, g = tiny_layer(1)
    ck, cv = encode_prefix(cfg, w, g, 64)
    x = np64(synth.hidden_states(32, cfg["hidden"], g, "f32"))
    _, _, _, ex = O.attn_layer(cfg, w, ck, cv, 64, x, 0, "f32", want_probs=True)
    assert np.all(ex["probs"] > 0.0)


def test_single_key_returns_its_value():
    for lt in (0, 1):
        cfg, w, g = tiny_layer(lt)
        x = np64(synth.hidden_states(1, cfg["hidden"], g, "f32"))
        Hkv, dh = cfg["n_kv_heads"], cfg["head_dim"]
        _, k, v, ex = O.attn_layer(cfg, w, np.zeros((Hkv, 1, dh)), np.zeros((Hkv, 1, dh)), 0, x, 0,
                                   "f32", want_probs=True)
        n_rep = cfg["n_q_heads"] // Hkv
        # output of head h equals the single value row of its kv head
        h = O.rms(x, w["w_in_norm"], cfg["rms_eps"])
        o_expected = np.concatenate([v[hq // n_rep, 0] for hq in range(cfg["n_q_heads"])])
        np.testing.assert_allclose(ex["probs"], 1.0)
        out_expected = x + o_expected[None, :] @ w["w_o"].T
        out, _, _ = O.attn_layer(cfg, w, np.zeros((Hkv, 1, dh)), np.zeros((Hkv, 1, dh)), 0, x, 0, "f32")
        np.testing.assert_allclose(out, out_expected, rtol=1e-12, atol=1e-12)
        del h


@pytest.mark.parametrize("layer_type", [0, 1])
def test_incremental_encode_equals_one_shot(layer_type):
    """A KV cache is only consistent if encoding [A; B] at once equals encoding A
    then B against A's cache (pins the causal mask, window and positions)."""
    cfg, w, g = tiny_layer(layer_type)
    Hkv, dh = cfg["n_kv_heads"], cfg["head_dim"]
    xa = np64(synth.hidden_states(48, cfg["hidden"], g, "f32"))
    xb = np64(synth.hidden_states(40, cfg["hidden"], g, "f32"))
    z = np.zeros((Hkv, 128, dh))
    out_ab, k_ab, v_ab = O.attn_layer(cfg, w, z, z, 0, np.concatenate([xa, xb]), 1, "f32")
    out_a, k_a, v_a = O.attn_layer(cfg, w, z, z, 0, xa, 1, "f32")
    ck, cv = z.copy(), z.copy()
    ck[:, :48], cv[:, :48] = k_a, v_a
    out_b, k_b, v_b = O.attn_layer(cfg, w, ck, cv, 48, xb, 1, "f32")
    np.testing.assert_allclose(out_ab[48:], out_b, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(out_ab[:48], out_a, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(k_ab[:, 48:], k_b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(v_ab[:, 48:], v_b, rtol=1e-12, atol=1e-12)


def test_causal_encode_first_token_sees_only_itself():
    cfg, w, g = tiny_layer(0)
    x = np64(synth.hidden_states(40, cfg["hidden"], g, "f32"))
    z = np.zeros((cfg["n_kv_heads"], 64, cfg["head_dim"]))
    _, _, _, ex = O.attn_layer(cfg, w, z, z, 0, x, 1, "f32", want_probs=True)
    a = ex["probs"]
    W = cfg["window"]
    np.testing.assert_allclose(a[:, 0, 0], 1.0)
    for j in range(40):
        assert np.all(a[:, j, j + 1:] == 0)                 # no future keys
        assert np.all(a[:, j, : max(0, j - W + 1)] == 0)     # per-query window
        np.testing.assert_allclose(a[:, j].sum(-1), 1.0, rtol=1e-12)


def test_shared_kv_projection_global_layer():
    """[AIT] attention paragraph: W_v = W_k; only K gets gamma_k and RoPE, V is
    unit-RMS.  So k = gamma_k * v on every dim RoPE leaves alone."""
    cfg, w, g = tiny_layer(1)
    x = np64(synth.hidden_states(16, cfg["hidden"], g, "f32"))
    q, k, v = O.project_qkv(cfg, w, x, 100, "f32")
    dh = cfg["head_dim"]
    keep = int(0.25 * dh / 2)
    gk = w["k_norm"][0]
    np.testing.assert_allclose(k[..., keep:dh // 2], gk * v[..., keep:dh // 2], rtol=1e-12)
    np.testing.assert_allclose(k[..., dh // 2 + keep:], gk * v[..., dh // 2 + keep:], rtol=1e-12)
    np.testing.assert_allclose(np.sqrt(np.mean(v * v, -1)), 1.0, rtol=1e-6)
    # pre-RoPE: same vector up to gamma_k (rotation is a pair-norm-preserving map)
    h = dh // 2
    np.testing.assert_allclose(k[..., :h] ** 2 + k[..., h:] ** 2,
                               gk ** 2 * (v[..., :h] ** 2 + v[..., h:] ** 2), rtol=1e-10)


def _rms_by_hand(vec, w, eps):
    """w_t * x_t * sqrt(d) / (||x|| + eps) written as scalar loops."""
    d = len(vec)
    nrm = math.sqrt(sum(float(a) * float(a) for a in vec))
    return [float(w[t]) * float(vec[t]) * math.sqrt(d) / (nrm + eps) for t in range(d)]


@pytest.mark.parametrize("layer_type", [0, 1])
def test_head_major_split_by_hand(layer_type):
    """[AIT] projection code: the projection output is split 'l (n h) -> n l h',
    so head n owns columns [n*d_h, (n+1)*d_h), i.e. rows [n*d_h, (n+1)*d_h) of
    W_q (W_k for kv head g).  Each head is rebuilt here from those weight rows
    with the pre-norm, QK-norm and split-half rotation as scalar loops; a
    split taking columns n, n+H, n+2H, ... (the '(h n)' order) fails."""
    cfg, w, g = tiny_layer(layer_type)
    x = np64(synth.hidden_states(3, cfg["hidden"], g, "f32"))
    pos0 = 37
    q, k, v = O.project_qkv(cfg, w, x, pos0, "f32")
    dh, half, eps = cfg["head_dim"], cfg["head_dim"] // 2, cfg["rms_eps"]
    rf = cfg["rotary_factor"] if layer_type == 1 else 1.0
    n_keep = int(round(rf * half))

    def head(W, gamma, n, j):
        h = _rms_by_hand(x[j], w["w_in_norm"], eps)
        raw = [sum(h[d] * float(W[n * dh + t, d]) for d in range(len(h))) for t in range(dh)]
        nr = _rms_by_hand(raw, gamma, eps)
        out = list(nr)
        p = pos0 + j
        for t in range(half):
            f = cfg["rope_base"] ** (-2.0 * t / dh) if t < n_keep else 0.0
            c, s = math.cos(p * f), math.sin(p * f)
            out[t] = nr[t] * c - nr[t + half] * s
            out[t + half] = nr[t + half] * c + nr[t] * s
        return np.array(out), np.array(raw)

    for n, j in ((0, 0), (cfg["n_q_heads"] - 1, 2), (1, 1)):
        ref, _ = head(w["w_q"], w["q_norm"], n, j)
        np.testing.assert_allclose(q[n, j], ref, rtol=1e-10, atol=1e-12)
    for gi, j in ((0, 1), (cfg["n_kv_heads"] - 1, 2)):
        ref, raw = head(w["w_k"], w["k_norm"], gi, j)
        np.testing.assert_allclose(k[gi, j], ref, rtol=1e-10, atol=1e-12)
        if layer_type == 1:
            # shared projection: the value is the raw key of the same head at unit RMS
            np.testing.assert_allclose(v[gi, j], _rms_by_hand(raw, np.ones(dh), eps), rtol=1e-10,
                                       atol=1e-12)


def test_selfcond_adds_swiglu_of_u_by_hand():
    """[AIT] glossary "Self-conditioning"; [VLG] soft embedding: the expected
    embedding u passes through the small MLP and is ADDED to the token
    embedding (x_j = E[c_j] + MLP_sc(u_j), no sqrt(D) scale).  The MLP
    (bias-free SwiGLU) is evaluated here with scalar loops for u != 0, so
    'replace' instead of 'add', a dropped gate, or a swapped gate/up fails."""
    D, V, F = 12, 40, 5
    g = synth.generator(12)
    E = np64(synth.embed_table(V, D, g, "f32"))
    sc = {k: v * 10.0 for k, v in npw(synth.selfcond_weights(D, F, g, "f32")).items()}
    u = np64(synth.hidden_states(3, D, g, "f32"))
    tok = np.array([5, 39, 0])
    x = O.embed_selfcond(tok, E, u, sc, "f32")
    for j in range(3):
        a = []
        for f in range(F):
            zg = sum(float(sc["sc_gate"][f, d]) * float(u[j, d]) for d in range(D))
            zu = sum(float(sc["sc_up"][f, d]) * float(u[j, d]) for d in range(D))
            a.append(zg / (1.0 + math.exp(-zg)) * zu)
        for d in range(D):
            mlp = sum(float(sc["sc_down"][d, f]) * a[f] for f in range(F))
            assert abs(x[j, d] - (E[tok[j], d] + mlp)) <= 1e-12 * (1.0 + abs(E[tok[j], d]))
    # the MLP term is not negligible here: replacing instead of adding would fail
    assert np.max(np.abs(x - E[tok])) > 1e-2


def test_shared_kv_keys_are_rotated_scaled_values():
    """The identity behind a value-only cache in W_v = W_k layers ([AIT]
    attention paragraph: KV saving / reconstruction): the stored key equals
    the split-half rotation, at the key's own position, of gamma_k times the
    stored value, on every dim (float64, no rounding)."""
    cfg, w, g = tiny_layer(1)
    x = np64(synth.hidden_states(9, cfg["hidden"], g, "f32"))
    pos0 = 1234
    _, k, v = O.project_qkv(cfg, w, x, pos0, "f32")
    dh, half = cfg["head_dim"], cfg["head_dim"] // 2
    keep = int(round(cfg["rotary_factor"] * half))
    for j in range(9):
        p = pos0 + j
        for t in range(half):
            f = cfg["rope_base"] ** (-2.0 * t / dh) if t < keep else 0.0
            c, s_ = math.cos(p * f), math.sin(p * f)
            a = w["k_norm"][t] * v[:, j, t]
            b = w["k_norm"][t + half] * v[:, j, t + half]
            np.testing.assert_allclose(k[:, j, t], a * c - b * s_, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(k[:, j, t + half], b * c + a * s_, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------
# MoE
# ----------------------------------------------------------------------------


def tiny_moe(seed=0, **over):
    cfg = synth.tiny_moe_cfg("f32")
    cfg.update(over)
    g = synth.generator(seed)
    w = npw(synth.moe_weights(cfg, g))
    x = np64(synth.hidden_states(24, cfg["hidden"], g, "f32"))
    return cfg, w, x, g


def test_router_topk_matches_stable_argsort():
    rng = np.random.default_rng(5)
    r = rng.normal(size=(50, 16))
    r[3, 4] = r[3, 9] = r[3].max() + 1.0           # exact tie: lower id first
    idx, wts = O.router_topk(r, 4, route_scale=2.5)
    ref = np.argsort(-r, axis=1, kind="stable")[:, :4]
    np.testing.assert_array_equal(idx, ref)
    assert idx[3, 0] == 4 and idx[3, 1] == 9
    np.testing.assert_allclose(wts.sum(1), 2.5, rtol=1e-13)
    # weights are the softmax restricted to the chosen experts
    p = scipy.special.softmax(r, axis=1)
    sel = np.take_along_axis(p, idx, 1)
    np.testing.assert_allclose(wts, 2.5 * sel / sel.sum(1, keepdims=True), rtol=1e-12)


def test_moe_all_experts_reduces_to_dense_softmax_mixture():
    cfg, w, x, _ = tiny_moe(top_k=8)
    out, idx, wts, r = O.moe_block(cfg, w, x, "f32")
    h = O.rms(x, w["w_in_norm"], cfg["rms_eps"])
    p = scipy.special.softmax(h @ w["w_router"].T, axis=1)
    y = O.swiglu_ffn(h, w["ws_gate"], w["ws_up"], w["ws_down"], "f32")
    for e in range(8):
        y = y + p[:, e:e + 1] * O.swiglu_ffn(h, w["w_gate"][e], w["w_up"][e], w["w_down"][e], "f32")
    np.testing.assert_allclose(out, x + y, rtol=1e-11, atol=1e-11)


def test_moe_identical_experts_weights_sum_to_scale():
    cfg, w, x, _ = tiny_moe(route_scale=1.7)
    for name in ("w_gate", "w_up", "w_down"):
        w[name] = np.repeat(w[name][:1], cfg["n_experts"], axis=0)
    out, _, _, _ = O.moe_block(cfg, w, x, "f32")
    h = O.rms(x, w["w_in_norm"], cfg["rms_eps"])
    y = O.swiglu_ffn(h, w["ws_gate"], w["ws_up"], w["ws_down"], "f32") + \
        1.7 * O.swiglu_ffn(h, w["w_gate"][0], w["w_up"][0], w["w_down"][0], "f32")
    np.testing.assert_allclose(out, x + y, rtol=1e-11, atol=1e-11)


def test_route_scale_scales_only_the_routed_experts():
    # O11: the scale multiplies the renormalised top-k weights, never the
    # shared expert: the routed part of the update is linear in it
    cfg, w, x, _ = tiny_moe()
    h = O.rms(x, w["w_in_norm"], cfg["rms_eps"])
    shared = O.swiglu_ffn(h, w["ws_gate"], w["ws_up"], w["ws_down"], "f32")
    o1, i1, w1, _ = O.moe_block(dict(cfg, route_scale=1.0), w, x, "f32")
    o3, i3, w3, _ = O.moe_block(dict(cfg, route_scale=0.3), w, x, "f32")
    np.testing.assert_array_equal(i1, i3)
    np.testing.assert_allclose(w1.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(w3, 0.3 * w1, rtol=1e-14)
    np.testing.assert_allclose(o3 - x - shared, 0.3 * (o1 - x - shared), rtol=1e-10, atol=1e-12)


def test_swiglu_silu_closed_form():
    z = np.array([-3.0, -0.5, 0.0, 0.5, 3.0])
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-15)
    # a 1-wide expert: down * silu(gate*h) * (up*h)
    h = np.array([[2.0]])
    out = O.swiglu_ffn(h, np.array([[0.5]]), np.array([[3.0]]), np.array([[4.0]]), "f32")
    np.testing.assert_allclose(out, 4.0 * (1.0 * scipy.special.expit(1.0)) * 6.0, rtol=1e-15)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_moe_grouped_equals_per_token_loop(dtype):
    cfg, w, x, g = tiny_moe(seed=3)
    r = np64(synth.router_logits(24, cfg["n_experts"], g))
    a = O.moe_block(cfg, w, x, dtype, router_logits=r)
    b = O.moe_block_grouped(cfg, w, x, dtype, router_logits=r)
    np.testing.assert_array_equal(a[1], b[1])
    tol = 1e-12 if dtype == "f32" else 1e-2
    np.testing.assert_allclose(a[0], b[0], rtol=tol, atol=tol)


def test_layer_scalar_identity_and_linear():
    cfg, w, x, _ = tiny_moe()
    o1, _, _, _ = O.moe_block(dict(cfg, layer_scalar=1.0), w, x, "f32")
    o2, _, _, _ = O.moe_block(dict(cfg, layer_scalar=2.0), w, x, "f32")
    np.testing.assert_allclose(o2, 2.0 * o1, rtol=1e-14)


# ----------------------------------------------------------------------------
# sampler
# ----------------------------------------------------------------------------


def scfg(V, **kw):
    return synth.sampler_cfg(V, **kw)


def test_entropy_uniform_and_peaked_rows():
    V = 4096
    logits = np.zeros((3, V))
    logits[1, 17] = 80.0           # one dominant logit
    logits[2, [5, 9]] = 80.0       # tie at the max: lowest id wins
    out = O.sample_renoise(logits, scfg(V))
    assert abs(out["entropy"][0] - math.log(V)) < 1e-12
    assert out["entropy"][1] < 1e-20
    assert abs(out["entropy"][2] - math.log(2)) < 1e-12
    assert list(out["commit"]) == [False, True, True]
    assert out["tokens"][1] == 17 and out["tokens"][2] == 5
    assert out["n_renoised"] == 1


def test_entropy_matches_library_and_commit_sets():
    V = 4096
    g = synth.generator(7)
    logits = np64(synth.sampler_logits(64, V, g))
    for t in (1.0, 0.7):
        s = scfg(V, t_max=t, t_min=t)
        out = O.sample_renoise(logits, s)
        p = scipy.special.softmax(logits / t, axis=1)
        np.testing.assert_allclose(out["entropy"], scipy.stats.entropy(p, axis=1), rtol=1e-9, atol=1e-12)
        c = out["commit"]
        np.testing.assert_array_equal(c, out["entropy"] < s["tau"])
        assert out["n_renoised"] == int(np.sum(out["entropy"] >= s["tau"]))
        # committed positions carry the argmax; the rest carry the noise tokens
        noise = O.renoise_tokens(64, V, s["seed"], s["step"], s["canvas_idx"])
        np.testing.assert_array_equal(out["tokens"][c], np.argmax(logits, 1)[c])
        np.testing.assert_array_equal(out["tokens"][~c], noise[~c])
        assert 0 < c.sum() < 64
        # probabilities from the row statistics are the tempered softmax
        pr = O.probs(logits, out["row_max"], out["row_z"], out["temperature"])
        np.testing.assert_allclose(pr, p, rtol=1e-10, atol=1e-300)


def test_nonfinite_rows_counted_and_proposals_skip_nan():
    """Failure detection (a reading: the pages never meet non-finite logits).
    Rows with a NaN or +-inf are counted, their entropy is NaN so they are
    re-noised, a NaN is never proposed, and an all-NaN row proposes 0."""
    V = 64
    lg = np.zeros((5, V))
    lg[0, 10] = 5.0                          # ordinary peaked row
    lg[1, 0] = np.nan
    lg[1, 7] = 9.0                           # NaN ignored: 7 is the argmax
    lg[2, :] = np.nan                        # no number at all
    lg[3, 3] = np.inf
    lg[4, :] = -np.inf
    lg[4, 0] = np.nan                        # -inf is a value: first -inf after the NaN
    with np.errstate(invalid="ignore"):
        out = O.sample_renoise(lg, scfg(V, final_step=False))
        fin = O.sample_renoise(lg, scfg(V, final_step=True))
    assert out["n_nonfinite"] == 4
    np.testing.assert_array_equal(fin["tokens"], [10, 7, 0, 3, 1])
    assert np.isfinite(out["entropy"][0]) and np.isnan(out["entropy"][1:]).all()
    noise = O.renoise_tokens(5, V, 1, 0, 0)
    np.testing.assert_array_equal(out["tokens"][1:], noise[1:])
    assert out["commit"][0] and out["n_renoised"] == 4


def test_final_step_commits_everything():
    V = 4096
    logits = np.zeros((4, V))
    out = O.sample_renoise(logits, scfg(V, final_step=True))
    assert out["commit"].all() and out["n_renoised"] == 0
    assert (out["tokens"] == 0).all()


def test_temperature_schedule_endpoints():
    assert O.temperature(1.5, 0.5, 0, 48) == 1.5
    assert abs(O.temperature(1.5, 0.5, 47, 48) - 0.5) < 1e-15
    vals = [O.temperature(1.5, 0.5, i, 48) for i in range(48)]
    np.testing.assert_allclose(np.diff(vals), -1.0 / 47, rtol=1e-12)


# ----------------------------------------------------------------------------
# self-conditioning, head
# ----------------------------------------------------------------------------


def test_selfcond_zero_input_is_noop_and_one_hot_picks_row():
    D, V, F = 64, 512, 32
    g = synth.generator(9)
    E = np64(synth.embed_table(V, D, g, "bf16"))
    sc = npw(synth.selfcond_weights(D, F, g, "bf16"))
    tok = np.array([3, 7, 511])
    a = O.embed_selfcond(tok, E, np.zeros((3, D)), sc, "bf16")
    b = O.embed_selfcond(tok, E, None, None, "bf16")
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(b, E[tok])
    p = np.zeros((2, V))
    p[0, 11] = 1.0
    p[1, 400] = 1.0
    np.testing.assert_array_equal(O.soft_embed(p, E, "bf16"), E[[11, 400]])


def test_lm_head_tied_is_textbook_product():
    D, V = 64, 1000
    g = synth.generator(10)
    E = np64(synth.embed_table(V, D, g, "f32"))
    x = np64(synth.hidden_states(5, D, g, "f32"))
    w = np.ones(D)
    lg = O.lm_head(x, w, E, 0.0, "f32")
    h = x / np.sqrt(np.mean(x * x, -1, keepdims=True))
    np.testing.assert_allclose(lg, np.einsum("nd,vd->nv", h, E), rtol=1e-11, atol=1e-11)


# ----------------------------------------------------------------------------
# configuration wiring
# ----------------------------------------------------------------------------


def test_parameter_count_matches_pages():
    """[THK] Architecture: 25.2B total, 3.8B active (the latter includes parts
    outside this text stack, so it only bounds the count loosely)."""
    m = synth.full_model_cfg()
    total, active = O.param_count(2816, 30, 6, m["sliding"], m["global"], 128, 8, 704, 704,
                                  262144, sc_ffn=704)
    assert abs(total / 25.2e9 - 1) < 0.02, total
    assert abs(active / 3.8e9 - 1) < 0.10, active


def test_layer_schedule_every_sixth_is_global():
    types = [O.layer_type(l, 6) for l in range(30)]
    assert sum(types) == 5
    assert [l for l in range(30) if types[l]] == [5, 11, 17, 23, 29]


def test_tiny_step_and_commit_run_and_step0_selfcond_noop():
    mcfg = synth.tiny_model_cfg()
    w = synth.model_weights(mcfg, seed=0)
    wn = dict(embed=np64(w["embed"]), w_final_norm=np64(w["w_final_norm"]), sc=npw(w["sc"]),
              attn=[npw(a) for a in w["attn"]], moe=[npw(m) for m in w["moe"]],
              layer_scalar=w["layer_scalar"])
    g = synth.generator(1)
    L, Hkv, dh = 2, 2, 64
    kv = dict(k=[np.zeros((Hkv, 256, dh)) for _ in range(L)],
              v=[np.zeros((Hkv, 256, dh)) for _ in range(L)], kv_len=0)
    prompt = synth.tokens(64, 4096, g).numpy()
    kn, vn = O.commit_canvas(mcfg, wn, kv, prompt, "f32")
    for l in range(L):
        kv["k"][l][:, :64], kv["v"][l][:, :64] = kn[l], vn[l]
    kv["kv_len"] = 64
    c0 = O.canvas_noise(32, 4096, 1, 0)
    s = scfg(4096)
    a = O.canvas_step(mcfg, wn, kv, dict(tokens=c0, u=np.zeros((32, 256))), s, "f32")
    b = O.canvas_step(mcfg, dict(wn, sc=None), kv, dict(tokens=c0, u=None), s, "f32")
    np.testing.assert_array_equal(a["logits"], b["logits"])
    assert a["tokens"].shape == (32,) and a["u_next"].shape == (32, 256)
    assert np.all((a["tokens"] >= 0) & (a["tokens"] < 4096))
