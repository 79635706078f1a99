"""Plain, slow CPU oracle for one DiffusionGemma-style canvas denoising step.

TEST INFRASTRUCTURE ONLY.  This module is the reference the HIP library is
checked against.  Only the test-suite, the smoke check and the CPU-baseline
leg of the benchmark may import it; the product library never calls it and
shares no code with it.

Arithmetic is float64 throughout.  Inputs arrive as float arrays (bfloat16
values widen to float64 exactly).  When the model dtype is bfloat16, values
are rounded to bfloat16 at the points where the model stores a tensor in its
own dtype: the pages' ``rms`` helper casts its result back to the input dtype
(aitrends.kr notebook summary, QK-norm paragraph and its rms code), and the
projections, attention output and residual stream of a bf16 model are bf16
tensors.  The storage points are listed next to each function.  With
``dtype='f32'`` nothing is rounded (pure float64).

Sources (the five web pages on DiffusionGemma), cited by page and section:
  [AIT]  aitrends.kr summary of a DiffusionGemma-26B notebook: details
         paragraphs (QK-norm + rms code, RoPE + rotate code, attention +
         projection code, sampler) and the glossary (Scalar QK Norm,
         Partial RoPE, Layer Scalar, Self-conditioning, MoE, Sliding-window).
  [THK]  thakicloud.github.io "DiffusionGemma 26B-A4B" post: Architecture.
  [VLG]  velog.io "DiffusionGemma Self-conditioning" post: Self-conditioning,
         DiffusionGemma structure (block diffusion, soft embedding).
  [REV]  blog.secrett2633.cloud review of the DiffusionGemma Technical
         Report: section 1 (Canvas, Adaptive Stopping).
  [ABN]  aibars.net news item: block-autoregressive denoising and
         self-correction; text diffusion.

Every function states the reading it takes where the pages leave a step open.
"""
import math

import numpy as np

from .philox import philox4x32_10, uniform_token

_COLS = 16384   # output-column slice for the vocabulary-wide products

# ----------------------------------------------------------------------------
# precision helpers
# ----------------------------------------------------------------------------


def round_bf16(x):
    """Round to bfloat16 (round-to-nearest-even) and return float64.

    Goes through float32 first, as a device converts an fp32 register.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    out = u.astype(np.uint32).view(np.float32).astype(np.float64)
    return out.reshape(np.shape(x))


def store(x, dtype):
    """Value of ``x`` after storing it as a tensor of the model dtype."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# A1 RMSNorm  [AIT] QK-norm paragraph, rms code
# ----------------------------------------------------------------------------


def rms(x, w=1.0, eps=1e-6):
    """w * x * sqrt(d) / (||x||_2 + eps) along the last axis.

    The eps is added to the L2 norm itself, not inside a square root of the
    mean square, as the rms code on [AIT] writes it.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.asarray(w, dtype=np.float64) * x * math.sqrt(d) / (nrm + eps)


# ----------------------------------------------------------------------------
# A3/A4 split-half RoPE, partial in global layers  [AIT] RoPE paragraph,
# rotate code, glossary "Partial RoPE"
# ----------------------------------------------------------------------------


def rope_freqs(head_dim, base, rotary_factor=1.0):
    """Per-pair angular frequencies f_t, t < head_dim/2.

    f_t = base**(-2t/head_dim) over the full spectrum; with a partial rotary
    factor r only the first r fraction of the frequencies is kept and the
    rest is set to zero (no rotation on those dims).  Reading: the spectrum
    is not re-spaced over the kept part; the tail is zeroed.
    """
    half = head_dim // 2
    t = np.arange(half, dtype=np.float64)
    f = np.power(float(base), -2.0 * t / head_dim)
    keep = int(round(rotary_factor * half))
    f[keep:] = 0.0
    return f


def rope(x, positions, freqs):
    """Split-half rotation: pair (t, t + d/2) rotated by angle p * f_t.

    x: [..., n, d]; positions: [n] absolute positions.
    out_t = x_t cos - x_{t+d/2} sin ; out_{t+d/2} = x_{t+d/2} cos + x_t sin.
    """
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * freqs[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ----------------------------------------------------------------------------
# attention layer  [AIT] attention paragraph + projection code, glossary
# "Scalar QK Norm", "Sliding-window Attention"
# ----------------------------------------------------------------------------


def visible_keys(cfg, kv_len, n_tok, causal):
    """Boolean mask [n_tok, kv_len + n_tok]: may query j see key m?

    Keys 0..kv_len-1 are committed cache rows, kv_len.. are this call's rows.
    Decode (causal=0): every canvas row, plus committed rows
      [max(0, kv_len - W), kv_len) in sliding layers, all of them in global
      layers ([AIT] glossary "Sliding-window Attention": all canvas tokens
      plus a fixed-length committed prefix in front of the canvas).
    Encode (causal=1): key m is visible to the query at position p = kv_len+j
      iff m <= p, and, in sliding layers, m > p - W (a per-query window).
    """
    n_keys = kv_len + n_tok
    m = np.arange(n_keys)[None, :]
    p = kv_len + np.arange(n_tok)[:, None]
    sliding = cfg["layer_type"] == 0
    W = cfg["window"]
    if causal:
        vis = m <= p
        if sliding:
            vis &= m > p - W
    else:
        vis = np.ones((n_tok, n_keys), dtype=bool)
        if sliding:
            lo = max(0, kv_len - W)
            vis[:, :lo] = False
    return vis


def project_qkv(cfg, w, x, pos0, dtype):
    """Pre-norm, projections, QK-norm, V-norm and RoPE for one layer.

    Storage points (model dtype): h after the pre-norm; the raw projections;
    q, k after norm + rotation; v after its unit-RMS norm.
    Global layers share the K/V projection (W_v = W_k, [AIT] attention
    paragraph): the raw value equals the raw key; only the key gets the
    gamma_k norm and the rotation, the value is normalised to unit RMS.
    Returns q [Hq, n, d], k [Hkv, n, d], v [Hkv, n, d].
    """
    eps = cfg["rms_eps"]
    Hq, Hkv, dh = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    n = x.shape[0]
    h = store(rms(x, w["w_in_norm"], eps), dtype)
    q = store(h @ w["w_q"].T, dtype)
    k = store(h @ w["w_k"].T, dtype)
    if cfg["shared_kv"]:
        v = k.copy()
    else:
        v = store(h @ w["w_v"].T, dtype)
    # 'l (n h) -> n l h': head n owns columns [n*dh, (n+1)*dh)
    q = q.reshape(n, Hq, dh).transpose(1, 0, 2)
    k = k.reshape(n, Hkv, dh).transpose(1, 0, 2)
    v = v.reshape(n, Hkv, dh).transpose(1, 0, 2)
    freqs = rope_freqs(dh, cfg["rope_base"],
                       cfg["rotary_factor"] if cfg["layer_type"] == 1 else 1.0)
    pos = pos0 + np.arange(n)
    q = store(rope(rms(q, w["q_norm"], eps), pos, freqs), dtype)
    k = store(rope(rms(k, w["k_norm"], eps), pos, freqs), dtype)
    if cfg["v_unit_rms"]:
        v = store(rms(v, 1.0, eps), dtype)
    return q, k, v


def attention_core(q, K, V, vis, n_rep):
    """softmax(q K^T * 1) V per q head over the visible keys.

    The softmax scale is 1: with scalar QK-norm weights the logit is already
    d_h * gamma_q * gamma_k * cos(theta), a fixed per-layer temperature
    ([AIT] QK-norm paragraph, glossary "Scalar QK Norm").
    Query head n reads kv head n // n_rep (contiguous grouping; reading).
    q [Hq, n, d]; K, V [Hkv, n_keys, d]; vis [n, n_keys].
    Returns o [Hq, n, d], scores [Hq, n, n_keys], probs [Hq, n, n_keys].
    """
    Hq = q.shape[0]
    o = np.empty_like(q)
    scores = np.zeros((Hq, q.shape[1], K.shape[1]))
    probs = np.zeros_like(scores)
    cols = np.nonzero(vis.any(axis=0))[0]      # keys no query can see are never read
    vv = vis[:, cols]
    for hq in range(Hq):
        g = hq // n_rep
        s = q[hq] @ K[g][cols].T
        scores[hq][:, cols] = s
        s = np.where(vv, s, -np.inf)
        mx = np.max(s, axis=-1, keepdims=True)
        e = np.exp(s - mx)
        a = e / np.sum(e, axis=-1, keepdims=True)
        probs[hq][:, cols] = a
        o[hq] = a @ V[g][cols]
    return o, scores, probs


def attn_layer(cfg, w, cache_k, cache_v, kv_len, x, causal, dtype, want_probs=False):
    """x + Attention(x) for one layer; returns (x_out, k_new, v_new[, extras]).

    cache_k, cache_v: [Hkv, >=kv_len, d] committed rows (post-norm/rotation).
    Decode (causal=0) is the canvas pass; encode (causal=1) is the commit
    pass whose k_new/v_new rows the caller appends at [kv_len, kv_len+n)
    ([AIT] attention paragraph: decode attends to committed|canvas, encode
    behaves like a causal prefill).
    Storage points: attention output o, and x_out = x + o W_o^T (one rounding).
    """
    Hq, Hkv, dh = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    q, k, v = project_qkv(cfg, w, x, kv_len, dtype)
    K = np.concatenate([np.asarray(cache_k, np.float64)[:, :kv_len], k], axis=1)
    V = np.concatenate([np.asarray(cache_v, np.float64)[:, :kv_len], v], axis=1)
    vis = visible_keys(cfg, kv_len, n, causal)
    o, scores, probs = attention_core(q, K, V, vis, Hq // Hkv)
    o = store(o.transpose(1, 0, 2).reshape(n, Hq * dh), dtype)
    x_out = store(x + o @ w["w_o"].T, dtype)
    if want_probs:
        return x_out, k, v, dict(q=q, K=K, V=V, vis=vis, scores=scores, probs=probs)
    return x_out, k, v


# ----------------------------------------------------------------------------
# MoE block  [AIT] glossary "MoE"; [THK] Architecture (128 experts, 8 active
# + 1 shared)
# ----------------------------------------------------------------------------


def silu(z):
    return z / (1.0 + np.exp(-z))


def router_topk(r, top_k, route_scale=1.0):
    """Top-k experts per token and their mixing weights.

    Scores are exp(router_key . x), renormalised over the chosen experts and
    scaled ([AIT] glossary "MoE").  Reading: p = softmax(r) over all
    experts; the top_k largest logits are chosen (ties to the lower expert
    id); w = p_T / sum(p_T) * route_scale.
    r: [n, E].  Returns idx int64 [n, k] (in descending-score order) and w.
    """
    r = np.asarray(r, dtype=np.float64)
    n, E = r.shape
    p = np.exp(r - r.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    idx = np.zeros((n, top_k), dtype=np.int64)
    wts = np.zeros((n, top_k))
    for t in range(n):
        order = sorted(range(E), key=lambda e: (-r[t, e], e))[:top_k]
        idx[t] = order
        pt = p[t, order]
        wts[t] = pt / pt.sum() * route_scale
    return idx, wts


def swiglu_ffn(h, wg, wu, wd, dtype):
    """W_d (silu(W_g h) * (W_u h)); the hidden activation is a model-dtype tensor."""
    a = store(silu(h @ wg.T) * (h @ wu.T), dtype)
    return a @ wd.T


def moe_block(cfg, w, x, dtype, router_logits=None):
    """x_out = s_l * (x + MoE(rms(x))) with a brute-force per-token loop.

    y_t = shared(h_t) + sum over the top-k experts e of w_e * expert_e(h_t);
    the shared expert is always added ([AIT] glossary "MoE"; [THK]).
    The layer scalar s_l rescales the layer's residual-stream output
    ([AIT] glossary "Layer Scalar"); reading: applied once, after the MoE
    residual, so s_l = 1 is the identity.
    Storage points: h, each expert's hidden activation, and x_out.
    Router logits are kept in float64 (the device keeps them in fp32).
    Returns x_out, idx, wts, router_logits.
    """
    eps = cfg["rms_eps"]
    x = np.asarray(x, dtype=np.float64)
    h = store(rms(x, w["w_in_norm"], eps), dtype)
    if router_logits is None:
        r = h @ w["w_router"].T
    else:
        r = np.asarray(router_logits, dtype=np.float64)
    idx, wts = router_topk(r, cfg["top_k"], cfg["route_scale"])
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        ht = h[t:t + 1]
        acc = swiglu_ffn(ht, w["ws_gate"], w["ws_up"], w["ws_down"], dtype)[0]
        for j in range(cfg["top_k"]):
            e = idx[t, j]
            acc = acc + wts[t, j] * swiglu_ffn(ht, w["w_gate"][e], w["w_up"][e],
                                               w["w_down"][e], dtype)[0]
        y[t] = acc
    x_out = store(cfg["layer_scalar"] * (x + y), dtype)
    return x_out, idx, wts, r


def moe_block_grouped(cfg, w, x, dtype, router_logits=None):
    """Same result as moe_block, with the per-token expert calls batched by
    expert (one product per expert over the tokens routed to it) so that the
    full-size shapes finish in seconds.  Each token's terms are added in the
    same order as the per-token loop: shared expert first, then the chosen
    experts in descending-score order.
    """
    eps = cfg["rms_eps"]
    x = np.asarray(x, dtype=np.float64)
    h = store(rms(x, w["w_in_norm"], eps), dtype)
    if router_logits is None:
        r = h @ w["w_router"].T
    else:
        r = np.asarray(router_logits, dtype=np.float64)
    idx, wts = router_topk(r, cfg["top_k"], cfg["route_scale"])
    n = x.shape[0]
    terms = np.zeros((cfg["top_k"], n, x.shape[1]))
    for e in np.unique(idx):
        tok, slot = np.nonzero(idx == e)
        out = swiglu_ffn(h[tok], w["w_gate"][e], w["w_up"][e], w["w_down"][e], dtype)
        terms[slot, tok] = wts[tok, slot][:, None] * out
    y = swiglu_ffn(h, w["ws_gate"], w["ws_up"], w["ws_down"], dtype)
    for j in range(cfg["top_k"]):
        y = y + terms[j]
    x_out = store(cfg["layer_scalar"] * (x + y), dtype)
    return x_out, idx, wts, r


# ----------------------------------------------------------------------------
# LM head, sampler, self-conditioning
# ----------------------------------------------------------------------------


def lm_head(x, w_final_norm, embed, eps, dtype):
    """logits = rms(x, w_final) E^T with the head tied to the embedding table.

    Reading: a final RMSNorm precedes the tied head; no soft-cap.
    Storage point: the normed hidden (model dtype).  Logits stay float64.
    """
    h = store(rms(x, w_final_norm, eps), dtype)
    V = embed.shape[0]
    out = np.empty((h.shape[0], V))
    for c0 in range(0, V, _COLS):      # output columns in slices: no sum is split
        out[:, c0:c0 + _COLS] = h @ np.asarray(embed[c0:c0 + _COLS], np.float64).T
    return out


def temperature(t_max, t_min, step, n_steps):
    """Linear schedule from t_max at step 0 to t_min at step n_steps-1.

    [AIT] sampler paragraph: the temperature is lowered linearly over the
    denoising steps.  Reading: t_i = t_max + (t_min - t_max) * i / (S - 1).
    """
    if n_steps <= 1:
        return float(t_max)
    return float(t_max) + (float(t_min) - float(t_max)) * step / (n_steps - 1)


def first_argmax(s):
    """Per row, the index of the largest entry that is a number (lowest id on
    ties).  Reading for non-finite logits, which the pages never meet: a NaN
    is never a candidate, -inf is an ordinary (smallest) value, and a row with
    no number at all proposes token 0."""
    s = np.asarray(s, dtype=np.float64)
    nan = np.isnan(s)
    filled = np.where(nan, -np.inf, s)
    idx = np.argmax(filled, axis=1)
    for r in np.nonzero(np.isneginf(filled[np.arange(len(s)), idx]))[0]:
        cand = np.nonzero(~nan[r])[0]
        idx[r] = cand[0] if len(cand) else 0
    return idx


def row_stats(logits, t):
    """Per row of l/t: max m, Z = sum e^d, S = sum e^d d (d = l/t - m), entropy H.

    H = ln Z - S/Z equals -sum p ln p for p = softmax(l/t), in nats.
    Also the argmax of the raw logits, lowest id on ties (first_argmax).
    A row holding a NaN or +-inf has a NaN entropy (so it never commits on
    its own).
    """
    l = np.asarray(logits, dtype=np.float64) / t
    m = l.max(axis=1, keepdims=True)
    d = l - m
    e = np.exp(d)
    Z = e.sum(axis=1)
    S = (e * d).sum(axis=1)
    H = np.log(Z) - S / Z
    with np.errstate(invalid="ignore"):
        H = np.where(np.isfinite(np.asarray(logits, np.float64)).all(axis=1), H, np.nan)
    amax = first_argmax(logits)
    return m[:, 0], Z, S, H, amax


def renoise_tokens(n_pos, vocab, seed, step, canvas_idx):
    """Uniform random tokens for positions 0..n_pos-1 at one denoising step.

    Philox4x32-10, key = (seed low word, seed high word), counter =
    (position, step, canvas index, 0); token = floor(X0 * V / 2**32).
    The initial canvas uses step = 0xFFFFFFFF.
    """
    ctr = np.zeros((n_pos, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n_pos)
    ctr[:, 1] = step & 0xFFFFFFFF
    ctr[:, 2] = canvas_idx & 0xFFFFFFFF
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    x = philox4x32_10(ctr, key)
    return uniform_token(x[:, 0], vocab)


def canvas_noise(n_pos, vocab, seed, canvas_idx):
    """Initial canvas: a block of uniform random tokens ([ABN] text diffusion:
    generation starts from a random-noise block)."""
    return renoise_tokens(n_pos, vocab, seed, 0xFFFFFFFF, canvas_idx)


def gumbel_noise(rows, vocab, seed, step, canvas_idx):
    """Gumbel(0, 1) noise g[j, v] for the sampled-token variant.

    Gumbel-max: argmax_v (l_v/t + g_v) is a draw from softmax(l/t)
    (textbook; used here for the reading "sample the committed token"
    instead of taking the argmax).  Uniforms: Philox4x32-10 with key
    (seed lo, seed hi) and counter (position, step, canvas, 1 + v // 4); word
    v % 4 gives k = word >> 9 (23 bits) and u = (k + 1/2) 2^-23, exact in
    fp32; E = -ln u, taken as -ln(1 - w) with w = 1 - u (exact) through
    log1p when u >= 1/2; g = -ln E.  Float64 throughout.
    rows: position indices.  Returns float64 [len(rows), vocab].
    """
    rows = np.asarray(rows, dtype=np.int64)
    nq = (vocab + 3) // 4
    ctr = np.zeros((len(rows), nq, 4), dtype=np.uint64)
    ctr[..., 0] = rows[:, None]
    ctr[..., 1] = step & 0xFFFFFFFF
    ctr[..., 2] = canvas_idx & 0xFFFFFFFF
    ctr[..., 3] = 1 + np.arange(nq)[None, :]
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    x = philox4x32_10(ctr, key).reshape(len(rows), nq * 4)[:, :vocab].astype(np.int64)
    k = x >> 9
    u = (k + 0.5) * 2.0 ** -23
    w = ((2 ** 23 - 1 - k) + 0.5) * 2.0 ** -23
    e = np.where(u < 0.5, -np.log(u), -np.log1p(-w))
    return -np.log(e)


def sorted_cumulative_commit(H, bound):
    """Commit rule "prefix within the entropy bound" read as a sorted
    cumulative bound ([AIT] sampler paragraph and its generation-config
    note; the EB-sampler of Ben-Hamu et al. 2025 is the published form).

    Positions are taken in ascending entropy (ties: lower position first);
    the position at each rank commits iff the summed entropy of the
    positions ranked before it is <= bound.  The committed set is the
    longest low-entropy prefix whose entropy sum minus its largest member
    stays within the bound; the lowest-entropy position always commits
    (bound >= 0).  Returns (commit bool [n], prior_sum float64 [n]).
    """
    H = np.asarray(H, dtype=np.float64)
    order = sorted(range(len(H)), key=lambda j: (H[j], j))
    commit = np.zeros(len(H), dtype=bool)
    prior = np.zeros(len(H))
    cum = 0.0
    for j in order:
        prior[j] = cum
        commit[j] = cum <= bound
        cum += H[j]
    return commit, prior


def sample_renoise(logits, scfg, pred_prev=None):
    """Entropy-bound commit / uniform re-noise for every canvas position.

    [AIT] sampler paragraph: per-position entropy of the tempered
    distribution; low-entropy positions are fixed, the rest re-noised with
    uniform random tokens ([ABN] self-correction).  Reading (the configs fix
    it): position j commits iff H_j < tau; committed positions take the
    argmax token (lowest id on ties); on the final step every position
    commits.
    scfg: dict(vocab, tau, t_max, t_min, n_steps, step, canvas_idx, seed,
    final_step).  Returns a dict.

    Variants (alternative readings of the same passages):
      scfg["commit_rule"] = "sorted_cumulative": sorted_cumulative_commit
        with bound tau;
      scfg["token_rule"] = "gumbel": the proposal is the Gumbel-max draw
        argmax_v (l_v/t + g_v) (lowest id on ties) instead of the argmax;
      pred_prev: the previous step's proposals; n_changed counts the
        positions whose proposal differs (output stability, [REV] section 1
        Adaptive Stopping).
    """
    t = temperature(scfg["t_max"], scfg["t_min"], scfg["step"], scfg["n_steps"])
    m, Z, S, H, amax = row_stats(logits, t)
    n = logits.shape[0]
    margin = None
    if scfg.get("token_rule", "argmax") == "gumbel":
        sc = np.asarray(logits, dtype=np.float64) / t + gumbel_noise(
            np.arange(n), scfg["vocab"], scfg["seed"], scfg["step"], scfg["canvas_idx"])
        pred = first_argmax(sc)
        top2 = -np.sort(-sc, axis=1)[:, :2]
        margin = top2[:, 0] - top2[:, 1]
    else:
        pred = amax
    prior = None
    if scfg.get("commit_rule", "entropy") == "sorted_cumulative":
        commit, prior = sorted_cumulative_commit(H, scfg["tau"])
    else:
        commit = H < scfg["tau"]
    if scfg.get("final_step", False):
        commit[:] = True
    noise = renoise_tokens(n, scfg["vocab"], scfg["seed"], scfg["step"], scfg["canvas_idx"])
    tokens = np.where(commit, pred, noise)
    n_changed = None if pred_prev is None else int(np.sum(np.asarray(pred_prev) != pred))
    n_nonfinite = int(np.sum(~np.isfinite(np.asarray(logits, np.float64)).all(axis=1)))
    return dict(tokens=tokens.astype(np.int64), commit=commit, entropy=H,
                n_renoised=int(np.sum(~commit)), n_nonfinite=n_nonfinite, argmax=amax, pred=pred.astype(np.int64),
                n_changed=n_changed, gumbel_margin=margin, prior_sum=prior, row_max=m,
                row_z=Z, temperature=t)


def probs(logits, row_max, row_z, t):
    """Tempered softmax p = exp(l/t - m) / Z."""
    l = np.asarray(logits, dtype=np.float64) / t
    return np.exp(l - row_max[:, None]) / row_z[:, None]


def soft_embed(p, embed, dtype):
    """Expected embedding u = P E ([AIT] glossary "Self-conditioning").

    Storage points: P and u (model dtype)."""
    p = store(p, dtype)
    D = embed.shape[1]
    u = np.empty((p.shape[0], D))
    for c0 in range(0, D, 256):        # output columns in slices: no sum is split
        u[:, c0:c0 + 256] = p @ np.asarray(embed[:, c0:c0 + 256], np.float64)
    return store(u, dtype)


def embed_selfcond(tokens, embed, u, sc, dtype):
    """x_j = E[c_j] + MLP_sc(u_j).

    [AIT] glossary "Self-conditioning"; [VLG] soft embedding: the expected
    embedding passes through a small MLP and is added to the canvas input.
    Reading: bias-free SwiGLU MLP D -> F_sc -> D, so MLP_sc(0) = 0 and the
    first step (u = 0) is unaffected.  No sqrt(D) embedding scale.
    sc = None disables self-conditioning.
    Storage points: the MLP hidden activation and x.
    """
    x = np.asarray(np.asarray(embed)[np.asarray(tokens)], np.float64)   # gather, then widen
    if sc is None or u is None:
        return store(x, dtype)
    add = swiglu_ffn(np.asarray(u, np.float64), sc["sc_gate"], sc["sc_up"], sc["sc_down"], dtype)
    return store(x + add, dtype)


# ----------------------------------------------------------------------------
# whole step and commit
# ----------------------------------------------------------------------------


def layer_type(l, global_every):
    """Hybrid schedule: one global layer every `global_every` layers (l % 6 == 5)."""
    return 1 if (l % global_every) == global_every - 1 else 0


def _injected(weights, l):
    rl = weights.get("router_logits")
    return None if rl is None else rl[l]


def canvas_step(model, weights, kv, state, scfg, dtype):
    """One denoising step over the canvas (decode mode through every layer).

    model: dict(n_layers, global_every, sliding=cfg, global=cfg, moe=cfg,
                rms_eps, vocab).
    weights: dict(embed, w_final_norm, sc (or None), attn[l], moe[l],
    layer_scalar[l], optionally router_logits[l]: injected router logits of
    layer l used in place of the router product, None entries computed).
    kv: dict(k[l], v[l], kv_len).  state: dict(tokens, u (or None)).
    Returns dict(sample outputs, logits, u_next, x_final).
    """
    x = embed_selfcond(state["tokens"], weights["embed"], state.get("u"),
                       weights.get("sc"), dtype)
    P = kv["kv_len"]
    for l in range(model["n_layers"]):
        acfg = model["global"] if layer_type(l, model["global_every"]) else model["sliding"]
        x, _, _ = attn_layer(acfg, weights["attn"][l], kv["k"][l], kv["v"][l], P, x, 0, dtype)
        x, _, _, _ = moe_block_grouped(dict(model["moe"], layer_scalar=weights["layer_scalar"][l]),
                                       weights["moe"][l], x, dtype, router_logits=_injected(weights, l))
    logits = lm_head(x, weights["w_final_norm"], weights["embed"], model["rms_eps"], dtype)
    out = sample_renoise(logits, scfg)
    p = probs(logits, out["row_max"], out["row_z"], out["temperature"])
    out["u_next"] = soft_embed(p, weights["embed"], dtype)
    out["logits"] = logits
    out["x_final"] = x
    return out


def commit_canvas(model, weights, kv, tokens, dtype):
    """Encode pass: append the final tokens' K/V to every layer's cache.

    Causal attention over [committed ; these tokens] ([AIT] attention
    paragraph: encode behaves like a causal prefill; [ABN] block-
    autoregressive: a finished block is committed to the KV cache).  No
    self-conditioning input (reading).  Nothing after the last layer's K/V
    is needed, so the last layer stops after its projections ([AIT]:
    work after the last layer is skipped).
    Returns lists k_new[l], v_new[l]; the caller appends and advances kv_len.
    """
    x = embed_selfcond(tokens, weights["embed"], None, None, dtype)
    P = kv["kv_len"]
    k_new, v_new = [], []
    L = model["n_layers"]
    for l in range(L):
        acfg = model["global"] if layer_type(l, model["global_every"]) else model["sliding"]
        if l == L - 1:
            _, k, v = project_qkv(acfg, weights["attn"][l], x, P, dtype)
        else:
            x, k, v = attn_layer(acfg, weights["attn"][l], kv["k"][l], kv["v"][l], P, x, 1, dtype)
            x, _, _, _ = moe_block_grouped(dict(model["moe"], layer_scalar=weights["layer_scalar"][l]),
                                           weights["moe"][l], x, dtype, router_logits=_injected(weights, l))
        k_new.append(k)
        v_new.append(v)
    return k_new, v_new


def param_count(D, n_layers, global_every, sliding, glob, n_experts, top_k, ffn, shared_ffn,
                vocab, sc_ffn=0):
    """Parameter total and active-per-token count for a model configuration.

    Counts weights only (norm vectors included); the head is tied to E.
    """
    def attn_params(c):
        q = c["n_q_heads"] * c["head_dim"] * D
        k = c["n_kv_heads"] * c["head_dim"] * D
        v = 0 if c["shared_kv"] else k
        o = D * c["n_q_heads"] * c["head_dim"]
        return q + k + v + o + 2 * c["head_dim"] + D
    total = vocab * D + D + 3 * D * sc_ffn
    active = total
    for l in range(n_layers):
        a = attn_params(glob if layer_type(l, global_every) else sliding)
        router = n_experts * D
        experts = n_experts * 3 * ffn * D
        shared = 3 * shared_ffn * D
        total += a + router + experts + shared + D
        active += a + router + top_k * 3 * ffn * D + shared + D
    return total, active


def generate(model, weights, kv, prompt, n_canvases, canvas_len, max_steps, seed, t_max, t_min, tau, dtype,
             stop_rule="renoised"):
    """Block-autoregressive generation from the step and commit above.

    [ABN] block-autoregressive denoising: the prompt is committed, then each
    block of canvas_len positions starts from uniform noise, is denoised, and
    is committed to the KV cache before the next block.  [REV] section 1
    (Adaptive Stopping): the loop stops early once the prediction settles.
    stop_rule "renoised": stop after a step that re-noised no position.
    stop_rule "stable": from the second step on, stop once no position's
    proposal changed since the previous step; the canvas then takes the
    proposals everywhere.  The last allowed step commits every position.
    kv: dict(k[l], v[l], kv_len) with room for the prompt and the canvases;
    it is copied, not modified.
    Returns dict(tokens [n_canvases, canvas_len], steps [n_canvases],
    min_entropy_gap: the smallest |H - tau| met, min_lead: the smallest
    argmax lead met on any position, kv: the cache after the last commit).
    """
    kv = dict(k=[np.array(a, np.float64) for a in kv["k"]], v=[np.array(a, np.float64) for a in kv["v"]],
              kv_len=kv["kv_len"])
    V = model["vocab"]

    def append(tok):
        k_new, v_new = commit_canvas(model, weights, kv, tok, dtype)
        P, n = kv["kv_len"], len(tok)
        for l in range(model["n_layers"]):
            kv["k"][l][:, P:P + n] = k_new[l]
            kv["v"][l][:, P:P + n] = v_new[l]
        kv["kv_len"] = P + n

    if prompt is not None and len(prompt):
        append(np.asarray(prompt))
    out, steps = [], []
    gap, lead = np.inf, np.inf
    for c in range(n_canvases):
        tokens, u, pred_prev = canvas_noise(canvas_len, V, seed, c), None, None
        used = 0
        for i in range(max_steps):
            final = i == max_steps - 1
            s = dict(vocab=V, tau=tau, t_max=t_max, t_min=t_min, n_steps=max_steps, step=i, canvas_idx=c,
                     seed=seed, final_step=final)
            r = canvas_step(model, weights, kv, dict(tokens=tokens, u=u), s, dtype)
            used += 1
            gap = min(gap, float(np.min(np.abs(r["entropy"] - tau))))
            top = -np.partition(-r["logits"], 1, axis=1)[:, :2]
            lead = min(lead, float(np.min(top[:, 0] - top[:, 1])))
            tokens, u = r["tokens"], r["u_next"]
            if final:
                break
            if stop_rule == "stable":
                changed = None if pred_prev is None else int(np.sum(r["pred"] != pred_prev))
                pred_prev = r["pred"]
                if changed == 0:
                    tokens = r["pred"]
                    break
            elif r["n_renoised"] == 0:
                break
        out.append(tokens)
        steps.append(used)
        append(tokens)
    return dict(tokens=np.array(out), steps=steps, min_entropy_gap=gap, min_lead=lead, kv=kv)
