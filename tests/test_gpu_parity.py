"""HIP path vs the CPU oracle, entry point by entry point, through the C ABI.

Bars: fp32 path max relative error 1e-4, bf16 path 2e-2 (max |gpu - ref| /
max |ref| per tensor); integer outputs (router indices, commit masks,
re-noise tokens, counts) bit-exact where the oracle's deciding margin
exceeds the stated band.
"""
import math

import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from oracle import dg_oracle as O
from tests.helpers import (assert_close, assert_delta_close, check_router_sets, check_sampler_outputs, cuda, np64,
                           npw, rel_err)

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    torch.manual_seed(0)
    yield


def sync():
    torch.cuda.synchronize()


# ----------------------------------------------------------------- RMSNorm


@pytest.mark.parametrize("dtype,n,D", [("f32", 37, 256), ("bf16", 200, 2816), ("bf16", 1, 64)])
def test_rmsnorm(dtype, n, D):
    g = synth.generator(11)
    x = synth.hidden_states(n, D, g, dtype) * 3
    w = synth._uniform(g, (D,), 0.5, 1.5, dtype, "cpu")
    y = B.dg_rmsnorm(x.cuda(), w.cuda(), 1e-6)
    sync()
    ref = O.store(O.rms(np64(x), np64(w), 1e-6), dtype)
    assert_close(np64(y), ref, dtype, "rmsnorm")


# ----------------------------------------------------------------- sampler


def sampler_case(n, V, seed, dtype="f32"):
    """Logits whose rows stay clear of the commit threshold by > 1e-3 nats."""
    g = synth.generator(seed)
    lg = synth.sampler_logits(n, V, g)
    if dtype == "bf16":
        lg = lg.to(torch.bfloat16)
    tau = 0.5 * math.log(V)
    for _ in range(20):
        _, _, _, H, _ = O.row_stats(np64(lg), 1.0)
        bad = np.abs(H - tau) <= 1e-3
        if not bad.any():
            break
        lg[torch.from_numpy(bad)] = (lg[torch.from_numpy(bad)].float() * 1.01).to(lg.dtype)
    return lg


@pytest.mark.parametrize("n,V,dtype,temp", [(32, 4096, "f32", 1.0), (256, 262144, "f32", 1.0),
                                             (77, 262144, "bf16", 1.0), (64, 4096, "f32", 0.7)])
def test_sample_renoise(n, V, dtype, temp):
    lg = sampler_case(n, V, 5 + n, dtype)
    s = synth.sampler_cfg(V, t_max=temp, t_min=temp, step=3, canvas_idx=2)
    out = B.dg_sample_renoise(s, lg.cuda())
    sync()
    ref = O.sample_renoise(np64(lg), s)
    commit = out["commit"].cpu().numpy().astype(bool)
    np.testing.assert_array_equal(commit, ref["commit"])
    np.testing.assert_array_equal(out["tokens"].cpu().numpy(), ref["tokens"])
    assert int(out["n_renoised"].item()) == ref["n_renoised"]
    # entropy lives on the scale [0, ln V]: its error is measured against ln V
    assert np.max(np.abs(out["entropy"].cpu().numpy() - ref["entropy"])) < 1e-4 * math.log(V)
    rs = out["rowstats"].cpu().numpy()
    np.testing.assert_allclose(rs[:, 0], ref["row_max"], rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(rs[:, 1], ref["row_z"], rtol=1e-4)
    # committed positions are never re-noised; the count matches the threshold
    assert (commit == (ref["entropy"] < s["tau"])).all()
    assert int(out["n_renoised"].item()) == int((~commit).sum())


def test_sample_final_step_and_ties():
    V = 4096
    lg = torch.zeros(8, V)
    lg[1, 100] = lg[1, 7] = 50.0        # tie: lowest id wins
    s = synth.sampler_cfg(V, final_step=True)
    out = B.dg_sample_renoise(s, lg.cuda())
    sync()
    assert out["commit"].cpu().numpy().all()
    assert int(out["n_renoised"].item()) == 0
    assert int(out["tokens"][1].item()) == 7
    assert int(out["tokens"][0].item()) == 0
    np.testing.assert_allclose(out["entropy"][0].item(), math.log(V), rtol=1e-5)


def test_canvas_noise():
    for V, ci in ((262144, 0), (4096, 5), (1000, 3)):
        t = B.dg_canvas_noise(300, V, 1, ci)
        sync()
        np.testing.assert_array_equal(t.cpu().numpy(), O.canvas_noise(300, V, 1, ci))


# ----------------------------------------------------------------- LM head / soft embedding


@pytest.mark.parametrize("dtype,n,D,V", [("f32", 32, 256, 4096), ("bf16", 45, 256, 4096),
                                         ("bf16", 45, 320, 4040), ("bf16", 256, 2816, 262144)])
def test_lm_head(dtype, n, D, V):
    g = synth.generator(21)
    E = synth.embed_table(V, D, g, dtype)
    x = synth.hidden_states(n, D, g, dtype)
    wn = synth._uniform(g, (D,), 0.5, 1.5, dtype, "cpu")
    lg = B.dg_lm_head(x.cuda(), wn.cuda(), E.cuda(), 1e-6)
    sync()
    # every column (the oracle slices the vocabulary, never a sum)
    ref = O.lm_head(np64(x), np64(wn), E.float().numpy(), 1e-6, dtype)
    assert_close(lg.cpu().numpy(), ref, "f32" if dtype == "f32" else "bf16", "logits")


@pytest.mark.parametrize("dtype,n,D,V", [("f32", 32, 256, 4096), ("bf16", 45, 320, 8000),
                                         ("bf16", 256, 2816, 262144)])
def test_soft_embed(dtype, n, D, V):
    g = synth.generator(31)
    E = synth.embed_table(V, D, g, dtype)
    lg = synth.sampler_logits(n, V, g)
    s = synth.sampler_cfg(V, t_max=0.8, t_min=0.8)
    Ed = E.cuda()
    out = B.dg_sample_renoise(s, lg.cuda())
    u = B.dg_soft_embed(s, lg.cuda(), out["rowstats"], B.dg_embed_transpose(Ed), dtype)
    sync()
    ref = O.sample_renoise(np64(lg), s)
    p = O.probs(np64(lg), ref["row_max"], ref["row_z"], ref["temperature"])
    uref = O.soft_embed(p, E.float().numpy(), dtype)      # every column
    assert_close(np64(u), uref, dtype, "u = P.E")


def test_embed_transpose():
    E = torch.randn(1000, 192).to(torch.bfloat16).cuda()
    Et = B.dg_embed_transpose(E)
    sync()
    assert torch.equal(Et.cpu(), E.cpu().t().contiguous())


# ----------------------------------------------------------------- attention


def run_gpu_attn(cfg, w, ck, cv, P, x, causal):
    """ck, cv: [Hkv][cap][dh] (the oracle's layout); the device cache holds V
    transposed.  Returns the device x and the cache with V back in row layout."""
    xd = x.clone().cuda()
    kd, vtd = ck.cuda(), cv.transpose(1, 2).contiguous().cuda()
    new_len = B.dg_attn_layer(cfg, cuda(w), kd, vtd, P, xd, causal)
    sync()
    return xd, kd, vtd.transpose(1, 2), new_len


@pytest.mark.parametrize("layer_type", [0, 1])
def test_attn_tiny_encode_then_decode(layer_type):
    """fp32 tiny layer: encode a 64-token prefix into the cache (both sides
    separately), then decode a 32-token canvas against it."""
    cfg = synth.tiny_attn_cfg(layer_type, "f32")
    g = synth.generator(3 + layer_type)
    w = synth.attn_weights(cfg, g)
    Hkv, dh = cfg["n_kv_heads"], cfg["head_dim"]
    xp = synth.hidden_states(64, cfg["hidden"], g, "f32")
    xc = synth.hidden_states(32, cfg["hidden"], g, "f32")
    ck = torch.zeros(Hkv, 128, dh)
    cv = torch.zeros(Hkv, 128, dh)
    xo, kd, vd, n1 = run_gpu_attn(cfg, w, ck, cv, 0, xp, 1)
    assert n1 == 64
    wn = npw(w)
    ref_x, ref_k, ref_v = O.attn_layer(cfg, wn, np.zeros((Hkv, 0, dh)), np.zeros((Hkv, 0, dh)), 0, np64(xp), 1, "f32")
    assert_close(np64(xo), ref_x, "f32", "encode x")
    assert_close(np64(kd)[:, :64], ref_k, "f32", "encode k")
    assert_close(np64(vd)[:, :64], ref_v, "f32", "encode v")
    # decode over the GPU's own cache vs the oracle's own cache
    xd = xc.clone().cuda()
    B.dg_attn_layer(cfg, cuda(w), kd, vd.transpose(1, 2).contiguous(), 64, xd, 0)
    sync()
    ckr = np.zeros((Hkv, 128, dh))
    cvr = np.zeros((Hkv, 128, dh))
    ckr[:, :64], cvr[:, :64] = ref_k, ref_v
    ref_d, _, _ = O.attn_layer(cfg, wn, ckr, cvr, 64, np64(xc), 0, "f32")
    assert_close(np64(xd), ref_d, "f32", "decode x")


@pytest.mark.parametrize("n_tok,P", [(256, 2048), (200, 700)])
def test_attn_sliding_bf16(n_tok, P):
    """Sliding layer at canvas shape: cache N(0,1), window 1024."""
    cfg = synth.sliding_cfg()
    g = synth.generator(41)
    w = synth.attn_weights(cfg, g)
    cap = (P + n_tok + 7) // 8 * 8          # capacity: a multiple of 8 holding the canvas rows
    ck, cv = synth.kv_cache_random(cfg["n_kv_heads"], cap, cfg["head_dim"], g, "bf16")
    x = synth.hidden_states(n_tok, cfg["hidden"], g, "bf16")
    xo, _, _, n1 = run_gpu_attn(cfg, w, ck, cv, P, x, 0)
    assert n1 == P
    ref, _, _ = O.attn_layer(cfg, npw(w), np64(ck), np64(cv), P, np64(x), 0, "bf16")
    assert_close(np64(xo), ref, "bf16", "sliding x")
    # the residual update itself (x_out - x) to the same bar
    assert_delta_close(np64(xo), ref, np64(x), "bf16", "sliding delta")


def test_attn_global_bf16_32k():
    cfg = synth.global_cfg()
    g = synth.generator(43)
    w = synth.attn_weights(cfg, g)
    P = 32768
    ck, cv = synth.kv_cache_random(cfg["n_kv_heads"], P + 256, cfg["head_dim"], g, "bf16")
    x = synth.hidden_states(256, cfg["hidden"], g, "bf16")
    xo, _, _, _ = run_gpu_attn(cfg, w, ck, cv, P, x, 0)
    ref, _, _ = O.attn_layer(cfg, npw(w), np64(ck), np64(cv), P, np64(x), 0, "bf16")
    assert_delta_close(np64(xo), ref, np64(x), "bf16", "global delta")


def test_attn_encode_bf16_ragged():
    """Causal encode of 300 tokens after 100 committed ones (sliding, W=128)."""
    cfg = dict(synth.sliding_cfg(), window=128)
    g = synth.generator(47)
    w = synth.attn_weights(cfg, g)
    Hkv, dh = cfg["n_kv_heads"], cfg["head_dim"]
    ck, cv = synth.kv_cache_random(Hkv, 512, dh, g, "bf16")
    x = synth.hidden_states(300, cfg["hidden"], g, "bf16")
    xo, kd, vd, n1 = run_gpu_attn(cfg, w, ck, cv, 100, x, 1)
    assert n1 == 400
    ref, rk, rv = O.attn_layer(cfg, npw(w), np64(ck), np64(cv), 100, np64(x), 1, "bf16")
    assert_delta_close(np64(xo), ref, np64(x), "bf16", "encode delta")
    assert_close(np64(kd)[:, 100:400], rk, "bf16", "appended k")
    assert_close(np64(vd)[:, 100:400], rv, "bf16", "appended v")
    # rows outside [100, 400) untouched
    assert torch.equal(kd.cpu()[:, :100], ck[:, :100]) and torch.equal(kd.cpu()[:, 400:], ck[:, 400:])


@pytest.mark.parametrize("layer_type", [0, 1])
def test_attn_encode_bf16_ragged_aligned_start(layer_type):
    """Causal encode of 300 tokens after 96 committed ones: the cache
    columns start on an 8-column boundary, so the V heads go from the
    projection straight to the transposed cache (64-token tiles, the last
    one ragged, 4 tokens in its last 8-token chunk); global layers add the
    unit-RMS value norm at d_h = 512."""
    cfg = synth.sliding_cfg() if layer_type == 0 else synth.global_cfg()
    if layer_type == 0:
        cfg = dict(cfg, window=128)
    g = synth.generator(48 + layer_type)
    w = synth.attn_weights(cfg, g)
    Hkv, dh = cfg["n_kv_heads"], cfg["head_dim"]
    ck, cv = synth.kv_cache_random(Hkv, 512, dh, g, "bf16")
    x = synth.hidden_states(300, cfg["hidden"], g, "bf16")
    xo, kd, vd, n1 = run_gpu_attn(cfg, w, ck, cv, 96, x, 1)
    assert n1 == 396
    ref, rk, rv = O.attn_layer(cfg, npw(w), np64(ck), np64(cv), 96, np64(x), 1, "bf16")
    assert_delta_close(np64(xo), ref, np64(x), "bf16", "encode delta")
    assert_close(np64(kd)[:, 96:396], rk, "bf16", "appended k")
    assert_close(np64(vd)[:, 96:396], rv, "bf16", "appended v")
    # value columns outside [96, 396) untouched
    v = vd.cpu()
    assert torch.equal(v[:, :96], cv[:, :96]) and torch.equal(v[:, 396:], cv[:, 396:])


def test_attn_poisoned_out_of_window_rows_are_not_read():
    cfg = synth.sliding_cfg()
    g = synth.generator(49)
    w = synth.attn_weights(cfg, g)
    ck, cv = synth.kv_cache_random(cfg["n_kv_heads"], 2048 + 256, cfg["head_dim"], g, "bf16")
    x = synth.hidden_states(256, cfg["hidden"], g, "bf16")
    a, _, _, _ = run_gpu_attn(cfg, w, ck, cv, 2048, x, 0)
    ck2, cv2 = ck.clone(), cv.clone()
    ck2[:, :1024] = float("nan")
    cv2[:, :1024] = float("nan")
    b, _, _, _ = run_gpu_attn(cfg, w, ck2, cv2, 2048, x, 0)
    assert torch.equal(a.cpu(), b.cpu())


# ----------------------------------------------------------------- MoE


@pytest.mark.parametrize("n,inject", [(24, False), (37, True)])
def test_moe_tiny_f32(n, inject):
    cfg = synth.tiny_moe_cfg("f32")
    g = synth.generator(51)
    w = synth.moe_weights(cfg, g)
    x = synth.hidden_states(n, cfg["hidden"], g, "f32")
    rl = synth.router_logits(n, cfg["n_experts"], g) if inject else None
    xd = x.clone().cuda()
    idx, wts = B.dg_moe_block(cfg, cuda(w), xd, None if rl is None else rl.cuda(), want_topk=True)
    sync()
    ref, ridx, rw, r = O.moe_block(cfg, npw(w), np64(x), "f32", router_logits=None if rl is None else np64(rl))
    # indices bit-exact where the k-th / (k+1)-th logit gap is clear, valid inside the band
    clear = check_router_sets(idx.cpu().numpy(), ridx, r, cfg["top_k"])
    assert rel_err(wts.cpu().numpy()[clear], rw[clear]) < 1e-5
    assert_close(np64(xd), ref, "f32", "moe x")


@pytest.mark.parametrize("layer_scalar,route_scale", [(1.0, 1.0), (1.15, 1.3), (0.85, 0.7)])
def test_moe_bf16_full_injected(layer_scalar, route_scale):
    """128 experts top-8 + shared at the canvas shape, router logits N(0,1);
    the layer scalar rescales x + y and the route scale the routed weights
    (aitrends glossary "Layer Scalar", "MoE")."""
    cfg = synth.moe_cfg(2816, 128, 8, 704, 704, layer_scalar=layer_scalar, route_scale=route_scale)
    g = synth.generator(53)
    w = synth.moe_weights(cfg, g, with_router=False)
    x = synth.hidden_states(256, cfg["hidden"], g, "bf16")
    rl = synth.router_logits(256, 128, g)
    xd = x.clone().cuda()
    idx, wts = B.dg_moe_block(cfg, cuda(w), xd, rl.cuda(), want_topk=True)
    sync()
    wn = {k: (v.float().numpy() if isinstance(v, torch.Tensor) else v) for k, v in w.items()}
    ref, ridx, rw, _ = O.moe_block_grouped(cfg, wn, np64(x), "bf16", router_logits=np64(rl))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert rel_err(wts.cpu().numpy(), rw) < 1e-5
    assert_close(np64(xd), ref, "bf16", "moe x")
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "moe delta")


def test_moe_bf16_router_computed():
    """Full-size block with the router product on the device (split-K partials
    summed by the top-k pass): indices bit-exact where the oracle's 8th/9th
    logit gap exceeds 1e-3, outputs on those tokens at the bf16 bar."""
    cfg = synth.moe_cfg(2816, 128, 8, 704, 704)
    g = synth.generator(59)
    w = synth.moe_weights(cfg, g, with_router=True)
    x = synth.hidden_states(256, cfg["hidden"], g, "bf16")
    xd = x.clone().cuda()
    idx, wts = B.dg_moe_block(cfg, cuda(w), xd, None, want_topk=True)
    sync()
    ref, ridx, rw, r = O.moe_block_grouped(cfg, npw(w), np64(x), "bf16")
    # exact where the 8th/9th logit gap is clear; inside the band the sets may
    # differ only by experts within 1e-3 of the oracle's 8th logit
    clear = check_router_sets(idx.cpu().numpy(), ridx, r, 8)
    assert clear.mean() > 0.9
    assert rel_err(wts.cpu().numpy()[clear], rw[clear]) < 1e-2
    assert_delta_close(np64(xd)[clear], ref[clear], np64(x)[clear], "bf16", "moe (router computed) delta")


def test_moe_bf16_ragged_groups():
    """45 tokens over 16 experts (top-4): short groups, ragged column tiles
    (ffn 192, shared 128, hidden 320)."""
    cfg = synth.moe_cfg(320, 16, 4, 192, 128, dtype="bf16")
    g = synth.generator(57)
    w = synth.moe_weights(cfg, g)
    x = synth.hidden_states(45, 320, g, "bf16")
    rl = synth.router_logits(45, 16, g)
    xd = x.clone().cuda()
    idx, _ = B.dg_moe_block(cfg, cuda(w), xd, rl.cuda(), want_topk=True)
    sync()
    ref, ridx, _, _ = O.moe_block_grouped(cfg, npw(w), np64(x), "bf16", router_logits=np64(rl))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert_close(np64(xd), ref, "bf16", "moe x")
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "moe ragged delta")


@pytest.mark.parametrize("D,E,k,F,n", [(2752, 16, 4, 704, 45), (320, 16, 4, 320, 45), (256, 8, 2, 512, 100)])
def test_moe_bf16_down_ring_groups(D, E, k, F, n):
    """Expert down product with several (expert, column tile, row block)
    items per workgroup: skewed router logits leave experts 0-2 without rows
    and give expert 5 most tokens (several row blocks); D = 2784 ends in a
    half column tile; ffn 704 / 320 / 512 give waves 3 / 2 / 1 and 2 / 1
    stages of 64 per item."""
    cfg = synth.moe_cfg(D, E, k, F, F, dtype="bf16")
    g = synth.generator(61)
    w = synth.moe_weights(cfg, g)
    x = synth.hidden_states(n, D, g, "bf16")
    rl = synth.router_logits(n, E, g)
    rl[:, :3] -= 20.0
    rl[:, 5] += 4.0
    xd = x.clone().cuda()
    idx, _ = B.dg_moe_block(cfg, cuda(w), xd, rl.cuda(), want_topk=True)
    sync()
    ref, ridx, _, _ = O.moe_block_grouped(cfg, npw(w), np64(x), "bf16", router_logits=np64(rl))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    counts = np.bincount(ridx.ravel(), minlength=E)
    assert counts[:3].sum() == 0 and counts[5] > 32
    assert_close(np64(xd), ref, "bf16", "moe x")
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "moe down-ring delta")


@pytest.mark.parametrize("n", [1, 3])
def test_moe_bf16_few_tokens(n):
    """A handful of tokens: fewer (expert, column tile, row block) items than
    resident workgroups in the down product, so most workgroups have none."""
    cfg = synth.moe_cfg(2816, 16, 4, 704, 704, dtype="bf16")
    g = synth.generator(67 + n)
    w = synth.moe_weights(cfg, g)
    x = synth.hidden_states(n, 2816, g, "bf16")
    rl = synth.router_logits(n, 16, g)
    xd = x.clone().cuda()
    idx, _ = B.dg_moe_block(cfg, cuda(w), xd, rl.cuda(), want_topk=True)
    sync()
    ref, ridx, _, _ = O.moe_block_grouped(cfg, npw(w), np64(x), "bf16", router_logits=np64(rl))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert_close(np64(xd), ref, "bf16", "moe x")
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "moe few-token delta")


def test_moe_bf16_prefill_rows():
    """2048 tokens: ~128 rows per expert exercises the 128-row tiles."""
    cfg = synth.moe_cfg(256, 16, 8, 128, 128, dtype="bf16")
    g = synth.generator(55)
    w = synth.moe_weights(cfg, g)
    x = synth.hidden_states(2048, 256, g, "bf16")
    rl = synth.router_logits(2048, 16, g)
    xd = x.clone().cuda()
    idx, _ = B.dg_moe_block(cfg, cuda(w), xd, rl.cuda(), want_topk=True)
    sync()
    ref, ridx, _, _ = O.moe_block_grouped(cfg, npw(w), np64(x), "bf16", router_logits=np64(rl))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "moe prefill delta")


# ----------------------------------------------------------------- whole step / commit (tiny)


def tiny_model(dtype="f32"):
    mcfg = synth.tiny_model_cfg(dtype=dtype)
    w = synth.model_weights(mcfg, seed=0)
    return mcfg, w


def oracle_weights(w):
    return dict(embed=np64(w["embed"]), w_final_norm=np64(w["w_final_norm"]), sc=npw(w["sc"]),
                attn=[npw(a) for a in w["attn"]], moe=[npw(m) for m in w["moe"]],
                layer_scalar=w["layer_scalar"])


def gpu_weights(w):
    return dict(embed=w["embed"].cuda(), w_final_norm=w["w_final_norm"].cuda(), sc=cuda(w["sc"]),
                attn=[cuda(a) for a in w["attn"]], moe=[cuda(m) for m in w["moe"]],
                layer_scalar=list(w["layer_scalar"]))


def test_tiny_commit_then_two_steps():
    mcfg, w = tiny_model("f32")
    model = B.Model(mcfg, gpu_weights(w))
    wn = oracle_weights(w)
    V, C = mcfg["vocab"], 32
    kv = B.KV(mcfg, 128)
    prompt = synth.tokens(64, V, synth.generator(2))
    B.dg_commit_canvas(model, kv, prompt.cuda())
    sync()
    assert kv.kv_len == 64
    L, Hkv, dh = 2, 2, 64
    rkv = dict(k=[np.zeros((Hkv, 128, dh)) for _ in range(L)], v=[np.zeros((Hkv, 128, dh)) for _ in range(L)],
               kv_len=0)
    kn, vn = O.commit_canvas(mcfg, wn, rkv, prompt.numpy(), "f32")
    for l in range(L):
        assert_close(np64(kv.k[l])[:, :64], kn[l], "f32", f"commit k[{l}]")
        assert_close(np64(kv.v[l].transpose(1, 2))[:, :64], vn[l], "f32", f"commit v[{l}]")
        rkv["k"][l][:, :64], rkv["v"][l][:, :64] = kn[l], vn[l]
    rkv["kv_len"] = 64

    canvas = B.Canvas(C, mcfg["hidden"], "f32", keep_logits_vocab=V)
    canvas.tokens.copy_(B.dg_canvas_noise(C, V, 1, 0))
    tokens = O.canvas_noise(C, V, 1, 0)
    u = None
    for step in range(2):
        s = synth.sampler_cfg(V, t_max=2.0, t_min=0.5, n_steps=4, step=step)
        B.dg_canvas_step(model, kv, canvas, s)
        sync()
        ref = O.canvas_step(mcfg, wn, rkv, dict(tokens=tokens, u=u), s, "f32")
        assert_close(canvas.logits.cpu().numpy(), ref["logits"], "f32", f"step {step} logits")
        assert np.max(np.abs(canvas.entropy.cpu().numpy() - ref["entropy"])) < 1e-4 * math.log(V)
        noise = O.renoise_tokens(C, V, s["seed"], s["step"], s["canvas_idx"])
        dl = float(np.max(np.abs(canvas.logits.cpu().numpy() - ref["logits"])))
        check_sampler_outputs(canvas.tokens.cpu().numpy(), canvas.commit.cpu().numpy(), ref, ref["logits"], noise,
                              s["tau"], band_logit=max(2 * dl, 1e-6), band_h=1e-3)
        assert_close(np64(canvas.u), ref["u_next"], "f32", f"step {step} u")
        tokens, u = ref["tokens"], ref["u_next"]   # each side continues from its own state
