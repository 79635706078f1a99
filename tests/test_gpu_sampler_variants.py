"""Sampler variants on the GPU against the oracle: Gumbel-max proposals, the
sorted cumulative entropy bound, the proposal-stability count, and both
rules inside a whole (tiny) denoising step.

Integer results are compared bit for bit where floating point does not
decide them within a stated band: Gumbel proposals where the oracle's
best-minus-second score margin exceeds 1e-4 (fp32 logits/t + g against
float64), sorted-cumulative commits where the oracle's prior entropy sum is
more than 2e-3 nats from the bound.  Re-noise tokens are integer-only and
always bit-exact given the commit decision.
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


def logits_case(n, V, seed, dtype):
    lg = synth.sampler_logits(n, V, synth.generator(seed), n_flat=3, n_peaked=3)
    return lg.to(torch.bfloat16) if dtype == "bf16" else lg


def gumbel_scores(lg64, rows, scfg):
    """The oracle's proposal scores l/t + g for `rows`, 32 rows at a time."""
    t = O.temperature(scfg["t_max"], scfg["t_min"], scfg["step"], scfg["n_steps"])
    out = np.empty((len(rows), scfg["vocab"]))
    for r0 in range(0, len(rows), 32):
        rr = rows[r0:r0 + 32]
        out[r0:r0 + 32] = lg64[rr] / t + O.gumbel_noise(rr, scfg["vocab"], scfg["seed"], scfg["step"],
                                                        scfg["canvas_idx"])
    return out


def gumbel_ref(lg64, rows, scfg):
    sc = gumbel_scores(lg64, rows, scfg)
    top2 = -np.partition(-sc, 1, axis=1)[:, :2]
    return np.argmax(sc, axis=1), top2[:, 0] - top2[:, 1], sc


@pytest.mark.parametrize("n,V,dtype,temp", [(45, 8000, "f32", 1.0), (33, 4096, "bf16", 0.7),
                                             (256, 262144, "f32", 1.0)])
def test_gumbel_proposals(n, V, dtype, temp):
    lg = logits_case(n, V, 11 + n, dtype)
    s = dict(synth.sampler_cfg(V, t_max=temp, t_min=temp, step=5, canvas_idx=3), token_rule="gumbel")
    pred = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    out = B.dg_sample_renoise(s, lg.cuda(), pred=pred)
    sync()
    lg64 = np64(lg)
    rows = np.arange(n)                 # every row, also at V = 262,144
    ref_pred, margin, sc = gumbel_ref(lg64, rows, s)
    got = pred.cpu().numpy()[rows]
    clear = margin > 1e-4
    assert clear.mean() > 0.9
    np.testing.assert_array_equal(got[clear], ref_pred[clear])
    # where the margin is inside the band the GPU draw must be one of the near-best
    t = O.temperature(s["t_max"], s["t_min"], s["step"], s["n_steps"])
    for r in np.nonzero(~clear)[0]:
        assert sc[r].max() - sc[r, got[r]] <= 1e-4
    # commit rule unchanged (H < tau); committed positions take the draw,
    # the others the Philox re-noise token
    H = O.row_stats(lg64, t)[3]
    commit = out["commit"].cpu().numpy().astype(bool)
    band = np.abs(H - s["tau"]) > 1e-3
    np.testing.assert_array_equal(commit[band], (H < s["tau"])[band])
    tok = out["tokens"].cpu().numpy()
    noise = O.renoise_tokens(n, V, s["seed"], s["step"], s["canvas_idx"])
    np.testing.assert_array_equal(tok[~commit], noise[~commit])
    np.testing.assert_array_equal(tok[commit], pred.cpu().numpy()[commit])
    assert int(out["n_changed"].item()) == n          # previous proposals were -1
    # the draws differ from the argmax on flat / warm rows, as sampling should
    assert (pred.cpu().numpy() != np.argmax(lg64, axis=1)).sum() > 0


@pytest.mark.parametrize("n,V,dtype,bound", [(256, 4096, "f32", 40.0), (77, 262144, "bf16", 25.0),
                                              (300, 4096, "f32", 0.0)])
def test_sorted_cumulative_commit(n, V, dtype, bound):
    lg = logits_case(n, V, 21 + n, dtype)
    s = dict(synth.sampler_cfg(V, tau=bound, step=2, canvas_idx=1), commit_rule="sorted_cumulative")
    out = B.dg_sample_renoise(s, lg.cuda())
    sync()
    ref = O.sample_renoise(np64(lg), s)
    commit = out["commit"].cpu().numpy().astype(bool)
    clear = np.abs(ref["prior_sum"] - bound) > 2e-3
    assert clear.mean() > 0.9
    np.testing.assert_array_equal(commit[clear], ref["commit"][clear])
    tok = out["tokens"].cpu().numpy()
    np.testing.assert_array_equal(tok[clear], ref["tokens"][clear])
    assert int(out["n_renoised"].item()) == int((~commit).sum())
    # the GPU's own commit set is a prefix of its own entropy order, never empty
    Hg = out["entropy"].cpu().numpy()
    order = sorted(range(n), key=lambda j: (Hg[j], j))
    flags = commit[order]
    k = int(flags.sum())
    assert k >= 1 and flags[:k].all() and not flags[k:].any()


def test_sorted_cumulative_final_step_and_ties():
    V = 4096
    lg = torch.zeros(8, V)           # eight flat rows: equal entropies, ties by position
    s = dict(synth.sampler_cfg(V, tau=2 * math.log(V) + 1e-2), commit_rule="sorted_cumulative")
    out = B.dg_sample_renoise(s, lg.cuda())
    sync()
    # prior sums 0, ln V, 2 ln V, ...: positions 0..2 commit
    assert list(out["commit"].cpu().numpy()) == [1, 1, 1, 0, 0, 0, 0, 0]
    fin = B.dg_sample_renoise(dict(s, final_step=True), lg.cuda())
    sync()
    assert fin["commit"].cpu().numpy().all() and int(fin["n_renoised"].item()) == 0


def test_stability_count():
    n, V = 64, 4096
    lg = logits_case(n, V, 31, "f32")
    s = synth.sampler_cfg(V)
    pred = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    a = B.dg_sample_renoise(s, lg.cuda(), pred=pred)
    sync()
    assert int(a["n_changed"].item()) == n
    np.testing.assert_array_equal(pred.cpu().numpy(), np.argmax(np64(lg), axis=1))
    b = B.dg_sample_renoise(dict(s, step=1), lg.cuda(), pred=pred)
    sync()
    assert int(b["n_changed"].item()) == 0
    lg2 = lg.clone()
    hit = [5, 9, 40]
    for j in hit:
        lg2[j, (int(np.argmax(np64(lg)[j])) + 17) % V] = 1e3
    prev = pred.cpu().numpy().copy()
    c = B.dg_sample_renoise(dict(s, step=2), lg2.cuda(), pred=pred)
    sync()
    ref = O.sample_renoise(np64(lg2), dict(s, step=2), pred_prev=prev)
    assert int(c["n_changed"].item()) == ref["n_changed"] == len(hit)


@pytest.mark.parametrize("rules", [("sorted_cumulative", "gumbel"), ("entropy", "gumbel")])
def test_tiny_step_with_variants(rules):
    """Two tiny fp32 denoising steps through dg_canvas_step with the variant
    rules, against the oracle's whole step."""
    from tests.test_gpu_parity import gpu_weights, oracle_weights, tiny_model
    mcfg, w = tiny_model("f32")
    model = B.Model(mcfg, gpu_weights(w))
    wn = oracle_weights(w)
    V, C, L, Hkv, dh = mcfg["vocab"], 32, 2, 2, 64
    kv = B.KV(mcfg, 128)
    prompt = synth.tokens(64, V, synth.generator(2))
    B.dg_commit_canvas(model, kv, prompt.cuda())
    sync()
    rkv = dict(k=[np.zeros((Hkv, 128, dh)) for _ in range(L)], v=[np.zeros((Hkv, 128, dh)) for _ in range(L)],
               kv_len=0)
    kn, vn = O.commit_canvas(mcfg, wn, rkv, prompt.numpy(), "f32")
    for l in range(L):
        rkv["k"][l][:, :64], rkv["v"][l][:, :64] = kn[l], vn[l]
    rkv["kv_len"] = 64
    canvas = B.Canvas(C, mcfg["hidden"], "f32", keep_logits_vocab=V)
    canvas.tokens.copy_(B.dg_canvas_noise(C, V, 1, 0))
    tokens = O.canvas_noise(C, V, 1, 0)
    u = None
    prev = None
    for step in range(2):
        s = dict(synth.sampler_cfg(V, tau=30.0 if rules[0] == "sorted_cumulative" else None, t_max=2.0,
                                   t_min=0.5, n_steps=4, step=step), commit_rule=rules[0], token_rule=rules[1])
        B.dg_canvas_step(model, kv, canvas, s)
        sync()
        ref = O.canvas_step(mcfg, wn, rkv, dict(tokens=tokens, u=u), s, "f32")
        assert_close(canvas.logits.cpu().numpy(), ref["logits"], "f32", f"step {step} logits")
        # proposals and commits compared where no float decision is close
        gm = ref["gumbel_margin"]
        clear = gm > 1e-4
        if rules[0] == "sorted_cumulative":
            clear &= np.abs(ref["prior_sum"] - s["tau"]) > 2e-3
        else:
            clear &= np.abs(ref["entropy"] - s["tau"]) > 1e-3
        assert clear.mean() > 0.8
        np.testing.assert_array_equal(canvas.pred.cpu().numpy()[clear], ref["pred"][clear])
        np.testing.assert_array_equal(canvas.commit.cpu().numpy().astype(bool)[clear], ref["commit"][clear])
        np.testing.assert_array_equal(canvas.tokens.cpu().numpy()[clear], ref["tokens"][clear])
        if prev is not None:
            assert int(canvas.n_changed.item()) == int((canvas.pred.cpu().numpy() != prev).sum())
        prev = canvas.pred.cpu().numpy().copy()
        tokens, u = ref["tokens"], ref["u_next"]
