"""dg_sample_renoise_noalloc (no workspace argument, built-in per-GPU scratch)
against dg_sample_renoise through the C ABI: the same kernels, so every
output must be bit-identical.  Two calls in a row, the second smaller, so
the second reads nothing the first left in the scratch."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth

pytestmark = pytest.mark.gpu


def _same(a, b):
    for k in ("tokens", "commit", "entropy", "rowstats", "n_renoised", "n_changed", "n_nonfinite"):
        if a[k] is None:
            assert b[k] is None
            continue
        x, y = a[k].cpu(), b[k].cpu()
        if x.dtype == torch.float32:     # bit patterns: the planted NaN row compares equal to itself
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), k


def test_noalloc_sampler_matches_workspace_entry_point(gpu_lib):
    cases = [(256, 262144, "f32", 5), (45, 4096, "bf16", 6)]
    for n, V, dtype, seed in cases:
        print(f"[no-alloc] n={n} V={V} {dtype}", flush=True)
        lg = synth.sampler_logits(n, V, synth.generator(seed))
        lg[3, 17] = float("nan")
        lg = (lg.to(torch.bfloat16) if dtype == "bf16" else lg).cuda()
        s = dict(synth.sampler_cfg(V, t_max=0.9, t_min=0.9, step=2, canvas_idx=1), token_rule="gumbel")
        pa = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        pb = pa.clone()
        a = B.dg_sample_renoise(s, lg, pred=pa)
        b = B.dg_sample_renoise_noalloc(s, lg, pred=pb)
        torch.cuda.synchronize()
        _same(a, b)
        assert torch.equal(pa.cpu(), pb.cpu())
        assert int(b["n_nonfinite"].item()) == 1
        # the entropy rule too, without the optional outputs
        s2 = synth.sampler_cfg(V, step=3)
        a = B.dg_sample_renoise(s2, lg, want_rowstats=False)
        b = B.dg_sample_renoise_noalloc(s2, lg, want_rowstats=False)
        torch.cuda.synchronize()
        _same(a, b)
        assert 0 <= int(b["n_renoised"].item()) <= n
        assert np.isfinite(b["entropy"].cpu().numpy()[[0, 1, 2]]).all()
