"""The library's launch timer (dg_set_kernel_timer): with `every` = n it
records HIP events around launches 0, n, 2n, ... of its kernel class and
counts every launch it sees; the bench's live roofline figure relies on it."""
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from tests.helpers import cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("every,expect", [(1, 7), (3, 3), (31, 1)])
def test_timer_samples_every_nth_launch(every, expect):
    cfg = synth.moe_cfg(320, 16, 4, 192, 128, dtype="bf16")
    g = synth.generator(81)
    w = cuda(synth.moe_weights(cfg, g))
    x = synth.hidden_states(45, 320, g, "bf16").cuda()
    rl = synth.router_logits(45, 16, g).cuda()
    B.dg_moe_block(cfg, w, x.clone(), rl)
    torch.cuda.synchronize()
    t = B.kernel_timer("moe_gateup", capacity=16, every=every)
    with t:
        for _ in range(7):
            B.dg_moe_block(cfg, w, x.clone(), rl)
    d = t.durations_ms()
    assert t.t.seen == 7
    assert t.t.count == expect and len(d) == expect
    assert all(v > 0.0 for v in d)
    # detached: further launches are not recorded
    B.dg_moe_block(cfg, w, x.clone(), rl)
    torch.cuda.synchronize()
    assert t.t.seen == 7 and t.t.count == expect
