"""FP8 (OCP E4M3) expert weights: the HIP quantiser and the fp8 expert
products against the oracle (oracle/fp8.py quantises the same bf16 weights on
its own; its dequantised experts go through the oracle's MoE block).

Codes and scales are integer / exactly-defined fp32 results: bit-exact.
MoE outputs: the bf16 bar (2e-2), router indices bit-exact.
"""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B
from discrete_text_diffusion_step_amd import synth
from oracle import dg_oracle as O
from oracle import fp8 as F8
from tests.helpers import assert_close, assert_delta_close, cuda, np64, npw

pytestmark = pytest.mark.gpu

TD = {"f32": torch.float32, "bf16": torch.bfloat16}
SCALE_NAME = {"w_gate": "s_gate", "w_up": "s_up", "w_down": "s_down",
              "ws_gate": "ss_gate", "ws_up": "ss_up", "ws_down": "ss_down"}


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    torch.manual_seed(0)
    yield


def edge_rows(rows, cols, dtype, seed):
    """N(0, 0.02) rows plus edge rows: all zero, one tiny value, a row spanning
    16 binades (subnormal codes), a row of exact powers of two."""
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(rows, cols, generator=g) * 0.02
    w[0] = 0.0
    w[1] = 0.0
    w[1, cols // 3] = -3.0e-5
    w[2] = w[2].sign() * torch.logspace(-16, 0, cols, base=2.0)
    w[3] = torch.exp2(torch.randint(-20, 3, (cols,), generator=g).float())
    return w.to(TD[dtype])


@pytest.mark.parametrize("dtype,rows,cols", [("bf16", 300, 2816), ("bf16", 130, 704), ("f32", 33, 320)])
def test_quantize_fp8_bitexact(dtype, rows, cols):
    w = edge_rows(rows, cols, dtype, 61 + rows)
    q, s = B.dg_quantize_fp8(w.cuda())
    torch.cuda.synchronize()
    rq, rs = F8.quantize_rows(np64(w))
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def _run_gpu(cfg, w, x, rl):
    wq = B.quantize_moe_weights(cuda(w))
    xd = x.clone().cuda()
    idx, wts = B.dg_moe_block(dict(cfg, expert_format="fp8_e4m3"), wq, xd, rl.cuda(), want_topk=True)
    torch.cuda.synchronize()
    return wq, xd, idx


def _check_codes(wq, codes, scales, experts=None):
    for n, sn in SCALE_NAME.items():
        got_q, got_s = wq[n].cpu().numpy(), wq[sn].cpu().numpy()
        if n.startswith("w_") and experts is not None:
            for e in experts:
                np.testing.assert_array_equal(got_q[e], codes[n][e])
                np.testing.assert_array_equal(got_s[e], scales[n][e])
        else:
            np.testing.assert_array_equal(got_q, codes[n])
            np.testing.assert_array_equal(got_s, scales[n])


@pytest.mark.parametrize("D,E,k,F,Fs,n,seed", [
    (320, 16, 4, 192, 128, 45, 71),     # ragged: depths 320 and 192 end on a 64-deep half stage
    (256, 16, 8, 128, 128, 2048, 73),   # ~1024 rows per expert: the 64-row tiles
])
def test_moe_fp8_small(D, E, k, F, Fs, n, seed):
    cfg = synth.moe_cfg(D, E, k, F, Fs, dtype="bf16")
    g = synth.generator(seed)
    w = synth.moe_weights(cfg, g, with_router=False)
    x = synth.hidden_states(n, D, g, "bf16")
    rl = synth.router_logits(n, E, g)
    wq, xd, idx = _run_gpu(cfg, w, x, rl)
    codes, scales, deq = F8.quantize_experts(npw(w))
    _check_codes(wq, codes, scales)
    wn = npw(w)
    wn.update(deq)
    ref, ridx, _, _ = O.moe_block_grouped(cfg, wn, np64(x), "bf16", router_logits=np64(rl))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert_close(np64(xd), ref, "bf16", "fp8 moe x")
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "fp8 moe delta")


@pytest.mark.parametrize("D,E,k,F,n", [(2752, 16, 4, 704, 45), (320, 16, 4, 576, 45), (256, 8, 2, 640, 100)])
def test_moe_fp8_down_ring_groups(D, E, k, F, n):
    """fp8 down product with several (expert, column tile, row block) items per
    workgroup: skewed router logits leave experts 0-2 without rows and give
    expert 5 most tokens (several row blocks); ffn 704 and 576 end on a
    64-deep half stage (held by wave 1 and by wave 0), 640 on whole stages;
    the waves own 2/2/1/1, 2/1/1/1 and 2/1/1/1 stages of 128 per item."""
    cfg = synth.moe_cfg(D, E, k, F, F, dtype="bf16")
    g = synth.generator(63)
    w = synth.moe_weights(cfg, g, with_router=False)
    x = synth.hidden_states(n, D, g, "bf16")
    rl = synth.router_logits(n, E, g)
    rl[:, :3] -= 20.0
    rl[:, 5] += 4.0
    wq, xd, idx = _run_gpu(cfg, w, x, rl)
    codes, scales, deq = F8.quantize_experts(npw(w))
    wn = npw(w)
    wn.update(deq)
    ref, ridx, _, _ = O.moe_block_grouped(cfg, wn, np64(x), "bf16", router_logits=np64(rl))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    counts = np.bincount(ridx.ravel(), minlength=E)
    assert counts[:3].sum() == 0 and counts[5] > 32
    assert_close(np64(xd), ref, "bf16", "fp8 moe x")
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "fp8 moe down-ring delta")


def test_moe_fp8_single_token():
    """One token: fewer down-product items than resident workgroups."""
    cfg = synth.moe_cfg(2816, 16, 4, 704, 704, dtype="bf16")
    g = synth.generator(69)
    w = synth.moe_weights(cfg, g, with_router=False)
    x = synth.hidden_states(1, 2816, g, "bf16")
    rl = synth.router_logits(1, 16, g)
    wq, xd, idx = _run_gpu(cfg, w, x, rl)
    codes, scales, deq = F8.quantize_experts(npw(w))
    wn = npw(w)
    wn.update(deq)
    ref, ridx, _, _ = O.moe_block_grouped(cfg, wn, np64(x), "bf16", router_logits=np64(rl))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert_close(np64(xd), ref, "bf16", "fp8 moe x")
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "fp8 moe single-token delta")


def _quantize_stack(stack, ex):
    """The oracle's codes, scales and dequantised values of an expert stack
    [E, N, K] (bf16 tensor), one expert per task."""
    res = list(ex.map(lambda e: F8.quantize_rows(np64(stack[e])), range(stack.shape[0])))
    q = np.stack([r[0] for r in res])
    sc = np.stack([r[1] for r in res])
    deq = np.stack(list(ex.map(lambda e: F8.dequantize_rows(q[e], sc[e]), range(stack.shape[0]))))
    return q, sc, deq


def test_moe_fp8_full_all_tokens():
    """128 experts top-8 + shared at the canvas shape (256 tokens): codes and
    scales of every expert bit-exact, and every token's output against the
    oracle's MoE on the oracle's own dequantised weights."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = synth.moe_cfg(2816, 128, 8, 704, 704)
    g = synth.generator(53)
    w = synth.moe_weights(cfg, g, with_router=False)
    x = synth.hidden_states(256, cfg["hidden"], g, "bf16")
    rl = synth.router_logits(256, 128, g)
    wq, xd, idx = _run_gpu(cfg, w, x, rl)
    wn = {"w_in_norm": np64(w["w_in_norm"])}
    with ThreadPoolExecutor(16) as ex:
        for n in ("w_gate", "w_up", "w_down"):
            q, sc, wn[n] = _quantize_stack(w[n], ex)
            np.testing.assert_array_equal(wq[n].cpu().numpy(), q)
            np.testing.assert_array_equal(wq[SCALE_NAME[n]].cpu().numpy(), sc)
    for n in ("ws_gate", "ws_up", "ws_down"):
        q, sc = F8.quantize_rows(np64(w[n]))
        np.testing.assert_array_equal(wq[n].cpu().numpy(), q)
        np.testing.assert_array_equal(wq[SCALE_NAME[n]].cpu().numpy(), sc)
        wn[n] = F8.dequantize_rows(q, sc)
    ref, ridx, _, _ = O.moe_block_grouped(cfg, wn, np64(x), "bf16", router_logits=np64(rl))
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    assert_close(np64(xd), ref, "bf16", "fp8 moe x (all tokens)")
    assert_delta_close(np64(xd), ref, np64(x), "bf16", "fp8 moe delta (all tokens)")
