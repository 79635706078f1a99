"""The roof probes return exactly what they read and compute, so the rates
bench.py derives from them measure work that was done."""
import numpy as np
import pytest
import torch

from discrete_text_diffusion_step_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("n_bytes,n_groups", [(64 << 20, 2048), ((8 << 20) + 48, 300), (16, 1)])
def test_hbm_read_probe_sums_every_word(n_bytes, n_groups):
    """Random 32-bit words; the workgroup sums add up (mod 2^32) to the sum of
    every word, including a tail shorter than one unrolled round."""
    g = torch.Generator().manual_seed(5)
    words = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_bytes // 4,), generator=g, dtype=torch.int64).to(torch.int32)
    sink = B.dg_probe_hbm_read(words.cuda(), n_groups=n_groups)
    torch.cuda.synchronize()
    got = int(sink.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % 2 ** 32
    want = int(words.numpy().view(np.uint32).astype(np.uint64).sum()) % 2 ** 32
    assert got == want


@pytest.mark.parametrize("iters,a,b", [(64, 1.0, 2.0 ** -10), (16, 0.5, 0.25), (0, 1.0, 1.0)])
def test_mfma_probe_exact(iters, a, b):
    n_groups = 40
    sink = B.dg_probe_mfma_bf16(iters, a, b, n_groups=n_groups)
    torch.cuda.synchronize()
    want = 16.0 * iters * 32 * a * b
    assert torch.equal(sink.cpu(), torch.full((4 * n_groups,), want))
    assert B.dg_probe_mfma_flops(iters, n_groups) == n_groups * 4 * iters * 16 * 2 * 16 * 16 * 32
