"""The achievable-peak probes: the copy copies, the MFMA loop computes the
closed form of its accumulators."""

import numpy as np
import pytest
import torch

from uniform_noise_diffusion_amd import probe

from gpu_common import DEV

pytestmark = pytest.mark.gpu


def test_copy_is_exact_including_a_ragged_block():
    n = (1 << 20) + 3 * 16   # not a multiple of the 256-element block
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros_like(src)
    probe.copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_mfma_loop_matches_its_closed_form():
    # every accumulator of every chain is incremented by the same 32x32x16
    # product each iteration; the wave's written value is the sum over the 8
    # chains of all 32x32 entries of iters * (A B)
    blocks, iters = 4, 3
    out = torch.zeros(blocks * 8, dtype=torch.float32, device=DEV)
    flops = probe.mfma(out, blocks, iters)
    torch.cuda.synchronize()
    assert flops == blocks * 8 * iters * 8 * 32768
    lane = np.arange(64)
    e = np.arange(8)
    bf = lambda x: torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).float().numpy()
    a = bf(0.001 * (lane[:, None] + e[None, :]))        # lane l, element e
    b = bf(0.002 * (lane[:, None] - e[None, :]))
    # A row i (lanes i and i + 32 hold k 0..7 and 8..15), B column j likewise
    A = np.concatenate([a[:32], a[32:]], axis=1)          # [32 rows, 16 k]
    B = np.concatenate([b[:32], b[32:]], axis=1).T        # [16 k, 32 cols]
    want = 8 * iters * (A.astype(np.float64) @ B.astype(np.float64)).sum()
    got = out.cpu().numpy()
    assert np.allclose(got, want, rtol=1e-4)
