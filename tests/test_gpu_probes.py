"""The measurement probes (vae_probe_mfma_f32, vae_probe_hbm) compute what
their declarations state: the MFMA probe's per-wave output sums match the
closed form of its register operands, the read probe's sums add up to the
buffer's sum, the copy is exact."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    from diffusion_vae_decoder_amd import api as a
    return a


def test_mfma_probe_closed_form(api):
    blocks, iters = 8, 32
    out, flops = api.probe_mfma_f32(blocks, iters)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * iters * 8 * 2 * 32 * 32 * 2
    a = 1.0 + np.arange(64) / 64.0
    b = 1.0 - np.arange(64) / 128.0
    # every round adds sum_k a(m + 32k) b(n + 32k) to C[m][n]; over the
    # wave's 32 x 32 outputs and 8 chains
    per_wave = 8 * iters * sum(a[32 * k:32 * k + 32].sum() * b[32 * k:32 * k + 32].sum() for k in range(2))
    got = out.cpu().double().numpy().reshape(blocks * 4, 64).sum(axis=1)
    np.testing.assert_allclose(got, per_wave, rtol=1e-5)


def test_hbm_read_probe_sums_the_buffer(api):
    n = (1 << 20) + 4 * 37   # not a multiple of the grid's stride
    g = torch.Generator().manual_seed(3)
    x = torch.randint(-8, 9, (n,), generator=g).float()
    part = api.probe_hbm(x.cuda(), blocks=64)
    torch.cuda.synchronize()
    # small integers: every partial sum is exact in float32
    assert part.numel() == 64 * 256
    assert float(part.double().sum()) == float(x.double().sum())


def test_hbm_copy_probe_is_exact(api):
    n = (1 << 20) + 4 * 37
    x = torch.randn(n, generator=torch.Generator().manual_seed(4)).cuda()
    y = torch.full_like(x, math.nan)
    api.probe_hbm(x, y, blocks=64)
    torch.cuda.synchronize()
    assert torch.equal(x, y)
