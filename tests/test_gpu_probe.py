"""The matrix-core probe (a measurement hook of libbasa) through the C ABI.
Its result has a closed form in both modes: with constant operands every
product step adds 16 * 2^-12 = 2^-8 to each accumulator element, so each sink
element is 4 * iters * 2^-8 exactly; with switching operands every pair of
steps adds a product and its exact negation, so the sink is 0 exactly.  The
clock readings must be ordered and give a plausible clock."""
import numpy as np
import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from video_gen_amd import basa

    basa.load()
    return torch, basa


@pytest.mark.parametrize("iters,mode,n_wg", [(1, 0, 3), (1001, 0, 8), (5000, 0, 512),
                                             (2, 1, 3), (1000, 1, 8), (5000, 1, 512)])
def test_probe_mfma_closed_form_and_clocks(env, iters, mode, n_wg):
    torch, basa = env
    say(f"[probe] iters={iters} mode={mode} workgroups={n_wg}")
    sink = torch.full((n_wg * 256,), -1.0, dtype=torch.float32, device="cuda")
    clocks = torch.zeros((n_wg, 4), dtype=torch.int64, device="cuda")
    flops = basa.basa_probe_mfma(iters, n_wg, sink, clocks, mode=mode)
    torch.cuda.synchronize()
    assert flops == 2 * 32 * 32 * 16 * 4 * 4 * iters * n_wg
    got = sink.cpu().numpy()
    want = np.float32(4 * iters / 256.0) if mode == 0 else np.float32(0.0)
    assert (got == want).all(), np.unique(got)[:8]
    c = clocks.cpu().numpy()
    assert (c[:, 1] > c[:, 0]).all() and (c[:, 3] >= c[:, 2]).all()
    if iters >= 5000:
        ghz = (c[:, 1] - c[:, 0]) / ((c[:, 3] - c[:, 2]) / 100e6) / 1e9
        say(f"  clock under load: median {np.median(ghz):.3f} GHz")
        assert 0.5 < np.median(ghz) < 3.0
