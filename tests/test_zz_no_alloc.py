"""Allocation-free routing: basa_route_windows_noalloc (the library's own
per-GPU scratch) against basa_route_windows with a caller workspace, through
the C ABI.  Route tables must be identical (bit-exact index work), on calls in
a row where the later ones are smaller, so a later call cannot lean on what an
earlier one left in the shared scratch."""
import numpy as np
import pytest

from tests.gpu_util import basa_plan, say
from video_gen_amd.synth import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from video_gen_amd import basa

    basa.load()
    return torch, basa


def _both(torch, basa, plan, q, k):
    blk = basa.Block(plan)                       # route table + workspace of the plain call
    basa.basa_route_windows(plan, q, k, blk.route, blk.workspace)
    plain = blk.route.clone()
    na = torch.full_like(blk.route, -7)
    basa.basa_route_windows_noalloc(plan, q, k, na)
    torch.cuda.synchronize()
    return plain.cpu().numpy(), na.cpu().numpy()


def test_route_noalloc_matches_workspace_entry_point(env):
    torch, basa = env
    small = Workload("small3d", 1, 2, 64, (3, 12, 20), (2, 5, 6), (1, 2, 3), (1, 4, 4), 3, "bf16",
                     71, True, "small routed grid with short windows")
    cases = [(WORKLOADS["wan"], None), (WORKLOADS["wan"], 3), (small, None)]
    for w, heads in cases:
        say(f"[noalloc] {w.name} heads={heads or w.heads}")
        inp = make_inputs(w, heads=heads)
        plan = basa_plan(basa, w, w.shift, heads=heads)
        assert plan.info["route_workspace_bytes"] <= 64 << 20
        plain, na = _both(torch, basa, plan, inp.torch("q"), inp.torch("k"))
        assert (na >= 0).all()
        np.testing.assert_array_equal(na, plain)
