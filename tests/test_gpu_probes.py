"""GPU test of the LDS-ring load probe (proj_ring_probe), a measurement aid:
every compiled combination runs, and each wave reports the number of stages
it issued, (stages - 1) + chunks."""
import pytest
import torch

import tp1_skinny_bf16_amd as tp
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

# (rows, piece, depth, barrier, what) for every compiled instance
CASES = [(64, 256, 5, 1, 1), (64, 256, 5, 0, 2), (128, 256, 3, 1, 3), (64, 512, 3, 1, 1),
         (64, 512, 3, 0, 1), (64, 1024, 2, 1, 2), (64, 1024, 2, 0, 1), (64, 256, 9, 1, 1),
         (128, 256, 5, 1, 3), (64, 128, 9, 1, 2), (128, 128, 9, 1, 3)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(DEV)


@pytest.mark.parametrize("shared", [0, 1])
def test_ring_probe_runs_every_instance(shared):
    K, grid = 2048, 6
    x = torch.randn((64, K), device=DEV).to(torch.bfloat16)
    w = torch.randn(((1 if shared else grid) * 64, K), device=DEV).to(torch.bfloat16)
    for rows, piece, depth, barrier, what in CASES:
        sink = torch.full((grid * 8,), -1.0, dtype=torch.float32, device=DEV)
        tp.ring_probe(x, w, rows=rows, piece=piece, depth=depth, barrier=bool(barrier),
                      what=what, shared_w=bool(shared), grid=grid, sink=sink)
        torch.cuda.synchronize()
        want = (depth - 1) + K * 2 // piece
        say(f"ring probe rows={rows} piece={piece} depth={depth} barrier={barrier} "
            f"what={what} shared={shared}: stages {sink[0].item():.0f} (want {want})")
        assert bool((sink == want).all()), sink
