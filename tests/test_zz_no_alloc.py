"""GPU test of proj_run_noalloc, the entry point that allocates nothing.

It must give the same bits as proj_run with a plan for the batches 1, 2, 4,
..., 256 (both take the tactic of the smallest power of two >= B), on calls
that use the static split-K scratch, one after another with the second
smaller, and every output must pass the parity gates against the oracle.  A
call whose tactic needs more scratch than the static buffer is refused
before any launch.
"""
import numpy as np
import pytest
import torch

import tp1_skinny_bf16_amd as tp
import workloads as wl
from gpu_util import DEV, check_random, gpu_run, say, tactic_label

pytestmark = pytest.mark.gpu

POW2 = [1, 2, 4, 8, 16, 32, 64, 128, 256]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(DEV)


def _noalloc(x_cpu, Wd):
    B, K = x_cpu.shape
    N = Wd.shape[0]
    xd = x_cpu.contiguous().to(DEV)
    y = torch.empty((B, N), dtype=torch.bfloat16, device=DEV)
    tp.run_noalloc(xd, Wd, y)
    torch.cuda.synchronize()
    return wl.bits(y.cpu())


@pytest.mark.parametrize("cases", [
    # (N, K, B): a large split-K call, then smaller ones
    [(wl.DSA_N, wl.DSA_K, 256), (wl.OPROJ_N, wl.OPROJ_K, 64), (wl.DSA_N, wl.DSA_K, 5)],
    [(wl.OPROJ_N, wl.OPROJ_K, 128), (1000, 1032, 40)],
])
def test_noalloc_matches_proj_run(cases):
    for i, (N, K, B) in enumerate(cases):
        x, W = wl.random_case(B, N, K, seed=100 + i)
        Wd = W.to(DEV)
        plan = tp.Plan(N, K, POW2)
        t, _ = plan.tactic(B)
        want = gpu_run(plan, x, Wd)
        got = _noalloc(x, Wd)
        say(f"noalloc N={N} K={K} B={B} {tactic_label(plan, B)}: "
            f"{int(np.count_nonzero(got != want))} differ from proj_run")
        assert np.array_equal(got, want), (N, K, B)
        check_random(f"noalloc N={N} K={K} B={B}", got, x, W)
        plan.close()


def test_noalloc_refuses_more_scratch_than_it_has():
    # an unmeasured shape whose default tactic at B = 256 splits K in two:
    # 2 x 256 x 16896 FP32 partials = 33 MiB, above the 32 MiB buffer
    N, K, B = 16896, 8192, 256
    plan = tp.Plan(N, K, POW2, host_only=True)
    t, _ = plan.tactic(B)
    assert t.split * 256 * N * 4 > 32 << 20, t
    W = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    x = torch.empty((B, K), dtype=torch.bfloat16, device=DEV)
    y = torch.full((B, N), 3.0, dtype=torch.bfloat16, device=DEV)
    rc = tp.run_noalloc_ptr(N, K, B, x.data_ptr(), K, W.data_ptr(), y.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    assert rc == tp.PROJ_ESCRATCH, rc
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())        # nothing was launched
