"""Weight prefetch beside a stand-in for the attention core.

The runtime page ("vllm.models.kimi_k3.nvidia.specialized_decode.runtime")
lists an L2 weight prefetch among its modules, and the hybrid page's
"NoPrefetch" gives its fork/join interface: a prefetcher forked before the
attention core and joined after it.  proj_run_layers_overlap puts a
fixed-duration, memory-free stand-in for the core between each layer's
input projection and o_proj, and prefetches the head of the o_proj weight
while it runs: on a second stream, or inside the stand-in's own launch.
None of it may change a single output bit.
"""
import numpy as np
import pytest
import torch

import tp1_skinny_bf16_amd as tp
import workloads as wl
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(DEV)


def _weights(n, N, K, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return [(torch.randn((N, K), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
            for _ in range(n)]


@pytest.mark.parametrize("B", [8, 64])
def test_overlap_outputs_equal_the_plain_chain(B):
    L = 3
    w_in = _weights(L, wl.DSA_N, wl.DSA_K, 11)
    w_o = _weights(L, wl.OPROJ_N, wl.OPROJ_K, 12)
    x0 = torch.randn((B, wl.DSA_K), device=DEV).to(torch.bfloat16)
    stack = tp.LayerStack(tp.Plan(wl.DSA_N, wl.DSA_K, [B]), tp.Plan(wl.OPROJ_N, wl.OPROJ_K, [B]),
                          w_in, w_o)
    ref_in, ref_o = stack.run(x0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()              # default priority, like the main stream
    wo_bytes = wl.OPROJ_N * wl.OPROJ_K * 2
    cases = [(0.0, 0, False), (5.0, 0, False), (5.0, 64 << 20, False), (2.0, wo_bytes, False),
             (0.0, 1 << 20, False), (5.0, 64 << 20, True), (0.0, wo_bytes, True),
             (3.0, 1000, True)]
    for core_us, pf, in_core in cases:
        y_in, y_o = stack.buffers(B)
        y_in.fill_(7.0)
        y_o.fill_(7.0)
        stack.run_overlap(x0, y_in, y_o, core_us=core_us, prefetch_bytes=pf,
                          side_stream=side if pf and not in_core else None,
                          prefetch_in_core=in_core)
        torch.cuda.synchronize()
        same = torch.equal(y_in.view(torch.int16), ref_in.view(torch.int16)) and \
            torch.equal(y_o.view(torch.int16), ref_o.view(torch.int16))
        say(f"B={B} core {core_us} us prefetch {pf} bytes ({'in the core launch' if in_core else 'side stream'}): "
            f"outputs equal = {same}")
        assert same


def test_prefetch_alone_writes_nothing():
    W = _weights(1, 4096, 4096, 5)[0]
    before = W.clone()
    tp.prefetch(W, W.numel() * 2)
    tp.prefetch(W, 1000)                     # rounded down to whole 16-byte pieces
    torch.cuda.synchronize()
    assert torch.equal(W.view(torch.int16), before.view(torch.int16))
