"""Graph capture of the projection path.

A decode step can replay its layer loop as a captured graph: the vLLM API
page "vllm.models.kimi_k3.nvidia.specialized_decode.runtime", section
"specialized_decode_config", configures the decode runtime with the
engine's graph capture sizes.  Here the graphs are HIP graphs recorded
through torch.cuda.CUDAGraph.  proj_run and proj_run_layers only enqueue
kernels on the stream they are given: no memset, no allocation and no
synchronisation, so both can be captured.  Every tactic is deterministic, so
each replay must equal the eager result bit for bit.  Replays read their
inputs by address, so a new x0 copied into the captured buffer must give the
eager result for that x0.  Between replays the program does eager work of its
own (fills of the outputs, other projections) and synchronises.
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


def _capture(fn):
    """Run fn once eagerly on a side stream (the usual pattern before a
    capture), then capture it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


def test_graph_capture_without_warmup():
    """Capture straight away, with no eager call before: building the plan
    sets every kernel's LDS allowance, so no launch changes a function
    attribute, and the first launches in the process may be recorded into a
    graph.  (First in this file, so in a GPU-only run it precedes every
    other launch of these instances.)"""
    N, K = 3000, 4096
    plan = tp.Plan(N, K, [1, 16, 64])
    W = _weights(1, N, K, 45)[0]
    g = torch.Generator(device=DEV)
    g.manual_seed(46)
    x = torch.randn((64, K), generator=g, device=DEV).to(torch.bfloat16)
    outs = {B: torch.empty((B, N), dtype=torch.bfloat16, device=DEV) for B in (1, 16, 64)}
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for B, o in outs.items():
            plan.run(x[:B], W, o)
    for rep in range(2):
        for o in outs.values():
            o.fill_(0.5)
        graph.replay()
        torch.cuda.synchronize()
        for B, o in outs.items():
            want = _bits(plan.run(x[:B], W))
            torch.cuda.synchronize()
            assert np.array_equal(_bits(o), want), f"replay {rep} B={B} ({plan.kernel_name(B)})"
    say("capture without warm-up: replays equal eager")


def test_graph_replay_layer_chain():
    B, L = 64, 2
    pin = tp.Plan(wl.DSA_N, wl.DSA_K, [16, B])
    po = tp.Plan(wl.OPROJ_N, wl.OPROJ_K, [16, B])
    say(f"chain kernels: {pin.kernel_name(B)} / {po.kernel_name(B)}")
    stack = tp.LayerStack(pin, po, _weights(L, wl.DSA_N, wl.DSA_K, 40),
                          _weights(L, wl.OPROJ_N, wl.OPROJ_K, 41))
    g = torch.Generator(device=DEV)
    g.manual_seed(42)
    xs = [torch.randn((B, wl.DSA_K), generator=g, device=DEV).to(torch.bfloat16)
          for _ in range(2)]
    x0 = xs[0].clone()
    y_in, y_o = stack.buffers(B)
    graph = _capture(lambda: stack.run(x0, y_in, y_o))

    for i, xv in enumerate(xs):
        ref_in, ref_o = stack.run(xv)          # eager, into fresh buffers
        torch.cuda.synchronize()
        ref_in, ref_o = _bits(ref_in), _bits(ref_o)
        x0.copy_(xv)
        for rep in range(3):
            y_in.fill_(7.0)
            y_o.fill_(-3.0)
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(_bits(y_in), ref_in), f"x{i} replay {rep}: in-proj differs"
            assert np.array_equal(_bits(y_o), ref_o), f"x{i} replay {rep}: o_proj differs"
            # eager work of the program between replays, on the same plans
            stack.run(xs[1 - i])
            torch.cuda.synchronize()
    say("chain graph: 2 inputs x 3 replays bitwise equal to eager")


def test_graph_replay_every_bin_one_graph():
    """One graph holding a call per planned bin (B = bin and one ragged B
    below it) of the DSA shape: split-K tactics put two kernels in the graph
    per call and share the plan's workspace in stream order."""
    N, K = wl.DSA_N, wl.DSA_K
    bins = [1, 2, 4, 8, 16, 32, 64, 128, 256]
    plan = tp.Plan(N, K, bins)
    W = _weights(1, N, K, 43)[0]
    g = torch.Generator(device=DEV)
    g.manual_seed(44)
    x = torch.randn((256, K), generator=g, device=DEV).to(torch.bfloat16)
    Bs = sorted({b for bin_ in bins for b in (bin_, max(1, bin_ - 3))})
    outs = {B: torch.empty((B, N), dtype=torch.bfloat16, device=DEV) for B in Bs}

    def calls():
        for B in Bs:
            plan.run(x[:B], W, outs[B])

    graph = _capture(calls)
    refs = {}
    for B in Bs:
        refs[B] = _bits(plan.run(x[:B], W))
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs.values():
            o.fill_(1.0)
        graph.replay()
        torch.cuda.synchronize()
        for B in Bs:
            assert np.array_equal(_bits(outs[B]), refs[B]), \
                f"replay {rep} B={B} ({plan.kernel_name(B)}) differs from eager"
    say(f"per-bin graph: {len(Bs)} calls x 3 replays bitwise equal to eager")
