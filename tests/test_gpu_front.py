"""GPU tests of the MoE layer's split-K front (proj_pack_rows + one plan over
the packed [shared gate_up | latent down] weight, the vLLM API page
"vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep": opening text and
section "DepMoe").  The pages print neither part's size, so the parts here
are ragged and full-width shapes with the model's row length 7168."""
import numpy as np
import pytest
import torch

import tp1_skinny_bf16_amd as tp
import workloads as wl
from gpu_util import DEV, check_exact, check_random, say, tactic_label

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(DEV)


@pytest.mark.parametrize("rows,K", [([1000, 24, 536], 2056), ([4096, 2048], 7168)])
def test_pack_rows_stacks_bit_for_bit(rows, K):
    g = torch.Generator().manual_seed(sum(rows) + K)
    parts = [torch.randn((r, K), generator=g).to(torch.bfloat16) for r in rows]
    packed = tp.pack_rows([p.to(DEV) for p in parts])
    torch.cuda.synchronize()
    assert torch.equal(packed.cpu().view(torch.int16), torch.cat(parts).view(torch.int16))


def test_pack_rows_refuses_overlap_and_bad_shapes():
    a = torch.zeros((64, 1024), dtype=torch.bfloat16, device=DEV)
    # the destination (16 rows from row 0) overlaps the source (16 rows from
    # row 8): refused before anything is enqueued
    rc = tp.pack_rows_ptr(a.data_ptr(), [a[8:].data_ptr()], [16], 1024,
                          torch.cuda.current_stream().cuda_stream)
    assert rc == tp.PROJ_EINVAL
    with pytest.raises(ValueError):
        tp.pack_rows([a, torch.zeros((8, 512), dtype=torch.bfloat16, device=DEV)])
    with pytest.raises(ValueError):
        tp.pack_rows([a.t()])


def _parts(rows, K, seed, exact):
    out = []
    for i, r in enumerate(rows):
        if exact:
            _, W = wl.exact_sum_case(1, r, K, seed=seed + i)
        else:
            _, W = wl.random_case(1, r, K, seed=seed + i)
        out.append(W)
    return out


@pytest.mark.parametrize("rows,K", [([1000, 536], 2056), ([300, 40, 77], 1032)])
def test_front_exact_on_small_shapes(rows, K):
    # exact-sum inputs: every planned tactic of the packed shape is bitwise
    # equal to the oracle on each part
    parts = _parts(rows, K, seed=11, exact=True)
    x, _ = wl.exact_sum_case(64, 8, K, seed=5)
    front = tp.MoeFront([p.to(DEV) for p in parts], [1, 2, 4, 8, 16, 32, 64])
    for B in (1, 3, 16, 29, 64):
        views = front.run(x[:B].to(DEV))
        torch.cuda.synchronize()
        for i, (v, W) in enumerate(zip(views, parts)):
            check_exact(f"front part {i} rows={rows} K={K} B={B} {tactic_label(front.plan, B)}",
                        wl.bits(v.contiguous().cpu()), x[:B], W)
    front.close()


@pytest.mark.parametrize("rows", [[4096, 2048], [2048, 1024, 512]])
def test_front_random_full_width(rows):
    # random N(0, 0.02) weights at the model's row length: the parity gates on
    # every output of every part
    K = wl.DSA_K
    parts = _parts(rows, K, seed=21, exact=False)
    x = wl.random_case(64, 8, K, seed=6)[0]
    front = tp.MoeFront([p.to(DEV) for p in parts], [1, 4, 16, 64])
    for B in (1, 4, 13, 64):
        views = front.run(x[:B].to(DEV))
        torch.cuda.synchronize()
        for i, (v, W) in enumerate(zip(views, parts)):
            check_random(f"front part {i} rows={rows} B={B} {tactic_label(front.plan, B)}",
                         wl.bits(v.contiguous().cpu()), x[:B], W)
    with pytest.raises(ValueError):
        front.run(torch.zeros((65, K), dtype=torch.bfloat16, device=DEV))
    front.close()
