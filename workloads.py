"""Seeded synthetic workloads for the TP1 decode projection.

This module only draws inputs: it holds none of the projection's arithmetic,
so both the GPU path's tests/benchmark and the CPU oracle can take their
inputs from it.

Shapes are the Kimi K3 decode projections named on the vLLM API page
"vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep" (opening text):
the packed DSA input projection 14560 x 7168, the o_proj 7168 x 12288 (its
input is 96 heads x 128 = 12288 wide, section "DepAttention") and the packed
KDA input projection 49376 x 7168.  The pages give no data, so the values are
synthetic stand-ins for RMS-normalised rows times trained weights: x ~ N(0,1),
W ~ N(0, 0.02) (0.02 read as the standard deviation), both drawn as float32
from a seeded CPU torch generator and rounded to BF16 by torch's
round-to-nearest-even cast.  Within a configuration the weight is drawn first,
then x for the largest batch; a smaller batch uses the leading rows of x.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

DSA_N, DSA_K = 14560, 7168        # packed [q_a | kv_a | gate | wk | wv]
OPROJ_N, OPROJ_K = 7168, 12288    # o_proj, input 96 heads x 128
KDA_N, KDA_K = 49376, 7168        # packed KDA in_proj_qkvgfab

W_STD = 0.02
X_STD = 1.0


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    N: int
    K: int
    batches: tuple
    seed: int
    layers: int = 1               # >1 only for the multi-layer stream

    @property
    def bmax(self) -> int:
        return max(self.batches)


CONFIGS = (
    Config("dsa_b1", DSA_N, DSA_K, (1,), 0),
    Config("oproj_sweep", OPROJ_N, OPROJ_K, (1, 2, 4, 8, 16), 1),
    Config("kda_sweep", KDA_N, KDA_K, (1, 4, 8, 16, 32), 2),
    Config("dsa_sweep", DSA_N, DSA_K, (1, 2, 4, 8, 16, 32, 64, 128, 256), 3),
    # 8 layers of (W_in 14560x7168 then W_o 7168x12288) at B=64; the o_proj
    # input is columns 0..12287 of the in-projection output.
    Config("multilayer", DSA_N, DSA_K, (64,), 4, layers=8),
)
BY_NAME = {c.name: c for c in CONFIGS}


def normal_bf16(shape, std: float, gen: torch.Generator,
                device: str | torch.device = "cpu") -> torch.Tensor:
    """BF16 tensor with N(0, std) values: float32 draw, scale, RNE cast."""
    t = torch.randn(*shape, generator=gen, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def config_tensors(cfg: Config) -> dict:
    """CPU BF16 tensors of a configuration, drawn in a fixed order.

    single-layer: {"W": [N,K], "x": [bmax,K]}
    multi-layer:  {"W_in": [L x [N,K]], "W_o": [L x [7168,12288]], "x": [64,7168]}
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(cfg.seed)
    if cfg.layers == 1:
        W = normal_bf16((cfg.N, cfg.K), W_STD, g)
        x = normal_bf16((cfg.bmax, cfg.K), X_STD, g)
        return {"W": W, "x": x}
    w_in, w_o = [], []
    for _ in range(cfg.layers):
        w_in.append(normal_bf16((cfg.N, cfg.K), W_STD, g))
        w_o.append(normal_bf16((OPROJ_N, OPROJ_K), W_STD, g))
    x = normal_bf16((cfg.bmax, cfg.K), X_STD, g)
    return {"W_in": w_in, "W_o": w_o, "x": x}


def random_case(B: int, N: int, K: int, seed: int, w_std: float = W_STD,
                x_std: float = X_STD) -> tuple:
    """(x[B,K], W[N,K]) BF16 CPU tensors for an arbitrary shape."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    W = normal_bf16((N, K), w_std, g)
    x = normal_bf16((B, K), x_std, g)
    return x, W


def exact_sum_case(B: int, N: int, K: int, seed: int) -> tuple:
    """Integer workload whose every partial sum is exact in float32.

    x in {-3..3}, W in {-3..3} * 2^-5: every product and every partial sum
    is a multiple of 2^-5 of magnitude <= 9 * K * 2^-5 (3456 < 2^12 for
    K = 12288), so it needs at most 17 significant bits and any float32
    summation order gives the exact sum.  The result (an integer multiple of
    2^-5 below 2^12) still rounds to BF16, identically on every path.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    W = (torch.randint(-3, 4, (N, K), generator=g).to(torch.float32)
         * 2.0 ** -5).to(torch.bfloat16)
    x = torch.randint(-3, 4, (B, K), generator=g).to(torch.bfloat16)
    return x, W


def one_hot_weight(N: int, K: int, scale: float = 1.0) -> torch.Tensor:
    """W[n,k] = scale if k == n mod K else 0 (identity for N == K)."""
    W = torch.zeros((N, K), dtype=torch.bfloat16)
    n = torch.arange(N)
    W[n, n % K] = scale
    return W


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 numpy view of a CPU BF16 tensor's bit patterns."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(b: np.ndarray) -> torch.Tensor:
    """CPU BF16 tensor from uint16 bit patterns."""
    arr = np.ascontiguousarray(b, dtype=np.uint16)
    return torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16)


def algorithmic_bytes(B: int, N: int, K: int) -> int:
    """Bytes a projection call must move: W once, x once, y once (BF16)."""
    return 2 * N * K + 2 * B * K + 2 * B * N
