"""TP1 BF16 decode projection for MI355X (gfx950).

y[B, N] = x[B, K] . W^T with BF16 x and W (nn.Linear N x K layout), FP32
accumulation and BF16 output, for decode batches B = 1..256, as the TP1 linear
of the vLLM API page "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep"
(section "DepProjection") defines it.  The work runs in hand-written HIP
kernels behind the C ABI of include/tp1_proj.h; this package is the thin
Python binding (torch supplies device memory and streams only).
"""
from ._binding import (EXPORTS, KERNEL_IDS, KERNEL_NAMES,  # noqa: F401
                       KERNEL_MFMA_PIPE, KERNEL_MFMA_XS, KERNEL_STREAM,
                       KERNEL_STREAM_DOT2,
                       LIB_PATH, MAX_BATCH, MAX_BATCHES, MAX_PACK, PROJ_EALIGN, PROJ_EBATCH,
                       PROJ_EHIP, PROJ_EINVAL, PROJ_ENODEV, PROJ_ENOMEM, PROJ_ESCRATCH,
                       PROJ_OK, Plan, ProjError, Tactic, library, pack_rows, pack_rows_ptr,
                       prefetch, read_probe, ring_probe, run_noalloc, run_noalloc_ptr,
                       strerror)
from .front import MoeFront  # noqa: F401
from .layers import LayerStack  # noqa: F401
