"""The MoE layer's split-K front over a packed weight (argument marshalling).

On the vLLM API page "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.
dep" (its opening text and section "DepMoe"), every MoE layer of a decode step
starts with a split-K front: one projection of the layer's rows over the
shared expert's gate_up weight and the latent down-projection weight packed
into one [shared gate_up | latent down] matrix, for batches up to the front's
limit (wider batches take the stock module).  Here the parts are stacked once
with proj_pack_rows, one plan covers the packed shape, and each call is one
proj_run whose output columns hold the parts side by side.  The pages print
neither part's size: any row counts with one row length K work.
"""
from __future__ import annotations

from ._binding import Plan, pack_rows


def _stream_object(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


class MoeFront:
    """A split-K front over BF16 weights [rows_i, K] that share the input x."""

    def __init__(self, parts, batches, *, stream=None):
        parts = list(parts)
        if not parts:
            raise ValueError("a front needs at least one weight")
        self.rows = [int(p.shape[0]) for p in parts]
        self.N = sum(self.rows)
        self.K = int(parts[0].shape[1])
        self.weight = pack_rows(parts, stream=stream)   # one [N, K] weight
        # packing is a one-time preparation: wait for it here, so that a call
        # on any stream reads the packed weight
        _stream_object(stream).synchronize()
        self.plan = Plan(self.N, self.K, batches)
        self.front_max = max(batches)

    def buffer(self, B: int):
        import torch
        return torch.empty((B, self.N), dtype=torch.bfloat16, device=self.weight.device)

    def run(self, x, y=None, *, stream=None):
        """Enqueue y = x . [part_0; part_1; ...]^T; returns the list of column
        views y[:, r0_i : r0_i + rows_i], one per part (x . part_i^T)."""
        B = x.shape[0]
        if B > self.front_max:
            raise ValueError(f"batch {B} is above the front's limit {self.front_max}")
        if y is None:
            y = self.buffer(B)
        self.plan.run(x, self.weight, y, stream=stream)
        out, r0 = [], 0
        for r in self.rows:
            out.append(y[:, r0:r0 + r])
            r0 += r
        return out

    def close(self):
        self.plan.close()
