"""Multi-layer decode streaming over proj_run_layers (argument marshalling).

Each layer runs its input projection, then o_proj on the first K_o columns of
that output (read in place through the row stride), feeding the next layer,
as DepAttention chains the two projections on the vLLM API page
"vllm.models.kimi_k3.nvidia.specialized_decode.runtime.dep" (section
"DepAttention"; the attention core between them is outside this library).
The chain is enqueued by one native call.
"""
from __future__ import annotations

import ctypes

from ._binding import Plan, _check, _lib, _stream_handle


class LayerStack:
    """L layers of (W_in [N_in, K_in], W_o [N_o, K_o]) with distinct weights."""

    def __init__(self, in_plan: Plan, out_plan: Plan, w_in, w_o):
        if len(w_in) != len(w_o):
            raise ValueError("need one o_proj weight per input projection")
        if out_plan.N != in_plan.K or out_plan.K > in_plan.N:
            raise ValueError("o_proj must map K_o <= N_in columns back to K_in")
        for w in list(w_in) + list(w_o):
            if not w.is_contiguous() or not w.is_cuda:
                raise ValueError("weights must be contiguous device tensors")
        weights = list(w_in) + list(w_o)
        devs = {p.device for p in (in_plan, out_plan)} | {w.device.index for w in weights}
        if len(devs) != 1:
            raise ValueError("the plans and every weight must be on one device")
        self.in_plan, self.out_plan = in_plan, out_plan
        self.w_in, self.w_o = list(w_in), list(w_o)   # keep the tensors alive
        L = len(self.w_in)
        self._pin = (ctypes.c_void_p * max(1, L))(*[w.data_ptr() for w in self.w_in])
        self._po = (ctypes.c_void_p * max(1, L))(*[w.data_ptr() for w in self.w_o])

    def _check_operands(self, x0, y_in, y_o):
        """bfloat16 device tensors on the weights' device: the library takes
        raw device pointers, so a host tensor's address must never reach it."""
        import torch
        ops = (x0, y_in, y_o)
        if any(t.dtype != torch.bfloat16 for t in ops):
            raise TypeError("x0, y_in and y_o must be bfloat16")
        devs = {t.device for t in ops} | {w.device for w in self.w_in[:1]}
        if not all(t.is_cuda for t in ops) or len(devs) != 1:
            raise ValueError("x0, y_in and y_o must be device tensors on the weights' device")

    @property
    def layers(self) -> int:
        return len(self.w_in)

    def buffers(self, B: int, device=None):
        import torch
        dev = device or self.w_in[0].device
        y_in = torch.empty((self.layers, B, self.in_plan.N), dtype=torch.bfloat16, device=dev)
        y_o = torch.empty((self.layers, B, self.out_plan.N), dtype=torch.bfloat16, device=dev)
        return y_in, y_o

    def run(self, x0, y_in=None, y_o=None, *, stream=None):
        """Enqueue every layer; returns (y_in [L,B,N_in], y_o [L,B,N_o])."""
        B = x0.shape[0]
        if y_in is None or y_o is None:
            y_in, y_o = self.buffers(B, x0.device)
        if tuple(y_in.shape) != (self.layers, B, self.in_plan.N) or not y_in.is_contiguous():
            raise ValueError("y_in must be contiguous [L, B, N_in]")
        if tuple(y_o.shape) != (self.layers, B, self.out_plan.N) or not y_o.is_contiguous():
            raise ValueError("y_o must be contiguous [L, B, N_o]")
        if x0.stride(1) != 1 or x0.shape[1] != self.in_plan.K:
            raise ValueError("x0 must be [B, K_in] with unit column stride")
        self._check_operands(x0, y_in, y_o)
        ldx = x0.stride(0) if B > 1 else self.in_plan.K
        rc = _lib().proj_run_layers(self.in_plan.handle, self.out_plan.handle, self.layers,
                                    B, ctypes.c_void_p(x0.data_ptr()), ldx, self._pin,
                                    self._po, ctypes.c_void_p(y_in.data_ptr()),
                                    ctypes.c_void_p(y_o.data_ptr()),
                                    ctypes.c_void_p(_stream_handle(stream)))
        _check(rc, f"proj_run_layers(L={self.layers}, B={B})")
        return y_in, y_o

    def run_overlap(self, x0, y_in, y_o, *, core_us: float, prefetch_bytes: int = 0,
                    stream=None, side_stream=None, prefetch_in_core: bool = False):
        """The chain with a fixed-duration stand-in for the attention core
        between each layer's projections and the prefetch of the head of
        that layer's o_proj weight: beside the core on `side_stream`, or,
        with prefetch_in_core, inside the core's own launch on `stream`."""
        B = x0.shape[0]
        if tuple(y_in.shape) != (self.layers, B, self.in_plan.N) or not y_in.is_contiguous():
            raise ValueError("y_in must be contiguous [L, B, N_in]")
        if tuple(y_o.shape) != (self.layers, B, self.out_plan.N) or not y_o.is_contiguous():
            raise ValueError("y_o must be contiguous [L, B, N_o]")
        if x0.stride(1) != 1 or x0.shape[1] != self.in_plan.K:
            raise ValueError("x0 must be [B, K_in] with unit column stride")
        self._check_operands(x0, y_in, y_o)
        ldx = x0.stride(0) if B > 1 else self.in_plan.K
        if prefetch_in_core:
            side = _stream_handle(stream)
        else:
            side = _stream_handle(side_stream) if side_stream is not None else 0
        rc = _lib().proj_run_layers_overlap(
            self.in_plan.handle, self.out_plan.handle, self.layers, B,
            ctypes.c_void_p(x0.data_ptr()), ldx, self._pin, self._po,
            ctypes.c_void_p(y_in.data_ptr()), ctypes.c_void_p(y_o.data_ptr()),
            float(core_us), int(prefetch_bytes), ctypes.c_void_p(_stream_handle(stream)),
            ctypes.c_void_p(side))
        _check(rc, f"proj_run_layers_overlap(L={self.layers}, B={B})")
        return y_in, y_o
