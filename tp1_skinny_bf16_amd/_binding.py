"""ctypes binding of the C ABI in include/tp1_proj.h (argument marshalling only).

Every step of the projection runs in the HIP library libtp1proj.so; this
module only turns torch tensors into device pointers and streams.  If the
library is not built, importing the binding raises: there is no CPU or
PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtp1proj.so")

PROJ_OK = 0
PROJ_EINVAL = -1
PROJ_EBATCH = -2
PROJ_EALIGN = -3
PROJ_EHIP = -4
PROJ_ENOMEM = -5
PROJ_ENODEV = -6
PROJ_ESCRATCH = -7

KERNEL_STREAM = 1
KERNEL_STREAM_DOT2 = 3
KERNEL_MFMA_XS = 5
KERNEL_MFMA_PIPE = 6
KERNEL_NAMES = {KERNEL_STREAM: "stream", KERNEL_STREAM_DOT2: "stream_dot2",
                KERNEL_MFMA_XS: "mfma_xs", KERNEL_MFMA_PIPE: "mfma_pipe"}
KERNEL_IDS = {v: k for k, v in KERNEL_NAMES.items()}

PLAN_HOST_ONLY = 0x1
PLAN_SPLIT_FUSED = 0x2
MAX_BATCH = 256
MAX_BATCHES = 64
MAX_PACK = 64

# every symbol include/tp1_proj.h declares
EXPORTS = ("proj_plan", "proj_run", "proj_free", "proj_strerror",
           "proj_plan_tactic", "proj_plan_set_tactic",
           "proj_plan_workspace_bytes", "proj_read_probe", "proj_run_layers",
           "proj_plan_kernel_name", "proj_run_noalloc", "proj_prefetch",
           "proj_run_layers_overlap", "proj_pack_rows", "proj_ring_probe")


class ProjError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        msg = _lib().proj_strerror(code).decode() if _LIB is not None else str(code)
        super().__init__(f"{what}: {msg} ({code})" if what else f"{msg} ({code})")


class _Tactic(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("bcap", ctypes.c_int),
                ("split", ctypes.c_int), ("rows", ctypes.c_int),
                ("waves", ctypes.c_int), ("wpc", ctypes.c_int), ("kc", ctypes.c_int),
                ("depth", ctypes.c_int), ("kw", ctypes.c_int), ("nw", ctypes.c_int),
                ("stagger", ctypes.c_int)]


@dataclasses.dataclass(frozen=True)
class Tactic:
    kernel: int
    bcap: int
    split: int
    rows: int
    waves: int
    wpc: int
    kc: int = 0
    depth: int = 0
    kw: int = 0
    nw: int = 0
    stagger: int = 0

    @property
    def kernel_name(self) -> str:
        return KERNEL_NAMES.get(self.kernel, str(self.kernel))

    def as_dict(self) -> dict:
        d = dataclasses.asdict(self)
        d["kernel"] = self.kernel_name
        return d

    def _c(self) -> _Tactic:
        return _Tactic(self.kernel, self.bcap, self.split, self.rows, self.waves,
                       self.wpc, self.kc, self.depth, self.kw, self.nw, self.stagger)


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run __graft_entry__.build() (or "
            "python tp1_skinny_bf16_amd/build.py); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.proj_plan.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                              ctypes.c_int, ctypes.c_uint, ctypes.POINTER(vp)]
    lib.proj_plan.restype = ctypes.c_int
    lib.proj_run.argtypes = [vp, ctypes.c_int, vp, ctypes.c_long, vp, vp, vp]
    lib.proj_run.restype = ctypes.c_int
    lib.proj_free.argtypes = [vp]
    lib.proj_free.restype = None
    lib.proj_strerror.argtypes = [ctypes.c_int]
    lib.proj_strerror.restype = ctypes.c_char_p
    lib.proj_plan_tactic.argtypes = [vp, ctypes.c_int, ctypes.POINTER(_Tactic),
                                     ctypes.POINTER(ctypes.c_int)]
    lib.proj_plan_tactic.restype = ctypes.c_int
    lib.proj_plan_set_tactic.argtypes = [vp, ctypes.c_int, ctypes.POINTER(_Tactic)]
    lib.proj_plan_set_tactic.restype = ctypes.c_int
    lib.proj_plan_workspace_bytes.argtypes = [vp]
    lib.proj_plan_workspace_bytes.restype = ctypes.c_size_t
    lib.proj_plan_kernel_name.argtypes = [vp, ctypes.c_int, ctypes.c_char_p, ctypes.c_size_t]
    lib.proj_plan_kernel_name.restype = ctypes.c_int
    lib.proj_run_layers.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_long,
                                    ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp]
    lib.proj_run_layers.restype = ctypes.c_int
    lib.proj_prefetch.argtypes = [vp, ctypes.c_size_t, vp]
    lib.proj_prefetch.restype = ctypes.c_int
    lib.proj_pack_rows.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_int),
                                   ctypes.c_int, ctypes.c_int, vp]
    lib.proj_pack_rows.restype = ctypes.c_int
    ci = ctypes.c_int
    lib.proj_ring_probe.argtypes = [vp, vp, ci, ci, ci, ci, ci, ci, ci, ci, vp, vp]
    lib.proj_ring_probe.restype = ctypes.c_int
    lib.proj_run_layers_overlap.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp, ctypes.c_long,
                                            ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp,
                                            ctypes.c_double, ctypes.c_size_t, vp, vp]
    lib.proj_run_layers_overlap.restype = ctypes.c_int
    lib.proj_run_noalloc.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp,
                                     ctypes.c_long, vp, vp, vp]
    lib.proj_run_noalloc.restype = ctypes.c_int
    lib.proj_read_probe.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    lib.proj_read_probe.restype = ctypes.c_int
    _LIB = lib
    return lib


def library():
    """The loaded ctypes library (raises ImportError when not built)."""
    return _lib()


def strerror(code: int) -> str:
    return _lib().proj_strerror(code).decode()


def _check(rc: int, what: str):
    if rc != PROJ_OK:
        raise ProjError(rc, what)


def _stream_handle(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """A plan for an N x K BF16 weight and a list of batch sizes.

    Mirrors the page's DepProjection: `run(x, W, out)` writes
    y = x . W^T into `out` (BF16 [B, N]) and returns it.
    """

    def __init__(self, N: int, K: int, batches, *, host_only: bool = False,
                 fused_split: bool = False):
        self.N, self.K = int(N), int(K)
        self.batches = tuple(int(b) for b in batches)
        arr = (ctypes.c_int * max(1, len(self.batches)))(*self.batches)
        h = ctypes.c_void_p()
        flags = (PLAN_HOST_ONLY if host_only else 0) | (PLAN_SPLIT_FUSED if fused_split else 0)
        rc = _lib().proj_plan(self.N, self.K, arr, len(self.batches), flags, ctypes.byref(h))
        _check(rc, f"proj_plan(N={N}, K={K}, batches={self.batches})")
        self._h = h
        self.host_only = host_only
        # the device the plan's workspace lives on (the current one now)
        self.device = None
        if not host_only:
            import torch
            self.device = torch.cuda.current_device()

    def close(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            _lib().proj_free(h)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    @property
    def handle(self):
        return self._h

    @property
    def workspace_bytes(self) -> int:
        return int(_lib().proj_plan_workspace_bytes(self._h))

    def tactic(self, B: int):
        """(Tactic, bin) proj_run would use for batch B."""
        t = _Tactic()
        b = ctypes.c_int()
        _check(_lib().proj_plan_tactic(self._h, int(B), ctypes.byref(t), ctypes.byref(b)),
               f"proj_plan_tactic(B={B})")
        return (Tactic(t.kernel, t.bcap, t.split, t.rows, t.waves, t.wpc, t.kc, t.depth, t.kw,
                       t.nw, t.stagger), b.value)

    def kernel_name(self, B: int) -> str:
        """Kernel instance(s) proj_run launches for batch B (profiler names)."""
        buf = ctypes.create_string_buffer(128)
        _check(_lib().proj_plan_kernel_name(self._h, int(B), buf, 128),
               f"proj_plan_kernel_name(B={B})")
        return buf.value.decode()

    def set_tactic(self, bin_: int, tactic: Tactic):
        c = tactic._c()
        _check(_lib().proj_plan_set_tactic(self._h, int(bin_), ctypes.byref(c)),
               f"proj_plan_set_tactic(bin={bin_}, {tactic})")

    def run_ptr(self, B: int, x_ptr: int, ldx: int, w_ptr: int, y_ptr: int,
                stream: int = 0) -> int:
        """Raw call: returns the status code instead of raising."""
        return _lib().proj_run(self._h, int(B), ctypes.c_void_p(x_ptr), int(ldx),
                               ctypes.c_void_p(w_ptr), ctypes.c_void_p(y_ptr),
                               ctypes.c_void_p(stream))

    def run(self, x, W, out=None, *, stream=None):
        """y[B, N] = x[B, K] . W^T on the GPU; x may have a row stride > K."""
        import torch
        if x.dtype != torch.bfloat16 or W.dtype != torch.bfloat16:
            raise TypeError("x and W must be bfloat16")
        if x.dim() != 2 or W.dim() != 2 or x.shape[1] != self.K or \
                tuple(W.shape) != (self.N, self.K):
            raise ValueError(f"shapes x{tuple(x.shape)} W{tuple(W.shape)} do not "
                             f"match the plan ({self.N} x {self.K})")
        if not (x.is_cuda and W.is_cuda):
            raise ValueError("x and W must be device tensors")
        if x.stride(1) != 1 or not W.is_contiguous():
            raise ValueError("x needs unit column stride and W must be contiguous")
        B = x.shape[0]
        if out is None:
            out = torch.empty((B, self.N), dtype=torch.bfloat16, device=x.device)
        if tuple(out.shape) != (B, self.N) or not out.is_contiguous() or \
                out.dtype != torch.bfloat16:
            raise ValueError("out must be a contiguous bfloat16 [B, N] tensor")
        _same_device(x, W, out)
        if self.device is not None and x.device.index != self.device:
            raise ValueError(f"operands on cuda:{x.device.index}, the plan on cuda:{self.device}")
        ldx = x.stride(0) if B > 1 else self.K
        rc = self.run_ptr(B, x.data_ptr(), ldx, W.data_ptr(), out.data_ptr(),
                          _stream_handle(stream))
        _check(rc, f"proj_run(B={B})")
        return out


def _same_device(*tensors):
    """Every operand a device tensor on one device (the kernels take raw
    device pointers: a host tensor's address must never reach them)."""
    if not all(t.is_cuda for t in tensors):
        raise ValueError("every operand must be a device tensor")
    if len({t.device for t in tensors}) != 1:
        raise ValueError("operands on different devices")


def run_noalloc_ptr(N: int, K: int, B: int, x_ptr: int, ldx: int, w_ptr: int, y_ptr: int,
                    stream: int = 0) -> int:
    """Raw proj_run_noalloc call: returns the status code."""
    return _lib().proj_run_noalloc(int(N), int(K), int(B), ctypes.c_void_p(x_ptr), int(ldx),
                                   ctypes.c_void_p(w_ptr), ctypes.c_void_p(y_ptr),
                                   ctypes.c_void_p(stream))


def run_noalloc(x, W, out, *, stream=None):
    """y[B, N] = x[B, K] . W^T into the preallocated `out`, with no plan and
    no device allocation (the library's static split-K scratch)."""
    import torch
    if x.dtype != torch.bfloat16 or W.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise TypeError("x, W and out must be bfloat16")
    N, K = W.shape
    B = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K or x.stride(1) != 1 or not W.is_contiguous():
        raise ValueError("x must be [B, K] with unit column stride and W contiguous [N, K]")
    if tuple(out.shape) != (B, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, N] tensor")
    _same_device(x, W, out)
    ldx = x.stride(0) if B > 1 else K
    rc = run_noalloc_ptr(N, K, B, x.data_ptr(), ldx, W.data_ptr(), out.data_ptr(),
                         _stream_handle(stream))
    _check(rc, f"proj_run_noalloc(N={N}, K={K}, B={B})")
    return out


def prefetch(W, nbytes: int, stream=None):
    """Enqueue the prefetch of the leading `nbytes` of weight tensor W (at most
    its size: the library cannot see the tensor's extent)."""
    size = W.numel() * W.element_size()
    if int(nbytes) > 0 and not W.is_cuda:
        raise ValueError("prefetch needs a device tensor")
    if not 0 <= int(nbytes) <= size:
        raise ValueError(f"prefetch of {nbytes} bytes from a {size}-byte tensor")
    if not W.is_contiguous():
        raise ValueError("prefetch needs a contiguous tensor")
    rc = _lib().proj_prefetch(ctypes.c_void_p(W.data_ptr()), int(nbytes),
                              ctypes.c_void_p(_stream_handle(stream)))
    _check(rc, "proj_prefetch")


def pack_rows_ptr(dst: int, srcs, rows, K: int, stream: int = 0) -> int:
    """proj_pack_rows on raw device pointers; returns the status code."""
    n = len(srcs)
    src_arr = (ctypes.c_void_p * max(1, n))(*[int(p) for p in srcs])
    row_arr = (ctypes.c_int * max(1, n))(*[int(r) for r in rows])
    return _lib().proj_pack_rows(ctypes.c_void_p(int(dst)), src_arr, row_arr, n, int(K),
                                 ctypes.c_void_p(int(stream)))


def pack_rows(weights, out=None, stream=None):
    """Stack BF16 [rows_i, K] device tensors into one [sum(rows_i), K] weight
    (allocated unless `out` is given) with proj_pack_rows; returns it."""
    import torch
    weights = list(weights)
    if not weights:
        raise ValueError("nothing to pack")
    K = weights[0].shape[1]
    for w in weights:
        if w.dtype != torch.bfloat16 or w.dim() != 2 or w.shape[1] != K:
            raise ValueError("weights must be 2-D bfloat16 tensors with one row length")
        if not w.is_contiguous():
            raise ValueError("weights must be contiguous")
    rows = [w.shape[0] for w in weights]
    if out is None:
        out = torch.empty((sum(rows), K), dtype=torch.bfloat16, device=weights[0].device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (sum(rows), K) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 [{sum(rows)}, {K}] tensor")
    _same_device(out, *weights)
    _check(pack_rows_ptr(out.data_ptr(), [w.data_ptr() for w in weights], rows, K,
                         _stream_handle(stream)), "proj_pack_rows")
    return out


def ring_probe(x, w, *, rows: int, piece: int, depth: int, barrier: bool, what: int,
               shared_w: bool, grid: int, sink, stream=None):
    """Enqueue the LDS-ring load probe (measurement aid): x [64, K] and w
    [grid * 64, K] (or [64, K] with shared_w) BF16 device tensors, sink a
    float32 device tensor of at least grid * 8 elements."""
    K = x.shape[1]
    need_w = 64 if shared_w else grid * 64
    if tuple(x.shape) != (64, K) or w.shape[1] != K or w.shape[0] < need_w:
        raise ValueError("x must be [64, K] and w at least [grid * 64, K] (or [64, K] shared)")
    if sink.numel() < grid * 8 or sink.dtype.itemsize != 4:
        raise ValueError("sink needs grid * 8 float32 elements")
    if not (x.is_contiguous() and w.is_contiguous() and sink.is_contiguous()):
        raise ValueError("x, w and sink must be contiguous")
    _same_device(x, w, sink)
    rc = _lib().proj_ring_probe(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()), K,
                                int(rows), int(piece), int(depth), int(bool(barrier)), int(what),
                                int(bool(shared_w)), int(grid), ctypes.c_void_p(sink.data_ptr()),
                                ctypes.c_void_p(_stream_handle(stream)))
    _check(rc, "proj_ring_probe")


def read_probe(buf, sink, waves_per_cu: int = 0, stream=None):
    """Enqueue the streaming-read probe over tensor `buf` (measurement aid)."""
    rc = _lib().proj_read_probe(ctypes.c_void_p(buf.data_ptr()),
                                buf.numel() * buf.element_size(),
                                ctypes.c_void_p(sink.data_ptr()), int(waves_per_cu),
                                ctypes.c_void_p(_stream_handle(stream)))
    _check(rc, "proj_read_probe")
