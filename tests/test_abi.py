"""CPU tests of the C ABI: symbols, host-only plans, bins and validation.

No compute call is made here (there is no GPU); host-only plans exercise the
plan logic and every argument check of proj_run up to the launch.
"""
import ctypes
import os
import re
import subprocess

import pytest

import tp1_skinny_bf16_amd as tp
from tp1_skinny_bf16_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp1_proj.h")

SHAPES = [(14560, 7168), (7168, 12288), (49376, 7168)]
ALL_B = [1, 2, 4, 8, 16, 32, 64, 128, 256]


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(proj_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(tp.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = tp.library()
    out = subprocess.run(["nm", "-D", "--defined-only", tp.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in header_functions():
        assert name in exported, f"{name} not exported"
        assert hasattr(lib, name)


def test_strerror_covers_every_status():
    for code in (tp.PROJ_OK, tp.PROJ_EINVAL, tp.PROJ_EBATCH, tp.PROJ_EALIGN,
                 tp.PROJ_EHIP, tp.PROJ_ENOMEM, tp.PROJ_ENODEV, tp.PROJ_ESCRATCH):
        assert tp.strerror(code) and tp.strerror(code) != "unknown status"
    assert tp.strerror(12345) == "unknown status"


def _plan_rc(N, K, batches, flags=bd.PLAN_HOST_ONLY):
    lib = tp.library()
    arr = (ctypes.c_int * max(1, len(batches)))(*batches)
    h = ctypes.c_void_p()
    rc = lib.proj_plan(N, K, arr, len(batches), flags, ctypes.byref(h))
    if h:
        lib.proj_free(h)
    return rc


@pytest.mark.parametrize("N,K,batches", [
    (0, 7168, [1]), (-1, 7168, [1]), (100, 0, [1]), (100, 7164, [1]),
    (100, 64, []), (100, 64, [2, 1]), (100, 64, [1, 1]), (100, 64, [0]),
    (100, 64, [257]), (100, 64, list(range(1, 66))),
])
def test_plan_rejects_bad_arguments(N, K, batches):
    assert _plan_rc(N, K, batches) == tp.PROJ_EINVAL


def test_plan_rejects_unknown_flags_and_null_out():
    assert _plan_rc(100, 64, [1], flags=0x80) == tp.PROJ_EINVAL
    arr = (ctypes.c_int * 1)(1)
    assert tp.library().proj_plan(100, 64, arr, 1, 1, None) == tp.PROJ_EINVAL


def test_bins_follow_the_smallest_key_at_or_above():
    # the page's _bins: the smallest key >= batch; above the largest key
    # this library refuses instead of falling back.
    p = tp.Plan(14560, 7168, [4, 16, 64], host_only=True)
    assert p.tactic(1)[1] == 4
    assert p.tactic(4)[1] == 4
    assert p.tactic(5)[1] == 16
    assert p.tactic(17)[1] == 64
    assert p.tactic(64)[1] == 64
    for bad in (0, -3, 65, 1000):
        with pytest.raises(tp.ProjError) as e:
            p.tactic(bad)
        assert e.value.code == tp.PROJ_EBATCH


TP_SHARDS = [(14560 // g, 7168) for g in (2, 4, 8)] + [(7168, 12288 // g) for g in (2, 4, 8)] + \
            [(49376 // g, 7168) for g in (2, 4, 8)]


@pytest.mark.parametrize("N,K", SHAPES + TP_SHARDS +
                         [(1000, 1032), (777, 2056), (33, 8), (5, 12288)])
def test_every_planned_bin_gets_a_valid_tactic(N, K):
    p = tp.Plan(N, K, ALL_B, host_only=True)
    for b in range(1, 257):
        t, bin_ = p.tactic(b)
        assert bin_ >= b and t.bcap >= bin_
        assert t.kernel in tp.KERNEL_NAMES
        # setting the chosen tactic back must validate
        p.set_tactic(bin_, t)


def test_set_tactic_validation():
    p = tp.Plan(14560, 7168, [1, 16], host_only=True)
    good = tp.Tactic(tp.KERNEL_STREAM, 1, 2, 2, 4, 8)
    p.set_tactic(1, good)
    assert p.tactic(1)[0] == good
    assert p.workspace_bytes >= 2 * 1 * 14560 * 4
    for bad in [tp.Tactic(tp.KERNEL_STREAM, 1, 1, 3, 4, 8),       # no instance
                tp.Tactic(tp.KERNEL_STREAM, 1, 1, 1, 9, 8),       # too many waves
                tp.Tactic(tp.KERNEL_STREAM, 1, 0, 1, 4, 8),       # split 0
                tp.Tactic(2, 16, 1, 1, 4, 0),                     # retired kernel ids
                tp.Tactic(4, 16, 1, 1, 2, 4),
                tp.Tactic(7, 1, 1, 1, 1, 1)]:
        with pytest.raises(tp.ProjError):
            p.set_tactic(1, bad)
    with pytest.raises(tp.ProjError):                           # bcap < bin
        p.set_tactic(16, tp.Tactic(tp.KERNEL_STREAM, 8, 1, 1, 4, 8))
    with pytest.raises(tp.ProjError):                           # not a bin
        p.set_tactic(3, good)
    # x for 8 rows of K = 12288 in one slice does not fit the LDS
    q = tp.Plan(7168, 12288, [8], host_only=True)
    with pytest.raises(tp.ProjError):
        q.set_tactic(8, tp.Tactic(tp.KERNEL_STREAM, 8, 1, 1, 4, 8))


def test_stream_lds_counts_the_static_partials():
    """The stream kernel keeps [8 waves][2][rows * bcap] floats of static LDS
    beside the staged x slice: a slice whose staged x alone fills the LDS
    exactly is refused at plan time instead of failing at launch."""
    # bcap 8, one 10240-wide slice: 8 * 10240 * 2 = 163840 bytes of x = all of it
    p = tp.Plan(1000, 10240, [8], host_only=True)
    with pytest.raises(tp.ProjError):
        p.set_tactic(8, tp.Tactic(tp.KERNEL_STREAM, 8, 1, 4, 4, 8))
    # two slices of 5120 leave room for the partials
    p.set_tactic(8, tp.Tactic(tp.KERNEL_STREAM, 8, 2, 4, 4, 8))
    # a slice of 10240 - 512 = 9728 for bcap 8: 155648 + 2048 + 16 bytes fit
    q = tp.Plan(1000, 19456, [8], host_only=True)
    q.set_tactic(8, tp.Tactic(tp.KERNEL_STREAM, 8, 2, 4, 4, 8))


def test_run_argument_checks_on_a_host_only_plan():
    p = tp.Plan(128, 256, [1, 8], host_only=True)
    X, Wp, Y = 0x10000, 0x200000, 0x800000      # never dereferenced
    assert p.run_ptr(0, X, 256, Wp, Y) == tp.PROJ_OK              # no-op
    assert p.run_ptr(9, X, 256, Wp, Y) == tp.PROJ_EBATCH
    assert p.run_ptr(-1, X, 256, Wp, Y) == tp.PROJ_EBATCH
    assert p.run_ptr(1, 0, 256, Wp, Y) == tp.PROJ_EINVAL
    assert p.run_ptr(1, X, 256, 0, Y) == tp.PROJ_EINVAL
    assert p.run_ptr(1, X, 256, Wp, 0) == tp.PROJ_EINVAL
    assert p.run_ptr(1, X, 255, Wp, Y) == tp.PROJ_EINVAL          # ldx < K
    assert p.run_ptr(2, X, 260, Wp, Y) == tp.PROJ_EALIGN          # ldx % 8
    assert p.run_ptr(1, X + 2, 256, Wp, Y) == tp.PROJ_EALIGN
    assert p.run_ptr(1, X, 256, Wp + 8, Y) == tp.PROJ_EALIGN
    assert p.run_ptr(1, X, 256, Wp, Y + 4) == tp.PROJ_EALIGN
    assert p.run_ptr(1, X, 256, Wp, X + 16) == tp.PROJ_EINVAL     # y overlaps x
    assert p.run_ptr(1, X, 256, Wp, Wp + 4096) == tp.PROJ_EINVAL  # y overlaps W
    assert p.run_ptr(8, X, 0, Wp, Y) == tp.PROJ_ENODEV            # ldx 0 = K
    assert p.run_ptr(1, X, 256, Wp, Y) == tp.PROJ_ENODEV
    lib = tp.library()
    assert lib.proj_run(None, 1, X, 256, Wp, Y, None) == tp.PROJ_EINVAL
    lib.proj_free(None)                                           # NULL-safe


def test_run_layers_argument_checks():
    lib = tp.library()
    pin = tp.Plan(14560, 7168, [64], host_only=True)
    po = tp.Plan(7168, 12288, [64], host_only=True)
    bad_o = tp.Plan(7000, 12288, [64], host_only=True)
    W = (ctypes.c_void_p * 2)(0x100000, 0x200000)
    Wz = (ctypes.c_void_p * 2)(0x100000, None)
    X, Y1, Y2 = 0x10000000, 0x20000000, 0x30000000
    call = lambda a, b, L, B, w=W: lib.proj_run_layers(  # noqa: E731
        a.handle, b.handle, L, B, ctypes.c_void_p(X), 0, w, w,
        ctypes.c_void_p(Y1), ctypes.c_void_p(Y2), None)
    assert call(pin, po, 2, 64) == tp.PROJ_ENODEV
    assert call(pin, po, 0, 64) == tp.PROJ_OK
    assert call(pin, po, 2, 65) == tp.PROJ_EBATCH
    assert call(pin, bad_o, 2, 64) == tp.PROJ_EINVAL     # o_proj N != K_in
    assert call(po, pin, 2, 64) == tp.PROJ_EINVAL        # wrong chain order
    assert call(pin, po, 2, 64, Wz) == tp.PROJ_EINVAL    # a NULL weight
    assert call(pin, po, -1, 64) == tp.PROJ_EINVAL
    # an input projection of 1820 rows cannot feed o_proj in place (rows of
    # 3640 bytes are not 16-byte aligned): refused before any launch
    shard_in = tp.Plan(1820, 7168, [64], host_only=True)
    shard_o = tp.Plan(7168, 1536, [64], host_only=True)
    assert call(shard_in, shard_o, 2, 64) == tp.PROJ_EALIGN
    assert lib.proj_run_layers(pin.handle, po.handle, 2, 64, ctypes.c_void_p(X + 8), 0, W, W,
                               ctypes.c_void_p(Y1), ctypes.c_void_p(Y2), None) == tp.PROJ_EALIGN


def test_run_layers_overlap_argument_checks():
    lib = tp.library()
    pin = tp.Plan(14560, 7168, [64], host_only=True)
    po = tp.Plan(7168, 12288, [64], host_only=True)
    W = (ctypes.c_void_p * 2)(0x100000, 0x200000)
    X, Y1, Y2, S1, S2 = 0x10000000, 0x20000000, 0x30000000, 0x1234, 0x5678
    call = lambda L, B, core, pf, st, side: lib.proj_run_layers_overlap(  # noqa: E731
        pin.handle, po.handle, L, B, ctypes.c_void_p(X), 0, W, W, ctypes.c_void_p(Y1),
        ctypes.c_void_p(Y2), core, pf, ctypes.c_void_p(st), ctypes.c_void_p(side))
    assert call(2, 64, 5.0, 1 << 20, S1, S2) == tp.PROJ_ENODEV    # host-only plans
    assert call(2, 64, -1.0, 0, S1, 0) == tp.PROJ_EINVAL          # negative core time
    assert call(2, 64, float("nan"), 0, S1, 0) == tp.PROJ_EINVAL
    assert call(2, 64, 5.0, 1 << 20, S1, 0) == tp.PROJ_EINVAL     # prefetch, no side stream
    # side == main stream: the prefetch runs inside the stand-in's launch (valid;
    # host-only plans cannot run it)
    assert call(2, 64, 5.0, 1 << 20, S1, S1) == tp.PROJ_ENODEV
    assert call(2, 64, 5.0, 1 << 20, 0, 0) == tp.PROJ_ENODEV
    assert call(2, 65, 5.0, 0, S1, 0) == tp.PROJ_EBATCH
    assert call(0, 64, 5.0, 1 << 20, S1, S2) == tp.PROJ_OK        # nothing to do
    assert lib.proj_prefetch(None, 16, None) == tp.PROJ_EINVAL
    assert lib.proj_prefetch(ctypes.c_void_p(0x1008), 16, None) == tp.PROJ_EALIGN
    assert lib.proj_prefetch(ctypes.c_void_p(0x1000), 0, None) == tp.PROJ_OK


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bd, "_LIB", None)
    monkeypatch.setattr(bd, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        bd.library()


def test_product_package_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "tp1_skinny_bf16_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), f"{f} mentions the oracle"


def test_unlisted_bins_take_the_next_measured_tactic():
    # verify-step batches (requests x (1 + speculative tokens)) are not powers
    # of two; each takes the measured tactic of the next measured bin above it
    p = tp.Plan(14560, 7168, [3, 6, 12, 24, 48, 96, 192], host_only=True)
    q = tp.Plan(14560, 7168, [4, 8, 16, 32, 64, 128, 256], host_only=True)
    for b, ref in zip([3, 6, 12, 24, 48, 96, 192], [4, 8, 16, 32, 64, 128, 256]):
        assert p.tactic(b)[0] == q.tactic(ref)[0]
    # above the largest measured bin there is nothing to borrow: default rule
    r = tp.Plan(14560, 7168, [1], host_only=True)
    assert r.tactic(1)[0].kernel in tp.KERNEL_NAMES


def test_stagger_is_validated():
    p = tp.Plan(14560, 7168, [1, 16], host_only=True)
    for ok in [tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8, stagger=1),
               tp.Tactic(tp.KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, stagger=1)]:
        p.set_tactic(16, ok)
        assert p.tactic(16)[0] == ok
    for bin_, bad in [(16, tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8,
                                     stagger=2)),
                      (16, tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8,
                                     stagger=-1)),
                      (1, tp.Tactic(tp.KERNEL_STREAM, 1, 1, 4, 4, 8, stagger=1))]:
        with pytest.raises(tp.ProjError):
            p.set_tactic(bin_, bad)


def test_pipe_only_fields_are_validated():
    p = tp.Plan(14560, 7168, [16], host_only=True)
    ok = tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 8)
    p.set_tactic(16, ok)
    for bad in [tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 0, 8),    # kw 0
                tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 256, 3, 2, 4),    # not compiled
                tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 1, 4, 1, 3, 256, 3, 2, 8),    # wpc 3
                tp.Tactic(tp.KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 1, 0),      # kw on XS
                tp.Tactic(tp.KERNEL_MFMA_XS, 16, 1, 8, 1, 2, 128, 1, 0, 4),      # nw on XS
                tp.Tactic(tp.KERNEL_STREAM, 1, 1, 4, 4, 8, 0, 0, 0, 8)]:         # nw on STREAM
        with pytest.raises(tp.ProjError):
            p.set_tactic(16, bad)


def test_split_reduction_pass_named_by_output_count():
    """A split-K call launches the four-outputs-per-thread reduction when
    B * N is a multiple of four and the one-per-thread pass otherwise, each
    compiled for S = 2..8 slices (<0>: any S); the kernel name says which
    (rocprof summaries and traffic figures key on it)."""
    t = tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 2, 4, 1, 1, 128, 4, 1, 4)
    p = tp.Plan(1001, 1024, [16], host_only=True)       # N odd
    p.set_tactic(16, t)
    assert p.kernel_name(16).endswith("+splitk_reduce4<2>")    # 16 * 1001 % 4 == 0
    assert p.kernel_name(4).endswith("+splitk_reduce4<2>")
    assert p.kernel_name(3).endswith("+splitk_reduce<2>")      # 3 * 1001 odd
    q = tp.Plan(1002, 1024, [16], host_only=True)
    q.set_tactic(16, t)
    assert q.kernel_name(2).endswith("+splitk_reduce4<2>")     # 2 * 1002 % 4 == 0
    assert q.kernel_name(1).endswith("+splitk_reduce<2>")      # 1002 % 4 == 2
    # slices of 32 (the pipe kernel's K step): 8 of them, then 32
    q.set_tactic(16, tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 8, 4, 1, 1, 128, 4, 1, 4))
    assert q.kernel_name(16).endswith("+splitk_reduce4<8>")
    s = tp.Plan(1002, 4096, [8], host_only=True)
    s.set_tactic(8, tp.Tactic(tp.KERNEL_STREAM, 8, 12, 1, 4, 8))
    assert s.kernel_name(8).endswith("+splitk_reduce4<0>")     # 12 slices
    r = tp.Plan(1001, 1024, [16], host_only=True)
    r.set_tactic(16, tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4))
    assert "splitk" not in r.kernel_name(16)                # no split, no pass


def test_noalloc_argument_checks_return_before_any_device_call():
    """proj_run_noalloc validates shape, batch, stride, alignment and overlap
    on the host and returns before touching a device (these calls run here,
    without a GPU; the pointers are never dereferenced)."""
    run = tp.run_noalloc_ptr
    a, b, c = 0x10000, 0x20000000, 0x40000000        # 16-byte aligned, disjoint
    assert run(0, 64, 1, a, 64, b, c) == tp.PROJ_EINVAL          # N <= 0
    assert run(100, 60, 1, a, 60, b, c) == tp.PROJ_EINVAL        # K % 8
    assert run(100, 64, -1, a, 64, b, c) == tp.PROJ_EBATCH
    assert run(100, 64, 257, a, 64, b, c) == tp.PROJ_EBATCH      # above 256
    assert run(100, 64, 0, 0, 64, 0, 0) == tp.PROJ_OK            # B == 0: no-op
    assert run(100, 64, 2, a, 32, b, c) == tp.PROJ_EINVAL        # ldx < K
    assert run(100, 64, 2, 0, 64, b, c) == tp.PROJ_EINVAL        # null x
    assert run(100, 64, 2, a + 2, 64, b, c) == tp.PROJ_EALIGN    # misaligned x
    assert run(100, 64, 2, a, 68, b, c) == tp.PROJ_EALIGN        # ldx % 8
    assert run(100, 64, 2, a, 64, b, b + 64) == tp.PROJ_EINVAL   # y overlaps W


def test_prefetch_binding_refuses_more_than_the_tensor():
    """The C ABI cannot see a buffer's extent, so the binding checks it: a
    prefetch longer than the tensor (or of a negative size) never reaches the
    library."""
    import torch
    W = torch.empty((4, 8), dtype=torch.bfloat16)          # 64 bytes, CPU: never launched
    with pytest.raises(ValueError):
        tp.prefetch(W, 65)
    with pytest.raises(ValueError):
        tp.prefetch(W, -1)
    with pytest.raises(ValueError):
        tp.prefetch(W.t(), 16)


def test_bindings_refuse_host_tensors():
    """The kernels take raw device pointers, so the Python entry points check
    that every operand is a device tensor before any call into the library."""
    import torch
    x = torch.zeros((2, 64), dtype=torch.bfloat16)
    W = torch.zeros((32, 64), dtype=torch.bfloat16)
    y = torch.zeros((2, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tp.run_noalloc(x, W, y)
    p = tp.Plan(32, 64, [2], host_only=True)
    with pytest.raises(ValueError):
        p.run(x, W, y)


def test_pack_rows_argument_checks_on_the_host():
    # every case is refused before any HIP call: the pointers are never used
    st = 0
    good_dst, good_src = 0x100000, 0x400000
    assert tp.pack_rows_ptr(0, [good_src], [4], 64, st) == tp.PROJ_EINVAL          # no dst
    assert tp.pack_rows_ptr(good_dst, [], [], 64, st) == tp.PROJ_EINVAL           # n = 0
    assert tp.pack_rows_ptr(good_dst, [good_src] * (tp.MAX_PACK + 1),
                            [1] * (tp.MAX_PACK + 1), 64, st) == tp.PROJ_EINVAL    # n too large
    assert tp.pack_rows_ptr(good_dst, [good_src], [4], 60, st) == tp.PROJ_EINVAL  # K % 8
    assert tp.pack_rows_ptr(good_dst, [good_src], [4], 0, st) == tp.PROJ_EINVAL   # K = 0
    assert tp.pack_rows_ptr(good_dst, [good_src], [0], 64, st) == tp.PROJ_EINVAL  # empty part
    assert tp.pack_rows_ptr(good_dst, [0], [4], 64, st) == tp.PROJ_EINVAL         # no source
    assert tp.pack_rows_ptr(good_dst + 8, [good_src], [4], 64, st) == tp.PROJ_EALIGN
    assert tp.pack_rows_ptr(good_dst, [good_src + 8], [4], 64, st) == tp.PROJ_EALIGN
    # a source inside the destination's 2 x 4 x 64 x 2 = 1 KiB, or the other way round
    assert tp.pack_rows_ptr(good_dst, [good_src, good_dst + 512], [4, 4], 64, st) == tp.PROJ_EINVAL
    assert tp.pack_rows_ptr(good_dst, [good_dst - 256], [4], 64, st) == tp.PROJ_EINVAL


def test_unmeasured_shape_takes_the_nearest_measured_tactic():
    # 3072 x 7168 is within a factor of two of the measured 3640 x 7168 (and
    # nearer to it than to 1820 or 6172 rows): it takes that shape's tactic at
    # every bin where the tactic is valid for it
    bins = [1, 2, 4, 8, 16, 32, 64, 128, 256]
    near = tp.Plan(3072, 7168, bins, host_only=True)
    ref = tp.Plan(3640, 7168, bins, host_only=True)
    for b in bins:
        assert near.tactic(b)[0] == ref.tactic(b)[0], b
    # an in-between bin takes the neighbour's tactic for the next measured bin
    mid = tp.Plan(3072, 7168, [3, 12, 100], host_only=True)
    for b, up in ((3, 4), (12, 16), (100, 128)):
        assert mid.tactic(b)[0] == ref.tactic(up)[0], b
    # nothing measured within a factor of two: the default rule (the weight
    # stream for one row, the pipelined kernel above)
    far = tp.Plan(1000, 1032, bins, host_only=True)
    assert far.tactic(1)[0].kernel == tp.KERNEL_STREAM
    assert far.tactic(64)[0].kernel == tp.KERNEL_MFMA_PIPE
    # the measured shapes themselves are unchanged
    assert ref.tactic(1)[0] != far.tactic(1)[0]


def test_ring_probe_argument_checks_on_the_host():
    # refused before any HIP call (the pointers are never used)
    p, s = 0x100000, 0x800000
    lib = tp.library()
    def probe(*a):
        import ctypes
        x, w, K, rows, piece, depth, barrier, what, shared, grid, sink = a
        return lib.proj_ring_probe(ctypes.c_void_p(x), ctypes.c_void_p(w), K, rows, piece,
                                   depth, barrier, what, shared, grid, ctypes.c_void_p(sink),
                                   ctypes.c_void_p(0))
    assert probe(0, p, 7168, 64, 256, 5, 1, 1, 0, 4, s) == tp.PROJ_EINVAL       # no x
    assert probe(p, p, 7168, 64, 256, 5, 1, 3, 0, 4, s) == tp.PROJ_EINVAL       # both needs 128 rows
    assert probe(p, p, 7168, 128, 256, 3, 1, 1, 0, 4, s) == tp.PROJ_EINVAL      # 128 rows needs both
    assert probe(p, p, 7168, 64, 256, 7, 1, 1, 0, 4, s) == tp.PROJ_EINVAL       # not compiled
    assert probe(p, p, 7000, 64, 1024, 2, 1, 1, 0, 4, s) == tp.PROJ_EINVAL      # K*2 % piece
    assert probe(p, p, 7168, 64, 256, 5, 1, 1, 0, 0, s) == tp.PROJ_EINVAL       # empty grid
    assert probe(p + 8, p, 7168, 64, 256, 5, 1, 1, 0, 4, s) == tp.PROJ_EALIGN


def test_every_table_row_is_the_plans_choice():
    # each measured row must pass the library's checks for its own shape and
    # bin: a row that failed them would fall through to another rule unseen
    import os
    import re
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "tp1_skinny_bf16_amd", "csrc", "tactics_table.cpp")).read()
    names = {"PROJ_KERNEL_STREAM": tp.KERNEL_STREAM, "PROJ_KERNEL_STREAM_DOT2": tp.KERNEL_STREAM_DOT2,
             "PROJ_KERNEL_MFMA_XS": tp.KERNEL_MFMA_XS, "PROJ_KERNEL_MFMA_PIPE": tp.KERNEL_MFMA_PIPE}
    pat = r"\{(\d+), (\d+), (\d+), \{(PROJ_KERNEL_\w+), ([\d, ]+)\}\}"
    rows = re.findall(pat, src)
    assert len(rows) > 100
    for N, K, b, kern, fields in rows:
        vals = [int(v) for v in fields.split(",")]
        want = tp.Tactic(names[kern], *vals)
        plan = tp.Plan(int(N), int(K), [int(b)], host_only=True)
        assert plan.tactic(int(b))[0] == want, (N, K, b)
