"""CPU model of the pipelined MFMA kernel's indexing (mfma_pipe_kernel).

The kernel fills LDS with direct-to-LDS loads, so a lane's load address and
the LDS position it lands in are tied by the load instruction (1 KB blocks,
16 bytes per lane); the MFMA fragment reads then find each 16-byte piece by
a per-row rotation.  These tests re-derive that arithmetic for every
compiled instance and check, without a GPU:
  - the loaders fill every (row, piece) position of a stage exactly once and
    the fragment reads look each piece up where it was loaded;
  - the 16 rows of every fragment read fall in 16 distinct bank groups;
  - fragment reads stay inside the x rows / weight rows of the stage;
  - every global address a lane loads at the extreme steps of a workgroup is
    inside x or W, for ragged and full shapes, batches and K splits;
  - the LDS the plan reserves covers the ring and the partial tiles, and the
    library accepts every instance as a tactic.
"""
import os
import re

import numpy as np
import pytest

import tp1_skinny_bf16_amd as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LDS_BYTES = 160 * 1024


def pipe_instances():
    src = open(os.path.join(ROOT, "tp1_skinny_bf16_amd", "csrc", "plan.hpp")).read()
    blk = src[src.index("TP1_PIPE_INSTANCES(X)"):]
    blk = blk[:blk.index("\n\n")]
    pat = r"X\((\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\)"
    return [tuple(map(int, m)) for m in re.findall(pat, blk)]


INSTANCES = pipe_instances()


def ceil(a, b):
    return -(-a // b)


class Geometry:
    """The kernel's compile-time geometry for one instance."""

    def __init__(self, bcap, ntb, wm, wk, kc, depth, nw):
        self.MT, self.NTB, self.WM, self.WK, self.KC, self.D, self.NW = (
            bcap // 16, ntb, wm, wk, kc, depth, nw)
        self.WN = nw // (wm * wk)
        self.MTW, self.NTW = self.MT // wm, ntb // self.WN
        self.XR, self.GR, self.PP = 16 * self.MT, 16 * ntb, kc // 8
        self.SH = 0 if self.PP >= 16 else (1 if self.PP == 8 else 2)
        self.STAGE = (self.XR + self.GR) * self.PP * 16
        self.NB = (self.XR + self.GR) * self.PP // 64
        self.XB = self.XR * self.PP // 64
        self.NI = self.NB // nw

    def slot_of(self, r, p):
        return r * self.PP + ((p + (r >> self.SH)) & (self.PP - 1))

    def loader_pieces(self):
        """(wave, block index, lane) -> (stage row, piece)."""
        out = {}
        for wave in range(self.NW):
            for i in range(self.NI):
                bi = i * self.NW + wave
                for lane in range(64):
                    slot = bi * 64 + lane
                    r = slot // self.PP
                    p = ((slot % self.PP) - (r >> self.SH)) & (self.PP - 1)
                    out[(wave, bi, lane)] = (r, p, slot)
        return out


@pytest.mark.parametrize("inst", INSTANCES, ids=lambda t: "x".join(map(str, t)))
def test_static_constraints(inst):
    g = Geometry(*inst)
    assert g.WN * g.WM * g.WK == g.NW and g.NW in (4, 8)
    assert g.MT % g.WM == 0 and g.NTB % g.WN == 0
    assert (g.KC // 32) % g.WK == 0
    assert g.PP in (4, 8) or g.PP % 16 == 0 and g.PP <= 64
    assert g.NB % g.NW == 0 and (g.XR * g.PP) % 64 == 0
    assert 2 <= g.D and g.NI * (g.D - 2) <= 63          # vmcnt immediate range
    parts = (g.WK - 1) * g.MT * g.NTB * 1024
    assert parts == (g.WK - 1) * g.WM * g.WN * g.MTW * g.NTW * 64 * 16
    assert g.D * g.STAGE + parts + 16 <= LDS_BYTES      # + the fixup's shared flag


@pytest.mark.parametrize("inst", INSTANCES, ids=lambda t: "x".join(map(str, t)))
def test_loader_and_reader_agree(inst):
    g = Geometry(*inst)
    pieces = g.loader_pieces()
    seen = {}
    for (wave, bi, lane), (r, p, slot) in pieces.items():
        assert (bi < g.XB) == (r < g.XR)                 # x blocks hold x rows only
        assert (r, p) not in seen
        seen[(r, p)] = slot
        assert g.slot_of(r, p) == slot                    # the read finds the piece
    assert len(seen) == (g.XR + g.GR) * g.PP             # every position filled once
    for r0 in range(0, g.XR + g.GR, 16):
        for p in range(g.PP):
            groups = {g.slot_of(r, p) % 16 for r in range(r0, r0 + 16)}
            assert len(groups) == 16, (r0, p)             # conflict-free fragment read
    for wave in range(g.NW):
        wk = wave // (g.WM * g.WN)
        wmn = wave % (g.WM * g.WN)
        wm, wn = wmn // g.WN, wmn % g.WN
        for jj in range(g.KC // 32 // g.WK):
            j = jj * g.WK + wk
            for lgrp in range(4):
                assert j * 4 + lgrp < g.PP
            for n in range(g.NTW):
                r = g.XR + (wn * g.NTW + n) * 16
                assert g.XR <= r and r + 15 < g.XR + g.GR
            for m in range(g.MTW):
                assert (wm * g.MTW + m) * 16 + 15 < g.XR


def _slices(K, KC, split):
    step = max(KC, 32)
    ks = max(ceil(ceil(K, split), step) * step, step)
    return ks, ceil(K, ks)


SHAPES = [(1000, 1032), (77, 520), (33, 8), (300, 2056), (14560, 7168), (7168, 12288),
          (49376, 7168)]


@pytest.mark.parametrize("inst", INSTANCES, ids=lambda t: "x".join(map(str, t)))
def test_global_loads_in_bounds(inst):
    g = Geometry(*inst)
    pieces = list(g.loader_pieces().values())
    r = np.array([q[0] for q in pieces], dtype=np.int64)
    kp = np.array([q[1] for q in pieces], dtype=np.int64) * 8
    is_x = r < g.XR
    bcap = 16 * g.MT
    for N, K in SHAPES:
        for B in sorted({bcap, max(1, bcap // 2 + 1), 1}):
            for split in (1, 3, 8):
                for wpc in (1, 2):
                    ks, S = _slices(K, g.KC, split)
                    grid = max(1, min(256 * wpc // S, N))
                    blocks = range(grid) if grid <= 6 else [0, 1, grid // 2, grid - 2, grid - 1]
                    for s in range(S):
                        k0 = s * ks
                        klen = min(K - k0, ks)
                        assert klen > 0
                        C = ceil(klen, g.KC)
                        for bx in blocks:
                            row0 = N * bx // grid
                            rows = N * (bx + 1) // grid - row0
                            assert rows >= 1
                            T = ceil(rows, g.GR) * C
                            for it in sorted({0, C - 1, T - C, T - 1}):
                                ig, ic = it // C, it % C
                                k = ic * g.KC + kp
                                live_k = k < klen          # else the zero block loads
                                xl = is_x & live_k & (r < B)
                                assert np.all(r[xl] * K + k0 + k[xl] + 8 <= B * K)
                                rr = ig * g.GR + r - g.XR
                                wl = ~is_x & live_k & (rr < rows)
                                assert np.all(row0 + rr[wl] < N)
                                assert np.all(k0 + k[wl] + 8 <= K)
                                assert np.all(rr[wl] >= 0)


@pytest.mark.parametrize("inst", INSTANCES, ids=lambda t: "x".join(map(str, t)))
def test_library_accepts_every_instance(inst):
    bcap, rows, waves, kw, kc, depth, nw = inst
    plan = tp.Plan(14560, 7168, [bcap], host_only=True)
    for wpc in (1, 2):
        t = tp.Tactic(tp.KERNEL_MFMA_PIPE, bcap, 1, rows, waves, wpc, kc, depth, kw, nw)
        g = Geometry(*inst)
        lds = g.D * g.STAGE + (g.WK - 1) * g.MT * g.NTB * 1024
        if wpc == 1:
            plan.set_tactic(bcap, t)
            assert plan.tactic(bcap)[0] == t
        assert lds <= LDS_BYTES
    # an instance that is not compiled is refused
    bad = tp.Tactic(tp.KERNEL_MFMA_PIPE, bcap, 1, rows, waves, 1, kc, depth + 100, kw, nw)
    with pytest.raises(tp.ProjError):
        plan.set_tactic(bcap, bad)
