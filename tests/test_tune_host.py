"""Host logic of the tactic tuner (no GPU): the candidate lists against the
compiled kernel instances, and the merging of tuning runs into table rows."""
import json
import os
import re

import pytest

import tp1_skinny_bf16_amd as tp
from tp1_skinny_bf16_amd import tune

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BINS = [1, 2, 4, 8, 16, 32, 64, 128, 256]


def _instances(macro):
    src = open(os.path.join(ROOT, "tp1_skinny_bf16_amd", "csrc", "plan.hpp")).read()
    blk = src[src.index(f"{macro}(X)"):]
    blk = blk[:blk.index("\n\n")]
    return {tuple(int(v) for v in m.split(", ")) for m in re.findall(r"X\(([\d, ]+)\)", blk)}


def test_every_pipe_candidate_is_a_compiled_instance_and_vice_versa():
    """A listed candidate without a compiled instance would be skipped
    silently by the tuner; a compiled instance no bin lists is never
    measured."""
    compiled = _instances("TP1_PIPE_INSTANCES")
    listed = set()
    for b in BINS:
        for t in tune.candidates(b):
            if t.kernel == tp.KERNEL_MFMA_PIPE:
                listed.add((t.bcap, t.rows, t.waves, t.kw, t.kc, t.depth, t.nw))
    assert listed <= compiled, sorted(listed - compiled)
    assert compiled <= listed, sorted(compiled - listed)


def test_every_xs_candidate_is_a_compiled_instance():
    compiled = _instances("TP1_XS_INSTANCES")
    listed = {(t.bcap, t.rows, t.waves, t.kc, t.depth)
              for b in BINS for t in tune.candidates(b) if t.kernel == tp.KERNEL_MFMA_XS}
    assert listed <= compiled, sorted(listed - compiled)


@pytest.mark.parametrize("N,K", [(14560, 7168), (7168, 12288), (1820, 7168)])
def test_candidates_validate_on_a_host_plan(N, K):
    """Every candidate of the batch-16 and batch-64 bins either validates or is
    refused with PROJ_EINVAL; each kernel family keeps valid candidates."""
    p = tp.Plan(N, K, [16, 64], host_only=True)
    for b in (16, 64):
        ok = {}
        for t in tune.candidates(b):
            try:
                p.set_tactic(b, t)
                ok[t.kernel] = ok.get(t.kernel, 0) + 1
            except tp.ProjError as e:
                assert e.code == tp.PROJ_EINVAL
        assert ok.get(tp.KERNEL_MFMA_PIPE, 0) > 0 and ok.get(tp.KERNEL_MFMA_XS, 0) > 0


def _run(N, K, bins):
    """A tuner result in the JSON layout measure() writes."""
    out = {"N": N, "K": K, "bins": {}}
    for b, (us, kernel) in bins.items():
        t = tp.Tactic(tp.KERNEL_MFMA_PIPE, max(16, b), 1, 2, 1, 1, kernel, 4, 4, 8, 1).as_dict()
        out["bins"][str(b)] = {"chosen": {"tactic": t, "us": us, "kernel": "k"},
                               "GBps": 1.0, "n_candidates": 3,
                               "best_stream_us": None, "best_mfma_us": us}
    return out


def test_emit_table_keeps_the_fastest_run_per_bin(tmp_path):
    a = tmp_path / "a.json"
    b = tmp_path / "b.json"
    a.write_text(json.dumps([_run(7168, 12288, {1: (29.0, 256), 2: (28.0, 256)})]))
    b.write_text(json.dumps([_run(7168, 12288, {1: (28.5, 512), 2: (28.9, 512)})]))
    rows = tune.emit_table([str(a), str(b)]).splitlines()
    assert len(rows) == 2
    # bin 1 from run b (512-wide chunks), bin 2 from run a (256-wide)
    assert rows[0].startswith("    {7168, 12288, 1, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 512,")
    assert "// 28.5 us" in rows[0]
    assert rows[1].startswith("    {7168, 12288, 2, {PROJ_KERNEL_MFMA_PIPE, 16, 1, 2, 1, 1, 256,")
    assert "// 28.0 us" in rows[1]
    md = tune.summarize([str(a), str(b)])
    assert "## 7168 x 12288" in md and "Crossover (first bin whose best tactic is an MFMA kernel): 1" in md


def test_recheck_picks_only_bins_whose_choice_beat_the_table_tactic():
    """The paired re-check looks at a bin only when the run's choice beat the
    table's own tactic, timed in the same run, by more than the margin;
    fields missing from older runs read as 0."""
    table = {(100, 256, 8): tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 1, 4, 1, 1, 128, 4, 1, 4),
             (100, 256, 16): tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 2, 4, 1, 1, 128, 4, 1, 4)}
    other = tp.Tactic(tp.KERNEL_STREAM, 8, 1, 4, 4, 8)

    def row(t, us):
        d = t.as_dict()
        return {"tactic": d, "us": us}

    old_style = table[(100, 256, 16)].as_dict()
    del old_style["stagger"]                       # an older run without the field
    run = [{"N": 100, "K": 256, "bins": {
        "8": {"chosen": row(other, 9.0), "all": [row(other, 9.0), row(table[(100, 256, 8)], 10.0)]},
        "16": {"chosen": row(table[(100, 256, 16)], 11.0),
               "all": [{"tactic": old_style, "us": 11.0}]}}}]
    got = tune.recheck_candidates(run, lambda N, K, b: table[(N, K, b)], 0.015)
    assert [(N, K, b) for N, K, b, _, _ in got] == [(100, 256, 8)]
    assert got[0][3] == table[(100, 256, 8)] and got[0][4] == other
    # within the margin: nothing to re-check
    assert tune.recheck_candidates(run, lambda N, K, b: table[(N, K, b)], 0.2) == []
