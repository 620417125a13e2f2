"""CPU tests of the rocprofv3 summarisers (profile_summary, counter_summary)
on small synthetic CSV files in rocprofv3's layout."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]
COPY = "__amd_rocclr_copyBuffer"
KERN = "void tp1::mfma_pipe_kernel<4, 8, 2, 1, 128, 3, 8>(tp1::MfmaArgs)"


def _counters(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (name, grid, counter, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Agent_Id": "Agent 1",
                        "Queue_Id": 1, "Process_Id": 1, "Thread_Id": 1, "Grid_Size": grid,
                        "Kernel_Id": 1, "Kernel_Name": name, "Workgroup_Size": 512,
                        "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 8,
                        "Accum_VGPR_Count": 0, "SGPR_Count": 8, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": 0, "End_Timestamp": 1})


def _run(module, *args, cwd):
    env = dict(os.environ, PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-m", module, *args], cwd=cwd, env=env,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return r.stdout


def test_traffic_scale_comes_from_the_largest_copy(tmp_path):
    # two smaller copies (a weight being packed) share the reference copy's
    # grid: the scale must come from the 256 MiB copies alone.  FETCH_SIZE
    # reads half the bytes, WRITE_SIZE all of them, as measured on the GPU.
    ref = 268435456 / 1024
    kt = tmp_path / "kt"
    kt.mkdir()
    with open(kt / "kt_kernel_stats.csv", "w") as f:
        f.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        f.write(f'"{KERN}",2,60000,30000.0,90.0,29000,31000,1.0\n')
        f.write(f'"{COPY}",5,500000,100000.0,10.0,8000,110000,1.0\n')
    fetch = [(COPY, 131072, "FETCH_SIZE", ref * 0.5)] * 2 + \
            [(COPY, 131072, "FETCH_SIZE", ref * 0.05)] * 2 + \
            [(KERN, 131072, "FETCH_SIZE", 100e6 / 1024 * 0.5)] * 2
    write = [(COPY, 131072, "WRITE_SIZE", ref)] * 2 + \
            [(COPY, 131072, "WRITE_SIZE", ref * 0.1)] * 2 + \
            [(KERN, 131072, "WRITE_SIZE", 2e6 / 1024)] * 2
    _counters(str(tmp_path / "f" / "f_counter_collection.csv"), fetch)
    _counters(str(tmp_path / "w" / "w_counter_collection.csv"), write)
    line = {"moe_front": {"points": [{"kernel": "mfma_pipe_kernel<4, 8, 2, 1, 128, 3, 8>",
                                      "B": 1, "N": 6000, "K": 8000}]}}
    (tmp_path / "bench.json").write_text(json.dumps(line) + "\n")
    out = tmp_path / "out"
    _run("tp1_skinny_bf16_amd.profile_summary", "--kt", str(kt), "--fetch",
         str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--bench-json",
         str(tmp_path / "bench.json"), "--name", "t", "--command", "c", "--out", str(out),
         cwd=ROOT)
    traffic = json.load(open(out / "traffic.json"))["kernels"]
    k = traffic["mfma_pipe_kernel<4, 8, 2, 1, 128, 3, 8>"]
    assert abs(k["read_bytes"] - 100e6) < 1e3 and abs(k["write_bytes"] - 2e6) < 1e3
    text = (out / "t_traffic.md").read_text()
    assert "/ 0.50000" in text and "/ 1.00000" in text
    # algorithmic bytes of the front point: 2NK + 2BK + 2BN
    alg = (2 * 6000 * 8000 + 2 * 8000 + 2 * 6000) / 1e6
    assert f"{alg:.2f}" in text


def test_counter_passes_merge_with_l2_hit_rate(tmp_path):
    a, b = tmp_path / "a", tmp_path / "b"
    _counters(str(a / "m_counter_collection.csv"),
              [(KERN, 131072, "SQ_VALU_MFMA_BUSY_CYCLES", 1024.0 * 4 * 10),
               (KERN, 131072, "GRBM_GUI_ACTIVE", 8 * 100.0)])
    _counters(str(b / "m_counter_collection.csv"),
              [(KERN, 131072, "TCC_HIT_sum", 30.0), (KERN, 131072, "TCC_MISS_sum", 70.0)])
    out = tmp_path / "out"
    _run("tp1_skinny_bf16_amd.counter_summary", "--dir", str(a), str(b), "--name", "t",
         "--command", "c", "--cus", "1024", "--out", str(out), cwd=ROOT)
    row = [l for l in (out / "t_counters.md").read_text().splitlines()
           if l.startswith("| `mfma_pipe")][0]
    # MFMA busy = 40960 / ((800 / 8) * 1024 * 4) = 10%; L2 hit = 30 / 100
    assert "| 10.0% |" in row and row.rstrip().endswith("| 30.0% |")
