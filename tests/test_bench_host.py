"""Host logic of bench.py, no GPU: the counting rule, the kernel-name mapping used to read
rocprofv3 output, the one-GPU guard, the source digest that gates stored counters, and the
profile summary written from synthetic counter files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from attention_forward_06_amd.inputs import WORKLOADS  # noqa: E402


@pytest.mark.parametrize("mode", ["none", "causal", "block_diag"])
def test_visible_pairs_counts_the_mask(mode):
    # brute-force count of the (query, key) pairs each mode keeps
    for L in range(1, 13):
        for bs in [b for b in range(1, L + 1) if L % b == 0] if mode == "block_diag" else [0]:
            keep = {"none": lambda i, j: True,
                    "causal": lambda i, j: j <= i,
                    "block_diag": lambda i, j: i // bs == j // bs}[mode]
            n = sum(1 for i in range(L) for j in range(L) if keep(i, j))
            assert bench.visible_pairs(mode, L, bs) == n


def test_kernel_of_names_the_launched_instance():
    dt_code = {"f16": 0, "bf16": 1, "bf16_v_e5m2": 2, "f16_v_e5m2": 3}
    mode_code = {"none": 0, "causal": 1, "block_diag": 2}
    for n in bench.BENCH_WORKLOADS:
        w = WORKLOADS[n]
        name, grid = bench.kernel_of(n)
        if w["D"] <= 64 and w["mode"] != "block_diag":
            # 64 query rows per wave: one 256-thread workgroup per 256 query rows
            assert name == f"attn_fwd_rows64_kernel<{w['D']}, {dt_code[w['dtype']]}, {mode_code[w['mode']]}, false>"
            assert grid == -(-w["L"] // 256) * w["B"] * w["H"] * 256
            continue
        bn, kw = (128, w["block_size"]) if w["mode"] == "block_diag" else (64, 64)
        assert name == (f"attn_fwd_kernel<{w['D']}, {dt_code[w['dtype']]}, {mode_code[w['mode']]}, 4, "
                        f"{bn}, {kw}, false>")
        # one 256-thread workgroup per 128 query rows of every (batch, head)
        assert grid == -(-w["L"] // 128) * w["B"] * w["H"] * 256
    assert bench.kernel_of(bench.HEADLINE) == ("attn_fwd_kernel<128, 1, 1, 4, 64, 64, false>", 32 * 128 * 256)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_source_digest_ignores_comments_and_layout(tmp_path, monkeypatch):
    a, b, c = tmp_path / "a.h", tmp_path / "b.h", tmp_path / "c.h"
    a.write_text("int x = 1;  // one\n/* block\n comment */ int y;\n")
    b.write_text("int x = 1;\n\n   int y;   // other words\n")
    c.write_text("int x = 2;\nint y;\n")
    digest = lambda p: (monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(p)]), bench.source_digest())[1]
    assert digest(a) == digest(b)
    assert digest(a) != digest(c)
    assert len(digest(a)) == 64


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)


def test_summary_from_synthetic_counters(tmp_path):
    name = bench.HEADLINE
    kname, grid = bench.kernel_of(name)
    full = f"void (anonymous namespace)::{kname}(Params)"
    copy = "__amd_rocclr_copyBuffer"
    d = tmp_path / "run"

    def pmc(pass_name, values, copy_values=None):
        rows = [{"Kernel_Name": full, "Grid_Size": grid, "Counter_Name": c, "Counter_Value": v}
                for c, v in values.items()]
        for c, v in (copy_values or {}).items():
            rows.append({"Kernel_Name": copy, "Grid_Size": 1 << 20, "Counter_Name": c, "Counter_Value": v})
        _write_csv(str(d / pass_name / "run_counter_collection.csv"), rows)

    # a 1 GiB copy reads FETCH_SIZE = 512 MiB-in-KiB and writes the full 1 GiB: scales x2, x1
    pmc("pmc_fetch", {"FETCH_SIZE": 300000.0}, {"FETCH_SIZE": 524288.0})
    pmc("pmc_write", {"WRITE_SIZE": 131072.0}, {"WRITE_SIZE": 1048576.0})
    gui = 8 * 1_000_000.0
    pmc("pmc_mfma", {"SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1_000_000 * 1024, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1.0e9,
                     "SQ_INSTS_VALU_MFMA_MOPS_F16": 0.0, "SQ_INSTS_VALU_MFMA_MOPS_F8": 0.0, "GRBM_GUI_ACTIVE": gui})
    pmc("pmc_lds", {"SQ_LDS_BANK_CONFLICT": 0.0, "SQ_LDS_IDX_ACTIVE": 2.56e7, "SQ_INSTS_VALU": 6.0e6,
                    "SQ_INSTS_LDS": 1.5e6, "SQ_INSTS_MFMA": 1.0e6, "SQ_WAVE_CYCLES": 4.0e8, "GRBM_GUI_ACTIVE": gui})
    trace = [{"Kernel_Name": full, "Grid_Size_X": grid, "Start_Timestamp": 1000 * i,
              "End_Timestamp": 1000 * i + 500_000 + i} for i in range(40)]
    _write_csv(str(d / "prof_trace" / "run_kernel_trace.csv"), trace)
    _write_csv(str(d / "prof_trace" / "run_kernel_stats.csv"),
               [{"Name": full, "Calls": 40, "AverageNs": 500_020.0}, {"Name": copy, "Calls": 3, "AverageNs": 17_000.0}])

    out = tmp_path / "out"
    out.mkdir()
    bench.summarize_profiles(str(d), out=str(out))

    t = json.loads((out / "traffic.json").read_text())
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["kernel_source_sha256"] == bench.source_digest()
    row = t["workloads"][name]
    assert row["hbm_bytes_per_launch"] == round((300000.0 * 2 + 131072.0) * 1024)
    w = WORKLOADS[name]
    assert row["algorithmic_bytes"] == w["B"] * w["H"] * w["L"] * w["D"] * 8
    # only the workload with counters is listed
    assert set(t["workloads"]) == {name}
    trace_md = (out / "attn_fwd_kernel_trace_all_workloads.md").read_text()
    assert name in trace_md and "| 40 |" in trace_md
    counters_md = (out / "attn_fwd_mfma_lds_counters_all_workloads.md").read_text()
    assert "50.0%" in counters_md          # MFMA busy = busy cycles / (GUI clocks x 1024 SIMDs)
    assert (out / "attn_fwd_hbm_traffic_all_workloads.md").exists()
    # the stall passes are optional: no summary without them
    assert not (out / "attn_fwd_issue_and_wait_counters_all_workloads.md").exists()
