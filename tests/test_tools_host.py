"""Host logic of the measurement tools (no GPU): bench.py's argument handling and the
arithmetic of profile_summary.py's summaries on small synthetic rocprofv3 CSV files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_py(*args):
    return subprocess.run([sys.executable, *args], cwd=ROOT, capture_output=True, text=True, timeout=120)


def test_bench_refuses_more_than_one_gpu():
    r = run_py("bench.py", "--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_rejects_unknown_secondary_workload():
    r = run_py("bench.py", "--secondary", "zigzag_rank3,nonsense")
    assert r.returncode == 2
    assert "nonsense" in r.stderr


TRACE_FIELDS = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]
PMC_FIELDS = ["Dispatch_Id", "Agent_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
              "Start_Timestamp", "End_Timestamp"]


def write_csv(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def trace_rows(spec):
    """spec: list of (kernel, grid, duration ns); dispatches back to back in that order."""
    rows, t = [], 0
    for i, (k, g, d) in enumerate(spec, start=1):
        rows.append({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": i, "Kernel_Name": k, "Start_Timestamp": t,
                     "End_Timestamp": t + d, "Grid_Size_X": g})
        t += d + 10
    return rows


def test_trace_groups_by_kernel_grid_and_run_order(tmp_path):
    k = "void ra::(anonymous namespace)::attn_bf16_kernel<128, OutBf16>(ra::AttnArgs)"
    spec = [(k, 1024, 3_000_000), (k, 1024, 5_000_000), ("copy", 64, 1000), (k, 1024, 2_000_000),
            (k, 1024, 4_000_000), (k, 256, 1_000_000)]
    write_csv(tmp_path / "kt.csv", TRACE_FIELDS, trace_rows(spec))
    out = tmp_path / "t.md"
    r = run_py("profile_summary.py", "trace", str(tmp_path / "kt.csv"), "--out", str(out), "--title", "T",
               "--cmd", "C", "--split", "attn_bf16_kernel<128, OutBf16>@1024=first,second")
    assert r.returncode == 0, r.stderr
    rows = {tuple(c.strip() for c in line.split("|")[1:4]): line for line in out.read_text().splitlines()
            if line.startswith("| attn")}
    first = rows[("attn_bf16_kernel<128, OutBf16>", "1024", "first")].split("|")
    second = rows[("attn_bf16_kernel<128, OutBf16>", "1024", "second")].split("|")
    assert first[4].strip() == "2" and float(first[5]) == pytest.approx(4.0)  # (3 + 5) / 2 ms
    assert second[4].strip() == "2" and float(second[5]) == pytest.approx(3.0)  # (2 + 4) / 2 ms
    assert ("attn_bf16_kernel<128, OutBf16>", "256", "") in rows


def test_trace_reports_the_last_calls_of_a_run(tmp_path):
    # a benchmark's warm-up calls come first: --last reports the timed calls on their own row
    k = "void ra::(anonymous namespace)::attn_bf16_kernel<128, OutBf16>(ra::AttnArgs)"
    spec = [(k, 1024, 9_000_000), (k, 1024, 3_000_000), (k, 1024, 5_000_000)]
    write_csv(tmp_path / "kt.csv", TRACE_FIELDS, trace_rows(spec))
    out = tmp_path / "t.md"
    r = run_py("profile_summary.py", "trace", str(tmp_path / "kt.csv"), "--out", str(out), "--title", "T",
               "--cmd", "C", "--split", "attn_bf16_kernel<128, OutBf16>@1024=bench",
               "--last", "attn_bf16_kernel<128, OutBf16>@1024=bench:2")
    assert r.returncode == 0, r.stderr
    rows = {tuple(c.strip() for c in line.split("|")[1:4]): line.split("|") for line in out.read_text().splitlines()
            if line.startswith("| attn")}
    allr = rows[("attn_bf16_kernel<128, OutBf16>", "1024", "bench")]
    last = rows[("attn_bf16_kernel<128, OutBf16>", "1024", "bench, last 2 calls")]
    assert allr[4].strip() == "3" and float(allr[5]) == pytest.approx(17.0 / 3, abs=1e-3)
    assert last[4].strip() == "2" and float(last[5]) == pytest.approx(4.0)   # (3 + 5) / 2 ms
    assert float(last[6]) == pytest.approx(3.0) and float(last[7]) == pytest.approx(5.0)


def pmc_rows(spec, counter):
    """spec: list of (kernel, grid, value); one row per dispatch for ``counter``."""
    return [{"Dispatch_Id": i, "Agent_Id": "Agent 1", "Kernel_Name": k, "Grid_Size": g, "Counter_Name": counter,
             "Counter_Value": v, "Start_Timestamp": 0, "End_Timestamp": 1}
            for i, (k, g, v) in enumerate(spec, start=1)]


def test_hbm_scales_counters_by_the_plain_copy(tmp_path):
    copy, perm = "__amd_rocclr_copyBuffer", "void ra::(anonymous namespace)::permute_kernel<16>(char const*)"
    mib64 = 64 << 20
    # trace: the copy and the permute each take 25 us
    write_csv(tmp_path / "kt.csv", TRACE_FIELDS,
              trace_rows([(copy, 131072, 25_000), (perm, 4096, 25_000), (perm, 4096, 25_000)]))
    # the counters see half the copy's reads (FETCH_SIZE) and all of its writes, in KiB
    write_csv(tmp_path / "f.csv", PMC_FIELDS,
              pmc_rows([(copy, 131072, mib64 / 2048), (perm, 4096, mib64 / 2048), (perm, 4096, mib64 / 2048)],
                       "FETCH_SIZE"))
    write_csv(tmp_path / "w.csv", PMC_FIELDS,
              pmc_rows([(copy, 131072, mib64 / 1024), (perm, 4096, mib64 / 1024), (perm, 4096, mib64 / 1024)],
                       "WRITE_SIZE"))
    out = tmp_path / "h.md"
    r = run_py("profile_summary.py", "hbm", "--trace", str(tmp_path / "kt.csv"), "--fetch", str(tmp_path / "f.csv"),
               "--write", str(tmp_path / "w.csv"), "--calib", f"{copy}@131072={mib64}",
               "--kernel", f"permute_kernel<16>@4096=:{2 * mib64}", "--title", "T", "--cmd", "C", "--out", str(out))
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    assert "FETCH_SIZE x 2.0000, WRITE_SIZE x 1.0000" in text
    row = [line for line in text.splitlines() if line.startswith("| permute_kernel")][0].split("|")
    assert float(row[4]) == pytest.approx(0.025)                       # ms
    assert float(row[6]) == pytest.approx(2 * mib64 / 25e-6 / 1e9, rel=1e-3)  # algorithmic GB/s
    assert float(row[10]) == pytest.approx(1.0, abs=1e-3)               # counted / algorithmic


def test_traffic_json_from_counters(tmp_path):
    copy, attn = "__amd_rocclr_copyBuffer", "void ra::(anonymous namespace)::attn_bf16_kernel<128, OutBf16>(x)"
    mib64 = 64 << 20
    write_csv(tmp_path / "f.csv", PMC_FIELDS,
              pmc_rows([(attn, 1024, 1000.0), (copy, 131072, mib64 / 2048), (attn, 1024, 3000.0)], "FETCH_SIZE"))
    write_csv(tmp_path / "w.csv", PMC_FIELDS,
              pmc_rows([(attn, 1024, 10.0), (copy, 131072, mib64 / 1024), (attn, 1024, 30.0)], "WRITE_SIZE"))
    src = tmp_path / "k.hip"
    src.write_text("kernel source")
    out = tmp_path / "t.json"
    r = run_py("profile_summary.py", "traffic", "--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
               "--kernel", "attn_bf16_kernel", "--grid", "1024", "--calib-kernel", copy, "--calib-grid", "131072",
               "--calib-bytes", str(mib64), "--src", str(src), "--cmd", "C", "--out", str(out))
    assert r.returncode == 0, r.stderr
    t = json.loads(out.read_text())
    assert t["fetch_bytes"] == round(2000.0 * 1024 * 2)  # mean KiB x 1024 x fetch factor 2
    assert t["write_bytes"] == round(20.0 * 1024)
    assert t["bytes_per_launch"] == t["fetch_bytes"] + t["write_bytes"]
    assert len(t["kernel_sha256_16"]) == 16


def test_short_names_of_mangled_template_kernels():
    # the tracer leaves kernels with a __bf16 parameter mangled; the summaries show them by name
    sys.path.insert(0, ROOT)
    import profile_summary as ps
    assert ps._short("_ZN2ra12_GLOBAL__N_112delta_kernelILi128EEEvPKDF16bS3_PKfPfS6_lll") == "delta_kernel<128>"
    assert ps._short("_ZN2ra12_GLOBAL__N_112delta_kernelILi64EEEvPKDF16bS3_PKfPfS6_lll") == "delta_kernel<64>"
    assert ps._short("void ra::(anonymous namespace)::dq_kernel<128>(ra::BwdArgs)") == "dq_kernel<128>"
    assert ps._short("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_grid_of_a_dispatch_counts_every_dimension():
    # a multi-tensor launch puts the tensor in blockIdx.y: its trace row must not share a grid
    # key with the one-tensor launch of the same x extent
    sys.path.insert(0, ROOT)
    import profile_summary as ps
    assert ps._grid({"Grid_Size_X": "4194304", "Grid_Size_Y": "3", "Grid_Size_Z": "1"}) == 12582912
    assert ps._grid({"Grid_Size_X": "4194304"}) == 4194304
    assert ps._grid({"Grid_Size": "12582912"}) == 12582912
