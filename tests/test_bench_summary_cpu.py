"""bench.py's profile summarizer on a synthetic rocprofv3 output (no GPU):
kernel times, the achieved rate over the algorithmic bytes, counter bytes
scaled by the calibration copy, and the traffic file that bench.py reads
back only while its kernel-source hash matches."""

import csv
import os

import pytest

import bench

KERNEL = "fold_table_kernel<4, OpSumI32, 1, true>"  # 8 KiB per workgroup
MANGLED = f"void rc::(anonymous namespace)::{KERNEL}(rc::FoldTable)"
COPY = "__amd_rocclr_copyBuffer"
WGS = 65_536  # 4 jobs x 16,384 tiles: 536,870,912 algorithmic bytes per launch


def write_csv(path, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def fake_run(tmp_path, fetch_kib, write_kib, copy_fetch_kib, copy_write_kib, durations_us):
    d = tmp_path / "prof"
    t, trace = 0, []
    for us in durations_us:
        trace.append({"Kernel_Name": MANGLED, "Start_Timestamp": t, "End_Timestamp": t + int(us * 1000),
                      "Grid_Size_X": 64 * WGS // 4, "Grid_Size_Y": 4, "Grid_Size_Z": 1,
                      "Workgroup_Size_X": 64, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1})
        t += int(us * 1000) + 5000
    trace.append({"Kernel_Name": COPY, "Start_Timestamp": t, "End_Timestamp": t + 200_000,
                  "Grid_Size_X": 1 << 20, "Grid_Size_Y": 1, "Grid_Size_Z": 1,
                  "Workgroup_Size_X": 256, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1})
    write_csv(d / "trace" / "x" / "run_kernel_trace.csv", trace)
    for ctr, sub, v, cv in (("FETCH_SIZE", "fetch", fetch_kib, copy_fetch_kib),
                            ("WRITE_SIZE", "write", write_kib, copy_write_kib)):
        rows = [{"Kernel_Name": MANGLED, "Counter_Name": ctr, "Counter_Value": v, "Grid_Size": 64 * WGS}
                for _ in durations_us]
        rows.append({"Kernel_Name": COPY, "Counter_Name": ctr, "Counter_Value": cv, "Grid_Size": 1 << 20})
        write_csv(d / sub / "x" / "run_counter_collection.csv", rows)
    return d


@pytest.fixture
def profiles(tmp_path, monkeypatch):
    out = tmp_path / "profiles"
    monkeypatch.setattr(bench, "PROFILES", out)
    return out


def test_summary_rates_and_scaled_traffic(tmp_path, profiles):
    # FETCH_SIZE counts half the bytes read (the copy's 512 MiB read as 256 MiB)
    d = fake_run(tmp_path, fetch_kib=131_072, write_kib=262_144, copy_fetch_kib=262_144,
                 copy_write_kib=524_288, durations_us=[100.0] * 18 + [81.4] * 30)
    bench.summarize_profile(d, "int32_r4_64MiB")
    md = (profiles / "int32_r4_64MiB_kernel_stats.md").read_text()
    row = next(line for line in md.splitlines() if line.startswith(f"| `{KERNEL}`"))
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "48"                  # every launch counted
    assert cells[5] == "30" and cells[6] == "81.4"   # the steady launches only
    assert cells[7] == "536870912"           # 8 KiB x 65,536 workgroups
    gbps = 536_870_912 / 81.4e-6 / 1e9
    assert cells[8] == f"{gbps:.1f}" and cells[9] == f"{100 * gbps / 8000:.1f}%"
    assert cells[10] == "1.0000"             # 2 x 128 MiB fetched + 256 MiB written
    tr = (profiles / "traffic_int32_r4_64MiB.txt").read_text()
    assert "fetch_scale = 2.000000" in tr and "write_scale = 1.000000" in tr
    assert f"{KERNEL}.fetch_bytes_per_launch = 268435456" in tr
    assert f"{KERNEL}.write_bytes_per_launch = 268435456" in tr
    assert f"kernels_sha256 = {bench.kernels_sha()}" in tr
    # bench.py reads the traffic back for the current sources only
    path = profiles / "traffic_int32_r4_64MiB.txt"
    assert bench.read_traffic_file(path, KERNEL) == 536_870_912
    path.write_text(tr.replace(bench.kernels_sha(), "0" * 64))
    assert bench.read_traffic_file(path, KERNEL) is None


def test_summary_without_calibration_copy_reports_no_traffic(tmp_path, profiles):
    d = fake_run(tmp_path, fetch_kib=131_072, write_kib=262_144, copy_fetch_kib=0, copy_write_kib=0,
                 durations_us=[81.4] * 30)
    bench.summarize_profile(d, "int32_r4_64MiB")
    tr = (profiles / "traffic_int32_r4_64MiB.txt").read_text()
    assert "fetch_scale = none" in tr and f"{KERNEL}.fetch_bytes_per_launch" not in tr
    assert bench.read_traffic_file(profiles / "traffic_int32_r4_64MiB.txt", KERNEL) is None


def test_summary_commands_name_the_given_folder(tmp_path, profiles):
    d = fake_run(tmp_path, 1, 1, 1, 1, [10.0] * 4)
    bench.summarize_profile(d, "int32_r4_64MiB")
    md = (profiles / "int32_r4_64MiB_kernel_stats.md").read_text()
    rel = os.path.relpath(d, bench.ROOT)  # commands run from the repository root
    for sub in ("trace", "fetch", "write"):
        assert f"-d $OLDPWD/{rel}/{sub} -o run -- python3 $OLDPWD/bench.py --profile int32_r4_64MiB" in md
    assert f"--summarize-profile {rel} --profile int32_r4_64MiB" in md
