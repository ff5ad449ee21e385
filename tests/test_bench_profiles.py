"""The profile summariser of bench.py on small synthetic rocprofv3 CSV files
(no GPU): kinds are taken in order of first appearance, counters are scaled by
the 1 GiB copy, and the traffic record carries the current qmm.hip digest."""
import csv
import hashlib
import json
import os

import bench
from speculative_decoding_verify_vq_amd.stack import StackConfig, qmm_algorithmic_bytes

QMM = "void vq::(anonymous namespace)::qmm_kernel<4, 4, 2, {e}, {n}, {c}>(vq::(anonymous namespace)::QmmArgs)"
KINDS = [("qkv", QMM.format(e=0, n="true", c="false"), (64, 7)), ("o", QMM.format(e=1, n="false", c="false"), (40, 12)),
         ("gate_up", QMM.format(e=2, n="true", c="false"), (272, 5)),
         ("down", QMM.format(e=1, n="false", c="false"), (40, 17)),
         ("lm_head", QMM.format(e=0, n="true", c="true"), (1940, 1))]
COPY = "__amd_rocclr_copyBuffer"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _make(tmp):
    stats_h = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]
    _write(os.path.join(tmp, "kt", "kt_kernel_stats.csv"), stats_h,
           [[name, 10, 10000.0 * (i + 1), 1000.0 * (i + 1), 10.0, 900.0, 1100.0, 1.0]
            for i, (_, name, _) in enumerate(KINDS)])
    trace_h = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X",
               "Grid_Size_Y"]
    rows = []
    for rep in range(2):
        for i, (_, name, (gx, gy)) in enumerate(KINDS):
            rows.append(["KERNEL_DISPATCH", name, 0, 1000 * (i + 1), 256, gx * 256, gy])
    _write(os.path.join(tmp, "kt", "kt_kernel_trace.csv"), trace_h, rows)
    ctr_h = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    for ctr, sub, copy_val in (("FETCH_SIZE", "fetch", 524288.0), ("WRITE_SIZE", "write", 1048576.0)):
        rows = [[COPY, 131072, ctr, copy_val]]
        for rep in range(3):
            for i, (_, name, (gx, gy)) in enumerate(KINDS):
                rows.append([name, gx * gy * 256, ctr, 100.0 * (i + 1)])
        _write(os.path.join(tmp, sub, f"{sub}_counter_collection.csv"), ctr_h, rows)
    with open(os.path.join(tmp, "kt.out"), "w") as f:
        f.write("[bench] log line\n")
        f.write(json.dumps({"ms_per_step": 4.7, "value": 3000.0, "roofline": {
            "avg_launch_us": 16.0, "per_kind": {k: {"us": 1.0} for k, _, _ in KINDS}}}) + "\n")


def test_summarize_profiles(tmp_path):
    prof, out = str(tmp_path / "prof"), str(tmp_path / "out")
    os.makedirs(out)
    _make(prof)
    bench.summarize_profiles(prof, out, "cmd-kt", "cmd-fetch", "cmd-write")
    rec = json.load(open(os.path.join(out, "qmm_traffic_4bit_M4.json")))
    assert abs(rec["fetch_scale"] - 2.0) < 1e-9 and abs(rec["write_scale"] - 1.0) < 1e-9
    cfg = StackConfig()
    sh = cfg.shapes()
    tot = 0
    for i, (kind, _, _) in enumerate(KINDS):
        r = rec["per_kind"][kind]
        # FETCH counts are scaled by 2, WRITE by 1; counters are KiB
        assert r["hbm_bytes"] == 1024 * (2 * 100 * (i + 1) + 100 * (i + 1))
        out_b = {"qkv": 2, "o": 4, "gate_up": 1, "down": 4, "lm_head": 4}[kind]
        assert r["algorithmic_bytes"] == qmm_algorithmic_bytes(cfg.M, *sh[kind], cfg.bits, out_bytes=out_b)
        assert r["dispatches"] == 3
        tot += rec["step_launch_counts"][kind] * r["hbm_bytes"]
    assert rec["hbm_bytes_per_launch"] == int(tot / 257)
    src = os.path.join(bench.ROOT, "speculative_decoding_verify_vq_amd", "csrc", "qmm.hip")
    assert rec["qmm_hip_sha256"] == hashlib.sha256(open(src, "rb").read()).hexdigest()
    kt = open(os.path.join(out, "qmm_kernel_verify_step_4bit_M4.md")).read()
    # trace averages: kind i lasts (i + 1) us; weighted by 64, 64, 64, 64, 1
    want = (64 * (1 + 2 + 3 + 4) + 5) / 257
    assert f"{want:.2f} us" in kt and "cmd-kt" in kt
    assert "| gate_up | 64 |" in open(os.path.join(out, "qmm_traffic_4bit_M4.md")).read()


def test_summarize_curve_counters(tmp_path):
    """Per-width counter summary: CURVE_PACKS dispatches per width, in order."""
    prof, out = str(tmp_path / "prof"), str(tmp_path / "out")
    os.makedirs(out)
    name = QMM.format(e=0, n="false", c="false")
    ctr_h = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    for ctr, sub, copy_val in (("FETCH_SIZE", "fetch", 524288.0), ("WRITE_SIZE", "write", 1048576.0)):
        rows = [[COPY, 131072, ctr, copy_val]]
        for i, m in enumerate(bench.CURVE_MS):
            rows += [[name, 136 * 5 * 256, ctr, 1000.0 + 10 * i]] * bench.CURVE_PACKS
        _write(os.path.join(prof, sub, f"{sub}_counter_collection.csv"), ctr_h, rows)
    bench.summarize_curve_counters(prof, out, 4, "f", "w")
    md = open(os.path.join(out, "qmm_traffic_by_M_4bit.md")).read()
    # width 3 (index 2): fetch 1020 KiB x 2 + write 1020 KiB x 1
    assert f"| 3 | 1020.0 | 1020.0 | {1024 * 3 * 1020} |" in md


def test_summarize_profiles_config4(tmp_path):
    """The 8-bit M=8 step: the same summaries under the configuration's tag, with
    its own algorithmic bytes."""
    prof, out = str(tmp_path / "prof"), str(tmp_path / "out")
    os.makedirs(out)
    _make(prof)
    bench.summarize_profiles(prof, out, "cmd-kt", "cmd-fetch", "cmd-write", 4)
    rec = json.load(open(os.path.join(out, "qmm_traffic_8bit_M8.json")))
    assert rec["bits"] == 8 and rec["M"] == 8
    cfg = StackConfig(bits=8, lm_bits=8, M=8)
    assert rec["per_kind"]["o"]["algorithmic_bytes"] == qmm_algorithmic_bytes(8, 5120, 6144, 8, out_bytes=4)
    assert os.path.exists(os.path.join(out, "qmm_kernel_verify_step_8bit_M8.md"))
    assert "| down | 64 |" in open(os.path.join(out, "qmm_traffic_8bit_M8.md")).read()
    assert cfg.M == 8


def test_summarize_attn_counters(tmp_path):
    """Attention counter summary: partial + combine dispatches per call, in width order."""
    prof, out = str(tmp_path / "prof"), str(tmp_path / "out")
    os.makedirs(out)
    part = "void vq::(anonymous namespace)::attn_partial_kernel<256, 2, false>(unsigned short const*)"
    comb = "void vq::(anonymous namespace)::attn_combine_kernel(float const*)"
    ctr_h = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    for ctr, sub, copy_val in (("FETCH_SIZE", "fetch", 524288.0), ("WRITE_SIZE", "write", 1048576.0)):
        rows = [[COPY, 131072, ctr, copy_val]]
        for i, m in enumerate(bench.ATTN_MS):
            for _ in range(bench.ATTN_COUNTER_CACHES):
                rows += [[part, 512 * 256, ctr, 1000.0 + 10 * i], [comb, 96 * 256, ctr, 5.0]]
        _write(os.path.join(prof, sub, f"{sub}_counter_collection.csv"), ctr_h, rows)
    bench.summarize_attn_counters(prof, out, "f", "w")
    md = open(os.path.join(out, "attn_traffic_by_M_32k.md")).read()
    # width 2 (index 1): fetch (1010 + 5) KiB x 2 + write (1010 + 5) KiB x 1
    assert f"| 2 | 1015.0 | 1015.0 | {1024 * 3 * 1015} |" in md
