"""Host logic of the profile summaries: synthetic rocprofv3 CSVs in the
tool's column layout, summarised into a scratch directory, and the derived
figures checked against hand-computed values (launch means over the timed
launches, the byte counters scaled by the calibration copy, the matrix-core
counters over the algorithmic flops)."""

import csv
import json

import pytest

import bench
from paged_kv_cache_412_amd import profiling, workloads

KERNEL = "void pa::decode_mfma_kernel<2, 2, 128, 16, 2>(pa::DecodeParams)"
REDUCE = "void pa::decode_reduce_kernel<true, 2, 1>(pa::DecodeParams)"
COPY = "__amd_rocclr_copyBuffer"
COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Kernel_Name", "Counter_Name",
                "Counter_Value"]


def write_csv(path, cols, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols, quoting=csv.QUOTE_NONNUMERIC)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def counters(path, name, per_dispatch, kernel=KERNEL, split=1):
    """One row per (dispatch, instance); each dispatch's value split evenly
    over `split` instances, as rocprofv3 reports per-instance values."""
    rows, cid = [], 0
    for d, v in enumerate(per_dispatch):
        for _ in range(split):
            cid += 1
            rows.append({"Correlation_Id": cid, "Dispatch_Id": d + 1, "Agent_Id": "Agent 1",
                         "Kernel_Name": kernel, "Counter_Name": name, "Counter_Value": v / split})
    write_csv(path, COUNTER_COLS, rows)


@pytest.fixture
def runs(tmp_path, monkeypatch):
    d = tmp_path / "prof"
    d.mkdir()
    out = tmp_path / "profiles"
    monkeypatch.setattr(profiling, "PROFILES", str(out))
    w = "llama70b"
    # kernel trace: the warm-up launches at 700 us, then the 50 timed ones at 640 us
    S, W = profiling.STEPS, profiling.WARMUP
    durs = [700.0] * W + [640.0] * S
    rows, t = [], 1_000_000
    for i, us in enumerate(durs):
        rows.append({"Kernel_Name": KERNEL, "Start_Timestamp": t, "End_Timestamp": t + int(us * 1e3)})
        t += int(us * 1e3) + 5_000
        rows.append({"Kernel_Name": REDUCE, "Start_Timestamp": t, "End_Timestamp": t + 4_000})
        t += 10_000
    write_csv(d / f"trace_{w}_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    total = sum(durs) * 1e3
    write_csv(d / f"trace_{w}_kernel_stats.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"],
              [{"Name": KERNEL, "Calls": len(durs), "TotalDurationNs": total,
                "AverageNs": total / len(durs), "Percentage": 99.0},
               {"Name": REDUCE, "Calls": len(durs), "TotalDurationNs": 4000.0 * len(durs),
                "AverageNs": 4000.0, "Percentage": 1.0}])
    # byte counters (KiB per dispatch): the calibration copy of 1 GiB reads
    # half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    counters(d / f"pmc_FETCH_SIZE_{w}_counter_collection.csv", "FETCH_SIZE", [2.0e6, 2.2e6, 2.4e6], split=16)
    counters(d / f"pmc_WRITE_SIZE_{w}_counter_collection.csv", "WRITE_SIZE", [1.0e3, 3.0e3, 2.0e3], split=16)
    gib_kib = bench.CALIBRATION_BYTES / 1024
    counters(d / "pmc_FETCH_SIZE_calibration_counter_collection.csv", "FETCH_SIZE", [gib_kib / 2] * 3, COPY)
    counters(d / "pmc_WRITE_SIZE_calibration_counter_collection.csv", "WRITE_SIZE", [gib_kib] * 3, COPY)
    alg = profiling.bench_decode_flops(workloads.CONFIGS[w])
    counters(d / f"pmc_MfmaUtil_{w}_counter_collection.csv", "MfmaUtil", [6.0, 7.0, 8.0])
    counters(d / f"pmc_MfmaFlops_{w}_counter_collection.csv", "MfmaFlops", [2.0 * alg] * 3)
    # where the time goes: 1000 wave-cycles split 350 issuing / 400 waiting
    # for a slot / 250 on a dependency; 8 XCDs of 1000 cycles; the matrix
    # cores of 1024 SIMDs busy 40 %, a quarter of that beside vector issue
    pipe = {"SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 250.0, "SQ_WAIT_INST_LDS": 30.0,
            "SQ_ACTIVE_INST_LDS": 40.0, "SQ_LDS_IDX_ACTIVE": 200.0, "SQ_LDS_BANK_CONFLICT": 20.0,
            "LdsUtil": 19.0, "VALUBusy": 40.0, "SQ_ACTIVE_INST_ANY": 350.0, "SQ_WAIT_INST_ANY": 400.0,
            "GRBM_GUI_ACTIVE": 8000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 409600.0,
            "SQ_VALU_MFMA_COEXEC_CYCLES": 102400.0, "SQ_INSTS_MFMA": 25600.0, "SQ_INSTS_VALU": 1.0e5,
            "SQ_INSTS_VALU_TRANS_F32": 1.0e4}
    assert set(pipe) == set(profiling.PIPE_COUNTERS + profiling.ISSUE_COUNTERS)
    for name, v in pipe.items():
        counters(d / f"pmc_{name}_{w}_counter_collection.csv", name, [v] * 3, split=4)
    profiling.summarize(w, str(d))
    rec = json.loads((out / f"traffic_decode_mfma_kernel_{w}.json").read_text())
    md = (out / f"decode_mfma_kernel_{w}.md").read_text()
    return rec, md, alg


def test_summary_launch_means(runs):
    rec, md, _ = runs
    assert rec["timed_avg_launch_us"] == pytest.approx(640.0)
    assert rec["avg_launch_us"] == pytest.approx((700.0 * profiling.WARMUP + 640.0 * profiling.STEPS)
                                                 / (profiling.WARMUP + profiling.STEPS))
    kv = profiling.bench_kv_bytes(workloads.CONFIGS["llama70b"])
    assert f"{kv / 640e-6 / 1e9:.1f} GB/s" in md


def test_summary_scales_the_byte_counters(runs):
    rec, md, _ = runs
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    assert rec["fetch_kib_per_launch"] == pytest.approx(2.2e6)   # instances summed per dispatch
    assert rec["write_kib_per_launch"] == pytest.approx(2.0e3)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(2.2e6 * 1024 * 2 + 2.0e3 * 1024)
    assert rec["kernel_hash"] == bench.kernel_hash("decode_mfma_kernel")


def test_summary_matrix_core_counters(runs):
    rec, md, alg = runs
    assert rec["mfma_util_pct"] == pytest.approx(7.0)
    assert rec["algorithmic_flops"] == alg
    assert rec["mfma_flops_per_launch"] / alg == pytest.approx(2.0)
    assert "| issued / algorithmic | 2.000 |" in md


def test_bench_reads_back_the_record(runs, monkeypatch, tmp_path):
    rec, _, _ = runs
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path / "profiles"))
    assert bench.measured_traffic("decode_mfma_kernel", "llama70b") == pytest.approx(rec["hbm_bytes_per_launch"])
    m = bench.measured_mfma("decode_mfma_kernel", "llama70b")
    assert m["busy_pct"] == 7.0 and m["issued_over_algorithmic"] == 2.0
    # a record taken on other kernel sources is not reported
    p = tmp_path / "profiles" / "traffic_decode_mfma_kernel_llama70b.json"
    stale = dict(rec, kernel_hash="0" * 16)
    p.write_text(json.dumps(stale))
    assert bench.measured_traffic("decode_mfma_kernel", "llama70b") is None
    assert bench.measured_mfma("decode_mfma_kernel", "llama70b") is None


def test_summary_pipe_and_issue_counters(runs):
    rec, md, _ = runs
    assert rec["pipe"]["SQ_WAVE_CYCLES"] == pytest.approx(1000.0)   # instances summed per dispatch
    assert "| 10.0 % of LDS active cycles |" in md                  # bank conflicts 20 of 200
    shares = [float(x) for x in
              [md.split(f"| {c}")[1].split("|")[2].split("%")[0] for c in
               ("SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY (above)")]]
    assert shares == [35.0, 40.0, 25.0] and sum(shares) == pytest.approx(100.0)
    assert "| 1000 cycles per XCD |" in md
    assert "| 40.0 % of SIMD cycles |" in md
    assert "| 25.0 % of matrix-core busy cycles |" in md
    assert "| 16.0 busy cycles each |" in md
    assert rec["issue"]["SQ_INSTS_VALU_TRANS_F32"] == pytest.approx(1.0e4)
