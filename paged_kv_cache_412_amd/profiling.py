"""rocprofv3 runs of bench.py and the summaries kept under ``profiles/``.

Three steps, run from the repository root:

``python -m paged_kv_cache_412_amd.profiling trace --workload W --out DIR``
    (GPU) ``rocprofv3 --kernel-trace --stats -f csv`` around a short bench.py
    run of workload W.
``python -m paged_kv_cache_412_amd.profiling pmc --workload W --out DIR``
    (GPU) four ``rocprofv3 --pmc`` passes, one counter each: FETCH_SIZE and
    WRITE_SIZE around the same bench.py run, and around
    ``bench.py --copy-calibration`` (a plain 1 GiB device copy); with
    ``--no-calibration`` only the first two (``calibration`` takes the other
    two once for several workloads profiled into one DIR).
``python -m paged_kv_cache_412_amd.profiling mfma --workload W --out DIR``
    (GPU) two more ``rocprofv3 --pmc`` passes, one derived counter each:
    ``MfmaUtil`` (matrix-core busy cycles over active cycles times SIMDs, in
    percent) and ``MfmaFlops`` (matrix-core operations issued, 512 flops per
    MOP), for the kernels that run on the matrix cores.
``python -m paged_kv_cache_412_amd.profiling vmem --workload W --out DIR``
    (GPU) one ``rocprofv3 --pmc`` pass per vector-memory counter
    (VMEM_COUNTERS): address-unit busy and stall cycles, vector-L1 stalls,
    vector-memory read instructions, waves, and the GPU busy cycles they are
    shares of.
``python -m paged_kv_cache_412_amd.profiling pipe --workload W --out DIR``
    (GPU) one ``rocprofv3 --pmc`` pass per counter of PIPE_COUNTERS and
    ISSUE_COUNTERS: where the waves' time goes (issuing, waiting for an issue
    slot or on a dependency, LDS issue and bank conflicts, VALU), and how
    often vector instructions issue while the matrix cores are busy.
``python -m paged_kv_cache_412_amd.profiling summarize --workload W --dir DIR``
    (any machine) reads those CSVs and writes
    ``profiles/<kernel>_<workload>.md`` (per-kernel durations; HBM bytes per
    launch and matrix-core activity when those PMC passes are there) and
    ``profiles/traffic_<kernel>_<workload>.json`` (what bench.py reports as
    ``roofline.traffic`` while the kernel sources are unchanged).

FETCH_SIZE and WRITE_SIZE count KiB per dispatch.  Each is scaled by the
factor that makes it read exactly 1 GiB for the calibration copy, so the
figure is in bytes of HBM traffic as a plain copy would count them.
Every rocprofv3 call runs as a child process with the program itself after
``--`` and a hard time limit.
"""

from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
ROCPROF = "rocprofv3"
STEPS, WARMUP = 50, 200         # bench.py's defaults: the profiled run is the bench run
PMC_STEPS, PMC_WARMUP = 3, 1


def _bench_cmd(workload: str, steps: int, warmup: int, extra=()) -> list:
    return [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", workload, "--steps",
            str(steps), "--warmup", str(warmup), "--no-cpu-baseline", "--batches", "0", *extra]


def _run(cmd: list, limit: int) -> None:
    print("[profiling] " + " ".join(cmd), flush=True)
    r = subprocess.run(cmd, timeout=limit)
    if r.returncode != 0:
        raise SystemExit(f"command failed with status {r.returncode}")


def trace(workload: str, out: str) -> None:
    cmd = [ROCPROF, "--kernel-trace", "--stats", "-f", "csv", "-d", out, "-o", f"trace_{workload}",
           "--", *_bench_cmd(workload, STEPS, WARMUP)]
    _run(cmd, 300)


def calibration(out: str) -> None:
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        _run([ROCPROF, "--pmc", counter, "-f", "csv", "-d", out, "-o", f"pmc_{counter}_calibration",
              "--", *_bench_cmd("llama13b", 1, 0, ("--copy-calibration",))], 180)


def pmc(workload: str, out: str, with_calibration: bool = True) -> None:
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        _run([ROCPROF, "--pmc", counter, "-f", "csv", "-d", out, "-o", f"pmc_{counter}_{workload}",
              "--", *_bench_cmd(workload, PMC_STEPS, PMC_WARMUP)], 180)
    if with_calibration:
        calibration(out)


MFMA_COUNTERS = ("MfmaUtil", "MfmaFlops")


def mfma(workload: str, out: str) -> None:
    for counter in MFMA_COUNTERS:
        _run([ROCPROF, "--pmc", counter, "-f", "csv", "-d", out, "-o", f"pmc_{counter}_{workload}",
              "--", *_bench_cmd(workload, PMC_STEPS, PMC_WARMUP)], 180)


# The vector-memory path of the decode kernels: how busy the per-CU address
# unit (TA) is, how often the vector L1 (TCP, "TC" to the TA) holds it up,
# and how many vector-memory read instructions carry the bytes.  One counter
# per pass.  GRBM_GUI_ACTIVE (GPU busy cycles of the dispatch) normalises the
# others: TA_BUSY_avr is already a mean over the TA instances, the *_sum
# counters add up one instance per compute unit.
VMEM_COUNTERS = ("GRBM_GUI_ACTIVE", "TA_BUSY_avr", "TA_ADDR_STALLED_BY_TC_CYCLES_sum",
                 "TA_DATA_STALLED_BY_TC_CYCLES_sum", "TCP_PENDING_STALL_CYCLES_sum",
                 "TCP_TCR_TCP_STALL_CYCLES_sum", "SQ_INSTS_VMEM_RD", "SQ_WAVES")


def vmem(workload: str, out: str) -> None:
    for counter in VMEM_COUNTERS:
        _run([ROCPROF, "--pmc", counter, "-f", "csv", "-d", out, "-o", f"pmc_{counter}_{workload}",
              "--", *_bench_cmd(workload, PMC_STEPS, PMC_WARMUP)], 180)


# Where the waves' time goes (one counter per pass): wave cycles and the
# share of them spent waiting (for anything; for an LDS instruction to
# issue), LDS instruction issue and bank-conflict cycles against the LDS's
# active cycles, and the derived LDS and VALU utilisations.
PIPE_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_LDS",
                 "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "LdsUtil", "VALUBusy")


# Issue and co-execution (one counter per pass, same step): the wave-cycles
# spent issuing, waiting for an issue slot and (SQ_WAIT_ANY above) waiting
# on a dependency, which add up to SQ_WAVE_CYCLES; the matrix cores' busy
# cycles, and those in which a vector instruction issued beside them; the
# instruction mix; and the dispatch's length in cycles for the clock.
ISSUE_COUNTERS = ("SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_VALU_MFMA_BUSY_CYCLES",
                  "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                  "SQ_INSTS_VALU_TRANS_F32", "GRBM_GUI_ACTIVE")


def pipe(workload: str, out: str) -> None:
    for counter in PIPE_COUNTERS + ISSUE_COUNTERS:
        _run([ROCPROF, "--pmc", counter, "-f", "csv", "-d", out, "-o", f"pmc_{counter}_{workload}",
              "--", *_bench_cmd(workload, PMC_STEPS, PMC_WARMUP)], 180)


def _find(d: str, pattern: str):
    hits = sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))
    return hits[-1] if hits else None


def _counter_per_dispatch(path: str, counter: str) -> dict:
    """kernel name -> list of counter values, one per dispatch (summed over
    the counter's instances within a dispatch)."""
    per = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            key = (row["Kernel_Name"], row.get("Dispatch_Id") or row.get("Correlation_Id"))
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def _gpu_shape(agent_info: str):
    """(XCD count, compute-unit count) of the GPU agent in a rocprofv3
    agent-info CSV; (8, 256) when the file is missing."""
    try:
        with open(agent_info, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Agent_Type", "").upper().endswith("GPU"):
                    return int(row["Num_Xcc"]), int(row["Cu_Count"])
    except (OSError, KeyError, ValueError):
        pass
    return 8, 256


def _short(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")


def summarize(workload: str, d: str) -> None:
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (kernel naming and source hash)
    from paged_kv_cache_412_amd import workloads

    cfg = workloads.CONFIGS[workload]
    kernel = bench.decode_kernel_name(cfg)
    stats = _find(d, f"trace_{workload}_kernel_stats.csv")
    if stats is None:
        raise SystemExit(f"no kernel stats for {workload} under {d}")
    with open(stats, newline="") as f:
        rows = list(csv.DictReader(f))
    lines = [f"# {kernel} -- {workload}", "",
             "Kernel durations from `rocprofv3 --kernel-trace --stats` around the bench.py run (no CPU baseline).",
             "", "Commands (repository root, MI355X):", "", "```",
             f"python -m paged_kv_cache_412_amd.profiling trace --workload {workload} --out rocprof_out",
             "  # = " + " ".join([ROCPROF, "--kernel-trace", "--stats", "-f", "csv", "-d", "rocprof_out",
                                   "-o", f"trace_{workload}", "--", "python3", "bench.py", "--workload",
                                   workload, "--steps", str(STEPS), "--warmup", str(WARMUP),
                                   "--no-cpu-baseline"]),
             f"python -m paged_kv_cache_412_amd.profiling summarize --workload {workload} --dir rocprof_out",
             "```", "", "| kernel | calls | average us | total us | % |", "|---|---|---|---|---|"]
    avg_us = None
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = _short(r["Name"])
        if not name.startswith("pa::"):
            continue
        a = float(r["AverageNs"]) / 1e3
        lines.append(f"| `{name}` | {r['Calls']} | {a:.2f} | {float(r['TotalDurationNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
        if name.startswith(f"pa::{kernel}") and avg_us is None:
            avg_us = a
    # bench.py times the dominant kernel over its last launches (one per
    # step, two for swap: evict and restore); the clock is still rising
    # during the warm-up, so those launches are the ones to compare with
    timed_us = None
    ktrace = _find(d, f"trace_{workload}_kernel_trace.csv")
    if ktrace is not None:
        with open(ktrace, newline="") as f:
            trace_rows = list(csv.DictReader(f))

        def durations(name):
            return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                    for r in trace_rows if _short(r["Kernel_Name"]).startswith(f"pa::{name}")]

        durs = durations(kernel)
        last = durs[-STEPS * (2 if cfg.swap else 1):]
        if last:
            timed_us = sum(last) / len(last)
            lines += ["", f"`{kernel}`: mean over the {len(last)} launches bench.py times (the last ones of "
                          f"the run, from the kernel trace): {timed_us:.2f} us; over all {len(durs)} "
                          f"launches, warm-up included: {sum(durs) / len(durs):.2f} us."]
        plan = durations("decode_plan_kernel")[-STEPS:]
        if plan and last and not cfg.prefill and not cfg.swap:
            plan_us = sum(plan) / len(plan)
            lines += [f"bench.py's events bracket the `pa_decode_partition` call, which launches "
                      f"`decode_plan_kernel` ({plan_us:.2f} us) and then `{kernel}`: "
                      f"{plan_us + timed_us:.2f} us together on the kernel trace, launch gap excluded."]
    kvb = bench_kv_bytes(cfg)
    rate_us = timed_us or avg_us
    if avg_us and cfg.swap:
        lines += ["", f"Bytes per launch (one direction, K and V): {kvb}; at the average duration of "
                      f"`{kernel}` over the timed launches (evictions and restores together) that is "
                      f"{kvb / (rate_us * 1e-6) / 1e9:.1f} GB/s over the host link, "
                      f"{100 * kvb / (rate_us * 1e-6) / 63e9:.1f} % of PCIe 5.0 x16 (63 GB/s)."]
    elif avg_us and cfg.prefill:
        fl = bench_prefill_flops(cfg)
        lines += ["", f"Algorithmic flops per launch: {fl} (4*D per query head and visible key); at the "
                      f"timed launches' mean duration that is {fl / (rate_us * 1e-6) / 1e12:.1f} TFLOP/s, "
                      f"{100 * fl / (rate_us * 1e-6) / 2.5e15:.1f} % of the 2.5 PFLOP/s 16-bit matrix peak. "
                      f"Bytes a launch must move at least (every sequence's K and V read once, "
                      f"q read once, out written once): {kvb}."]
    elif avg_us:
        lines += ["", f"Algorithmic KV bytes per launch: {kvb} (valid tokens' K and V); at the "
                      f"timed launches' mean duration that is {kvb / (rate_us * 1e-6) / 1e9:.1f} GB/s, "
                      f"{100 * kvb / (rate_us * 1e-6) / 8e12:.1f} % of 8 TB/s."]
    rec = {"kernel": kernel, "workload": workload, "kernel_hash": bench.kernel_hash(kernel),
           "avg_launch_us": avg_us, "timed_avg_launch_us": timed_us, "algorithmic_bytes": kvb}
    fetch = _find(d, f"pmc_FETCH_SIZE_{workload}_counter_collection.csv")
    write = _find(d, f"pmc_WRITE_SIZE_{workload}_counter_collection.csv")
    cfetch = _find(d, "pmc_FETCH_SIZE_calibration_counter_collection.csv")
    cwrite = _find(d, "pmc_WRITE_SIZE_calibration_counter_collection.csv")

    def kernel_avg(path, counter):
        vals = [v for n, vs in _counter_per_dispatch(path, counter).items() if kernel in n
                for v in vs]
        return sum(vals) / len(vals), len(vals)

    if fetch and write and cfetch and cwrite:
        def calib(path, counter):
            per = _counter_per_dispatch(path, counter)
            name, vals = max(per.items(), key=lambda kv: max(kv[1]))
            return max(vals), _short(name)

        f_kib, nf = kernel_avg(fetch, "FETCH_SIZE")
        w_kib, nw = kernel_avg(write, "WRITE_SIZE")
        cf_kib, cname = calib(cfetch, "FETCH_SIZE")
        cw_kib, _ = calib(cwrite, "WRITE_SIZE")
        ref = bench.CALIBRATION_BYTES
        kf, kw = ref / (cf_kib * 1024), ref / (cw_kib * 1024)
        hbm = f_kib * 1024 * kf + w_kib * 1024 * kw
        rec.update({"fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
                    "calibration_kernel": cname, "calibration_fetch_kib": cf_kib,
                    "calibration_write_kib": cw_kib, "fetch_factor": kf, "write_factor": kw,
                    "hbm_bytes_per_launch": hbm, "dispatches": [nf, nw]})
        lines += ["", "## HBM traffic (rocprofv3 --pmc, one counter per pass)", "", "```",
                  f"python -m paged_kv_cache_412_amd.profiling pmc --workload {workload} --out rocprof_out",
                  "  # = rocprofv3 --pmc FETCH_SIZE -f csv ... -- python3 bench.py --workload "
                  f"{workload} --steps {PMC_STEPS} --warmup {PMC_WARMUP} --no-cpu-baseline",
                  "  #   rocprofv3 --pmc FETCH_SIZE -f csv ... -- python3 bench.py --copy-calibration",
                  "  #   and the same two with WRITE_SIZE", "```", "",
                  "| quantity | value |", "|---|---|",
                  f"| FETCH_SIZE per `{kernel}` dispatch (KiB, mean of {nf}) | {f_kib:.0f} |",
                  f"| WRITE_SIZE per dispatch (KiB, mean of {nw}) | {w_kib:.0f} |",
                  f"| calibration: 1 GiB copy (`{cname}`) FETCH / WRITE (KiB) | {cf_kib:.0f} / {cw_kib:.0f} |",
                  f"| scale factors fetch / write | {kf:.4f} / {kw:.4f} |",
                  f"| HBM bytes per launch (scaled) | {hbm:.4g} |",
                  f"| algorithmic bytes per launch | {kvb:.4g} |",
                  f"| traffic / algorithmic | {hbm / kvb:.3f} |"]
    util = _find(d, f"pmc_MfmaUtil_{workload}_counter_collection.csv")
    mops = _find(d, f"pmc_MfmaFlops_{workload}_counter_collection.csv")
    if util and mops:
        u, nu = kernel_avg(util, "MfmaUtil")
        issued, nm = kernel_avg(mops, "MfmaFlops")
        alg = bench_prefill_flops(cfg) if cfg.prefill else bench_decode_flops(cfg)
        rec.update({"mfma_util_pct": u, "mfma_flops_per_launch": issued, "algorithmic_flops": alg})
        lines += ["", "## Matrix-core activity (rocprofv3 --pmc, one derived counter per pass)", "", "```",
                  f"python -m paged_kv_cache_412_amd.profiling mfma --workload {workload} --out rocprof_out",
                  "  # = rocprofv3 --pmc MfmaUtil -f csv ... -- python3 bench.py --workload "
                  f"{workload} --steps {PMC_STEPS} --warmup {PMC_WARMUP} --no-cpu-baseline",
                  "  #   and the same with MfmaFlops", "```", "",
                  "| quantity | value |", "|---|---|",
                  f"| MfmaUtil per `{kernel}` dispatch (% of SIMD cycles with the matrix core busy, "
                  f"mean of {nu}) | {u:.1f} |",
                  f"| MfmaFlops per dispatch (flops issued to the matrix cores, mean of {nm}) | {issued:.4g} |",
                  f"| algorithmic flops per launch | {alg:.4g} |",
                  f"| issued / algorithmic | {issued / alg:.3f} |"]
        if rate_us:
            lines.append(f"| issued matrix-core TFLOP/s at the timed launches' mean duration | "
                         f"{issued / (rate_us * 1e-6) / 1e12:.1f} |")
    vm = {c: _find(d, f"pmc_{c}_{workload}_counter_collection.csv") for c in VMEM_COUNTERS}
    if all(vm.values()):
        val = {c: kernel_avg(vm[c], c)[0] for c in VMEM_COUNTERS}
        xcc, cus = _gpu_shape(vm["GRBM_GUI_ACTIVE"].replace("_counter_collection.csv", "_agent_info.csv"))
        # GRBM_GUI_ACTIVE adds one busy-cycle count per XCD: the dispatch's
        # own length in cycles is that over the XCD count.
        cyc = val["GRBM_GUI_ACTIVE"] / xcc
        rec["vmem"] = val
        lines += ["", "## Vector-memory path (rocprofv3 --pmc, one counter per pass)", "", "```",
                  f"python -m paged_kv_cache_412_amd.profiling vmem --workload {workload} --out rocprof_out",
                  "  # = rocprofv3 --pmc <counter> -f csv ... -- python3 bench.py --workload "
                  f"{workload} --steps {PMC_STEPS} --warmup {PMC_WARMUP} --no-cpu-baseline --batches 0",
                  "  #   for each of: " + ", ".join(VMEM_COUNTERS), "```", "",
                  f"Per `{kernel}` dispatch (mean over the run's dispatches).  GRBM_GUI_ACTIVE is summed "
                  f"over the {xcc} XCDs; shares are of the dispatch's length in cycles (that sum over "
                  f"{xcc}), and of that length times {cus} compute units for the summed counters.", "",
                  "| counter | per dispatch | share |", "|---|---|---|",
                  f"| GRBM_GUI_ACTIVE (cycles, all XCDs) | {val['GRBM_GUI_ACTIVE']:.4g} | "
                  f"{cyc:.4g} cycles per XCD |",
                  f"| TA_BUSY_avr: address unit busy | {val['TA_BUSY_avr']:.4g} | "
                  f"{100 * val['TA_BUSY_avr'] / cyc:.1f} % |"]
        for c, what in (("TA_ADDR_STALLED_BY_TC_CYCLES_sum", "address unit stalled by the vector L1 (addresses)"),
                        ("TA_DATA_STALLED_BY_TC_CYCLES_sum", "address unit stalled by the vector L1 (data)"),
                        ("TCP_PENDING_STALL_CYCLES_sum", "vector L1 stalled on pending misses"),
                        ("TCP_TCR_TCP_STALL_CYCLES_sum", "vector L1 stalled by the L2 request path")):
            lines.append(f"| {c}: {what} | {val[c]:.4g} | {100 * val[c] / (cus * cyc):.1f} % |")
        insts = val["SQ_INSTS_VMEM_RD"]
        lines += [f"| SQ_INSTS_VMEM_RD: vector-memory read instructions | {insts:.4g} | "
                  f"{kvb / insts:.0f} algorithmic bytes per instruction |",
                  f"| SQ_WAVES | {val['SQ_WAVES']:.4g} | |"]
    pp = {c: _find(d, f"pmc_{c}_{workload}_counter_collection.csv") for c in PIPE_COUNTERS}
    if all(pp.values()):
        val = {c: kernel_avg(pp[c], c)[0] for c in PIPE_COUNTERS}
        rec["pipe"] = val
        wc = val["SQ_WAVE_CYCLES"]
        lds = val["SQ_LDS_IDX_ACTIVE"]
        lines += ["", "## Where the waves' time goes (rocprofv3 --pmc, one counter per pass)", "", "```",
                  f"python -m paged_kv_cache_412_amd.profiling pipe --workload {workload} --out rocprof_out",
                  "  # = rocprofv3 --pmc <counter> -f csv ... -- python3 bench.py --workload "
                  f"{workload} --steps {PMC_STEPS} --warmup {PMC_WARMUP} --no-cpu-baseline --batches 0",
                  "  #   for each of: " + ", ".join(PIPE_COUNTERS), "```", "",
                  f"Per `{kernel}` dispatch (mean over the run's dispatches).", "",
                  "| counter | per dispatch | share |", "|---|---|---|",
                  f"| SQ_WAVE_CYCLES: wave-cycles | {wc:.4g} | |",
                  f"| SQ_WAIT_ANY: wave-cycles waiting for anything | {val['SQ_WAIT_ANY']:.4g} | "
                  f"{100 * val['SQ_WAIT_ANY'] / wc:.1f} % of wave-cycles |",
                  f"| SQ_WAIT_INST_LDS: wave-cycles waiting to issue an LDS instruction | "
                  f"{val['SQ_WAIT_INST_LDS']:.4g} | {100 * val['SQ_WAIT_INST_LDS'] / wc:.1f} % of wave-cycles |",
                  f"| SQ_ACTIVE_INST_LDS: cycles issuing LDS instructions | {val['SQ_ACTIVE_INST_LDS']:.4g} | |",
                  f"| SQ_LDS_IDX_ACTIVE: LDS active cycles | {lds:.4g} | |",
                  f"| SQ_LDS_BANK_CONFLICT: LDS bank-conflict cycles | {val['SQ_LDS_BANK_CONFLICT']:.4g} | "
                  f"{100 * val['SQ_LDS_BANK_CONFLICT'] / lds:.1f} % of LDS active cycles |",
                  f"| LdsUtil (derived, %) | {val['LdsUtil']:.3g} | |",
                  f"| VALUBusy (derived, %) | {val['VALUBusy']:.3g} | |"]
        ip = {c: _find(d, f"pmc_{c}_{workload}_counter_collection.csv") for c in ISSUE_COUNTERS}
        if all(ip.values()):
            iv = {c: kernel_avg(ip[c], c)[0] for c in ISSUE_COUNTERS}
            rec["issue"] = iv
            xcc, cus = _gpu_shape(ip["GRBM_GUI_ACTIVE"].replace("_counter_collection.csv", "_agent_info.csv"))
            cyc = iv["GRBM_GUI_ACTIVE"] / xcc  # the dispatch's length in cycles
            simds = 4 * cus
            busy = iv["SQ_VALU_MFMA_BUSY_CYCLES"]
            lines += ["",
                      f"Issue and co-execution (same step, one counter per pass: "
                      f"{', '.join(ISSUE_COUNTERS)}).  The first three rows split the wave-cycles.", "",
                      "| counter | per dispatch | share |", "|---|---|---|",
                      f"| SQ_ACTIVE_INST_ANY: wave-cycles issuing | {iv['SQ_ACTIVE_INST_ANY']:.4g} | "
                      f"{100 * iv['SQ_ACTIVE_INST_ANY'] / wc:.1f} % of wave-cycles |",
                      f"| SQ_WAIT_INST_ANY: wave-cycles waiting for an issue slot | {iv['SQ_WAIT_INST_ANY']:.4g} | "
                      f"{100 * iv['SQ_WAIT_INST_ANY'] / wc:.1f} % of wave-cycles |",
                      f"| SQ_WAIT_ANY (above): wave-cycles waiting on a dependency | {val['SQ_WAIT_ANY']:.4g} | "
                      f"{100 * val['SQ_WAIT_ANY'] / wc:.1f} % of wave-cycles |",
                      f"| GRBM_GUI_ACTIVE (cycles, all {xcc} XCDs) | {iv['GRBM_GUI_ACTIVE']:.4g} | "
                      f"{cyc:.4g} cycles per XCD |",
                      f"| SQ_VALU_MFMA_BUSY_CYCLES: matrix-core busy cycles, all {simds} SIMDs | {busy:.4g} | "
                      f"{100 * busy / (simds * cyc):.1f} % of SIMD cycles |",
                      f"| SQ_VALU_MFMA_COEXEC_CYCLES: busy with a vector instruction issued beside | "
                      f"{iv['SQ_VALU_MFMA_COEXEC_CYCLES']:.4g} | "
                      f"{100 * iv['SQ_VALU_MFMA_COEXEC_CYCLES'] / busy:.1f} % of matrix-core busy cycles |",
                      f"| SQ_INSTS_MFMA: matrix instructions | {iv['SQ_INSTS_MFMA']:.4g} | "
                      f"{busy / iv['SQ_INSTS_MFMA']:.1f} busy cycles each |",
                      f"| SQ_INSTS_VALU: vector instructions (matrix ones included) | {iv['SQ_INSTS_VALU']:.4g} | |",
                      f"| SQ_INSTS_VALU_TRANS_F32: fp32 transcendentals | {iv['SQ_INSTS_VALU_TRANS_F32']:.4g} | |"]
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"{kernel}_{workload}.md"), "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(PROFILES, f"traffic_{kernel}_{workload}.json"), "w", encoding="utf-8") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print("\n".join(lines))


def bench_kv_bytes(cfg) -> int:
    """Algorithmic bytes of the workload's dominant kernel (its seeded
    lengths, no GPU): for decode the valid tokens' K and V; for prefill
    those plus q read once and out written once."""
    import numpy as np

    from paged_kv_cache_412_amd import workloads
    if cfg.swap:
        return 2 * int(cfg.swap["blocks"]) * cfg.block_size * cfg.Hkv * cfg.D * \
            workloads.ELEM_BYTES[cfg.kv_dtype]
    if cfg.prefill:
        news, ctx, _ = workloads.prefill_lengths(cfg)
        lens = news + ctx
        qo = int(np.sum(news)) * cfg.Hq * cfg.D * (workloads.ELEM_BYTES[cfg.q_dtype] +
                                                   workloads.ELEM_BYTES[cfg.out_dtype])
        return int(np.sum(lens)) * 2 * cfg.Hkv * cfg.D * workloads.ELEM_BYTES[cfg.kv_dtype] + qo
    else:
        lens = workloads.seq_lengths(cfg)
    return int(np.sum(lens)) * 2 * cfg.Hkv * cfg.D * workloads.ELEM_BYTES[cfg.kv_dtype]


def bench_decode_flops(cfg) -> int:
    """Algorithmic flops of a decode launch (its seeded lengths, no GPU):
    4*D per (valid token, query head), 2*D for q.k and 2*D for p.v."""
    import numpy as np

    from paged_kv_cache_412_amd import workloads
    return 4 * cfg.D * cfg.Hq * int(np.sum(workloads.seq_lengths(cfg)))


def bench_prefill_flops(cfg) -> int:
    """Algorithmic flops of the prefill workload (its seeded lengths, no GPU)."""
    from paged_kv_cache_412_amd import workloads
    news, ctx, _ = workloads.prefill_lengths(cfg)
    pairs = sum(int(n) * int(c) + int(n) * (int(n) + 1) // 2 for n, c in zip(news, ctx))
    return 4 * cfg.D * cfg.Hq * pairs


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("step", choices=["trace", "pmc", "calibration", "mfma", "vmem", "pipe", "summarize"])
    ap.add_argument("--no-calibration", action="store_true",
                    help="pmc: skip the calibration copy (taken once by the calibration step)")
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--out", default="rocprof_out")
    ap.add_argument("--dir", default="rocprof_out")
    a = ap.parse_args(argv)
    if a.step == "trace":
        trace(a.workload, a.out)
    elif a.step == "pmc":
        pmc(a.workload, a.out, not a.no_calibration)
    elif a.step == "calibration":
        calibration(a.out)
    elif a.step == "mfma":
        mfma(a.workload, a.out)
    elif a.step == "vmem":
        vmem(a.workload, a.out)
    elif a.step == "pipe":
        pipe(a.workload, a.out)
    else:
        summarize(a.workload, a.dir)
    return 0


if __name__ == "__main__":
    sys.exit(main())
