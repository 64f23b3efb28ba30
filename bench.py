"""Benchmark of the paged decode path on one MI355X.

One step = the whole hot path over one batch: slot mapping, copy-on-write
block copies (when the workload shares blocks), the cache write of one new
token per sequence, the split-K decode partitions and the combine of split
sequences (in the partition launch or a reduce launch, ``--combine``).  With a
prefill workload (``--workload prefill13b | prefill70b | prefill_fp8``) a
step is the prefill path instead: slot mapping of every new token, the cache
write, and causal paged attention, reported in algorithmic TFLOP/s against
the matrix-core peak.  Inputs
are seeded synthetic data already resident in HBM; the timed region holds
exactly ``--steps`` steps between a synchronise and two HIP events.

Printed: one JSON line with the metric (effective KV GB/s: bytes of the valid
tokens' K and V, sum_b L_b * 2 * Hkv * D * elem, per step time), the roofline
of the dominant kernel (the decode partition kernel, timed with HIP events on
the stream it runs on), the per-step time as the median of 5 batches beside
the contract's single timed batch, the GPU, ROCm release and host, and the
CPU oracle timed on a bounded sample twice (every affinity core, one
thread) with the GPU output's max abs error against the oracle on it.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
METRIC = "paged decode attention: effective KV GB/s and % of HBM peak; seqs/s per layer"
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
_COMMON_SOURCES = ["paged_kv_cache_412_amd/csrc/pa_device.h",
                   "paged_kv_cache_412_amd/csrc/pa_mfma.h",
                   "paged_kv_cache_412_amd/csrc/pa_decode_common.h",
                   "paged_kv_cache_412_amd/csrc/pa_internal.h",
                   "paged_kv_cache_412_amd/csrc/pa_api.hip"]
# sources a kernel's measured counters depend on (the counters are dropped
# when any of them changes)
KERNEL_SOURCES = {
    "decode": ["paged_kv_cache_412_amd/csrc/pa_decode.hip",
               "paged_kv_cache_412_amd/csrc/pa_decode_valu.hip",
               "paged_kv_cache_412_amd/csrc/pa_decode_mfma.hip"] + _COMMON_SOURCES,
    "prefill": ["paged_kv_cache_412_amd/csrc/pa_prefill.hip"] + _COMMON_SOURCES,
    "cache": ["paged_kv_cache_412_amd/csrc/pa_cache.hip"] + _COMMON_SOURCES,
}
CALIBRATION_BYTES = 1 << 30  # size of the plain copy used to scale the PMC byte counters
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # MI355X dense 16-bit matrix peak


def kernel_hash(kernel: str) -> str:
    family = ("prefill" if kernel.startswith("prefill") else
              "cache" if kernel.startswith("copy_blocks") else "decode")
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kv_bytes(wl) -> int:
    from paged_kv_cache_412_amd.workloads import ELEM_BYTES
    c = wl.cfg
    return int(np.sum(wl.seq_lens)) * 2 * c.Hkv * c.D * ELEM_BYTES[c.kv_dtype]


def decode_kernel_name(cfg) -> str:
    """The dominant kernel the library dispatches for this workload: the
    prefill kernel for prefill workloads; for decode, the library's rule
    (include/pa.h, decode workspace layout): the matrix-core partition kernel
    for query groups of 3 to 16 with a 16-bit query over a cache of the same
    16-bit type or an 8-bit cache, the vector-ALU kernel otherwise."""
    if cfg.prefill:
        return "prefill_kernel"
    if cfg.swap:
        return "copy_blocks_kernel"
    pair = cfg.q_dtype == cfg.kv_dtype in ("f16", "bf16") or (
        cfg.kv_dtype in ("e4m3", "e5m2") and cfg.q_dtype in ("f16", "bf16"))
    return "decode_mfma_kernel" if 3 <= cfg.G <= 16 and pair else "decode_valu_kernel"


def prefill_flops(wl) -> int:
    """Algorithmic flops of one prefill call: 4*D per (query head, visible
    key) pair -- 2*D for the score, 2*D for the weighted sum -- over the
    causal pairs: new token i of sequence b sees ctx_b + i + 1 keys."""
    c = wl.cfg
    pairs = 0
    for n, L in zip(wl.news, wl.seq_lens):
        n, L = int(n), int(L)
        ctx = L - n
        pairs += n * ctx + n * (n + 1) // 2
    return 4 * c.D * c.Hq * pairs


def prefill_bytes(wl) -> int:
    """Bytes a prefill call must move at least: every sequence's L_b tokens
    of K and V (all KV heads) read once, q read once, out written once."""
    from paged_kv_cache_412_amd.workloads import ELEM_BYTES
    c = wl.cfg
    kv = int(np.sum(wl.seq_lens)) * 2 * c.Hkv * c.D * ELEM_BYTES[c.kv_dtype]
    return kv + wl.T * c.Hq * c.D * (ELEM_BYTES[c.q_dtype] + ELEM_BYTES[c.out_dtype])


def _counter_record(kernel: str, workload: str) -> dict:
    """The committed PMC counter record of this kernel and workload, if it was
    taken on the current kernel source; else {}."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path, encoding="utf-8") as f:
        rec = json.load(f)
    return rec if rec.get("kernel_hash") == kernel_hash(kernel) else {}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed PMC counter runs, if they were taken
    on the current kernel source."""
    return _counter_record(kernel, workload).get("hbm_bytes_per_launch")


def measured_mfma(kernel: str, workload: str):
    """Matrix-core counters per launch (busy percent of SIMD cycles, flops
    issued, and those over the algorithmic flops) from committed PMC runs on
    the current kernel source, or None."""
    rec = _counter_record(kernel, workload)
    if "mfma_util_pct" not in rec:
        return None
    return {"busy_pct": round(rec["mfma_util_pct"], 1),
            "issued_flops": rec["mfma_flops_per_launch"],
            "issued_over_algorithmic": round(rec["mfma_flops_per_launch"] / rec["algorithmic_flops"], 3)}


def read_ceiling(args):
    """The practical HBM read rate of a block gather on this part: a 4 GiB
    pool read whole, piece by piece in a seeded random order, through
    pa_read_blocks (the attention kernels' non-temporal 16-byte buffer
    loads), for pieces of 1 to 32 KiB; beside it, torch's own device copy
    (bytes read plus bytes written per second).  Prints one JSON line."""
    import torch

    from paged_kv_cache_412_amd import binding
    total = 4 << 30
    pool = torch.empty(total, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    reps = max(3, args.steps // 5)
    res = {}
    for kib in (1, 2, 4, 8, 16, 32):
        piece = kib << 10
        ids = torch.from_numpy(np.random.default_rng(412).permutation(total // piece).astype(np.int32)).cuda()
        for _ in range(2):
            binding.read_blocks(pool, piece, ids, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            binding.read_blocks(pool, piece, ids, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        res[f"{kib}KiB"] = round(total / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)
    del pool
    src = torch.empty(2 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    print(json.dumps({"read_ceiling_gbs": res, "pool_bytes": total, "reps": reps,
                      "torch_copy_gbs_read_plus_write": round(copy_gbs, 1),
                      "peak_gbs": HBM_PEAK_GBS}), flush=True)
    return 0


def copy_calibration():
    """A plain device-to-device copy of CALIBRATION_BYTES, three times: the
    reference the PMC byte counters are scaled by."""
    import torch
    src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": CALIBRATION_BYTES, "copies": 3}), flush=True)
    return 0


def host_facts() -> dict:
    """Where the CPU baseline ran: affinity cores, os.cpu_count(), the CPU
    model, NumPy's BLAS backend and its default thread count."""
    from threadpoolctl import threadpool_info
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
            for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"affinity_cores": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "cpu_model": model, "numpy_blas": blas}


def cpu_legs(run_leg, budget_s: float) -> dict:
    """The oracle timed twice on the host: with every core this process may
    run on as BLAS threads, then with one.  run_leg(threads, budget) returns
    the leg's result dict; the all-core leg is the reported value."""
    host = host_facts()
    n = host["affinity_cores"]
    many = run_leg(n, budget_s)
    one = run_leg(1, budget_s)
    out = dict(many)
    out["cores"] = n
    out["single_thread"] = {k: one[k] for k in ("value", "seconds", "sample") if k in one}
    out["host"] = host
    return out


def cpu_baseline(wl, step, budget_s: float, check=None):
    """The oracle as it stands, on host copies of the pools, over as many
    sequences as fit in ``budget_s`` seconds (at least one), with every
    affinity core and with one BLAS thread.  ``check`` receives the oracle's
    output for the sequences it computed (max abs error of the GPU's)."""
    from threadpoolctl import threadpool_limits

    from oracle import paged
    from paged_kv_cache_412_amd.workloads import ELEM_BYTES
    from tests import parity

    cfg = wl.cfg
    k = parity.storage(wl.k_pool)
    v = parity.storage(wl.v_pool)
    q = parity.widen(parity.storage(wl.q), cfg.q_dtype)
    tab = step.tables_np
    order = np.random.default_rng(0).permutation(cfg.B)

    def leg(threads, budget):
        done, nbytes = [], 0
        outs = []
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            for b in order:
                o = paged.decode(q, k, v, tab, wl.seq_lens, cfg.block_size, wl.scale, seqs=[int(b)],
                                 widen_k=lambda x: parity.widen(x, cfg.kv_dtype, wl.k_scale),
                                 widen_v=lambda x: parity.widen(x, cfg.kv_dtype, wl.v_scale))
                outs.append(o[int(b)])
                done.append(int(b))
                nbytes += int(wl.seq_lens[b]) * 2 * cfg.Hkv * cfg.D * ELEM_BYTES[cfg.kv_dtype]
                if time.perf_counter() - t0 >= budget:
                    break
            dt = time.perf_counter() - t0
        if check is not None and threads != 1:
            check(done, np.stack(outs))
        return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "kind": "oracle",
                "sample": f"{len(done)} of {cfg.B} sequences (all {cfg.Hq} heads), {dt:.1f} s, "
                          f"fp64 NumPy, BLAS limited to {threads} thread(s)",
                "seconds": round(dt, 3), "seq_layers_per_s": round(len(done) / dt, 3)}
    return cpu_legs(leg, budget_s)


def cpu_baseline_prefill(wl, step, budget_s: float, check=None):
    """The oracle as it stands over a bounded sample of new tokens: each
    sampled token's attention as a one-row prefill over its sequence's first
    p + 1 tokens, all query heads; every affinity core, then one thread."""
    from threadpoolctl import threadpool_limits

    from oracle import paged
    from tests import parity

    cfg = wl.cfg
    k = parity.storage(wl.k_pool)
    v = parity.storage(wl.v_pool)
    q = parity.widen(parity.storage(wl.q), cfg.q_dtype)
    tab = step.tables_np.astype(np.int64)
    rows = np.random.default_rng(0).permutation(wl.T)
    owner = np.searchsorted(wl.q_starts, rows, side="right") - 1

    def leg(threads, budget):
        done, flops = [], 0
        outs = []
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            for r, b in zip(rows, owner):
                pos = int(wl.seq_lens[b]) - int(wl.news[b]) + int(r - wl.q_starts[b])
                o = paged.prefill(q[r:r + 1], k, v, tab[b:b + 1], np.array([pos + 1]), np.array([0, 1]),
                                  cfg.block_size, wl.scale,
                                  widen_k=lambda x: parity.widen(x, cfg.kv_dtype, wl.k_scale),
                                  widen_v=lambda x: parity.widen(x, cfg.kv_dtype, wl.v_scale))
                done.append(int(r))
                outs.append(o[0])
                flops += 4 * cfg.D * cfg.Hq * (pos + 1)
                if time.perf_counter() - t0 >= budget:
                    break
            dt = time.perf_counter() - t0
        if check is not None and threads != 1:
            check(done, np.stack(outs))
        return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
                "sample": f"{len(done)} of {wl.T} new tokens (all {cfg.Hq} heads), {dt:.1f} s, "
                          f"fp64 NumPy, BLAS limited to {threads} thread(s)",
                "seconds": round(dt, 3)}
    return cpu_legs(leg, budget_s)


def gpu_facts() -> dict:
    """The GPU and the ROCm release the numbers come from."""
    import torch
    ver = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(path) as f:
                ver = f.read().strip()
                break
        except OSError:
            continue
    props = torch.cuda.get_device_properties(0)
    name = torch.cuda.get_device_name(0)
    # without libdrm's marketing-name table the runtime reports no name or a
    # generic one; the kernel driver's sysfs entries still carry the product
    # name, the PCI device id and the VBIOS part number
    sysfs = {}
    for card in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        for key in ("product_name", "device", "vbios_version"):
            try:
                with open(os.path.join(card, key)) as f:
                    sysfs.setdefault(key, f.read().strip())
            except OSError:
                pass
        if sysfs:
            break
    return {"gpu_name": name or sysfs.get("product_name", ""), "gpu_product": sysfs.get("product_name"),
            "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "pci_device_id": sysfs.get("device"),
            "vbios": sysfs.get("vbios_version"), "rocm_version": ver, "hip_runtime": torch.version.hip}


def median_batches(run_step, stream, batches=5, steps=100) -> dict:
    """Per-step time as the median of `batches` batches of `steps` back-to-back
    steps (events on the stream around each batch)."""
    import torch
    ms = []
    for _ in range(batches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            run_step()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / steps)
    return {"median_ms_per_step": round(float(np.median(ms)), 5),
            "batches_ms_per_step": [round(x, 5) for x in ms], "steps_per_batch": steps}


def error_check(gpu_out, kv_dtype, out_dtype):
    """A `check` callback for the CPU legs: max abs error of the GPU output
    (first axis: sequences or new-token rows) against the oracle on the
    sampled rows, and whether every element is
    within the parity tolerance (that of the KV dtype plus half an ulp of
    the output dtype)."""
    from tests import parity
    result = {}

    def check(rows, ref):
        g = parity.gpu_out(gpu_out)[rows]
        err = np.abs(g - ref)
        p, emin = parity.OUT_FORMAT[out_dtype]
        from oracle import numerics
        bound = parity.TOL[kv_dtype] + numerics.half_ulp(ref, p, emin)
        result.update({"value": float(np.max(err)), "within_tolerance": bool(np.all(err <= bound)),
                       "tolerance": parity.TOL[kv_dtype], "rows": len(rows)})
    return check, result


def bench_prefill(args, cfg):
    """Prefill workloads: one step = slot mapping, cache write and causal
    paged attention of every sequence's new tokens."""
    import torch

    from paged_kv_cache_412_amd import workloads
    from paged_kv_cache_412_amd.step import PrefillStep

    print(f"[bench] building prefill workload {cfg.name}", file=sys.stderr, flush=True)
    wl = workloads.make_prefill(cfg, device="cuda")
    step = PrefillStep(wl)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps, {ms_step:.4f} ms/step", file=sys.stderr, flush=True)
    stages = ["slot_mapping", "cache_write", "attention"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, s in enumerate(stages):
            getattr(step, s)()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {s: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, s in enumerate(stages)}
    batches = median_batches(step.run, stream, args.batches, steps=20) if args.batches else None
    flops = prefill_flops(wl)
    tflops = flops / (ms_step * 1e-3) / 1e12
    attn_ms = stage_ms["attention"]
    achieved = flops / (attn_ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS["bf16" if cfg.q_dtype == "bf16" else "f16"]
    kernel = decode_kernel_name(cfg)
    out = {
        "metric": "paged prefill attention: algorithmic TFLOP/s and % of the MFMA peak; tokens/s per layer",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.q_dtype,
        "accum_dtype": "f32",
        "data": "synthetic (seeded N(0,1) queries, new rows and caches, scattered block tables)",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "block_size": cfg.block_size, "kv_dtype": cfg.kv_dtype, "q_dtype": cfg.q_dtype,
                   "new_tokens": f"U[{cfg.prefill['new'][0]},{cfg.prefill['new'][1]}]",
                   "cached_tokens": f"U[{cfg.prefill['ctx'][0]},{cfg.prefill['ctx'][1]}]",
                   "total_new_tokens": wl.T, "pool_blocks": wl.num_blocks},
        "tokens_per_s": round(wl.T / (ms_step * 1e-3), 1),
        "flops_per_step": flops,
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "median_of_batches": (dict(batches, tflops=round(flops / (batches["median_ms_per_step"] * 1e-3) / 1e12, 2))
                              if batches else None),
        "system": gpu_facts(),
        "roofline": {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(kernel, cfg.name),
                     "algorithmic_bytes": prefill_bytes(wl), "avg_launch_ms": round(attn_ms, 5),
                     "mfma": measured_mfma(kernel, cfg.name)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        check, err = error_check(step.out, cfg.kv_dtype, cfg.out_dtype)
        out["cpu_baseline"] = cpu_baseline_prefill(wl, step, args.cpu_budget, check)
        out["max_abs_err_vs_oracle"] = err
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


# the library computes the balanced schedule's plan inside the attention
# kernel up to this many sequences (a separate plan kernel beyond)
INLINE_PLAN_MAX_B = 1024

HOST_LINK_PEAK_GBS = 63.0  # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes, 128b/130b)


def bench_swap(args, cfg):
    """Swap workloads: one step = evict N blocks (K and V) from the device
    pools to pinned host pools, then restore them to other device blocks,
    two pa_swap_blocks calls.  Bytes move over the host link both ways."""
    import torch

    from paged_kv_cache_412_amd import binding, workloads

    print(f"[bench] building swap workload {cfg.name}", file=sys.stderr, flush=True)
    wl = workloads.make_swap(cfg)
    N = wl.out_pairs.shape[0]
    nbytes = 2 * N * wl.block_bytes          # K and V, one direction
    stream = torch.cuda.current_stream()

    def out():
        binding.swap_blocks(wl.k_dev, wl.v_dev, wl.k_host, wl.v_host, wl.out_map)

    def back():
        binding.swap_blocks(wl.k_host, wl.v_host, wl.k_dev, wl.v_dev, wl.in_map)

    for _ in range(args.warmup):
        out()
        back()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        out()
        ev[i][1].record(stream)
        back()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    out_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    in_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    ms_step = out_ms + in_ms
    # the link's practical ceiling: the runtime's own pinned copies of the same bytes
    dev_chunk = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    host_chunk = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    for _ in range(2):
        host_chunk.copy_(dev_chunk, non_blocking=True)
        dev_chunk.copy_(host_chunk, non_blocking=True)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    host_chunk.copy_(dev_chunk, non_blocking=True)
    e[1].record(stream)
    dev_chunk.copy_(host_chunk, non_blocking=True)
    e[2].record(stream)
    torch.cuda.synchronize()
    copy_d2h, copy_h2d = e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])
    gbs = 2 * nbytes / (ms_step * 1e-3) / 1e9
    out_gbs = nbytes / (out_ms * 1e-3) / 1e9
    in_gbs = nbytes / (in_ms * 1e-3) / 1e9
    res = {
        "metric": "page-granular swap: GB/s over the host link (evict + restore), % of the link peak",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic (seeded N(0,1) fp16 pools, seeded random victim and target blocks)",
        "config": {"workload": cfg.name, "blocks_each_way": N, "block_bytes_per_pool": wl.block_bytes,
                   "block_size": cfg.block_size, "Hkv": cfg.Hkv, "D": cfg.D, "kv_dtype": cfg.kv_dtype,
                   "bytes_each_way": nbytes},
        "evict_gbs": round(out_gbs, 2),
        "restore_gbs": round(in_gbs, 2),
        "runtime_pinned_copy_gbs": {"d2h": round(nbytes / (copy_d2h * 1e-3) / 1e9, 2),
                                    "h2d": round(nbytes / (copy_h2d * 1e-3) / 1e9, 2)},
        "roofline": {"kernel": "copy_blocks_kernel", "bound": "host_link",
                     "achieved": round(min(out_gbs, in_gbs), 2), "peak": HOST_LINK_PEAK_GBS,
                     "unit": "GB/s", "frac": round(min(out_gbs, in_gbs) / HOST_LINK_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes": nbytes,
                     "avg_launch_ms": {"evict": round(out_ms, 5), "restore": round(in_ms, 5)}},
    }
    if not args.no_cpu_baseline:
        from oracle import paged
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        kd = parity_storage(wl.k_dev)
        kh = parity_storage(wl.k_host)
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < min(args.cpu_budget, 5.0) or done == 0:
            paged.swap_blocks(kd, kh, wl.out_pairs)
            done += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(done * N * wl.block_bytes / dt / 1e9, 3), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{done} evictions of the K pool's {N} blocks in host memory, {dt:.1f} s"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


def replay(manager, ops, budget_s=None, on_add=None):
    """Run a request-stream trace on a block manager (the library's or the
    oracle's); returns (operations done, seconds, peak blocks in use)."""
    is_native = hasattr(manager, "_h")
    total = manager.free_blocks()
    peak, done = 0, 0
    t0 = time.perf_counter()
    for op in ops:
        kind = op[0]
        if kind == "add":
            sid, cached = manager.add(op[1])
            if on_add:
                on_add(len(op[1]), cached)
        elif kind == "append":
            manager.append(op[1], op[2])
        elif kind == "fork":
            manager.fork(op[1])
        else:
            manager.free(op[1]) if is_native else manager.free_seq(op[1])
        done += 1
        if kind != "append" or done % 64 == 0:
            peak = max(peak, total - manager.free_blocks())
        if budget_s is not None and done % 256 == 0 and time.perf_counter() - t0 > budget_s:
            break
    return done, time.perf_counter() - t0, peak


def bench_stream(args, cfg):
    """Block-manager workloads: the library's native manager replays a
    seeded continuous-batching request stream (host code; no GPU kernel)."""
    from paged_kv_cache_412_amd import binding, workloads

    print(f"[bench] building request stream {cfg.name}", file=sys.stderr, flush=True)
    ops = workloads.make_stream(cfg)
    lens = {}
    NB = cfg.B * -(-(cfg.stream["system_len"][1] + cfg.stream["user_len"][1] +
                     cfg.stream["gen_len"][1]) // cfg.block_size)
    stats = {"prompt_tokens": 0, "cached_tokens": 0}

    def count(n, cached):
        stats["prompt_tokens"] += n
        stats["cached_tokens"] += cached

    times = []
    for rep in range(max(1, args.steps)):
        m = binding.BlockManager(NB, cfg.block_size, True)
        done, dt, peak_on = replay(m, ops, on_add=count if rep == 0 else None)
        m.close()
        times.append(dt)
    dt = float(np.median(times))
    m = binding.BlockManager(NB, cfg.block_size, False)
    _, _, peak_off = replay(m, ops)
    m.close()
    kinds = {k: sum(1 for o in ops if o[0] == k) for k in ("add", "append", "fork", "free")}
    res = {
        "metric": "host block manager with prefix caching: operations/s; blocks saved by caching",
        "value": round(len(ops) / dt, 1),
        "unit": "ops/s",
        "n_gpus": 1,
        "steps": max(1, args.steps),
        "warmup": 0,
        "ms_per_step": round(dt * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic request stream (seeded token ids, shared system prompts, n=3 samples)",
        "config": {"workload": cfg.name, "max_live": cfg.B, "block_size": cfg.block_size,
                   "pool_blocks": NB, **{k: (list(v) if isinstance(v, tuple) else v)
                                         for k, v in cfg.stream.items()}, "ops": kinds},
        "prompt_tokens_from_cache": round(stats["cached_tokens"] / max(1, stats["prompt_tokens"]), 4),
        "peak_blocks_in_use": {"prefix_caching": peak_on, "no_caching": peak_off},
        "blocks_saved_frac": round(1.0 - peak_on / max(1, peak_off), 4),
        "note": "host code through the ctypes binding (call overhead included); no device kernel",
        "roofline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import prefix_cache as opc
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        o = opc.PrefixCache(NB, cfg.block_size, caching=True)
        done, odt, _ = replay(o, ops, budget_s=min(args.cpu_budget, 10.0))
        res["cpu_baseline"] = {"value": round(done / odt, 1), "unit": "ops/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {done} of {len(ops)} operations of the same stream, {odt:.1f} s"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)
    return 0


def parity_storage(t):
    from tests import parity
    return parity.storage(t)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps before the timed ones: with 10, the first timed decode "
                         "steps still run below the steady rate (long 8-bit contexts 10 %% slower)")
    ap.add_argument("--workload", default="llama13b")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--combine", choices=["auto", "in_launch", "reduce"], default="auto",
                    help="who combines sequences split across work-groups (pa_decode_args.combine)")
    ap.add_argument("--cpu-budget", type=float, default=8.0,
                    help="seconds of oracle work per CPU leg (all cores, then one thread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--batches", type=int, default=5,
                    help="extra batches of 100 steps for the median step time (0: none)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="measure the block-gather read ceiling and torch's copy rate, then exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the plain copy the PMC byte counters are scaled by")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path is measured on one GPU's share of "
              f"the batch; --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import torch

    from paged_kv_cache_412_amd import binding, workloads
    from paged_kv_cache_412_amd.step import DecodeStep

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration()
    if args.read_ceiling:
        return read_ceiling(args)
    if workloads.CONFIGS[args.workload].stream:
        return bench_stream(args, workloads.CONFIGS[args.workload])
    binding.lib()
    cfg = workloads.CONFIGS[args.workload]
    if cfg.prefill:
        return bench_prefill(args, cfg)
    if cfg.swap:
        return bench_swap(args, cfg)
    print(f"[bench] building workload {cfg.name}", file=sys.stderr, flush=True)
    wl = workloads.make(cfg, device="cuda")
    combine = {"auto": binding.PA_COMBINE_AUTO, "in_launch": binding.PA_COMBINE_IN_LAUNCH,
               "reduce": binding.PA_COMBINE_REDUCE}[args.combine]
    step = DecodeStep(wl, partition_size=args.partition_size, combine=combine)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    # timed region: exactly --steps whole steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] {args.steps} steps, {ms_step:.4f} ms/step", file=sys.stderr, flush=True)

    # per-stage durations, events on the same stream around each C-ABI call
    stages = list(DecodeStep.STAGES)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, s in enumerate(stages):
            getattr(step, s)()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {s: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, s in enumerate(stages)}

    batches = median_batches(step.run, stream, args.batches) if args.batches else None
    nbytes = kv_bytes(wl)
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    part_ms = stage_ms["decode_partition"]
    achieved = nbytes / (part_ms * 1e-3) / 1e9
    kernel = decode_kernel_name(cfg)
    traffic = measured_traffic(kernel, cfg.name)
    partition = binding.partition_size(step.args)
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.kv_dtype,
        "accum_dtype": "f32",
        "data": "synthetic (seeded N(0,1) queries and caches, scattered block tables)",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D,
                   "block_size": cfg.block_size, "kv_dtype": cfg.kv_dtype, "q_dtype": cfg.q_dtype,
                   "seq_lens": (f"U[{cfg.len_range[0]},{cfg.len_range[1]}]" if cfg.len_range
                                else "fixed"),
                   "total_tokens": int(np.sum(wl.seq_lens)), "pool_blocks": wl.num_blocks,
                   "partition_size": partition, "combine": args.combine,
                   "cow_copies": len(step.copies)},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "seq_layers_per_s": round(cfg.B / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": nbytes,
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "median_of_batches": (dict(batches, gbs=round(nbytes / (batches["median_ms_per_step"] * 1e-3) / 1e9, 2))
                              if batches else None),
        "system": gpu_facts(),
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": nbytes, "avg_launch_ms": round(part_ms, 5),
                     "launch_scope": ("pa_decode_partition call: plan kernel, then the attention kernel"
                                      if partition == 0 and cfg.B > INLINE_PLAN_MAX_B
                                      else "pa_decode_partition call: the attention kernel"),
                     "mfma": measured_mfma(kernel, cfg.name)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        check, err = error_check(step.out, cfg.kv_dtype, cfg.out_dtype)
        out["cpu_baseline"] = cpu_baseline(wl, step, args.cpu_budget, check)
        out["max_abs_err_vs_oracle"] = err
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
