"""pa_decode_no_alloc through the C ABI against pa_decode on the same inputs.

The allocation-free entry point runs the same kernels on the library's own
fixed workspace instead of the caller's, so its outputs must equal
pa_decode's bit for bit.  Each case makes two calls in a row on the shared
array, the second with a smaller input (fewer sequences, other lengths), so
that what the first call left in the array (partial rows, counters) cannot
leak into the second; the first case is also checked against the oracle.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

from paged_kv_cache_412_amd import binding, workloads
from paged_kv_cache_412_amd.step import DecodeStep
from tests import parity

pytestmark = pytest.mark.gpu

C = workloads.CONFIGS
SMALL = {
    "tiny": C["tiny"],
    "llama13b": replace(C["llama13b"], B=6, Hq=4, Hkv=4, len_range=(100, 1600)),
    "llama70b": replace(C["llama70b"], B=4, Hq=16, Hkv=2, lens=(4096, 777, 1, 513)),
    "long_fp8": replace(C["long_fp8"], B=2, Hq=8, Hkv=2),
    "llama13b_bs8": replace(C["llama13b"], name="llama13b_bs8", B=6, Hq=4, Hkv=4, block_size=8,
                            len_range=(100, 1600)),
}
COMBINES = {"auto": binding.PA_COMBINE_AUTO, "in_launch": binding.PA_COMBINE_IN_LAUNCH,
            "reduce": binding.PA_COMBINE_REDUCE}


def both(step, wl, part, combine, rows=None):
    """pa_decode (torch workspace) and pa_decode_no_alloc on the step's
    post-write state, for sequences `rows` (all by default)."""
    rows = slice(None) if rows is None else rows
    q = wl.q[rows].contiguous()
    tables = step.block_tables[rows].contiguous()
    lens = step.seq_lens[rows].contiguous()
    ref = torch.full((q.shape[0], q.shape[1], q.shape[2]), float("nan"), dtype=torch.float32, device="cuda")
    got = torch.full_like(ref, float("nan"))
    kw = dict(kv_dtype=step.kv_dtype, k_scales=step.k_scales, v_scales=step.v_scales, combine=combine)
    binding.decode(ref, q, wl.k_pool, wl.v_pool, tables, lens, wl.scale, step.k_scale, step.v_scale,
                   partition_size=part, **kw)
    binding.decode_no_alloc(got, q, wl.k_pool, wl.v_pool, tables, lens, wl.scale, step.k_scale,
                            step.v_scale, partition_size=part, **kw)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("mode", list(COMBINES))
@pytest.mark.parametrize("part", [0, 64])
@pytest.mark.parametrize("name", list(SMALL))
def test_no_alloc_equals_pa_decode_twice(name, part, mode):
    cfg = SMALL[name]
    if part % cfg.block_size:
        part = cfg.block_size
    print(f"\n[case] no-alloc {name} part={part} combine={mode}", flush=True)
    wl = workloads.make(cfg, device="cuda")
    pre = parity.snapshot(wl)
    step = DecodeStep(wl, partition_size=part, out_dtype="f32", combine=COMBINES[mode])
    step.run()
    torch.cuda.synchronize()
    ref, got = both(step, wl, part, COMBINES[mode])
    assert torch.equal(ref.view(torch.int32), got.view(torch.int32)), "first call differs from pa_decode"
    exp = parity.oracle_step(wl, pre)
    parity.assert_close(parity.gpu_out(got), exp.out, cfg.kv_dtype, "f32", f"{name} no-alloc")
    # second call: fewer sequences (the last ones, other lengths), same array
    keep = slice(cfg.B // 2, cfg.B)
    ref2, got2 = both(step, wl, part, COMBINES[mode], keep)
    assert torch.equal(ref2.view(torch.int32), got2.view(torch.int32)), "second call differs"
    print(f"[ok] {name} part={part} combine={mode}", flush=True)


def test_no_alloc_many_sequences_then_one():
    """A batch past the inline plan (the plan kernel's prefix sums live in the
    array too), then one long sequence split over every work-group."""
    base = SMALL["llama70b"]
    lens = tuple(int(x) for x in np.random.default_rng(8).integers(0, 70, 1500))
    for cfg in (replace(base, B=1500, lens=lens, pool_blocks=0),
                replace(base, B=1, lens=(20001,), pool_blocks=0)):
        print(f"\n[case] no-alloc B={cfg.B}", flush=True)
        wl = workloads.make(cfg, device="cuda")
        step = DecodeStep(wl, out_dtype="f32")
        step.run()
        torch.cuda.synchronize()
        for mode in COMBINES.values():
            ref, got = both(step, wl, 0, mode)
            assert torch.equal(ref.view(torch.int32), got.view(torch.int32)), (cfg.B, mode)


def test_no_alloc_rejects_what_does_not_fit():
    """More counters than the fixed region holds: PA_ERR_WORKSPACE, nothing
    written."""
    B, Hq, Hkv, D, bs = 2048, 40, 40, 64, 16       # B * Hkv = 81,920 > 65,536
    q = torch.zeros((B, Hq, D), dtype=torch.float16, device="cuda")
    k = torch.zeros((4, bs, Hkv, D), dtype=torch.float16, device="cuda")
    tables = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(binding.PaError) as e:
        binding.decode_no_alloc(out, q, k, k, tables, lens, 0.1)
    assert e.value.status == 4                     # PA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
