"""The decode and prefill steps captured in a HIP graph and replayed.

A serving loop captures its steps once and replays them; every call on the
path must then be capturable: no allocation, no host synchronisation, no
memset node (the arrival counters are cleared by the kernels themselves).
Each case runs the step eagerly, captures the same step (copy-on-write
copies, cache write, attention and the combine) on a side stream, and
replays it four times with eager work and synchronisations between the
replays.  Every replay must give the eager step's outputs bit for bit, and
the pools and outputs must match the oracle.  The steps are idempotent, so
replaying one leaves the same state as running it once.
"""

from dataclasses import replace

import pytest
import torch

from paged_kv_cache_412_amd import binding, workloads
from paged_kv_cache_412_amd.step import DecodeStep, PrefillStep
from tests import parity
from tests.test_gpu_parity import COMBINES, COOP, SMALL, check_step
from tests.test_gpu_prefill import SMALL as PREFILL_SMALL
from tests.test_gpu_prefill import check as check_prefill

pytestmark = pytest.mark.gpu

REPLAYS = 4


def capture(run):
    """The graph of one call of `run`, captured after a warm-up call on the
    side stream that capture uses."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    return g


def replay_matches(g, out, eager):
    for i in range(REPLAYS):
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), eager.view(torch.uint8)), f"replay {i} differs"


DECODE = {"llama13b": SMALL["llama13b"], "llama70b": SMALL["llama70b"], "shared": SMALL["shared"],
          "long_fp8": SMALL["long_fp8"], "coop_e4m3": COOP["coop_e4m3"],
          "llama13b_bs8": SMALL["llama13b_bs8"], "long_fp8_bs64": SMALL["long_fp8_bs64"],
          # past the 1,024 sequences one work-group's plan covers: the plan kernel runs too
          "many_short": replace(SMALL["llama70b"], name="many_short", B=1100,
                                lens=tuple(i % 70 for i in range(1100)), len_range=(), pool_blocks=0)}


@pytest.mark.parametrize("mode", ["auto"] + list(COMBINES))
@pytest.mark.parametrize("part", [0, 64])
@pytest.mark.parametrize("name", list(DECODE))
def test_decode_step_replays_from_a_graph(name, part, mode):
    cfg = DECODE[name]
    if part % cfg.block_size:
        part = cfg.block_size
    combine = binding.PA_COMBINE_AUTO if mode == "auto" else COMBINES[mode]
    print(f"\n[case] graph decode {name} part={part} combine={mode}", flush=True)
    wl = workloads.make(cfg, device="cuda")
    pre = parity.snapshot(wl)
    step = DecodeStep(wl, partition_size=part, out_dtype="f32", combine=combine)
    step.run()
    torch.cuda.synchronize()
    eager = step.out.clone()
    g = capture(step.run)
    replay_matches(g, step.out, eager)
    exp = parity.oracle_step(wl, pre)
    err = check_step(wl, step, exp, out_dtype="f32")
    print(f"[ok] {name} part={part} combine={mode}: {REPLAYS} replays bit-equal, "
          f"max abs err {err:.3e}", flush=True)


@pytest.mark.parametrize("name", ["prefill13b", "prefill70b", "prefill_fp8", "prefill70b_bs8"])
def test_prefill_step_replays_from_a_graph(name):
    cfg = PREFILL_SMALL[name]
    print(f"\n[case] graph prefill {name}", flush=True)
    wl = workloads.make_prefill(cfg, device="cuda")
    pre = parity.snapshot(wl)
    step = PrefillStep(wl, out_dtype="f32")
    step.run()
    torch.cuda.synchronize()
    eager = step.out.clone()
    g = capture(step.run)
    replay_matches(g, step.out, eager)
    exp = parity.oracle_prefill(wl, pre)
    err = check_prefill(wl, step, exp, out_dtype="f32")
    print(f"[ok] {name}: {REPLAYS} replays bit-equal, max abs err {err:.3e}", flush=True)
