"""GPU: seeded random sweeps of decode steps and prefill calls against the
fp64 oracle.

The hand-picked parity cases fix a few head counts and length sets; here
each case draws its own shape from the supported set -- KV heads 1..12 (most
not a multiple of a work-group's heads), group size, head dim, block size,
dtype pair (new-row source dtype included), output dtype, batch 1..24 with
lengths 0..2500, the balanced or a fixed partition size, per-head scales for
8-bit caches, query spread -- and runs the whole step (slot mapping,
copy-on-write, cache write, partitions, reduce).  The prefill sweep draws
group size 1..16, KV heads, head dim, block size, dtype pair, new-token and
cached-context ranges and query scale, and runs slot mapping, cache write
and causal paged attention.  Same bars as the parity suites: slots and pools
bit-exact, every output within the KV dtype's tolerance plus half an ulp of
the output dtype.
"""

import numpy as np
import pytest

from paged_kv_cache_412_amd import workloads
from tests.test_gpu_parity import check_step, run_step

pytestmark = pytest.mark.gpu

PAIRS = [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"), ("bf16", "e4m3"), ("f16", "e4m3"),
         ("bf16", "e5m2"), ("f16", "e5m2")]
CASES = 200


def draw(i):
    rng = np.random.default_rng(41_200 + i)
    qd, kvd = PAIRS[int(rng.integers(len(PAIRS)))]
    fp8 = kvd in ("e4m3", "e5m2")
    G = int(rng.choice([1, 2, 4, 8])) if kvd == "f32" else int(rng.integers(1, 17))
    Hkv = int(rng.integers(1, 13))
    while G * Hkv > 48:
        Hkv -= 1
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32, 64]))
    B = int(rng.integers(1, 25))
    lens = rng.integers(0, 2501, size=B)
    lens[rng.random(B) < 0.15] = 0                        # empty sequences
    edge = rng.random(B) < 0.2                             # block-boundary lengths
    lens[edge] = (rng.integers(0, 40, size=int(edge.sum())) * bs + rng.integers(-1, 2, size=int(edge.sum())))
    lens = np.clip(lens, 0, 2500)
    if rng.random() < 0.6:
        part = 0
    else:
        unit = max(bs, 16)
        part = unit * int(rng.integers(1, 1024 // unit + 1))
    src = str(rng.choice(["f32", "f16", "bf16"])) if fp8 else kvd
    sigma = float(rng.choice([1.0, 4.0]))
    out = "f32" if (sigma > 1 or rng.random() < 0.3) else qd
    cfg = workloads.Config(f"sweep{i}-{qd}-{kvd}-G{G}-Hkv{Hkv}-D{D}-bs{bs}", 1000 + i, B=B, Hq=G * Hkv,
                           Hkv=Hkv, D=D, block_size=bs, kv_dtype=kvd, q_dtype=qd, out_dtype=qd,
                           src_dtype=src, lens=tuple(int(x) for x in lens),
                           head_scales=bool(fp8 and rng.random() < 0.3))
    return cfg, part, out, sigma


@pytest.mark.parametrize("i", range(CASES))
def test_random_decode_step(i):
    cfg, part, out, sigma = draw(i)
    wl, step, exp = run_step(cfg, partition_size=part, out_dtype=out, q_sigma=sigma)
    err = check_step(wl, step, exp, out_dtype=out)
    print(f"[ok] {cfg.name} part={part} out={out} sigma={sigma} max abs err {err:.3e}", flush=True)


PREFILL_PAIRS = [p for p in PAIRS if p[1] != "f32"]
PREFILL_CASES = 60


def draw_prefill(i):
    rng = np.random.default_rng(41_700 + i)
    qd, kvd = PREFILL_PAIRS[int(rng.integers(len(PREFILL_PAIRS)))]
    fp8 = kvd in ("e4m3", "e5m2")
    G = int(rng.integers(1, 17))
    Hkv = int(rng.integers(1, 7))
    while G * Hkv > 24:
        Hkv -= 1
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32, 64]))
    B = int(rng.integers(1, 4))
    n_hi = int(rng.integers(1, 201))
    c_hi = int(rng.choice([0, int(rng.integers(1, 301))]))
    q_scale = float(rng.choice([1.0, 4.0]))
    out = "f32" if (q_scale > 1 or rng.random() < 0.3) else qd
    cfg = workloads.Config(f"psweep{i}-{qd}-{kvd}-G{G}-Hkv{Hkv}-D{D}-bs{bs}", 1500 + i, B=B, Hq=G * Hkv,
                           Hkv=Hkv, D=D, block_size=bs, kv_dtype=kvd, q_dtype=qd, out_dtype=qd,
                           src_dtype=qd, prefill=dict(new=(1, n_hi), ctx=(0, c_hi)),
                           head_scales=bool(fp8 and rng.random() < 0.3))
    return cfg, out, q_scale


@pytest.mark.parametrize("i", range(PREFILL_CASES))
def test_random_prefill_call(i):
    from tests.test_gpu_prefill import check, run
    cfg, out, q_scale = draw_prefill(i)
    wl, step, exp = run(cfg, out_dtype=out, q_scale=q_scale)
    err = check(wl, step, exp, out_dtype=out)
    print(f"[ok] {cfg.name} out={out} q_scale={q_scale} max abs err {err:.3e}", flush=True)
