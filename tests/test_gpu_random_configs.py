"""Seeded random configurations: HIP path vs the fp64 oracle through the C ABI.

Each case draws, from a fixed seed, an entry point (slidingDecodeGQA,
decodeGQA, the runtime-window sliding call, or decodeGQA over a values-only
cache), a dtype, a cache form, a batch size and a capacity. The per-sequence
lengths mix 0, 1, the capacity, page and tile edges and uniform draws. Every
output element is compared with the oracle at the usual tolerances: max-abs
1e-4 for float32 inputs and 2e-2 for bfloat16 inputs. The configurations span
both launch modes and the window edge, at sizes the oracle finishes in seconds.
"""
import numpy as np
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import synth
from gpu_cases import (TOL, hip_run, hip_run_k_eq_v, max_err, oracle_run, oracle_run_k_eq_v,
                       to_f64, to_gpu)

pytestmark = pytest.mark.gpu

KINDS = ("sliding", "global", "window", "k_eq_v")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


def draw_config(i: int):
    rng = np.random.default_rng(7000 + i)
    kind = KINDS[i % len(KINDS)]
    dtype = ("f32", "bf16")[int(rng.integers(2))]
    paged = bool(rng.integers(2))
    B = int(rng.choice([1, 2, 3, 5, 8, 17, 32, 48]))
    cap = int(rng.integers(1, 2600 if kind in ("global", "k_eq_v") else 3200))
    if paged:
        cap = -(-cap // 16) * 16  # a paged capacity is whole pages
    specials = [0, 1, 15, 16, 17, cap, max(cap - 1, 0), min(1024, cap), min(1025, cap)]
    lens = [int(rng.choice(specials)) if rng.random() < 0.4 else int(rng.integers(0, cap + 1))
            for _ in range(B)]
    window = int(rng.choice([1, 7, 16, 100, 1023, 2048, 4000])) if kind == "window" else None
    return kind, dtype, paged, B, cap, lens, window


@pytest.mark.parametrize("i", range(24))
def test_random_config_parity(i):
    kind, dtype, paged, B, cap, lens, window = draw_config(i)
    variant = "sliding" if kind in ("sliding", "window") else "global"
    print(f"case {i}: {kind} {dtype} paged={paged} B={B} cap={cap} window={window}", flush=True)
    c = synth.make_case(variant, dtype, B, cap, lens, paged=paged, seed=9000 + i, window=window,
                        extra_pages=3)
    if kind == "k_eq_v":
        ref = oracle_run_k_eq_v(c)
        got = to_f64(hip_run_k_eq_v(to_gpu(c)))
    else:
        ref = oracle_run(c, window=window)
        got = to_f64(hip_run(to_gpu(c), window=window))
    err = max_err(got, ref)
    assert err <= TOL[dtype], (i, kind, dtype, paged, B, cap, lens, window, err)
