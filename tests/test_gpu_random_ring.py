"""Seeded random ring-cache configurations vs the fp64 oracle.

The sliding layers' cache can be capped at R positions: position s lives in
slot s mod R. Each case draws, from a fixed seed:
- a ring size R (a multiple of 16 from 16 to 4096, powers of two and others) and a window W <= R;
- 1 to 40 sequences, a dtype;
- lengths mixing 1, W, R, their neighbours, many wraps, and the longest
  sequence the library accepts (262144).

Every output element is compared with the oracle at the usual tolerances.
Never-written slots hold NaN and must never be read.
"""
import numpy as np
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import oracle
import synth
from gpu_cases import TOL, max_err, to_f64

pytestmark = pytest.mark.gpu


def draw_ring_config(i: int):
    rng = np.random.default_rng(8500 + i)
    R = int(rng.choice([16, 48, 112, 512, 1008, 1024, 2048, 3008, 4096]))  # whole pages
    W = int(rng.choice([1, 2, R // 2 or 1, R - 1 or 1, R]))
    dtype = ("f32", "bf16")[int(rng.integers(2))]
    B = int(rng.integers(1, 41))
    specials = [1, W, W + 1, R - 1 or 1, R, R + 1, 3 * R + 5, 262144]
    lens = [int(rng.choice(specials)) if rng.random() < 0.5 else int(rng.integers(1, 20000))
            for _ in range(B)]
    return R, W, dtype, lens


@pytest.mark.parametrize("i", range(12))
def test_random_ring_parity(i):
    R, W, dtype, lens = draw_ring_config(i)
    print(f"case {i}: ring={R} window={W} {dtype} B={len(lens)}", flush=True)
    c = synth.make_ring_case(dtype, len(lens), R, lens, seed=9800 + i, window=W)
    got = to_f64(gqa.gqa_decode_sliding_ring(*(x.cuda() for x in (c.q, c.k, c.v, c.seq_lens)),
                                             window=W))
    torch.cuda.synchronize()
    assert np.isfinite(got).all()
    ref = oracle.gqa_decode_ring(*(synth.to_numpy(x) for x in (c.q, c.k, c.v, c.seq_lens)),
                                 window=W)
    err = max_err(got, ref)
    assert err <= TOL[dtype], (i, R, W, dtype, lens, err)
