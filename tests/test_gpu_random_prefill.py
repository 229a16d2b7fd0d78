"""Seeded random prefill / chunked-prefill configurations vs the fp64 oracle.

Each case draws, from a fixed seed:
- an entry point: sliding, global, or the runtime-window sliding call;
- a dtype and a cache form;
- 1 to 6 sequences, a capacity, and per sequence a cache length and a chunk length.

The chunk lengths include empty chunks, single tokens, a whole fresh prompt
and, now and then, a chunk longer than the sequence, whose rows before
position 0 are zero. Every output element is compared with the oracle at the
usual tolerances, and the rows outside every attended range, filled with NaN,
must never be read.
"""
import numpy as np
import pytest

import decode_attention_slidingdecodegqa_amd as gqa
import synth
from gpu_cases import TOL, max_err, to_f64
from test_gpu_prefill import hip_prefill, oracle_prefill, to_gpu

pytestmark = pytest.mark.gpu

KINDS = ("sliding", "global", "window")


def draw_prefill_config(i: int):
    rng = np.random.default_rng(8000 + i)
    kind = KINDS[i % len(KINDS)]
    dtype = ("f32", "bf16")[int(rng.integers(2))]
    paged = bool(rng.integers(2))
    B = int(rng.integers(1, 7))
    cap = int(rng.integers(1, 1200 if kind == "global" else 2400))
    if paged:
        cap = -(-cap // 16) * 16  # a paged capacity is whole pages
    lens, q_lens = [], []
    for _ in range(B):
        L = int(rng.choice([0, 1, 17, cap])) if rng.random() < 0.3 else int(rng.integers(0, cap + 1))
        u = rng.random()
        if u < 0.15:
            T = 0
        elif u < 0.3:
            T = min(1, L)
        elif u < 0.4:
            T = L  # a fresh prompt
        elif u < 0.45:
            T = L + int(rng.integers(1, 4))  # longer than the sequence: leading zero rows
        else:
            T = int(rng.integers(0, min(L, 160) + 1))
        lens.append(L)
        q_lens.append(T)
    window = int(rng.choice([1, 5, 64, 1023, 2048])) if kind == "window" else None
    return kind, dtype, paged, cap, lens, q_lens, window


@pytest.mark.parametrize("i", range(18))
def test_random_prefill_parity(i):
    kind, dtype, paged, cap, lens, q_lens, window = draw_prefill_config(i)
    variant = "global" if kind == "global" else "sliding"
    print(f"case {i}: {kind} {dtype} paged={paged} cap={cap} lens={lens} q_lens={q_lens} "
          f"window={window}", flush=True)
    c = synth.make_prefill_case(variant, dtype, cap, lens, q_lens, paged=paged, seed=9500 + i,
                                window=window, extra_pages=3)
    d = to_gpu(c)
    if kind == "window":
        got = to_f64(gqa.gqa_prefill_sliding_window(d.q, d.k, d.v, d.cu_q, d.seq_lens, window,
                                                    block_table=d.block_table))
    else:
        got = to_f64(hip_prefill(d))
    assert np.isfinite(got).all()
    err = max_err(got, oracle_prefill(c)) if got.size else 0.0
    assert err <= TOL[dtype], (i, kind, dtype, paged, cap, lens, q_lens, window, err)
