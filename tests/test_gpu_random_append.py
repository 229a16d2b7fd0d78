"""Seeded random KV-append configurations vs the fp64 oracle.

Each case draws, from a fixed seed:
- a variant, a dtype and a cache form;
- 1 to 64 sequences and a capacity: contiguous up to 1,024 positions, paged up to 262,144;
- per sequence a length mixing 0, 1, page edges, the capacity and uniform draws.

The new token's query (RMS-normed, weighted, rotated) and its cache rows are
compared with the oracle. Every other byte of the cache must be left
untouched, and a sequence of length 0 writes nothing and returns a zero query.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_cases import TOL, max_err, to_f64
from test_gpu_append import GEOM, cache_row, oracle_rows, raw_token, run_append

pytestmark = pytest.mark.gpu


def draw_append_config(i: int):
    rng = np.random.default_rng(8800 + i)
    variant = ("sliding", "global")[i % 2]
    dtype = ("f32", "bf16")[int(rng.integers(2))]
    paged = bool(rng.integers(2))
    B = int(rng.integers(1, 65))
    cap = 16 * int(rng.integers(1, 16385)) if paged else int(rng.integers(1, 1025))
    specials = [0, 1, 15, 16, 17, cap, max(cap - 1, 1), max(cap - 16, 1)]
    lens = [int(rng.choice(specials)) if rng.random() < 0.4 else int(rng.integers(0, cap + 1))
            for _ in range(B)]
    return variant, dtype, paged, cap, lens


@pytest.mark.parametrize("i", range(12))
def test_random_append_parity(i):
    variant, dtype, paged, cap, lens = draw_append_config(i)
    print(f"case {i}: {variant} {dtype} paged={paged} cap={cap} B={len(lens)}", flush=True)
    KV, D = GEOM[variant]
    B = len(lens)
    q, k, v, wq, wk = raw_token(variant, dtype, B, seed=8900 + i)
    tdt = synth.TORCH_DTYPES[dtype]
    if paged:
        # one physical page per sequence, holding the new token's slot
        npages = B + 2
        perm = torch.randperm(npages, generator=torch.Generator().manual_seed(8950 + i))
        bt = torch.full((B, cap // 16), -1, dtype=torch.int32)
        for b, L in enumerate(lens):
            if L >= 1:
                bt[b, (L - 1) // 16] = int(perm[b])
        kc = torch.full((npages, 16, KV, D), float("nan"), dtype=tdt)
        bt_d = bt.cuda()
    else:
        bt, bt_d = None, None
        kc = torch.full((B, cap, KV, D), float("nan"), dtype=tdt)
    vc = kc.clone()
    kc_d, vc_d = kc.cuda(), vc.cuda()
    q_out = run_append(variant, q, k, v, wq, wk, lens, kc_d, vc_d, bt_d)
    torch.cuda.synchronize()
    eq, ek, ev, pos = oracle_rows(variant, q, k, v, wq, wk, lens)
    live = [b for b, L in enumerate(lens) if L >= 1]
    if live:
        assert max_err(to_f64(q_out)[live], eq[live]) <= TOL[dtype], i
    kc2, vc2 = kc_d.cpu(), vc_d.cpu()
    for b, L in enumerate(lens):
        if L < 1:
            assert torch.count_nonzero(q_out[b]) == 0, (i, b)
            continue
        p = int(pos[b])
        assert max_err(cache_row(kc2, bt, b, p).double().numpy(), ek[b]) <= TOL[dtype], (i, b, L)
        assert max_err(cache_row(vc2, bt, b, p).double().numpy(), ev[b]) <= TOL[dtype], (i, b, L)
        cache_row(kc2, bt, b, p).fill_(float("nan"))
        cache_row(vc2, bt, b, p).fill_(float("nan"))
    view = torch.int16 if dtype == "bf16" else torch.int32
    for got, orig in ((kc2, kc), (vc2, vc)):
        assert torch.equal(got.view(view), orig.view(view)), i
