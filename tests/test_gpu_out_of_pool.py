"""Block-table entries outside the page pool (a device-resident precondition
the host cannot check): their positions are dropped, and nothing the kernels
read in their place reaches the output.

The kernels read physical page 0 in place of a page id outside
[0, num_pages) and must select its rows out, never multiply them by a zero
weight (0 * NaN = NaN): a real cache's page 0 may hold stale data.  Each case
makes physical page 0 a page no block-table entry references, points one
attended page of a sequence outside the pool, and runs the call twice, with
page 0 all NaN and all zero.  The outputs must be finite and bit-identical,
and must match the oracle on the same cache with that page's positions
removed (a contiguous copy of each sequence's remaining rows in order; for
decodeGQA and causal prefill that is the same set of keys in the same order,
the definition's sum without those positions).
"""
import numpy as np
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import oracle
import synth
from gpu_cases import TOL, hip_run, max_err, oracle_run, to_f64, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


def _free_page0(k, v, bt):
    """Swap physical pages so that page 0 is referenced by no block-table entry."""
    used = set(bt[bt >= 0].tolist())
    u = next(p for p in range(k.shape[0]) if p not in used)
    if u != 0:
        k[[0, u]] = k[[u, 0]]
        v[[0, u]] = v[[u, 0]]
        bt[bt == 0] = u
    return k, v, bt


def _with_page0(k, v, fill):
    k, v = k.clone(), v.clone()
    k[0] = fill
    v[0] = fill
    return k, v


def _compact(k, v, bt, lens, drop):
    """Contiguous [B, cap, KV, D] copy of each sequence's rows in position
    order, without the positions of the (sequence, logical page) pairs in
    `drop`; returns k, v and the shortened lengths."""
    B = bt.shape[0]
    KV, D = k.shape[2], k.shape[3]
    cap = bt.shape[1] * 16
    kc = torch.full((B, cap, KV, D), float("nan"), dtype=k.dtype)
    vc = torch.full_like(kc, float("nan"))
    out_lens = []
    for b in range(B):
        L = int(lens[b])
        n = 0
        for p in range((L + 15) // 16):
            if (b, p) in drop:
                continue
            cnt = min(16, L - 16 * p)
            kc[b, n:n + cnt] = k[int(bt[b, p]), :cnt]
            vc[b, n:n + cnt] = v[int(bt[b, p]), :cnt]
            n += cnt
        out_lens.append(n)
    return kc, vc, torch.tensor(out_lens, dtype=torch.int32)


BAD_IDS = lambda num_pages: (num_pages, num_pages + 1000, -1, -7)  # noqa: E731


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,cap,mode", [(3, 4096, "group"), (64, 512, "unit")],
                         ids=["group", "unit"])
def test_decode_global_drops_out_of_pool_pages(B, cap, mode, dtype):
    assert gqa.gqa_decode_plan("global", B, cap)["mode"] == mode
    lens = synth.draw_seq_lens(("uniform", 40, cap), B, 51).tolist()
    lens[0] = cap
    c = synth.make_case("global", dtype, B, cap, lens, paged=True, seed=400, extra_pages=3)
    k, v, bt = _free_page0(c.k, c.v, c.block_table.clone())
    num_pages = k.shape[0]
    drop = {}
    for i, b in enumerate(range(min(B, 4))):
        p = (int(lens[b]) // 16) // 2          # a full page in the middle of the range
        drop[(b, p)] = BAD_IDS(num_pages)[i % 4]
    for (b, p), bad in drop.items():
        bt[b, p] = bad
    outs = []
    for fill in (float("nan"), 0.0):
        kf, vf = _with_page0(k, v, fill)
        case = synth.Case("global", dtype, c.q, kf, vf, c.seq_lens, bt, cap, 0)
        outs.append(hip_run(to_gpu(case)).cpu())
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1])
    kc, vc, lc = _compact(k, v, bt, c.seq_lens, set(drop))
    ref = oracle_run(synth.Case("global", dtype, c.q, kc, vc, lc, None, cap, 0))
    assert max_err(to_f64(outs[0]), ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,cap,mode", [(2, 4096, "stream"), (8, 1104 + 16, "unit")],
                         ids=["stream", "unit"])
def test_decode_sliding_drops_out_of_pool_pages(B, cap, mode, dtype):
    assert gqa.gqa_decode_plan("sliding", B, cap)["mode"] == mode
    lens = synth.draw_seq_lens(("uniform", 600, cap), B, 52).tolist()
    lens[0] = cap
    c = synth.make_case("sliding", dtype, B, cap, lens, paged=True, seed=401, extra_pages=3,
                        alloc_all_pages=True)
    k, v, bt = _free_page0(c.k, c.v, c.block_table.clone())
    num_pages = k.shape[0]
    drop = {}
    for i, b in enumerate(range(min(B, 4))):
        lo, L = c.attended(b)
        p = ((lo + L) // 2) // 16
        drop[(b, p)] = BAD_IDS(num_pages)[i % 4]
    for (b, p), bad in drop.items():
        bt[b, p] = bad
    outs = []
    for fill in (float("nan"), 0.0):
        kf, vf = _with_page0(k, v, fill)
        case = synth.Case("sliding", dtype, c.q, kf, vf, c.seq_lens, bt, cap, 1024)
        outs.append(hip_run(to_gpu(case)).cpu())
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1])
    # the oracle over each window's rows without the dropped page (re-based so
    # that the window is exactly the kept rows: window 0 on the compact copy)
    G = 2
    for b in range(B):
        lo, L = c.attended(b)
        keep = [s for s in range(lo, L) if (b, s // 16) not in drop]
        rows_k = torch.stack([k[int(bt[b, s // 16]), s % 16] for s in keep])[None]
        rows_v = torch.stack([v[int(bt[b, s // 16]), s % 16] for s in keep])[None]
        sub = synth.Case("sliding", dtype, c.q[b:b + 1], rows_k, rows_v,
                         torch.tensor([len(keep)], dtype=torch.int32), None, len(keep), 0)
        ref = oracle_run(sub, window=0)
        assert max_err(to_f64(outs[0][b:b + 1]), ref) <= TOL[dtype], (b, G)


def _prefill(variant, q, k, v, cu, sl, bt):
    fn = gqa.gqa_prefill_sliding if variant == "sliding" else gqa.gqa_prefill_global
    return fn(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), sl.cuda(), block_table=bt.cuda())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_prefill_drops_out_of_pool_pages(variant, dtype):
    cap = 1600
    lens, q_lens = [1600, 900], [300, 64]
    pc = synth.make_prefill_case(variant, dtype, cap, lens, q_lens, paged=True, seed=402,
                                 extra_pages=3, window=0 if variant == "global" else None)
    k, v, bt = _free_page0(pc.k, pc.v, pc.block_table.clone())
    num_pages = k.shape[0]
    # a page of the past every chunk row attends to (below the chunk; for the
    # sliding layer inside every row's window)
    drop = {(0, 1290 // 16): num_pages + 3, (1, 500 // 16): -2}
    for (b, p), bad in drop.items():
        bt[b, p] = bad
    outs = []
    for fill in (float("nan"), 0.0):
        kf, vf = _with_page0(k, v, fill)
        outs.append(_prefill(variant, pc.q, kf, vf, pc.cu_q, pc.seq_lens, bt).cpu())
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1])
    if variant == "global":
        # causal prefill: every row's keys are [0, p] without the dropped page,
        # which lies below every row, so the compact copy shifts rows and keys alike
        kc, vc, lc = _compact(k, v, bt, pc.seq_lens, set(drop))
        ref = oracle.gqa_prefill("global", synth.to_numpy(pc.q), synth.to_numpy(kc),
                                 synth.to_numpy(vc), synth.to_numpy(pc.cu_q), lc.numpy(),
                                 nthreads=16)
        assert max_err(to_f64(outs[0]), ref) <= TOL[dtype]
