"""KV append (norms + RoPE of the new token, cache write) vs the fp64 oracle,
through the C ABI, on an MI355X."""
import numpy as np
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import oracle
import synth
from gpu_cases import TOL, hip_run, max_err, oracle_run, to_f64, to_gpu

pytestmark = pytest.mark.gpu
HEADS = 32
GEOM = {"sliding": (16, 256), "global": (4, 512)}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


def raw_token(variant, dtype, B, seed):
    KV, D = GEOM[variant]
    g = torch.Generator().manual_seed(seed)
    tdt = synth.TORCH_DTYPES[dtype]
    q = (torch.randn(B, HEADS, D, generator=g) * 2).to(tdt)
    k = (torch.randn(B, KV, D, generator=g) * 3).to(tdt)
    v = torch.randn(B, KV, D, generator=g).to(tdt)
    wq = torch.empty(D).uniform_(0.2, 0.4, generator=g).to(tdt)
    wk = torch.empty(D).uniform_(0.2, 0.4, generator=g).to(tdt)
    return q, k, v, wq, wk


def oracle_rows(variant, q, k, v, wq, wk, lens):
    n = synth.to_numpy
    return oracle.gqa_append_rows(variant, n(q), n(k), None if variant == "global" else n(v),
                                  n(wq), n(wk), np.asarray(lens, dtype=np.int32))


def run_append(variant, q, k, v, wq, wk, lens, kc, vc, bt=None, q_out=None):
    d = "cuda"
    args = [q.to(d), k.to(d)] + ([v.to(d)] if variant == "sliding" else []) + \
        [wq.to(d), wk.to(d), torch.as_tensor(lens, dtype=torch.int32).to(d), kc, vc]
    fn = gqa.gqa_append_sliding if variant == "sliding" else gqa.gqa_append_global
    return fn(*args, block_table=bt, q_out=q_out)


def cache_row(cache, bt, b, pos):
    if bt is None:
        return cache[b, pos]
    return cache[int(bt[b, pos // 16]), pos % 16]


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_append_parity(variant, dtype, paged):
    KV, D = GEOM[variant]
    cap = 262144 if paged else 320
    lens = [1, 17, cap, 0, 160, cap - 15] if not paged else [1, 17, cap, 0, 131072, 99999]
    B = len(lens)
    q, k, v, wq, wk = raw_token(variant, dtype, B, seed=300)
    tdt = synth.TORCH_DTYPES[dtype]
    if paged:
        # one physical page per sequence, holding the new token's slot
        npages = B + 3
        perm = torch.randperm(npages, generator=torch.Generator().manual_seed(301))
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
    assert max_err(to_f64(q_out), eq) <= TOL[dtype]
    kc2, vc2 = kc_d.cpu(), vc_d.cpu()
    for b, L in enumerate(lens):
        if L < 1:
            assert torch.count_nonzero(q_out[b]) == 0
            continue
        p = int(pos[b])
        assert max_err(cache_row(kc2, bt, b, p).double().numpy(), ek[b]) <= TOL[dtype], (b, L)
        assert max_err(cache_row(vc2, bt, b, p).double().numpy(), ev[b]) <= TOL[dtype], (b, L)
        # mark the written rows, then every other byte must be untouched
        cache_row(kc2, bt, b, p).fill_(float("nan"))
        cache_row(vc2, bt, b, p).fill_(float("nan"))
    for got, orig in ((kc2, kc), (vc2, vc)):
        assert torch.equal(got.view(torch.int16 if dtype == "bf16" else torch.int32),
                           orig.view(torch.int16 if dtype == "bf16" else torch.int32))


def test_append_q_in_place():
    q, k, v, wq, wk = raw_token("sliding", "bf16", 3, seed=302)
    lens = [5, 1, 64]
    kc = torch.zeros(3, 64, 16, 256, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    ref = run_append("sliding", q, k, v, wq, wk, lens, kc.clone(), vc.clone()).cpu()
    qd = q.cuda()
    out = run_append("sliding", qd, k, v, wq, wk, lens, kc, vc, q_out=qd)
    assert out.data_ptr() == qd.data_ptr()
    assert torch.equal(out.cpu(), ref)


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_append_then_attend(variant, paged):
    """Append the new token on the GPU, then attend; the oracle appends the same
    token (fp64) into a copy of the cache and attends."""
    KV, D = GEOM[variant]
    lens = [1300, 1, 700, 1025]
    cap = 1312
    c = synth.make_case(variant, "bf16", 4, cap, lens, paged=paged, seed=303, fill=0.0,
                        alloc_all_pages=True)
    q, k, v, wq, wk = raw_token(variant, "bf16", 4, seed=304)
    g = to_gpu(c)
    q_out = run_append(variant, q, k, v, wq, wk, lens, g.k, g.v, g.block_table)
    o = hip_run(synth.Case(c.variant, c.dtype, q_out, g.k, g.v, g.seq_lens, g.block_table,
                           c.cap, c.window))
    eq, ek, ev, pos = oracle_rows(variant, q, k, v, wq, wk, lens)
    host = synth.Case(c.variant, c.dtype, torch.from_numpy(eq).to(torch.bfloat16), c.k.clone(),
                      c.v.clone(), c.seq_lens, c.block_table, c.cap, c.window)
    for b in range(4):
        p = int(pos[b])
        cache_row(host.k, c.block_table, b, p).copy_(torch.from_numpy(ek[b]).to(torch.bfloat16))
        cache_row(host.v, c.block_table, b, p).copy_(torch.from_numpy(ev[b]).to(torch.bfloat16))
    err = max_err(to_f64(o), oracle_run(host))
    assert err <= TOL["bf16"], err
