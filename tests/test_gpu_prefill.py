"""Prefill / chunked prefill (a chunk of new tokens per sequence, causal and
sliding masks) vs the fp64 oracle, through the C ABI, on an MI355X."""
import numpy as np
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import oracle
import synth
from gpu_cases import TOL, max_err, to_f64

pytestmark = pytest.mark.gpu
HEADS = 32


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


def to_gpu(c: synth.PrefillCase) -> synth.PrefillCase:
    d = "cuda"
    return synth.PrefillCase(c.variant, c.dtype, c.q.to(d), c.k.to(d), c.v.to(d), c.cu_q.to(d),
                             c.seq_lens.to(d),
                             None if c.block_table is None else c.block_table.to(d), c.cap,
                             c.window)


def to_cpu(c: synth.PrefillCase) -> synth.PrefillCase:
    return synth.PrefillCase(c.variant, c.dtype, c.q.cpu(), c.k.cpu(), c.v.cpu(), c.cu_q.cpu(),
                             c.seq_lens.cpu(),
                             None if c.block_table is None else c.block_table.cpu(), c.cap,
                             c.window)


def hip_prefill(c: synth.PrefillCase, o=None, stream=None) -> torch.Tensor:
    fn = gqa.gqa_prefill_sliding if c.variant == "sliding" else gqa.gqa_prefill_global
    return fn(c.q, c.k, c.v, c.cu_q, c.seq_lens, block_table=c.block_table, o=o, stream=stream)


def oracle_prefill(c: synth.PrefillCase, rows=None) -> np.ndarray:
    n = synth.to_numpy
    bt = None if c.block_table is None else n(c.block_table)
    return oracle.gqa_prefill((c.KV, c.D, c.window), n(c.q), n(c.k), n(c.v), n(c.cu_q),
                              n(c.seq_lens), block_table=bt, rows=rows, nthreads=16)


# lengths: a chunk after a long past (crossing the window), a fresh prompt, a
# single token, an empty chunk, a chunk starting at position 0 with the cache
# full
CASES = {
    "sliding": dict(cap=2112, seq_lens=[1300, 40, 7, 900, 2100], q_lens=[77, 40, 1, 0, 300]),
    "global": dict(cap=720, seq_lens=[700, 33, 1, 260, 64], q_lens=[50, 33, 1, 0, 64]),
}


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_prefill_parity(variant, dtype, paged):
    kw = CASES[variant]
    c = synth.make_prefill_case(variant, dtype, kw["cap"], kw["seq_lens"], kw["q_lens"],
                                paged=paged, seed=500, extra_pages=3)
    got = to_f64(hip_prefill(to_gpu(c)))
    assert np.isfinite(got).all()  # NaN outside every attended range is never read
    err = max_err(got, oracle_prefill(c))
    assert err <= TOL[dtype], err


def test_prefill_fresh_prompt_first_token_exact():
    # position 0 attends only to itself: o = v[0] bit for bit
    for variant, G in (("sliding", 2), ("global", 8)):
        c = synth.make_prefill_case(variant, "bf16", 64, [20, 64], [20, 64], seed=501)
        got = hip_prefill(to_gpu(c)).cpu()
        for b, n in enumerate((0, 20)):
            for h in range(HEADS):
                assert torch.equal(got[n, h], c.v[b, 0, h // G])


def test_prefill_paged_equals_contiguous():
    for variant in ("sliding", "global"):
        kw = dict(seed=502, fill=0.0)
        a = synth.make_prefill_case(variant, "bf16", 1040, [1040, 300], [200, 300], **kw)
        b = synth.make_prefill_case(variant, "bf16", 1040, [1040, 300], [200, 300], paged=True,
                                    **kw)
        assert torch.equal(hip_prefill(to_gpu(a)).cpu(), hip_prefill(to_gpu(b)).cpu())


def test_prefill_deterministic_on_a_side_stream():
    c = to_gpu(synth.make_prefill_case("global", "bf16", 1024, [1024, 512], [300, 100],
                                       seed=503))
    a = hip_prefill(c).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o = torch.full_like(c.q, float("nan"))
        b = hip_prefill(c, o=o, stream=s)
    s.synchronize()
    assert torch.equal(a, b)


def test_prefill_profile_kind():
    c = to_gpu(synth.make_prefill_case("sliding", "bf16", 256, [256], [64], seed=504))
    gqa.profile_begin(8)
    hip_prefill(c)
    res = gqa.profile_read()
    assert res[("sliding", "prefill")][0] == 1 and res[("global", "prefill")][0] == 0


@pytest.mark.parametrize("name", sorted(synth.PREFILL_WORKLOADS))
def test_prefill_workload_sampled(name):
    c = synth.make_prefill_workload(name, seed=0, device="cuda")
    got = hip_prefill(c)
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all()
    host = to_cpu(c)
    cu = host.cu_q.tolist()
    # first, middle and last query rows of the first and last sequence, a few heads
    ns = sorted({cu[0], (cu[0] + cu[1]) // 2, cu[1] - 1, cu[-2], cu[-1] - 1})
    rows = [(n, h) for n in ns for h in (0, 7, 8, 31)]
    ref = oracle_prefill(host, rows=rows)
    g = to_f64(got)
    for i, (n, h) in enumerate(rows):
        assert max_err(g[n, h], ref[i]) <= TOL["bf16"], (name, n, h)


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_prefill_many_sequences(variant):
    # B = 256 sequences (the whole work-group prefix over cu_q), chunks of 0..40
    # tokens after pasts of 0..1500 positions; sampled rows vs the oracle
    g = torch.Generator().manual_seed(505)
    B, cap = 256, 1552
    q_lens = torch.randint(0, 41, (B,), generator=g)
    past = torch.randint(0, 1501, (B,), generator=g)
    lens = (past + q_lens).clamp(max=cap)
    c = synth.make_prefill_case(variant, "bf16", cap, lens.tolist(), q_lens.tolist(), seed=505,
                                device="cuda")
    got = to_f64(hip_prefill(c))
    assert np.isfinite(got).all()
    cu = c.cu_q.tolist()
    for b in (0, 1, 97, 128, 200, 254, 255):
        T = cu[b + 1] - cu[b]
        if T == 0:
            continue
        # the oracle on this sequence alone (its rows, its cache slice)
        sub = synth.PrefillCase(c.variant, c.dtype, c.q[cu[b]:cu[b + 1]].cpu(),
                                c.k[b:b + 1].cpu(), c.v[b:b + 1].cpu(),
                                torch.tensor([0, T], dtype=torch.int32),
                                c.seq_lens[b:b + 1].cpu(), None, c.cap, c.window)
        rows = [(n, h) for n in (0, T - 1) for h in (0, 13, 31)]
        ref = oracle_prefill(sub, rows=rows)
        for i, (n, h) in enumerate(rows):
            assert max_err(got[cu[b] + n, h], ref[i]) <= TOL["bf16"], (b, n, h)


def test_prefill_many_items_per_block_all_rows():
    # more work-groups than CUs, so each persistent block of the bf16 sliding
    # kernel takes a list of them: 96 sequences of 0..24 new tokens after pasts
    # of 0..200 positions, a few with chunks longer than the sequence (their
    # rows before position 0 are zero, some whole work-groups of them); every
    # row vs the oracle, for both geometries (the global layer as a control)
    g = torch.Generator().manual_seed(509)
    B, cap = 96, 240
    q_lens = torch.randint(0, 25, (B,), generator=g)
    past = torch.randint(0, 201, (B,), generator=g)
    lens = (past + q_lens).clamp(max=cap)
    for b in (3, 40, 77):  # the chunk reaches before position 0 (b = 40: all of it)
        q_lens[b] = 24
        lens[b] = 0 if b == 40 else 5 + b % 7
    for variant in ("sliding", "global"):
        c = synth.make_prefill_case(variant, "bf16", cap, lens.tolist(), q_lens.tolist(), seed=509)
        got = to_f64(hip_prefill(to_gpu(c)))
        ref = oracle_prefill(c)
        assert max_err(got, ref) <= TOL["bf16"], variant
        cu = c.cu_q.tolist()
        for b in (3, 40, 77):
            before = q_lens[b].item() - lens[b].item()
            assert not got[cu[b]:cu[b] + before].any(), (variant, b)


def test_prefill_chunk_longer_than_sequence():
    # outside the domain: rows before position 0 are zero, the rest as defined
    c = synth.make_prefill_case("sliding", "bf16", 64, [5, 30], [8, 10], seed=506, fill=0.0)
    got = to_f64(hip_prefill(to_gpu(c)))
    ref = oracle_prefill(c)
    assert not got[:3].any()           # tokens 0..2 of sequence 0 sit before position 0
    assert max_err(got, ref) <= TOL["bf16"]


# Runtime windows of the sliding geometry (the Retrofit page's per-layer
# windows): chunks after pasts around the window edge, a single token, a fresh
# prompt and an empty chunk.
@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("window", [1, 17, 2048, 8192])
def test_prefill_window_parity(window, dtype, paged):
    cap = max(window + 64, 608)
    lens = [cap - 3, min(cap, window + 20), min(cap, window), 40, 7]
    q_lens = [60, 25, 1, 40, 0]
    c = synth.make_prefill_case("sliding", dtype, cap, lens, q_lens, paged=paged, seed=510 + window,
                                window=window, extra_pages=3)
    d = to_gpu(c)
    got = to_f64(gqa.gqa_prefill_sliding_window(d.q, d.k, d.v, d.cu_q, d.seq_lens, window,
                                                block_table=d.block_table))
    assert np.isfinite(got).all()  # NaN outside every attended range is never read
    err = max_err(got, oracle_prefill(c))
    assert err <= TOL[dtype], (window, dtype, paged, err)


def test_prefill_window_1024_matches_the_default_entry_point():
    c = to_gpu(synth.make_prefill_case("sliding", "bf16", 2112, [1300, 40, 2100], [77, 40, 300],
                                       seed=511))
    a = hip_prefill(c)
    b = gqa.gqa_prefill_sliding_window(c.q, c.k, c.v, c.cu_q, c.seq_lens, 1024)
    assert torch.equal(a, b)


def test_prefill_window_8192_sampled():
    # 2 x 1024 new tokens after 8192 cached positions, window 8192: sampled rows
    W = 8192
    c = synth.make_prefill_case("sliding", "bf16", 9232, [9216, 9000], [1024, 1024], seed=512,
                                window=W, device="cuda", fill=0.0)
    got = to_f64(gqa.gqa_prefill_sliding_window(c.q, c.k, c.v, c.cu_q, c.seq_lens, W))
    assert np.isfinite(got).all()
    rows = [(n, h) for n in (0, 511, 1023, 1024, 2047) for h in (0, 17, 31)]
    ref = oracle_prefill(to_cpu(c), rows=rows)
    for i, (n, h) in enumerate(rows):
        assert max_err(got[n, h], ref[i]) <= TOL["bf16"], (n, h)
