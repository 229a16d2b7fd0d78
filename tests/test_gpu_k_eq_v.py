"""decodeGQA over a values-only cache (keys rebuilt in the kernel as
rope(w_k * v_s, s): values = keys on the global layers) vs the fp64 oracle,
through the C ABI, on an MI355X."""
import numpy as np
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import oracle
import synth
from gpu_cases import TOL, hip_run_k_eq_v, max_err, oracle_run_k_eq_v, to_f64, to_gpu

pytestmark = pytest.mark.gpu
HEADS = 32


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


def _host(c):
    return synth.Case(c.variant, c.dtype, c.q.cpu(), c.k.cpu(), c.v.cpu(), c.seq_lens.cpu(),
                      None if c.block_table is None else c.block_table.cpu(), c.cap, c.window,
                      c.w_k.cpu())


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_k_eq_v_parity(dtype, paged):
    # ragged lengths: one position, one tile, a tile plus one, several tiles with
    # a ragged tail, nothing attended; NaN everywhere outside the attended rows
    lens = [700, 1, 16, 17, 333, 0]
    c = synth.make_case("global", dtype, len(lens), 704, lens, paged=paged, seed=410,
                        extra_pages=3)
    got = hip_run_k_eq_v(to_gpu(c))
    torch.cuda.synchronize()
    g = to_f64(got)
    assert np.isfinite(g).all()
    err = max_err(g, oracle_run_k_eq_v(c))
    assert err <= TOL[dtype], err
    assert not g[5].any()  # seq_len 0: zero rows


def test_k_eq_v_single_position_is_the_value_row():
    # softmax over one position is exactly 1: o = v_0 bit for bit, whatever the key
    c = synth.make_case("global", "bf16", 3, 64, [1, 1, 1], seed=411)
    got = hip_run_k_eq_v(to_gpu(c)).cpu()
    for h in range(HEADS):
        assert torch.equal(got[:, h], c.v[:, 0, h // 8])


def test_k_eq_v_paged_equals_contiguous():
    lens = [300, 47, 1]
    kw = dict(seed=412, fill=0.0)
    a = synth.make_case("global", "bf16", 3, 304, lens, **kw)
    b = synth.make_case("global", "bf16", 3, 304, lens, paged=True, **kw)
    assert torch.equal(a.v[0, :300], b.v[b.block_table[0, :19].long()].reshape(-1, 4, 512)[:300])
    ga, gb = hip_run_k_eq_v(to_gpu(a)).cpu(), hip_run_k_eq_v(to_gpu(b)).cpu()
    assert torch.equal(ga, gb)


def test_k_eq_v_deterministic_and_workspace_reuse():
    c = to_gpu(synth.make_case("global", "bf16", 4, 4096, [4096, 2500, 17, 999], seed=413))
    ws = torch.empty(gqa.gqa_decode_workspace_bytes("global", 4, 4096), dtype=torch.uint8,
                     device="cuda")
    ws.fill_(0xFF)
    a = hip_run_k_eq_v(c, workspace=ws).clone()
    b = hip_run_k_eq_v(c, workspace=ws)
    assert torch.equal(a, b)


def test_k_eq_v_unit_mode():
    # 256 sequences x 4 kv heads = 1024 units of <= 128 tiles: one work-group per unit
    B, cap = 256, 2048
    assert gqa.gqa_decode_plan("global", B, cap)["mode"] == "unit"
    lens = synth.draw_seq_lens(("uniform", 1, cap), B, seed=414)
    lens[0], lens[1] = 1, cap
    c = synth.make_case("global", "bf16", B, cap, lens, seed=414, device="cuda")
    got = to_f64(hip_run_k_eq_v(c))
    assert np.isfinite(got).all()
    rows = [(b, h) for b in (0, 1, 77, 200, 255) for h in (0, 7, 8, 31)]
    ref = oracle_run_k_eq_v(_host(c), rows=rows)
    for i, (b, h) in enumerate(rows):
        assert max_err(got[b, h], ref[i]) <= TOL["bf16"], (b, h, int(lens[b]))


def test_k_eq_v_unit_mode_f32_paged():
    B, cap = 256, 320
    lens = synth.draw_seq_lens(("uniform", 1, cap), B, seed=415)
    c = synth.make_case("global", "f32", B, cap, lens, paged=True, seed=415, device="cuda")
    assert gqa.gqa_decode_plan("global", B, cap)["mode"] == "unit"
    got = to_f64(hip_run_k_eq_v(c))
    rows = [(b, h) for b in (3, 100, 254) for h in range(0, HEADS, 5)]
    ref = oracle_run_k_eq_v(_host(c), rows=rows)
    for i, (b, h) in enumerate(rows):
        assert max_err(got[b, h], ref[i]) <= TOL["f32"], (b, h)


def test_k_eq_v_workload_b32_paged_sampled():
    c = synth.make_workload("global_bf16_b32_paged_s16k_128k", seed=0, device="cuda")
    got = hip_run_k_eq_v(c)
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all()
    host = _host(c)
    order = torch.argsort(host.seq_lens)
    bs = [int(order[0]), int(order[-1]), int(order[len(order) // 2])]
    rows = [(b, h) for b in bs for h in (0, 7, 8, 31)]
    ref = oracle_run_k_eq_v(host, rows=rows)
    gh = to_f64(got)
    for i, (b, h) in enumerate(rows):
        assert max_err(gh[b, h], ref[i]) <= TOL["bf16"], (b, h, int(host.seq_lens[b]))


def test_k_eq_v_longest_sequence():
    # positions up to 262143: the largest RoPE angles of the shape domain
    c = synth.make_workload("global_bf16_b1_paged_s262144", seed=0, device="cuda")
    got = to_f64(hip_run_k_eq_v(c))
    rows = [(0, h) for h in (0, 9, 22, 31)]
    ref = oracle_run_k_eq_v(_host(c), rows=rows)
    for i, (b, h) in enumerate(rows):
        assert max_err(got[b, h], ref[i]) <= TOL["bf16"], h


def test_k_eq_v_append_then_attend():
    """Append the new token to a values-only cache on the GPU, then attend; the
    oracle appends the same token (fp64) into a copy of the cache and attends."""
    lens = [1300, 1, 700, 1025]
    cap = 1312
    for paged in (False, True):
        c = synth.make_case("global", "bf16", 4, cap, lens, paged=paged, seed=416, fill=0.0,
                            alloc_all_pages=True)
        g = torch.Generator().manual_seed(417)
        q_raw = (torch.randn(4, HEADS, 512, generator=g) * 2).to(torch.bfloat16)
        k_raw = (torch.randn(4, 4, 512, generator=g) * 3).to(torch.bfloat16)
        w_q = torch.empty(512).uniform_(0.2, 0.4, generator=g).to(torch.bfloat16)
        w_k = c.w_k
        d = to_gpu(c)
        v_before = d.v.clone()
        q_out = gqa.gqa_append_global_k_eq_v(q_raw.cuda(), k_raw.cuda(), w_q.cuda(), w_k.cuda(),
                                             d.seq_lens, d.v, block_table=d.block_table)
        o = gqa.gqa_decode_global_k_eq_v_paged(q_out, d.v, w_k.cuda(), d.block_table,
                                               d.seq_lens) if paged else \
            gqa.gqa_decode_global_k_eq_v(q_out, d.v, w_k.cuda(), d.seq_lens)
        n = synth.to_numpy
        eq, ek, ev, pos = oracle.gqa_append_rows("global", n(q_raw), n(k_raw), None, n(w_q),
                                                 n(w_k), np.asarray(lens, dtype=np.int32))
        host = _host(c)
        host.q = torch.from_numpy(eq).to(torch.bfloat16)
        v_after = d.v.cpu()
        for b in range(4):
            p = int(pos[b])
            row = host.v[b, p] if not paged else \
                host.v[int(host.block_table[b, p // 16]), p % 16]
            row.copy_(torch.from_numpy(ev[b]).to(torch.bfloat16))
            got_row = v_after[b, p] if not paged else \
                v_after[int(host.block_table[b, p // 16]), p % 16]
            assert max_err(got_row.double().numpy(), ev[b]) <= TOL["bf16"], (paged, b)
            # the written row aside, the cache is untouched
            got_row.copy_(v_before.cpu()[b, p] if not paged else
                          v_before.cpu()[int(host.block_table[b, p // 16]), p % 16])
        assert torch.equal(v_after.view(torch.int16), v_before.cpu().view(torch.int16))
        assert max_err(to_f64(q_out), eq) <= TOL["bf16"]
        err = max_err(to_f64(o), oracle_run_k_eq_v(host))
        assert err <= TOL["bf16"], (paged, err)


def test_k_eq_v_profile_kinds():
    c = to_gpu(synth.make_case("global", "bf16", 2, 4096, [4096, 100], seed=418))
    gqa.profile_begin(16)
    for _ in range(2):
        hip_run_k_eq_v(c)
    res = gqa.profile_read()
    assert res[("global_k_eq_v", "main")][0] == 2 and res[("global_k_eq_v", "main")][1] > 0
    assert res[("global_k_eq_v", "combine")][0] == 2
    assert res[("global", "main")][0] == 0
