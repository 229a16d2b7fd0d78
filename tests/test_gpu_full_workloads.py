"""Every output element of the full-size workloads against the fp64 oracle.

The workloads are the shape domain of the gemma-4-31B Model Spec page ("At a
glance" table, Shape domain row: B <= 256, S <= 262144, page 16): the sliding
B=256 contiguous cache (S_max 8192), the global B=32 paged cache (lengths in
[16384, 131072]) and one sequence of 262144 positions in both geometries.
The HIP call runs once on the whole batch, in the launch configuration the
benchmark times, with NaN in every unattended cache slot and unreferenced
page.  The oracle then runs sequence by sequence (or in small batches) on
host copies of the attended rows only, so host memory stays bounded:

  * a contiguous sliding sequence is copied as its attended rows [lo, L),
    re-based to positions [0, n): the oracle then attends to exactly these
    rows in the same order (its window covers all n <= 1024 of them), the
    same sum as on the full layout;
  * a paged sequence is copied as its own pages, in block-table order, with
    an identity block table.

Tolerances: max-abs 2e-2 for bf16 inputs (unit-RMS values).  A CPU test
checks that both host copies give the oracle the same sums as the full
layout, bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_cases import TOL, hip_run, max_err, oracle_run, to_f64

HEADS = 32


@pytest.fixture
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")


def _say(msg):
    print(f"[full] {msg}", flush=True)


def _window_batch(c, bs):
    """Host case holding the attended rows of contiguous sequences bs, re-based
    to position 0 (sequence i holds n_i = L_i - lo_i rows)."""
    spans = [c.attended(b) for b in bs]
    n_max = max(1, max(L - lo for lo, L in spans))
    KV, D = c.KV, c.D
    k = torch.full((len(bs), n_max, KV, D), float("nan"), dtype=c.k.dtype)
    v = torch.full_like(k, float("nan"))
    for i, (b, (lo, L)) in enumerate(zip(bs, spans)):
        if L > lo:
            k[i, :L - lo] = c.k[b, lo:L].cpu()
            v[i, :L - lo] = c.v[b, lo:L].cpu()
    lens = torch.tensor([L - lo for lo, L in spans], dtype=torch.int32)
    q = c.q[list(bs)].cpu()
    return synth.Case(c.variant, c.dtype, q, k, v, lens, None, n_max, c.window)


def _paged_sequence(c, b):
    """Host case holding sequence b of a paged case: its pages in block-table
    order, an identity block table."""
    L = int(c.seq_lens[b])
    lo, _ = c.attended(b)
    p0, p1 = lo // 16, (L + 15) // 16
    bt_row = c.block_table[b].cpu()
    phys = bt_row[p0:p1].to(torch.int64).to(c.k.device)
    k = c.k[phys].cpu()
    v = c.v[phys].cpu()
    bt = torch.full((1, c.block_table.shape[1]), -1, dtype=torch.int32)
    bt[0, p0:p1] = torch.arange(p1 - p0, dtype=torch.int32)
    return synth.Case(c.variant, c.dtype, c.q[b:b + 1].cpu(), k, v, c.seq_lens[b:b + 1].cpu(),
                      bt, c.cap, c.window)


@pytest.mark.gpu
def test_sliding_b256_every_sequence(need_gpu):
    c = synth.make_workload("sliding_bf16_b256_s8192", seed=0, device="cuda")
    got = hip_run(c)
    torch.cuda.synchronize()
    gh = to_f64(got)
    del got
    worst = 0.0
    for b0 in range(0, c.B, 32):
        bs = list(range(b0, min(c.B, b0 + 32)))
        host = _window_batch(c, bs)
        ref = oracle_run(host)
        err = max_err(gh[b0:b0 + len(bs)], ref)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (bs[0], bs[-1], err)
    _say(f"sliding B=256: {c.B * HEADS} rows, max abs err {worst:.3e}")


@pytest.mark.gpu
def test_global_b32_paged_every_row(need_gpu):
    c = synth.make_workload("global_bf16_b32_paged_s16k_128k", seed=0, device="cuda")
    got = hip_run(c)
    torch.cuda.synchronize()
    gh = to_f64(got)
    del got
    worst = 0.0
    for b in range(c.B):
        host = _paged_sequence(c, b)
        ref = oracle_run(host)
        err = max_err(gh[b:b + 1], ref)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (b, int(c.seq_lens[b]), err)
    _say(f"global B=32 paged: {c.B * HEADS} rows, max abs err {worst:.3e}")


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["sliding_bf16_b1_paged_s262144",
                                  "global_bf16_b1_paged_s262144"])
def test_long_single_sequence_every_head(need_gpu, name):
    c = synth.make_workload(name, seed=0, device="cuda")
    got = hip_run(c)
    torch.cuda.synchronize()
    host = _paged_sequence(c, 0)
    ref = oracle_run(host)
    err = max_err(to_f64(got), ref)
    _say(f"{name}: all {HEADS} heads, max abs err {err:.3e}")
    assert err <= TOL["bf16"], err


def test_host_copies_give_the_oracle_the_same_sums():
    # (CPU) the re-based window copy and the per-sequence page copy used above
    # give the oracle the same rows in the same order: on small cases they
    # reproduce the oracle on the full layout bit for bit
    c = synth.make_case("sliding", "bf16", 6, 2112, [1, 700, 1024, 1025, 2000, 2112], seed=31)
    full = oracle_run(c)
    rebased = oracle_run(_window_batch(c, list(range(6))))
    assert np.array_equal(full, rebased)
    p = synth.make_case("global", "bf16", 3, 640, [640, 17, 300], paged=True, seed=32,
                        extra_pages=4)
    full = oracle_run(p)
    for b in range(3):
        assert np.array_equal(full[b:b + 1], oracle_run(_paged_sequence(p, b)))
    ps = synth.make_case("sliding", "bf16", 2, 2112, [2112, 1500], paged=True, seed=33)
    full = oracle_run(ps)
    for b in range(2):
        assert np.array_equal(full[b:b + 1], oracle_run(_paged_sequence(ps, b)))
