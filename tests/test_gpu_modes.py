"""The two split launch modes forced on both geometries, vs the fp64 oracle,
through the C ABI, on an MI355X: stream (the tile partition over waves) and
group (the same partition over work-groups, each merging its four waves in
LDS), both finished by the combine kernel.  The planner takes stream mode on
the sliding geometry and group mode on the global one; the other parity tests
run those, and this module runs each geometry in the other mode as well.

Every call here runs with the mode forced (gqa_decode_force_mode), on the
shapes the other parity tests run in unit or split mode: ragged lengths
across tiles, pages and window edges, empty sequences, both cache forms, f32
and bf16, the runtime window, the ring, the values-only calls, the online-
softmax stress inputs and the longest single sequence, each into a NaN-filled
output.  Bars: 1e-4 (f32), 2e-2 (bf16) max-abs; one-hot selections bit for
bit.
"""
import numpy as np
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import oracle
import oracle_pins
import synth
from gpu_cases import (TOL, hip_run, hip_run_k_eq_v, max_err, oracle_run, oracle_run_k_eq_v,
                       to_f64, to_gpu)
from stress_cases import stress_decode_case

pytestmark = pytest.mark.gpu
HEADS = 32


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


@pytest.fixture(params=["group", "stream"], autouse=True)
def mode(request):
    gqa.force_mode(request.param)
    yield request.param
    gqa.force_mode(None)


def _nan_out(c):
    return torch.full_like(c.q, float("nan"))


SMALL = {
    "sliding": (2096, [1, 15, 16, 17, 1023, 1024, 1025, 1041, 2047, 2096]),
    "global": (1312, [1, 15, 16, 17, 100, 513, 1024, 1299, 1312]),
}


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_mode_parity_small(variant, dtype, paged, mode):
    cap, lens = SMALL[variant]
    assert gqa.gqa_decode_plan(variant, len(lens), cap)["mode"] == mode
    c = synth.make_case(variant, dtype, len(lens), cap, lens, paged=paged, seed=601,
                        extra_pages=5)
    g = to_gpu(c)
    got = to_f64(hip_run(g, o=_nan_out(g)))
    err = max_err(got, oracle_run(c))
    assert err <= TOL[dtype], (variant, dtype, paged, err)


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_mode_batch_shapes(variant):
    # many units, one long unit per kv head, a few ragged ones
    for B, cap, seed in ((64, 1100, 611), (1, 9000, 612), (3, 4096, 613), (256, 200, 614)):
        lens = synth.draw_seq_lens(("uniform", 1, cap), B, seed)
        c = synth.make_case(variant, "bf16", B, cap, lens, seed=seed)
        g = to_gpu(c)
        err = max_err(to_f64(hip_run(g, o=_nan_out(g))), oracle_run(c))
        assert err <= TOL["bf16"], (B, cap, err)


def slice_boundary_positions(variant, dtype, lens, cap, mode):
    """For each sequence, the first position of a tile where two slices meet
    inside kv head 0's unit (the middle if one slice holds it).  Slices: the
    launch's waves (half the plan's for the f32 sliding kernel, only
    max(T, 256) of them for fewer tiles) in stream mode; its work-groups
    (fewer when the tiles give fewer than four per work-group) in group mode."""
    KV = 16 if variant == "sliding" else 4
    plan = gqa.gqa_decode_plan(variant, len(lens), cap)
    waves = plan["waves"]
    if variant == "sliding" and dtype == "f32":
        waves //= 2
    rng = []
    for L in lens:
        L = min(L, cap)
        lo = max(0, L - 1024) if variant == "sliding" else 0
        t0 = lo // 16
        rng.append((lo, L, t0, (L + 15) // 16 - t0))
    T = KV * sum(n for *_, n in rng)
    if mode == "group":
        NS = min(waves // 4, max(1, -(-T // 4)))
    else:
        NS = min(waves, max(256, T))
    out, first = [], 0
    for lo, L, t0, n in rng:
        pos = (lo + L) // 2
        for w in range(NS):
            st = w * T // NS
            if first < st < first + n:
                pos = max(lo, (t0 + st - first) * 16)
                break
        out.append(min(pos, L - 1))
        first += KV * n
    return out


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_mode_one_hot_selects_exactly(variant, dtype, paged, mode):
    # a dominant logit at the window start, the last position, a page's first
    # and last rows, and the first tile of a slice inside a split unit: the
    # merged weights are exactly one-hot, o is that value row
    lens = [1030, 200, 47, 1024, 1296]
    cap = 1296
    for pick in ("lo", "last", "page0", "page15", "slice"):
        if pick == "slice":
            pos = slice_boundary_positions(variant, dtype, lens, cap, mode)
        else:
            pos = []
            for L in lens:
                lo = max(0, L - 1024) if variant == "sliding" else 0
                first = ((lo + 15) // 16) * 16
                p = {"lo": lo, "last": L - 1, "page0": first, "page15": first + 15}[pick]
                pos.append(min(p, L - 1))
        c = oracle_pins.one_hot_case(variant, dtype, len(lens), cap, lens, pos, seed=603,
                                     paged=paged)
        g = to_gpu(c)
        got = hip_run(g, o=_nan_out(g)).cpu()
        G = HEADS // c.KV
        for b in range(len(lens)):
            for h in range(HEADS):
                exp = oracle_pins.value_row(c, b, pos[b], h // G)
                assert torch.equal(got[b, h], exp), (pick, b, h)


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_mode_lengths_and_empty_sequences(variant):
    # seq_len 0 and negative give zero rows (written by the kernel: o starts as
    # NaN), above the capacity clamps; a call with nothing attended at all
    cap = 320
    c = synth.make_case(variant, "bf16", 4, cap, [0, -5, cap, 17], seed=609, fill=0.0)
    g = to_gpu(c)
    got = hip_run(g, o=_nan_out(g)).cpu()
    assert torch.count_nonzero(got[0]) == 0 and torch.count_nonzero(got[1]) == 0
    assert max_err(to_f64(got), oracle_run(c)) <= TOL["bf16"]
    e = synth.make_case(variant, "bf16", 3, cap, [0, 0, -1], seed=610, fill=0.0)
    ge = to_gpu(e)
    got_e = hip_run(ge, o=_nan_out(ge)).cpu()
    assert torch.count_nonzero(got_e) == 0


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_mode_prefix_across_lane_rows(variant):
    # the split kernels scan the sequences' tile counts four to a lane, in
    # 16-lane rows: batches that end one sequence into the second, third and
    # fourth row, with empty sequences among them
    for B, seed in ((65, 615), (129, 616), (193, 617)):
        lens = [int(x) for x in synth.draw_seq_lens(("uniform", 1, 300), B, seed)]
        lens[3::7] = [0] * len(lens[3::7])
        c = synth.make_case(variant, "bf16", B, 300, lens, seed=seed)
        g = to_gpu(c)
        err = max_err(to_f64(hip_run(g, o=_nan_out(g))), oracle_run(c))
        assert err <= TOL["bf16"], (B, err)


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_mode_consecutive_calls_and_side_stream(variant):
    # calls of different shapes one after another on one stream, each into a
    # NaN output, then the same on a side stream
    cap = 4096
    shapes = [([4096, 5, 3000, 1], 620), ([17, 4000, 64, 2222, 4096, 1], 621),
              ([4096], 622), ([4096, 5, 3000, 1], 620)]
    cases = [synth.make_case(variant, "bf16", len(l), cap, l, seed=s) for l, s in shapes]
    refs = [oracle_run(c) for c in cases]
    side = torch.cuda.Stream()
    for stream in (None, side):
        outs = []
        for c, ref in zip(cases, refs):
            g = to_gpu(c)
            o = _nan_out(g)
            if stream is not None:
                stream.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(stream):
                    hip_run(g, o=o, stream=stream)
                stream.synchronize()
            else:
                hip_run(g, o=o)
            outs.append(o)
            err = max_err(to_f64(o), ref)
            assert err <= TOL["bf16"], (stream is not None, err)
        assert torch.equal(outs[0], outs[3])


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mode_runtime_window(dtype, paged):
    window, cap = 4096, 9008
    lens = [9008, 4097, 2500, 6000, 1]
    c = synth.make_case("sliding", dtype, len(lens), cap, lens, paged=paged, seed=630,
                        window=window, extra_pages=3)
    g = to_gpu(c)
    got = to_f64(hip_run(g, o=_nan_out(g), window=window))
    err = max_err(got, oracle_run(c, window=window))
    assert err <= TOL[dtype], (dtype, paged, err)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mode_ring(dtype):
    ring, window = 2048, 1500
    lens = [1499, 1500, 1501, 2047, 2048, 2049, 10007]
    c = synth.make_ring_case(dtype, len(lens), ring, lens, seed=640, window=window)
    got = to_f64(gqa.gqa_decode_sliding_ring(*(x.cuda() for x in (c.q, c.k, c.v, c.seq_lens)),
                                             window=window))
    n = synth.to_numpy
    ref = oracle.gqa_decode_ring(n(c.q), n(c.k), n(c.v), n(c.seq_lens), window=window)
    assert max_err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mode_values_only(dtype, paged):
    lens = [700, 1, 16, 17, 333, 0, 4000]
    c = synth.make_case("global", dtype, len(lens), 4000, lens, paged=paged, seed=650,
                        extra_pages=3)
    g = to_gpu(c)
    got = to_f64(hip_run_k_eq_v(g, o=_nan_out(g)))
    assert np.isfinite(got).all()
    err = max_err(got, oracle_run_k_eq_v(c))
    assert err <= TOL[dtype], (dtype, paged, err)


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pattern", ["ramp", "large"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_mode_softmax_stress(variant, pattern, dtype, paged):
    # rising logits (repeated rescales, partials whose maxima differ by
    # hundreds) and large random ones, through the in-kernel merge
    B, cap, lens = (4, 4096, [4096, 1025, 3000, 17]) if variant == "sliding" else \
        (3, 16384, [16384, 9000, 333])
    c = stress_decode_case(pattern, variant, dtype, B, cap, lens, seed=660, paged=paged)
    g = to_gpu(c)
    got = to_f64(hip_run(g, o=_nan_out(g)))
    err = max_err(got, oracle_run(c))
    assert err <= TOL[dtype], (variant, pattern, dtype, paged, err)


@pytest.mark.parametrize("name", ["sliding_bf16_b1_paged_s262144",
                                  "global_bf16_b1_paged_s262144"])
def test_mode_long_single_sequence(name):
    c = synth.make_workload(name, seed=0, device="cuda")
    got = to_f64(hip_run(c, o=_nan_out(c)))
    host = synth.Case(c.variant, c.dtype, c.q.cpu(), c.k.cpu(), c.v.cpu(), c.seq_lens.cpu(),
                      c.block_table.cpu(), c.cap, c.window)
    err = max_err(got, oracle_run(host))
    assert err <= TOL["bf16"], (name, err)


def test_mode_noalloc_matches_workspace_call():
    # the allocation-free entry point in the forced mode: two calls in a row,
    # the second smaller
    for lens, seed in (([16384, 9000, 333, 4096], 670), ([777, 20], 671)):
        c = to_gpu(synth.make_case("global", "bf16", len(lens), 16384, lens, paged=True,
                                   seed=seed))
        want = hip_run(c)
        o = _nan_out(c)
        gqa.gqa_decode_global_paged_noalloc(c.q, c.k, c.v, c.block_table, c.seq_lens, o)
        torch.cuda.synchronize()
        assert torch.equal(o, want)
