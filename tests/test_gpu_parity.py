"""HIP path vs the fp64 oracle, through the C ABI, on an MI355X.

Every case is seeded and synthetic (synth.py).  Tolerances: max-abs error 1e-4
for float32 inputs, 2e-2 for bfloat16 inputs (unit-RMS values).  Invariants
that the method makes exact are checked bit for bit.
"""
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import oracle_pins
import synth
from gpu_cases import SPLIT_MODE, TOL, hip_run, max_err, oracle_run, to_f64, to_gpu

pytestmark = pytest.mark.gpu

HEADS = 32


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


SMALL = {
    # variant: (cap, seq_lens) spanning several tiles, the window edge and ragged tails
    "sliding": (2096, [1, 15, 16, 17, 1023, 1024, 1025, 1041, 2047, 2096]),
    "global": (1312, [1, 15, 16, 17, 100, 513, 1024, 1299, 1312]),
}


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_parity_small(variant, dtype, paged):
    cap, lens = SMALL[variant]
    c = synth.make_case(variant, dtype, len(lens), cap, lens, paged=paged, seed=101,
                        extra_pages=5)
    ref = oracle_run(c)
    got = to_f64(hip_run(to_gpu(c)))
    err = max_err(got, ref)
    assert err <= TOL[dtype], (variant, dtype, paged, err)


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_parity_batch_shapes(variant):
    # many sequences (direct path) and one sequence (split path) of one dtype
    for B, cap, seed in ((64, 1100, 1), (1, 9000, 2), (3, 4096, 3)):
        lens = synth.draw_seq_lens(("uniform", 1, cap), B, seed)
        c = synth.make_case(variant, "bf16", B, cap, lens, seed=seed)
        err = max_err(to_f64(hip_run(to_gpu(c))), oracle_run(c))
        assert err <= TOL["bf16"], (B, cap, err)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_combine_d_parts(variant, dtype):
    # split units (stream mode, group mode on the global geometry) at batch
    # sizes that give the combine 8, 4, 2 and 1 d parts per head
    # (fewer than 256 (sequence, head) rows split each head's D across work-groups)
    # and work-groups of eight and of four waves (above 512 groups); sliding with a
    # 2048 window, whose 129-tile units keep these batches in stream mode
    cap = SMALL[variant][0]
    window = 2048 if variant == "sliding" else None
    for B in ((1, 2, 5, 16, 24, 31, 33) if dtype == "bf16" else (1, 16, 33)):
        assert gqa.gqa_decode_plan(variant, B, cap, window=window)["mode"] == SPLIT_MODE[variant]
        lens = synth.draw_seq_lens(("uniform", 1, cap), B, 200 + B)
        lens[0] = cap
        c = synth.make_case(variant, dtype, B, cap, lens, seed=200 + B, window=window)
        err = max_err(to_f64(hip_run(to_gpu(c), window=window)), oracle_run(c, window=window))
        assert err <= TOL[dtype], (variant, dtype, B, err)


UNIT_MODE = {"sliding": (64, 1104), "global": (256, 512)}  # B, capacity


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_parity_unit_mode(variant, dtype, paged):
    # many short units: one work-group per (sequence, kv head)
    B, cap = UNIT_MODE[variant]
    assert gqa.gqa_decode_plan(variant, B, cap)["mode"] == "unit"
    lens = synth.draw_seq_lens(("uniform", 1, cap), B, 7)
    lens[0], lens[1], lens[2] = 1, cap, 0
    c = synth.make_case(variant, dtype, B, cap, lens, paged=paged, seed=113)
    err = max_err(to_f64(hip_run(to_gpu(c))), oracle_run(c))
    assert err <= TOL[dtype], (variant, dtype, paged, err)


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_single_position_is_exact(variant, dtype, paged):
    c = synth.make_case(variant, dtype, 3, 64, [1, 1, 1], paged=paged, seed=102)
    got = hip_run(to_gpu(c)).cpu()
    G = HEADS // c.KV
    for b in range(3):
        for h in range(HEADS):
            exp = oracle_pins.value_row(c, b, 0, h // G)
            assert torch.equal(got[b, h], exp), (b, h)


def stream_waves(variant, dtype, plan_waves, T):
    """Waves sharing T tiles in stream mode: the launch (half the plan's waves
    for the f32 sliding kernel, which fits one wave per SIMD), only
    max(T, 256) of them when T is smaller."""
    W = plan_waves // 2 if (variant == "sliding" and dtype == "f32") else plan_waves
    return min(W, max(256, T))


def slice_boundary_positions(variant, lens, cap, dtype="bf16"):
    """For each sequence, the first position of a tile that starts a new slice
    inside kv head 0's unit (where two wave slices of the stream partition, or
    two work-group slices of the group partition, meet), or the unit's middle
    if one slice holds it."""
    KV = 16 if variant == "sliding" else 4
    plan = gqa.gqa_decode_plan(variant, len(lens), cap)
    rng = []
    for L in lens:
        L = min(L, cap)
        lo = max(0, L - 1024) if variant == "sliding" else 0
        t0 = lo // 16
        rng.append((lo, L, t0, (L + 15) // 16 - t0))
    T = KV * sum(n for *_, n in rng)
    if plan["mode"] == "stream":
        W = stream_waves(variant, dtype, plan["waves"], T)
    elif plan["mode"] == "group":
        # work-groups: the launch's, or one per 4 tiles when that is fewer
        groups = plan["waves"] // 4
        W = min(groups, max(1, -(-T // 4)))
    else:
        W = 1
    out, first = [], 0
    for lo, L, t0, n in rng:
        s0 = first                       # flattened first tile of unit (b, g=0)
        pos = (lo + L) // 2
        for w in range(W):
            st = w * T // W
            if s0 < st < s0 + n:
                pos = max(lo, (t0 + st - s0) * 16)
                break
        out.append(min(pos, L - 1))
        first += KV * n
    return out


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_one_hot_dominant_logit_selects_exactly(variant, dtype, paged):
    lens = [1030, 200, 47, 1024, 1296]
    cap = 1296
    for pick in ("lo", "last", "page0", "page15", "slice"):
        if pick == "slice":
            pos = slice_boundary_positions(variant, lens, cap, dtype)
        else:
            pos = []
            for L in lens:
                lo = max(0, L - 1024) if variant == "sliding" else 0
                first = ((lo + 15) // 16) * 16
                p = {"lo": lo, "last": L - 1, "page0": first, "page15": first + 15}[pick]
                pos.append(min(p, L - 1))
        c = oracle_pins.one_hot_case(variant, dtype, len(lens), cap, lens, pos, seed=103,
                                     paged=paged)
        got = hip_run(to_gpu(c)).cpu()
        G = HEADS // c.KV
        for b in range(len(lens)):
            for h in range(HEADS):
                exp = oracle_pins.value_row(c, b, pos[b], h // G)
                assert torch.equal(got[b, h], exp), (pick, b, h)


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_poison_outside_the_range_is_never_read(variant, paged):
    lens = [1300, 20, 1025, 16, 2000]
    kw = dict(paged=paged, seed=104, extra_pages=6)
    a = synth.make_case(variant, "bf16", 5, 2000, lens, fill=float("nan"), **kw)
    z = synth.make_case(variant, "bf16", 5, 2000, lens, fill=0.0, **kw)
    ga = hip_run(to_gpu(a)).cpu()
    gz = hip_run(to_gpu(z)).cpu()
    assert torch.isfinite(ga.float()).all()
    assert torch.equal(ga, gz)


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_paged_equals_contiguous_bitwise(variant):
    lens = [1, 95, 1040, 700]
    c = synth.make_case(variant, "bf16", 4, 1040, lens, seed=105)
    p = oracle_pins._contig_to_paged(c, seed=106)
    a = hip_run(to_gpu(c)).cpu()
    b = hip_run(to_gpu(p)).cpu()
    assert torch.equal(a, b)


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_gqa_group_sharing_bitwise(variant):
    c = synth.make_case(variant, "bf16", 2, 700, [700, 333], seed=107)
    G = HEADS // c.KV
    for h in range(HEADS):
        c.q[:, h] = c.q[:, (h // G) * G]
    got = hip_run(to_gpu(c)).cpu()
    for h in range(HEADS):
        assert torch.equal(got[:, h], got[:, (h // G) * G])


def test_sliding_equals_full_below_the_window():
    c = synth.make_case("sliding", "f32", 4, 1024, [1, 513, 1000, 1024], seed=108)
    got = to_f64(hip_run(to_gpu(c)))
    full = oracle_run(c, window=0)
    assert max_err(got, full) <= TOL["f32"]


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_length_edge_cases(variant):
    # seq_len 0 and negative give zero rows; above the capacity clamps to it
    cap = 320
    c = synth.make_case(variant, "bf16", 4, cap, [0, -5, cap, 17], seed=109, fill=0.0)
    got = hip_run(to_gpu(c)).cpu()
    assert torch.count_nonzero(got[0]) == 0 and torch.count_nonzero(got[1]) == 0
    c2 = synth.Case(c.variant, c.dtype, c.q, c.k, c.v,
                    torch.tensor([0, -5, cap + 1000, 17], dtype=torch.int32), None, cap, c.window)
    got2 = hip_run(to_gpu(c2)).cpu()
    assert torch.equal(got, got2)
    ref = oracle_run(c)
    assert max_err(to_f64(got), ref) <= TOL["bf16"]


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_deterministic_and_workspace_reuse(variant):
    cap = 4096
    lens_a = [4096, 5, 3000, 1]
    lens_b = [17, 4000, 64, 2222]
    a = to_gpu(synth.make_case(variant, "bf16", 4, cap, lens_a, seed=110))
    b = to_gpu(synth.make_case(variant, "bf16", 4, cap, lens_b, seed=111))
    need = gqa.gqa_decode_workspace_bytes(variant, 4, cap)
    ws = torch.full((max(need, 16),), 255, dtype=torch.uint8, device="cuda")  # NaN-patterned
    s = torch.cuda.Stream()
    # the inputs and the NaN fill were queued on the current stream
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o1 = hip_run(a, workspace=ws, stream=s)
        ob = hip_run(b, workspace=ws, stream=s)
        o2 = hip_run(a, workspace=ws, stream=s)
    s.synchronize()
    assert torch.equal(o1, o2)
    assert max_err(to_f64(ob), oracle_run(b)) <= TOL["bf16"]


@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_side_stream_without_entering_it(variant):
    # stream= names a side stream while the current stream stays the default
    # one; the binding allocates o and the workspace itself.  Work queued on
    # the default stream right after the call allocates and fills memory of
    # the workspace's size: the binding must keep the blocks it handed to the
    # side stream's kernels from being reused before they complete.
    cap = 4096
    c = to_gpu(synth.make_case(variant, "bf16", 4, cap, [4096, 5, 3000, 1], seed=115))
    assert gqa.gqa_decode_plan(variant, 4, cap)["mode"] == SPLIT_MODE[variant]
    need = gqa.gqa_decode_workspace_bytes(variant, 4, cap)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        o = hip_run(c, stream=s)
        junk = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
        junk2 = torch.full_like(o, float("nan"))
        outs.append(o)
        del junk, junk2
    s.synchronize()
    torch.cuda.synchronize()
    ref = oracle_run(c)
    for o in outs:
        assert max_err(to_f64(o), ref) <= TOL["bf16"]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_profile_hooks_count_launches():
    c = to_gpu(synth.make_case("global", "bf16", 2, 4096, [4096, 100], seed=112))
    gqa.profile_begin(16)
    for _ in range(3):
        hip_run(c)
    res = gqa.profile_read()
    assert res[("global", "main")][0] == 3 and res[("global", "main")][1] > 0
    assert res[("global", "combine")][0] == 3
    assert res[("sliding", "main")][0] == 0


def test_measurement_probes():
    src = torch.rand(1 << 20, device="cuda")
    dst = torch.zeros_like(src)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    gqa.hbm_read_probe(src, sink)
    gqa.hbm_copy_probe(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    # a size that is not a multiple of the wave stride
    s2 = torch.rand(1000 * 4 + 4, device="cuda")
    d2 = torch.zeros_like(s2)
    gqa.hbm_copy_probe(s2, d2)
    torch.cuda.synchronize()
    assert torch.equal(s2, d2)


# --------------------------------------------------------------- runtime window

@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("window", [1, 17, 512, 2048, 4096, 8192])
def test_window_parity(window, paged):
    cap = 9008
    lens = [1, window, window + 1, 4000, 9008, 8191]
    c = synth.make_case("sliding", "bf16", len(lens), cap, lens, paged=paged, seed=120,
                        window=window, extra_pages=3)
    got = to_f64(hip_run(to_gpu(c), window=window))
    err = max_err(got, oracle_run(c, window=window))
    assert err <= TOL["bf16"], (window, paged, err)


@pytest.mark.parametrize("window,B,expect", [(512, 64, "unit"), (2048, 64, "unit"),
                                             (2048, 32, "stream")])
def test_window_parity_unit_mode_and_f32(window, B, expect):
    cap = 4096
    mode = gqa.gqa_decode_plan("sliding", B, cap, window=window)["mode"]
    assert mode == expect
    lens = synth.draw_seq_lens(("uniform", 1, cap), B, 9)
    c = synth.make_case("sliding", "f32", B, cap, lens, seed=121, window=window)
    err = max_err(to_f64(hip_run(to_gpu(c), window=window)), oracle_run(c, window=window))
    assert err <= TOL["f32"], (window, err)


def test_window_1024_matches_the_default_entry_point():
    c = to_gpu(synth.make_case("sliding", "bf16", 5, 3000, [3000, 1025, 1024, 5, 2500], seed=122))
    assert torch.equal(hip_run(c), hip_run(c, window=1024))


@pytest.mark.parametrize("window", [2048, 8192])
def test_window_one_hot_edges_exact(window):
    lens = [window + 37, window, 9000]
    cap = 9008
    for pick in ("lo", "last"):
        pos = [max(0, L - window) if pick == "lo" else L - 1 for L in lens]
        c = synth.make_case("sliding", "f32", 3, cap, lens, seed=123, window=window)
        G = 2
        js = [(h * 37 + 5) % 256 for h in range(HEADS)]
        q = torch.zeros(3, HEADS, 256)
        for h in range(HEADS):
            q[:, h, js[h]] = 1.0
        c.q = q
        for b in range(3):
            lo, L = c.attended(b)
            for h in range(HEADS):
                c.k[b, lo:L, h // G, js[h]] = torch.linspace(-4, 4, L - lo)
                c.k[b, pos[b], h // G, js[h]] = 160.0
        got = hip_run(to_gpu(c), window=window).cpu()
        for b in range(3):
            for h in range(HEADS):
                assert torch.equal(got[b, h], c.v[b, pos[b], h // G]), (pick, b, h)


def test_window_poison_never_read():
    lens = [5000, 20, 9000]
    kw = dict(paged=True, seed=124, window=4096, extra_pages=4)
    a = synth.make_case("sliding", "bf16", 3, 9008, lens, fill=float("nan"), **kw)
    z = synth.make_case("sliding", "bf16", 3, 9008, lens, fill=0.0, **kw)
    ga, gz = hip_run(to_gpu(a), window=4096).cpu(), hip_run(to_gpu(z), window=4096).cpu()
    assert torch.isfinite(ga.float()).all() and torch.equal(ga, gz)


# --------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", ["sliding_f32_b4_s2048", "global_bf16_b4_s4096"])
def test_workload_small_full_parity(name):
    c = synth.make_workload(name, seed=0)
    got = to_f64(hip_run(to_gpu(c)))
    err = max_err(got, oracle_run(c))
    assert err <= TOL[c.dtype], (name, err)
