"""Host-side checks of the C ABI: the library loads, exports what the header
declares, plans sensibly and rejects bad arguments before launching anything.
No call here reaches the GPU: every entry-point call below fails validation."""
import ctypes
import os
import re

import pytest

import decode_attention_slidingdecodegqa_amd as gqa
from decode_attention_slidingdecodegqa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_decode.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIBRARY_PATH):
        from decode_attention_slidingdecodegqa_amd import build
        build.build()
    return gqa.library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_\w+)\s*\(", src)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(gqa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_constants_match_pages(lib):
    gold = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "model_constants.txt")):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = (x.strip() for x in line.split("="))
            gold[k] = int(v)
    s = gqa.constants("sliding")
    gl = gqa.constants("global")
    assert s == dict(heads=gold["heads"], kv_heads=gold["sliding.kv_heads"],
                     head_dim=gold["sliding.head_dim"], window=gold["sliding.window"],
                     page=gold["page_size"])
    assert gl == dict(heads=gold["heads"], kv_heads=gold["global.kv_heads"],
                      head_dim=gold["global.head_dim"], window=0, page=gold["page_size"])


@pytest.mark.parametrize("variant", ["sliding", "global"])
@pytest.mark.parametrize("B,cap", [(1, 1), (1, 262144), (4, 2048), (4, 4096), (32, 131072),
                                   (256, 8192), (256, 262144), (7, 33), (8, 8192), (32, 1024),
                                   (64, 2048), (128, 4096), (256, 4096)])
def test_plan_and_workspace(lib, variant, B, cap):
    plan = gqa.gqa_decode_plan(variant, B, cap)
    KV = 16 if variant == "sliding" else 4
    G, D = 32 // KV, (256 if variant == "sliding" else 512)
    tiles = (cap + 15) // 16
    if variant == "sliding":
        tiles = min(tiles, 1024 // 16 + 1)
    ws = gqa.gqa_decode_workspace_bytes(variant, B, cap)
    units = B * KV
    if (units >= 1024 and tiles <= 320) or (units >= 256 and tiles <= 128) or \
            (D == 256 and units >= 128 and tiles <= 65):
        # many short units: one work-group of four waves per unit, no workspace
        assert plan == {"mode": "unit", "waves": 4 * B * KV, "slots": 0}
        assert ws == 0
    else:
        # split units: wave slices (stream mode) on the sliding geometry, work-group
        # slices (group mode) on the global one and on tiny sliding calls (at most
        # 2048 tiles in all); slot u + w for every (unit, slice), and in group mode
        # over at least 2^19 tiles the dynamic tail's chunks (up to 768 more
        # slices) and its counter
        group = variant == "global" or units * tiles <= 2048
        assert plan["mode"] == ("group" if group else "stream")
        assert plan["waves"] == (2048 if variant == "sliding" else 1024)
        slices = plan["waves"] // 4 if group else plan["waves"]
        dyn = variant == "global" and units * tiles >= 1 << 19
        assert plan["slots"] == B * KV + slices + (768 if dyn else 0)
        assert ws >= (B + 1) * 4 + (4 if dyn else 0) + plan["slots"] * G * (D + 2) * 4


def test_plan_modes_of_the_workloads(lib):
    assert gqa.gqa_decode_plan("sliding", 256, 8192)["mode"] == "unit"
    assert gqa.gqa_decode_plan("global", 32, 131072)["mode"] == "group"
    assert gqa.gqa_decode_plan("global", 1, 262144)["mode"] == "group"
    assert gqa.gqa_decode_plan("sliding", 4, 2048)["mode"] == "stream"
    assert gqa.gqa_decode_plan("sliding", 1, 262144)["mode"] == "group"


def tail_plan(T, dyn):
    """The group partition's dynamic tail, as the kernels compute it: static
    slices over [0, S), then nch chunks of C tiles."""
    if not dyn or T < 1 << 19:
        return T, 1, 0
    Td = T // 12
    C = max(128, -(-Td // 768))
    nch = Td // C
    return T - nch * C, C, nch


def test_dynamic_tail_partitions_exactly():
    # static slices [w*S//W, (w+1)*S//W) and chunks [S + c*C, S + (c+1)*C) cover
    # [0, T) once; slice_of(t) names the slice or chunk holding t; at most 768
    # chunks (the slots the plan adds) of at least 128 tiles
    import random
    rnd = random.Random(7)
    for _ in range(300):
        T = rnd.choice([(1 << 19) - 1, 1 << 19, 600_000, 1_221_000, 16_777_216, rnd.randint(1, 4_000_000)])
        W = rnd.choice([64, 256])
        S, C, nch = tail_plan(T, True)
        assert S + nch * C == T and nch <= 768
        if T < 1 << 19:
            assert (S, nch) == (T, 0)
            continue
        assert C >= 128 and nch >= 1 and S >= W
        for t in sorted({0, S - 1, S, T - 1} | {rnd.randrange(T) for _ in range(50)}):
            sl = ((t + 1) * W - 1) // S if t < S else W + (t - S) // C
            if sl < W:
                assert sl * S // W <= t < (sl + 1) * S // W
            else:
                c = sl - W
                assert 0 <= c < nch and S + c * C <= t < S + (c + 1) * C


def test_slice_arithmetic_partitions_exactly():
    # the stream partition: slice w = [w*T//W, (w+1)*T//W); the wave holding
    # tile t is ((t+1)*W - 1)//T (the same integer formula runs on the device)
    import random
    rnd = random.Random(5)
    for _ in range(2000):
        T = rnd.randint(1, 10**7)
        W = rnd.choice([1024, 2048, 7])
        t = rnd.randrange(T)
        w = ((t + 1) * W - 1) // T
        assert w * T // W <= t < (w + 1) * T // W


def test_bad_arguments_fail_before_launch(lib):
    P = ctypes.c_void_p
    ok = P(0x10000)  # aligned non-null stand-ins; never dereferenced: validation fails first
    mis = P(0x10008)
    sl = lib.gqa_decode_sliding
    gl = lib.gqa_decode_global_paged
    E = {"NULL": -1, "SHAPE": -2, "DTYPE": -3, "ALIGN": -4, "WS": -5}
    # null pointers
    assert sl(None, ok, ok, ok, ok, 4, 2048, 1, None, 0, None) == E["NULL"]
    assert sl(ok, ok, ok, None, ok, 4, 2048, 1, None, 0, None) == E["NULL"]
    assert gl(ok, ok, ok, None, 10, ok, ok, 4, 10, 1, None, 0, None) == E["NULL"]
    # batch and capacity ranges
    assert sl(ok, ok, ok, ok, ok, 0, 2048, 1, None, 0, None) == E["SHAPE"]
    assert sl(ok, ok, ok, ok, ok, 257, 2048, 1, None, 0, None) == E["SHAPE"]
    assert sl(ok, ok, ok, ok, ok, 4, 0, 1, None, 0, None) == E["SHAPE"]
    assert sl(ok, ok, ok, ok, ok, 4, 262145, 1, None, 0, None) == E["SHAPE"]
    assert gl(ok, ok, ok, ok, 0, ok, ok, 4, 10, 1, None, 0, None) == E["SHAPE"]
    assert gl(ok, ok, ok, ok, 16385, ok, ok, 4, 10, 1, None, 0, None) == E["SHAPE"]
    assert gl(ok, ok, ok, ok, 10, ok, ok, 4, 0, 1, None, 0, None) == E["SHAPE"]
    # dtype
    assert sl(ok, ok, ok, ok, ok, 4, 2048, 2, None, 0, None) == E["DTYPE"]
    assert sl(ok, ok, ok, ok, ok, 4, 2048, -1, None, 0, None) == E["DTYPE"]
    # alignment
    assert sl(mis, ok, ok, ok, ok, 256, 8192, 1, None, 0, None) == E["ALIGN"]
    assert sl(ok, ok, mis, ok, ok, 256, 8192, 1, None, 0, None) == E["ALIGN"]
    assert sl(ok, ok, ok, ok, mis, 256, 8192, 1, None, 0, None) == E["ALIGN"]
    # workspace: B=32 global paged over 131072 positions needs one
    need = lib.gqa_decode_workspace_bytes(1, 32, 131072)
    assert need > 0
    assert gl(ok, ok, ok, ok, 8192, ok, ok, 32, 9000, 1, None, 0, None) == E["WS"]
    assert gl(ok, ok, ok, ok, 8192, ok, ok, 32, 9000, 1, ok, need - 1, None) == E["WS"]
    assert gl(ok, ok, ok, ok, 8192, ok, ok, 32, 9000, 1, mis, need, None) == E["ALIGN"]
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert gqa.gqa_status_str(code)
    assert gqa.gqa_status_str(-99) == "unknown status"


def test_window_arguments(lib):
    P = ctypes.c_void_p
    ok = P(0x10000)
    f = lib.gqa_decode_sliding_window
    fp = lib.gqa_decode_sliding_window_paged
    for w in (0, -1, 262145):
        assert f(ok, ok, ok, ok, ok, 4, 2048, w, 1, None, 0, None) == -2
        assert fp(ok, ok, ok, ok, 16, ok, ok, 4, 16, w, 1, None, 0, None) == -2
        assert lib.gqa_decode_sliding_window_workspace_bytes(4, 2048, w) == 0
    # the default window reproduces the sliding plan; larger windows leave unit mode
    assert gqa.gqa_decode_plan("sliding", 256, 8192, window=1024) == \
        gqa.gqa_decode_plan("sliding", 256, 8192)
    assert gqa.gqa_decode_plan("sliding", 256, 8192, window=8192)["mode"] == "stream"
    assert gqa.gqa_decode_plan("sliding", 256, 8192, window=2032)["mode"] == "unit"
    assert gqa.gqa_decode_workspace_bytes("sliding", 256, 8192, window=8192) > 0
    with pytest.raises(ValueError):
        gqa.gqa_decode_plan("global", 4, 4096, window=1024)


def test_ring_arguments_fail_before_launch(lib):
    P = ctypes.c_void_p
    ok, mis = P(0x10000), P(0x10008)
    f, ap = lib.gqa_decode_sliding_ring, lib.gqa_append_sliding_ring
    for ring, window in ((1000, 1000), (8, 8), (262160, 1024), (1024, 1025), (1024, 0),
                         (0, 1024), (-16, 8)):
        assert f(ok, ok, ok, ok, ok, 4, ring, window, 1, None, 0, None) == -2, (ring, window)
        assert lib.gqa_decode_sliding_ring_workspace_bytes(4, ring, window) == 0
    assert f(ok, ok, ok, ok, ok, 4, 1024, 1024, 7, None, 0, None) == -3
    assert f(ok, ok, ok, None, ok, 4, 1024, 1024, 1, None, 0, None) == -1
    assert f(ok, mis, ok, ok, ok, 4, 1024, 1024, 1, None, 0, None) == -4
    # a small batch runs in stream mode: its workspace is required
    assert gqa.gqa_decode_sliding_ring_workspace_bytes(4, 1024, 1024) > 0
    assert f(ok, ok, ok, ok, ok, 4, 1024, 1024, 1, None, 0, None) == -5
    # the ring plans over the position domain, as a full-length windowed call
    for B, ring, w in ((4, 1024, 1024), (256, 1024, 1024), (256, 8192, 8192), (7, 48, 17)):
        assert gqa.gqa_decode_sliding_ring_workspace_bytes(B, ring, w) == \
            gqa.gqa_decode_workspace_bytes("sliding", B, 262144, window=w)
    for ring in (1000, 8, 0):
        assert ap(ok, ok, ok, ok, ok, ok, ok, ok, ok, 4, ring, 1, None) == -2
    assert ap(ok, ok, None, ok, ok, ok, ok, ok, ok, 4, 1024, 1, None) == -1
    assert ap(ok, ok, ok, ok, ok, ok, ok, ok, ok, 4, 1024, 7, None) == -3
    assert ap(ok, ok, ok, ok, ok, ok, ok, mis, ok, 4, 1024, 1, None) == -4


def test_append_arguments_fail_before_launch(lib):
    P = ctypes.c_void_p
    ok, mis = P(0x10000), P(0x10008)
    sl, gl = lib.gqa_append_sliding, lib.gqa_append_global_paged
    assert sl(ok, ok, None, ok, ok, ok, ok, ok, ok, 4, 64, 1, None) == -1   # sliding needs v_raw
    assert sl(ok, ok, ok, ok, ok, ok, ok, ok, ok, 0, 64, 1, None) == -2
    assert sl(ok, ok, ok, ok, ok, ok, ok, ok, ok, 4, 262145, 1, None) == -2
    assert sl(ok, ok, ok, ok, ok, ok, ok, ok, ok, 4, 64, 7, None) == -3
    assert sl(ok, ok, ok, mis, ok, ok, ok, ok, ok, 4, 64, 1, None) == -4
    assert gl(ok, ok, ok, ok, None, 8, ok, ok, ok, ok, 4, 8, 1, None) == -1
    assert gl(ok, ok, ok, ok, ok, 0, ok, ok, ok, ok, 4, 8, 1, None) == -2
    assert gl(ok, ok, ok, ok, ok, 8, ok, ok, ok, mis, 4, 8, 1, None) == -4


def test_values_only_arguments_fail_before_launch(lib):
    P = ctypes.c_void_p
    ok, mis = P(0x10000), P(0x10008)
    f, fp = lib.gqa_decode_global_k_eq_v, lib.gqa_decode_global_k_eq_v_paged
    # f(q, v, w_k, seq_lens, o, B, S_max, dtype, ws, ws_bytes, stream)
    assert f(ok, ok, None, ok, ok, 4, 64, 1, None, 0, None) == -1   # w_k is required
    assert f(ok, None, ok, ok, ok, 4, 64, 1, None, 0, None) == -1
    assert f(ok, ok, ok, ok, ok, 0, 64, 1, None, 0, None) == -2
    assert f(ok, ok, ok, ok, ok, 4, 262145, 1, None, 0, None) == -2
    assert f(ok, ok, ok, ok, ok, 4, 64, 5, None, 0, None) == -3
    assert f(ok, ok, mis, ok, ok, 4, 64, 1, None, 0, None) == -4
    assert f(ok, ok, ok, ok, ok, 4, 64, 1, None, 0, None) == -5     # stream plan needs workspace
    # fp(q, v_pool, w_k, block_table, max_pages, seq_lens, o, B, num_pages, dtype, ws, ...)
    assert fp(ok, ok, ok, None, 8, ok, ok, 4, 8, 1, None, 0, None) == -1
    assert fp(ok, ok, ok, ok, 0, ok, ok, 4, 8, 1, None, 0, None) == -2
    a, ap = lib.gqa_append_global_k_eq_v, lib.gqa_append_global_k_eq_v_paged
    # a(q_raw, k_raw, w_q, w_k, seq_lens, q_out, v_cache, B, S_max, dtype, stream)
    assert a(ok, ok, ok, ok, ok, ok, None, 4, 64, 1, None) == -1
    assert a(ok, ok, ok, ok, ok, ok, ok, 0, 64, 1, None) == -2
    assert a(ok, ok, ok, ok, ok, ok, mis, 4, 64, 1, None) == -4
    assert ap(ok, ok, ok, ok, None, 8, ok, ok, ok, 4, 8, 1, None) == -1


def test_prefill_arguments_fail_before_launch(lib):
    P = ctypes.c_void_p
    ok, mis = P(0x10000), P(0x10008)
    f, fp = lib.gqa_prefill_sliding, lib.gqa_prefill_global_paged
    # f(q, k, v, cu_q, seq_lens, o, B, N, S_max, dtype, stream)
    assert f(ok, ok, ok, None, ok, ok, 2, 64, 128, 1, None) == -1   # cu_q is required
    assert f(ok, ok, ok, ok, ok, ok, 0, 64, 128, 1, None) == -2
    assert f(ok, ok, ok, ok, ok, ok, 257, 64, 128, 1, None) == -2
    assert f(ok, ok, ok, ok, ok, ok, 2, 0, 128, 1, None) == -2      # no query rows
    assert f(ok, ok, ok, ok, ok, ok, 2, (1 << 24) + 1, 128, 1, None) == -2
    assert f(ok, ok, ok, ok, ok, ok, 2, 64, 262145, 1, None) == -2
    assert f(ok, ok, ok, ok, ok, ok, 2, 64, 128, 3, None) == -3
    assert f(mis, ok, ok, ok, ok, ok, 2, 64, 128, 1, None) == -4
    assert f(ok, ok, ok, ok, ok, mis, 2, 64, 128, 1, None) == -4
    # fp(q, k_pool, v_pool, block_table, max_pages, cu_q, seq_lens, o, B, N, num_pages, dtype, s)
    assert fp(ok, ok, ok, None, 8, ok, ok, ok, 2, 64, 8, 1, None) == -1
    assert fp(ok, ok, ok, ok, 0, ok, ok, ok, 2, 64, 8, 1, None) == -2
    assert fp(ok, ok, ok, ok, 8, ok, ok, ok, 2, 64, 0, 1, None) == -2
    # runtime-window prefill: fw(q, k, v, cu_q, seq_lens, o, B, N, S_max, window, dtype, s)
    fw, fwp = lib.gqa_prefill_sliding_window, lib.gqa_prefill_sliding_window_paged
    for w in (0, -1, 262145):
        assert fw(ok, ok, ok, ok, ok, ok, 2, 64, 128, w, 1, None) == -2
        # fwp(q, k_pool, v_pool, bt, max_pages, cu_q, seq_lens, o, B, N, num_pages, window, dt, s)
        assert fwp(ok, ok, ok, ok, 8, ok, ok, ok, 2, 64, 8, w, 1, None) == -2
    assert fw(ok, ok, ok, None, ok, ok, 2, 64, 128, 2048, 1, None) == -1
    assert fw(ok, ok, ok, ok, ok, ok, 2, 64, 128, 2048, 3, None) == -3


def test_binding_refuses_host_tensors(lib):
    import torch
    q = torch.zeros(1, 32, 256, dtype=torch.bfloat16)
    k = torch.zeros(1, 16, 16, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gqa.gqa_decode_sliding(q, k, k, torch.ones(1, dtype=torch.int32))


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "decode_attention_slidingdecodegqa_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read().lower()
                assert "oracle" not in src, f
    assert "oracle" not in open(HEADER).read().lower()


def test_slice_bounds_in_fp64_are_exact():
    """The kernels take the slice bounds floor(w*T/W) and the slice of a tile,
    floor(((t+1)*W - 1)/T), as fp64 divisions truncated to integers, for
    numerators below 2^40 and denominators below 2^27 (tile counts stay below
    2^26, slice counts below 2^12).  IEEE double division, which Python's float
    shares, gives the integer quotient there: the operands are exact, the
    quotient is correctly rounded, and a quotient that is not an integer lies
    at least 1/den from one."""
    import random
    rng = random.Random(7)
    cases = []
    for den in (1, 2, 3, 12, 255, 256, 1023, 2048, (1 << 26) - 1, 1 << 26, (1 << 27) - 1):
        top = ((1 << 40) - 1) // den * den
        cases += [(0, den), (den - 1, den), (den, den), (den + 1, den), (top, den), (top - 1, den),
                  ((1 << 40) - 1, den)]
    cases += [(rng.randrange(1 << 40), rng.randrange(1, 1 << 27)) for _ in range(200000)]
    # slice bounds as the kernels form them, at the largest tile and slice counts
    for T in (1, 255, 1 << 20, (1 << 26) - 1, 1 << 26):
        for W in (1, 256, 1023, 1024, 2048):
            for w in (0, 1, W // 2, W - 1, W):
                cases.append((w * T, W))
            for t in (0, 1, T // 3, T - 1):
                cases.append(((t + 1) * W - 1, T))
    bad = [(n, d) for n, d in cases if int(float(n) / float(d)) != n // d]
    assert not bad, bad[:5]
