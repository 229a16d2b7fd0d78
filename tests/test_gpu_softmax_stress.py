"""Online-softmax stress: logits that keep rising across a unit, and large
random logits, HIP path vs the fp64 oracle through the C ABI.

The kernels keep a reference maximum per head and rescale their running sums
only when a tile's logits exceed it by more than 8 (natural-log units); the
combine kernel and the unit kernel's in-LDS merge weight partial results by
exp(m_i - M).  The synthetic caches of the other tests rarely exercise these
paths after the first tile, so the cases here build logits (tests/
stress_cases.py) that
  * rise by up to 24 per 16-position tile along whole sequences (bf16) or in
    16-tile sawteeth of +-100 (f32), with per-head coefficients that make
    other heads fall or stay flat: repeated rescales with factors strictly
    between 0 and 1 in every wave, and partials whose maxima differ widely;
  * are large and random (about +-100 bf16, +-25 f32; the values-only
    calls within their accuracy envelope, tests/stress_cases.py).
They run in the planner's launch modes (unit: one work-group per (sequence,
kv head); stream on the sliding geometry and group on the global one: units
split across waves or work-groups, merged by the combine kernel), both cache
forms, f32 and bf16, for the decode, runtime-window, values-only and prefill
calls.  The bars are the usual 1e-4 (f32) and 2e-2 (bf16) max-abs errors.
"""
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import oracle
import synth
from gpu_cases import (TOL, hip_run, hip_run_k_eq_v, max_err, oracle_run, oracle_run_k_eq_v,
                       to_f64, to_gpu)
from stress_cases import KFV_Q_SCALE, apply_large, stress_decode_case, stress_prefill_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


# (variant, window, B, capacity, lengths, expected launch mode)
DECODE_SHAPES = {
    "sliding-unit": ("sliding", None, 8, 1104, [1104, 1, 1041, 700, 1024, 16, 1103, 333], "unit"),
    "sliding-stream": ("sliding", None, 4, 4096, [4096, 1025, 3000, 17], "stream"),
    "window4096-stream": ("sliding", 4096, 4, 9008, [9008, 4097, 2500, 6000], "stream"),
    "global-unit": ("global", None, 64, 512, None, "unit"),
    "global-group": ("global", None, 3, 16384, [16384, 9000, 333], "group"),
}


def _lens(shape_key, B, cap):
    lens = DECODE_SHAPES[shape_key][4]
    if lens is None:
        lens = synth.draw_seq_lens(("uniform", 1, cap), B, 77).tolist()
        lens[0], lens[1] = cap, 1
    return lens


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pattern", ["ramp", "large"])
@pytest.mark.parametrize("shape", sorted(DECODE_SHAPES))
def test_decode_softmax_stress(shape, pattern, dtype, paged):
    variant, window, B, cap, _, mode = DECODE_SHAPES[shape]
    assert gqa.gqa_decode_plan(variant, B, cap, window=window)["mode"] == mode
    lens = _lens(shape, B, cap)
    c = stress_decode_case(pattern, variant, dtype, B, cap, lens, seed=300 + len(shape),
                           paged=paged, window=window)
    ref = oracle_run(c, window=window)
    got = to_f64(hip_run(to_gpu(c), window=window))
    err = max_err(got, ref)
    assert err <= TOL[dtype], (shape, pattern, dtype, paged, err)


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,cap", [(64, 512), (3, 16384)], ids=["unit", "group"])
def test_values_only_large_logits(B, cap, dtype, paged):
    # keys rebuilt from values: the query alone carries the scale (the values
    # are the keys, so scaling them would scale the outputs too), within the
    # accuracy envelope of the kernel's folded key weight (KFV_Q_SCALE)
    lens = synth.draw_seq_lens(("uniform", 1, cap), B, 78).tolist()
    lens[0] = cap
    c = synth.make_case("global", dtype, B, cap, lens, paged=paged, seed=310, extra_pages=2)
    apply_large(c, scale_k=False, scale=KFV_Q_SCALE[dtype])
    ref = oracle_run_k_eq_v(c)
    got = to_f64(hip_run_k_eq_v(to_gpu(c)))
    err = max_err(got, ref)
    assert err <= TOL[dtype], (B, dtype, paged, err)


def _prefill_oracle(pc):
    bt = None if pc.block_table is None else synth.to_numpy(pc.block_table)
    return oracle.gqa_prefill((pc.KV, pc.D, pc.window), synth.to_numpy(pc.q),
                              synth.to_numpy(pc.k), synth.to_numpy(pc.v),
                              synth.to_numpy(pc.cu_q), synth.to_numpy(pc.seq_lens),
                              block_table=bt, nthreads=16)


def _prefill_gpu(pc, window=None):
    dev = "cuda"
    q, k, v, cu, sl = (t.to(dev) for t in (pc.q, pc.k, pc.v, pc.cu_q, pc.seq_lens))
    bt = None if pc.block_table is None else pc.block_table.to(dev)
    if window is not None:
        return gqa.gqa_prefill_sliding_window(q, k, v, cu, sl, window, block_table=bt)
    fn = gqa.gqa_prefill_sliding if pc.variant == "sliding" else gqa.gqa_prefill_global
    return fn(q, k, v, cu, sl, block_table=bt)


@pytest.mark.parametrize("paged", [False, True], ids=["contig", "paged"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pattern", ["ramp", "large"])
@pytest.mark.parametrize("variant", ["sliding", "global"])
def test_prefill_softmax_stress(variant, pattern, dtype, paged):
    # a chunk after a long past (crossing the window), a fresh prompt, a short chunk
    cap = 1808
    lens, q_lens = [1800, 1100, 700], [200, 1100, 40]
    pc = stress_prefill_case(pattern, variant, dtype, cap, lens, q_lens, seed=320, paged=paged)
    ref = _prefill_oracle(pc)
    got = to_f64(_prefill_gpu(pc))
    err = max_err(got, ref)
    assert err <= TOL[dtype], (variant, pattern, dtype, paged, err)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_window_ramp(dtype):
    pc = stress_prefill_case("ramp", "sliding", dtype, 4608, [4600, 3000], [700, 64], seed=330,
                             paged=True, window=2048)
    ref = _prefill_oracle(pc)
    got = to_f64(_prefill_gpu(pc, window=2048))
    err = max_err(got, ref)
    assert err <= TOL[dtype], (dtype, err)
