"""The allocation-free entry point gqa_decode_global_paged_noalloc against
gqa_decode_global_paged, through the C ABI, on the GPU.

It runs the same kernels with the library's own device array as the
workspace, so its output must equal the workspace entry point's bit for bit
(and the fp64 oracle within the bf16/f32 bars).  Two calls in a row, the
second on a smaller input, check that a call does not depend on what the
previous one left in the shared array; a unit-mode batch (no workspace) and
a stream-mode batch of each dtype are covered.  Collected last: it is the
only test that touches the library-owned array.
"""
import pytest
import torch

import decode_attention_slidingdecodegqa_amd as gqa
import synth
from gpu_cases import TOL, hip_run, max_err, oracle_run, to_f64, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests selected but no GPU is visible")
    gqa.library()


def _noalloc(c):
    o = torch.empty_like(c.q)
    return gqa.gqa_decode_global_paged_noalloc(c.q, c.k, c.v, c.block_table, c.seq_lens, o)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_the_workspace_entry_point(dtype):
    big = to_gpu(synth.make_case("global", dtype, 12, 16384,
                                 synth.draw_seq_lens(("uniform", 1, 16384), 12, 61).tolist(),
                                 paged=True, seed=501, extra_pages=2))
    small = to_gpu(synth.make_case("global", dtype, 3, 2048, [2048, 700, 1], paged=True,
                                   seed=502, extra_pages=2))
    for c in (big, small):
        assert gqa.gqa_decode_plan("global", c.B, c.cap)["mode"] == "group"
    got_big = _noalloc(big)
    got_small = _noalloc(small)          # the second call, on a smaller input
    torch.cuda.synchronize()
    for c, got in ((big, got_big), (small, got_small)):
        ref = hip_run(c)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), c.B
        assert max_err(to_f64(got), oracle_run(c)) <= TOL[dtype]


def test_noalloc_unit_mode_and_repeat():
    c = to_gpu(synth.make_case("global", "bf16", 64, 512,
                               synth.draw_seq_lens(("uniform", 1, 512), 64, 62).tolist(),
                               paged=True, seed=503))
    assert gqa.gqa_decode_plan("global", c.B, c.cap)["mode"] == "unit"
    a = _noalloc(c)
    s = to_gpu(synth.make_case("global", "bf16", 2, 4096, [4096, 3000], paged=True, seed=504))
    b = _noalloc(s)
    a2 = _noalloc(c)
    torch.cuda.synchronize()
    assert torch.equal(a, hip_run(c)) and torch.equal(a, a2)
    assert torch.equal(b, hip_run(s))


def test_noalloc_rejects_bad_arguments_before_any_launch():
    c = to_gpu(synth.make_case("global", "bf16", 2, 64, [64, 5], paged=True, seed=505))
    lib = gqa.library()
    o = torch.empty_like(c.q)
    args = [c.q.data_ptr(), c.k.data_ptr(), c.v.data_ptr(), c.block_table.data_ptr(),
            c.block_table.shape[1], c.seq_lens.data_ptr(), o.data_ptr(), 2, c.k.shape[0], 1, None]
    bad_b = list(args)
    bad_b[7] = 257
    assert lib.gqa_decode_global_paged_noalloc(*bad_b) == -2
    bad_dt = list(args)
    bad_dt[9] = 5
    assert lib.gqa_decode_global_paged_noalloc(*bad_dt) == -3
    with pytest.raises(ValueError):
        gqa.gqa_decode_global_paged_noalloc(c.q, c.k, c.v, c.block_table, c.seq_lens, None)
