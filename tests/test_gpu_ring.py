"""slidingDecodeGQA over a cache capped at R positions (ring: position s in
slot s % R; the retrofit page's per-layer caches capped at the window) vs the
fp64 oracle, through the C ABI, on an MI355X."""
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


def _n(t):
    return synth.to_numpy(t)


def _gpu(c):
    return synth.Case(c.variant, c.dtype, c.q.cuda(), c.k.cuda(), c.v.cuda(), c.seq_lens.cuda(),
                      None, c.cap, c.window, c.w_k.cuda())


def _oracle(c, window, rows=None):
    return oracle.gqa_decode_ring(_n(c.q), _n(c.k), _n(c.v), _n(c.seq_lens), window=window,
                                  rows=rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ring,window,lens", [
    # not yet full, exactly full, one past, many wraps, the longest sequence
    (1024, 1024, [1, 1000, 1024, 1025, 5000, 262144]),
    # window below the ring; lengths around the ring and window edges
    (2048, 1500, [1499, 1500, 1501, 2047, 2048, 2049, 10007]),
    # a ring that is not a power of two, a window of 17
    (48, 17, [1, 16, 17, 47, 48, 49, 96, 1001]),
], ids=["r1024_w1024", "r2048_w1500", "r48_w17"])
def test_ring_parity(ring, window, lens, dtype):
    c = synth.make_ring_case(dtype, len(lens), ring, lens, seed=500 + ring, window=window)
    got = to_f64(gqa.gqa_decode_sliding_ring(*(x.cuda() for x in (c.q, c.k, c.v, c.seq_lens)),
                                             window=window))
    torch.cuda.synchronize()
    assert np.isfinite(got).all()  # the NaN in never-written slots is never read
    err = max_err(got, _oracle(c, window))
    assert err <= TOL[dtype], err


def test_ring_equals_linear_bitwise():
    """The same rows in a ring and in a linear cache give the same bits (the
    kernel reads the same positions in the same order; only the slot differs)."""
    R, W = 1024, 1024
    lens = [1, 700, 1024, 1025, 2500, 4000]
    ring = synth.make_ring_case("bf16", len(lens), R, lens, seed=510, window=W)
    lin = synth.make_case("sliding", "bf16", len(lens), max(lens), lens, seed=510, window=W,
                          draw_from=[max(0, L - R) for L in lens])
    a = gqa.gqa_decode_sliding_ring(*(x.cuda() for x in (ring.q, ring.k, ring.v, ring.seq_lens)),
                                    window=W)
    b = gqa.gqa_decode_sliding_window(*(x.cuda() for x in (lin.q, lin.k, lin.v, lin.seq_lens)),
                                      W)
    assert torch.equal(a.cpu(), b.cpu())


def test_ring_unit_mode_sampled():
    # B = 256: 4096 units, unit mode; ring = window = 1024; lengths up to 262144
    B, R = 256, 1024
    assert gqa.gqa_decode_sliding_ring_workspace_bytes(B, R, R) == 0
    lens = synth.draw_seq_lens(("uniform", 1, 262144), B, seed=511)
    lens[0], lens[1], lens[2] = 1, R, 262144
    c = synth.make_ring_case("bf16", B, R, lens, seed=511, window=R, device="cuda")
    got = to_f64(gqa.gqa_decode_sliding_ring(c.q, c.k, c.v, c.seq_lens, window=R))
    assert np.isfinite(got).all()
    host = synth.Case(c.variant, c.dtype, c.q.cpu(), c.k.cpu(), c.v.cpu(), c.seq_lens.cpu(),
                      None, c.cap, c.window, c.w_k.cpu())
    rows = [(b, h) for b in (0, 1, 2, 99, 255) for h in (0, 13, 31)]
    ref = _oracle(host, R, rows=rows)
    for i, (b, h) in enumerate(rows):
        assert max_err(got[b, h], ref[i]) <= TOL["bf16"], (b, h, int(lens[b]))


def test_ring_window_8192_stream_mode():
    # the widest window of the retrofit table in its own 8192-slot ring
    B, R = 8, 8192
    lens = [1, 8191, 8192, 8193, 20000, 100001, 262144, 16]
    c = synth.make_ring_case("bf16", B, R, lens, seed=512, window=R)
    got = to_f64(gqa.gqa_decode_sliding_ring(*(x.cuda() for x in (c.q, c.k, c.v, c.seq_lens)),
                                             window=R))
    rows = [(b, h) for b in range(B) for h in (0, 31)]
    ref = _oracle(c, R, rows=rows)
    for i, (b, h) in enumerate(rows):
        assert max_err(got[b, h], ref[i]) <= TOL["bf16"], (b, h)


def test_ring_append_then_attend():
    """Append the new token into the ring on the GPU (slot (L-1) % R), then
    attend; the oracle appends the same token (fp64) into a copy of the ring."""
    R, W = 64, 64
    lens = [1, 63, 64, 65, 128, 129, 1000]
    B = len(lens)
    for dtype in ("f32", "bf16"):
        c = synth.make_ring_case(dtype, B, R, lens, seed=513, window=W, fill=0.0)
        g = torch.Generator().manual_seed(514)
        tdt = synth.TORCH_DTYPES[dtype]
        q_raw = (torch.randn(B, HEADS, 256, generator=g) * 2).to(tdt)
        k_raw = (torch.randn(B, 16, 256, generator=g) * 3).to(tdt)
        v_raw = torch.randn(B, 16, 256, generator=g).to(tdt)
        w_q = torch.empty(256).uniform_(0.2, 0.4, generator=g).to(tdt)
        w_k = torch.empty(256).uniform_(0.2, 0.4, generator=g).to(tdt)
        kc, vc = c.k.cuda(), c.v.cuda()
        k_before, v_before = kc.clone(), vc.clone()
        sl = c.seq_lens.cuda()
        q_out = gqa.gqa_append_sliding_ring(q_raw.cuda(), k_raw.cuda(), v_raw.cuda(), w_q.cuda(),
                                            w_k.cuda(), sl, kc, vc)
        o = gqa.gqa_decode_sliding_ring(q_out, kc, vc, sl, window=W)
        eq, ek, ev, pos = oracle.gqa_append_rows("sliding", _n(q_raw), _n(k_raw), _n(v_raw),
                                                 _n(w_q), _n(w_k), np.asarray(lens, np.int32))
        k_after, v_after = kc.cpu(), vc.cpu()
        host_k, host_v = c.k.clone(), c.v.clone()
        for b in range(B):
            slot = int(pos[b]) % R
            assert max_err(k_after[b, slot].double().numpy(), ek[b]) <= TOL[dtype], (dtype, b)
            assert max_err(v_after[b, slot].double().numpy(), ev[b]) <= TOL[dtype], (dtype, b)
            host_k[b, slot] = torch.from_numpy(ek[b]).to(tdt)
            host_v[b, slot] = torch.from_numpy(ev[b]).to(tdt)
            # the written slot aside, the ring is untouched
            k_after[b, slot] = k_before[b, slot].cpu()
            v_after[b, slot] = v_before[b, slot].cpu()
        assert torch.equal(k_after, k_before.cpu()) and torch.equal(v_after, v_before.cpu())
        assert max_err(to_f64(q_out), eq) <= TOL[dtype]
        ref = oracle.gqa_decode_ring(_n(torch.from_numpy(eq).to(tdt)), _n(host_k), _n(host_v),
                                     np.asarray(lens, np.int32), window=W)
        assert max_err(to_f64(o), ref) <= TOL[dtype], dtype
