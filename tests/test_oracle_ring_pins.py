"""Pins of the fp64 oracle over a sliding-layer cache capped at R positions
(the retrofit page's "Progressive Window Assignment": each layer keeps its own
KV cache capped at its window size), read as a ring with position s in slot
s % R.  CPU only.

The reference is independent of the oracle's ring arithmetic: the test builds
the ring from a linear cache with numpy (ring[b, s % R] = lin[b, s] for the
last R positions, NaN in the slots nothing has reached), and the linear-cache
oracle -- pinned on its own by the brute-force masked softmax, torch SDPA and
the closed forms -- must agree bit for bit.  Planted mistakes in a copy of the
oracle must each be caught.
"""
import numpy as np
import pytest

import oracle
import synth

HEADS = 32


def _np(t):
    return synth.to_numpy(t)


def _linear(dtype, lens, R, window, seed):
    """A linear cache holding (at least) the last R positions of each sequence."""
    cap = max(max(lens), 1)
    return synth.make_case("sliding", dtype, len(lens), cap, lens, seed=seed, window=window,
                           draw_from=[max(0, L - R) for L in lens])


def _ring_from_linear(c, R):
    """ring[b, s % R] = lin[b, s] for s in [max(0, L - R), L); NaN elsewhere."""
    k, v = _np(c.k), _np(c.v)
    B = k.shape[0]
    nan = np.float32("nan")
    if k.dtype == np.uint16:
        nan = np.uint16(0x7FC0)  # a bf16 quiet NaN
    rk = np.full((B, R) + k.shape[2:], nan, dtype=k.dtype)
    rv = np.full((B, R) + v.shape[2:], nan, dtype=v.dtype)
    for b in range(B):
        L = int(c.seq_lens[b])
        for s in range(max(0, L - R), L):
            rk[b, s % R] = k[b, s]
            rv[b, s % R] = v[b, s]
    return rk, rv


CASES = [
    # (R, window, seq_lens)
    (32, 32, [1, 31, 32, 33, 100, 327]),      # window = ring; no wrap, exactly full, wraps
    (48, 17, [5, 47, 48, 49, 200, 481]),      # ring not a power of two, window < ring
    (64, 1, [1, 2, 64, 65, 130]),             # window of one position
    (16, 16, [16, 17, 31, 32, 33, 1000]),     # the smallest ring, many wraps
]


def check_ring_equals_linear(lib):
    for R, W, lens in CASES:
        for dtype in ("f32", "bf16"):
            c = _linear(dtype, lens, R, W, seed=70 + R)
            rk, rv = _ring_from_linear(c, R)
            got = oracle.gqa_decode_ring(_np(c.q), rk, rv, _np(c.seq_lens), window=W, lib=lib)
            ref = oracle.gqa_decode("sliding", _np(c.q), _np(c.k), _np(c.v), _np(c.seq_lens),
                                    window=W, lib=lib)
            assert np.isfinite(got).all(), (R, W, dtype)
            assert np.array_equal(got, ref), (R, W, dtype)


def check_synth_ring_is_the_definition(lib):
    # the GPU tests' ring builder lays out exactly the ring above
    R, W, lens = 48, 17, [5, 47, 48, 49, 200, 481]
    for dtype in ("f32", "bf16"):
        c = _linear(dtype, lens, R, W, seed=80)
        rk, rv = _ring_from_linear(c, R)
        s = synth.make_ring_case(dtype, len(lens), R, lens, seed=80, window=W)
        k, v = _np(s.k), _np(s.v)
        assert np.array_equal(k.view(np.uint8), rk.view(np.uint8))  # NaN fills included
        assert np.array_equal(v.view(np.uint8), rv.view(np.uint8))
        assert np.array_equal(_np(s.q), _np(c.q))


def check_single_position_is_the_value_row(lib):
    # L = 1 (and a window of one after many wraps): o = v of the newest position
    R = 32
    c = synth.make_ring_case("f32", 2, R, [1, 1000], seed=81, window=1)
    got = oracle.gqa_decode_ring(_np(c.q), _np(c.k), _np(c.v), _np(c.seq_lens), window=1,
                                 lib=lib)
    for b, L in enumerate([1, 1000]):
        for h in (0, 17, 31):
            assert np.array_equal(got[b, h], _np(c.v)[b, (L - 1) % R, h // 2].astype(np.float64))


def check_window_above_ring_rejected(lib):
    c = synth.make_ring_case("f32", 1, 32, [40], seed=82, window=32)
    try:
        oracle.gqa_decode_ring(_np(c.q), _np(c.k), _np(c.v), _np(c.seq_lens), window=33,
                               lib=lib)
    except ValueError:
        return
    raise AssertionError("a window above the ring was accepted")


ALL = [check_single_position_is_the_value_row, check_ring_equals_linear,
       check_synth_ring_is_the_definition, check_window_above_ring_rejected]


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("check", ALL, ids=lambda f: f.__name__)
def test_ring_pin(lib, check):
    check(lib)


# planted mistakes; none of them reads outside the arrays
MUTANTS = {
    "slot_one_ahead": ("if (j->ring > 0) return (((int64_t)b * j->ring + s % j->ring) * j->KV",
                       "if (j->ring > 0) return (((int64_t)b * j->ring + (s + 1) % j->ring) * j->KV"),
    "ring_read_as_linear": ("return orc_run(dtype, q, k, v, NULL, NULL, 0, seq_lens, NULL, B, ring, ring,",
                            "return orc_run(dtype, q, k, v, NULL, NULL, 0, seq_lens, NULL, B, ring, 0,"),
    "window_check_dropped": ("(block_table || cu_q || window < 1 || window > ring)",
                             "(block_table || cu_q || window < 1)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_ring_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    mlib = oracle.load(oracle.build(str(path), str(tmp_path / f"libmutant_{name}.so")))
    for check in ALL:
        try:
            check(mlib)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            return
    pytest.fail(f"planted mistake {name} passed every ring pin")
