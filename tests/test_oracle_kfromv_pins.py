"""Pins of the fp64 decodeGQA oracle over a values-only cache (keys rebuilt as
rope(w_k * v_s, s): values = keys on the global layers), CPU only.

The reference is the already pinned plain decode oracle run on a key cache
built here independently (RoPE as complex multiplication in numpy, fp64,
stored as float32), plus paged = contiguous and planted mistakes.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import synth


def _case(B, cap, lens, seed, paged=False):
    c = synth.make_case("global", "f32", B, cap, lens, seed=seed, paged=paged, fill=0.0)
    g = torch.Generator().manual_seed(seed + 1)
    w_k = torch.empty(512).uniform_(0.2, 0.4, generator=g)
    return c, w_k


def _keys_from_values(v, w_k, pos):
    """rope(w_k * v, pos) for rows v [..., 512] at positions pos [...] (complex form)."""
    u = v.astype(np.float64) * w_k.astype(np.float64)
    z = u[..., :256] + 1j * u[..., 256:]
    i = np.arange(256)
    f = np.where(i < 64, 1e6 ** (-2.0 * i / 512), 0.0)
    z = z * np.exp(1j * pos[..., None] * f)
    return np.concatenate([z.real, z.imag], axis=-1)


def check_matches_explicit_key_cache(lib):
    c, w_k = _case(3, 700, [700, 1, 333], seed=40)
    v = c.v.numpy()
    pos = np.arange(c.cap, dtype=np.float64)[None, :, None] * np.ones((c.B, 1, 4))
    k = _keys_from_values(v, w_k.numpy(), pos).astype(np.float32)
    ref = oracle.gqa_decode("global", c.q.numpy(), k, v, c.seq_lens.numpy(), lib=lib)
    got = oracle.gqa_decode_k_from_v(c.q.numpy(), v, w_k.numpy(), c.seq_lens.numpy(), lib=lib)
    assert np.abs(got - ref).max() <= 1e-5


def check_paged_equals_contiguous(lib):
    c, w_k = _case(3, 96, [96, 17, 50], seed=41)
    p = oracle_pins._contig_to_paged(c, seed=42)
    a = oracle.gqa_decode_k_from_v(c.q.numpy(), c.v.numpy(), w_k.numpy(), c.seq_lens.numpy(),
                                   lib=lib)
    b = oracle.gqa_decode_k_from_v(p.q.numpy(), p.v.numpy(), w_k.numpy(), p.seq_lens.numpy(),
                                   block_table=p.block_table.numpy(), lib=lib)
    assert np.array_equal(a, b)


def check_single_position(lib):
    # one position: the output is the value row whatever the key
    c, w_k = _case(2, 16, [1, 1], seed=43)
    got = oracle.gqa_decode_k_from_v(c.q.numpy(), c.v.numpy(), w_k.numpy(), c.seq_lens.numpy(),
                                     lib=lib)
    for h in range(32):
        assert np.array_equal(got[:, h], c.v[:, 0, h // 8].double().numpy())


ALL = [check_single_position, check_matches_explicit_key_cache, check_paged_equals_contiguous]


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("check", ALL, ids=lambda f: f.__name__)
def test_k_from_v_pin(lib, check):
    check(lib)


MUTANTS = {
    "position_one_late": ("orc_rope(k, j->D, (long)s, 1e6, 64);",
                          "orc_rope(k, j->D, (long)s + 1, 1e6, 64);"),
    "sliding_theta": ("orc_rope(k, j->D, (long)s, 1e6, 64);",
                      "orc_rope(k, j->D, (long)s, 1e4, 64);"),
    "all_pairs_active": ("orc_rope(k, j->D, (long)s, 1e6, 64);",
                         "orc_rope(k, j->D, (long)s, 1e6, 256);"),
    "weight_dropped": ("k[d] = orc_elem(j->w_k, j->dtype, (size_t)d) * orc_elem(j->v, j->dtype, (size_t)off + d);",
                       "k[d] = orc_elem(j->v, j->dtype, (size_t)off + d);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_k_from_v_mistake_is_caught(name, tmp_path):
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
    pytest.fail(f"planted mistake {name} passed every k-from-v pin")
