"""Pins of the fp64 prefill oracle (a chunk of new tokens per sequence attending
causally, or within the sliding window, to a cache that already holds the
chunk), CPU only.

The references are independent formulations: the masked score matrix of the
architecture page's compact forward pass written out in numpy (positions =
past + arange(T), full mask s <= t, sliding mask t - W < s <= t, scores +
mask, softmax, P @ V, repeat_kv), torch's SDPA in float64 with an explicit
boolean mask, closed forms (a fresh prompt's first token returns its own value
row; a dominant key at the window edge is selected exactly), and invariants
(keys after the query never matter; paged = contiguous).  Planted mistakes in
a copy of the oracle must each be caught.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import synth

F = torch.nn.functional


def _np(t):
    return t.detach().cpu().double().numpy()


def _numpy_reference(c: synth.PrefillCase) -> np.ndarray:
    """Compact forward pass, one sequence at a time, with the masks as matrices."""
    G = 32 // c.KV
    out = np.zeros((c.N, 32, c.D))
    cu = c.cu_q.tolist()
    for b in range(c.B):
        L = int(c.seq_lens[b])
        T = cu[b + 1] - cu[b]
        past = L - T
        t_pos = past + np.arange(T)                    # query positions
        s_pos = np.arange(L)                           # key positions (cache incl. chunk)
        keep = s_pos[None, :] <= t_pos[:, None]        # causal
        if c.window > 0:
            keep &= s_pos[None, :] > t_pos[:, None] - c.window
        mask = np.where(keep, 0.0, -np.inf)
        K = _np(c.k[b, :L])                            # [L, KV, D]
        V = _np(c.v[b, :L])
        Q = _np(c.q[cu[b]:cu[b + 1]])                  # [T, 32, D]
        for h in range(32):
            scores = Q[:, h] @ K[:, h // G].T * 1.0 + mask
            P = np.exp(scores - scores.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            out[cu[b]:cu[b + 1], h] = P @ V[:, h // G]
    return out


def _run(c, lib, rows=None):
    bt = None if c.block_table is None else synth.to_numpy(c.block_table)
    n = synth.to_numpy
    return oracle.gqa_prefill((c.KV, c.D, c.window), n(c.q), n(c.k), n(c.v), n(c.cu_q),
                              n(c.seq_lens), block_table=bt, rows=rows, lib=lib)


def _small(variant, window, seed, dtype="f32"):
    # one chunk after a cache, one fresh prompt, one single-token chunk
    return synth.make_prefill_case(variant, dtype, 48, [40, 7, 33], [9, 7, 1], seed=seed,
                                   window=window, fill=0.0)


def check_numpy_masked_matrix(lib):
    for variant, window in (("sliding", 5), ("sliding", 16), ("global", 0), ("sliding", 1)):
        for dtype in ("f32", "bf16"):
            c = _small(variant, window, seed=60, dtype=dtype)
            got = _run(c, lib)
            ref = _numpy_reference(c)
            assert np.abs(got - ref).max() <= 1e-12, (variant, window, dtype)


def check_torch_sdpa(lib):
    c = _small("global", 0, seed=61)
    got = _run(c, lib)
    cu = c.cu_q.tolist()
    for b in range(c.B):
        L, T = int(c.seq_lens[b]), cu[b + 1] - cu[b]
        q = c.q[cu[b]:cu[b + 1]].double().transpose(0, 1)               # [32, T, D]
        k = c.k[b, :L].double().repeat_interleave(8, dim=1).transpose(0, 1).contiguous()
        v = c.v[b, :L].double().repeat_interleave(8, dim=1).transpose(0, 1).contiguous()
        pos = torch.arange(L - T, L)[:, None]
        allowed = torch.arange(L)[None, :] <= pos
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=allowed, scale=1.0)
        assert np.abs(got[cu[b]:cu[b + 1]] - o.transpose(0, 1).numpy()).max() <= 1e-12


def check_fresh_prompt_first_token(lib):
    # a fresh prompt (past 0): token 0 attends only to itself, o = v[0] exactly
    c = _small("sliding", 1024, seed=62)
    got = _run(c, lib)
    for h in range(32):
        assert np.array_equal(got[9, h], _np(c.v[1, 0, h // 2]))
    # window 1: every token returns its own value row
    c1 = _small("sliding", 1, seed=63)
    got1 = _run(c1, lib)
    cu = c1.cu_q.tolist()
    for b in range(c1.B):
        L, T = int(c1.seq_lens[b]), cu[b + 1] - cu[b]
        for t in range(T):
            for h in (0, 31):
                assert np.array_equal(got1[cu[b] + t, h], _np(c1.v[b, L - T + t, h // 2]))


def check_window_edge_one_hot(lib):
    # a dominant key at the oldest kept position is selected exactly; moved one
    # step older it must be ignored
    W = 6
    c = _small("sliding", W, seed=64)
    b, t = 0, 4
    n = int(c.cu_q[b]) + t
    p = int(c.seq_lens[b]) - (int(c.cu_q[1]) - int(c.cu_q[0])) + t
    h = 5
    k = c.k.clone()
    k[b, p - W + 1, h // 2] = c.q[n, h] * 1e4
    c2 = synth.PrefillCase(c.variant, c.dtype, c.q, k, c.v, c.cu_q, c.seq_lens, None, c.cap, W)
    got = _run(c2, lib, rows=[(n, h)])
    assert np.array_equal(got[0], _np(c.v[b, p - W + 1, h // 2]))
    k = c.k.clone()
    k[b, p - W, h // 2] = c.q[n, h] * 1e4
    c3 = synth.PrefillCase(c.variant, c.dtype, c.q, k, c.v, c.cu_q, c.seq_lens, None, c.cap, W)
    assert np.array_equal(_run(c3, lib, rows=[(n, h)]), _run(c, lib, rows=[(n, h)]))


def check_future_keys_never_matter(lib):
    # keys and values after a query's position (later tokens of the chunk) are
    # poisoned: the earlier tokens' rows are unchanged and finite
    c = _small("global", 0, seed=65)
    base = _run(c, lib)
    cu = c.cu_q.tolist()
    b, t = 0, 3
    L, T = int(c.seq_lens[b]), cu[1] - cu[0]
    p = L - T + t
    k, v = c.k.clone(), c.v.clone()
    k[b, p + 1:], v[b, p + 1:] = float("nan"), float("nan")
    c2 = synth.PrefillCase(c.variant, c.dtype, c.q, k, v, c.cu_q, c.seq_lens, None, c.cap, 0)
    rows = [(cu[0] + tt, h) for tt in range(t + 1) for h in (0, 9, 31)]
    got = _run(c2, lib, rows=rows)
    ref = np.stack([base[n, h] for n, h in rows])
    assert np.isfinite(got).all() and np.array_equal(got, ref)


def check_last_token_matches_decode(lib):
    # the chunk's last token sits at L-1: the (separately pinned) decode
    # definition of the same cache
    c = _small("sliding", 1024, seed=66)
    got = _run(c, lib)
    n = synth.to_numpy
    last = [int(x) - 1 for x in c.cu_q[1:]]
    q_last = c.q[last].contiguous()
    dec = oracle.gqa_decode("sliding", n(q_last), n(c.k), n(c.v), n(c.seq_lens), lib=lib)
    assert np.abs(got[last] - dec).max() <= 1e-13


def check_paged_equals_contiguous(lib):
    c = synth.make_prefill_case("global", "bf16", 64, [60, 20], [12, 20], seed=67, fill=0.0)
    paged = synth.make_prefill_case("global", "bf16", 64, [60, 20], [12, 20], seed=67, fill=0.0,
                                    paged=True, extra_pages=2)
    assert np.array_equal(_run(c, lib), _run(paged, lib))
    # the same through the pins' own contiguous-to-paged shuffle
    d = oracle_pins._contig_to_paged(
        synth.Case(c.variant, c.dtype, c.q[:2], c.k, c.v, c.seq_lens, None, c.cap, c.window),
        seed=68)
    pc = synth.PrefillCase(c.variant, c.dtype, c.q, d.k, d.v, c.cu_q, c.seq_lens, d.block_table,
                           d.cap, c.window)
    assert np.array_equal(_run(c, lib), _run(pc, lib))


ALL = [check_fresh_prompt_first_token, check_numpy_masked_matrix, check_torch_sdpa,
       check_window_edge_one_hot, check_future_keys_never_matter,
       check_last_token_matches_decode, check_paged_equals_contiguous]


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("check", ALL, ids=lambda f: f.__name__)
def test_prefill_pin(lib, check):
    check(lib)


MUTANTS = {
    "window_one_long": ("(j->window > 0 && pos - j->window + 1 > 0) ? pos - j->window + 1 : 0;",
                        "(j->window > 0 && pos - j->window > 0) ? pos - j->window : 0;"),
    "kv_head_modulo": ("const int kvh = h / (ORC_HEADS / j->KV);",
                       "const int kvh = h % j->KV;"),
    "sequence_lookup_off_by_one": ("while (b < j->B && j->cu_q[b + 1] <= n) ++b;",
                                   "while (b < j->B && j->cu_q[b + 1] < n) ++b;"),
    "query_row_of_sequence": ("const size_t q_at = ((size_t)n * ORC_HEADS + h) * (size_t)D;",
                              "const size_t q_at = ((size_t)b * ORC_HEADS + h) * (size_t)D;"),
    "position_one_early": ("const int64_t pos = Lb - T_b + (n - j->cu_q[b]);",
                           "const int64_t pos = Lb - T_b + (n - j->cu_q[b]) - 1;"),
    "positions_ignore_the_past": ("const int64_t pos = Lb - T_b + (n - j->cu_q[b]);",
                                  "const int64_t pos = (n - j->cu_q[b]);"),
    "no_max_subtraction_sign": ("score[i] = exp(score[i] - top);",
                                "score[i] = exp(top - score[i]);"),
    "normaliser_dropped": ("for (int d = 0; d < D; ++d) out[d] = out[d] / total;", ""),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_prefill_mistake_is_caught(name, tmp_path):
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
    pytest.fail(f"planted mistake {name} passed every prefill pin")
