"""Pins that tie the fp64 oracle to something other than itself.

Each ``check_*`` takes an oracle library handle (``oracle.load(path)``) and
raises AssertionError (or any exception) when the oracle disagrees with:
  * a brute force of the masked-softmax forward pass written the way the
    "Gemma 4 31B-it Text Architecture" page's compact forward pass spells it
    (repeat_kv materialised, scores = Q K^T * 1.0 + additive mask with keys
    t-1024 < s <= t, softmax, P @ V), in numpy float64;
  * torch's scaled_dot_product_attention in float64 on the CPU (a library
    routine: the special case with an explicit boolean mask and scale 1);
  * closed forms (one position, equal keys, a hand-computed three-position
    softmax), exact selection by a dominant logit, the GQA head mapping, the
    IEEE definition of bfloat16 widening;
  * invariants (window = full attention when L <= 1024, paged = contiguous,
    position permutation, poison outside the attended range).
The same checks run against copies of the oracle with planted mistakes (see
test_oracle_pins.py), each of which at least one check must catch.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import synth

HEADS = 32


def _np(t):
    return synth.to_numpy(t)


def _f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def run_oracle(lib, case: synth.Case, window=None, rows=None, nthreads=4):
    bt = None if case.block_table is None else _np(case.block_table)
    return oracle.gqa_decode((case.KV, case.D, case.window if window is None else window),
                             _np(case.q), _np(case.k), _np(case.v), _np(case.seq_lens),
                             block_table=bt, rows=rows, nthreads=nthreads, lib=lib)


def brute_force(q, k, v, seq_lens, KV, window):
    """Compact forward pass of the architecture page, one decode query per sequence.

    q [B,32,D], k/v [B,S,KV,D] float64; the cache holds positions 0..L-1, the
    query is position t = L-1.
    """
    B, H, D = q.shape
    G = H // KV
    out = np.zeros((B, H, D))
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        t = L - 1
        K = np.repeat(k[b, :L], G, axis=1)  # repeat_kv -> [L, 32, D]
        V = np.repeat(v[b, :L], G, axis=1)
        s = np.arange(L)
        allowed = s <= t
        if window > 0:
            allowed &= s > t - window
        mask = np.where(allowed, 0.0, -np.inf)
        scores = np.einsum("hd,shd->hs", q[b], K) * 1.0 + mask[None, :]
        P = np.exp(scores - scores.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        out[b] = np.einsum("hs,shd->hd", P, V)
    return out


def _full_case(variant, dtype, B, cap, lens, seed):
    """All positions [0, L) drawn (no window in the generator) so brute force can read them."""
    return synth.make_case(variant, dtype, B, cap, lens, seed=seed, window=0, fill=0.0)


def check_bruteforce_small(lib):
    for variant in ("sliding", "global"):
        for dtype in ("f32", "bf16"):
            c = _full_case(variant, dtype, 3, 48, [1, 17, 48], seed=11)
            for W in (1, 3, 16, 17, 0):
                got = run_oracle(lib, c, window=W)
                ref = brute_force(_f64(c.q), _f64(c.k), _f64(c.v), _np(c.seq_lens), c.KV, W)
                err = np.abs(got - ref).max()
                assert err <= 1e-12, (variant, dtype, W, err)


def check_bruteforce_window1024(lib):
    c = _full_case("sliding", "f32", 4, 2048, [1100, 1024, 1025, 2047], seed=12)
    got = run_oracle(lib, c, window=1024)
    ref = brute_force(_f64(c.q), _f64(c.k), _f64(c.v), _np(c.seq_lens), c.KV, 1024)
    err = np.abs(got - ref).max()
    assert err <= 1e-12, err


def check_sdpa(lib):
    F = torch.nn.functional
    for variant, dtype, lens, W in (("global", "bf16", [5, 40], 0), ("sliding", "f32", [30, 9], 7)):
        c = _full_case(variant, dtype, 2, 40, lens, seed=13)
        got = run_oracle(lib, c, window=W)
        G = HEADS // c.KV
        for b in range(c.B):
            L = int(c.seq_lens[b])
            q = c.q[b].to(torch.float64)[:, None, :]                      # [32,1,D]
            K = c.k[b, :L].to(torch.float64).repeat_interleave(G, 1).transpose(0, 1)
            V = c.v[b, :L].to(torch.float64).repeat_interleave(G, 1).transpose(0, 1)
            s = torch.arange(L)
            allowed = s <= L - 1
            if W > 0:
                allowed &= s > L - 1 - W
            ref = F.scaled_dot_product_attention(q, K.contiguous(), V.contiguous(),
                                                 attn_mask=allowed[None, None, :], scale=1.0)
            err = np.abs(got[b] - ref[:, 0, :].numpy()).max()
            assert err <= 1e-12, (variant, b, err)


def check_L1_exact(lib):
    for variant in ("sliding", "global"):
        for dtype in ("f32", "bf16"):
            c = synth.make_case(variant, dtype, 3, 32, [1, 1, 1], seed=14)
            got = run_oracle(lib, c)
            G = HEADS // c.KV
            for b in range(3):
                for h in range(HEADS):
                    exp = _f64(c.v[b, 0, h // G])
                    assert np.array_equal(got[b, h], exp), (variant, dtype, b, h)


def check_all_keys_equal(lib):
    for variant, dtype, cap, lens in (("sliding", "f32", 1600, [1025, 1500, 600, 1024]),
                                      ("global", "bf16", 4000, [300, 4000])):
        c = synth.make_case(variant, dtype, len(lens), cap, lens, seed=15)
        for b in range(c.B):
            lo, L = c.attended(b)
            c.k[b, lo:L] = c.k[b, lo:lo + 1].clone()  # every key of the range equal
        got = run_oracle(lib, c)
        G = HEADS // c.KV
        for b in range(c.B):
            lo, L = c.attended(b)
            mean = c.v[b, lo:L].to(torch.float64).mean(0)  # [KV, D]
            for h in range(HEADS):
                err = np.abs(got[b, h] - mean[h // G].numpy()).max()
                assert err <= 1e-13, (variant, b, h, err)


def one_hot_case(variant, dtype, B, cap, lens, positions, seed, paged=False):
    """q[b,h] = e_{j_h}; k[.,g,j_h] in [-4,4] except 160 at positions[b]."""
    c = synth.make_case(variant, dtype, B, cap, lens, seed=seed, paged=paged)
    KV, D = c.KV, c.D
    G = HEADS // KV
    gen = torch.Generator().manual_seed(seed + 99)
    js = [(h * 37 + 5) % D for h in range(HEADS)]
    q = torch.zeros(B, HEADS, D)
    for h in range(HEADS):
        q[:, h, js[h]] = 1.0
    c.q = q.to(c.q.dtype)
    for b in range(B):
        lo, L = c.attended(b)
        s = torch.arange(lo, L)
        if c.block_table is None:
            page, slot = None, None
        else:
            page = c.block_table[b, s // 16].long()
            slot = s % 16
        for h in range(HEADS):
            g = h // G
            vals = torch.empty(L - lo).uniform_(-4, 4, generator=gen)
            vals[s == positions[b]] = 160.0
            vals = vals.to(c.k.dtype)
            if page is None:
                c.k[b, lo:L, g, js[h]] = vals
            else:
                c.k[page, slot, g, js[h]] = vals
    # the dominant key component of every head of the group at positions[b]
    for b in range(B):
        p = positions[b]
        for h in range(HEADS):
            if c.block_table is None:
                c.k[b, p, h // G, js[h]] = 160.0
            else:
                c.k[int(c.block_table[b, p // 16]), p % 16, h // G, js[h]] = 160.0
    return c


def value_row(c, b, s, g):
    if c.block_table is None:
        return c.v[b, s, g]
    return c.v[int(c.block_table[b, s // 16]), s % 16, g]


def check_one_hot(lib):
    for variant, dtype, paged in (("sliding", "bf16", False), ("global", "f32", True),
                                  ("sliding", "f32", True)):
        lens = [1030, 200, 47, 1024]
        cap = 1040
        for pick in ("lo", "last", "page0", "page15"):
            pos = []
            for L in lens:
                lo = max(0, L - 1024) if variant == "sliding" else 0
                p = {"lo": lo, "last": L - 1, "page0": ((lo + 15) // 16) * 16,
                     "page15": ((lo + 15) // 16) * 16 + 15}[pick]
                pos.append(min(p, L - 1))
            c = one_hot_case(variant, dtype, 4, cap, lens, pos, seed=16, paged=paged)
            got = run_oracle(lib, c)
            G = HEADS // c.KV
            for b in range(4):
                for h in range(HEADS):
                    exp = _f64(value_row(c, b, pos[b], h // G))
                    assert np.array_equal(got[b, h], exp), (variant, paged, pick, b, h)


def check_three_position_closed_form(lib):
    # logits 0, 1, 2 on head 0 and value rows e_0, e_1, e_2:
    # o[0] = (1, e, e^2, 0, ...) / (1 + e + e^2)
    c = synth.make_case("sliding", "f32", 1, 8, [3], seed=17)
    c.q.zero_()
    c.q[0, 0, 0] = 1.0
    c.k.zero_()
    c.v.zero_()
    for s in range(3):
        c.k[0, s, 0, 0] = float(s)
        c.v[0, s, 0, s] = 1.0
    got = run_oracle(lib, c)
    den = 1.0 + math.e + math.e ** 2
    exp = np.zeros(256)
    exp[:3] = [1.0 / den, math.e / den, math.e ** 2 / den]
    assert np.abs(got[0, 0] - exp).max() <= 1e-15, got[0, 0, :4]
    # head 1 shares kv head 0 with q = 0: uniform weights
    assert np.abs(got[0, 1, :3] - 1.0 / 3).max() <= 1e-15


def check_sliding_equals_full(lib):
    c = synth.make_case("sliding", "f32", 4, 1024, [1, 513, 1000, 1024], seed=18)
    a = run_oracle(lib, c, window=1024)
    b = run_oracle(lib, c, window=0)
    assert np.array_equal(a, b)
    c2 = _full_case("sliding", "f32", 1, 1100, [1100], seed=18)
    assert not np.array_equal(run_oracle(lib, c2, window=1024), run_oracle(lib, c2, window=0))


def _contig_to_paged(c: synth.Case, seed: int) -> synth.Case:
    """The same logical cache through a random page permutation (built here, not by synth)."""
    B, cap = c.B, c.cap
    npg = cap // 16
    gen = torch.Generator().manual_seed(seed)
    need = [(int(c.seq_lens[b]) + 15) // 16 for b in range(B)]
    total = sum(need) + 3  # three unreferenced pages
    perm = torch.randperm(total, generator=gen)
    pool_k = torch.full((total, 16, c.KV, c.D), float("nan"), dtype=c.k.dtype)
    pool_v = torch.full_like(pool_k, float("nan"))
    bt = torch.full((B, npg), -1, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        for p in range(need[b]):
            phys = int(perm[nxt])
            nxt += 1
            bt[b, p] = phys
            pool_k[phys] = c.k[b, p * 16:(p + 1) * 16]
            pool_v[phys] = c.v[b, p * 16:(p + 1) * 16]
    return synth.Case(c.variant, c.dtype, c.q, pool_k, pool_v, c.seq_lens, bt, cap, c.window)


def check_paged_equals_contiguous(lib):
    for variant, dtype, lens in (("global", "bf16", [1, 95, 33]), ("sliding", "f32", [96, 16, 50])):
        c = synth.make_case(variant, dtype, 3, 96, lens, seed=19)
        p = _contig_to_paged(c, seed=20)
        for W in (0, 20):
            assert np.array_equal(run_oracle(lib, c, window=W), run_oracle(lib, p, window=W)), \
                (variant, W)


def check_permutation(lib):
    c = synth.make_case("sliding", "f32", 2, 1500, [700, 1400], seed=21)
    a = run_oracle(lib, c)
    gen = torch.Generator().manual_seed(22)
    for b in range(2):
        lo, L = c.attended(b)
        perm = torch.randperm(L - lo, generator=gen) + lo
        c.k[b, lo:L] = c.k[b, perm].clone()
        c.v[b, lo:L] = c.v[b, perm].clone()
    assert np.abs(run_oracle(lib, c) - a).max() <= 1e-13


def check_poison(lib):
    for variant, paged in (("sliding", False), ("sliding", True), ("global", True)):
        lens = [1300, 20, 1025]
        a = synth.make_case(variant, "bf16", 3, 1328, lens, paged=paged, seed=23,
                            fill=float("nan"), extra_pages=4)
        z = synth.make_case(variant, "bf16", 3, 1328, lens, paged=paged, seed=23, fill=0.0,
                            extra_pages=4)
        ra, rz = run_oracle(lib, a), run_oracle(lib, z)
        assert np.isfinite(ra).all() and np.array_equal(ra, rz), (variant, paged)
        if paged and variant == "sliding":
            # pages entirely below the window are not even in the table
            assert int(a.block_table[0, 0]) == -1


def check_bf16_widening(lib):
    pats = [0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0xC2C8, 0x0000, 0x3C00]
    vals = [1.0, -1.0, 3.140625, 2.0 ** -133, 2.0 ** 127 * (1 + 127 / 128), -100.0, 0.0,
            2.0 ** -7]
    c = synth.make_case("global", "bf16", 1, 16, [1], seed=24)
    row = torch.tensor(pats * (512 // len(pats)), dtype=torch.int32).to(torch.int16)
    for g in range(4):
        c.v[0, 0, g] = row.view(torch.bfloat16)
    got = run_oracle(lib, c)
    exp = np.array(vals * (512 // len(vals)))
    for h in range(HEADS):
        assert np.array_equal(got[0, h], exp), h


def check_gqa_mapping(lib):
    for variant in ("sliding", "global"):
        c = synth.make_case(variant, "f32", 2, 64, [64, 9], seed=25)
        for g in range(c.KV):
            c.v[:, :, g, :] = float(g + 1)
        got = run_oracle(lib, c)
        G = HEADS // c.KV
        for h in range(HEADS):
            assert np.abs(got[:, h] - (h // G + 1)).max() <= 1e-14 * (h // G + 1), (variant, h)


ALL_CHECKS = [
    check_three_position_closed_form,
    check_L1_exact,
    check_bf16_widening,
    check_gqa_mapping,
    check_all_keys_equal,
    check_bruteforce_small,
    check_sdpa,
    check_one_hot,
    check_sliding_equals_full,
    check_paged_equals_contiguous,
    check_permutation,
    check_poison,
    check_bruteforce_window1024,
]
