"""Seeded inputs whose logits stress the online softmax (test inputs only).

The synthetic caches of synth.py give logits of a few units (unit-RMS q and k
times weights in [0.2, 0.4], scale 1), so a wave's running maximum is set by
its first tile and an online-softmax rescale almost never fires after it.
The attention of the gemma-4-31B Model Spec page has scale 1 and no soft-cap
on the logits ("Compute-graph nodes", attn.core rows; the soft-cap is on the
LM head only), so larger and trending logits are in its domain.  Two
patterns, applied to a case built by synth on the host:

  ramp   one key coordinate per kv head carries a ramp along the positions,
         and every query head weights it by its own coefficient, so the
         logits of a head rise (or fall, or stay flat) by a fixed amount per
         16-position tile on top of the random part.  bf16: a plain ramp,
         per-tile rises up to 24 over whole sequences (repeated rescales in
         every wave, partials whose maxima differ by hundreds).  f32: a
         sawtooth of the same slope with a period of 16 tiles, so the logits
         stay within about +-100 (the f32 bar of 1e-4 assumes fp32 logits
         whose rounding is small next to it) while every slice still sees
         several rises of more than 8.
  large  q and k scaled up so that the logits are about +-100 (bf16, scale
         10: weights about 3) or +-25 (f32, scale 2.5).  The f32 bar is an
         absolute 1e-4 while the fp32 rounding of a logit grows with its
         magnitude: at scale 5 the global geometry (D = 512) measured
         1.0-2.0e-4, all of it logit rounding (an fp32 emulation of the
         products on the host gives the same trend: 1.1e-5 at scale 2,
         2.0e-5 at 2.5, 7.9e-5 at 5 on a subsample of the prefill case).

The ramp coordinate of kv head g is D-1-g, one of the last coordinates of
the head dimension, so that the large ramp term enters the fp32 dot product
late and its rounding stays small next to the f32 bar.
"""
from __future__ import annotations

import torch

import synth

HEADS = 32
# per-query-head multipliers of the ramp (head h uses RAMP_COEF[h % 8]);
# f32 keeps the sawtooth amplitude within about +-100 with |coef| <= 1
RAMP_COEF = {"bf16": (0.5, 1.0, 1.5, -1.0, 0.25, 2.0, 0.0, -0.5),
             "f32": (1.0, 0.75, -1.0, 0.5, 0.0, -0.5, 0.25, 1.0)}
RAMP_SLOPE = 0.75          # per position: a 12-unit rise per tile at coefficient 1
SAW_PERIOD = 256           # positions (16 tiles) of the f32 sawtooth
LARGE_SCALE = {"bf16": 10.0, "f32": 2.5}


def ramp_coord(D: int, g: int) -> int:
    return D - 1 - g


def _rows_of(c, b, positions):
    """(index tuple) addressing the cache rows of sequence b at `positions`."""
    pos = torch.as_tensor(positions, dtype=torch.int64)
    if c.block_table is None:
        return (torch.full_like(pos, b), pos)
    page = c.block_table[b].cpu().to(torch.int64)[pos // 16]
    return (page, pos % 16)


def ramp_value(dtype: str, pos: torch.Tensor, lo: int, L: int) -> torch.Tensor:
    """The ramp key component at positions pos of a sequence drawn on [lo, L)."""
    if dtype == "f32":
        return RAMP_SLOPE * ((pos - lo) % SAW_PERIOD - SAW_PERIOD // 2).to(torch.float32)
    return RAMP_SLOPE * (pos - (lo + L) // 2).to(torch.float32)


def apply_ramp(c, ranges):
    """Put the ramp into case c (synth.Case or synth.PrefillCase, on the host).

    ranges: per sequence, the drawn positions [lo, L) whose key rows exist;
    every query row gets the same head coefficients."""
    KV, D = c.KV, c.D
    G = HEADS // KV
    coef = RAMP_COEF[c.dtype]
    q = c.q.to(torch.float32)
    for h in range(HEADS):
        q[:, h, ramp_coord(D, h // G)] = coef[h % 8]
    c.q = q.to(c.q.dtype)
    for b, (lo, L) in enumerate(ranges):
        if L <= lo:
            continue
        pos = torch.arange(lo, L)
        idx = _rows_of(c, b, pos)
        vals = ramp_value(c.dtype, pos, lo, L).to(c.k.dtype)
        for g in range(KV):
            c.k[idx[0], idx[1], g, ramp_coord(D, g)] = vals
    return c


# The values-only global calls rebuild each key from its value row and fold
# the key weight into the query (rounded to bf16 on the 448 coordinates that
# do not rotate), where the oracle rounds the rebuilt key as a stored key
# would be.  The two roundings differ by about 2^-9 of each product, so their
# max-abs difference grows with the logit scale: an exact host emulation of
# the kernel's rounding against the oracle, on the two shapes tested below,
# gives 0.002-0.013 at the synthetic scale, 0.005-0.013 at 1.25x, 0.010-0.022
# at 1.5x and 0.14 at 10x (the GPU measured 0.12-0.14 at 10x).  Their
# large-logit case therefore scales q by 1.25 in bf16; f32 keys are rebuilt in
# fp32 and take the f32 scale of the other calls.
KFV_Q_SCALE = {"bf16": 1.25, "f32": 2.5}


def apply_large(c, scale_k: bool = True, scale: float | None = None):
    """Scale q (and k) so that the logits are tens to hundreds of units."""
    s = LARGE_SCALE[c.dtype] if scale is None else scale
    c.q = (c.q.to(torch.float32) * s).to(c.q.dtype)
    if scale_k:
        c.k = (c.k.to(torch.float32) * s).to(c.k.dtype)
    return c


def decode_ranges(c):
    return [c.attended(b) for b in range(c.B)]


def stress_decode_case(pattern, variant, dtype, B, cap, lens, seed, paged=False, window=None):
    c = synth.make_case(variant, dtype, B, cap, lens, paged=paged, seed=seed, window=window,
                        extra_pages=3)
    if pattern == "ramp":
        return apply_ramp(c, decode_ranges(c))
    return apply_large(c)


def prefill_ranges(pc):
    """Drawn positions of each sequence of a prefill case: from the first
    chunk token's window start to seq_lens[b]."""
    out = []
    cu = pc.cu_q.tolist()
    for b, L in enumerate(pc.seq_lens.tolist()):
        T = cu[b + 1] - cu[b]
        p0 = L - T
        lo = max(0, p0 - pc.window + 1) if pc.window > 0 else 0
        out.append((min(lo, max(L, 0)), max(L, 0)))
    return out


def stress_prefill_case(pattern, variant, dtype, cap, lens, q_lens, seed, paged=False,
                        window=None):
    pc = synth.make_prefill_case(variant, dtype, cap, lens, q_lens, paged=paged, seed=seed,
                                 window=window, extra_pages=3)
    if pattern == "ramp":
        return apply_ramp(pc, prefill_ranges(pc))
    return apply_large(pc)
