"""Seeded synthetic inputs for Gemma-4-31B decode attention.

This module is shared by both sides of every parity check: the fp64 oracle
(``oracle/``) and the HIP library (``decode_attention_slidingdecodegqa_amd``)
receive the very same bytes from it.  It holds none of the attention
arithmetic: it draws random numbers, shapes them like the tensors the upstream
nodes produce, lays them out in a contiguous or paged cache and fills the
unused cache space.

Value recipe (the attention inputs are outputs of upstream nodes of the
gemma-4-31B Model Spec page, "Compute-graph nodes" table):
  * q, k: per-head RMS-normalised N(0,1) draws (attn.qk_norm, eps 1e-6) times a
    per-channel weight of length D drawn U(0.2, 0.4), one weight for q and one
    for k, shared across heads, batch and positions;
  * v: per-head RMS-normalised N(0,1) draw with no weight (attn.v_norm,
    "rmsnormUnit"), i.e. unit RMS;
  * decodeGQA ("values = keys"): k and v come from the same raw draw r,
    v = unit-RMS(r), k = w_k * unit-RMS(r); RoPE is not applied (it is an
    upstream node; the kernel sees post-RoPE keys whatever they are).  The
    values-only calls take v and w_k (kept in ``Case.w_k``, rounded to the
    dtype) and rebuild their own keys.
Only positions inside the attended range [max(0, L-W), L) are drawn; every
other cache slot (and every unreferenced page) holds ``fill``: NaN for
correctness runs (so a stray read shows up), zero for timing runs.  Block-table
entries no position inside the attended range needs are -1.
"""
from __future__ import annotations

import dataclasses
import torch

HEADS = 32
PAGE = 16
EPS = 1e-6
# variant -> (kv heads, head dim, window); window 0 = none
VARIANTS = {"sliding": (16, 256, 1024), "global": (4, 512, 0)}

# The workloads (shape domain of the Model Spec page's "At a glance" table:
# B <= 256, S <= 262144, page 16).  Keys are descriptive workload names.
WORKLOADS = {
    "sliding_f32_b4_s2048": dict(variant="sliding", dtype="f32", B=4, cap=2048, paged=False,
                                 lens=("uniform_straddle", 1, 2048)),
    "global_bf16_b4_s4096": dict(variant="global", dtype="bf16", B=4, cap=4096, paged=False,
                                 lens=("uniform", 1, 4096)),
    "sliding_bf16_b256_s8192": dict(variant="sliding", dtype="bf16", B=256, cap=8192,
                                    paged=False, lens=("uniform", 1, 8192)),
    "global_bf16_b32_paged_s16k_128k": dict(variant="global", dtype="bf16", B=32, cap=131072,
                                            paged=True, lens=("uniform", 16384, 131072)),
    "sliding_bf16_b1_paged_s262144": dict(variant="sliding", dtype="bf16", B=1, cap=262144,
                                          paged=True, lens=("fixed", 262144, 262144)),
    "global_bf16_b1_paged_s262144": dict(variant="global", dtype="bf16", B=1, cap=262144,
                                         paged=True, lens=("fixed", 262144, 262144)),
}

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Case:
    variant: str
    dtype: str               # "f32" | "bf16"
    q: torch.Tensor          # [B, 32, D]
    k: torch.Tensor          # [B, cap, KV, D] or [num_pages, 16, KV, D]
    v: torch.Tensor
    seq_lens: torch.Tensor   # [B] int32
    block_table: torch.Tensor | None  # [B, max_pages] int32 or None
    cap: int                 # S_max (contiguous) or max_pages*16 (paged)
    window: int
    w_k: torch.Tensor | None = None  # [D] the k weight the keys were drawn with, in dtype

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def paged(self):
        return self.block_table is not None

    @property
    def KV(self):
        return VARIANTS[self.variant][0]

    @property
    def D(self):
        return VARIANTS[self.variant][1]

    def attended(self, b: int, window: int | None = None) -> tuple[int, int]:
        """[lo, L) of sequence b under `window` (default: the case's window; 0 = none)."""
        W = self.window if window is None else window
        L = int(self.seq_lens[b])
        L = max(0, min(L, self.cap))
        lo = max(0, L - W) if W > 0 else 0
        return lo, L

    def kv_bytes(self, window: int | None = None) -> int:
        """Algorithmic K+V bytes one call reads (each attended row once)."""
        eb = 4 if self.dtype == "f32" else 2
        lens = self.seq_lens.tolist()
        W = self.window if window is None else window
        n = 0
        for L in lens:
            L = max(0, min(int(L), self.cap))
            n += L - (max(0, L - W) if W > 0 else 0)
        return n * self.KV * self.D * 2 * eb


def _gen(seed: int, tag: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag) % (2**63 - 1))
    return g


def rms_unit(x: torch.Tensor) -> torch.Tensor:
    """Per-row RMS normalisation over the last axis, no weight (eps 1e-6)."""
    return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + EPS)


def draw_seq_lens(lens, B: int, seed: int) -> torch.Tensor:
    kind, lo, hi = lens
    g = _gen(seed, 1, "cpu")
    if kind == "fixed":
        return torch.full((B,), hi, dtype=torch.int32)
    s = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    if kind == "uniform_straddle" and B >= 2:
        # at least one sequence below and one above the 1024 window
        if not bool((s < 1024).any()):
            s[0] = int(torch.randint(1, 1024, (1,), generator=g))
        if not bool((s > 1024).any()):
            s[-1] = int(torch.randint(1025, hi + 1, (1,), generator=g))
    return s


def make_case(variant: str, dtype: str, B: int, cap: int, seq_lens, paged: bool = False,
              seed: int = 0, device="cpu", fill: float = float("nan"), window: int | None = None,
              extra_pages: int = 0, alloc_all_pages: bool = False, draw_from=None) -> Case:
    """Build one seeded case.

    seq_lens: int list/tensor [B] (values outside [0, cap] are the caller's
    business).  paged: lay K/V out as a page pool with a random page
    permutation; the pool holds exactly the pages the attended ranges touch
    (all pages below L when ``alloc_all_pages``) plus ``extra_pages``
    unreferenced ones.  window: override of the variant's window.  draw_from:
    optional per-sequence first position to draw (instead of L - window).
    """
    KV, D, W = VARIANTS[variant]
    if window is not None:
        W = window
    tdt = TORCH_DTYPES[dtype]
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32).cpu()
    assert seq_lens.shape == (B,)
    g_w = _gen(seed, 2, device)
    w_q = torch.empty(D, device=device).uniform_(0.2, 0.4, generator=g_w)
    w_k = torch.empty(D, device=device).uniform_(0.2, 0.4, generator=g_w)
    g_q = _gen(seed, 3, device)
    q = (w_q * rms_unit(torch.randn(B, HEADS, D, generator=g_q, device=device))).to(tdt)

    def rng_of(b):
        return _gen(seed, 1000 + b, device)

    def rows(b, n):
        """K and V rows for n attended positions of sequence b, fp32 [n, KV, D]."""
        g = rng_of(b)
        if variant == "global":
            r = rms_unit(torch.randn(n, KV, D, generator=g, device=device))
            return w_k * r, r
        kx = rms_unit(torch.randn(n, KV, D, generator=g, device=device))
        vx = rms_unit(torch.randn(n, KV, D, generator=g, device=device))
        return w_k * kx, vx

    ranges = []
    for b in range(B):
        L = max(0, min(int(seq_lens[b]), cap))
        lo = max(0, L - W) if W > 0 else 0
        if draw_from is not None:
            lo = max(0, min(int(draw_from[b]), L))
        ranges.append((lo, L))

    if not paged:
        k = torch.full((B, cap, KV, D), fill, dtype=tdt, device=device)
        v = torch.full((B, cap, KV, D), fill, dtype=tdt, device=device)
        for b, (lo, L) in enumerate(ranges):
            if L > lo:
                kr, vr = rows(b, L - lo)
                k[b, lo:L] = kr.to(tdt)
                v[b, lo:L] = vr.to(tdt)
        return Case(variant, dtype, q, k, v, seq_lens.to(device), None, cap, W, w_k.to(tdt))

    assert cap % PAGE == 0
    max_pages = cap // PAGE
    first_last = []
    for lo, L in ranges:
        if L <= lo:
            first_last.append((0, 0))
            continue
        p0 = 0 if alloc_all_pages else lo // PAGE
        first_last.append((p0, (L + PAGE - 1) // PAGE))
    n_used = sum(p1 - p0 for p0, p1 in first_last)
    num_pages = max(1, n_used + extra_pages)
    perm = torch.randperm(num_pages, generator=_gen(seed, 4, "cpu"))
    bt = torch.full((B, max_pages), -1, dtype=torch.int32)
    k = torch.full((num_pages, PAGE, KV, D), fill, dtype=tdt, device=device)
    v = torch.full((num_pages, PAGE, KV, D), fill, dtype=tdt, device=device)
    nxt = 0
    for b, ((lo, L), (p0, p1)) in enumerate(zip(ranges, first_last)):
        if p1 <= p0:
            continue
        phys = perm[nxt:nxt + (p1 - p0)]
        nxt += p1 - p0
        bt[b, p0:p1] = phys.to(torch.int32)
        if L <= lo:
            continue
        kr, vr = rows(b, L - lo)
        # logical positions lo..L-1 -> (page, slot); pad to whole pages with fill
        a0 = p0 * PAGE
        span = (p1 - p0) * PAGE
        kb = torch.full((span, KV, D), fill, dtype=tdt, device=device)
        vb = torch.full((span, KV, D), fill, dtype=tdt, device=device)
        kb[lo - a0:L - a0] = kr.to(tdt)
        vb[lo - a0:L - a0] = vr.to(tdt)
        idx = phys.to(device=device, dtype=torch.int64)
        k[idx] = kb.view(p1 - p0, PAGE, KV, D)
        v[idx] = vb.view(p1 - p0, PAGE, KV, D)
    return Case(variant, dtype, q, k, v, seq_lens.to(device), bt.to(device), cap, W,
                w_k.to(tdt))


def make_ring_case(dtype: str, B: int, ring: int, seq_lens, seed: int = 0, device="cpu",
                   fill: float = float("nan"), window: int = 1024) -> Case:
    """A sliding-layer cache capped at ``ring`` positions: k, v [B, ring, 16, 256]
    with position s in slot s % ring, holding the last min(L, ring) positions
    of each sequence.  The rows are the ones ``make_case(..., draw_from=L -
    ring)`` draws for the same positions (same seed and order); unused slots
    hold ``fill``.  seq_lens may exceed ring."""
    KV, D, _ = VARIANTS["sliding"]
    tdt = TORCH_DTYPES[dtype]
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32).cpu()
    assert seq_lens.shape == (B,)
    g_w = _gen(seed, 2, device)
    w_q = torch.empty(D, device=device).uniform_(0.2, 0.4, generator=g_w)
    w_k = torch.empty(D, device=device).uniform_(0.2, 0.4, generator=g_w)
    g_q = _gen(seed, 3, device)
    q = (w_q * rms_unit(torch.randn(B, HEADS, D, generator=g_q, device=device))).to(tdt)
    k = torch.full((B, ring, KV, D), fill, dtype=tdt, device=device)
    v = torch.full((B, ring, KV, D), fill, dtype=tdt, device=device)
    for b in range(B):
        L = int(seq_lens[b])
        n = max(0, min(L, ring))
        if n == 0:
            continue
        g = _gen(seed, 1000 + b, device)
        kx = rms_unit(torch.randn(n, KV, D, generator=g, device=device))
        vx = rms_unit(torch.randn(n, KV, D, generator=g, device=device))
        slots = torch.arange(L - n, L, device=device) % ring
        k[b, slots] = (w_k * kx).to(tdt)
        v[b, slots] = vx.to(tdt)
    return Case("sliding", dtype, q, k, v, seq_lens.to(device), None, ring, window, w_k.to(tdt))


@dataclasses.dataclass
class PrefillCase:
    """A chunk of T_b new tokens per sequence, already appended to the cache:
    sequence b holds seq_lens[b] positions, its query rows cu_q[b] .. cu_q[b+1]-1
    are its last T_b positions."""
    variant: str
    dtype: str
    q: torch.Tensor          # [N, 32, D]
    k: torch.Tensor          # as Case
    v: torch.Tensor
    cu_q: torch.Tensor       # [B+1] int32
    seq_lens: torch.Tensor   # [B] int32
    block_table: torch.Tensor | None
    cap: int
    window: int

    @property
    def B(self):
        return self.seq_lens.shape[0]

    @property
    def N(self):
        return self.q.shape[0]

    @property
    def KV(self):
        return VARIANTS[self.variant][0]

    @property
    def D(self):
        return VARIANTS[self.variant][1]

    def attended_pairs(self) -> int:
        """Unmasked (query token, key) pairs of one kv head and one query head."""
        n = 0
        lens = self.seq_lens.tolist()
        cu = self.cu_q.tolist()
        for b, L in enumerate(lens):
            T = cu[b + 1] - cu[b]
            for t in range(T):
                p = L - T + t
                if p < 0:
                    continue
                n += p + 1 - (max(0, p - self.window + 1) if self.window > 0 else 0)
        return n

    def flops(self) -> int:
        """Algorithmic flops: QK^T and PV over every unmasked pair, all 32 heads."""
        return 4 * HEADS * self.D * self.attended_pairs()


def make_prefill_case(variant: str, dtype: str, cap: int, seq_lens, q_lens, paged: bool = False,
                      seed: int = 0, device="cpu", fill: float = float("nan"),
                      window: int | None = None, extra_pages: int = 0) -> PrefillCase:
    """Seeded prefill case: the cache rows every query of the chunk attends to are
    drawn like make_case's (positions from the first chunk token's window start
    to seq_lens[b]); every other slot holds ``fill``.  q [N,32,D] is drawn like
    the decode queries (per-head RMS-normalised times w_q)."""
    KV, D, W = VARIANTS[variant]
    if window is not None:
        W = window
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int32).cpu()
    q_lens = torch.as_tensor(q_lens, dtype=torch.int32).cpu()
    B = seq_lens.shape[0]
    draw_from = []
    for b in range(B):
        p0 = int(seq_lens[b]) - int(q_lens[b])  # position of the first chunk token
        draw_from.append(max(0, p0 - W + 1) if W > 0 else 0)
    c = make_case(variant, dtype, B, cap, seq_lens, paged=paged, seed=seed, device=device,
                  fill=fill, window=W, extra_pages=extra_pages, draw_from=draw_from)
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(q_lens, 0)
    N = int(cu[-1])
    g_w = _gen(seed, 5, device)
    w_q = torch.empty(D, device=device).uniform_(0.2, 0.4, generator=g_w)
    g_q = _gen(seed, 6, device)
    q = (w_q * rms_unit(torch.randn(N, HEADS, D, generator=g_q, device=device)))
    return PrefillCase(variant, dtype, q.to(TORCH_DTYPES[dtype]), c.k, c.v, cu.to(device),
                       c.seq_lens, c.block_table, cap, W)


# Prefill workloads (no page names one; shapes inside the Spec's domain): a
# chunk of T new tokens after a cached past, every sequence alike.
PREFILL_WORKLOADS = {
    "sliding_bf16_prefill_b8_past4096_chunk2048": dict(variant="sliding", dtype="bf16", B=8,
                                                        past=4096, chunk=2048, paged=False),
    "global_bf16_prefill_b2_past8192_chunk2048_paged": dict(variant="global", dtype="bf16", B=2,
                                                            past=8192, chunk=2048, paged=True),
}


def make_prefill_workload(name: str, seed: int = 0, device="cpu",
                          fill: float = float("nan"), window: int | None = None) -> PrefillCase:
    """One of PREFILL_WORKLOADS by name; `window` overrides the sliding window."""
    w = PREFILL_WORKLOADS[name]
    L = w["past"] + w["chunk"]
    cap = (L + PAGE - 1) // PAGE * PAGE
    return make_prefill_case(w["variant"], w["dtype"], cap, [L] * w["B"], [w["chunk"]] * w["B"],
                             paged=w["paged"], seed=seed, device=device, fill=fill, window=window)


def make_workload(name: str, seed: int = 0, device="cpu", fill: float = float("nan"),
                  B: int | None = None, window: int | None = None) -> Case:
    """One of WORKLOADS by name (B may be cut down for a quick CPU-sized run; `window`
    overrides the variant's window, which decides the rows drawn)."""
    w = WORKLOADS[name]
    nb = w["B"] if B is None else B
    lens = draw_seq_lens(w["lens"], w["B"], seed)[:nb]
    return make_case(w["variant"], w["dtype"], nb, w["cap"], lens, paged=w["paged"], seed=seed,
                     device=device, fill=fill, window=window)


def to_numpy(t: torch.Tensor):
    """Host numpy view of a tensor as the oracle takes it (bf16 -> uint16 bits)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def expected_kv_bytes(name: str) -> float:
    """Expected algorithmic K+V bytes per call of a workload (over its seq_len law)."""
    w = WORKLOADS[name]
    KV, D, W = VARIANTS[w["variant"]]
    eb = 4 if w["dtype"] == "f32" else 2
    kind, lo, hi = w["lens"]
    vals = range(lo, hi + 1) if kind != "fixed" else [hi]
    n = sum(min(L, W) if W > 0 else L for L in vals) / len(vals)
    return w["B"] * n * KV * D * 2 * eb


__all__ = ["Case", "make_case", "make_workload", "PrefillCase", "make_prefill_case",
           "PREFILL_WORKLOADS", "make_prefill_workload", "WORKLOADS", "VARIANTS", "to_numpy",
           "draw_seq_lens", "rms_unit", "expected_kv_bytes", "HEADS", "PAGE"]

if __name__ == "__main__":  # pragma: no cover - quick look at the workloads
    for n in WORKLOADS:
        print(n, f"{expected_kv_bytes(n) / 1e9:.3f} GB/call")
