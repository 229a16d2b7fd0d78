"""fp64 CPU oracle for Gemma-4-31B decode attention (slidingDecodeGQA / decodeGQA).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and
the benchmark's ``cpu_baseline`` leg may import this package.  The HIP library
never imports, links or calls it, and it imports nothing from the HIP side.

The arithmetic lives in ``gqa_oracle.c`` (plain C, double precision); this
module only compiles it with gcc and marshals numpy arrays into it.  It
follows the attn.core rows of the "Compute-graph nodes" table of the
gemma-4-31B Model Spec page and the tensor shapes of its "Tensors of the main
nodes" table.

Parity status of every function here: pinned by ``tests/test_oracle_pins.py``
(brute-force masked softmax, torch SDPA in float64, closed forms, bit-exact
selection, invariants and planted-mistake checks), and for the other entry
points by ``tests/test_oracle_{append,kfromv,prefill,ring}_pins.py``.  The only unpinned reading
is the zero row for seq_len <= 0 ("parity unpinned": the pages' shape domain
starts at S = 1).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gqa_oracle.c")
LIBRARY = os.path.join(_HERE, "libgqaoracle.so")

HEADS = 32
PAGE = 16
F32, BF16 = 0, 1

# variant -> (kv heads, head dim, window); attn.core rows of the Model Spec page
VARIANTS = {
    "sliding": (16, 256, 1024),
    "global": (4, 512, 0),
}

_ERRORS = {-1: "bad argument", -2: "seq_len above capacity", -3: "page id outside pool",
           -4: "out of memory"}


def build(source: str = SOURCE, out: str = LIBRARY, extra=()) -> str:
    """Compile the oracle with gcc (no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           *extra, source, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_libs: dict = {}


def load(path: str = LIBRARY):
    """Load (building first if absent) an oracle shared library."""
    path = os.path.abspath(path)
    if path in _libs:
        return _libs[path]
    if path == os.path.abspath(LIBRARY) and not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    fn = lib.oracle_gqa_decode
    p = ctypes.c_void_p
    i32 = ctypes.c_int32
    fn.argtypes = [ctypes.c_int, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, p, i32,
                   p, i32]
    fn.restype = ctypes.c_int
    kv = lib.oracle_gqa_decode_k_from_v
    kv.argtypes = [ctypes.c_int, p, p, p, p, p, i32, i32, i32, i32, p, i32, p, i32]
    kv.restype = ctypes.c_int
    pf = lib.oracle_gqa_prefill
    pf.argtypes = [ctypes.c_int, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, i32, p,
                   i32, p, i32]
    pf.restype = ctypes.c_int
    ap = lib.oracle_gqa_append_rows
    ap.argtypes = [ctypes.c_int, p, p, p, p, p, p, i32, i32, i32, p, p, p, p]
    ap.restype = ctypes.c_int
    rg = lib.oracle_gqa_decode_ring
    rg.argtypes = [ctypes.c_int, p, p, p, p, i32, i32, i32, i32, i32, p, i32, p, i32]
    rg.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # raw bfloat16 bit patterns
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits) arrays, got {a.dtype}")


def gqa_decode(variant, q, k, v, seq_lens, block_table=None, num_pages=None, rows=None,
               nthreads: int | None = None, window: int | None = None, lib=None) -> np.ndarray:
    """Reference decode attention in fp64.

    variant: "sliding" or "global" (or an explicit (KV, D, window) tuple).
    q [B,32,D]; k, v [B,S,KV,D] (contiguous) or [num_pages,16,KV,D] (paged, with
    block_table [B,max_pages] int32); seq_lens [B] int32.  q/k/v are float32
    arrays or uint16 arrays holding bf16 bits.  ``window`` overrides the
    variant's window (<= 0: none).  ``rows``: optional list of (b, h) pairs.
    Returns float64 [B,32,D], or [len(rows), D] when rows is given.
    """
    KV, D, W = VARIANTS[variant] if isinstance(variant, str) else variant
    if window is not None:
        W = window
    lib = lib or load()
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share a dtype")
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = q.shape[0]
    if q.shape != (B, HEADS, D) or seq_lens.shape != (B,):
        raise ValueError("q must be [B,32,D] and seq_lens [B]")
    if block_table is None:
        if k.ndim != 4 or k.shape[0] != B or k.shape[2:] != (KV, D) or v.shape != k.shape:
            raise ValueError("contiguous k/v must be [B,S,KV,D]")
        cap, max_pages, n_pages, bt = k.shape[1], 0, 0, None
    else:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        if bt.ndim != 2 or bt.shape[0] != B:
            raise ValueError("block_table must be [B,max_pages]")
        if k.ndim != 4 or k.shape[1:] != (PAGE, KV, D) or v.shape != k.shape:
            raise ValueError("paged k/v must be [num_pages,16,KV,D]")
        max_pages = bt.shape[1]
        n_pages = k.shape[0] if num_pages is None else num_pages
        cap = max_pages * PAGE
    if rows is None:
        rows_arr, n_rows = None, B * HEADS
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        n_rows = rows_arr.shape[0]
    out = np.zeros((n_rows, D), dtype=np.float64)
    nthreads = nthreads or min(os.cpu_count() or 1, 16)
    rc = lib.oracle_gqa_decode(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(bt), B, cap,
                               max_pages, n_pages, KV, D, W, _ptr(rows_arr), n_rows, _ptr(out),
                               nthreads)
    if rc != 0:
        raise ValueError(f"oracle error {rc}: {_ERRORS.get(rc, '?')}")
    return out.reshape(B, HEADS, D) if rows is None else out


def gqa_decode_ring(q, k, v, seq_lens, window: int = 1024, rows=None,
                    nthreads: int | None = None, lib=None) -> np.ndarray:
    """Reference slidingDecodeGQA over a cache capped at R positions, in fp64.

    k, v [B,R,16,256]: position s in slot s % R (the retrofit page's per-layer
    caches capped at the window, read as a ring); window <= R; seq_lens may
    exceed R.  Otherwise as gqa_decode.
    """
    KV, D, _ = VARIANTS["sliding"]
    lib = lib or load()
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share a dtype")
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = q.shape[0]
    if q.shape != (B, HEADS, D) or seq_lens.shape != (B,):
        raise ValueError("q must be [B,32,D] and seq_lens [B]")
    if k.ndim != 4 or k.shape[0] != B or k.shape[2:] != (KV, D) or v.shape != k.shape:
        raise ValueError("ring k/v must be [B,R,16,256]")
    ring = k.shape[1]
    if rows is None:
        rows_arr, n_rows = None, B * HEADS
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        n_rows = rows_arr.shape[0]
    out = np.zeros((n_rows, D), dtype=np.float64)
    nthreads = nthreads or min(os.cpu_count() or 1, 16)
    rc = lib.oracle_gqa_decode_ring(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), B, ring, KV,
                                    D, window, _ptr(rows_arr), n_rows, _ptr(out), nthreads)
    if rc != 0:
        raise ValueError(f"oracle error {rc}: {_ERRORS.get(rc, '?')}")
    return out.reshape(B, HEADS, D) if rows is None else out


def gqa_append_rows(variant, q_raw, k_raw, v_raw, w_q, w_k, seq_lens, lib=None):
    """Norms + RoPE of the new token of every sequence (attn.qk_norm, attn.v_norm,
    attn.rope of the Model Spec page), in fp64.

    q_raw [B,32,D], k_raw/v_raw [B,KV,D] (v_raw ignored for "global": values =
    keys), w_q/w_k [D]; float32 arrays or uint16 bf16 bits.  Returns
    (q_out [B,32,D], k_row [B,KV,D], v_row [B,KV,D], pos [B]) with pos =
    seq_lens - 1 (-1 and zero rows where seq_lens < 1).
    """
    KV, D, _ = VARIANTS[variant]
    lib = lib or load()
    q_raw, k_raw = np.ascontiguousarray(q_raw), np.ascontiguousarray(k_raw)
    w_q, w_k = np.ascontiguousarray(w_q), np.ascontiguousarray(w_k)
    dt = _dtype_code(q_raw)
    v_raw = None if v_raw is None else np.ascontiguousarray(v_raw)
    for a in (k_raw, w_q, w_k) + ((v_raw,) if v_raw is not None else ()):
        if _dtype_code(a) != dt:
            raise TypeError("inputs must share a dtype")
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = q_raw.shape[0]
    if q_raw.shape != (B, HEADS, D) or k_raw.shape != (B, KV, D) or w_q.shape != (D,) or \
            w_k.shape != (D,) or seq_lens.shape != (B,):
        raise ValueError("bad shapes")
    q_out = np.zeros((B, HEADS, D))
    k_row = np.zeros((B, KV, D))
    v_row = np.zeros((B, KV, D))
    pos = np.zeros(B, dtype=np.int32)
    rc = lib.oracle_gqa_append_rows(dt, _ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(w_q),
                                    _ptr(w_k), _ptr(seq_lens), B, KV, D, _ptr(q_out),
                                    _ptr(k_row), _ptr(v_row), _ptr(pos))
    if rc != 0:
        raise ValueError(f"oracle error {rc}: {_ERRORS.get(rc, '?')}")
    return q_out, k_row, v_row, pos


def gqa_decode_k_from_v(q, v, w_k, seq_lens, block_table=None, num_pages=None, rows=None,
                        nthreads: int | None = None, lib=None) -> np.ndarray:
    """decodeGQA over a values-only cache: the key of position s is
    rope(w_k * v_s, s) (values = keys on the global layers), in fp64.

    q [B,32,512]; v [B,S,4,512] or [num_pages,16,4,512] with block_table; w_k [512].
    """
    lib = lib or load()
    q, v, w_k = (np.ascontiguousarray(a) for a in (q, v, w_k))
    dt = _dtype_code(q)
    if _dtype_code(v) != dt or _dtype_code(w_k) != dt:
        raise TypeError("q, v, w_k must share a dtype")
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = q.shape[0]
    if q.shape != (B, HEADS, 512) or w_k.shape != (512,) or seq_lens.shape != (B,):
        raise ValueError("bad shapes")
    if block_table is None:
        if v.ndim != 4 or v.shape[0] != B or v.shape[2:] != (4, 512):
            raise ValueError("v must be [B,S,4,512]")
        cap, max_pages, n_pages, bt = v.shape[1], 0, 0, None
    else:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        if v.ndim != 4 or v.shape[1:] != (PAGE, 4, 512):
            raise ValueError("paged v must be [num_pages,16,4,512]")
        max_pages = bt.shape[1]
        n_pages = v.shape[0] if num_pages is None else num_pages
        cap = max_pages * PAGE
    if rows is None:
        rows_arr, n_rows = None, B * HEADS
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        n_rows = rows_arr.shape[0]
    out = np.zeros((n_rows, 512), dtype=np.float64)
    nthreads = nthreads or min(os.cpu_count() or 1, 16)
    rc = lib.oracle_gqa_decode_k_from_v(dt, _ptr(q), _ptr(v), _ptr(w_k), _ptr(seq_lens), _ptr(bt),
                                        B, cap, max_pages, n_pages, _ptr(rows_arr), n_rows,
                                        _ptr(out), nthreads)
    if rc != 0:
        raise ValueError(f"oracle error {rc}: {_ERRORS.get(rc, '?')}")
    return out.reshape(B, HEADS, 512) if rows is None else out


def gqa_prefill(variant, q, k, v, cu_q, seq_lens, block_table=None, num_pages=None, rows=None,
                nthreads: int | None = None, window: int | None = None, lib=None) -> np.ndarray:
    """Reference prefill attention in fp64: query row n of sequence b (cu_q[b] <= n
    < cu_q[b+1]) sits at position seq_lens[b] - T_b + (n - cu_q[b]) and attends
    to the keys at positions p - W < s <= p (sliding) or s <= p (global).

    q [N,32,D]; cu_q [B+1] int32; k, v and block_table as gqa_decode.  rows:
    optional list of (query row, head) pairs.  Returns [N,32,D] or [len(rows), D].
    """
    KV, D, W = VARIANTS[variant] if isinstance(variant, str) else variant
    if window is not None:
        W = window
    lib = lib or load()
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share a dtype")
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int32)
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = seq_lens.shape[0]
    N = q.shape[0]
    if q.shape != (N, HEADS, D) or cu_q.shape != (B + 1,):
        raise ValueError("q must be [N,32,D] and cu_q [B+1]")
    if block_table is None:
        if k.ndim != 4 or k.shape[0] != B or k.shape[2:] != (KV, D) or v.shape != k.shape:
            raise ValueError("contiguous k/v must be [B,S,KV,D]")
        cap, max_pages, n_pages, bt = k.shape[1], 0, 0, None
    else:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        if bt.ndim != 2 or bt.shape[0] != B:
            raise ValueError("block_table must be [B,max_pages]")
        if k.ndim != 4 or k.shape[1:] != (PAGE, KV, D) or v.shape != k.shape:
            raise ValueError("paged k/v must be [num_pages,16,KV,D]")
        max_pages = bt.shape[1]
        n_pages = k.shape[0] if num_pages is None else num_pages
        cap = max_pages * PAGE
    if rows is None:
        rows_arr, n_rows = None, N * HEADS
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        n_rows = rows_arr.shape[0]
    out = np.zeros((n_rows, D), dtype=np.float64)
    nthreads = nthreads or min(os.cpu_count() or 1, 16)
    rc = lib.oracle_gqa_prefill(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(cu_q), _ptr(seq_lens),
                                _ptr(bt), B, N, cap, max_pages, n_pages, KV, D, W, _ptr(rows_arr),
                                n_rows, _ptr(out), nthreads)
    if rc != 0:
        raise ValueError(f"oracle error {rc}: {_ERRORS.get(rc, '?')}")
    return out.reshape(N, HEADS, D) if rows is None else out
