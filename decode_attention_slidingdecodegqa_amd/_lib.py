"""ctypes marshalling for libgqadecode.so (argument plumbing only)."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_PKG, "libgqadecode.so")

GQA_F32, GQA_BF16 = 0, 1
GQA_SLIDING, GQA_GLOBAL = 0, 1
HEADS, PAGE = 32, 16
_VARIANT = {"sliding": GQA_SLIDING, "global": GQA_GLOBAL}

EXPORTED_SYMBOLS = (
    "gqa_decode_sliding", "gqa_decode_global", "gqa_decode_sliding_paged",
    "gqa_decode_global_paged", "gqa_decode_workspace_bytes", "gqa_decode_plan",
    "gqa_decode_constants", "gqa_status_str", "gqa_profile_begin", "gqa_profile_read",
    "gqa_hbm_read_probe", "gqa_hbm_copy_probe", "gqa_decode_sliding_window",
    "gqa_decode_sliding_window_paged", "gqa_decode_sliding_window_workspace_bytes",
    "gqa_decode_sliding_window_plan", "gqa_append_sliding", "gqa_append_sliding_paged",
    "gqa_append_global", "gqa_append_global_paged", "gqa_decode_global_k_eq_v",
    "gqa_decode_global_k_eq_v_paged", "gqa_append_global_k_eq_v",
    "gqa_append_global_k_eq_v_paged", "gqa_prefill_sliding", "gqa_prefill_global",
    "gqa_prefill_sliding_paged", "gqa_prefill_global_paged", "gqa_decode_sliding_ring",
    "gqa_decode_sliding_ring_workspace_bytes", "gqa_append_sliding_ring",
    "gqa_prefill_sliding_window", "gqa_prefill_sliding_window_paged",
    "gqa_decode_global_paged_noalloc", "gqa_decode_force_mode",
)


class GqaError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: status {status} ({gqa_status_str(status)})")
        self.status = status


_lib = None


def library():
    """Load libgqadecode.so (built in-tree by build.py); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise RuntimeError(f"{LIBRARY_PATH} is missing: build it with "
                           "`python -m decode_attention_slidingdecodegqa_amd.build`")
    lib = ctypes.CDLL(LIBRARY_PATH)
    p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    contig = [p, p, p, p, p, i32, i32, i32, p, sz, p]
    paged = [p, p, p, p, i32, p, p, i32, i32, i32, p, sz, p]
    for name, args in (("gqa_decode_sliding", contig), ("gqa_decode_global", contig),
                       ("gqa_decode_sliding_paged", paged), ("gqa_decode_global_paged", paged)):
        f = getattr(lib, name)
        f.argtypes, f.restype = args, ctypes.c_int
    lib.gqa_decode_force_mode.argtypes = [i32]
    lib.gqa_decode_force_mode.restype = ctypes.c_int
    lib.gqa_decode_global_paged_noalloc.argtypes = [p, p, p, p, i32, p, p, i32, i32, i32, p]
    lib.gqa_decode_global_paged_noalloc.restype = ctypes.c_int
    lib.gqa_decode_sliding_window.argtypes = [p, p, p, p, p, i32, i32, i32, i32, p, sz, p]
    lib.gqa_decode_sliding_window.restype = ctypes.c_int
    lib.gqa_decode_sliding_window_paged.argtypes = [p, p, p, p, i32, p, p, i32, i32, i32, i32, p,
                                                    sz, p]
    lib.gqa_decode_sliding_window_paged.restype = ctypes.c_int
    lib.gqa_decode_sliding_window_workspace_bytes.argtypes = [i32, i32, i32]
    lib.gqa_decode_sliding_window_workspace_bytes.restype = sz
    lib.gqa_decode_sliding_window_plan.argtypes = [i32, i32, i32] + [ctypes.POINTER(i32)] * 3
    lib.gqa_decode_sliding_window_plan.restype = ctypes.c_int
    lib.gqa_decode_sliding_ring.argtypes = [p, p, p, p, p, i32, i32, i32, i32, p, sz, p]
    lib.gqa_decode_sliding_ring.restype = ctypes.c_int
    lib.gqa_decode_sliding_ring_workspace_bytes.argtypes = [i32, i32, i32]
    lib.gqa_decode_sliding_ring_workspace_bytes.restype = sz
    lib.gqa_append_sliding_ring.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, p]
    lib.gqa_append_sliding_ring.restype = ctypes.c_int
    lib.gqa_append_sliding.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, p]
    lib.gqa_append_sliding_paged.argtypes = [p, p, p, p, p, p, i32, p, p, p, p, i32, i32, i32, p]
    lib.gqa_append_global.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, p]
    lib.gqa_append_global_paged.argtypes = [p, p, p, p, p, i32, p, p, p, p, i32, i32, i32, p]
    lib.gqa_decode_global_k_eq_v.argtypes = [p, p, p, p, p, i32, i32, i32, p, sz, p]
    lib.gqa_decode_global_k_eq_v_paged.argtypes = [p, p, p, p, i32, p, p, i32, i32, i32, p, sz,
                                                   p]
    lib.gqa_append_global_k_eq_v.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, p]
    lib.gqa_append_global_k_eq_v_paged.argtypes = [p, p, p, p, p, i32, p, p, p, i32, i32, i32, p]
    for name in ("gqa_prefill_sliding", "gqa_prefill_global"):
        getattr(lib, name).argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, p]
        getattr(lib, name).restype = ctypes.c_int
    for name in ("gqa_prefill_sliding_paged", "gqa_prefill_global_paged"):
        getattr(lib, name).argtypes = [p, p, p, p, i32, p, p, p, i32, i32, i32, i32, p]
        getattr(lib, name).restype = ctypes.c_int
    lib.gqa_prefill_sliding_window.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, p]
    lib.gqa_prefill_sliding_window.restype = ctypes.c_int
    lib.gqa_prefill_sliding_window_paged.argtypes = [p, p, p, p, i32, p, p, p, i32, i32, i32, i32,
                                                     i32, p]
    lib.gqa_prefill_sliding_window_paged.restype = ctypes.c_int
    for name in ("gqa_append_sliding", "gqa_append_sliding_paged", "gqa_append_global",
                 "gqa_append_global_paged", "gqa_decode_global_k_eq_v",
                 "gqa_decode_global_k_eq_v_paged", "gqa_append_global_k_eq_v",
                 "gqa_append_global_k_eq_v_paged"):
        getattr(lib, name).restype = ctypes.c_int
    lib.gqa_decode_workspace_bytes.argtypes = [i32, i32, i32]
    lib.gqa_decode_workspace_bytes.restype = sz
    lib.gqa_decode_plan.argtypes = [i32, i32, i32] + [ctypes.POINTER(i32)] * 3
    lib.gqa_decode_plan.restype = ctypes.c_int
    lib.gqa_decode_constants.argtypes = [i32] + [ctypes.POINTER(i32)] * 5
    lib.gqa_decode_constants.restype = ctypes.c_int
    lib.gqa_status_str.argtypes = [i32]
    lib.gqa_status_str.restype = ctypes.c_char_p
    lib.gqa_profile_begin.argtypes = [i32]
    lib.gqa_profile_begin.restype = ctypes.c_int
    lib.gqa_profile_read.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double), i32]
    lib.gqa_profile_read.restype = ctypes.c_int
    lib.gqa_hbm_read_probe.argtypes = [p, sz, p, p]
    lib.gqa_hbm_read_probe.restype = ctypes.c_int
    lib.gqa_hbm_copy_probe.argtypes = [p, p, sz, p]
    lib.gqa_hbm_copy_probe.restype = ctypes.c_int
    _lib = lib
    return lib


def gqa_status_str(status: int) -> str:
    return library().gqa_status_str(int(status)).decode()


def _variant(v) -> int:
    return _VARIANT[v] if isinstance(v, str) else int(v)


def constants(variant) -> dict:
    vals = [ctypes.c_int32() for _ in range(5)]
    rc = library().gqa_decode_constants(_variant(variant), *[ctypes.byref(x) for x in vals])
    if rc:
        raise GqaError("gqa_decode_constants", rc)
    return dict(zip(("heads", "kv_heads", "head_dim", "window", "page"), (x.value for x in vals)))


def gqa_decode_workspace_bytes(variant, B: int, capacity: int, window: int | None = None) -> int:
    """Workspace bytes; `window` (sliding only) selects the windowed calls' size."""
    if window is not None:
        if _variant(variant) != GQA_SLIDING:
            raise ValueError("a runtime window applies to the sliding variant only")
        return int(library().gqa_decode_sliding_window_workspace_bytes(int(B), int(capacity),
                                                                       int(window)))
    return int(library().gqa_decode_workspace_bytes(_variant(variant), int(B), int(capacity)))


GQA_MODE_UNIT, GQA_MODE_STREAM, GQA_MODE_GROUP = 0, 1, 2
_MODE_NAMES = {GQA_MODE_UNIT: "unit", GQA_MODE_STREAM: "stream", GQA_MODE_GROUP: "group"}


def gqa_decode_plan(variant, B: int, capacity: int, window: int | None = None) -> dict:
    """Launch plan: {'mode': 'unit'|'stream'|'group', 'waves': W, 'slots': workspace slots}."""
    mode, n, t = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    if window is not None:
        if _variant(variant) != GQA_SLIDING:
            raise ValueError("a runtime window applies to the sliding variant only")
        rc = library().gqa_decode_sliding_window_plan(int(B), int(capacity), int(window),
                                                      ctypes.byref(mode), ctypes.byref(n),
                                                      ctypes.byref(t))
    else:
        rc = library().gqa_decode_plan(_variant(variant), int(B), int(capacity),
                                       ctypes.byref(mode), ctypes.byref(n), ctypes.byref(t))
    if rc:
        raise GqaError("gqa_decode_plan", rc)
    return {"mode": _MODE_NAMES[mode.value], "waves": n.value, "slots": t.value}


def force_mode(mode: str | None) -> None:
    """Make later plans and calls take launch mode 'unit', 'stream' or 'group'
    whatever the planner would choose (None: the planner's choice again).
    Process-wide; for measurement and tests."""
    code = -1 if mode is None else {v: k for k, v in _MODE_NAMES.items()}[mode]
    rc = library().gqa_decode_force_mode(code)
    if rc:
        raise GqaError("gqa_decode_force_mode", rc)


def profile_begin(capacity: int) -> None:
    rc = library().gqa_profile_begin(int(capacity))
    if rc:
        raise GqaError("gqa_profile_begin", rc)


def profile_read() -> dict:
    """{(variant, kernel): (launches, total_ms)} for variant in sliding / global /
    global_k_eq_v (global layers over a values-only cache) and kernel in
    main/combine/append."""
    n = 11
    counts = (ctypes.c_int32 * n)()
    ms = (ctypes.c_double * n)()
    rc = library().gqa_profile_read(counts, ms, n)
    if rc:
        raise GqaError("gqa_profile_read", rc)
    out = {}
    for vi, vname in enumerate(("sliding", "global")):
        for kind, kname in ((2 * vi, "main"), (2 * vi + 1, "combine"), (4 + vi, "append")):
            out[(vname, kname)] = (counts[kind], ms[kind])
    for kind, kname in ((6, "main"), (7, "combine"), (8, "append")):
        out[("global_k_eq_v", kname)] = (counts[kind], ms[kind])
    for vi, vname in enumerate(("sliding", "global")):
        out[(vname, "prefill")] = (counts[9 + vi], ms[9 + vi])
    return out


def hbm_read_probe(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Plain read stream over src (measurement only)."""
    nbytes = src.numel() * src.element_size()
    rc = library().gqa_hbm_read_probe(_dev(src, "src"), nbytes, _dev(sink, "sink"),
                                      _stream(stream, src.device))
    if rc:
        raise GqaError("gqa_hbm_read_probe", rc)


def hbm_copy_probe(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """Plain copy src -> dst (measurement only)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    rc = library().gqa_hbm_copy_probe(_dev(src, "src"), _dev(dst, "dst"), nbytes,
                                      _stream(stream, src.device))
    if rc:
        raise GqaError("gqa_hbm_copy_probe", rc)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GQA_F32
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _for_stream(t: torch.Tensor, stream) -> torch.Tensor:
    """A tensor this binding allocated, used by a launch on `stream`.

    torch's caching allocator ties a block to the stream that was current when
    it was allocated and may hand it out again as soon as the tensor is freed,
    ordered only against that stream.  When the launch runs on another stream,
    record_stream makes the free wait for the work queued on `stream` up to
    the moment of the free, so the caller keeps the tensor alive until the
    launch has been queued (the workspace is then freed when the call
    returns)."""
    if stream is not None:
        t.record_stream(stream)
    return t


def _prepare(variant, q, seq_lens, o, workspace, capacity, window=None, stream=None):
    B = q.shape[0]
    D = 256 if variant == GQA_SLIDING else 512
    if q.dim() != 3 or q.shape[1:] != (HEADS, D):
        raise ValueError(f"q must be [B,32,{D}]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if o is None:
        o = _for_stream(torch.empty_like(q), stream)
    elif o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("o must match q in shape and dtype")
    need = gqa_decode_workspace_bytes(variant, B, capacity, window)
    if workspace is None and need > 0:
        workspace = _for_stream(torch.empty(need, dtype=torch.uint8, device=q.device), stream)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    # the workspace tensor goes back to the caller, which holds it across the
    # launch (see _for_stream)
    return B, o, (workspace, ws_ptr), ws_bytes


def _stream(stream, device):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _contiguous_call(name, variant, q, k, v, seq_lens, o, workspace, stream, window=None):
    KV = 16 if variant == GQA_SLIDING else 4
    D = 256 if variant == GQA_SLIDING else 512
    if k.dim() != 4 or k.shape[0] != q.shape[0] or k.shape[2:] != (KV, D) or v.shape != k.shape:
        raise ValueError(f"k/v must be [B,S_max,{KV},{D}]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    S_max = k.shape[1]
    B, o, (ws_keep, ws), ws_bytes = _prepare(variant, q, seq_lens, o, workspace, S_max, window, stream)
    fn = getattr(library(), name)
    shape = (B, S_max) if window is None else (B, S_max, int(window))
    rc = fn(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(seq_lens, "seq_lens"), _dev(o, "o"),
            *shape, _dtype_code(q), ws, ws_bytes, _stream(stream, q.device))
    del ws_keep  # held until the launch was queued (see _for_stream)
    if rc:
        raise GqaError(name, rc)
    return o


def _paged_call(name, variant, q, k_pool, v_pool, block_table, seq_lens, o, workspace, stream,
                window=None):
    KV = 16 if variant == GQA_SLIDING else 4
    D = 256 if variant == GQA_SLIDING else 512
    if k_pool.dim() != 4 or k_pool.shape[1:] != (PAGE, KV, D) or v_pool.shape != k_pool.shape:
        raise ValueError(f"k_pool/v_pool must be [num_pages,16,{KV},{D}]")
    if not (q.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("q, k_pool, v_pool must share a dtype")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
            block_table.shape[0] != q.shape[0]:
        raise ValueError("block_table must be int32 [B,max_pages]")
    max_pages = block_table.shape[1]
    num_pages = k_pool.shape[0]
    B, o, (ws_keep, ws), ws_bytes = _prepare(variant, q, seq_lens, o, workspace, max_pages * PAGE, window,
                                  stream)
    fn = getattr(library(), name)
    shape = (B, num_pages) if window is None else (B, num_pages, int(window))
    rc = fn(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
            _dev(block_table, "block_table"), max_pages, _dev(seq_lens, "seq_lens"), _dev(o, "o"),
            *shape, _dtype_code(q), ws, ws_bytes, _stream(stream, q.device))
    del ws_keep  # held until the launch was queued (see _for_stream)
    if rc:
        raise GqaError(name, rc)
    return o


def gqa_decode_sliding(q, k, v, seq_lens, o=None, workspace=None, stream=None):
    """slidingDecodeGQA on a contiguous cache k, v [B,S_max,16,256]."""
    return _contiguous_call("gqa_decode_sliding", GQA_SLIDING, q, k, v, seq_lens, o, workspace,
                            stream)


def gqa_decode_global(q, k, v, seq_lens, o=None, workspace=None, stream=None):
    """decodeGQA on a contiguous cache k, v [B,S_max,4,512]."""
    return _contiguous_call("gqa_decode_global", GQA_GLOBAL, q, k, v, seq_lens, o, workspace,
                            stream)


def gqa_decode_sliding_paged(q, k_pool, v_pool, block_table, seq_lens, o=None, workspace=None,
                             stream=None):
    """slidingDecodeGQA on a paged cache k_pool, v_pool [num_pages,16,16,256]."""
    return _paged_call("gqa_decode_sliding_paged", GQA_SLIDING, q, k_pool, v_pool, block_table,
                       seq_lens, o, workspace, stream)


def gqa_decode_global_paged(q, k_pool, v_pool, block_table, seq_lens, o=None, workspace=None,
                            stream=None):
    """decodeGQA on a paged cache k_pool, v_pool [num_pages,16,4,512]."""
    return _paged_call("gqa_decode_global_paged", GQA_GLOBAL, q, k_pool, v_pool, block_table,
                       seq_lens, o, workspace, stream)


def gqa_decode_global_paged_noalloc(q, k_pool, v_pool, block_table, seq_lens, o, stream=None):
    """decodeGQA on a paged cache through the entry point that allocates
    nothing: its split-S partials use the library's own device array (shared
    by every call on the device; calls that can overlap must be ordered by the
    caller).  `o` is required: this call allocates no tensor either."""
    if not isinstance(o, torch.Tensor) or o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("o must be given and match q in shape and dtype")
    if q.dim() != 3 or q.shape[1:] != (HEADS, 512):
        raise ValueError("q must be [B,32,512]")
    if k_pool.dim() != 4 or k_pool.shape[1:] != (PAGE, 4, 512) or v_pool.shape != k_pool.shape:
        raise ValueError("k_pool/v_pool must be [num_pages,16,4,512]")
    if not (q.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("q, k_pool, v_pool must share a dtype")
    B = q.shape[0]
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B,max_pages]")
    name = "gqa_decode_global_paged_noalloc"
    rc = getattr(library(), name)(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                  _dev(block_table, "block_table"), block_table.shape[1],
                                  _dev(seq_lens, "seq_lens"), _dev(o, "o"), B, k_pool.shape[0],
                                  _dtype_code(q), _stream(stream, q.device))
    if rc:
        raise GqaError(name, rc)
    return o


def gqa_decode_sliding_window(q, k, v, seq_lens, window, o=None, workspace=None, stream=None):
    """slidingDecodeGQA geometry with a runtime window on a contiguous cache."""
    return _contiguous_call("gqa_decode_sliding_window", GQA_SLIDING, q, k, v, seq_lens, o,
                            workspace, stream, window=window)


def gqa_decode_sliding_window_paged(q, k_pool, v_pool, block_table, seq_lens, window, o=None,
                                    workspace=None, stream=None):
    """slidingDecodeGQA geometry with a runtime window on a paged cache."""
    return _paged_call("gqa_decode_sliding_window_paged", GQA_SLIDING, q, k_pool, v_pool,
                       block_table, seq_lens, o, workspace, stream, window=window)


def _append_call(variant, q_raw, k_raw, v_raw, w_q, w_k, seq_lens, k_cache, v_cache,
                 block_table, q_out, stream, ring=False):
    KV = 16 if variant == GQA_SLIDING else 4
    D = 256 if variant == GQA_SLIDING else 512
    B = q_raw.shape[0]
    if q_raw.shape != (B, HEADS, D) or k_raw.shape != (B, KV, D):
        raise ValueError(f"q_raw must be [B,32,{D}] and k_raw [B,{KV},{D}]")
    if variant == GQA_SLIDING and (v_raw is None or v_raw.shape != k_raw.shape):
        raise ValueError("v_raw must be [B,16,256]")
    if w_q.shape != (D,) or w_k.shape != (D,):
        raise ValueError(f"w_q and w_k must be [{D}]")
    dts = {t.dtype for t in (q_raw, k_raw, w_q, w_k, k_cache, v_cache)
           if t is not None}
    if v_raw is not None and variant == GQA_SLIDING:
        dts.add(v_raw.dtype)
    if len(dts) != 1:
        raise TypeError("inputs, weights and caches must share a dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if q_out is None:
        q_out = _for_stream(torch.empty_like(q_raw), stream)
    lib = library()
    st = _stream(stream, q_raw.device)
    ptrs = [_dev(q_raw, "q_raw"), _dev(k_raw, "k_raw")]
    if variant == GQA_SLIDING:
        ptrs.append(_dev(v_raw, "v_raw"))
    ptrs += [_dev(w_q, "w_q"), _dev(w_k, "w_k")]
    dt = _dtype_code(q_raw)
    name = "gqa_append_" + ("sliding" if variant == GQA_SLIDING else "global")
    if ring:
        name += "_ring"
    if block_table is None:
        if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[2:] != (KV, D) or \
                v_cache.shape != k_cache.shape:
            raise ValueError(f"k_cache/v_cache must be [B,S_max,{KV},{D}]")
        rc = getattr(lib, name)(*ptrs, _dev(seq_lens, "seq_lens"), _dev(q_out, "q_out"),
                                _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), B,
                                k_cache.shape[1], dt, st)
    else:
        name += "_paged"
        if k_cache.dim() != 4 or k_cache.shape[1:] != (PAGE, KV, D) or \
                v_cache.shape != k_cache.shape:
            raise ValueError(f"k_pool/v_pool must be [num_pages,16,{KV},{D}]")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
                block_table.shape[0] != B:
            raise ValueError("block_table must be int32 [B,max_pages]")
        rc = getattr(lib, name)(*ptrs, _dev(block_table, "block_table"), block_table.shape[1],
                                _dev(seq_lens, "seq_lens"), _dev(q_out, "q_out"),
                                _dev(k_cache, "k_pool"), _dev(v_cache, "v_pool"), B,
                                k_cache.shape[0], dt, st)
    if rc:
        raise GqaError(name, rc)
    return q_out


def gqa_decode_sliding_ring_workspace_bytes(B: int, ring: int, window: int = 1024) -> int:
    """Workspace bytes of gqa_decode_sliding_ring (0: none needed, or bad arguments)."""
    return int(library().gqa_decode_sliding_ring_workspace_bytes(int(B), int(ring), int(window)))


def gqa_decode_sliding_ring(q, k, v, seq_lens, window: int = 1024, o=None, workspace=None,
                            stream=None):
    """slidingDecodeGQA over a cache capped at R positions: k, v [B,R,16,256] with
    position s in slot s % R (R a multiple of 16, window <= R); seq_lens may
    exceed R."""
    if k.dim() != 4 or k.shape[0] != q.shape[0] or k.shape[2:] != (16, 256) or \
            v.shape != k.shape:
        raise ValueError("k/v must be [B,R,16,256]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    ring = k.shape[1]
    B = q.shape[0]
    need = gqa_decode_sliding_ring_workspace_bytes(B, ring, window)
    if workspace is None and need > 0:
        workspace = _for_stream(torch.empty(need, dtype=torch.uint8, device=q.device), stream)
    B, o, (ws_keep, ws), ws_bytes = _prepare(GQA_SLIDING, q, seq_lens, o, workspace, ring, window, stream)
    rc = library().gqa_decode_sliding_ring(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                           _dev(seq_lens, "seq_lens"), _dev(o, "o"), B, ring,
                                           int(window), _dtype_code(q), ws, ws_bytes,
                                           _stream(stream, q.device))
    del ws_keep  # held until the launch was queued (see _for_stream)
    if rc:
        raise GqaError("gqa_decode_sliding_ring", rc)
    return o


def gqa_append_sliding_ring(q_raw, k_raw, v_raw, w_q, w_k, seq_lens, k_cache, v_cache,
                            q_out=None, stream=None):
    """The sliding append into a cache capped at R positions (k_cache, v_cache
    [B,R,16,256]): the new token's rows go to slot (seq_lens-1) % R."""
    return _append_call(GQA_SLIDING, q_raw, k_raw, v_raw, w_q, w_k, seq_lens, k_cache, v_cache,
                        None, q_out, stream, ring=True)


def gqa_append_sliding(q_raw, k_raw, v_raw, w_q, w_k, seq_lens, k_cache, v_cache,
                       block_table=None, q_out=None, stream=None):
    """Norms + RoPE of the new token (position seq_lens-1) of the sliding layers;
    writes q_out (returned) and the token's K/V rows into the cache (contiguous,
    or paged when block_table is given)."""
    return _append_call(GQA_SLIDING, q_raw, k_raw, v_raw, w_q, w_k, seq_lens, k_cache, v_cache,
                        block_table, q_out, stream)


def gqa_append_global(q_raw, k_raw, w_q, w_k, seq_lens, k_cache, v_cache, block_table=None,
                      q_out=None, stream=None):
    """As gqa_append_sliding for the global layers (values = keys: no v_raw)."""
    return _append_call(GQA_GLOBAL, q_raw, k_raw, None, w_q, w_k, seq_lens, k_cache, v_cache,
                        block_table, q_out, stream)


def _check_w_k(w_k, q):
    if w_k.shape != (512,) or w_k.dtype != q.dtype:
        raise ValueError("w_k must be [512] in the dtype of q")


def gqa_decode_global_k_eq_v(q, v, w_k, seq_lens, o=None, workspace=None, stream=None):
    """decodeGQA over a values-only cache v [B,S_max,4,512]: the key of position
    s is rope(w_k * v_s, s), rebuilt in the kernel (values = keys)."""
    if v.dim() != 4 or v.shape[0] != q.shape[0] or v.shape[2:] != (4, 512):
        raise ValueError("v must be [B,S_max,4,512]")
    if q.dtype != v.dtype:
        raise TypeError("q and v must share a dtype")
    _check_w_k(w_k, q)
    S_max = v.shape[1]
    B, o, (ws_keep, ws), ws_bytes = _prepare(GQA_GLOBAL, q, seq_lens, o, workspace, S_max, stream=stream)
    name = "gqa_decode_global_k_eq_v"
    rc = getattr(library(), name)(_dev(q, "q"), _dev(v, "v"), _dev(w_k, "w_k"),
                                  _dev(seq_lens, "seq_lens"), _dev(o, "o"), B, S_max,
                                  _dtype_code(q), ws, ws_bytes, _stream(stream, q.device))
    del ws_keep  # held until the launch was queued (see _for_stream)
    if rc:
        raise GqaError(name, rc)
    return o


def gqa_decode_global_k_eq_v_paged(q, v_pool, w_k, block_table, seq_lens, o=None,
                                   workspace=None, stream=None):
    """As gqa_decode_global_k_eq_v on a paged values-only pool [num_pages,16,4,512]."""
    if v_pool.dim() != 4 or v_pool.shape[1:] != (PAGE, 4, 512):
        raise ValueError("v_pool must be [num_pages,16,4,512]")
    if q.dtype != v_pool.dtype:
        raise TypeError("q and v_pool must share a dtype")
    _check_w_k(w_k, q)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
            block_table.shape[0] != q.shape[0]:
        raise ValueError("block_table must be int32 [B,max_pages]")
    max_pages = block_table.shape[1]
    B, o, (ws_keep, ws), ws_bytes = _prepare(GQA_GLOBAL, q, seq_lens, o, workspace, max_pages * PAGE,
                                  stream=stream)
    name = "gqa_decode_global_k_eq_v_paged"
    rc = getattr(library(), name)(_dev(q, "q"), _dev(v_pool, "v_pool"), _dev(w_k, "w_k"),
                                  _dev(block_table, "block_table"), max_pages,
                                  _dev(seq_lens, "seq_lens"), _dev(o, "o"), B, v_pool.shape[0],
                                  _dtype_code(q), ws, ws_bytes, _stream(stream, q.device))
    del ws_keep  # held until the launch was queued (see _for_stream)
    if rc:
        raise GqaError(name, rc)
    return o


def gqa_append_global_k_eq_v(q_raw, k_raw, w_q, w_k, seq_lens, v_cache, block_table=None,
                             q_out=None, stream=None):
    """Append of the global layers to a values-only cache: writes q_out (returned)
    and the unit-RMS value row of the new token; no key row is stored."""
    B = q_raw.shape[0]
    if q_raw.shape != (B, HEADS, 512) or k_raw.shape != (B, 4, 512):
        raise ValueError("q_raw must be [B,32,512] and k_raw [B,4,512]")
    if w_q.shape != (512,) or w_k.shape != (512,):
        raise ValueError("w_q and w_k must be [512]")
    if len({t.dtype for t in (q_raw, k_raw, w_q, w_k, v_cache)}) != 1:
        raise TypeError("inputs, weights and cache must share a dtype")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if q_out is None:
        q_out = _for_stream(torch.empty_like(q_raw), stream)
    lib = library()
    st = _stream(stream, q_raw.device)
    ptrs = [_dev(q_raw, "q_raw"), _dev(k_raw, "k_raw"), _dev(w_q, "w_q"), _dev(w_k, "w_k")]
    dt = _dtype_code(q_raw)
    if block_table is None:
        name = "gqa_append_global_k_eq_v"
        if v_cache.dim() != 4 or v_cache.shape[0] != B or v_cache.shape[2:] != (4, 512):
            raise ValueError("v_cache must be [B,S_max,4,512]")
        rc = getattr(lib, name)(*ptrs, _dev(seq_lens, "seq_lens"), _dev(q_out, "q_out"),
                                _dev(v_cache, "v_cache"), B, v_cache.shape[1], dt, st)
    else:
        name = "gqa_append_global_k_eq_v_paged"
        if v_cache.dim() != 4 or v_cache.shape[1:] != (PAGE, 4, 512):
            raise ValueError("v_pool must be [num_pages,16,4,512]")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
                block_table.shape[0] != B:
            raise ValueError("block_table must be int32 [B,max_pages]")
        rc = getattr(lib, name)(*ptrs, _dev(block_table, "block_table"), block_table.shape[1],
                                _dev(seq_lens, "seq_lens"), _dev(q_out, "q_out"),
                                _dev(v_cache, "v_pool"), B, v_cache.shape[0], dt, st)
    if rc:
        raise GqaError(name, rc)
    return q_out


def _prefill_call(variant, q, k, v, cu_q, seq_lens, block_table, o, stream, window=None):
    KV = 16 if variant == GQA_SLIDING else 4
    D = 256 if variant == GQA_SLIDING else 512
    if q.dim() != 3 or q.shape[1:] != (HEADS, D):
        raise ValueError(f"q must be [N,32,{D}]")
    B = seq_lens.shape[0]
    if seq_lens.dtype != torch.int32 or seq_lens.dim() != 1:
        raise ValueError("seq_lens must be int32 [B]")
    if cu_q.dtype != torch.int32 or cu_q.shape != (B + 1,):
        raise ValueError("cu_q must be int32 [B+1]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if o is None:
        o = _for_stream(torch.empty_like(q), stream)
    elif o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("o must match q in shape and dtype")
    N = q.shape[0]
    lib = library()
    st = _stream(stream, q.device)
    kind = "sliding" if variant == GQA_SLIDING else "global"
    if block_table is None:
        if k.dim() != 4 or k.shape[0] != B or k.shape[2:] != (KV, D) or v.shape != k.shape:
            raise ValueError(f"k/v must be [B,S_max,{KV},{D}]")
        args = [_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(cu_q, "cu_q"),
                _dev(seq_lens, "seq_lens"), _dev(o, "o"), B, N, k.shape[1]]
        if window is None:
            name = f"gqa_prefill_{kind}"
            rc = getattr(lib, name)(*args, _dtype_code(q), st)
        else:
            name = "gqa_prefill_sliding_window"
            rc = lib.gqa_prefill_sliding_window(*args, int(window), _dtype_code(q), st)
    else:
        if k.dim() != 4 or k.shape[1:] != (PAGE, KV, D) or v.shape != k.shape:
            raise ValueError(f"k_pool/v_pool must be [num_pages,16,{KV},{D}]")
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
                block_table.shape[0] != B:
            raise ValueError("block_table must be int32 [B,max_pages]")
        args = [_dev(q, "q"), _dev(k, "k_pool"), _dev(v, "v_pool"),
                _dev(block_table, "block_table"), block_table.shape[1], _dev(cu_q, "cu_q"),
                _dev(seq_lens, "seq_lens"), _dev(o, "o"), B, N, k.shape[0]]
        if window is None:
            name = f"gqa_prefill_{kind}_paged"
            rc = getattr(lib, name)(*args, _dtype_code(q), st)
        else:
            name = "gqa_prefill_sliding_window_paged"
            rc = lib.gqa_prefill_sliding_window_paged(*args, int(window), _dtype_code(q), st)
    if rc:
        raise GqaError(name, rc)
    return o


def gqa_prefill_sliding(q, k, v, cu_q, seq_lens, block_table=None, o=None, stream=None):
    """Prefill of the sliding layers: query rows q [N,32,256] of the last
    cu_q[b+1]-cu_q[b] positions of each sequence, causal within the 1024-window;
    the cache (contiguous, or paged with block_table) already holds the chunk."""
    return _prefill_call(GQA_SLIDING, q, k, v, cu_q, seq_lens, block_table, o, stream)


def gqa_prefill_global(q, k, v, cu_q, seq_lens, block_table=None, o=None, stream=None):
    """Prefill of the global layers (q [N,32,512], full causal mask)."""
    return _prefill_call(GQA_GLOBAL, q, k, v, cu_q, seq_lens, block_table, o, stream)


def gqa_prefill_sliding_window(q, k, v, cu_q, seq_lens, window, block_table=None, o=None,
                               stream=None):
    """Prefill of the sliding geometry with a runtime window (1 <= window <=
    262144; the gqa_prefill_sliding_window[_paged] entry points), otherwise as
    gqa_prefill_sliding."""
    return _prefill_call(GQA_SLIDING, q, k, v, cu_q, seq_lens, block_table, o, stream,
                         window=window)
