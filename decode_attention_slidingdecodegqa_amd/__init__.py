"""MI355X (gfx950) decode attention for the Gemma-4-31B text decoder.

Thin Python binding over the C ABI of ``libgqadecode.so`` (declared in
``include/gqa_decode.h``).  The functions carry the C names and only marshal
arguments: torch tensors provide device memory and the current stream, every
step of the computation runs in the HIP kernels.  There is no fallback: when
the library is missing or no GPU is present the calls raise.

    gqa_decode_sliding(q, k, v, seq_lens)               slidingDecodeGQA, contiguous cache
    gqa_decode_global(q, k, v, seq_lens)                decodeGQA, contiguous cache
    gqa_decode_sliding_paged(q, k_pool, v_pool, block_table, seq_lens)
    gqa_decode_global_paged(q, k_pool, v_pool, block_table, seq_lens)
    gqa_decode_sliding_window(q, k, v, seq_lens, window)    sliding geometry, runtime window
    gqa_decode_sliding_window_paged(q, k_pool, v_pool, block_table, seq_lens, window)
    gqa_decode_sliding_ring(q, k, v, seq_lens, window)  sliding cache capped at R positions
                                                        (k, v [B,R,16,256], slot s % R)
    gqa_append_sliding_ring(q_raw, k_raw, v_raw, w_q, w_k, seq_lens, k_cache, v_cache)
    gqa_append_sliding(q_raw, k_raw, v_raw, w_q, w_k, seq_lens, k_cache, v_cache[, block_table])
    gqa_append_global(q_raw, k_raw, w_q, w_k, seq_lens, k_cache, v_cache[, block_table])
                                                        new token: norms, RoPE, cache write
    gqa_decode_global_k_eq_v(q, v, w_k, seq_lens)       decodeGQA over a values-only cache
    gqa_decode_global_k_eq_v_paged(q, v_pool, w_k, block_table, seq_lens)
    gqa_append_global_k_eq_v(q_raw, k_raw, w_q, w_k, seq_lens, v_cache[, block_table])
    gqa_prefill_sliding(q, k, v, cu_q, seq_lens[, block_table])   prefill / chunked prefill
    gqa_prefill_global(q, k, v, cu_q, seq_lens[, block_table])
    gqa_prefill_sliding_window(q, k, v, cu_q, seq_lens, window[, block_table])

Shapes (attn.core of the gemma-4-31B Model Spec page): q [B,32,D]; contiguous
k/v [B,S_max,KV,D]; paged pools [num_pages,16,KV,D] with block_table
[B,max_pages] int32; seq_lens [B] int32; returns o [B,32,D] of q's dtype
(float32 or bfloat16).  Sliding: KV=16, D=256, window 1024.  Global: KV=4, D=512.
The values-only variants keep one [.,.,4,512] cache for the global layers,
whose values equal their keys before RoPE and the k weight: the key of
position s is rope(w_k * v_s, s), rebuilt inside the attention kernel.
"""
from __future__ import annotations

from ._lib import (  # noqa: F401
    GQA_BF16,
    GQA_F32,
    GQA_GLOBAL,
    GQA_SLIDING,
    GqaError,
    constants,
    force_mode,
    gqa_append_global,
    gqa_append_global_k_eq_v,
    gqa_append_sliding,
    gqa_append_sliding_ring,
    gqa_decode_global,
    gqa_decode_global_k_eq_v,
    gqa_decode_global_k_eq_v_paged,
    gqa_decode_global_paged,
    gqa_decode_global_paged_noalloc,
    gqa_decode_plan,
    gqa_decode_sliding,
    gqa_decode_sliding_paged,
    gqa_decode_sliding_window,
    gqa_decode_sliding_ring,
    gqa_decode_sliding_ring_workspace_bytes,
    gqa_decode_sliding_window_paged,
    gqa_decode_workspace_bytes,
    gqa_prefill_global,
    gqa_prefill_sliding,
    gqa_prefill_sliding_window,
    gqa_status_str,
    hbm_copy_probe,
    hbm_read_probe,
    library,
    profile_begin,
    profile_read,
    EXPORTED_SYMBOLS,
)
