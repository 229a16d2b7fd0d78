/*
 * gqa_decode.h -- C ABI of the MI355X (gfx950) decode-attention library.
 *
 * The operation is the attn.core node of the gemma-4-31B Model Spec page
 * (docs.theformalera.com/models/gemma-4-31b.md), "Compute-graph nodes" table:
 *
 *   slidingDecodeGQA  o[b,h] = sum_s softmax_s(1 * <q[b,h], k[b,s,h/2]>) * v[b,s,h/2]
 *                     over the last 1024 positions s < seq_lens[b]
 *                     (32 query heads, 16 kv heads, D = 256, scale 1, window 1024)
 *   decodeGQA         the same with kv head h/8 over every s < seq_lens[b]
 *                     (32 query heads, 4 kv heads, D = 512, scale 1)
 *
 * Argument order and shapes follow the page's "Tensors of the main nodes"
 * table (q [B,32,D], k [B,S,kv,D], v [B,S,kv,D], seq_lens [B], o [B,32,D]); the
 * paged forms use the page size 16 of the "At a glance" table (Shape domain
 * row), which also bounds B to [1,256] and S to [1,262144].
 *
 * Window reading: the newest token is already in the cache when attention
 * runs (the compact forward pass on the "Gemma 4 31B-it Text Architecture"
 * page appends K/V first and masks keys t-1024 < s <= t), so sequence b
 * attends to positions [max(0, L-1024), L) with L = seq_lens[b].
 *
 * Layouts (all row-major, D innermost, element type `dtype` for q/k/v/o):
 *   q            [B, 32, D]
 *   contiguous   k, v [B, S_max, KV, D]: row (b, s, g) at ((b*S_max + s)*KV + g)*D
 *   paged        k_pool, v_pool [num_pages, 16, KV, D]; logical position s of
 *                sequence b is physical page block_table[b*max_pages + s/16],
 *                slot s%16
 *   block_table  [B, max_pages] int32
 *   seq_lens     [B] int32
 *   o            [B, 32, D]
 *   workspace    fp32 scratch for split-S partial results, at least
 *                gqa_decode_workspace_bytes(...) bytes (may be NULL when that is 0)
 *
 * Ownership: every pointer is caller-owned device memory.  The library
 * allocates no device memory, keeps no pointer after return and does not
 * synchronise: work is queued on `stream` (a hipStream_t; NULL = the null
 * stream) and the buffers must stay valid until it completes.  Calls that
 * share one workspace must be ordered on one stream.
 *
 * Host-checked preconditions (a negative status is returned and nothing is
 * launched): non-null pointers; 1 <= B <= 256; 1 <= S_max <= 262144 or
 * 1 <= max_pages*16 <= 262144 with num_pages >= 1; a known dtype; 16-byte
 * aligned q, k, v, o and workspace; a large enough workspace.
 *
 * Device-resident preconditions (documented, not checked on the host, which
 * would need a synchronisation): 1 <= seq_lens[b] <= capacity, and
 * block_table[b][p] in [0, num_pages) for every page p holding an attended
 * position.  Device behaviour outside them is memory-safe: seq_lens is
 * clamped to the capacity, seq_lens <= 0 gives a zero output row, a page id
 * outside [0, num_pages) is never dereferenced: its positions are dropped
 * from the softmax (the kernels read a zero page the library holds in its
 * place and set those positions' logits to -inf, so no pool byte behind an
 * invalid id is read and nothing reaches o from it, NaN included), and
 * no K/V byte outside the attended range, and no block-table entry of a
 * page without an attended position, is ever read.
 *
 * Errors: HIP launch failures map to GQA_ERR_HIP.  The library never aborts
 * and never prints.
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of q, k, v and o */
enum { GQA_F32 = 0, GQA_BF16 = 1 };

/* variant selector for the query functions */
enum { GQA_SLIDING = 0, GQA_GLOBAL = 1 };

/* status codes */
enum {
  GQA_OK = 0,
  GQA_ERR_NULL = -1,      /* a required pointer is NULL */
  GQA_ERR_SHAPE = -2,     /* B, S_max, max_pages, num_pages or window out of range */
  GQA_ERR_DTYPE = -3,     /* unknown dtype or variant */
  GQA_ERR_ALIGN = -4,     /* a tensor base pointer is not 16-byte aligned */
  GQA_ERR_WORKSPACE = -5, /* workspace missing or smaller than required */
  GQA_ERR_HIP = -6        /* the HIP runtime reported an error */
};

/* slidingDecodeGQA on a contiguous cache: k, v [B, S_max, 16, 256]. */
int gqa_decode_sliding(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                       void* o, int32_t B, int32_t S_max, int32_t dtype, void* workspace,
                       size_t workspace_bytes, void* stream);

/* decodeGQA on a contiguous cache: k, v [B, S_max, 4, 512]. */
int gqa_decode_global(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                      void* o, int32_t B, int32_t S_max, int32_t dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/* slidingDecodeGQA on a paged cache: k_pool, v_pool [num_pages, 16, 16, 256]. */
int gqa_decode_sliding_paged(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, int32_t max_pages,
                             const int32_t* seq_lens, void* o, int32_t B, int32_t num_pages,
                             int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/* decodeGQA on a paged cache: k_pool, v_pool [num_pages, 16, 4, 512]. */
int gqa_decode_global_paged(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, void* o, int32_t B, int32_t num_pages,
                            int32_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/* slidingDecodeGQA with a runtime window: the kv-head geometry of the sliding
 * layers (32 query heads over 16 kv heads, D = 256, scale 1) attending to the
 * last `window` positions below seq_lens[b], i.e. [max(0, L-window), L).
 * This is the per-layer window of the Retrofit Plan page ("Progressive Window
 * Assignment" table: 1024, 2048, 4096, 8192 in the four sliding layers of a
 * block, each with its own full-length cache); any 1 <= window <= 262144 is
 * accepted (GQA_ERR_SHAPE otherwise).  Arguments, layouts and errors are those
 * of gqa_decode_sliding / gqa_decode_sliding_paged; the workspace size comes
 * from gqa_decode_sliding_window_workspace_bytes. */
int gqa_decode_sliding_window(const void* q, const void* k, const void* v,
                              const int32_t* seq_lens, void* o, int32_t B, int32_t S_max,
                              int32_t window, int32_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream);
int gqa_decode_sliding_window_paged(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* seq_lens, void* o, int32_t B,
                                    int32_t num_pages, int32_t window, int32_t dtype,
                                    void* workspace, size_t workspace_bytes, void* stream);
/* Workspace bytes and launch plan of the windowed calls (0 / GQA_ERR_SHAPE for
 * out-of-range arguments); see gqa_decode_workspace_bytes and gqa_decode_plan. */
size_t gqa_decode_sliding_window_workspace_bytes(int32_t B, int32_t capacity, int32_t window);
int gqa_decode_sliding_window_plan(int32_t B, int32_t capacity, int32_t window, int32_t* mode,
                                   int32_t* n_waves, int32_t* n_slots);

/* slidingDecodeGQA over a cache capped at `ring` positions.  The Retrofit Plan
 * page ("Progressive Window Assignment") gives each sliding layer its own KV
 * cache capped at its window size; read as a ring, k and v are
 * [B, ring, 16, 256] with position s in slot s % ring, so the slots hold the
 * last `ring` positions written (gqa_append_sliding_ring writes them).
 * seq_lens[b] may exceed ring (up to 262144); the call attends to
 * [max(0, L-window), L) as gqa_decode_sliding_window does.  Requires
 * 16 <= ring <= 262144, ring a multiple of 16 (a 16-position tile then never
 * wraps) and 1 <= window <= ring (GQA_ERR_SHAPE otherwise).  Other arguments,
 * ownership and errors as for gqa_decode_sliding; the workspace size comes from
 * gqa_decode_sliding_ring_workspace_bytes (0: none needed, or bad arguments). */
int gqa_decode_sliding_ring(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                            void* o, int32_t B, int32_t ring, int32_t window, int32_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream);
size_t gqa_decode_sliding_ring_workspace_bytes(int32_t B, int32_t ring, int32_t window);

/* KV append of the new token with its per-head norms and RoPE: the nodes
 * attn.qk_norm, attn.v_norm and attn.rope of the Model Spec page's
 * "Compute-graph nodes" table, applied to one new token per sequence at
 * position pos = seq_lens[b] - 1 (seq_lens already counts the new token: the
 * compact forward pass of the architecture page appends K/V before
 * attention), then written into the cache at pos:
 *   q_out[b,h]      = rope(q_raw[b,h] / rms * w_q)
 *   cache k[b,pos,g] = rope(k_raw[b,g] / rms * w_k)
 *   cache v[b,pos,g] = v_raw[b,g] / rms          (global: v_raw is k_raw)
 *   rms = sqrt(mean_d x^2 + 1e-6); rope rotates pairs (i, i + D/2) by
 *   pos * theta^(-2i/D), (a, b) -> (a cos - b sin, a sin + b cos), for
 *   i < active: sliding theta 1e4, 128 of 128 pairs; global theta 1e6, the
 *   first 64 of 256 pairs (the rest keep zero inverse frequency).
 * Layouts: q_raw, q_out [B,32,D]; k_raw, v_raw [B,KV,D]; w_q, w_k [D]; caches
 * as in the attention calls.  All share `dtype`; q_out may equal q_raw.
 * Angles are formed in double precision, norms and rotation in fp32, outputs
 * rounded to the dtype (RNE).  A sequence with seq_lens[b] outside
 * [1, capacity] gets zero q_out rows and no cache write; a page id outside
 * [0, num_pages) gets no cache write.  Nothing else in the cache is touched.
 * Host-checked errors as for the attention calls (pointers, B, capacity,
 * dtype, 16-byte alignment). */
int gqa_append_sliding(const void* q_raw, const void* k_raw, const void* v_raw, const void* w_q,
                       const void* w_k, const int32_t* seq_lens, void* q_out, void* k_cache,
                       void* v_cache, int32_t B, int32_t S_max, int32_t dtype, void* stream);
int gqa_append_sliding_paged(const void* q_raw, const void* k_raw, const void* v_raw,
                             const void* w_q, const void* w_k, const int32_t* block_table,
                             int32_t max_pages, const int32_t* seq_lens, void* q_out,
                             void* k_pool, void* v_pool, int32_t B, int32_t num_pages,
                             int32_t dtype, void* stream);
/* The sliding append into a cache capped at `ring` positions (layout and
 * requirements as gqa_decode_sliding_ring): the new token's rows go to slot
 * (seq_lens[b] - 1) % ring, the rotation uses the true position
 * seq_lens[b] - 1; seq_lens[b] outside [1, 262144] gets zero q_out rows and no
 * cache write. */
int gqa_append_sliding_ring(const void* q_raw, const void* k_raw, const void* v_raw,
                            const void* w_q, const void* w_k, const int32_t* seq_lens,
                            void* q_out, void* k_cache, void* v_cache, int32_t B, int32_t ring,
                            int32_t dtype, void* stream);
int gqa_append_global(const void* q_raw, const void* k_raw, const void* w_q, const void* w_k,
                      const int32_t* seq_lens, void* q_out, void* k_cache, void* v_cache,
                      int32_t B, int32_t S_max, int32_t dtype, void* stream);
int gqa_append_global_paged(const void* q_raw, const void* k_raw, const void* w_q,
                            const void* w_k, const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, void* q_out, void* k_pool, void* v_pool,
                            int32_t B, int32_t num_pages, int32_t dtype, void* stream);

/* decodeGQA over a values-only cache (global layers).  On the global layers
 * the values are the raw keys (the Model Spec page: "What to watch for" and
 * attention_k_eq_v in "Published configuration"; the architecture page's
 * compact forward pass takes V_raw = K_raw), so with u = K_raw / rms the
 * cache's value row is u and the key row is rope(w_k * u, s).  These calls
 * read only the value cache and rebuild each key in the kernel:
 *   k_s = rope(w_k * v_s, s), s = the position of the row in its sequence,
 * with the global RoPE of gqa_append_global (pairs (i, i+256), the first 64
 * rotating by s * 1e6^(-2i/512)), then attend exactly as gqa_decode_global.
 * That halves the bytes a decode step reads (4 KiB instead of 8 KiB per
 * position in bf16).  Keys are rebuilt in fp32 (angles in double) and
 * rounded to the dtype before the QK^T product, as a stored key would be;
 * the query is multiplied by w_k (rounded to the dtype) on the 448
 * coordinates that do not rotate.
 * Arguments: q [B,32,512]; v [B,S_max,4,512] (contiguous) or v_pool
 * [num_pages,16,4,512] with block_table [B,max_pages]; w_k [512] (the k_norm
 * weight), all of one dtype; other arguments, the workspace (the size of
 * gqa_decode_workspace_bytes(GQA_GLOBAL, ...)), the plan and errors are those
 * of gqa_decode_global / gqa_decode_global_paged.  w_k NULL -> GQA_ERR_NULL. */
int gqa_decode_global_k_eq_v(const void* q, const void* v, const void* w_k,
                             const int32_t* seq_lens, void* o, int32_t B, int32_t S_max,
                             int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream);
int gqa_decode_global_k_eq_v_paged(const void* q, const void* v_pool, const void* w_k,
                                   const int32_t* block_table, int32_t max_pages,
                                   const int32_t* seq_lens, void* o, int32_t B,
                                   int32_t num_pages, int32_t dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);
/* The append of the global layers for a values-only cache: as
 * gqa_append_global (q_out and the value row u = k_raw / rms at pos) but no
 * key row is stored. */
int gqa_append_global_k_eq_v(const void* q_raw, const void* k_raw, const void* w_q,
                             const void* w_k, const int32_t* seq_lens, void* q_out,
                             void* v_cache, int32_t B, int32_t S_max, int32_t dtype,
                             void* stream);
int gqa_append_global_k_eq_v_paged(const void* q_raw, const void* k_raw, const void* w_q,
                                   const void* w_k, const int32_t* block_table,
                                   int32_t max_pages, const int32_t* seq_lens, void* q_out,
                                   void* v_pool, int32_t B, int32_t num_pages, int32_t dtype,
                                   void* stream);

/* Prefill / chunked prefill: attention of a chunk of new tokens per sequence
 * whose K/V rows are already in the cache (the architecture page, "Prefill,
 * Cache, and Long Context", and the masks of its compact forward pass:
 * positions = past_seen_tokens + arange(T_current); full layers keep keys
 * s <= t, sliding layers t - 1024 < s <= t; K/V appended before attention).
 * Sequence b holds seq_lens[b] positions; its T_b = cu_q[b+1] - cu_q[b] query
 * rows are its last T_b positions, so query row n = cu_q[b] + t sits at
 *   p = seq_lens[b] - T_b + t
 * and, for every head h (kv head h/2 sliding, h/8 global, scale 1),
 *   o[n,h] = sum_s softmax_s(<q[n,h], k[b,s,h/G]>) * v[b,s,h/G]
 * over s in [max(0, p - 1023), p] (sliding) or [0, p] (global).
 * Arguments: q, o [N,32,D] (packed query rows of all sequences); cu_q [B+1]
 * int32 (cu_q[0] = 0, non-decreasing, cu_q[B] = N); seq_lens [B] int32; the
 * cache as in the decode calls (contiguous [B,S_max,KV,D] or paged pools with
 * block_table).  No workspace.  Host-checked: pointers, 1 <= B <= 256,
 * 1 <= N <= 2^24, the capacity, dtype, 16-byte alignment (status as the
 * decode calls).  Device-resident preconditions: cu_q as stated,
 * T_b <= seq_lens[b] <= capacity, block-table entries of the attended pages
 * in [0, num_pages).  Rows whose position would be negative are zero;
 * seq_lens is clamped to the capacity; a page id outside the pool drops its
 * positions as in the decode calls (the library's zero page is read in its
 * place and its logits are set to -inf).  Softmax in fp32, P rounded to bf16
 * for bf16 inputs. */
int gqa_prefill_sliding(const void* q, const void* k, const void* v, const int32_t* cu_q,
                        const int32_t* seq_lens, void* o, int32_t B, int32_t N, int32_t S_max,
                        int32_t dtype, void* stream);
int gqa_prefill_global(const void* q, const void* k, const void* v, const int32_t* cu_q,
                       const int32_t* seq_lens, void* o, int32_t B, int32_t N, int32_t S_max,
                       int32_t dtype, void* stream);
int gqa_prefill_sliding_paged(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, int32_t max_pages, const int32_t* cu_q,
                              const int32_t* seq_lens, void* o, int32_t B, int32_t N,
                              int32_t num_pages, int32_t dtype, void* stream);
int gqa_prefill_global_paged(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, int32_t max_pages, const int32_t* cu_q,
                             const int32_t* seq_lens, void* o, int32_t B, int32_t N,
                             int32_t num_pages, int32_t dtype, void* stream);

/* Prefill of the sliding geometry with a runtime window: each query row at
 * position p attends to [max(0, p - window + 1), p].  These are the per-layer
 * windows of the Retrofit Plan page ("Progressive Window Assignment": 1024,
 * 2048, 4096 and 8192 in the four sliding layers of a block); any
 * 1 <= window <= 262144 is accepted (GQA_ERR_SHAPE otherwise).  Arguments,
 * layouts and errors are those of gqa_prefill_sliding / _paged; window 1024
 * is the default entry points' own. */
int gqa_prefill_sliding_window(const void* q, const void* k, const void* v, const int32_t* cu_q,
                               const int32_t* seq_lens, void* o, int32_t B, int32_t N,
                               int32_t S_max, int32_t window, int32_t dtype, void* stream);
int gqa_prefill_sliding_window_paged(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, int32_t max_pages,
                                     const int32_t* cu_q, const int32_t* seq_lens, void* o,
                                     int32_t B, int32_t N, int32_t num_pages, int32_t window,
                                     int32_t dtype, void* stream);

/* decodeGQA on a paged cache without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Arguments, layouts, results and
 * errors are those of gqa_decode_global_paged with workspace and
 * workspace_bytes left out: the split-S partials go to a library-owned array
 * of GQA_NOALLOC_SCRATCH_BYTES bytes in device memory (the workspace of the
 * largest batch, B = 256), which each device that loads the library holds
 * until the process ends.  The call itself allocates nothing; a plan needing
 * more than that array returns GQA_ERR_WORKSPACE.  The first call on a device
 * looks up the array's address with that device current (HIP may load the
 * library's code object then), so make it outside graph capture.  All calls
 * on one device share the one array and every call overwrites it: calls that
 * can overlap on a device (other streams, other threads) race and must be
 * ordered by the caller.  Nothing in the array needs to start at zero. */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)33 << 20)
int gqa_decode_global_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* seq_lens, void* o, int32_t B,
                                    int32_t num_pages, int32_t dtype, void* stream);

/* Workspace bytes a call needs for `variant` (GQA_SLIDING / GQA_GLOBAL), batch B
 * and cache capacity (S_max, or max_pages*16 for the paged forms).  Depends on
 * nothing else (not on dtype, device or seq_lens).  0 means no split-S pass:
 * the workspace may then be NULL.  Returns 0 for out-of-range arguments too. */
size_t gqa_decode_workspace_bytes(int32_t variant, int32_t B, int32_t capacity);

/* launch modes reported by gqa_decode_plan */
enum { GQA_MODE_UNIT = 0, GQA_MODE_STREAM = 1, GQA_MODE_GROUP = 2 };

/* The launch plan for these arguments (a function of them alone).
 * GQA_MODE_UNIT: one work-group of four waves per (sequence, kv head), used
 *   when there are enough such units for their length (at least 1024 units
 *   of at most 320 tiles of 16 positions, 256 of at most 128, or on the
 *   sliding geometry 128 of at most 65); no workspace; *n_waves = 4 * units,
 *   *n_slots = 0.
 * GQA_MODE_STREAM (the sliding geometry's other calls): *n_waves persistent
 *   waves each take an equal share of all tiles, partials of units shared by
 *   several waves go to *n_slots workspace slots, and a combine kernel merges
 *   them.
 * GQA_MODE_GROUP (the global geometry's other calls, and sliding calls of at
 *   most 2048 tiles of 16 positions over all units at the capacity):
 *   *n_waves / 4 work-groups each take an equal share of all tiles (their four
 *   waves share each unit piece and merge it in LDS); partials of units shared
 *   by several work-groups go to *n_slots workspace slots, and the combine
 *   kernel merges them.
 * Returns GQA_OK or GQA_ERR_SHAPE / GQA_ERR_DTYPE. */
int gqa_decode_plan(int32_t variant, int32_t B, int32_t capacity, int32_t* mode,
                    int32_t* n_waves, int32_t* n_slots);

/* Compile-time constants of a variant (heads, kv heads, head dim, window, page).
 * window is 0 for decodeGQA.  Returns GQA_OK or GQA_ERR_DTYPE. */
int gqa_decode_constants(int32_t variant, int32_t* heads, int32_t* kv_heads, int32_t* head_dim,
                         int32_t* window, int32_t* page);

/* Static description of a status code. */
const char* gqa_status_str(int32_t status);

/* Measurement and test utility: every later plan (and call) takes launch mode
 * `mode` (GQA_MODE_*) whatever the planner would choose, or the planner's
 * choice again for mode = -1.  Process-wide and not thread-safe; each mode
 * computes the same attention.  Returns GQA_OK or GQA_ERR_SHAPE. */
int gqa_decode_force_mode(int32_t mode);

/* Measurement utilities, not part of the attention path: a plain read stream
 * of `bytes` bytes from `src` (non-temporal 16-byte loads, 1 KiB contiguous
 * per wave instruction; `sink` is a 4-byte device word the kernel may write)
 * and a plain copy of `bytes` bytes from `src` to `dst`.  They measure the
 * sustainable HBM rate and calibrate a profiler's byte counters.  bytes must
 * be a positive multiple of 16 and the pointers 16-byte aligned device
 * memory; asynchronous on `stream`.  Returns GQA_OK or a negative status. */
int gqa_hbm_read_probe(const void* src, size_t bytes, void* sink, void* stream);
int gqa_hbm_copy_probe(const void* src, void* dst, size_t bytes, void* stream);

/* Launch timing for measurement: while enabled, every kernel the library
 * launches is bracketed by HIP events recorded on its stream (at most
 * `capacity` launches are kept).  gqa_profile_read synchronises those events
 * and reports, per kernel kind, the number of launches and their summed
 * duration in milliseconds (kind 2*variant: main kernel of that variant,
 * 2*variant+1: its combine kernel, 4+variant: its append kernel; the
 * values-only global calls: 6 main, 7 combine, 8 append; prefill: 9+variant);
 * it also
 * disables recording and releases
 * the events.  Measurement only: not thread-safe, not for captured graphs. */
int gqa_profile_begin(int32_t capacity);
int gqa_profile_read(int32_t* counts, double* total_ms, int32_t n_kinds);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */
