// gqa_decode.hip -- gfx950 decode attention for the Gemma-4-31B text decoder.
//
// Implements the attn.core node of the gemma-4-31B Model Spec page
// ("Compute-graph nodes" table): slidingDecodeGQA (32 query heads over 16 kv
// heads, D = 256, scale 1, the last 1024 positions) and decodeGQA (32 over 4,
// D = 512, scale 1, every position below seq_lens[b]), on a contiguous
// [B,S,kv,D] cache or on a paged cache of 16-position pages (the "At a glance"
// table's Shape domain row).  The C ABI is declared in include/gqa_decode.h.
//
// Method: flash-decoding with an exactly balanced ("stream-K") partition.
//
//   Work.  A unit is one (sequence b, kv head g); its attended positions
//   [lo, L) are cut into 16-position tiles (a tile is one page).  All tiles of
//   all units form one sequence, unit-major.  A fixed number W of persistent
//   waves each take an equal contiguous slice of it, whatever the mix of
//   sequence lengths, and carry their softmax state across the slice.  When a
//   slice leaves a unit, the wave flushes that unit's partial (O, m, l) to
//   workspace slot unit + wave, or writes o itself when its slice held the
//   whole unit; a combine kernel merges the 1..n partials of split units.
//
//   Tile.  One wave64 consumes a tile with every query head of the GQA group:
//   QK^T  v_mfma_f32_16x16x32_bf16 (16x16x4_f32 for f32): A = the 16 key rows,
//         B = the group's query heads padded to 16 columns.  The
//         reduction index may be any permutation of d shared by A and B, so
//         each lane loads whole 16-byte chunks of one key row straight into
//         the operand registers.
//   softmax online, fp32: base-2 exponentials of (z - m) * log2(e).  The logit
//         accumulator layout (lane = head column, 4 consecutive positions) is
//         the B operand layout of the PV instruction, so P never moves.
//   PV    v_mfma_f32_16x16x16_bf16 (16x16x4_f32): O^T = V^T P^T with V^T built
//         by transposing in registers the 4 rows x 8 columns a lane loads.
//   The accumulator holds O^T, so the per-head rescale is a per-lane scalar.
//
// Every K/V byte of the attended range is read from HBM exactly once; no byte
// outside it is read (rows outside [lo, L) are clamped onto attended rows of
// the same tile and dropped through -inf logits, so NaN or stale data in
// unused cache space cannot reach the result).

#include <mutex>
#include <vector>

#include "gqa_common.h"

namespace {

struct KernelArgs {
  const char* q;
  const char* k;    // unused when keys are rebuilt from values
  const char* v;
  const char* w_k;  // key weight [512]: keys rebuilt from values (global layers) when set
  const int32_t* seq_lens;
  const int32_t* block_table;
  char* o;
  int32_t* prefix;  // [B+1] flattened tile index of each sequence's first unit
  float* ws_ml;     // [slot][G][2]  (m, l)
  float* ws_acc;    // [slot][G][D]
  int32_t B;
  int32_t cap;
  int32_t max_pages;
  int32_t num_pages;
  int32_t window;
  int32_t n_waves;
  int32_t ring;  // > 0: contiguous cache capped at `ring` positions, position s in slot s % ring
  int32_t* counter;  // group mode with a dynamic tail: the chunk counter (zero at launch)
  int32_t dyn;       // nonzero: group mode may take a dynamic tail (tail_plan)
};

// Capacity that bounds a sequence's positions: the cache's, or for a ring
// (whose slots hold the last `ring` positions) the position domain.
__device__ inline int position_cap(int cap, int ring) { return ring > 0 ? kMaxSeq : cap; }

// Attended range of one sequence: positions [lo, L), tiles [t0, t0 + n).
struct SeqRange {
  int lo, L, t0, n;
};

__device__ inline SeqRange seq_range(int L_raw, int cap, int window) {
  SeqRange s;
  const int L = L_raw < cap ? L_raw : cap;
  if (L <= 0) {
    s.lo = s.L = s.t0 = s.n = 0;
    return s;
  }
  s.L = L;
  s.lo = (window > 0 && L > window) ? L - window : 0;
  s.t0 = s.lo / kTile;
  s.n = (L + kTile - 1) / kTile - s.t0;
  return s;
}

// floor(num / den) for 0 <= num < 2^40 and 0 < den < 2^27 (tile counts are at
// most 2^26, slice counts below 2^12), in fp64: both operands are exact, the
// quotient is correctly rounded, and a quotient that is not an integer lies at
// least 1/den from one, far beyond its rounding error, so truncation gives the
// integer quotient.  A 64-bit integer division expands into a long sequence
// that would sit ahead of every work-group's first load.
__device__ inline long floor_div(long num, long den) {
  return (long)((double)num / (double)den);
}

// Cross-lane steps without LDS round trips (a ds_bpermute waits behind every
// LDS access in flight): the lane swaps exchange lanes l and l ^ 16 (l ^ 32),
// DPP row rotations move values within a 16-lane row.
__device__ inline float max_lanes_xor16_32(float x) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}
__device__ inline float sum_lanes_xor16_32(float x) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}
// DPP row rotation by K lanes (row_ror:K) of a float
template <int K>
__device__ inline float row_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + K, 0xf, 0xf, false));
}
// the maximum over all 64 lanes, in every lane
__device__ inline float max_wave(float x) {
  x = max_lanes_xor16_32(x);
  x = fmaxf(x, row_ror<8>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<2>(x));
  return fmaxf(x, row_ror<1>(x));
}
// DPP row shift right by K lanes (row_shr:K) of an int; lanes below K read 0
template <int K>
__device__ inline int row_shr(int x) {
  return __builtin_amdgcn_update_dpp(0, x, 0x110 + K, 0xf, 0xf, true);
}

// Wave whose slice holds flattened tile t: slice w is [w*T/W, (w+1)*T/W).
__device__ inline int wave_of(long t, long T, int W) {
  return (int)floor_div((t + 1) * W - 1, T);
}

// Dynamic tail of the group partition.  Equal static slices leave the XCDs
// that read HBM faster idle at the end (measured per work-group on the global
// B=32 step: four XCDs finished their slices in 2.53-2.57 ms, the other four
// in 2.77-2.84 ms).  So in a large group-mode call the static slices cover the
// first S tiles only, and the last ~1/12 of the tiles form nch chunks of C
// tiles that the work-groups take from a counter when their slice is done.
// Chunk c is slice W + c for the partial slots and the combine.
constexpr long kDynMinTiles = 1L << 19;  // smaller calls (under ~2048 tiles per
                                         // work-group): static slices only, a
                                         // chunk there would be a large share
constexpr int kDynMaxChunks = 768;    // partial slots a call may add
constexpr int kDynMinChunk = 128;     // tiles per chunk at least
struct TailPlan {
  long S;   // tiles of the static slices
  int C;    // tiles per chunk
  int nch;  // chunks
};
__host__ __device__ inline TailPlan tail_plan(long T, int dyn) {
  if (!dyn || T < kDynMinTiles) return TailPlan{T, 1, 0};
  const long Td = T / 12;
  long C = (Td + kDynMaxChunks - 1) / kDynMaxChunks;
  if (C < kDynMinChunk) C = kDynMinChunk;
  const int nch = (int)(Td / C);
  return TailPlan{T - (long)nch * C, (int)C, nch};
}
// the slice holding flattened tile t (W static slices over [0, S), then the chunks)
__device__ inline int slice_of(long t, const TailPlan& tp, int W) {
  return t < tp.S ? wave_of(t, tp.S, W) : W + (int)(t - tp.S) / tp.C;
}

// Waves that share the T tiles of a stream-mode call: the W launched, or
// only max(T, kMinStreamWaves) of them when the actual lengths give fewer
// tiles than waves (the rest leave at once and hold no slice, so the combine
// reads no empty slots).  Folding several tiles into each wave to save
// partials measured slower: a global call of 4 sequences over 4096 positions
// took 30.8 us in its main kernel at 256 waves of about 6 tiles, 21 us at
// 1024 waves of 1.6.  The main and combine kernels both derive it from T.
constexpr int kMinStreamWaves = 256;
__device__ inline int effective_waves(long T, int W) {
  const long w = T > kMinStreamWaves ? T : kMinStreamWaves;
  return w < W ? (int)w : W;
}

// Waves per SIMD the main kernels are compiled for: the sliding bf16 kernels
// fit two (<= 256 registers), the others need one.
template <int KV, bool BF16>
constexpr int main_waves_per_simd() {
  return (KV == 16 && BF16) ? 2 : 1;
}

// ---- keys rebuilt from values (global layers: values = keys)
// k_s = rope(w_k * v_s, s): pairs (i, i+256) rotate by s * 1e6^(-2i/512) for
// i < 64, the other 448 coordinates are w_k * v.  The unrotated coordinates
// fold w_k into the query once per unit; a rotated pair of position
// pos0 + r is R(pos0*f_i) * M[r][i] * (v_i, v_{i+256}) with the work-group
// table M[r][i] = R(r*f_i) * diag(w_i, w_{i+256}) (r < 16) and the wave's
// per-tile base R(pos0*f_i), both in LDS, the angles formed in double.
constexpr int kRopePairs = 64;
constexpr double kLog2ThetaGlobal = 19.931568569324174;  // log2(1e6)

struct RopeLds {
  // R(r f_i) diag(w_i, w_{i+256}) as a row-major 2x2, pair-major so that the
  // 16 rows of one pair are 16 consecutive 16-byte entries (no bank conflicts)
  float m[kRopePairs][kTile][4];
  float base[kWaves][kRopePairs][2];  // per wave: (cos, sin)(pos0 f_i)
  double freq[kRopePairs];        // f_i = 1e6^(-2i/512)
};

// The per-wave LDS tile of the staged (bf16 keys-from-values) path: 16 rows of
// 512 bf16 values, unpadded, chunk c of row r stored at chunk c ^ f(r) with
// f(r) = 4(r % 4) + 2((r / 4) % 2).  The rows arrive whole (as the stored
// keys below) and both operand layouts are read back: the key operand into
// the registers, where its rotated chunks are rebuilt, and the value operand.
// gfx950 serves a 16-byte-per-lane LDS read in groups of 16 lanes taking rows
// r = 0..7 of one 16-lane quarter and r = 8..15 of the next: the key-operand
// reads (row r, chunk 4c + j) split by parity and the value-operand reads
// (rows 4j + i, chunk r + 16 blk) by bit 3, so neither has bank conflicts (a
// 16-byte row pad would halve the rate).
template <bool KFV, bool BF16>
constexpr bool kStaged = KFV && BF16;
// bf16 stored keys: each tile's key rows are fetched whole (one 1 KiB load
// instruction per 1 KiB of rows, the pattern a plain read streams fastest)
// and reach the MFMA operand layout (lane (r, j): row r, chunks 4c + j)
// through a per-wave LDS tile of unpadded rows with the same chunk swizzle.
// Fetched in the operand layout directly, every load instruction took 64
// bytes of 16 rows, and consecutive lanes read different rows: a plain read
// in that pattern measured 6.0 TB/s, whole rows 7.37 TB/s, and the value
// rows' pattern (4 rows x 256 bytes) 7.1.
template <bool KFV, bool BF16>
constexpr bool kRowKeys = !KFV && BF16;
constexpr int kStageRow = 512 * 2;
__device__ __forceinline__ int stage_swz(int r) { return ((r & 3) << 2) | ((r & 4) >> 1); }
constexpr int kStageBytes = kTile * kStageRow;
// LDS bytes per wave of a main kernel: the keys-from-values tile, the
// whole-row keys' tile (16 rows of ROW bytes), or none
template <bool KFV, bool BF16, int ROW>
constexpr int wave_stage_bytes() {
  return kStaged<KFV, BF16> ? kStageBytes : kRowKeys<KFV, BF16> ? kTile * ROW : 0;
}

template <bool BF16>
__device__ inline float elem_f32(const char* base, int i) {
  if constexpr (BF16) return bf16_value(*reinterpret_cast<const unsigned short*>(base + 2 * i));
  return *reinterpret_cast<const float*>(base + 4 * i);
}

template <bool BF16>
__device__ void rope_tables_init(const char* w_k, RopeLds* rl) {
  for (int idx = threadIdx.x; idx < kTile * kRopePairs; idx += kThreads) {
    const int r = idx / kRopePairs, i = idx % kRopePairs;
    const double f = exp2(-2.0 * i / 512 * kLog2ThetaGlobal);
    if (r == 0) rl->freq[i] = f;
    double sd, cd;
    sincos(r * f, &sd, &cd);
    const float c = (float)cd, sn = (float)sd;
    const float wa = elem_f32<BF16>(w_k, i), wb = elem_f32<BF16>(w_k, i + 256);
    rl->m[i][r][0] = c * wa;
    rl->m[i][r][1] = -sn * wb;
    rl->m[i][r][2] = sn * wa;
    rl->m[i][r][3] = c * wb;
  }
}

// the calling wave's base rotation of the tile starting at position pos0
// The angle pos0 * f_i is formed in revolutions in double and reduced to
// [-1/2, 1/2]; the hardware sine and cosine (v_sin_f32 / v_cos_f32, argument in
// revolutions, absolute error near 1e-6 on that range) then take it.
__device__ inline void rope_base(RopeLds* rl, int wave, int pos0) {
  const int i = threadIdx.x & 63;
  const double rev = (double)pos0 * rl->freq[i] * 0.15915494309189535;  // / 2 pi
  const float red = (float)(rev - rint(rev));
  rl->base[wave][i][0] = __builtin_amdgcn_cosf(red);
  rl->base[wave][i][1] = __builtin_amdgcn_sinf(red);
}

// Accumulates into st the tiles k_begin, k_begin + step, ... (< k_end) of unit
// (b, g), whose attended range is sr, with the calling wave.  myq is the wave's
// LDS slice for the unit's query heads.
template <int KV, int D, bool PAGED, bool BF16, bool KFV>
__device__ __forceinline__ void accumulate_tiles(const KernelArgs& a, int b, int g,
                                                 const SeqRange& sr, int k_begin, int k_end,
                                                 int step, u32x4* myq, RopeLds* rl, char* stage,
                                                 WaveState<KV, D, BF16>& st) {
  static_assert(!KFV || (KV == 4 && D == 512), "keys from values: global layers only");
  // wave-uniform in every caller, but derived from the lane's thread index or
  // from LDS reads: taken through a scalar register so that the tile and row
  // addressing below runs on the scalar unit instead of in every lane
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  k_begin = __builtin_amdgcn_readfirstlane(k_begin);
  k_end = __builtin_amdgcn_readfirstlane(k_end);
  // bf16 keys from values: each tile is fetched once, in whole rows, and
  // staged in the wave's LDS buffer, from which both operands are read
  constexpr bool STAGED = kStaged<KFV, BF16>;
  using Gm = Geo<KV, D, BF16>;
  constexpr int G = Gm::G, E = Gm::E, ROW = Gm::ROW, NCH = Gm::NCH, KCH = Gm::KCH,
                VBLK = Gm::VBLK, QPL = Gm::QPL;
  constexpr size_t POS = Gm::POS;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;  // row (A) / column (B, C) index of the 16x16 tiles
  const int j = lane >> 4;  // k-group of the operands, row-group of C

#pragma unroll
  for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
    for (int e = 0; e < E; ++e) st.acc[blk][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The reference max is raised only when a tile's max exceeds it by more
  // than kRescaleGap, so weights stay below e^kRescaleGap and the O/l rescale
  // runs a few times per unit instead of every tile; the softmax is the same.
  st.m = -INFINITY;
  st.l = 0.f;
  const int n_it = k_end > k_begin ? (k_end - k_begin + step - 1) / step : 0;
  if (n_it == 0) return;

  // The group's query heads live in the wave's LDS slice (row h = head g*G+h,
  // NCH chunks); QK^T reads them back per tile as the B operand.  Columns
  // >= G of the 16-wide operand are never stored or merged: they are zero, or
  // repeat head 0 where an unconditional read pays (a select there becomes a
  // branch around every read).  The global loads go first and the LDS store
  // waits for the first tile's K/V loads to be in flight, so the two
  // latencies overlap.
  u32x4 qstage[QPL];
  {
    const char* qsrc = a.q + ((size_t)b * kHeads + g * G) * ROW;
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
      const int c = lane + 64 * i;
      if (c < G * NCH) qstage[i] = load16(qsrc + (size_t)c * 16);
    }
    if constexpr (KFV) {
      // w_k folded into the query on the coordinates that do not rotate
#pragma unroll
      for (int i = 0; i < QPL; ++i) {
        const int c = lane + 64 * i;
        const int cc = c % NCH;  // chunk within the head row
        if (c < G * NCH && (cc * E) % 256 >= kRopePairs) {
          const u32x4 w = load16(a.w_k + (size_t)cc * 16);
          if constexpr (BF16) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const unsigned x = qstage[i][q], y = w[q];
              const float lo = bf16_value(x & 0xffffu) * bf16_value(y & 0xffffu);
              const float hi = bf16_value(x >> 16) * bf16_value(y >> 16);
              qstage[i][q] = bf16_pack2(lo, hi);
            }
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              qstage[i][q] = __builtin_bit_cast(unsigned, chunk_f32(qstage[i], q) * chunk_f32(w, q));
          }
        }
      }
    }
  }
  // the wave's query rows in LDS, chunk c of head h at c ^ stage_swz(h) (the
  // operand reads, lane (r, j) at chunk 4t + j of head r, would otherwise put
  // eight heads on one bank)
  const int qh = r < G ? r : 0;
  const u32x4* qrow = myq + qh * NCH;
  const int qswz = stage_swz(qh);

  // Physical pages of iterations it0 + lane (cur) and it0 + 64 + lane (nxt);
  // block-table entries of pages without an attended position are never read.
  const int32_t* bt = PAGED ? a.block_table + (size_t)b * a.max_pages + sr.t0 : nullptr;
  int it0 = 0;
  int pg_cur = 0, pg_nxt = 0;
  if constexpr (PAGED) {
    if (lane < n_it) pg_cur = bt[k_begin + step * lane];
    if (64 + lane < n_it) pg_nxt = bt[k_begin + step * (64 + lane)];
  }

  // Per-tile addressing.  Rows outside [lo, L) are clamped onto the nearest
  // attended row of the same tile: every load is unconditional yet never
  // leaves the attended range; the clamped duplicates are dropped below by
  // -inf logits (their softmax weight is exactly 0).
  struct TileAt {
    const char* kb;
    const char* vb;
    int pos0;
    int ok;  // page id inside the pool (an int: the struct has no padding bytes,
             // which the compiler would otherwise copy through LDS)
  };
  auto tile_at = [&](int it) {
    TileAt ta;
    ta.pos0 = (sr.t0 + k_begin + step * it) * kTile;
    size_t off;
    if constexpr (PAGED) {
      const int i = it - it0;
      const int page = i < 64 ? __builtin_amdgcn_readlane(pg_cur, i)
                              : __builtin_amdgcn_readlane(pg_nxt, i - 64);
      ta.ok = page >= 0 && page < a.num_pages;
      if (!ta.ok) {
        // a page id outside the pool is never dereferenced: its rows come
        // from the library's zero page (a scalar select) and its logits are
        // set to -inf below, so its positions drop out of the softmax
        ta.kb = ta.vb = zero_page() + (size_t)g * ROW;
        return ta;
      }
      off = ((size_t)page * kPage * KV + g) * (size_t)ROW;
    } else {
      ta.ok = true;
      // a ring of a multiple of 16 slots never splits a 16-aligned tile
      const int slot0 = a.ring > 0 ? ta.pos0 % a.ring : ta.pos0;
      off = (((size_t)b * a.cap + slot0) * KV + g) * (size_t)ROW;
    }
    ta.kb = (KFV ? a.v : a.k) + off;
    ta.vb = a.v + off;
    return ta;
  };
  auto clamp_row = [&](int pos0, int row) {
    const int p = min(max(pos0 + row, sr.lo), sr.L - 1);
    return p - pos0;
  };

  constexpr bool ROWK = kRowKeys<KFV, BF16>;
  // whole-row key fetch: instruction c takes the 1 KiB of tile rows
  // RPI*c .. RPI*c + RPI-1, lane l its 16-byte chunk l % NCH of row
  // RPI*c + l / NCH (KCH instructions either way: the same registers)
  constexpr int RPI = 1024 / ROW > 0 ? 1024 / ROW : 1;  // rows per load instruction
  auto krow_of = [&](int c) { return RPI * c + lane / NCH; };
  u32x4 kreg[KCH];      // key row r of the tile, chunks 4t+j (ROWK: the raw rows)
  u32x4 vreg[4][VBLK];  // value rows 4j+i of the tile, chunks r+16*blk
  auto load_k = [&](const TileAt& ta) {
    if constexpr (ROWK || STAGED) {
      static_assert(KCH * 64 * 16 == kTile * ROW, "whole-row key fetch: one register per chunk");
#pragma unroll
      for (int c = 0; c < KCH; ++c)
        kreg[c] = load16_stream(ta.kb + (size_t)clamp_row(ta.pos0, krow_of(c)) * POS +
                                16 * (lane % NCH));
    } else {
      const char* row = ta.kb + (size_t)clamp_row(ta.pos0, r) * POS;
#pragma unroll
      for (int c = 0; c < KCH; ++c) kreg[c] = load16(row + (4 * c + j) * 16);
    }
  };
  // the raw key rows into the wave's LDS tile (row-major, ROW bytes a row,
  // chunk p of row q at p ^ stage_swz(q)); written a whole row range per
  // instruction, so the writes are free of bank conflicts
  auto stage_keys = [&]() {
    if constexpr (ROWK || STAGED) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int q = krow_of(c);
        *reinterpret_cast<u32x4*>(stage + q * ROW + 16 * ((lane % NCH) ^ stage_swz(q))) = kreg[c];
      }
    }
  };
  auto load_v = [&](const TileAt& ta) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* row = ta.vb + (size_t)clamp_row(ta.pos0, 4 * j + i) * POS;
#pragma unroll
      for (int blk = 0; blk < VBLK; ++blk)
        vreg[i][blk] = load16_stream(row + (r + 16 * blk) * 16);
    }
  };

  // Keys rebuilt from the value row in src: the lane's rotated pairs are
  // chunks t < TA (coordinates < 64) and their partners t + TP (+256).  The
  // result goes back into src.
  constexpr int TA = kRopePairs / (4 * E), TP = 256 / (4 * E);
  // bf16: the lane's entries of M (its row r, its E pairs of chunks t < TA)
  // do not change from tile to tile, so they are read once here and kept in
  // registers, which the register allocator parks in AGPRs (1.8% faster than
  // reading them per tile; f32 has no room and reads them per tile)
  f32x4 Mreg[STAGED ? TA : 1][STAGED ? E : 1];
  if constexpr (STAGED) {
#pragma unroll
    for (int t = 0; t < TA; ++t)
#pragma unroll
      for (int e = 0; e < E; ++e)
        Mreg[t][e] = *reinterpret_cast<const f32x4*>(rl->m[E * (4 * t + j) + e][r]);
  }
  auto rebuild_keys = [&](u32x4 (&src)[KCH]) {
    if constexpr (KFV) {
      const int wave = threadIdx.x >> 6;
#pragma unroll
      for (int t = 0; t < TA; ++t) {
        float va[E], vb[E];
        if constexpr (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            va[2 * q] = bf16_value(src[t][q] & 0xffffu);
            va[2 * q + 1] = bf16_value(src[t][q] >> 16);
            vb[2 * q] = bf16_value(src[t + TP][q] & 0xffffu);
            vb[2 * q + 1] = bf16_value(src[t + TP][q] >> 16);
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            va[e] = chunk_f32(src[t], e);
            vb[e] = chunk_f32(src[t + TP], e);
          }
        }
        // the table entries of the E pairs first, all reads in flight, then the
        // math (interleaving them serialises the LDS latency)
        f32x4 Mt[E];
        f32x4 Bt[E / 2];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if constexpr (STAGED) {
            Mt[e] = Mreg[t][e];
          } else {
            // the row index opaque to the optimizer, so these reads are not
            // hoisted out of the tile loop into registers f32 does not have
            int rr = r;
            asm volatile("" : "+v"(rr));
            Mt[e] = *reinterpret_cast<const f32x4*>(rl->m[E * (4 * t + j) + e][rr]);
          }
        }
#pragma unroll
        for (int e = 0; e < E; e += 2)
          Bt[e / 2] = *reinterpret_cast<const f32x4*>(rl->base[wave][E * (4 * t + j) + e]);
        #pragma unroll
        for (int e = 0; e < E; ++e) {
          const f32x4 M = Mt[e];
          const float bc = Bt[e / 2][2 * (e & 1)], bs = Bt[e / 2][2 * (e & 1) + 1];
          const float xa = M[0] * va[e] + M[1] * vb[e];
          const float xb = M[2] * va[e] + M[3] * vb[e];
          va[e] = bc * xa - bs * xb;
          vb[e] = bs * xa + bc * xb;
        }
        u32x4 ka, kb;
        if constexpr (BF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            ka[q] = bf16_pack2(va[2 * q], va[2 * q + 1]);
            kb[q] = bf16_pack2(vb[2 * q], vb[2 * q + 1]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            ka[e] = __builtin_bit_cast(unsigned, va[e]);
            kb[e] = __builtin_bit_cast(unsigned, vb[e]);
          }
        }
        src[t] = ka;
        src[t + TP] = kb;
      }
    }
  };
  // the QK^T operand chunk c of the lane (compile-time c)
  auto key_op = [&](int c) -> u32x4 {
    if constexpr (ROWK) {
      return *reinterpret_cast<const u32x4*>(stage + r * ROW + 16 * ((4 * c + j) ^ stage_swz(r)));
    } else {
      return kreg[c];
    }
  };

  TileAt cur = tile_at(0);
  load_k(cur);
  if constexpr (!STAGED) load_v(cur);
  if constexpr (KFV) rope_base(rl, threadIdx.x >> 6, cur.pos0);
#pragma unroll
  for (int i = 0; i < QPL; ++i) {
    const int c = lane + 64 * i;
    if (c < G * NCH) myq[(c / NCH) * NCH + ((c % NCH) ^ stage_swz(c / NCH))] = qstage[i];
  }
  // one wave writes and reads its own slice: a wavefront-scope fence orders them
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();

  // bf16 keys from values: the query operand is the same for every tile of the
  // unit, so it is read from LDS once into registers
  u32x4 qreg[STAGED ? KCH : 1];
  if constexpr (STAGED) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) qreg[c] = qrow[(4 * c + j) ^ qswz];
  }

  for (int it = 0; it < n_it; ++it) {
    const bool more = it + 1 < n_it;
    const TileAt nxt = more ? tile_at(it + 1) : cur;

    if constexpr (STAGED) {
      // stage the fetched rows, read the key operand (row r, chunks 4c+j)
      // back into the registers and rebuild its rotated chunks there; QK^T
      // reads them as they are, and the registers take the next tile's rows
      // after QK^T.  On the global B=32 paged call, same machine: 1,526-1,536
      // us; the tile fetched in the key layout directly (no LDS round trip
      // before the rebuild), 1,599-1,600; that fetch with the rebuilt chunks
      // in an LDS area of their own, QK^T reading its keys from LDS and the
      // registers refilled right after staging, 1,608.
      stage_keys();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const char* srow = stage + r * kStageRow;
#pragma unroll
      for (int c = 0; c < KCH; ++c)
        kreg[c] = *reinterpret_cast<const u32x4*>(srow + 16 * ((4 * c + j) ^ stage_swz(r)));
      rebuild_keys(kreg);
    } else if constexpr (ROWK) {
      // this tile's key rows into the wave's LDS tile, then the registers
      // take the next tile's rows at once (fetched a whole QK^T earlier)
      stage_keys();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (more) load_k(nxt);
    } else {
      rebuild_keys(kreg);
    }

    // logits z[pos 4j+i][head r]
    f32x4 z;
    {
      f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
#pragma unroll
        for (int c = 0; c < KCH; c += 2) {
          // columns >= G: zero (stored-key kernels, HBM-bound: a branch around
          // the read costs nothing and the registers are full) or head 0
          // (keys from values, compute-bound)
          u32x4 q0, q1;
          if constexpr (STAGED) {
            q0 = qreg[c];
            q1 = qreg[c + 1];
          } else {
            q0 = KFV || r < G ? qrow[(4 * c + j) ^ qswz] : u32x4{0u, 0u, 0u, 0u};
            q1 = KFV || r < G ? qrow[(4 * c + 4 + j) ^ qswz] : u32x4{0u, 0u, 0u, 0u};
          }
          z0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, key_op(c)),
                                                       __builtin_bit_cast(bf16x8, q0), z0, 0, 0, 0);
          z1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, key_op(c + 1)),
                                                       __builtin_bit_cast(bf16x8, q1), z1, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
          const u32x4 qc = KFV || r < G ? qrow[(4 * c + j) ^ qswz] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            z0 = __builtin_amdgcn_mfma_f32_16x16x4f32(chunk_f32(kreg[c], e), chunk_f32(qc, e), z0,
                                                      0, 0, 0);
            z1 = __builtin_amdgcn_mfma_f32_16x16x4f32(chunk_f32(kreg[c], e + 1),
                                                      chunk_f32(qc, e + 1), z1, 0, 0, 0);
          }
        }
      }
      z = z0 + z1;
    }
    if constexpr (STAGED) {
      // the key registers are free: fetch the next tile; the staging writes
      // are complete before the value reads
      if (more) load_k(nxt);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // value operands: rows 4j+i (clamped as when fetched), chunks r+16*blk
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int blk = 0; blk < VBLK; ++blk)
          vreg[i][blk] = *reinterpret_cast<const u32x4*>(
              stage + (4 * j + i) * kStageRow + 16 * ((r ^ stage_swz(4 * j + i)) + 16 * blk));
    } else if constexpr (!ROWK) {
      // the key registers are free: fetch the next tile's keys
      if (more) load_k(nxt);
    }
    if constexpr (KFV) {
      if (more) {
        // the base of the next tile (this tile's rebuilt keys no longer read it)
        rope_base(rl, threadIdx.x >> 6, nxt.pos0);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = cur.pos0 + 4 * j + i;
      if (!(cur.ok && p >= sr.lo && p < sr.L)) z[i] = -INFINITY;
    }

    // online softmax (fp32)
    float tmax = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool grow = tmax > st.m + kRescaleGap;  // also when m = -inf and tmax is finite
    if (__any(grow)) {
      const float m_next = grow ? tmax : st.m;
      const float alpha = exp2_fast((st.m - (m_next == -INFINITY ? 0.f : m_next)) * kLog2e);
      if (grow) {
        st.l *= alpha;
#pragma unroll
        for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
          for (int e = 0; e < E; ++e) st.acc[blk][e] *= alpha;
      }
      st.m = m_next;
    }
    const float m_use = st.m == -INFINITY ? 0.f : st.m;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2_fast((z[i] - m_use) * kLog2e);

    if constexpr (BF16) {
      const unsigned p01 = bf16_pack2(p[0], p[1]), p23 = bf16_pack2(p[2], p[3]);
      st.l += (bf16_value(p01 & 0xffffu) + bf16_value(p01 >> 16)) +
              (bf16_value(p23 & 0xffffu) + bf16_value(p23 >> 16));
      const s16x4 pt = __builtin_bit_cast(s16x4, u32x2{p01, p23});
#pragma unroll
      for (int blk = 0; blk < VBLK; ++blk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const int dw = e >> 1;
          const unsigned lo = __builtin_amdgcn_perm(vreg[1][blk][dw], vreg[0][blk][dw], sel);
          const unsigned hi = __builtin_amdgcn_perm(vreg[3][blk][dw], vreg[2][blk][dw], sel);
          const s16x4 vt = __builtin_bit_cast(s16x4, u32x2{lo, hi});
          st.acc[blk][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pt, st.acc[blk][e], 0, 0, 0);
        }
      }
    } else {
      st.l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st.acc[blk][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(chunk_f32(vreg[i][blk], e), p[i],
                                                                  st.acc[blk][e], 0, 0, 0);
    }
    // the value registers are free: fetch the next tile's values
    if constexpr (!STAGED) {
      if (more) load_v(nxt);
    }
    if constexpr (PAGED) {
      if (it + 1 - it0 == 64) {
        it0 += 64;
        pg_cur = pg_nxt;
        pg_nxt = it0 + 64 + lane < n_it ? bt[k_begin + step * (it0 + 64 + lane)] : 0;
      }
    }
    cur = nxt;
  }
  // the lane's share of l summed over the 4 lanes of its column
  st.l = sum_lanes_xor16_32(st.l);
}

// Writes the wave's unnormalised O row of head r as fp32 (same ownership).
template <int KV, int D, bool BF16>
__device__ __forceinline__ void store_partial(const WaveState<KV, D, BF16>& st, float* ws_row) {
  using Gm = Geo<KV, D, BF16>;
  constexpr int E = Gm::E, VBLK = Gm::VBLK;
  const int j = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int blk = 0; blk < VBLK; ++blk) {
    float* dst = ws_row + 16 * E * blk + 4 * E * j;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < E; e += 4)
        *reinterpret_cast<f32x4*>(dst + E * i + e) =
            f32x4{st.acc[blk][e][i], st.acc[blk][e + 1][i], st.acc[blk][e + 2][i], st.acc[blk][e + 3][i]};
  }
}

// Tile counts of every sequence (s_cnt: tiles per unit), their lengths and
// the exclusive prefix sums of the counts (s_before[B]: the total), in LDS;
// work-group 0 also writes the prefix times KV to a.prefix for the combine.
// Called by wave 0 (lane l takes sequences 4l .. 4l+3); the caller then syncs.
template <int KV>
__device__ inline void tile_prefix(const KernelArgs& a, int* s_len, int* s_cnt, int* s_before) {
  const int lane = threadIdx.x & 63;
  int cnt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * lane + i;
    const int L = b < a.B ? a.seq_lens[b] : 0;
    cnt[i] = seq_range(L, position_cap(a.cap, a.ring), a.window).n;
    if (b < a.B) {
      s_len[b] = L;
      s_cnt[b] = cnt[i];
    }
  }
  const int lsum = cnt[0] + cnt[1] + cnt[2] + cnt[3];
  // inclusive scan over the lanes: within each 16-lane row by DPP row shifts
  // (lanes below the shift read 0), then the totals of the rows below added
  int incl = lsum;
  incl += row_shr<1>(incl);
  incl += row_shr<2>(incl);
  incl += row_shr<4>(incl);
  incl += row_shr<8>(incl);
  {
    const int r0 = __builtin_amdgcn_readlane(incl, 15);
    const int r1 = __builtin_amdgcn_readlane(incl, 31);
    const int r2 = __builtin_amdgcn_readlane(incl, 47);
    const int row = lane >> 4;
    incl += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
  }
  int run_b = incl - lsum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = 4 * lane + i;
    if (b < a.B) {
      s_before[b] = run_b;
      if (blockIdx.x == 0) a.prefix[b] = KV * run_b;
    }
    run_b += cnt[i];
  }
  if (lane == 63) {
    s_before[a.B] = incl;
    if (blockIdx.x == 0) a.prefix[a.B] = KV * incl;
  }
}

// ---- stream kernel: W persistent waves, each an equal slice of all tiles
template <int KV, int D, bool PAGED, bool BF16, bool KFV>
__global__ __launch_bounds__(kThreads, (main_waves_per_simd<KV, BF16>())) void gqa_stream_kernel(
    KernelArgs a) {
  using Gm = Geo<KV, D, BF16>;
  constexpr int G = Gm::G, ROW = Gm::ROW, NCH = Gm::NCH;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int j = lane >> 4;
  const int w = blockIdx.x * kWaves + (threadIdx.x >> 6);  // this wave's slice

  // ---- tile counts of every sequence and their prefix sums, once per
  // work-group in LDS (wave 0: lane l takes sequences 4l .. 4l+3)
  __shared__ int s_len[kMaxBatch];         // seq_lens
  __shared__ int s_cnt[kMaxBatch];         // tiles per unit of the sequence
  __shared__ int s_before[kMaxBatch + 1];  // tiles per unit summed over earlier sequences
  __shared__ u32x4 s_q[kWaves][G * NCH];   // per-wave query heads of the current unit
  __shared__ std::conditional_t<KFV, RopeLds, int> s_rope_buf;
  RopeLds* s_rope = KFV ? reinterpret_cast<RopeLds*>(&s_rope_buf) : nullptr;
  constexpr int SB = wave_stage_bytes<KFV, BF16, ROW>();  // per wave
  __shared__ __attribute__((aligned(16))) char s_stage[SB > 0 ? kWaves * SB : 16];
  char* stage = SB > 0 ? s_stage + (threadIdx.x >> 6) * SB : nullptr;
  if constexpr (KFV) rope_tables_init<BF16>(a.w_k, s_rope);
  if (threadIdx.x < 64) tile_prefix<KV>(a, s_len, s_cnt, s_before);
  __syncthreads();
  const long T = (long)KV * s_before[a.B];  // tiles of all units

  // ---- this wave's slice [s_begin, s_end) of the flattened tiles
  const int W = effective_waves(T, a.n_waves);
  if (w >= W) return;
  const long s_begin = floor_div((long)w * T, W);
  const long s_end = floor_div((long)(w + 1) * T, W);
  if (s_begin >= s_end) return;

  // the sequence holding s_begin: the last one whose first tile is <= s_begin
  int b = 0;
  {
    int lo_b = 0, hi_b = a.B - 1;
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if ((long)KV * s_before[mid] <= s_begin) lo_b = mid;
      else hi_b = mid - 1;
    }
    b = lo_b;
  }
  int n = s_cnt[b];
  int g, kk0;
  {
    const int rel = (int)(s_begin - (long)KV * s_before[b]);
    g = rel / n;
    kk0 = rel % n;
  }

  WaveState<KV, D, BF16> st;
  long t = s_begin;
  while (t < s_end) {
    // ---- one segment: tiles [k_begin, k_end) of unit (b, g)
    const SeqRange sr = seq_range(s_len[b], position_cap(a.cap, a.ring), a.window);
    const int k_begin = kk0;
    const int k_end = (int)min((long)n, (long)k_begin + (s_end - t));
    accumulate_tiles<KV, D, PAGED, BF16, KFV>(a, b, g, sr, k_begin, k_end, 1,
                                               s_q[threadIdx.x >> 6], s_rope, stage, st);

    // the wave writes o when its slice holds the whole unit, else a partial
    if (r < G) {
      if (k_begin == 0 && k_end == n) {
        const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
        store_o<KV, D, BF16>(st, a.o + ((size_t)b * kHeads + g * G + r) * ROW, inv);
      } else {
        const size_t slot = (size_t)(b * KV + g) + w;
        store_partial<KV, D, BF16>(st, a.ws_acc + (slot * G + r) * D);
        if (j == 0) *reinterpret_cast<f32x2*>(a.ws_ml + (slot * G + r) * 2) = f32x2{st.m, st.l};
      }
    }

    // ---- next unit (skipping sequences with nothing attended)
    t += k_end - k_begin;
    kk0 = 0;
    if (++g == KV) {
      g = 0;
      do {
        ++b;
      } while (b < a.B && s_cnt[b] == 0);
    }
    if (t < s_end) n = s_cnt[b];
  }
}

// The four waves' states of one unit (or unit piece) merged through LDS and
// written by all four waves, each a quarter of D: every wave stores its O rows
// and (m, l) (lanes r < G), then wave w folds the four rows on
// d in [wD/4, (w+1)D/4) with the common reference max.  Lane l of wave w takes
// the PER = G*D/256 consecutive values e0 = PER*l of that quarter's G x D/4
// block (head e0 / (D/4)).  Writes either o (whole unit: the merged row over
// the total weight, in the output dtype) or the unnormalised fp32 partial row
// and its (m, l) (the lane starting a head's quarter 0 writes the pair).
// s_acc holds 4 G rows of D + 4 floats, s_m and s_l 4 G floats; every wave of
// the work-group calls it (it holds a barrier, and a second one before the
// LDS rows may be reused).
template <int KV, int D, bool BF16>
__device__ __forceinline__ void merge_store_group(const WaveState<KV, D, BF16>& st, float* s_acc,
                                                  float* s_m, float* s_l, char* o_unit,
                                                  float* ws_acc_slot, float* ws_ml_slot) {
  using Gm = Geo<KV, D, BF16>;
  constexpr int G = Gm::G, E = Gm::E, VBLK = Gm::VBLK, EB = Gm::EB;
  constexpr int LROW = D + 4;  // padded LDS row (floats)
  constexpr int Q = D / kWaves;            // d values per wave
  constexpr int PER = G * Q / 64;          // values per lane
  static_assert(PER == 2 || PER % 4 == 0, "merge width");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int j = lane >> 4;
  if (r < G) {
    float* dst = s_acc + (wave * G + r) * LROW;
#pragma unroll
    for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) dst[16 * E * blk + 4 * E * j + E * i + e] = st.acc[blk][e][i];
    if (j == 0) {
      s_m[wave * G + r] = st.m;
      s_l[wave * G + r] = st.l;
    }
  }
  __syncthreads();
  const int e0 = PER * lane;
  const int h = e0 / Q;
  const int d = wave * Q + e0 % Q;
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) M = fmaxf(M, s_m[v * G + h]);
  const float Muse = M == -INFINITY ? 0.f : M;
  float sc[kWaves];
  float Lt = 0.f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    sc[v] = exp2_fast((s_m[v * G + h] - Muse) * kLog2e);
    Lt += sc[v] * s_l[v * G + h];
  }
  float x[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) x[k] = 0.f;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const float* row = s_acc + (v * G + h) * LROW + d;
#pragma unroll
    for (int k = 0; k < PER; ++k) x[k] += sc[v] * row[k];
  }
  if (o_unit != nullptr) {
    const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
    char* dst = o_unit + ((size_t)h * D + d) * EB;
    if constexpr (BF16) {
      if constexpr (PER == 2) {
        *reinterpret_cast<unsigned*>(dst) = bf16_pack2(x[0] * inv, x[1] * inv);
      } else {
#pragma unroll
        for (int c = 0; c < PER / 4; ++c)
          *reinterpret_cast<u32x2*>(dst + 8 * c) =
              u32x2{bf16_pack2(x[4 * c] * inv, x[4 * c + 1] * inv),
                    bf16_pack2(x[4 * c + 2] * inv, x[4 * c + 3] * inv)};
      }
    } else {
      if constexpr (PER == 2) {
        *reinterpret_cast<f32x2*>(dst) = f32x2{x[0] * inv, x[1] * inv};
      } else {
#pragma unroll
        for (int c = 0; c < PER / 4; ++c)
          *reinterpret_cast<f32x4*>(dst + 16 * c) =
              f32x4{x[4 * c] * inv, x[4 * c + 1] * inv, x[4 * c + 2] * inv, x[4 * c + 3] * inv};
      }
    }
  } else {
    float* dst = ws_acc_slot + (size_t)h * D + d;
    if constexpr (PER == 2) {
      *reinterpret_cast<f32x2*>(dst) = f32x2{x[0], x[1]};
    } else {
#pragma unroll
      for (int c = 0; c < PER / 4; ++c)
        *reinterpret_cast<f32x4*>(dst + 4 * c) = f32x4{x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]};
    }
    if (wave == 0 && e0 % Q == 0) *reinterpret_cast<f32x2*>(ws_ml_slot + 2 * h) = f32x2{M, Lt};
  }
  __syncthreads();  // the rows are read before anyone reuses the LDS
}

// ---- unit kernel: one work-group per unit (many short units); its four
// waves take interleaved tiles and merge their states in LDS, then write o
template <int KV, int D, bool PAGED, bool BF16, bool KFV>
__global__ __launch_bounds__(kThreads, (main_waves_per_simd<KV, BF16>())) void gqa_unit_kernel(
    KernelArgs a) {
  using Gm = Geo<KV, D, BF16>;
  constexpr int G = Gm::G, ROW = Gm::ROW, NCH = Gm::NCH;
  constexpr int LROW = D + 4;  // padded LDS row (floats)
  __shared__ u32x4 s_q[kWaves][G * NCH];
  // the merge rows of the four waves; the staged path's per-wave tiles share the
  // space (every wave has left its tile loop before the merge writes)
  constexpr int SB = wave_stage_bytes<KFV, BF16, ROW>();  // per wave
  constexpr int ACC_BYTES = kWaves * G * LROW * 4;
  constexpr int POOL = kWaves * SB > ACC_BYTES ? kWaves * SB : ACC_BYTES;
  __shared__ __attribute__((aligned(16))) char s_pool[POOL];
  float* s_acc = reinterpret_cast<float*>(s_pool);
  __shared__ float s_m[kWaves * G];
  __shared__ float s_l[kWaves * G];
  __shared__ std::conditional_t<KFV, RopeLds, int> s_rope_buf;
  RopeLds* s_rope = KFV ? reinterpret_cast<RopeLds*>(&s_rope_buf) : nullptr;
  if constexpr (KFV) {
    rope_tables_init<BF16>(a.w_k, s_rope);
    __syncthreads();
  }

  const int wave = threadIdx.x >> 6;
  const int r = threadIdx.x & 15;
  const int unit = blockIdx.x;
  const int b = unit / KV;
  const int g = unit % KV;
  const SeqRange sr = seq_range(a.seq_lens[b], position_cap(a.cap, a.ring), a.window);
  if (sr.n == 0) {  // nothing attended: zero rows
    for (int c = threadIdx.x; c < G * NCH; c += kThreads)
      *reinterpret_cast<u32x4*>(a.o + ((size_t)b * kHeads + g * G + c / NCH) * ROW + (c % NCH) * 16) =
          u32x4{0u, 0u, 0u, 0u};
    return;
  }

  WaveState<KV, D, BF16> st;
  accumulate_tiles<KV, D, PAGED, BF16, KFV>(a, b, g, sr, wave, sr.n, kWaves, s_q[wave], s_rope,
                                            SB > 0 ? s_pool + wave * SB : nullptr, st);
  if constexpr (SB > 0) __syncthreads();  // the tiles are dead before s_acc is written

  merge_store_group<KV, D, BF16>(st, s_acc, s_m, s_l, a.o + ((size_t)b * kHeads + g * G) * ROW,
                                 nullptr, nullptr);
}

// ---- group kernel: the stream partition over work-groups
// Work-group w takes the equal slice [w*T/NG, (w+1)*T/NG) of the flattened
// tiles; its four waves share each unit piece of the slice tile by tile (wave
// i takes the piece's tiles i, i+4, ...) and merge their states in LDS.  A
// piece that is a whole unit writes o; otherwise the work-group writes the
// merged partial to slot unit + w, and the combine kernel merges the
// partials as in stream mode (with the work-groups in the place of the
// waves).  A work-group's partial stands for four waves' tiles, so the
// workspace traffic is a quarter of stream mode's at the same parallelism.

// Work-groups that share the T tiles of a grouped call: the NG launched, or
// fewer when the lengths give fewer than kWaves tiles per work-group (every
// remaining slice then holds at least one tile).
__device__ inline int effective_groups(long T, int NG) {
  const long need = (T + kWaves - 1) / kWaves;
  return need < NG ? (int)(need > 1 ? need : 1) : NG;
}

template <int KV, int D, bool PAGED, bool BF16, bool KFV>
__global__ __launch_bounds__(kThreads, (main_waves_per_simd<KV, BF16>())) void gqa_group_kernel(
    KernelArgs a) {
  using Gm = Geo<KV, D, BF16>;
  constexpr int G = Gm::G, ROW = Gm::ROW, NCH = Gm::NCH;
  constexpr int LROW = D + 4;  // padded LDS row (floats)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int j = lane >> 4;
  const int grp = blockIdx.x;

  __shared__ int s_len[kMaxBatch];
  __shared__ int s_cnt[kMaxBatch];
  __shared__ int s_before[kMaxBatch + 1];
  __shared__ u32x4 s_q[kWaves][G * NCH];
  // the per-wave tiles and the merge rows of the four waves share the space (the
  // tile loops of a piece end before its merge writes, and a barrier ends
  // the merge before the next piece's tiles)
  constexpr int SB = wave_stage_bytes<KFV, BF16, ROW>();  // per wave
  constexpr int ACC_BYTES = kWaves * G * LROW * 4;
  constexpr int POOL = kWaves * SB > ACC_BYTES ? kWaves * SB : ACC_BYTES;
  __shared__ __attribute__((aligned(16))) char s_pool[POOL];
  float* s_acc = reinterpret_cast<float*>(s_pool);
  __shared__ float s_m[kWaves * G];
  __shared__ float s_l[kWaves * G];
  __shared__ std::conditional_t<KFV, RopeLds, int> s_rope_buf;
  RopeLds* s_rope = KFV ? reinterpret_cast<RopeLds*>(&s_rope_buf) : nullptr;
  if constexpr (KFV) rope_tables_init<BF16>(a.w_k, s_rope);
  if (threadIdx.x < 64) tile_prefix<KV>(a, s_len, s_cnt, s_before);
  __syncthreads();
  const long T = (long)KV * s_before[a.B];  // tiles of all units

  // (sequences with nothing attended get their zero rows from the combine)
  if (T == 0) return;
  const int NG = effective_groups(T, a.n_waves / kWaves);
  const TailPlan tp = tail_plan(T, a.dyn);

  // tiles [s_begin, s_end) of the flattened sequence (slice sl), unit piece by
  // unit piece
  auto run_range = [&](long s_begin, long s_end, int sl) {
    // the sequence holding s_begin: the last one whose first tile is <= s_begin
    int b = 0;
    {
      int lo_b = 0, hi_b = a.B - 1;
      while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if ((long)KV * s_before[mid] <= s_begin) lo_b = mid;
        else hi_b = mid - 1;
      }
      b = lo_b;
    }
    int n = s_cnt[b];
    int g, kk0;
    {
      const int rel = (int)(s_begin - (long)KV * s_before[b]);
      g = rel / n;
      kk0 = rel % n;
    }

    long t = s_begin;
    while (t < s_end) {
      // ---- one piece: tiles [k_begin, k_end) of unit (b, g), shared by the waves
      const SeqRange sr = seq_range(s_len[b], position_cap(a.cap, a.ring), a.window);
      const int k_begin = kk0;
      const int k_end = (int)min((long)n, (long)k_begin + (s_end - t));
      WaveState<KV, D, BF16> st;
      accumulate_tiles<KV, D, PAGED, BF16, KFV>(a, b, g, sr, k_begin + wave, k_end, kWaves,
                                                s_q[wave], s_rope,
                                                SB > 0 ? s_pool + wave * SB : nullptr, st);
      if constexpr (SB > 0) __syncthreads();  // the tiles are dead before s_acc is written
      // a whole unit writes o; a piece writes the work-group's partial to slot
      // unit + sl (the merge ends on a barrier: its LDS rows may then be reused)
      const size_t slot = (size_t)(b * KV + g) + sl;
      merge_store_group<KV, D, BF16>(
          st, s_acc, s_m, s_l,
          k_begin == 0 && k_end == n ? a.o + ((size_t)b * kHeads + g * G) * ROW : nullptr,
          a.ws_acc + slot * G * D, a.ws_ml + slot * G * 2);

      // ---- next unit (skipping sequences with nothing attended)
      t += k_end - k_begin;
      kk0 = 0;
      if (++g == KV) {
        g = 0;
        do {
          ++b;
        } while (b < a.B && s_cnt[b] == 0);
      }
      if (t < s_end) n = s_cnt[b];
    }
  };
  if (grp < NG) run_range(floor_div((long)grp * tp.S, NG), floor_div((long)(grp + 1) * tp.S, NG), grp);
  if (tp.nch > 0) {
    // the dynamic tail: chunks from the counter until none is left (one lane
    // takes the ticket; a value outside [0, nch) ends the loop)
    __shared__ int s_chunk;
    for (;;) {
      __syncthreads();  // every wave has read the last ticket
      if (threadIdx.x == 0) s_chunk = atomicAdd(a.counter, 1);
      __syncthreads();
      const int c = s_chunk;
      if (c < 0 || c >= tp.nch) break;
      run_range(tp.S + (long)c * tp.C, tp.S + (long)(c + 1) * tp.C, NG + c);
    }
  }
}

struct CombineArgs {
  const int32_t* prefix;
  const float* ws_ml;
  const float* ws_acc;
  char* o;
  int32_t B;
  int32_t n_waves;  // stream mode: the main kernel's waves; group mode: its work-groups
  int32_t groups;   // nonzero in group mode (slices per work-group, not per wave)
  int32_t dyn;      // group mode: the main kernel's dyn (its tail_plan)
};

// One work-group of CW waves (8, or 4 when that many work-groups would not
// fit the part in one round) per (sequence, query head, d part):
// the head's D values are cut into DS parts of D/DS (DS > 1 when there are
// few sequences, so that more work-groups share the reads).  Wave w merges the
// partials w, w + CW, ... of the unit: lane l owns PER = D/(64 DS)
// consecutive d values of the part, with U partials in flight (more for
// narrower lanes).  The waves' sums are then added in LDS in wave order.  The
// first batch of partial rows is loaded together with the (m, l) pairs the
// reference max needs, since those loads do not depend on it.  A unit held by
// one slice was written by its wave; a sequence with nothing attended gets a
// zero row.
constexpr int kCombineWavesMax = 8;
// work-groups of eight waves one combine launch may hold before it takes
// four-wave groups: about one round over 256 CUs at the kernel's occupancy
constexpr int kCombineWideGroups = 512;

// PER consecutive floats at p (16-, 8- or 4-byte aligned as PER asks)
template <int PER>
__device__ __forceinline__ void load_floats(const float* p, float (&v)[PER]) {
  if constexpr (PER % 4 == 0) {
#pragma unroll
    for (int c = 0; c < PER / 4; ++c) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(p + 4 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * c + e] = t[e];
    }
  } else if constexpr (PER == 2) {
    const f32x2 t = *reinterpret_cast<const f32x2*>(p);
    v[0] = t[0];
    v[1] = t[1];
  } else {
    static_assert(PER == 1, "lane width");
    v[0] = *p;
  }
}

template <int KV, int D, bool BF16, int DS, int CW>
__global__ __launch_bounds__(64 * CW) void gqa_combine_kernel(CombineArgs a) {
  constexpr int G = kHeads / KV;
  constexpr int EB = Elem<BF16>::bytes;
  constexpr int DW = D / DS;   // d values of this work-group
  constexpr int PER = DW / 64;  // d values per lane
  static_assert(PER == 1 || PER == 2 || PER % 4 == 0, "lane width");
  // partials in flight per lane: a batch is one round trip, so narrow lanes
  // take more of them (about 64 registers of partial rows either way)
  constexpr int U = PER >= 4 ? 8 : 16;
  __shared__ __attribute__((aligned(16))) float s_acc[CW][DW];
  __shared__ float s_l[CW];
  const int bh = blockIdx.x / DS;
  const int part = blockIdx.x % DS;
  const int b = bh / kHeads;
  const int h = bh % kHeads;
  const int g = h / G;
  const int hh = h % G;
  const int unit = b * KV + g;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int dl = lane * PER;        // within the part
  const int d = part * DW + dl;     // within the head row
  char* dst = a.o + ((size_t)b * kHeads + h) * D * EB + (size_t)d * EB;

  auto store = [&](const float (&run)[PER]) {
    if constexpr (BF16) {
      if constexpr (PER == 1) {
        *reinterpret_cast<unsigned short*>(dst) = (unsigned short)(bf16_pack2(run[0], 0.f) & 0xffffu);
      } else {
#pragma unroll
        for (int c = 0; c < PER; c += 2)
          *reinterpret_cast<unsigned*>(dst + c * EB) = bf16_pack2(run[c], run[c + 1]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < PER; ++c) *reinterpret_cast<float*>(dst + c * EB) = run[c];
    }
  };

  const int P0 = a.prefix[b];
  const int n = (a.prefix[b + 1] - P0) / KV;
  const long T = a.prefix[a.B];
  if (n <= 0) {
    if (wave == 0) {
      float zero[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) zero[e] = 0.f;
      store(zero);
    }
    return;
  }
  const long s0 = P0 + (long)g * n;
  const int W = a.groups ? effective_groups(T, a.n_waves) : effective_waves(T, a.n_waves);
  const TailPlan tp = tail_plan(T, a.groups ? a.dyn : 0);
  const int wf = slice_of(s0, tp, W);
  const int wl = slice_of(s0 + n - 1, tp, W);
  if (wf == wl) return;  // written by the wave that held the whole unit
  const int ns = wl - wf + 1;
  const f32x2* ml = reinterpret_cast<const f32x2*>(a.ws_ml) + ((size_t)unit + wf) * G + hh;
  const float* accp = a.ws_acc + (((size_t)unit + wf) * G + hh) * D + d;
  const size_t sstride = (size_t)G * D;
  // waves between wf and wl whose slices are empty (more waves than tiles)
  // wrote nothing: their slots are skipped.  With at least as many tiles as
  // waves every slice holds a tile; otherwise slice w = [wS/W, (w+1)S/W) is
  // tested with double divisions, exact here: (w+1)S < 2^53 is exact, the
  // quotient is correctly rounded, and a quotient that is not an integer lies
  // at least 1/W from one.  Every chunk of a dynamic tail holds C tiles.
  const bool all_hold = tp.S >= W;
  const double Td = (double)tp.S, Wd = (double)W;
  auto holds = [&](int s) {
    if (all_hold || wf + s >= W) return true;
    const double w = (double)(wf + s);
    return floor((w + 1.0) * Td / Wd) > floor(w * Td / Wd);
  };

  float x[U][PER];
  f32x2 e[U];
  bool okb[U];
  auto load_batch = [&](int s0u) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = s0u + CW * u;
      const int s = su < ns ? su : ns - 1;
      e[u] = ml[(size_t)s * G];
      okb[u] = su < ns && holds(s);
      load_floats<PER>(accp + (size_t)s * sstride, x[u]);
    }
  };
  load_batch(wave);

  // the reference max over the partials, lane-parallel in every wave
  float M = -INFINITY;
  for (int s = lane; s < ns; s += 64) {
    if (!holds(s)) continue;
    const f32x2 y = ml[(size_t)s * G];
    if (y[1] > 0.f) M = fmaxf(M, y[0]);
  }
  M = max_wave(M);

  float A[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) A[i] = 0.f;
  float Lt = 0.f;
  auto accumulate = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a slot nothing wrote may hold anything: select, never multiply by 0
      const bool ok = okb[u] && e[u][1] > 0.f;
      const float wgt = ok ? exp2_fast((e[u][0] - M) * kLog2e) : 0.f;
      Lt += ok ? wgt * e[u][1] : 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) A[i] += ok ? wgt * x[u][i] : 0.f;
    }
  };
  accumulate();
  for (int s0u = wave + CW * U; s0u < ns; s0u += CW * U) {
    load_batch(s0u);
    accumulate();
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) s_acc[wave][dl + i] = A[i];
  if (lane == 0) s_l[wave] = Lt;
  __syncthreads();
  if (wave != 0) return;
  float L = 0.f;
  float run[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) run[i] = 0.f;
#pragma unroll
  for (int w = 0; w < CW; ++w) {
    L += s_l[w];
#pragma unroll
    for (int i = 0; i < PER; ++i) run[i] += s_acc[w][dl + i];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) run[i] = L > 0.f ? run[i] * inv : 0.f;
  store(run);
}

// d parts per (sequence, head) of the combine: enough work-groups to spread
// the partial reads over the CUs (at least 256 when D allows it; one lane
// per d at most).  With 1024 groups of one float per lane, a global call of 4
// sequences spent 12.8 us in its combine, more than one sequence's 256
// groups merging four times the slices (8.6 us).
template <int D>
inline int combine_parts(int B) {
  int ds = 1;
  while (ds < D / 64 && (long)B * kHeads * ds < 256) ds *= 2;
  return ds;
}

// ------------------------------------------------------------- KV append
// The nodes between the projections and attn.core (Model Spec page,
// "Compute-graph nodes" table) for the new token of each sequence, at
// position pos = seq_lens[b] - 1:
//   q_out = rope(qk_norm(q_raw, w_q)), k_row = rope(qk_norm(k_raw, w_k)),
//   v_row = v_norm(v_raw) (global layers: values = keys, v_raw = k_raw);
//   qk_norm / v_norm: x / sqrt(mean(x^2) + 1e-6) (* w);
//   rope: rotate pairs (i, i + D/2) by pos * theta^(-2i/D) for i < active
//   (sliding theta 1e4, all 128 pairs; global theta 1e6, the first 64 pairs).
// k_row and v_row are written into the cache at pos.  Work-group (b, y) takes
// head rows 4y .. 4y+3 of sequence b (q heads, then k heads, then v heads),
// one row per wave, lane l holding elements [l*D/64, (l+1)*D/64), so the RoPE
// partner of a first-half element sits in lane l + 32; the group's cos/sin
// table is formed in double precision (angles reach 2.6e5 radians) in LDS.

struct AppendArgs {
  const char* q_raw;
  const char* k_raw;
  const char* v_raw;  // unused on global layers (values = keys)
  const char* w_q;
  const char* w_k;
  const int32_t* seq_lens;
  const int32_t* block_table;
  char* q_out;
  char* k_cache;  // nullptr: values-only cache (global layers), no key row
  char* v_cache;
  int32_t B;
  int32_t cap;
  int32_t max_pages;
  int32_t num_pages;
  int32_t ring;  // > 0: contiguous cache capped at `ring` positions (slot s % ring)
};

template <int N, bool BF16>
__device__ inline void load_elems(const char* p, float (&x)[N]) {
  if constexpr (BF16) {
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(p + 8 * c);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const unsigned d = w[q];
        x[4 * c + 2 * q] = bf16_value(d & 0xffffu);
        x[4 * c + 2 * q + 1] = bf16_value(d >> 16);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < N / 4; ++c) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(p + 16 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) x[4 * c + q] = w[q];
    }
  }
}

template <int N, bool BF16>
__device__ inline void store_elems(char* p, const float (&x)[N]) {
  if constexpr (BF16) {
#pragma unroll
    for (int c = 0; c < N / 4; ++c)
      *reinterpret_cast<u32x2*>(p + 8 * c) =
          u32x2{bf16_pack2(x[4 * c], x[4 * c + 1]),
                bf16_pack2(x[4 * c + 2], x[4 * c + 3])};
  } else {
#pragma unroll
    for (int c = 0; c < N / 4; ++c)
      *reinterpret_cast<f32x4*>(p + 16 * c) = f32x4{x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]};
  }
}

template <int KV, int D, bool PAGED, bool BF16>
__global__ __launch_bounds__(kThreads) void gqa_append_kernel(AppendArgs a) {
  constexpr bool GLOBAL = KV == 4;
  constexpr int H = D / 2;
  constexpr int N = D / 64;  // elements per lane
  constexpr int EB = Elem<BF16>::bytes;
  constexpr int ROW = D * EB;
  constexpr int ACTIVE = GLOBAL ? 64 : 128;
  constexpr double LOG2_THETA = GLOBAL ? 19.931568569324174 : 13.287712379549449;  // log2 1e6, 1e4
  constexpr int ROWS = kHeads + 2 * KV;  // q heads, then k heads, then v heads
  __shared__ float s_cos[H];
  __shared__ float s_sin[H];

  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int L = a.seq_lens[b];
  const bool live = L >= 1 && L <= position_cap(a.cap, a.ring);
  const int row = blockIdx.y * kWaves + wave;
  const int pos = L - 1;

  // destination of the new token's cache rows
  size_t row_off = 0;
  bool write_cache = live;
  if (live) {
    if constexpr (PAGED) {
      const int page = a.block_table[(size_t)b * a.max_pages + pos / kPage];
      write_cache = page >= 0 && page < a.num_pages;
      row_off = ((size_t)(write_cache ? page : 0) * kPage + pos % kPage) * KV * (size_t)ROW;
    } else {
      row_off = ((size_t)b * a.cap + (a.ring > 0 ? pos % a.ring : pos)) * KV * (size_t)ROW;
    }
  }

  for (int i = threadIdx.x; i < H; i += kThreads) {
    float c = 1.f, sn = 0.f;
    if (live && i < ACTIVE) {
      // theta^(-2i/D) and the angle in double, reduced to [-pi, pi] in double,
      // then an fp32 sin/cos of the reduced angle
      const double ang = (double)pos * exp2(-2.0 * i / D * LOG2_THETA);
      const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
      sincosf((float)red, &sn, &c);
    }
    s_cos[i] = c;
    s_sin[i] = sn;
  }
  __syncthreads();

  float wq[N], wk[N];
  load_elems<N, BF16>(a.w_q + (size_t)lane * N * EB, wq);
  load_elems<N, BF16>(a.w_k + (size_t)lane * N * EB, wk);

  if (row < ROWS) {
    const bool is_q = row < kHeads;
    const bool is_k = !is_q && row < kHeads + KV;
    if (is_k && a.k_cache == nullptr) return;  // values-only cache: no key row
    const int head = is_q ? row : (is_k ? row - kHeads : row - kHeads - KV);
    char* dst;
    const char* src;
    if (is_q) {
      src = a.q_raw + ((size_t)b * kHeads + head) * ROW;
      dst = a.q_out + ((size_t)b * kHeads + head) * ROW;
    } else {
      src = ((is_k || GLOBAL) ? a.k_raw : a.v_raw) + ((size_t)b * KV + head) * ROW;
      dst = (is_k ? a.k_cache : a.v_cache) + row_off + (size_t)head * ROW;
    }
    float y[N];
    if (!live) {
      // nothing to append: zero q rows, no cache write
#pragma unroll
      for (int e = 0; e < N; ++e) y[e] = 0.f;
      if (is_q) store_elems<N, BF16>(dst + (size_t)lane * N * EB, y);
      return;
    }
    float x[N];
    load_elems<N, BF16>(src + (size_t)lane * N * EB, x);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) ss += x[e] * x[e];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    const float inv = 1.f / sqrtf(ss / D + 1e-6f);
#pragma unroll
    for (int e = 0; e < N; ++e) y[e] = x[e] * inv * (is_q ? wq[e] : (is_k ? wk[e] : 1.f));
    if (is_q || is_k) {
      const bool first = lane < 32;
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float partner = __shfl_xor(y[e], 32);
        const int i = (lane & 31) * N + e;  // pair index
        const float c = s_cos[i], sn = s_sin[i];
        y[e] = first ? y[e] * c - partner * sn : y[e] * c + partner * sn;
      }
    }
    if (is_q || write_cache) store_elems<N, BF16>(dst + (size_t)lane * N * EB, y);
  }
}

// ------------------------------------------------------- measurement kernels
// Not part of the attention path: a plain read stream and a plain copy of a
// known byte count, used to measure the sustainable HBM read rate of the part
// and to calibrate a profiler's byte counters against the split kernels.  Each
// wave moves 8 KiB per iteration in 16-byte lanes (1 KiB contiguous per
// instruction).

constexpr int kProbeUnroll = 8;

// the dynamic tail's chunk counter to zero (lane 0 of one wave)
__global__ __launch_bounds__(64) void gqa_zero_counter_kernel(int32_t* counter) {
  if (threadIdx.x == 0) *counter = 0;
}

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* p, size_t n, unsigned* sink) {
  const size_t lane = threadIdx.x & 63;
  const size_t wave = (blockIdx.x * (size_t)blockDim.x + threadIdx.x) >> 6;
  const size_t n_waves = ((size_t)gridDim.x * blockDim.x) >> 6;
  unsigned acc = 0;
  for (size_t base = wave * 64 * kProbeUnroll; base < n; base += n_waves * 64 * kProbeUnroll) {
    u32x4 x[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const size_t i = base + (size_t)u * 64 + lane;
      x[u] = i < n ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
  }
  // data dependence on every load without a store per thread
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

__global__ __launch_bounds__(256) void hbm_copy_kernel(const u32x4* src, u32x4* dst, size_t n) {
  const size_t lane = threadIdx.x & 63;
  const size_t wave = (blockIdx.x * (size_t)blockDim.x + threadIdx.x) >> 6;
  const size_t n_waves = ((size_t)gridDim.x * blockDim.x) >> 6;
  for (size_t base = wave * 64 * kProbeUnroll; base < n; base += n_waves * 64 * kProbeUnroll) {
    u32x4 x[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const size_t i = base + (size_t)u * 64 + lane;
      if (i < n) x[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const size_t i = base + (size_t)u * 64 + lane;
      if (i < n) dst[i] = x[u];
    }
  }
}

// ---------------------------------------------------------------- host side
// ---------------------------------------------------------------- host side

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Launch plan, a function of (variant, B, capacity) only.  Enough short units
// fill the GPU one work-group per unit and need no workspace; otherwise the
// stream partition (over waves, or over work-groups on the global geometry)
// runs with workspace
//   [prefix: B+1 int32][ml: slots x G x 2 fp32][acc: slots x G x D fp32],
// slots = B*KV + W (a slice's partial of unit u sits in slot u + slice, W
// the waves or work-groups).
//
// Unit mode's time is set by its longest unit (a quarter of its tiles per
// wave, one after another), stream mode's by the bytes plus a combine, so
// unit mode needs more units the longer they are.  The tiers are measured
// (B uniform lengths, bf16):
//   - up to 320 tiles, from 1024 units: sliding windows 2048 / 4096 at B=256,
//     1,058 vs 1,105 and 1,791 vs 1,826 us; a 4096-position global cache at
//     B=256, 707 vs 722 us.  At 512 tiles it loses (window 8192: 2,481 vs
//     2,462; an 8192-position global cache: 1,495 vs 1,423 us), and at 256
//     tiles with 512 or 768 units it loses 3%;
//   - up to 128 tiles, from 256 units: global B=64 with a 2048-position
//     cache, 106 vs 113 us; sliding B=16, 37 vs 51 us.  Global B=32 with 128
//     tiles loses (87 vs 60 us);
//   - sliding geometry only, up to 65 tiles (one window), from 128 units:
//     sliding B=8, 27 vs 37 us.  Sliding B <= 4 loses (25 vs 16-23 us), and so
//     does global B=32 with a 1024-position cache (48.5 vs 43.8 us: its tiles
//     are twice the bytes, at one wave per SIMD).
constexpr int kUnitModeMinUnits = 1024;
constexpr int kUnitModeMaxTiles = 320;
inline bool unit_mode_fits(int units, int tiles_max, int D) {
  return (units >= kUnitModeMinUnits && tiles_max <= kUnitModeMaxTiles) ||
         (units >= 256 && tiles_max <= 128) || (D == 256 && units >= 128 && tiles_max <= 65);
}

// tiles (over all units, at the capacity) up to which a sliding call takes
// group mode
constexpr long kGroupSmallTiles = 2048;

struct Plan {
  int mode;  // GQA_MODE_UNIT, GQA_MODE_STREAM or GQA_MODE_GROUP
  int waves, slots;
  bool dyn;  // group mode with a dynamic tail (its counter zeroed before the launch)
  size_t prefix, counter, ml, acc, total;
};

// window: attended positions per sequence (0 = every position below L)
// Launch mode forced for measurement and tests (gqa_decode_force_mode), or -1
// for the planner's choice.
int g_force_mode = -1;

int make_plan(int variant, int B, int cap, int window, Plan* P) {
  VariantInfo vi;
  if (!variant_info(variant, &vi)) return GQA_ERR_DTYPE;
  if (B < 1 || B > kMaxBatch || cap < 1 || cap > kMaxSeq) return GQA_ERR_SHAPE;
  if (window < 0 || window > kMaxSeq) return GQA_ERR_SHAPE;
  int tiles_max = (cap + kTile - 1) / kTile;
  if (window > 0) {
    const int wt = (window + kTile - 1) / kTile + 1;
    tiles_max = tiles_max < wt ? tiles_max : wt;
  }
  const int units = B * vi.KV;
  *P = Plan{};
  // split units: work-group slices on the global geometry, wave slices on
  // the sliding one (group mode against stream mode, back-to-back calls on one
  // machine: global B=4 25.9 against 28.4 us, B=1 320 against 327, B=32 and
  // the values-only call equal; sliding f32 B=4 34.0 against 31.0)
  // A tiny sliding call (at most kGroupSmallTiles tiles in all, e.g. one
  // sequence's window) is latency-bound: group mode's LDS merge leaves a
  // quarter of the partials for the combine (one sequence of 262,144
  // positions, graph replay on one machine: 11.45 against 11.95 us per call).
  const bool tiny = (long)units * tiles_max <= kGroupSmallTiles;
  int mode = unit_mode_fits(units, tiles_max, vi.D)
                 ? GQA_MODE_UNIT
                 : (variant == GQA_GLOBAL || tiny ? GQA_MODE_GROUP : GQA_MODE_STREAM);
  if (g_force_mode >= 0) mode = g_force_mode;
  if (mode == GQA_MODE_UNIT) {
    P->mode = GQA_MODE_UNIT;
    P->waves = units * kWaves;
    return GQA_OK;
  }
  const int G = kHeads / vi.KV;
  P->mode = mode;
  P->waves = vi.waves;
  P->slots = units + (mode == GQA_MODE_GROUP ? vi.waves / kWaves : vi.waves);
  // a dynamic tail when the call may hold enough tiles (tail_plan decides on
  // the actual count); its chunks add up to kDynMaxChunks slots
  P->dyn = mode == GQA_MODE_GROUP && (long)units * tiles_max >= kDynMinTiles;
  if (P->dyn) P->slots += kDynMaxChunks;
  P->prefix = 0;
  P->counter = (size_t)(B + 1) * sizeof(int32_t);
  P->ml = align256(P->counter + sizeof(int32_t));
  P->acc = P->ml + align256((size_t)P->slots * G * 2 * sizeof(float));
  P->total = P->acc + (size_t)P->slots * G * vi.D * sizeof(float);
  return GQA_OK;
}

// ---- the workspace of the allocation-free entry point
// gqa_decode_global_paged_noalloc runs with this file-scope array as its
// workspace, for callers that cannot allocate device memory.  Its size is the
// workspace of the largest batch the global geometry accepts (B = 256 in
// stream mode: 1,280 + 131,072 + 33,554,432 bytes), rounded up to 33 MiB.
// Each device that loads the library holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = GQA_NOALLOC_SCRATCH_BYTES;
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream), looked up with that device current on the first call
// and kept; nullptr on a HIP error.
void* scratch_address(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// ---- launch timing (measurement only)
struct ProfRec {
  int kind;
  hipEvent_t start, stop;
};
std::vector<ProfRec> g_prof;
size_t g_prof_used = 0;
bool g_prof_on = false;

inline ProfRec* prof_slot(int kind) {
  if (!g_prof_on || g_prof_used >= g_prof.size()) return nullptr;
  ProfRec* r = &g_prof[g_prof_used++];
  r->kind = kind;
  return r;
}

typedef void (*MainFn)(KernelArgs);
typedef void (*CombineFn)(CombineArgs);

template <int KV, int D, bool KFV>
MainFn pick_main(int mode, bool paged, bool bf16) {
  if (mode == GQA_MODE_UNIT) {
    if (paged)
      return bf16 ? gqa_unit_kernel<KV, D, true, true, KFV> : gqa_unit_kernel<KV, D, true, false, KFV>;
    return bf16 ? gqa_unit_kernel<KV, D, false, true, KFV> : gqa_unit_kernel<KV, D, false, false, KFV>;
  }
  if (mode == GQA_MODE_GROUP) {
    if (paged)
      return bf16 ? gqa_group_kernel<KV, D, true, true, KFV> : gqa_group_kernel<KV, D, true, false, KFV>;
    return bf16 ? gqa_group_kernel<KV, D, false, true, KFV> : gqa_group_kernel<KV, D, false, false, KFV>;
  }
  if (paged)
    return bf16 ? gqa_stream_kernel<KV, D, true, true, KFV> : gqa_stream_kernel<KV, D, true, false, KFV>;
  return bf16 ? gqa_stream_kernel<KV, D, false, true, KFV> : gqa_stream_kernel<KV, D, false, false, KFV>;
}

template <int KV, int D, int DS>
CombineFn pick_combine_ds(bool bf16, int cw) {
  if (cw == kCombineWavesMax)
    return bf16 ? gqa_combine_kernel<KV, D, true, DS, kCombineWavesMax>
                : gqa_combine_kernel<KV, D, false, DS, kCombineWavesMax>;
  return bf16 ? gqa_combine_kernel<KV, D, true, DS, kCombineWavesMax / 2>
              : gqa_combine_kernel<KV, D, false, DS, kCombineWavesMax / 2>;
}

template <int KV, int D>
CombineFn pick_combine(bool bf16, int ds, int cw) {
  switch (ds) {
    case 1: return pick_combine_ds<KV, D, 1>(bf16, cw);
    case 2: return pick_combine_ds<KV, D, 2>(bf16, cw);
    case 4: return pick_combine_ds<KV, D, 4>(bf16, cw);
    default:
      if constexpr (D / 64 >= 8) return pick_combine_ds<KV, D, 8>(bf16, cw);
      return nullptr;
  }
}

// waves per combine work-group: eight while the launch holds at most
// kCombineWideGroups work-groups, four above (so that it stays about one
// round: eight-wave groups over 1024 (sequence, head, part) rows took two)
inline int combine_waves(int groups) {
  return groups <= kCombineWideGroups ? kCombineWavesMax : kCombineWavesMax / 2;
}

inline int default_window(int variant) { return variant == GQA_SLIDING ? kSlidingWindow : 0; }

// Profiling kinds: 2*variant main, 2*variant+1 combine, 4+variant append; the
// global layers over a values-only cache: 6 main, 7 combine, 8 append.
constexpr int kProfKeysFromValues = 6;

// w_k != nullptr: global layers over a values-only cache (k unused, keys
// rebuilt from v)
// ring > 0: sliding layers over a contiguous cache capped at `ring` positions
// (S_max = ring; 16 <= ring <= 262144, a multiple of 16, window <= ring)
int run(int variant, int window, bool paged, const void* q, const void* k, const void* v,
        const void* w_k, const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens,
        void* o, int32_t B, int32_t S_max, int32_t num_pages, int32_t dtype, void* workspace,
        size_t workspace_bytes_given, void* stream_, int32_t ring = 0,
        bool workspace_from_scratch = false) {
  const bool kfv = w_k != nullptr;
  if (kfv && variant != GQA_GLOBAL) return GQA_ERR_DTYPE;
  if (!q || (!k && !kfv) || !v || !seq_lens || !o || (paged && !block_table)) return GQA_ERR_NULL;
  if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_DTYPE;
  if (B < 1 || B > kMaxBatch) return GQA_ERR_SHAPE;
  int cap;
  if (paged) {
    if (max_pages < 1 || max_pages > kMaxSeq / kPage || num_pages < 1) return GQA_ERR_SHAPE;
    cap = max_pages * kPage;
  } else {
    if (S_max < 1 || S_max > kMaxSeq) return GQA_ERR_SHAPE;
    cap = S_max;
  }
  if (ring != 0) {
    if (variant != GQA_SLIDING || kfv || paged) return GQA_ERR_DTYPE;
    if (ring < kTile || ring > kMaxSeq || ring % kTile != 0 || ring != S_max) return GQA_ERR_SHAPE;
    if (window < 1 || window > ring) return GQA_ERR_SHAPE;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(w_k))
    return GQA_ERR_ALIGN;
  VariantInfo vi;
  variant_info(variant, &vi);
  Plan plan;
  int rc = make_plan(variant, B, ring ? kMaxSeq : cap, window, &plan);
  if (rc) return rc;
  const bool unit_mode = plan.mode == GQA_MODE_UNIT;
  const bool group_mode = plan.mode == GQA_MODE_GROUP;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  if (!unit_mode) {
    if (workspace_from_scratch) {
      // every host check above has passed: only now is HIP asked for the array
      if (plan.total > kScratchBytes) return GQA_ERR_WORKSPACE;
      workspace = scratch_address(stream);
      if (workspace == nullptr) return GQA_ERR_HIP;
      workspace_bytes_given = kScratchBytes;
    }
    if (!workspace || workspace_bytes_given < plan.total) return GQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return GQA_ERR_ALIGN;
  }
  const bool bf16 = dtype == GQA_BF16;
  char* ws = static_cast<char*>(workspace);

  KernelArgs ka;
  ka.q = static_cast<const char*>(q);
  ka.k = static_cast<const char*>(k);
  ka.v = static_cast<const char*>(v);
  ka.w_k = static_cast<const char*>(w_k);
  ka.seq_lens = seq_lens;
  ka.block_table = block_table;
  ka.o = static_cast<char*>(o);
  ka.prefix = unit_mode ? nullptr : reinterpret_cast<int32_t*>(ws + plan.prefix);
  ka.ws_ml = unit_mode ? nullptr : reinterpret_cast<float*>(ws + plan.ml);
  ka.ws_acc = unit_mode ? nullptr : reinterpret_cast<float*>(ws + plan.acc);
  ka.B = B;
  ka.cap = cap;
  ka.max_pages = paged ? max_pages : 0;
  ka.num_pages = paged ? num_pages : 0;
  ka.window = window;
  // stream and group modes launch one persistent wave per SIMD slot of the
  // variant's bf16 kernel; the f32 sliding kernel fits one wave per SIMD, so
  // it launches half as many (one round, the slots it leaves unused stay in
  // the workspace)
  const int launch_waves =
      !unit_mode && variant == GQA_SLIDING && !bf16 ? plan.waves / 2 : plan.waves;
  ka.n_waves = launch_waves;
  ka.ring = ring;
  ka.dyn = plan.dyn ? 1 : 0;
  ka.counter = plan.dyn ? reinterpret_cast<int32_t*>(ws + plan.counter) : nullptr;
  // the dynamic tail's counter starts at zero (a kernel, not a memset, so that
  // the call can be captured into a graph)
  if (plan.dyn) {
    hipLaunchKernelGGL(gqa_zero_counter_kernel, dim3(1), dim3(64), 0, stream, ka.counter);
    if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
  }

  MainFn main_fn = variant == GQA_SLIDING ? pick_main<16, 256, false>(plan.mode, paged, bf16)
                   : kfv                   ? pick_main<4, 512, true>(plan.mode, paged, bf16)
                                           : pick_main<4, 512, false>(plan.mode, paged, bf16);
  ProfRec* pr = prof_slot(kfv ? kProfKeysFromValues : 2 * variant);
  if (pr) (void)hipEventRecord(pr->start, stream);
  hipLaunchKernelGGL(main_fn, dim3((unsigned)(launch_waves / kWaves)), dim3(kThreads), 0, stream,
                     ka);
  if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
  if (pr) (void)hipEventRecord(pr->stop, stream);
  if (unit_mode) return GQA_OK;

  CombineArgs ca;
  ca.prefix = ka.prefix;
  ca.ws_ml = ka.ws_ml;
  ca.ws_acc = ka.ws_acc;
  ca.o = ka.o;
  ca.B = B;
  ca.n_waves = group_mode ? launch_waves / kWaves : launch_waves;
  ca.groups = group_mode ? 1 : 0;
  ca.dyn = ka.dyn;
  const int ds = variant == GQA_SLIDING ? combine_parts<256>(B) : combine_parts<512>(B);
  const int cw = combine_waves(B * kHeads * ds);
  CombineFn comb =
      variant == GQA_SLIDING ? pick_combine<16, 256>(bf16, ds, cw) : pick_combine<4, 512>(bf16, ds, cw);
  if (!comb) return GQA_ERR_SHAPE;
  ProfRec* pc = prof_slot(kfv ? kProfKeysFromValues + 1 : 2 * variant + 1);
  if (pc) (void)hipEventRecord(pc->start, stream);
  hipLaunchKernelGGL(comb, dim3((unsigned)(B * kHeads * ds)), dim3(64u * (unsigned)cw), 0, stream,
                     ca);
  if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
  if (pc) (void)hipEventRecord(pc->stop, stream);
  return GQA_OK;
}

typedef void (*AppendFn)(AppendArgs);

template <int KV, int D>
AppendFn pick_append(bool paged, bool bf16) {
  if (paged)
    return bf16 ? gqa_append_kernel<KV, D, true, true> : gqa_append_kernel<KV, D, true, false>;
  return bf16 ? gqa_append_kernel<KV, D, false, true> : gqa_append_kernel<KV, D, false, false>;
}

// k_cache == nullptr with values_only: global layers over a values-only cache
// (the key row is not written; attention rebuilds it from the value row)
// ring > 0: sliding layers over a contiguous cache capped at `ring` positions
int run_append(int variant, bool paged, bool values_only, const void* q_raw, const void* k_raw,
               const void* v_raw, const void* w_q, const void* w_k, const int32_t* block_table,
               int32_t max_pages, const int32_t* seq_lens, void* q_out, void* k_cache,
               void* v_cache, int32_t B, int32_t S_max, int32_t num_pages, int32_t dtype,
               void* stream_, int32_t ring = 0) {
  const bool global = variant == GQA_GLOBAL;
  if (values_only && !global) return GQA_ERR_DTYPE;
  if (!q_raw || !k_raw || (!global && !v_raw) || !w_q || !w_k || !seq_lens || !q_out ||
      (!k_cache && !values_only) || !v_cache || (paged && !block_table))
    return GQA_ERR_NULL;
  if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_DTYPE;
  if (B < 1 || B > kMaxBatch) return GQA_ERR_SHAPE;
  int cap;
  if (paged) {
    if (max_pages < 1 || max_pages > kMaxSeq / kPage || num_pages < 1) return GQA_ERR_SHAPE;
    cap = max_pages * kPage;
  } else {
    if (S_max < 1 || S_max > kMaxSeq) return GQA_ERR_SHAPE;
    cap = S_max;
  }
  if (ring != 0) {
    if (global || paged) return GQA_ERR_DTYPE;
    if (ring < kTile || ring > kMaxSeq || ring % kTile != 0 || ring != S_max) return GQA_ERR_SHAPE;
  }
  if (!aligned16(q_raw) || !aligned16(k_raw) || (!global && !aligned16(v_raw)) ||
      !aligned16(w_q) || !aligned16(w_k) || !aligned16(q_out) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return GQA_ERR_ALIGN;
  AppendArgs aa;
  aa.q_raw = static_cast<const char*>(q_raw);
  aa.k_raw = static_cast<const char*>(k_raw);
  aa.v_raw = static_cast<const char*>(v_raw);
  aa.w_q = static_cast<const char*>(w_q);
  aa.w_k = static_cast<const char*>(w_k);
  aa.seq_lens = seq_lens;
  aa.block_table = block_table;
  aa.q_out = static_cast<char*>(q_out);
  aa.k_cache = values_only ? nullptr : static_cast<char*>(k_cache);
  aa.v_cache = static_cast<char*>(v_cache);
  aa.B = B;
  aa.cap = cap;
  aa.max_pages = paged ? max_pages : 0;
  aa.num_pages = paged ? num_pages : 0;
  aa.ring = ring;
  const bool bf16 = dtype == GQA_BF16;
  AppendFn fn = global ? pick_append<4, 512>(paged, bf16) : pick_append<16, 256>(paged, bf16);
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  ProfRec* pr = prof_slot(values_only ? kProfKeysFromValues + 2 : 4 + variant);
  if (pr) (void)hipEventRecord(pr->start, stream);
  const unsigned rows = kHeads + 2 * (global ? 4 : 16);  // q, k and v head rows
  hipLaunchKernelGGL(fn, dim3((unsigned)B, (rows + kWaves - 1) / kWaves), dim3(kThreads), 0, stream,
                     aa);
  if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
  if (pr) (void)hipEventRecord(pr->stop, stream);
  return GQA_OK;
}

}  // namespace

namespace gqa_detail {
int prof_begin(int kind, hipStream_t stream) {
  if (!g_prof_on || g_prof_used >= g_prof.size()) return -1;
  const int slot = (int)g_prof_used++;
  g_prof[slot].kind = kind;
  (void)hipEventRecord(g_prof[slot].start, stream);
  return slot;
}
void prof_end(int slot, hipStream_t stream) {
  if (slot >= 0) (void)hipEventRecord(g_prof[slot].stop, stream);
}
}  // namespace gqa_detail

extern "C" {

int gqa_decode_sliding(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                       void* o, int32_t B, int32_t S_max, int32_t dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return run(GQA_SLIDING, kSlidingWindow, false, q, k, v, nullptr, nullptr, 0, seq_lens, o, B, S_max, 0, dtype, workspace,
             workspace_bytes, stream);
}

int gqa_decode_global(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                      void* o, int32_t B, int32_t S_max, int32_t dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return run(GQA_GLOBAL, 0, false, q, k, v, nullptr, nullptr, 0, seq_lens, o, B, S_max, 0, dtype, workspace,
             workspace_bytes, stream);
}

int gqa_decode_sliding_paged(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, int32_t max_pages,
                             const int32_t* seq_lens, void* o, int32_t B, int32_t num_pages,
                             int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return run(GQA_SLIDING, kSlidingWindow, true, q, k_pool, v_pool, nullptr, block_table, max_pages, seq_lens, o, B, 0,
             num_pages, dtype, workspace, workspace_bytes, stream);
}

int gqa_decode_global_paged(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, void* o, int32_t B, int32_t num_pages,
                            int32_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return run(GQA_GLOBAL, 0, true, q, k_pool, v_pool, nullptr, block_table, max_pages, seq_lens, o, B, 0,
             num_pages, dtype, workspace, workspace_bytes, stream);
}

int gqa_decode_global_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* seq_lens, void* o, int32_t B,
                                    int32_t num_pages, int32_t dtype, void* stream) {
  return run(GQA_GLOBAL, 0, true, q, k_pool, v_pool, nullptr, block_table, max_pages, seq_lens, o,
             B, 0, num_pages, dtype, nullptr, 0, stream, 0, true);
}

int gqa_decode_sliding_window(const void* q, const void* k, const void* v,
                              const int32_t* seq_lens, void* o, int32_t B, int32_t S_max,
                              int32_t window, int32_t dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (window < 1) return GQA_ERR_SHAPE;
  return run(GQA_SLIDING, window, false, q, k, v, nullptr, nullptr, 0, seq_lens, o, B, S_max, 0, dtype,
             workspace, workspace_bytes, stream);
}

int gqa_decode_sliding_window_paged(const void* q, const void* k_pool, const void* v_pool,
                                    const int32_t* block_table, int32_t max_pages,
                                    const int32_t* seq_lens, void* o, int32_t B,
                                    int32_t num_pages, int32_t window, int32_t dtype,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 1) return GQA_ERR_SHAPE;
  return run(GQA_SLIDING, window, true, q, k_pool, v_pool, nullptr, block_table, max_pages, seq_lens, o, B,
             0, num_pages, dtype, workspace, workspace_bytes, stream);
}

size_t gqa_decode_sliding_window_workspace_bytes(int32_t B, int32_t capacity, int32_t window) {
  Plan p;
  if (window < 1 || make_plan(GQA_SLIDING, B, capacity, window, &p)) return 0;
  return p.total;
}

int gqa_decode_sliding_window_plan(int32_t B, int32_t capacity, int32_t window, int32_t* mode,
                                   int32_t* n_waves, int32_t* n_slots) {
  if (window < 1) return GQA_ERR_SHAPE;
  Plan p;
  int rc = make_plan(GQA_SLIDING, B, capacity, window, &p);
  if (rc) return rc;
  if (mode) *mode = p.mode;
  if (n_waves) *n_waves = p.waves;
  if (n_slots) *n_slots = p.slots;
  return GQA_OK;
}

int gqa_decode_sliding_ring(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                            void* o, int32_t B, int32_t ring, int32_t window, int32_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 1) return GQA_ERR_SHAPE;
  return run(GQA_SLIDING, window, false, q, k, v, nullptr, nullptr, 0, seq_lens, o, B, ring, 0,
             dtype, workspace, workspace_bytes, stream, ring);
}

size_t gqa_decode_sliding_ring_workspace_bytes(int32_t B, int32_t ring, int32_t window) {
  Plan p;
  if (window < 1 || ring < kTile || ring > kMaxSeq || ring % kTile != 0 || window > ring ||
      make_plan(GQA_SLIDING, B, kMaxSeq, window, &p))
    return 0;
  return p.total;
}

int gqa_append_sliding_ring(const void* q_raw, const void* k_raw, const void* v_raw,
                            const void* w_q, const void* w_k, const int32_t* seq_lens,
                            void* q_out, void* k_cache, void* v_cache, int32_t B, int32_t ring,
                            int32_t dtype, void* stream) {
  return run_append(GQA_SLIDING, false, false, q_raw, k_raw, v_raw, w_q, w_k, nullptr, 0,
                    seq_lens, q_out, k_cache, v_cache, B, ring, 0, dtype, stream, ring);
}

int gqa_append_sliding(const void* q_raw, const void* k_raw, const void* v_raw, const void* w_q,
                       const void* w_k, const int32_t* seq_lens, void* q_out, void* k_cache,
                       void* v_cache, int32_t B, int32_t S_max, int32_t dtype, void* stream) {
  return run_append(GQA_SLIDING, false, false, q_raw, k_raw, v_raw, w_q, w_k, nullptr, 0, seq_lens, q_out,
                    k_cache, v_cache, B, S_max, 0, dtype, stream);
}

int gqa_append_sliding_paged(const void* q_raw, const void* k_raw, const void* v_raw,
                             const void* w_q, const void* w_k, const int32_t* block_table,
                             int32_t max_pages, const int32_t* seq_lens, void* q_out,
                             void* k_pool, void* v_pool, int32_t B, int32_t num_pages,
                             int32_t dtype, void* stream) {
  return run_append(GQA_SLIDING, true, false, q_raw, k_raw, v_raw, w_q, w_k, block_table, max_pages,
                    seq_lens, q_out, k_pool, v_pool, B, 0, num_pages, dtype, stream);
}

int gqa_append_global(const void* q_raw, const void* k_raw, const void* w_q, const void* w_k,
                      const int32_t* seq_lens, void* q_out, void* k_cache, void* v_cache,
                      int32_t B, int32_t S_max, int32_t dtype, void* stream) {
  return run_append(GQA_GLOBAL, false, false, q_raw, k_raw, nullptr, w_q, w_k, nullptr, 0, seq_lens,
                    q_out, k_cache, v_cache, B, S_max, 0, dtype, stream);
}

int gqa_append_global_paged(const void* q_raw, const void* k_raw, const void* w_q,
                            const void* w_k, const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, void* q_out, void* k_pool, void* v_pool,
                            int32_t B, int32_t num_pages, int32_t dtype, void* stream) {
  return run_append(GQA_GLOBAL, true, false, q_raw, k_raw, nullptr, w_q, w_k, block_table, max_pages,
                    seq_lens, q_out, k_pool, v_pool, B, 0, num_pages, dtype, stream);
}

int gqa_decode_global_k_eq_v(const void* q, const void* v, const void* w_k,
                             const int32_t* seq_lens, void* o, int32_t B, int32_t S_max,
                             int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!w_k) return GQA_ERR_NULL;
  return run(GQA_GLOBAL, 0, false, q, nullptr, v, w_k, nullptr, 0, seq_lens, o, B, S_max, 0,
             dtype, workspace, workspace_bytes, stream);
}

int gqa_decode_global_k_eq_v_paged(const void* q, const void* v_pool, const void* w_k,
                                   const int32_t* block_table, int32_t max_pages,
                                   const int32_t* seq_lens, void* o, int32_t B,
                                   int32_t num_pages, int32_t dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!w_k) return GQA_ERR_NULL;
  return run(GQA_GLOBAL, 0, true, q, nullptr, v_pool, w_k, block_table, max_pages, seq_lens, o,
             B, 0, num_pages, dtype, workspace, workspace_bytes, stream);
}

int gqa_append_global_k_eq_v(const void* q_raw, const void* k_raw, const void* w_q,
                             const void* w_k, const int32_t* seq_lens, void* q_out,
                             void* v_cache, int32_t B, int32_t S_max, int32_t dtype,
                             void* stream) {
  return run_append(GQA_GLOBAL, false, true, q_raw, k_raw, nullptr, w_q, w_k, nullptr, 0,
                    seq_lens, q_out, nullptr, v_cache, B, S_max, 0, dtype, stream);
}

int gqa_append_global_k_eq_v_paged(const void* q_raw, const void* k_raw, const void* w_q,
                                   const void* w_k, const int32_t* block_table,
                                   int32_t max_pages, const int32_t* seq_lens, void* q_out,
                                   void* v_pool, int32_t B, int32_t num_pages, int32_t dtype,
                                   void* stream) {
  return run_append(GQA_GLOBAL, true, true, q_raw, k_raw, nullptr, w_q, w_k, block_table,
                    max_pages, seq_lens, q_out, nullptr, v_pool, B, 0, num_pages, dtype, stream);
}

size_t gqa_decode_workspace_bytes(int32_t variant, int32_t B, int32_t capacity) {
  Plan p;
  if (make_plan(variant, B, capacity, default_window(variant), &p)) return 0;
  return p.total;
}

int gqa_decode_plan(int32_t variant, int32_t B, int32_t capacity, int32_t* mode,
                    int32_t* n_waves, int32_t* n_slots) {
  Plan p;
  int rc = make_plan(variant, B, capacity, default_window(variant), &p);
  if (rc) return rc;
  if (mode) *mode = p.mode;
  if (n_waves) *n_waves = p.waves;
  if (n_slots) *n_slots = p.slots;
  return GQA_OK;
}

int gqa_decode_constants(int32_t variant, int32_t* heads, int32_t* kv_heads, int32_t* head_dim,
                         int32_t* window, int32_t* page) {
  VariantInfo vi;
  if (!variant_info(variant, &vi)) return GQA_ERR_DTYPE;
  if (heads) *heads = kHeads;
  if (kv_heads) *kv_heads = vi.KV;
  if (head_dim) *head_dim = vi.D;
  if (window) *window = vi.window;
  if (page) *page = kPage;
  return GQA_OK;
}

const char* gqa_status_str(int32_t status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL: return "null pointer argument";
    case GQA_ERR_SHAPE: return "shape argument out of range";
    case GQA_ERR_DTYPE: return "unknown dtype or variant";
    case GQA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GQA_ERR_WORKSPACE: return "workspace missing or too small";
    case GQA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int gqa_decode_force_mode(int32_t mode) {
  if (mode < -1 || mode > GQA_MODE_GROUP) return GQA_ERR_SHAPE;
  g_force_mode = mode;
  return GQA_OK;
}

int gqa_hbm_read_probe(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return GQA_ERR_NULL;
  if (bytes == 0 || bytes % 16) return GQA_ERR_SHAPE;
  if (!aligned16(src)) return GQA_ERR_ALIGN;
  // 1024 waves (one per SIMD), 8 KiB in flight each: the fastest plain read
  // of a sweep over wave counts and depths (8192 waves read about 4% slower)
  hipLaunchKernelGGL(hbm_read_kernel, dim3(256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<unsigned*>(sink));
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_hbm_copy_probe(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return GQA_ERR_NULL;
  if (bytes == 0 || bytes % 16) return GQA_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return GQA_ERR_ALIGN;
  hipLaunchKernelGGL(hbm_copy_kernel, dim3(2048), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_profile_begin(int32_t capacity) {
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  g_prof_used = 0;
  g_prof_on = false;
  if (capacity < 1) return GQA_ERR_SHAPE;
  g_prof.resize((size_t)capacity);
  for (auto& r : g_prof) {
    if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess)
      return GQA_ERR_HIP;
  }
  g_prof_on = true;
  return GQA_OK;
}

int gqa_profile_read(int32_t* counts, double* total_ms, int32_t n_kinds) {
  for (int i = 0; i < n_kinds; ++i) {
    counts[i] = 0;
    total_ms[i] = 0.0;
  }
  int rc = GQA_OK;
  for (size_t i = 0; i < g_prof_used; ++i) {
    ProfRec& r = g_prof[i];
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess ||
        hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      rc = GQA_ERR_HIP;
      continue;
    }
    if (r.kind >= 0 && r.kind < n_kinds) {
      counts[r.kind] += 1;
      total_ms[r.kind] += ms;
    }
  }
  for (auto& r : g_prof) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  g_prof_used = 0;
  g_prof_on = false;
  return rc;
}

}  // extern "C"
