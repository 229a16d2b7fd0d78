// gqa_decode.hip -- gfx950 decode attention for the Gemma-4-31B text decoder.
//
// Implements the attn.core node of the gemma-4-31B Model Spec page
// ("Compute-graph nodes" table): slidingDecodeGQA (32 query heads over 16 kv
// heads, D = 256, scale 1, the last 1024 positions) and decodeGQA (32 over 4,
// D = 512, scale 1, every position below seq_lens[b]), on a contiguous
// [B,S,kv,D] cache or on a paged cache of 16-position pages (the "At a glance"
// table's Shape domain row).  The C ABI is declared in include/gqa_decode.h.
//
// Method: flash-decoding.  The attended positions of one (sequence, kv head)
// pair -- a "unit" -- are cut into tiles of 16 positions (one page).  A tile
// is consumed by one wave64 with every query head of the GQA group at once:
//
//   QK^T  v_mfma_f32_16x16x32_bf16 (or 16x16x4_f32): A = 16 key rows of the
//         tile, B = the group's query heads (padded to 16 columns with zeros).
//         The reduction index may be any permutation of d shared by A and B,
//         so each lane loads whole 16-byte chunks of one key row straight
//         from HBM in the order the instruction wants them.
//   softmax online, in fp32: running max m and sum l per head, base-2
//         exponentials of (z - m) * log2(e).  The logit accumulator layout
//         (lane = head column, 4 consecutive positions per lane) is exactly
//         the B operand layout of the PV instruction, so P never moves.
//   PV    v_mfma_f32_16x16x16_bf16 (or 16x16x4_f32) computing O^T = V^T P^T:
//         A = V^T, built by transposing in registers the 4 rows x 8 columns a
//         lane loads with 16-byte loads (one v_perm_b32 per output dword).
//
// The accumulator keeps O^T, so the per-head rescale factor of the online
// softmax is a per-lane scalar.  Four waves of a work-group take interleaved
// tiles of one split and merge their (m, l, O) through LDS; when the host
// plans more than one split per unit, each work-group stores its partial
// (O, m, l) in the fp32 workspace and a combine kernel merges the splits.
//
// Every K/V byte of the attended range is read from HBM exactly once; no byte
// outside it is read (masked rows are never loaded, so NaN or stale data in
// unused cache space cannot leak into the result).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "gqa_decode.h"

namespace {

constexpr int kHeads = 32;
constexpr int kPage = 16;
constexpr int kTile = 16;  // positions per tile: one page
constexpr int kWaves = 4;  // waves per work-group of the split kernel
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxBatch = 256;
constexpr int kMaxSeq = 262144;
constexpr int kSlidingWindow = 1024;
constexpr float kLog2e = 1.4426950408889634f;
// raise the softmax reference max only when a tile exceeds it by more than
// this (natural-log units): weights stay below e^8
constexpr float kRescaleGap = 8.0f;

// split planner: aim at ~8 work-groups per CU of a 256-CU part, with splits of
// 4..128 tiles (64..2048 positions)
constexpr long kTargetGroups = 2048;
constexpr int kMinTilesPerSplit = 4;
constexpr int kMaxTilesPerSplit = 128;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  static constexpr int E = 8;  // elements per 16-byte chunk
  static constexpr int bytes = 2;
};
template <>
struct Elem<false> {
  static constexpr int E = 4;
  static constexpr int bytes = 4;
};

struct SplitArgs {
  const char* q;
  const char* k;
  const char* v;
  const int32_t* seq_lens;
  const int32_t* block_table;
  char* o;
  float* ws_ml;   // [unit][split][G][2]  (m, l)
  float* ws_acc;  // [unit][split][G][D]
  int32_t cap;
  int32_t max_pages;
  int32_t num_pages;
  int32_t window;
  int32_t n_split;
  int32_t tps;  // tiles per split
};

struct Range {
  int lo, L;  // attended positions [lo, L)
  int t0, t1; // tiles [t0, t1) that hold them
};

// The attended range of sequence b; shared by the split and combine kernels so
// that both cut it identically.
__device__ inline Range unit_range(const int32_t* seq_lens, int b, int cap, int window) {
  int L = seq_lens[b];
  L = L < cap ? L : cap;
  Range r;
  if (L <= 0) {
    r.lo = r.L = r.t0 = r.t1 = 0;
    return r;
  }
  r.L = L;
  r.lo = (window > 0 && L > window) ? L - window : 0;
  r.t0 = r.lo / kTile;
  r.t1 = (L + kTile - 1) / kTile;
  return r;
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline u32x4 load16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

// Values are read exactly once, 256 contiguous bytes per row and instruction:
// non-temporal loads keep them out of the caches and raise the sustained read
// rate.  Keys are read in 64-byte halves of a 128-byte line by two consecutive
// instructions; they use ordinary loads so the line is still cached for the
// second half (non-temporal key loads measured slower).
__device__ inline u32x4 load16_stream(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ inline unsigned bf16_bits(float x) {
  return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)x);
}

__device__ inline float bf16_value(unsigned bits) {
  return __builtin_bit_cast(float, bits << 16);
}

// Component e of a 16-byte chunk as a float.  The component is copied into a
// scalar first: bit-casting a vector-component expression directly does not
// select the component.
__device__ inline float chunk_f32(const u32x4& c, int e) {
  const unsigned x = c[e];
  return __builtin_bit_cast(float, x);
}

// Store 4E consecutive fp32 values as E-sized output chunks (16 bytes each).
template <bool BF16>
__device__ inline void store_run(char* dst, const float* v, int n) {
  if constexpr (BF16) {
    for (int c = 0; c < n / 8; ++c) {
      u32x4 w;
      for (int q = 0; q < 4; ++q)
        w[q] = bf16_bits(v[8 * c + 2 * q]) | (bf16_bits(v[8 * c + 2 * q + 1]) << 16);
      *reinterpret_cast<u32x4*>(dst + 16 * c) = w;
    }
  } else {
    for (int c = 0; c < n / 4; ++c) {
      f32x4 w = {v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
      *reinterpret_cast<f32x4*>(dst + 16 * c) = w;
    }
  }
}

// Waves per SIMD the split kernel is compiled for: the sliding bf16 kernel fits
// two (<= 256 registers), the others need one.
template <int KV, bool BF16>
constexpr int split_waves_per_simd() {
  return (KV == 16 && BF16) ? 2 : 1;
}

template <int KV, int D, bool PAGED, bool BF16>
__global__ __launch_bounds__(kThreads, (split_waves_per_simd<KV, BF16>())) void gqa_split_kernel(
    SplitArgs a) {
  constexpr int G = kHeads / KV;  // query heads per kv head
  constexpr int E = Elem<BF16>::E;
  constexpr int EB = Elem<BF16>::bytes;
  constexpr int ROW = D * EB;                    // bytes of one head row
  constexpr size_t POS = (size_t)KV * D * EB;    // bytes between positions
  constexpr int NCH = D / E;                     // 16-byte chunks per row
  constexpr int KCH = NCH / 4;                   // key chunks per lane (chunk 4t+j)
  constexpr int VBLK = NCH / 16;                 // value chunks per lane and row (r+16*blk)
  constexpr int RUN = 4 * E;                     // contiguous d values per lane and blk
  constexpr int LROW = D + 4;                    // padded LDS row (floats)

  __shared__ float s_acc[(kWaves - 1) * G * LROW];
  __shared__ float s_m[(kWaves - 1) * G];
  __shared__ float s_l[(kWaves - 1) * G];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;  // row (A) / column (B, C) index of the 16x16 tiles
  const int j = lane >> 4;  // k-group of the operands, row-group of C
  const int split = blockIdx.x % a.n_split;
  const int unit = blockIdx.x / a.n_split;
  const int b = unit / KV;
  const int g = unit % KV;
  const bool direct = a.n_split == 1;

  const Range rg = unit_range(a.seq_lens, b, a.cap, a.window);
  const int wg_t0 = rg.t0 + split * a.tps;
  const int wg_t1 = min(rg.t1, wg_t0 + a.tps);

  if (wg_t0 >= wg_t1) {
    // nothing attended in this split
    if (direct) {
      for (int c = tid; c < G * NCH; c += kThreads) {
        char* dst = a.o + ((size_t)b * kHeads + g * G + c / NCH) * ROW + (c % NCH) * 16;
        *reinterpret_cast<u32x4*>(dst) = u32x4{0u, 0u, 0u, 0u};
      }
    } else if (tid < G) {
      float* ml = a.ws_ml + (((size_t)unit * a.n_split + split) * G + tid) * 2;
      ml[0] = -INFINITY;
      ml[1] = 0.f;
    }
    return;
  }

  // query heads of the group as the B operand of QK^T (columns >= G are zero)
  u32x4 qreg[KCH];
  {
    const char* qrow = a.q + ((size_t)b * kHeads + g * G + (r < G ? r : 0)) * ROW;
#pragma unroll
    for (int t = 0; t < KCH; ++t) {
      const u32x4 x = load16(qrow + (4 * t + j) * 16);
      qreg[t] = r < G ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // this wave takes tiles wg_t0 + wave + 4*i, i < n_mine; lane i holds the
  // physical page of its i-th tile (one vector load instead of one dependent
  // scalar load per tile)
  const int first = wg_t0 + wave;
  const int n_mine = first < wg_t1 ? (wg_t1 - first + kWaves - 1) / kWaves : 0;
  int pages = 0;
  if constexpr (PAGED) {
    if (lane < n_mine) pages = a.block_table[(size_t)b * a.max_pages + first + kWaves * lane];
  }

  // Per-tile addressing.  Rows outside [lo, L) are clamped onto the nearest
  // attended row of the same tile: every load is unconditional yet never
  // leaves the attended range; the clamped duplicates are dropped below by
  // setting their logits to -inf (so their softmax weight is exactly 0).
  struct TileAt {
    const char* kb;
    const char* vb;
    int pos0;
    bool ok;  // page id inside the pool
  };
  auto tile_at = [&](int i) {
    TileAt t;
    const int tile = first + kWaves * i;
    t.pos0 = tile * kTile;
    size_t off;
    if constexpr (PAGED) {
      const int page = __builtin_amdgcn_readlane(pages, i);
      t.ok = page >= 0 && page < a.num_pages;
      off = ((size_t)(t.ok ? page : 0) * kPage * KV + g) * (size_t)ROW;
    } else {
      t.ok = true;
      off = (((size_t)b * a.cap + t.pos0) * KV + g) * (size_t)ROW;
    }
    t.kb = a.k + off;
    t.vb = a.v + off;
    return t;
  };
  auto clamp_row = [&](int pos0, int row) {
    const int p = min(max(pos0 + row, rg.lo), rg.L - 1);
    return p - pos0;
  };

  u32x4 kreg[KCH];       // key row r of the tile, chunks 4t+j
  u32x4 vreg[4][VBLK];   // value rows 4j+i of the tile, chunks r+16*blk
  auto load_k = [&](const TileAt& t) {
    const char* row = t.kb + (size_t)clamp_row(t.pos0, r) * POS;
#pragma unroll
    for (int c = 0; c < KCH; ++c) kreg[c] = load16(row + (4 * c + j) * 16);
  };
  auto load_v = [&](const TileAt& t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* row = t.vb + (size_t)clamp_row(t.pos0, 4 * j + i) * POS;
#pragma unroll
      for (int blk = 0; blk < VBLK; ++blk) vreg[i][blk] = load16_stream(row + (r + 16 * blk) * 16);
    }
  };

  f32x4 acc[VBLK][E];
#pragma unroll
  for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[blk][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Reference max of head r (equal on the 4 lanes of a column).  It is raised
  // only when a tile's max exceeds it by more than kRescaleGap, so weights
  // stay below e^kRescaleGap and the O/l rescale runs a few times per wave
  // instead of every tile; the result is the same softmax either way.
  float m = -INFINITY;
  float l = 0.f;  // this lane's share of the sum of weights

  TileAt cur = tile_at(0);
  if (n_mine > 0) {
    load_k(cur);
    load_v(cur);
  }
  for (int it = 0; it < n_mine; ++it) {
    const bool more = it + 1 < n_mine;
    const TileAt nxt = more ? tile_at(it + 1) : cur;

    // logits z[pos 4j+i][head r]
    f32x4 z;
    {
      f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
#pragma unroll
        for (int t = 0; t < KCH; t += 2) {
          z0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kreg[t]), __builtin_bit_cast(bf16x8, qreg[t]), z0, 0, 0, 0);
          z1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kreg[t + 1]), __builtin_bit_cast(bf16x8, qreg[t + 1]), z1,
              0, 0, 0);
        }
      } else {
#pragma unroll
        for (int t = 0; t < KCH; ++t) {
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            z0 = __builtin_amdgcn_mfma_f32_16x16x4f32(chunk_f32(kreg[t], e),
                                                      chunk_f32(qreg[t], e), z0, 0, 0, 0);
            z1 = __builtin_amdgcn_mfma_f32_16x16x4f32(chunk_f32(kreg[t], e + 1),
                                                      chunk_f32(qreg[t], e + 1), z1, 0, 0, 0);
          }
        }
      }
      z = z0 + z1;
    }
    // the key registers are free: fetch the next tile's keys
    if (more) load_k(nxt);

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = cur.pos0 + 4 * j + i;
      if (!(cur.ok && p >= rg.lo && p < rg.L)) z[i] = -INFINITY;
    }

    // online softmax (fp32)
    float tmax = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool grow = tmax > m + kRescaleGap;  // also when m = -inf and tmax is finite
    if (__any(grow)) {
      const float m_next = grow ? tmax : m;
      const float alpha = exp2_fast((m - (m_next == -INFINITY ? 0.f : m_next)) * kLog2e);
      if (grow) {
        l *= alpha;
#pragma unroll
        for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[blk][e] *= alpha;
      }
      m = m_next;
    }
    const float m_use = m == -INFINITY ? 0.f : m;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2_fast((z[i] - m_use) * kLog2e);

    if constexpr (BF16) {
      unsigned pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = bf16_bits(p[i]);
      l += (bf16_value(pb[0]) + bf16_value(pb[1])) + (bf16_value(pb[2]) + bf16_value(pb[3]));
      const s16x4 pt =
          __builtin_bit_cast(s16x4, u32x2{pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)});
#pragma unroll
      for (int blk = 0; blk < VBLK; ++blk) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const int dw = e >> 1;
          const unsigned lo = __builtin_amdgcn_perm(vreg[1][blk][dw], vreg[0][blk][dw], sel);
          const unsigned hi = __builtin_amdgcn_perm(vreg[3][blk][dw], vreg[2][blk][dw], sel);
          const s16x4 vt = __builtin_bit_cast(s16x4, u32x2{lo, hi});
          acc[blk][e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pt, acc[blk][e], 0, 0, 0);
        }
      }
    } else {
      l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[blk][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(chunk_f32(vreg[i][blk], e), p[i],
                                                               acc[blk][e], 0, 0, 0);
    }
    // the value registers are free: fetch the next tile's values
    if (more) load_v(nxt);
    cur = nxt;
  }

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  // merge the four waves: lane (r, j) holds, for head r and each blk, the d
  // values 16E*blk + 4E*j + E*i + e  (i = C row within the lane, e = instruction)
  if (wave > 0 && r < G) {
    float* dst = s_acc + ((wave - 1) * G + r) * LROW;
#pragma unroll
    for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < E; ++e) dst[16 * E * blk + 4 * E * j + E * i + e] = acc[blk][e][i];
    if (j == 0) {
      s_m[(wave - 1) * G + r] = m;
      s_l[(wave - 1) * G + r] = l;
    }
  }
  __syncthreads();
  if (wave != 0 || r >= G) return;

  float M = m;
  float mw[kWaves - 1], lw[kWaves - 1];
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) {
    mw[w] = s_m[w * G + r];
    lw[w] = s_l[w * G + r];
    M = fmaxf(M, mw[w]);
  }
  const float Muse = M == -INFINITY ? 0.f : M;
  const float sc0 = exp2_fast((m - Muse) * kLog2e);
  float sc[kWaves - 1];
  float Lt = sc0 * l;
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) {
    sc[w] = exp2_fast((mw[w] - Muse) * kLog2e);
    Lt += sc[w] * lw[w];
  }

  const int head = g * G + r;
#pragma unroll
  for (int blk = 0; blk < VBLK; ++blk) {
    const int d0 = 16 * E * blk + 4 * E * j;
    float run[RUN];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = d0 + E * i + e;
        float x = sc0 * acc[blk][e][i];
#pragma unroll
        for (int w = 0; w < kWaves - 1; ++w) x += sc[w] * s_acc[(w * G + r) * LROW + d];
        run[E * i + e] = x;
      }
    if (direct) {
      const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
#pragma unroll
      for (int c = 0; c < RUN; ++c) run[c] = Lt > 0.f ? run[c] * inv : 0.f;
      store_run<BF16>(a.o + ((size_t)b * kHeads + head) * ROW + (size_t)d0 * EB, run, RUN);
    } else {
      float* dst = a.ws_acc + (((size_t)unit * a.n_split + split) * G + r) * D + d0;
#pragma unroll
      for (int c = 0; c < RUN; c += 4)
        *reinterpret_cast<f32x4*>(dst + c) = f32x4{run[c], run[c + 1], run[c + 2], run[c + 3]};
    }
  }
  if (!direct && j == 0) {
    float* ml = a.ws_ml + (((size_t)unit * a.n_split + split) * G + r) * 2;
    ml[0] = M;
    ml[1] = Lt;
  }
}

struct CombineArgs {
  const int32_t* seq_lens;
  const float* ws_ml;
  const float* ws_acc;
  char* o;
  int32_t cap;
  int32_t window;
  int32_t n_split;
  int32_t tps;
};

// One work-group per (sequence, query head); thread t owns d = 4t .. 4t+3.
// Splits whose l is 0 hold no result (their workspace slots may be stale):
// their weight is 0 and their values are selected away, never multiplied.
template <int KV, int D, bool BF16>
__global__ __launch_bounds__(D / 4) void gqa_combine_kernel(CombineArgs a) {
  constexpr int G = kHeads / KV;
  constexpr int EB = Elem<BF16>::bytes;
  constexpr int U = 8;  // partials in flight per thread
  const int b = blockIdx.x / kHeads;
  const int h = blockIdx.x % kHeads;
  const int g = h / G;
  const int hh = h % G;
  const int unit = b * KV + g;
  const Range rg = unit_range(a.seq_lens, b, a.cap, a.window);
  int n_used = rg.t1 > rg.t0 ? (rg.t1 - rg.t0 + a.tps - 1) / a.tps : 0;
  n_used = n_used < a.n_split ? n_used : a.n_split;

  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2* ml = reinterpret_cast<const f32x2*>(a.ws_ml) + (size_t)unit * a.n_split * G + hh;
  float M = -INFINITY;
  for (int s = 0; s < n_used; ++s) {
    const f32x2 x = ml[(size_t)s * G];
    if (x[1] > 0.f) M = fmaxf(M, x[0]);
  }
  const int d = threadIdx.x * 4;
  const float* accp = a.ws_acc + ((size_t)unit * a.n_split * G + hh) * D + d;
  const size_t sstride = (size_t)G * D;
  f32x4 A = {0.f, 0.f, 0.f, 0.f};
  float Lt = 0.f;
  for (int s0 = 0; s0 < n_used; s0 += U) {
    f32x4 x[U];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u < n_used ? s0 + u : n_used - 1;
      const f32x2 e = ml[(size_t)s * G];
      const bool ok = s0 + u < n_used && e[1] > 0.f;
      w[u] = ok ? exp2_fast((e[0] - M) * kLog2e) : 0.f;
      Lt += w[u] * (ok ? e[1] : 0.f);
      x[u] = *reinterpret_cast<const f32x4*>(accp + (size_t)s * sstride);
      x[u] = ok ? x[u] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) A += w[u] * x[u];
  }
  float run[4];
  const float inv = Lt > 0.f ? 1.f / Lt : 0.f;
  for (int c = 0; c < 4; ++c) run[c] = Lt > 0.f ? A[c] * inv : 0.f;
  char* dst = a.o + ((size_t)b * kHeads + h) * D * EB + (size_t)d * EB;
  if constexpr (BF16) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{bf16_bits(run[0]) | (bf16_bits(run[1]) << 16),
                                           bf16_bits(run[2]) | (bf16_bits(run[3]) << 16)};
  } else {
    *reinterpret_cast<f32x4*>(dst) = f32x4{run[0], run[1], run[2], run[3]};
  }
}

// ------------------------------------------------------- measurement kernels
// Not part of the attention path: a plain read stream and a plain copy of a
// known byte count, used to measure the sustainable HBM read rate of the part
// and to calibrate a profiler's byte counters against the split kernels.  Each
// wave moves 8 KiB per iteration in 16-byte lanes (1 KiB contiguous per
// instruction).

constexpr int kProbeUnroll = 8;

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

struct Plan {
  int n_split;
  int tps;
};

struct VariantInfo {
  int KV, D, window;
};

inline bool variant_info(int variant, VariantInfo* vi) {
  if (variant == GQA_SLIDING) {
    *vi = {16, 256, kSlidingWindow};
    return true;
  }
  if (variant == GQA_GLOBAL) {
    *vi = {4, 512, 0};
    return true;
  }
  return false;
}

int make_plan(int variant, int B, int cap, Plan* p) {
  VariantInfo vi;
  if (!variant_info(variant, &vi)) return GQA_ERR_DTYPE;
  if (B < 1 || B > kMaxBatch || cap < 1 || cap > kMaxSeq) return GQA_ERR_SHAPE;
  int tiles_max = (cap + kTile - 1) / kTile;
  if (vi.window > 0) {
    const int wt = (vi.window + kTile - 1) / kTile + 1;
    tiles_max = tiles_max < wt ? tiles_max : wt;
  }
  const long units = (long)B * vi.KV;
  long tps = ((long)tiles_max * units + kTargetGroups - 1) / kTargetGroups;
  if (tps < kMinTilesPerSplit) tps = kMinTilesPerSplit;
  if (tps > kMaxTilesPerSplit) tps = kMaxTilesPerSplit;
  long n_split = (tiles_max + tps - 1) / tps;
  if (n_split <= 1) {
    n_split = 1;
    tps = tiles_max;
  }
  p->n_split = (int)n_split;
  p->tps = (int)tps;
  return GQA_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t ml_bytes(int variant, int B, const Plan& p) {
  VariantInfo vi;
  variant_info(variant, &vi);
  return align256((size_t)B * vi.KV * p.n_split * (kHeads / vi.KV) * 2 * sizeof(float));
}

size_t workspace_bytes(int variant, int B, const Plan& p) {
  if (p.n_split <= 1) return 0;
  VariantInfo vi;
  variant_info(variant, &vi);
  return ml_bytes(variant, B, p) +
         (size_t)B * vi.KV * p.n_split * (kHeads / vi.KV) * vi.D * sizeof(float);
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

typedef void (*SplitFn)(SplitArgs);
typedef void (*CombineFn)(CombineArgs);

template <int KV, int D>
SplitFn pick_split(bool paged, bool bf16) {
  if (paged) return bf16 ? gqa_split_kernel<KV, D, true, true> : gqa_split_kernel<KV, D, true, false>;
  return bf16 ? gqa_split_kernel<KV, D, false, true> : gqa_split_kernel<KV, D, false, false>;
}

template <int KV, int D>
CombineFn pick_combine(bool bf16) {
  return bf16 ? gqa_combine_kernel<KV, D, true> : gqa_combine_kernel<KV, D, false>;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int run(int variant, bool paged, const void* q, const void* k, const void* v,
        const int32_t* block_table, int32_t max_pages, const int32_t* seq_lens, void* o,
        int32_t B, int32_t S_max, int32_t num_pages, int32_t dtype, void* workspace,
        size_t workspace_bytes_given, void* stream_) {
  if (!q || !k || !v || !seq_lens || !o || (paged && !block_table)) return GQA_ERR_NULL;
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
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GQA_ERR_ALIGN;
  VariantInfo vi;
  variant_info(variant, &vi);
  Plan plan;
  int rc = make_plan(variant, B, cap, &plan);
  if (rc) return rc;
  const size_t need = workspace_bytes(variant, B, plan);
  if (need > 0) {
    if (!workspace || workspace_bytes_given < need) return GQA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return GQA_ERR_ALIGN;
  }
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const bool bf16 = dtype == GQA_BF16;

  SplitArgs sa;
  sa.q = static_cast<const char*>(q);
  sa.k = static_cast<const char*>(k);
  sa.v = static_cast<const char*>(v);
  sa.seq_lens = seq_lens;
  sa.block_table = block_table;
  sa.o = static_cast<char*>(o);
  sa.ws_ml = need ? static_cast<float*>(workspace) : nullptr;
  sa.ws_acc = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ml_bytes(variant, B, plan))
                   : nullptr;
  sa.cap = cap;
  sa.max_pages = paged ? max_pages : 0;
  sa.num_pages = paged ? num_pages : 0;
  sa.window = vi.window;
  sa.n_split = plan.n_split;
  sa.tps = plan.tps;

  SplitFn split = variant == GQA_SLIDING ? pick_split<16, 256>(paged, bf16)
                                         : pick_split<4, 512>(paged, bf16);
  const unsigned groups = (unsigned)(B * vi.KV * plan.n_split);
  ProfRec* pr = prof_slot(2 * variant);
  if (pr) hipEventRecord(pr->start, stream);
  hipLaunchKernelGGL(split, dim3(groups), dim3(kThreads), 0, stream, sa);
  if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
  if (pr) hipEventRecord(pr->stop, stream);

  if (plan.n_split > 1) {
    CombineArgs ca;
    ca.seq_lens = seq_lens;
    ca.ws_ml = sa.ws_ml;
    ca.ws_acc = sa.ws_acc;
    ca.o = sa.o;
    ca.cap = cap;
    ca.window = vi.window;
    ca.n_split = plan.n_split;
    ca.tps = plan.tps;
    CombineFn comb = variant == GQA_SLIDING ? pick_combine<16, 256>(bf16) : pick_combine<4, 512>(bf16);
    ProfRec* pc = prof_slot(2 * variant + 1);
    if (pc) hipEventRecord(pc->start, stream);
    hipLaunchKernelGGL(comb, dim3((unsigned)(B * kHeads)), dim3((unsigned)(vi.D / 4)), 0, stream, ca);
    if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
    if (pc) hipEventRecord(pc->stop, stream);
  }
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_decode_sliding(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                       void* o, int32_t B, int32_t S_max, int32_t dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return run(GQA_SLIDING, false, q, k, v, nullptr, 0, seq_lens, o, B, S_max, 0, dtype, workspace,
             workspace_bytes, stream);
}

int gqa_decode_global(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                      void* o, int32_t B, int32_t S_max, int32_t dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return run(GQA_GLOBAL, false, q, k, v, nullptr, 0, seq_lens, o, B, S_max, 0, dtype, workspace,
             workspace_bytes, stream);
}

int gqa_decode_sliding_paged(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, int32_t max_pages,
                             const int32_t* seq_lens, void* o, int32_t B, int32_t num_pages,
                             int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return run(GQA_SLIDING, true, q, k_pool, v_pool, block_table, max_pages, seq_lens, o, B, 0,
             num_pages, dtype, workspace, workspace_bytes, stream);
}

int gqa_decode_global_paged(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, void* o, int32_t B, int32_t num_pages,
                            int32_t dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return run(GQA_GLOBAL, true, q, k_pool, v_pool, block_table, max_pages, seq_lens, o, B, 0,
             num_pages, dtype, workspace, workspace_bytes, stream);
}

size_t gqa_decode_workspace_bytes(int32_t variant, int32_t B, int32_t capacity) {
  Plan p;
  if (make_plan(variant, B, capacity, &p)) return 0;
  return workspace_bytes(variant, B, p);
}

int gqa_decode_plan(int32_t variant, int32_t B, int32_t capacity, int32_t* n_split,
                    int32_t* tiles_per_split) {
  Plan p;
  int rc = make_plan(variant, B, capacity, &p);
  if (rc) return rc;
  if (n_split) *n_split = p.n_split;
  if (tiles_per_split) *tiles_per_split = p.tps;
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

int gqa_hbm_read_probe(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return GQA_ERR_NULL;
  if (bytes == 0 || bytes % 16) return GQA_ERR_SHAPE;
  if (!aligned16(src)) return GQA_ERR_ALIGN;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(2048), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
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
    hipEventDestroy(r.start);
    hipEventDestroy(r.stop);
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
    hipEventDestroy(r.start);
    hipEventDestroy(r.stop);
  }
  g_prof.clear();
  g_prof_used = 0;
  g_prof_on = false;
  return rc;
}

}  // extern "C"
