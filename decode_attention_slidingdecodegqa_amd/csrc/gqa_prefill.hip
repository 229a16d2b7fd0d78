// gqa_prefill.hip -- gfx950 prefill / chunked-prefill attention for the
// Gemma-4-31B text decoder (both attention geometries of the decode kernels,
// with the causal and sliding masks of the architecture page's compact
// forward pass).  The C ABI is declared in include/gqa_decode.h.

#include <algorithm>
#include <atomic>

#include "gqa_common.h"

namespace {

// ----------------------------------------------------------------- prefill
// Attention of a chunk of new tokens per sequence (prefill / chunked prefill),
// the chunk's K/V rows already in the cache: query row n of sequence b
// (cu_q[b] <= n < cu_q[b+1], T_b rows) sits at position p = L_b - T_b + t and
// attends to the keys its mask keeps (global: s <= p; sliding: p - W < s <= p).
//
// Work: the query rows of one (sequence, kv head g) form T_b*G columns
// (token-major, the G heads of a token adjacent); a wave takes 16 of them, a
// work-group 64 or 128.  The work-group walks the union of its columns' key
// ranges in steps of PT positions (bf16: 32, two 16-key MFMA halves, or 64 on
// the sliding layer; f32: 16): each K/V step is fetched once with coalesced 16-byte loads into a
// double-buffered LDS tile with padded rows (operand reads free of bank
// conflicts, every operand address a lane base plus an immediate), which all
// waves use with every MFMA column masked to its own range.  bf16 P@V runs on 16x16x32 MFMAs over both halves
// of a step.  Under a windowed mask, work-groups of one (b, g) are placed on
// one XCD so their shared tiles stay in that XCD's L2; under the full causal
// mask they are dealt longest first over all XCDs.  bf16 sliding blocks are
// persistent, one per CU, each taking a list of work-groups.

struct PrefillArgs {
  const char* q;
  const char* k;
  const char* v;
  const int32_t* cu_q;
  const int32_t* seq_lens;
  const int32_t* block_table;
  char* o;
  int32_t B, N, cap, max_pages, num_pages, window;
};

constexpr int kXcds = 8;

// 16-column MFMA blocks per wave.  Two blocks would let every K/V operand read
// from LDS feed two MFMAs, but their queries and accumulators do not fit the
// 256 registers of two waves per SIMD (D = 256: 548 bytes per lane of spills;
// D = 512 needs the whole register file), and one wave per SIMD hides less
// latency (sliding: 1501 us against 1172 us when measured), so every variant
// runs one.
template <int KV, bool BF16>
constexpr int prefill_col_blocks() {
  return 1;
}

// bf16: two waves per SIMD (at most 256 VGPRs each; the library builds this
// file with the MFMA accumulators in VGPRs, so no AGPR is needed)
template <int KV, bool BF16>
constexpr int prefill_waves_per_simd() {
  return BF16 ? 2 : 1;
}

// waves per work-group and key positions per step.  bf16 runs eight waves
// (128 columns) on one K/V tile: each fetched step feeds twice the MFMA work
// of a four-wave group (global: 4.48 ms against 7.09 ms on 2 x 2048 tokens
// after 8192, where the 138 KB double buffer allows one work-group per CU;
// sliding: 0.85 ms against 1.08 ms on 8 x 2048 tokens after 4096).
template <int KV, bool BF16>
constexpr int prefill_waves() {
  return BF16 ? 8 : 4;
}
// The bf16 sliding layer takes 64 keys per step: each barrier, softmax
// reduction and rescale test then serves twice the MFMA work (measured 1%
// faster, 752-755 us against 761-767 on 8 x 2048 tokens after 4096); its
// double buffer (139 KB) still fits one work-group per CU.  The global
// layer's rows are twice as long and keep 32.
template <int KV, bool BF16>
constexpr int prefill_step() {
  return BF16 ? (KV == 16 ? 64 : 32) : 16;
}

// query columns per work-group
template <int KV, bool BF16>
constexpr int prefill_cols_per_wg() {
  return 16 * prefill_col_blocks<KV, BF16>() * prefill_waves<KV, BF16>();
}

// PERSIST: the block takes a list of items (the grid is sized from the CU
// count); otherwise one item per block.
template <int KV, int D, bool PAGED, bool BF16, bool PERSIST>
__global__ __launch_bounds__((64 * prefill_waves<KV, BF16>()), (prefill_waves_per_simd<KV, BF16>())) void gqa_prefill_kernel(
    PrefillArgs a) {
  using Gm = Geo<KV, D, BF16>;
  constexpr int G = Gm::G, E = Gm::E, ROW = Gm::ROW, NCH = Gm::NCH, KCH = Gm::KCH,
                VBLK = Gm::VBLK;
  constexpr size_t POS = Gm::POS;
  constexpr int CB = prefill_col_blocks<KV, BF16>();
  constexpr int CPW = prefill_cols_per_wg<KV, BF16>();  // columns per work-group
  constexpr int PT = prefill_step<KV, BF16>();      // key positions per step
  constexpr int NH = PT / 16;                       // 16-key halves per step
  // padded LDS row strides.  gfx950 serves a 16-byte-per-lane LDS read in
  // groups of 16 lanes that take rows r = 0..7 from one 16-lane quarter and
  // r = 8..15 from the next: the key operand (lane reads row r, chunk j) is
  // conflict-free with 32 bytes of padding, the f32 value operand (rows
  // 4j + i, chunk r) with 64, and the bf16 transposing value reads (rows
  // 4j + r/4, 8 bytes at 8(r%4)) run fastest with 32 (measured: 16 bytes
  // halve the first two to ~125 B/clk per CU)
  constexpr int RSK = ROW + 32;
  constexpr int RSV = BF16 ? ROW + 32 : ROW + 64;
  constexpr int TILE_K = PT * RSK;                  // one K step in LDS
  constexpr int TILE_BYTES = TILE_K + PT * RSV;     // K then V
  constexpr int NW = prefill_waves<KV, BF16>();     // waves per work-group
  constexpr int NT = 64 * NW;                       // threads per work-group
  constexpr int LDPT = 2 * PT * NCH / NT;           // 16-byte chunks per thread per step
  static_assert(LDPT * NT == 2 * PT * NCH, "step split");
  static_assert(NCH >= 64 || (NT % NCH) == 0, "rows per fetch instruction");
  const int lane = threadIdx.x & 63;
  // wave-uniform values go through readfirstlane so that the address math of
  // the tile fetch runs on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int j = lane >> 4;

  // ---- work-groups per sequence (ceil(T_b*G / 64)) and their prefix, in LDS
  __shared__ int s_wg0[kMaxBatch + 1];
  __shared__ int s_cu[kMaxBatch + 1];
  __shared__ int s_len[kMaxBatch];
  // two LDS buffers of one step each ([K, V]), separate variables so that the
  // compiler sees the LDS-DMA into one never aliases the reads of the other
  // (otherwise it waits for the next step's fetch before reading this one)
  __shared__ __attribute__((aligned(16))) char s_kv0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char s_kv1[TILE_BYTES];
  // LDS offset of row `row` of K (which = 0) or V (which = 1) in one buffer
  auto tile_row = [](int which, int row) { return which ? TILE_K + row * RSV : row * RSK; };
  if (threadIdx.x < 64) {
    int cnt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * lane + i;
      cnt[i] = 0;
      if (b < a.B) {
        const int c0 = a.cu_q[b], c1 = a.cu_q[b + 1];
        const int T = c1 > c0 ? c1 - c0 : 0;
        cnt[i] = (T * G + CPW - 1) / CPW;
        s_cu[b] = c0;
        s_len[b] = a.seq_lens[b];
        if (b == a.B - 1) s_cu[a.B] = c1;
      }
    }
    const int lsum = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    int incl = lsum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    int run_b = incl - lsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * lane + i;
      if (b < a.B) s_wg0[b] = run_b;
      run_b += cnt[i];
    }
    if (lane == 63) s_wg0[a.B] = incl;
  }
  __syncthreads();
  // ---- the work-groups of the call, flattened kv head major (item f is
  // work-group f % nwg of kv head f / nwg), and the block's items.  The
  // hardware deals block ids round-robin over the XCDs (gridDim.x is a
  // multiple of 8, so block x runs on XCD x % 8) and each XCD starts its
  // blocks in id order.  The host sizes the grid from an upper bound of the
  // items (one per block) or from the CU count (persistent blocks, each
  // taking a list of items, which saves a block launch and the prefix of
  // cu_q per item); the true count is only known here, and the map spreads
  // that count, not the bound, over the XCDs (an XCD given a larger share
  // finishes last while the others idle).
  // - windowed mask: items of one (b, g) with neighbouring columns share most
  //   of their keys, so XCD x takes a contiguous range of about 1/8 of them,
  //   which its blocks take in turn (the items running together on an XCD are
  //   neighbours and share the tiles in its L2; odd rounds take the slots in
  //   reverse, which evens out a length trend);
  // - full causal mask: a later column block attends to more keys, so the
  //   items are dealt longest first, round-robin over the XCDs, in rounds of
  //   gridDim.x that alternate direction (a persistent block's items then
  //   pair long with short).  Every item of a (b, g) reads that sequence's
  //   keys from position 0, so the L2s still share them.
  const int nwg = s_wg0[a.B];  // work-groups per kv head
  const int total = KV * nwg;
  auto item_at = [&](int k) -> int {
    if (a.window > 0) {
      const int xcd = (int)(blockIdx.x % kXcds), slot = (int)(blockIdx.x / kXcds);
      const int S = (int)(gridDim.x / kXcds);
      const int lo = (int)((long)xcd * total / kXcds), hi = (int)((long)(xcd + 1) * total / kXcds);
      const long f = (long)lo + (long)k * S + ((k & 1) ? S - 1 - slot : slot);
      return f < hi ? (int)f : -1;
    }
    const long P = gridDim.x;
    const long rank = (long)k * P + ((k & 1) ? P - 1 - (long)blockIdx.x : (long)blockIdx.x);
    return rank < total ? (int)(total - 1 - rank) : -1;
  };
  for (int k = 0; k == 0 || PERSIST; ++k) {
  const int f = item_at(k);
  if (f < 0) break;  // the whole work-group leaves together
  const int g = __builtin_amdgcn_readfirstlane(f / nwg);
  const int wg = f % nwg;
  int b = 0;
  {
    int lo_b = 0, hi_b = a.B - 1;
    while (lo_b < hi_b) {
      const int mid = (lo_b + hi_b + 1) >> 1;
      if (s_wg0[mid] <= wg) lo_b = mid;
      else hi_b = mid - 1;
    }
    b = __builtin_amdgcn_readfirstlane(lo_b);
  }
  const int cu = __builtin_amdgcn_readfirstlane(s_cu[b]);
  const int T = __builtin_amdgcn_readfirstlane(s_cu[b + 1]) - cu;
  const int cols = T * G;
  const int L = min(__builtin_amdgcn_readfirstlane(s_len[b]), a.cap);  // clamped for memory safety
  const int wcol0 = (wg - s_wg0[b]) * CPW;  // < cols
  const int col0 = wcol0 + wave * 16 * CB;
  const bool wave_live = col0 < cols;  // dead waves still take part in the barriers

  // ---- this lane's column r of each block: token, head, position, key range
  bool live[CB];
  int t_n[CB], head[CB], p_n[CB], lo_n[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int col = col0 + 16 * cb + r;
    live[cb] = col < cols;
    const int cl = live[cb] ? col : cols - 1;
    t_n[cb] = cl / G;
    head[cb] = g * G + cl % G;
    p_n[cb] = L - T + t_n[cb];
    lo_n[cb] = a.window > 0 ? max(0, p_n[cb] - a.window + 1) : 0;
  }
  // the work-group's key range: the union over its columns (token-major)
  const int wcol_end = min(wcol0 + CPW, cols);
  const int p_last = L - T + (wcol_end - 1) / G;
  const int p_first = max(L - T + wcol0 / G, 0);
  const int range_lo = a.window > 0 ? max(0, p_first - a.window + 1) : 0;
  const int range_hi = p_last;  // inclusive

  // bf16: acc[blk][e] is the O^T tile t = E*blk + e, lane (r, j) holding
  // d = 16t + 4j + i of column r; lsum[cb] is the column's sum of weights
  // (the same on all four lanes of the column), accumulated by an MFMA
  WaveState<KV, D, BF16> st[CB];
  f32x4 lsum[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    lsum[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
      for (int e = 0; e < E; ++e) st[cb].acc[blk][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    st[cb].m = -INFINITY;
    st[cb].l = 0.f;
  }

  if (range_hi >= 0) {
    // ---- the lane's query operands: column r, chunks 4c+j (bf16: registers;
    // f32, a parity case, reads them from global memory at every step)
    u32x4 qreg[CB][BF16 ? KCH : 1];
    const char* qsrc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      qsrc[cb] = a.q + ((size_t)(cu + t_n[cb]) * kHeads + head[cb]) * ROW;
      if constexpr (BF16) {
#pragma unroll
        for (int c = 0; c < KCH; ++c)
          qreg[cb][c] = live[cb] ? load16(qsrc[cb] + (4 * c + j) * 16) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    const int32_t* bt = PAGED ? a.block_table + (size_t)b * a.max_pages : nullptr;
    const int last_page = range_hi / kPage;
    // block-table entries of 64 consecutive pages, one per lane, refilled when
    // a step reaches the next 64 (a per-step load of the entry would stall
    // every step on its latency)
    int bt_chunk = -1, bt_lane = 0;

    // ---- cooperative step fetch.  Rows are clamped into the range (every step
    // lies within [range_lo & ~(PT-1), range_hi], so a clamped row stays in
    // the step's pages).  Rows of at least 1 KiB go straight to LDS (one
    // 16-byte-per-lane LDS-DMA load per KiB: LDS address = base + 16*lane, all
    // other addressing wave-uniform); shorter rows go through registers
    // (thread t takes chunks t + 256u of the K+V step).
    constexpr bool DMA = ROW % 1024 == 0;
    constexpr int IPR = DMA ? ROW / 1024 : 1;       // DMA loads per row
    constexpr int DMA_PER_WAVE = 2 * PT * IPR / NW;
    u32x4 ld[DMA ? 1 : LDPT];
    // register path: thread t stages chunk t % NCH of rows t / NCH + (256/NCH)*u
    const int ld_row0 = threadIdx.x / NCH;
    const int ld_c = threadIdx.x % NCH;
    static_assert(DMA || (NT / NCH <= 16 && 16 % (NT / NCH) == 0),
                  "register staging: a thread's rows stay within one 16-row half");
    const char* const k_base = a.k;
    const char* const v_base = a.v;
    auto fetch = [&](int step, int& okbits, auto& dst) {
      const int pos0 = step * PT;
      // offsets of the step's 16-row halves in the cache (wave-uniform); a
      // page id outside the pool is never dereferenced: its half reads the
      // library's zero page instead (half_ptr) and its keys are masked in
      // compute().  One offset per half keeps the scalar registers of the
      // fetch as few as a plain offset needs.
      size_t base[NH];
      okbits = 0;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        if constexpr (PAGED) {
          const int pi = pos0 / kPage + h;
          if ((pi >> 6) != bt_chunk) {
            bt_chunk = pi >> 6;
            const int e = 64 * bt_chunk + lane;
            bt_lane = e <= last_page ? bt[e] : 0;
          }
          const int page = __builtin_amdgcn_readlane(bt_lane, pi & 63);
          const bool ok = page >= 0 && page < a.num_pages;
          okbits |= ok ? (1 << h) : 0;
          base[h] = ((size_t)(ok ? page : 0) * kPage * KV + g) * (size_t)ROW;
        } else {
          okbits |= 1 << h;
          base[h] = (((size_t)b * a.cap + pos0 + 16 * h) * KV + g) * (size_t)ROW;
        }
      }
      // rows of half h of K (which = 0) or V (which = 1); the cache bases are
      // selected as values (selecting the argument fields themselves made the
      // compiler copy the argument block to scratch memory)
      auto half_ptr = [&](int which, int h) -> const char* {
        if (PAGED && !((okbits >> h) & 1)) return zero_page() + (size_t)g * ROW;
        // selects on the bits of h (a runtime index into base[] would put the
        // array in scratch memory)
        size_t off = base[0];
        if constexpr (NH == 2) {
          off = (h & 1) ? base[1] : base[0];
        } else if constexpr (NH == 4) {
          const size_t lo = (h & 1) ? base[1] : base[0];
          const size_t hi = (h & 1) ? base[3] : base[2];
          off = (h & 2) ? hi : lo;
        }
        return (which ? v_base : k_base) + off;
      };
      if constexpr (DMA) {
        // LDS-DMA through buffer descriptors, one per K/V and 16-row half of
        // the step, each spanning those 16 rows: the row's offset goes in the
        // scalar offset and 16*lane in the vector offset, so a load writes
        // LDS base + 16*lane.  (The flat form of this load makes the compiler
        // wait for every outstanding LDS read at each use, serialising the
        // operand reads of the step being computed.)
        auto dma = [&](int which, int h, int row_in_half, int part, int lds_off) {
          // the descriptor's base is wave-uniform: keep it in scalar registers
          const uint64_t addr = (uint64_t)half_ptr(which, NH == 1 || h == 0 ? 0 : NH - 1);
          const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
          const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
          const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(((uint64_t)hi << 32) | lo), 0, 16 * (int)POS, 0x00020000);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rsrc, (__attribute__((address_space(3))) void*)&dst[lds_off], 16,
              lane * 16 + part * 1024, row_in_half * (int)POS, 0, 0);
        };
        // interior step (one load per row): wave w loads rows w + NW*i, so K/V
        // and the half of load i are compile-time (no clamp)
        constexpr bool FAST = IPR == 1 && (PT % NW) == 0 && (16 % NW) == 0;
        if (FAST && pos0 >= range_lo && pos0 + PT - 1 <= range_hi) {
#pragma unroll
          for (int i = 0; i < (FAST ? DMA_PER_WAVE : 0); ++i) {
            constexpr int RPW = PT / NW;                 // loads per wave and K (or V)
            const int which = i / RPW;                   // 0: K, 1: V
            const int rin = NW * (i % RPW);              // + wave: row within the step
            dma(which, NH == 1 ? 0 : rin / 16, wave + rin % 16, 0, tile_row(which, wave + rin));
          }
        } else {
#pragma unroll
          for (int i = 0; i < DMA_PER_WAVE; ++i) {
            const int inst = wave + NW * i;  // wave-uniform
            const int which = inst / (PT * IPR);
            const int row = (inst / IPR) % PT;
            const int part = inst % IPR;
            const int rel = min(max(pos0 + row, range_lo), range_hi) - pos0;  // in [0, PT)
            dma(which, NH == 1 ? 0 : rel >> 4, rel & 15, part, tile_row(which, row) + part * 1024);
          }
        }
      } else if (pos0 >= range_lo && pos0 + PT - 1 <= range_hi) {
        // an interior step needs no clamp: row, K/V and page half of chunk u
        // are compile-time offsets from the thread's (row0, column chunk)
#pragma unroll
        for (int u = 0; u < LDPT; ++u) {
          constexpr int RPU = NT / NCH;                   // rows per u
          const int which = (RPU * u) / PT;               // 0: K, 1: V
          const int rin = (RPU * u) % PT;                 // + row0 < 16 within its half
          const int h = rin / 16;
          const size_t off = (size_t)(ld_row0 + rin % 16) * POS + ld_c * 16;
          ld[u] = load16(half_ptr(which, NH == 1 ? 0 : h) + off);
        }
      } else {
#pragma unroll
        for (int u = 0; u < LDPT; ++u) {
          const int q = threadIdx.x + NT * u;
          const int which = q / (PT * NCH);  // 0: K, 1: V
          const int row = (q / NCH) % PT;
          const int c = q % NCH;
          const int rel = min(max(pos0 + row, range_lo), range_hi) - pos0;  // in [0, PT)
          const int h = rel >> 4;
          const size_t off = (size_t)(rel & 15) * POS + c * 16;
          ld[u] = load16(half_ptr(which, h) + off);
        }
      }
    };
    auto stash = [&](auto& dst) {
      if constexpr (!DMA) {
#pragma unroll
        for (int u = 0; u < LDPT; ++u) {
          constexpr int RPU = NT / NCH;
          const int which = (RPU * u) / PT;
          const int row = ld_row0 + (RPU * u) % PT;
          *reinterpret_cast<u32x4*>(&dst[tile_row(which, row) + ld_c * 16]) = ld[u];
        }
      } else {
        // the step's LDS-DMA loads have landed before the barrier that follows
        __builtin_amdgcn_s_waitcnt(0);
      }
    };

    const int step_begin = range_lo / PT, step_end = range_hi / PT;  // inclusive
    const int kbase = r * RSK + j * 16;            // key operand: row r (+16h), chunk 4c+j
    // value operand.  bf16: transposing 8-byte reads, lane (r, j) at row
    // 4j + r/4 (+16 for the second half), d = 16t + 4(r%4); lane (r, j) then
    // holds V[4j + e][16t + r] (e = 0..3), the A operand of the tile-t MFMA.
    // f32: rows 4j+i (+16h), chunk r+16blk
    const int vbase = BF16 ? TILE_K + (4 * j + (r >> 2)) * RSV + 8 * (r & 3)
                           : TILE_K + 4 * j * RSV + r * 16;
    // a wave-uniform step that lies inside every column's key range needs no
    // mask (most steps: the mask only bites on the diagonal and the window edge)
    int w_lo = lo_n[0], w_hi = p_n[0];
#pragma unroll
    for (int cb = 1; cb < CB; ++cb) {
      w_lo = max(w_lo, lo_n[cb]);
      w_hi = min(w_hi, p_n[cb]);
    }
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      w_lo = max(w_lo, __shfl_xor(w_lo, d));
      w_hi = min(w_hi, __shfl_xor(w_hi, d));
    }
    w_lo = __builtin_amdgcn_readfirstlane(w_lo);
    w_hi = __builtin_amdgcn_readfirstlane(w_hi);
    auto compute = [&](int step, int ok_cur, auto& cur, auto&& after_qk) {
        const char* kt = cur + kbase;
        const char* vt = cur + vbase;
        // logits z[cb][h][key 16h+4j+i][column r of block cb]; each K operand
        // read from LDS feeds the MFMAs of every column block
        f32x4 z[CB][NH];
        if constexpr (BF16) {
          // the step's 2*KCH key operands (half h, chunk c: n = KCH*h + c) in a
          // software pipeline: the read of operand n + KDEPTH is issued before
          // the MFMA of operand n, so KDEPTH LDS reads are in flight
          constexpr int NK = NH * KCH, KDEPTH = 4;
          f32x4 zz[CB][NH][2];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int h = 0; h < NH; ++h) zz[cb][h][0] = zz[cb][h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
          auto kread = [&](int n) {
            return *reinterpret_cast<const u32x4*>(kt + (n / KCH) * 16 * RSK + (n % KCH) * 64);
          };
          // the wave in its QK^T phase runs at a raised priority: the eight
          // waves leave each step's barrier together, and the raised wave's
          // MFMAs and key reads issue ahead of the other wave of its SIMD,
          // which drifts into its softmax and PV products meanwhile
          // (measured 3-7% faster on the global layer, 1-2% on the sliding)
          __builtin_amdgcn_s_setprio(1);
          u32x4 kring[KDEPTH];
#pragma unroll
          for (int n = 0; n < KDEPTH; ++n) kring[n] = kread(n);
#pragma unroll
          for (int n = 0; n < NK; ++n) {
            const u32x4 kop = kring[n % KDEPTH];
            if (n + KDEPTH < NK) kring[n % KDEPTH] = kread(n + KDEPTH);
            const int h = n / KCH, c = n % KCH;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
              zz[cb][h][c & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, kop), __builtin_bit_cast(bf16x8, qreg[cb][c]),
                  zz[cb][h][c & 1], 0, 0, 0);
              if (c == KCH - 1) z[cb][h] = zz[cb][h][0] + zz[cb][h][1];
            }
          }
          // keep the pipeline order through scheduling: the first KDEPTH reads,
          // then each operand's MFMAs followed by the read KDEPTH ahead
          __builtin_amdgcn_sched_group_barrier(0x100, KDEPTH, 0);
#pragma unroll
          for (int n = 0; n < NK; ++n) {
            __builtin_amdgcn_sched_group_barrier(0x008, CB, 0);
            if (n + KDEPTH < NK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_s_setprio(0);
        } else {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          f32x4 z0[CB], z1[CB];
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            z0[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
            z1[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          const char* kh = kt + h * 16 * RSK;
          {
#pragma unroll
            for (int c = 0; c < KCH; ++c) {
              const u32x4 kc = *reinterpret_cast<const u32x4*>(kh + c * 64);
              const u32x4 qc =
                  live[0] ? load16(qsrc[0] + (4 * c + j) * 16) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
              for (int e = 0; e < 4; e += 2) {
                z0[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(chunk_f32(kc, e), chunk_f32(qc, e),
                                                             z0[0], 0, 0, 0);
                z1[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(chunk_f32(kc, e + 1),
                                                             chunk_f32(qc, e + 1), z1[0], 0, 0, 0);
              }
            }
          }
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) z[cb][h] = z0[cb] + z1[cb];
        }
        }
        after_qk();
        // each column keeps the keys of its own mask; online softmax per block
        const int pos0 = step * PT;
        float p[CB][NH][4];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          WaveState<KV, D, BF16>& sc = st[cb];
          const bool interior = ok_cur == (1 << NH) - 1 && pos0 >= w_lo && pos0 + PT - 1 <= w_hi;
          if (!interior) {
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int s_ = pos0 + 16 * h + 4 * j + i;
                if (!(((ok_cur >> h) & 1) && live[cb] && s_ >= lo_n[cb] && s_ <= p_n[cb]))
                  z[cb][h][i] = -INFINITY;
              }
          }
          float tmax = -INFINITY;
#pragma unroll
          for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, z[cb][h][i]);
          // the column's max over the four lanes (r, 0..3): lane swaps across
          // 16-lane rows, then across the 32-lane halves
          {
            const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax),
                                                              __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
            const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                              __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
          }
          const bool grow = tmax > sc.m + kRescaleGap;
          if (__any(grow)) {
            const float m_next = grow ? tmax : sc.m;
            const float alpha = exp2_fast((sc.m - (m_next == -INFINITY ? 0.f : m_next)) * kLog2e);
            if (grow) {
              sc.l *= alpha;
              lsum[cb] *= alpha;
#pragma unroll
              for (int blk = 0; blk < VBLK; ++blk)
#pragma unroll
                for (int e = 0; e < E; ++e) sc.acc[blk][e] *= alpha;
            }
            sc.m = m_next;
          }
          // exp(z - m) as 2^(z log2e - m log2e): one fused multiply-add per weight
          const float m_log = (sc.m == -INFINITY ? 0.f : sc.m) * kLog2e;
#pragma unroll
          for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) p[cb][h][i] = exp2_fast(fmaf(z[cb][h][i], kLog2e, -m_log));
        }
        if constexpr (BF16) {
          // P^T operands of each 32-key pair of halves hp (halves 2hp, 2hp+1):
          // k-slots 8j+e <-> keys 4j+e (e < 4), 16+4j+e-4 (e >= 4)
          constexpr int NP = NH / 2;
          u32x4 pt[CB][NP];
          const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int hp = 0; hp < NP; ++hp) {
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                pt[cb][hp][2 * h] = bf16_pack2(p[cb][2 * hp + h][0], p[cb][2 * hp + h][1]);
                pt[cb][hp][2 * h + 1] = bf16_pack2(p[cb][2 * hp + h][2], p[cb][2 * hp + h][3]);
              }
              // the column sums of the bf16 weights the P@V MFMAs use
              lsum[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, ones), __builtin_bit_cast(bf16x8, pt[cb][hp]),
                  lsum[cb], 0, 0, 0);
            }
          }
#pragma unroll
          for (int t = 0; t < D / 16; ++t) {
#pragma unroll
            for (int hp = 0; hp < NP; ++hp) {
              const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) s16x4*)(vt + 32 * hp * RSV + 32 * t));
              const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) s16x4*)(vt + (32 * hp + 16) * RSV + 32 * t));
              const bf16x8 vop = __builtin_bit_cast(
                  bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
              for (int cb = 0; cb < CB; ++cb)
                st[cb].acc[t / E][t % E] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    vop, __builtin_bit_cast(bf16x8, pt[cb][hp]), st[cb].acc[t / E][t % E], 0, 0,
                    0);
            }
          }
        } else {
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            st[0].l += (p[0][h][0] + p[0][h][1]) + (p[0][h][2] + p[0][h][3]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int blk = 0; blk < VBLK; ++blk) {
                const u32x4 vc =
                    *reinterpret_cast<const u32x4*>(vt + (16 * h + i) * RSV + blk * 256);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  st[0].acc[blk][e] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                      chunk_f32(vc, e), p[0][h][i], st[0].acc[blk][e], 0, 0, 0);
              }
          }
        }
    };

    // one step: fetch the next one into the other buffer, compute on this one,
    // publish the next (one barrier per step); the loop takes steps in pairs so
    // that each buffer is named statically.  The LDS-DMA fetch is issued after
    // the QK^T products: its LDS writes then meet the softmax and PV instead of
    // the key reads every wave issues at the start of the step (measured 3%
    // faster on the global layer); the register-staged fetch is issued first
    int ok_cur, ok_nxt = 0;
    fetch(step_begin, ok_cur, s_kv0);
    stash(s_kv0);
    __syncthreads();
    auto one_step = [&](int step, auto& cur, auto& nxt) {
      const bool more = step < step_end;
      if (!DMA && more) fetch(step + 1, ok_nxt, nxt);
      auto fetch_dma = [&] {
        if constexpr (DMA) {
          if (more) fetch(step + 1, ok_nxt, nxt);
        }
      };
      if (wave_live) compute(step, ok_cur, cur, fetch_dma);
      else fetch_dma();
      if (more) stash(nxt);
      __syncthreads();
      ok_cur = ok_nxt;
    };
    for (int step = step_begin; step <= step_end; step += 2) {
      one_step(step, s_kv0, s_kv1);
      if (step + 1 > step_end) break;
      one_step(step + 1, s_kv1, s_kv0);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      if constexpr (BF16) {
        st[cb].l = lsum[cb][0];
      } else {
        st[cb].l += __shfl_xor(st[cb].l, 16);
        st[cb].l += __shfl_xor(st[cb].l, 32);
      }
    }
  }
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    if (live[cb]) {
      const float inv = st[cb].l > 0.f ? 1.f / st[cb].l : 0.f;  // before position 0: zero row
      char* orow = a.o + ((size_t)(cu + t_n[cb]) * kHeads + head[cb]) * ROW;
      if constexpr (BF16) {
        // tile t: d = 16t + 4j + [0, 4), 8 bytes per lane
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          const f32x4 x = st[cb].acc[t / E][t % E] * inv;
          *reinterpret_cast<u32x2*>(orow + (16 * t + 4 * j) * 2) =
              u32x2{bf16_pack2(x[0], x[1]), bf16_pack2(x[2], x[3])};
        }
      } else {
        store_o<KV, D, BF16>(st[cb], orow, inv);
      }
    }
  }
  }  // items
}

typedef void (*PrefillFn)(PrefillArgs);

// bf16 sliding prefill blocks are persistent, one per CU (one work-group per
// CU fits the registers and LDS).  The global layer's items are long (an
// item's start is about 1% of one) and run one per block.
template <int KV, bool BF16>
constexpr bool prefill_persist() {
  return BF16 && KV == 16;
}

// compute units of the current device (cached per device; 256 on MI355X)
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < kXcds)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int KV, int D>
PrefillFn pick_prefill(bool paged, bool bf16) {
  if (paged)
    return bf16 ? gqa_prefill_kernel<KV, D, true, true, prefill_persist<KV, true>()>
                : gqa_prefill_kernel<KV, D, true, false, false>;
  return bf16 ? gqa_prefill_kernel<KV, D, false, true, prefill_persist<KV, true>()>
              : gqa_prefill_kernel<KV, D, false, false, false>;
}

constexpr int kMaxPrefillRows = 1 << 24;  // query rows per call
constexpr int kProfPrefill = 9;           // profiling kinds 9 (sliding), 10 (global)

int run_prefill(int variant, bool paged, const void* q, const void* k, const void* v,
                const int32_t* block_table, int32_t max_pages, const int32_t* cu_q,
                const int32_t* seq_lens, void* o, int32_t B, int32_t N, int32_t S_max,
                int32_t num_pages, int32_t dtype, void* stream_, int32_t window = -1) {
  if (!q || !k || !v || !cu_q || !seq_lens || !o || (paged && !block_table)) return GQA_ERR_NULL;
  if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_DTYPE;
  VariantInfo vi;
  if (!variant_info(variant, &vi)) return GQA_ERR_DTYPE;
  // window < 0: the variant's own (1024 sliding, none global); otherwise a
  // runtime window of the sliding geometry
  if (window >= 0 && (variant != GQA_SLIDING || window < 1 || window > kMaxSeq))
    return GQA_ERR_SHAPE;
  if (B < 1 || B > kMaxBatch || N < 1 || N > kMaxPrefillRows) return GQA_ERR_SHAPE;
  int cap;
  if (paged) {
    if (max_pages < 1 || max_pages > kMaxSeq / kPage || num_pages < 1) return GQA_ERR_SHAPE;
    cap = max_pages * kPage;
  } else {
    if (S_max < 1 || S_max > kMaxSeq) return GQA_ERR_SHAPE;
    cap = S_max;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GQA_ERR_ALIGN;
  PrefillArgs pa;
  pa.q = static_cast<const char*>(q);
  pa.k = static_cast<const char*>(k);
  pa.v = static_cast<const char*>(v);
  pa.cu_q = cu_q;
  pa.seq_lens = seq_lens;
  pa.block_table = block_table;
  pa.o = static_cast<char*>(o);
  pa.B = B;
  pa.N = N;
  pa.cap = cap;
  pa.max_pages = paged ? max_pages : 0;
  pa.num_pages = paged ? num_pages : 0;
  pa.window = window >= 0 ? window : vi.window;
  const bool bf16 = dtype == GQA_BF16;
  PrefillFn fn = variant == GQA_SLIDING ? pick_prefill<16, 256>(paged, bf16)
                                        : pick_prefill<4, 512>(paged, bf16);
  // an upper bound of the items, KV * sum_b ceil(T_b*G/CPW) (the kernel finds
  // the true count; blocks without an item leave at once), or persistent
  // blocks, one per CU, each taking a list of items.  The kernel's XCD map
  // needs a multiple of 8 blocks.
  const int G = kHeads / vi.KV;
  const int cpw = variant == GQA_SLIDING
                      ? (bf16 ? prefill_cols_per_wg<16, true>() : prefill_cols_per_wg<16, false>())
                      : (bf16 ? prefill_cols_per_wg<4, true>() : prefill_cols_per_wg<4, false>());
  int64_t n_items = (((int64_t)N * G + cpw - 1) / cpw + B) * vi.KV;
  const bool persist = variant == GQA_SLIDING
                           ? (bf16 ? prefill_persist<16, true>() : prefill_persist<16, false>())
                           : (bf16 ? prefill_persist<4, true>() : prefill_persist<4, false>());
  if (persist) n_items = std::min<int64_t>(n_items, device_cus() / kXcds * kXcds);
  n_items = (n_items + kXcds - 1) / kXcds * kXcds;
  const unsigned grid_x = (unsigned)n_items;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  const int slot = gqa_detail::prof_begin(kProfPrefill + variant, stream);
  const unsigned threads = 64u * (unsigned)(variant == GQA_SLIDING
                                                ? (bf16 ? prefill_waves<16, true>() : prefill_waves<16, false>())
                                                : (bf16 ? prefill_waves<4, true>() : prefill_waves<4, false>()));
  hipLaunchKernelGGL(fn, dim3(grid_x), dim3(threads), 0, stream, pa);
  if (hipGetLastError() != hipSuccess) return GQA_ERR_HIP;
  gqa_detail::prof_end(slot, stream);
  return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_prefill_sliding(const void* q, const void* k, const void* v, const int32_t* cu_q,
                        const int32_t* seq_lens, void* o, int32_t B, int32_t N, int32_t S_max,
                        int32_t dtype, void* stream) {
  return run_prefill(GQA_SLIDING, false, q, k, v, nullptr, 0, cu_q, seq_lens, o, B, N, S_max, 0,
                     dtype, stream);
}

int gqa_prefill_global(const void* q, const void* k, const void* v, const int32_t* cu_q,
                       const int32_t* seq_lens, void* o, int32_t B, int32_t N, int32_t S_max,
                       int32_t dtype, void* stream) {
  return run_prefill(GQA_GLOBAL, false, q, k, v, nullptr, 0, cu_q, seq_lens, o, B, N, S_max, 0,
                     dtype, stream);
}

int gqa_prefill_sliding_paged(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, int32_t max_pages, const int32_t* cu_q,
                              const int32_t* seq_lens, void* o, int32_t B, int32_t N,
                              int32_t num_pages, int32_t dtype, void* stream) {
  return run_prefill(GQA_SLIDING, true, q, k_pool, v_pool, block_table, max_pages, cu_q,
                     seq_lens, o, B, N, 0, num_pages, dtype, stream);
}

int gqa_prefill_global_paged(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_table, int32_t max_pages, const int32_t* cu_q,
                             const int32_t* seq_lens, void* o, int32_t B, int32_t N,
                             int32_t num_pages, int32_t dtype, void* stream) {
  return run_prefill(GQA_GLOBAL, true, q, k_pool, v_pool, block_table, max_pages, cu_q, seq_lens,
                     o, B, N, 0, num_pages, dtype, stream);
}

int gqa_prefill_sliding_window(const void* q, const void* k, const void* v, const int32_t* cu_q,
                               const int32_t* seq_lens, void* o, int32_t B, int32_t N,
                               int32_t S_max, int32_t window, int32_t dtype, void* stream) {
  if (window < 1) return GQA_ERR_SHAPE;  // (negative is the internal "variant default")
  return run_prefill(GQA_SLIDING, false, q, k, v, nullptr, 0, cu_q, seq_lens, o, B, N, S_max, 0,
                     dtype, stream, window);
}

int gqa_prefill_sliding_window_paged(const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, int32_t max_pages,
                                     const int32_t* cu_q, const int32_t* seq_lens, void* o,
                                     int32_t B, int32_t N, int32_t num_pages, int32_t window,
                                     int32_t dtype, void* stream) {
  if (window < 1) return GQA_ERR_SHAPE;
  return run_prefill(GQA_SLIDING, true, q, k_pool, v_pool, block_table, max_pages, cu_q,
                     seq_lens, o, B, N, 0, num_pages, dtype, stream, window);
}

}  // extern "C"
