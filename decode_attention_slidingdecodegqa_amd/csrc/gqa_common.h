// gqa_common.h -- constants, vector types and device helpers shared by the
// decode (gqa_decode.hip) and prefill (gqa_prefill.hip) kernels of the gfx950
// decode-attention library, plus the launch-timing hooks they share.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gqa_decode.h"

namespace {

constexpr int kHeads = 32;
constexpr int kPage = 16;
constexpr int kTile = 16;  // positions per tile: one page
constexpr int kWaves = 4;  // waves per work-group
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxBatch = 256;
constexpr int kMaxSeq = 262144;
constexpr int kSlidingWindow = 1024;
constexpr float kLog2e = 1.4426950408889634f;
// raise the softmax reference max only when a tile exceeds it by more than
// this (natural-log units): weights stay below e^8
constexpr float kRescaleGap = 8.0f;
// persistent waves per launch: the 1024 SIMDs of a 256-CU part at the
// occupancy of the variant's bf16 kernel (2 waves/SIMD sliding, 1 global)
constexpr int kWavesSliding = 2048;
constexpr int kWavesGlobal = 1024;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

// Sixteen positions of zeros in the widest row layout of any variant
// (16 kv heads x 256 f32, the same bytes as 4 x 512 f32): the rows a kernel
// reads in place of a page whose id lies outside the pool, so that such a page
// is never dereferenced and no other cache memory stands in for it.  Device
// code only reads it; a __device__ array without initializer is zero-filled
// when the code object is loaded.
constexpr size_t kZeroPageBytes = (size_t)kPage * 16 * 256 * 4;
__device__ __attribute__((aligned(256))) u32x4 g_zero_page[kZeroPageBytes / 16];

__device__ inline const char* zero_page() { return reinterpret_cast<const char*>(g_zero_page); }

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

// Two floats rounded to bf16 (RNE) and packed, the first in the low half: one
// v_cvt_pk_bf16_f32.
__device__ inline unsigned bf16_pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
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

// Compile-time geometry of one variant.
template <int KV, int D, bool BF16>
struct Geo {
  static constexpr int G = kHeads / KV;             // query heads per kv head
  static constexpr int E = Elem<BF16>::E;           // elements per 16-byte chunk
  static constexpr int EB = Elem<BF16>::bytes;      // bytes per element
  static constexpr int ROW = D * EB;                // bytes of one head row
  static constexpr size_t POS = (size_t)KV * D * EB;  // bytes between positions
  static constexpr int NCH = D / E;                 // 16-byte chunks per row
  static constexpr int KCH = NCH / 4;               // key chunks per lane (chunk 4t+j)
  static constexpr int VBLK = NCH / 16;             // value chunks per lane and row (r+16*blk)
  static constexpr int RUN = 4 * E;                 // contiguous d values per lane and blk
  static constexpr int QPL = (G * NCH + 63) / 64;   // query chunks per lane when staging
};

// The calling wave's online-softmax state for the heads of one unit.
template <int KV, int D, bool BF16>
struct WaveState {
  using Gm = Geo<KV, D, BF16>;
  f32x4 acc[Gm::VBLK][Gm::E];  // O^T: lane (r, j) holds head r, d = 16E*blk + 4E*j + E*i + e
  float m;                     // reference max of head r (equal on the 4 lanes of a column)
  float l;                     // this lane's share of the sum of weights
};

// Writes the wave's O row of head r (lane (r, j), r < G, owns the runs
// d = 16E*blk + 4E*j + [0, 4E)) scaled by inv, in the output dtype.
template <int KV, int D, bool BF16>
__device__ __forceinline__ void store_o(const WaveState<KV, D, BF16>& st, char* o_row, float inv) {
  using Gm = Geo<KV, D, BF16>;
  constexpr int E = Gm::E, EB = Gm::EB, VBLK = Gm::VBLK;
  const int j = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int blk = 0; blk < VBLK; ++blk) {
    char* dst = o_row + (size_t)(16 * E * blk + 4 * E * j) * EB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the E values d = 16E*blk + 4E*j + E*i + e, e = 0..E-1: one 16-byte chunk
      if constexpr (BF16) {
        u32x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = bf16_pack2(st.acc[blk][2 * q][i] * inv, st.acc[blk][2 * q + 1][i] * inv);
        *reinterpret_cast<u32x4*>(dst + 16 * i) = w;
      } else {
        *reinterpret_cast<f32x4*>(dst + 16 * i) =
            f32x4{st.acc[blk][0][i], st.acc[blk][1][i], st.acc[blk][2][i], st.acc[blk][3][i]} * inv;
      }
    }
  }
}

// ---------------------------------------------------------------- host side

struct VariantInfo {
  int KV, D, window, waves;
};

inline bool variant_info(int variant, VariantInfo* vi) {
  if (variant == GQA_SLIDING) {
    *vi = {16, 256, kSlidingWindow, kWavesSliding};
    return true;
  }
  if (variant == GQA_GLOBAL) {
    *vi = {4, 512, 0, kWavesGlobal};
    return true;
  }
  return false;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

namespace gqa_detail {
// Launch timing for measurement (see gqa_profile_begin): the slot recorded
// for a launch of `kind` on `stream` (-1 while timing is off), then its end.
__attribute__((visibility("hidden"))) int prof_begin(int kind, hipStream_t stream);
__attribute__((visibility("hidden"))) void prof_end(int slot, hipStream_t stream);
}  // namespace gqa_detail
