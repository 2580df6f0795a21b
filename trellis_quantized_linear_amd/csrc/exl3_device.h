// Device code of the EXL3 linear shared by the kernel translation units:
// codebook and trellis decode, the rotation and epilogue routines, every
// linear kernel template, and their dispatch by kernel form. Included by
// exl3_kernels.hip (rotation, test hooks, launchers) and exl3_linear_bits.hip
// (the linear kernels of one bit width per translation unit, so the widths
// compile in parallel). Everything is in an anonymous namespace: each
// translation unit emits only the kernels it instantiates.
//
// Every regime (1..16 decode rows, 17..128 mid-M rows, 128-row prompt blocks),
// every group and every column view runs the same per-output arithmetic: one
// MFMA shape, the same K chunks per split in ascending order, the splits added
// left to right in fp32, and one epilogue routine. A row's bits therefore do
// not depend on the row count (PR #1467, "The arithmetic": every mid-M form,
// a group member and the group rotation produce exactly what the single-weight
// launch produces).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdio>
#include <type_traits>

#include "exl3_internal.h"

namespace exl3 {
namespace {


typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// gfx9 raw buffer resource, dword 3: 32-bit data format, no swizzle. A raw
// load whose VGPR offset is past num_records returns zero, which pads the
// rows beyond M with zeros without a branch.
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;
// s_waitcnt operand for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (gfx9 encoding: vmcnt[3:0] bits 3:0, expcnt 6:4, lgkmcnt 11:8,
// vmcnt[5:4] bits 15:14).
constexpr int kWaitVmcnt0 = 0x0F70;
// Cache policy of buffer loads and stores that exchange data between
// workgroups: SC1, agent scope (written through / fetched past the XCD's
// non-coherent L2), the same bit LLVM sets for agent-scope atomics here.
constexpr int kAgentScope = 16;
// Cache policy of the weight stream of the 16- and 32-row launches of one
// row block: non-temporal (NT), the words are read once per call and should
// not displace the rotated input. A launch over several row blocks reads
// each block's words once per row block and keeps the normal policy, so the
// later row blocks find them in the last-level cache (3-bit {gate, up}
// spread launch at 32 / 48 rows 57 -> 54 / 85 -> 79 us; chained or
// exchanged 16-row forms: q/k/v at 24 rows 18.4 -> 16.6 us, down at 40 rows
// 34.2 -> 30.2 us; the normal policy costs 6-8 % at one row block).
constexpr int kStreamOnce = 2;
constexpr int kStreamAgain = 0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

// ---------------------------------------------------------------- codebook
// cb(s) = ((40503*s + 31161) mod 2^16 AND 0x8FFF) OR 0x3000, two states per
// 32-bit register: one packed 16-bit multiply-add and one and-or.
constexpr unsigned short kCbMul = 40503;
constexpr unsigned short kCbAdd = 31161;
constexpr uint32_t kCbMask2 = 0x8FFF8FFFu;
constexpr uint32_t kCbBase2 = 0x30003000u;

// The and-or constants live in VGPRs: gfx9 VOP3 instructions take no
// literal, and with the constants in registers the mask and the or fuse into
// one v_and_or_b32 per two weights.
struct CbConst {
  uint32_t mask2, base2;
};

__device__ __forceinline__ CbConst cb_const() {
  CbConst c{kCbMask2, kCbBase2};
  asm volatile("" : "+v"(c.mask2), "+v"(c.base2));
  return c;
}

__device__ __forceinline__ uint32_t codebook2(uint32_t states2, const CbConst &cb) {
  const u16x2 s = __builtin_bit_cast(u16x2, states2);
  const u16x2 t = s * u16x2{kCbMul, kCbMul} + u16x2{kCbAdd, kCbAdd};
  return (__builtin_bit_cast(uint32_t, t) & cb.mask2) | cb.base2;
}

// ------------------------------------------------------------ trellis decode
//
// MFMA B operand of v_mfma_f32_16x16x32_f16: lane l holds 8 K values of
// column l%16, K rows 8*(l/16) .. +7 of the 32-deep chunk. A chunk spans two
// tile rows (kt = 2c, 2c+1); lane group g = l/16 reads tile row 2c + g/2 and
// half h = g%2 of the column, i.e. weights i = 16*(l%16) + 8h + q, q = 0..7,
// which are consecutive in the tile's stream (the stream walks down a column).
// Those 8 windows start at bit 8*b*j, j = 2*(l%16) + h, and end 7b+16 bits
// later: at most three dwords of the tile, the last ones wrapping to the
// tile's start (tail-biting).
//
// Register r (r = 0..3) of the decoded operand holds window r in its low half
// and window r+4 in its high half ("slot order"); the rotated input Xr is
// stored in the same order, so the MFMA pairs every weight with its own input.

template <int BITS>
struct BitsTraits {
  static constexpr int kDwords = BITS <= 4 ? 2 : 3;     // dwords a lane reads per tile
  static constexpr int kTileBytes = 32 * BITS;
  static constexpr int kTileDwords = 8 * BITS;
  static constexpr bool kAligned = (BITS & 3) == 0;     // every lane's windows start at a dword
};

// Bits [P, P+32) of the 96-bit value (v2:v1:v0).
template <int P>
__device__ __forceinline__ uint32_t bits_at(uint32_t v0, uint32_t v1, uint32_t v2) {
  static_assert(P >= 0 && P < 96, "window outside the lane's dwords");
  if constexpr (P == 0) return v0;
  else if constexpr (P < 32) return __builtin_amdgcn_alignbit(v1, v0, P);
  else if constexpr (P == 32) return v1;
  else if constexpr (P < 64) return __builtin_amdgcn_alignbit(v2, v1, P - 32);
  else if constexpr (P == 64) return v2;
  else return v2 >> (P - 64);
}

// Windows Q (low half) and Q+4 (high half) of a lane whose windows start at
// bits 0, b, 2b, ... of (v2:v1:v0).
template <int BITS, int Q>
__device__ __forceinline__ uint32_t window_pair(uint32_t v0, uint32_t v1, uint32_t v2) {
  constexpr int lo = Q * BITS;
  constexpr int gap = 4 * BITS;
  if constexpr (gap == 16) {
    return bits_at<lo>(v0, v1, v2);
  } else if constexpr (gap < 16) {
    const uint32_t x = bits_at<lo>(v0, v1, v2);
    const uint32_t y = x << (16 - gap);
    return (x & 0xFFFFu) | (y & 0xFFFF0000u);
  } else {
    const uint32_t x = bits_at<lo>(v0, v1, v2);
    const uint32_t y = bits_at<lo + gap - 16>(v0, v1, v2);
    return (x & 0xFFFFu) | (y & 0xFFFF0000u);
  }
}

// Per-lane constants of the B operand stream.
template <int BITS>
struct BLane {
  uint32_t voff[BitsTraits<BITS>::kDwords];  // byte offsets of the lane's dwords in its tile row pair
  uint32_t shift;                            // bit offset of the lane's first window in voff[0]
};

template <int BITS>
__device__ __forceinline__ BLane<BITS> b_lane(int lane) {
  using T = BitsTraits<BITS>;
  BLane<BITS> r;
  const int c = lane & 15, g = lane >> 4;
  const int j = 2 * c + (g & 1);
  const int bj = BITS * j;
  const int d0 = bj >> 2;
  r.shift = 8u * (uint32_t)(bj & 3);
#pragma unroll
  for (int d = 0; d < T::kDwords; ++d) {
    int dw = d0 + d;
    if (dw >= T::kTileDwords) dw -= T::kTileDwords;   // tail-biting wrap inside the tile
    r.voff[d] = (uint32_t)((g >> 1) * 8 * T::kTileBytes + 4 * dw);
  }
  return r;
}

template <int BITS>
__device__ __forceinline__ half8 decode8(const uint32_t (&w)[BitsTraits<BITS>::kDwords], uint32_t shift,
                                        const CbConst &cb) {
  uint32_t v0, v1, v2;
  const uint32_t w2 = BitsTraits<BITS>::kDwords > 2 ? w[BitsTraits<BITS>::kDwords - 1] : 0u;
  if constexpr (BitsTraits<BITS>::kAligned) {
    v0 = w[0]; v1 = w[1]; v2 = w2;
  } else {
    v0 = __builtin_amdgcn_alignbit(w[1], w[0], shift);
    v1 = __builtin_amdgcn_alignbit(w2, w[1], shift);
    v2 = w2 >> shift;
  }
  u32x4 r;
  r[0] = codebook2(window_pair<BITS, 0>(v0, v1, v2), cb);
  r[1] = codebook2(window_pair<BITS, 1>(v0, v1, v2), cb);
  r[2] = codebook2(window_pair<BITS, 2>(v0, v1, v2), cb);
  r[3] = codebook2(window_pair<BITS, 3>(v0, v1, v2), cb);
  return __builtin_bit_cast(half8, r);
}

// ------------------------------------------------------------ conversions

__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ float fp16_to_f32(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ __forceinline__ uint16_t f32_to_fp16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ------------------------------------------------------------ epilogue
//
// A wave finishes 4*NQ rows of one block's Z (rows row0 .. row0 + 4NQ - 1,
// columns col0 .. col0 + 127): lane l, with c = l % 16 and g = l / 16, holds
// z[t][q] = Z[row0 + NQ*g + q][col0 + 16t + c]. With NQ = 4 that is the MFMA
// accumulator layout of a 16-row tile. Per column: times its scale, the
// unnormalised 128-point Sylvester transform by levels h = 1, 2, 4, ..., 64
// in that order (each pair (i, i + h) becomes (a + b, a - b) in fp32), times
// 2^-3 and the column's output sign, then bf16 with round to nearest even.
// The same arithmetic runs in every row regime.
//
// Column bits 0..3 are lane bits: levels 1, 2, 4 and 8 pair lanes c and c ^ h
// of one 16-lane DPP row. Column bits 4..6 are register bits: levels 16, 32
// and 64 pair registers t and t ^ (h / 16). The bf16 rows pass through NQ KB
// of LDS owned by the wave (`scratch`) so that each lane stores 16
// contiguous bytes of a row.

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Value of lane (c ^ H) of the lane's 16-lane row.
template <int H>
__device__ __forceinline__ float row_xor(float v) {
  int x = __float_as_int(v);
  if constexpr (H == 1) {
    x = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);      // quad_perm [1,0,3,2]
  } else if constexpr (H == 2) {
    x = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);      // quad_perm [2,3,0,1]
  } else if constexpr (H == 4) {
    x = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);     // row_half_mirror: c ^ 7
    x = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, true);      // quad_perm [3,2,1,0]: ^ 3
  } else {
    static_assert(H == 8, "lane levels are 1, 2, 4 and 8");
    x = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, true);     // row_ror:8
  }
  return __int_as_float(x);
}

// One lane level: the lower lane of a pair keeps a + b, the upper one a - b.
// With sgn = +1 (lower) or -1 (upper), fma(sgn, v, partner) rounds once, as
// v + partner or partner - v would.
template <int H, int NQ>
__device__ __forceinline__ void lane_level(float (&z)[8][NQ], int c) {
  const float sgn = (c & H) ? -1.0f : 1.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int q = 0; q < NQ; ++q) z[t][q] = __builtin_fmaf(sgn, z[t][q], row_xor<H>(z[t][q]));
}

template <int K, int NQ>
__device__ __forceinline__ void register_level(float (&z)[8][NQ]) {
#pragma unroll
  for (int t = 0; t < 8; ++t)
    if ((t & K) == 0) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float a = z[t][q], b = z[t + K][q];
        z[t][q] = a + b;
        z[t + K][q] = a - b;
      }
    }
}

// The lane's column constants: scales and 2^-3 * output signs of columns
// col0 + 16t + c. (v * 2^-3) * svh == v * (2^-3 * svh): the first product is
// exact. Loaded ahead of the epilogue to hide their latency.
struct EpiCols {
  float sc[8], so[8];
};

__device__ __forceinline__ EpiCols epi_cols(const MemberArgs &m, int col0, int lane) {
  const int c = lane & 15;
  EpiCols e;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    e.sc[t] = fp16_to_f32(m.scales[col0 + 16 * t + c]);
    e.so[t] = 0.125f * fp16_to_f32(m.svh[col0 + 16 * t + c]);
  }
  return e;
}

__device__ __forceinline__ void wave_lds_sync() {
  // a wave's LDS accesses complete in order; keep the compiler from moving
  // the reads of other lanes' writes above them
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int NQ>
__device__ __forceinline__ void epilogue_rows(float (&z)[8][NQ], const EpiCols &ec, int lane, const MemberArgs &m,
                                              int col0, int row0, int M, uint16_t *scratch) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int q = 0; q < NQ; ++q) z[t][q] = z[t][q] * ec.sc[t];
  lane_level<1>(z, c);
  lane_level<2>(z, c);
  lane_level<4>(z, c);
  lane_level<8>(z, c);
  register_level<1>(z);
  register_level<2>(z);
  register_level<4>(z);
  // bf16 (v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN), two
  // columns 16 apart per conversion, into scratch[row][column]
#pragma unroll
  for (int t = 0; t < 8; t += 2)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const bf16x2 h = __builtin_convertvector(f32x2{z[t][q] * ec.so[t], z[t + 1][q] * ec.so[t + 1]}, bf16x2);
      const uint32_t u = __builtin_bit_cast(uint32_t, h);
      uint16_t *row = scratch + (NQ * g + q) * kBlockCols;
      row[16 * t + c] = (uint16_t)(u & 0xFFFFu);
      row[16 * t + 16 + c] = (uint16_t)(u >> 16);
    }
  wave_lds_sync();
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int piece = lane + 64 * i;                  // 16 bytes: row piece/16, columns 8*(piece%16) ..
    const int r = piece >> 4, cc = 8 * (piece & 15);
    if (row0 + r < M) {
      const u32x4 v = *(const u32x4 *)(scratch + r * kBlockCols + cc);
      uint16_t *dst = m.y + (int64_t)(row0 + r) * m.ldy + col0 + cc;
      if (((uintptr_t)dst & 15) == 0) {
        *(u32x4 *)dst = v;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dst[2 * e] = (uint16_t)(v[e] & 0xFFFFu);
          dst[2 * e + 1] = (uint16_t)(v[e] >> 16);
        }
      }
    }
  }
}

// Rows row0 .. row0 + 4NQ - 1 of a block's Z from LDS (row pitch `pitch`
// floats; rows past M may hold anything) through the epilogue. The rows'
// LDS doubles as the wave's bf16 scratch once they are in registers.
template <int NQ>
__device__ __forceinline__ void epilogue_rows_lds(float *zrows, int pitch, const EpiCols &ec, int lane,
                                                  const MemberArgs &m, int col0, int row0, int M) {
  const int c = lane & 15, g = lane >> 4;
  float z[8][NQ];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int q = 0; q < NQ; ++q) z[t][q] = zrows[(NQ * g + q) * pitch + 16 * t + c];
  wave_lds_sync();
  epilogue_rows<NQ>(z, ec, lane, m, col0, row0, M, (uint16_t *)zrows);
}

// ------------------------------------------------------------ rot_in / rot_group
//
// Xr = fp16( FWHT128(X ⊙ suh) · 2^-4 ) per 128-chunk of K, the same
// butterflies as the output transform: levels h = 1, 2, ..., 64 in that order,
// each pair (i, i + h) -> (a + b, a - b) in fp32. One wave per (4 rows,
// 128-chunk), reading X once and rotating it for each member in turn (the
// in-launch rotation: per member and 128-chunk, all M <= 32 rows): lane l
// (c = l % 16, g = l / 16) holds elements 8c .. 8c+7 of row
// 4q + g, so levels 1, 2, 4 pair registers and levels 8, 16, 32, 64 pair
// lanes c ^ 1, c ^ 2, c ^ 4, c ^ 8 of a 16-lane DPP row. Each lane loads and
// stores 16 contiguous bytes; Xr leaves in the MFMA slot order (within each
// group of 8: k0 k4 k1 k5 k2 k6 k3 k7), or in natural order for the test hook,
// either row-major [M][K] or chunk-major [K/32][M][32]. The spread launch
// reads chunk-major: a chunk's 16 rows are then one contiguous 1 KB, 8 whole
// 128-byte lines per load instead of 16 half-used ones whose other halves its
// 16 streaming waves per CU evict from the L1 before the next chunk, and the
// L1's outstanding misses are what the weight stream shares with these loads
// (-5 % on {gate, up} at 16 rows). The 128-row tilings read chunk-major too:
// their workgroups all load the same chunk's 128 rows at about the same time,
// and row-major those rows lie 2K bytes apart, on few memory channels (-18 %
// on the 3-bit {gate, up} pair at 128 rows). The other 16- to 64-row launches
// (4 or 8 waves per CU, whose L1 keeps the row-major lines for the next
// chunk) measured as fast or faster row-major.

// 8 consecutive 16-bit values from p (any 2-byte alignment).
__device__ __forceinline__ u32x4 load8_u16(const uint16_t *p) {
  if (((uintptr_t)p & 15) == 0) return *(const u32x4 *)p;
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (uint32_t)p[2 * e] | ((uint32_t)p[2 * e + 1] << 16);
  return r;
}

// Lane (c, g)'s 8 outputs of one row from its 8 inputs xw (bf16, columns
// 128 k + 8c .. +7) and their signs sw, packed for one 16-byte store at
// xr + row * K + 128 k + 8c.
__device__ __forceinline__ u32x4 rot_lane(const u32x4 xw, const u32x4 sw, int c, bool natural) {
  float v[8][1];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e][0] = bf16_to_f32((uint16_t)(xw[e] & 0xFFFFu)) * fp16_to_f32((uint16_t)(sw[e] & 0xFFFFu));
    v[2 * e + 1][0] = bf16_to_f32((uint16_t)(xw[e] >> 16)) * fp16_to_f32((uint16_t)(sw[e] >> 16));
  }
  register_level<1>(v);
  register_level<2>(v);
  register_level<4>(v);
  lane_level<1>(v, c);
  lane_level<2>(v, c);
  lane_level<4>(v, c);
  lane_level<8>(v, c);
  uint16_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = f32_to_fp16(v[e][0] * 0.0625f);
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    out[e] = natural ? ((uint32_t)h[2 * e] | ((uint32_t)h[2 * e + 1] << 16))
                     : ((uint32_t)h[e] | ((uint32_t)h[e + 4] << 16));
  return out;
}


// ------------------------------------------------------------ rot_in inside a decode-row linear launch
//
// At up to 32 rows the rotation is a few microseconds of latency and almost
// no work, so the linear launch does it itself instead of a launch of its
// own. Member j's chunk k (128 columns of Xr, all M rows) is one item;
// item i = j * K/128 + k belongs to the wave with global index
// wave * gridDim.x + blockIdx.x == i (mod all waves), i.e. to the first
// dispatched workgroups. The owner writes the item with stores that reach
// the agent's coherence point, waits for them, and then sets the item's flag.
// A wave about to read Xr for chunks [c0, c1) first issues its weight loads,
// then polls the flags of the items they span (one flag per lane); no wave
// reads an item's lines before its flag is set or it wrote them itself, so no
// cache holds them stale. After spin_limit polls a wave rotates the items
// still unflagged itself (the same bits as their owner), so a launch whose
// workgroups are not all resident still ends. Each workgroup counts itself
// done once all its waves are past their last poll; the last one clears the
// flags and the count, which are thus zero at rest, as the split counters.

// Member j's chunk k of Xr (chunk-major for the spread launch, else
// row-major) for rows 0 .. M-1 (at most 4 Q rows): one wave,
// all of the lane's loads before any arithmetic; rows past M reread row
// M - 1 and are not stored (out-of-range buffer stores are dropped).
template <int Q>
__device__ __forceinline__ void rot_item(const LinearArgs &a, int j, int k, int lane, bool chunk_major) {
  const MemberArgs &m = a.m[j];
  const int c = lane & 15, g = lane >> 4;
  const int M = a.M;
  const int k0 = k * 128 + 8 * c;
  u32x4 xw[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) xw[q] = load8_u16(a.x + (int64_t)min(4 * q + g, M - 1) * a.ldx + k0);
  const u32x4 sw = load8_u16(m.suh + k0);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(m.xr, (uint32_t)((uint64_t)M * a.K * 2));
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int row = 4 * q + g;
    const int64_t at = chunk_major ? ((int64_t)(k0 >> 5) * M + row) * 32 + (k0 & 31) : (int64_t)row * a.K + k0;
    const uint32_t off = row < M ? (uint32_t)(at * 2) : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b128(rot_lane(xw[q], sw, c, false), rx, (int)off, 0, kAgentScope);
  }
}

// The items this wave owns, then their flags.
template <int Q>
__device__ __forceinline__ void rot_produce(const LinearArgs &a, int wave, int lane, bool chunk_major) {
  const int kc = a.K >> 7;
  const int items = a.n_members * kc;
  const int all = (int)(gridDim.x * (blockDim.x >> 6));
  for (int i = wave * (int)gridDim.x + (int)blockIdx.x; i < items; i += all) {
    const int j = i / kc;
    rot_item<Q>(a, j, i - j * kc, lane, chunk_major);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);             // the item's stores are complete
    if (lane == 0) __hip_atomic_store(a.sync + 1 + i, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Member j's items k0 .. k1 are in Xr when this returns.
template <int Q>
__device__ __forceinline__ void rot_wait(const LinearArgs &a, int j, int k0, int k1, int lane, bool chunk_major) {
  const uint32_t *flags = a.sync + 1 + j * (a.K >> 7);
  for (int kb = k0; kb <= k1; kb += 64) {
    const int k = kb + lane;
    for (int polls = 0;; ++polls) {
      const uint32_t v = k <= k1 ? __hip_atomic_load(flags + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1u;
      uint64_t missing = __builtin_amdgcn_ballot_w64(v == 0u);
      if (missing == 0) break;
      if (polls >= a.spin_limit) {
        while (missing) {
          rot_item<Q>(a, j, kb + __builtin_ctzll(missing), lane, chunk_major);
          missing &= missing - 1;
        }
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  asm volatile("" ::: "memory");
}

// One thread per workgroup, once every wave of it is past its last poll and
// its own items are flagged: true for the launch's last workgroup.
__device__ __forceinline__ bool rot_count_done(const LinearArgs &a) {
  return __hip_atomic_fetch_add(a.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
         (uint32_t)(gridDim.x - 1);
}

// Every thread of the last workgroup: flags and count back to zero.
__device__ __forceinline__ void rot_clear(const LinearArgs &a) {
  const int n = a.n_members * (a.K >> 7);
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    __hip_atomic_store(a.sync + 1 + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0) __hip_atomic_store(a.sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ linear

// Chunks in flight per wave: deeper where a stage is small.
template <int MT>
struct Depth { static constexpr int P = MT == 1 ? 8 : (MT == 2 ? 4 : 2); };

template <int BITS, int MT>
struct Stage {
  u32x4 a[MT];
  uint32_t b[2][BitsTraits<BITS>::kDwords];
};

template <int BITS, int MT>
__device__ __forceinline__ void load_stage(Stage<BITS, MT> &st, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, const uint32_t (&voff_a)[MT],
                                           const uint32_t (&voff_b)[2][BitsTraits<BITS>::kDwords],
                                           int chunk) {
  const int soff_a = chunk * 64;                 // 32 fp16 per row per chunk
  const int soff_b = chunk * 512 * BITS;         // two tile rows of 8 tiles
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    st.a[mt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)voff_a[mt], soff_a, 0));
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int d = 0; d < BitsTraits<BITS>::kDwords; ++d)
      st.b[i][d] = __builtin_amdgcn_raw_buffer_load_b32(rb, (int)voff_b[i][d], soff_b, 0);
}

template <int BITS, int MT>
__device__ __forceinline__ void compute_stage(const Stage<BITS, MT> &st, uint32_t shift, const CbConst &cb,
                                              f32x4 (&acc)[MT][2]) {
  half8 bf[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) bf[i] = decode8<BITS>(st.b[i], shift, cb);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const half8 af = __builtin_bit_cast(half8, st.a[mt]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      acc[mt][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[i], acc[mt][i], 0, 0, 0);
  }
}

template <int BITS, int MT, bool CHAINED>
__global__ __launch_bounds__(kThreads) void linear_ntile_kernel(const LinearArgs a) {
  using T = BitsTraits<BITS>;
  constexpr int R = 16 * MT;                      // rows per workgroup
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: everything derived from it (split, chunk,
  // buffer offsets) stays in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bid = blockIdx.x;

  // member of this workgroup (uniform)
  int j = 0;
  if (a.n_members > 1 && bid >= a.m[1].wg_begin) j = 1;
  if (a.n_members > 2 && bid >= a.m[2].wg_begin) j = 2;
  const MemberArgs &m = a.m[j];
  const int S = m.splits;
  const int groups = m.groups;                    // workgroups per (row block, column block): 1 or S
  const int local = bid - m.wg_begin;
  const int per_rb = m.n_blocks * groups;
  const int rb = local / per_rb;
  const int rem = local - rb * per_rb;
  const int nb = rem / groups;
  const int sg = rem - nb * groups;
  const int s_begin = CHAINED ? 0 : sg;
  const int s_end = CHAINED ? S : sg + 1;
  const int M = a.M, K = a.K, C = a.chunks;
  const int row_base = rb * R;
  const int col0 = nb * kBlockCols;

  // buffer resources: this member's rotated input, this block's words
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(m.xr, (uint32_t)((uint64_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t rbuf = make_rsrc(m.words + (int64_t)nb * m.block_stride, (uint32_t)(16u * K * BITS));

  const int c = lane & 15, g = lane >> 4;
  uint32_t voff_a[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = row_base + 16 * mt + c;
    voff_a[mt] = row < M ? (uint32_t)(row * 2 * K + 16 * g) : kOutOfRange;
  }
  const BLane<BITS> bl = b_lane<BITS>(lane);
  uint32_t voff_b[2][T::kDwords];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int d = 0; d < T::kDwords; ++d) voff_b[i][d] = bl.voff[d] + (uint32_t)((2 * wave + i) * T::kTileBytes);

  // Chains s_begin .. s_end-1, one after another; split s covers chunks
  // [floor(s*C/S), floor((s+1)*C/S)). Each chain starts from zero and is
  // folded into z in split order (z = P0, then z + P1, ...), exactly as if
  // every chain ran in its own workgroup.
  constexpr int P = Depth<MT>::P;
  const CbConst cbc = cb_const();
  f32x4 acc[MT][2];
  f32x4 z[CHAINED ? MT : 1][2];
  for (int s = s_begin; s < s_end; ++s) {
    const int c0 = (int)(((int64_t)s * C) / S);
    const int c1 = (int)(((int64_t)(s + 1) * C) / S);
    const int last = c1 - 1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // stage loads are issued strictly in stage order (the scheduling
    // barriers keep them from being regrouped), so the outstanding-load count
    // when a stage is consumed is the same on entry and on the back edge
    Stage<BITS, MT> st[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      load_stage<BITS, MT>(st[p], ra, rbuf, voff_a, voff_b, min(c0 + p, last));
      __builtin_amdgcn_sched_barrier(0);
    }
    const int n = c1 - c0;
    const int full_end = c0 + (n - n % P);
    for (int cc0 = c0; cc0 < full_end; cc0 += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        compute_stage<BITS, MT>(st[p], bl.shift, cbc, acc);
        load_stage<BITS, MT>(st[p], ra, rbuf, voff_a, voff_b, min(cc0 + p + P, last));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int p = 0; p < P - 1; ++p)
      if (p < n % P) compute_stage<BITS, MT>(st[p], bl.shift, cbc, acc);
    if constexpr (CHAINED) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 2; ++i) z[mt][i] = (s == 0) ? acc[mt][i] : z[mt][i] + acc[mt][i];
    }
  }

  __shared__ float zbuf[R][132];
  const EpiCols ec = epi_cols(m, col0, lane);
  if constexpr (CHAINED) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) zbuf[16 * mt + 4 * g + r][16 * (2 * wave + i) + c] = z[mt][i][r];
  } else {
    // Write this split's fp32 partial P_s[row][col] with agent-scope stores
    // (written through the XCD's non-coherent L2), wait until every wave's
    // stores have completed, then count the arrival. The last arriver reads
    // all partials with agent-scope loads (fetched past stale cache lines),
    // adds them in split order and resets the counter: no L2 write-back or
    // invalidation is needed on either side.
    const int N = m.N;
    float *P = m.partials + (int64_t)s_begin * M * N + col0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = row_base + 16 * mt + 4 * g + r;
          if (row < M)
            __hip_atomic_store(P + (int64_t)row * N + 16 * (2 * wave + i) + c, acc[mt][i][r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);        // this wave's stores are complete
    __syncthreads();
    __shared__ int s_last;
    uint32_t *counter = m.counters + (int64_t)rb * m.n_blocks + nb;
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (uint32_t)(groups - 1);
    }
    __syncthreads();
    if (!s_last) return;
    // the last arriver resets the counter it consumed: zero at rest
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float *P0 = m.partials + col0;
    const int64_t split_stride = (int64_t)M * N;
    for (int rr = wave; rr < R; rr += kWaves) {
      const int row = row_base + rr;
      if (row >= M) break;
      const float *p = P0 + (int64_t)row * N;
      float z0 = __hip_atomic_load(p + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      float z1 = __hip_atomic_load(p + lane + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int sp = 1; sp < S; ++sp) {
        p += split_stride;
        z0 = z0 + __hip_atomic_load(p + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        z1 = z1 + __hip_atomic_load(p + lane + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      zbuf[rr][lane] = z0;
      zbuf[rr][lane + 64] = z1;
    }
  }
  __syncthreads();
  if (wave < MT && row_base + 16 * wave < M)
    epilogue_rows_lds<4>(&zbuf[16 * wave][0], 132, ec, lane, m, col0, row_base + 16 * wave, M);
}


// ------------------------------------------------------------ linear, one split per wave
//
// Row tilings of 16 and 32 rows, W waves per workgroup. Wave w runs whole
// K-split chains over all 8 column tiles of the block, so one A fragment (the
// rotated input, 16 rows x 32 K) feeds 8 MFMAs. Chains are assigned
// round-robin: when the workgroup owns every split of its block (chained),
// wave w runs splits w, w+W, ... and the workgroup folds them in split order
// in LDS; otherwise workgroup g owns splits Wg .. Wg+W-1, one per wave, and
// the split partials meet through the workspace.
//
// Weight stream. A chunk of a block is two tile rows of 8 tiles, 512*b
// contiguous bytes. Each wave fetches its chunks with 128-bit loads (b/2
// instructions per chunk instead of one or two per tile and lane: the address
// unit spends about the same time on a 64-lane load whatever its width), and
// stages them in its own LDS region: tile tau at tau * (32b + 16), followed by
// a copy of the tile's first dword, so the windows that wrap past the tile's
// end (tail-biting) read on contiguously. Each lane then reads its 2 or 3
// dwords per tile with ds_read2_b32 (+ ds_read_b32). LDS is double-buffered
// one chunk ahead of the decode; a wave's region is its own, so no barrier is
// needed.

// A wave streams CT column tiles of each chunk's two tile rows: all 8 (one
// wave per split), or 4 (two waves per split, each with half the columns).
template <int BITS, int CT = 8>
struct Stream {
  static constexpr int kFullChunkBytes = 512 * BITS;             // 16 tiles: the chunk's bytes in memory
  static constexpr int kChunkBytes = 64 * CT * BITS;             // the wave's 2 CT tiles
  static constexpr int kLoads = (kChunkBytes + 1023) / 1024;     // 128-bit loads per chunk
  static constexpr int kStride = 32 * BITS + 16;                 // padded tile in LDS
  static constexpr int kSlot = 2 * CT * kStride + 16;            // the tiles + a dump for idle lanes
  static constexpr int kWave = 2 * kSlot;                        // double buffer
};

template <int MT>
struct ChainDepth { static constexpr int P = 4; };   // chunks in flight per wave

template <int BITS, int MT, int CT = 8>
struct ChainStage {
  u32x4 a[MT];
  u32x4 b[Stream<BITS, CT>::kLoads];
};

template <int BITS, int MT, int CT = 8, int POL = kStreamOnce>
__device__ __forceinline__ void load_chain_stage(ChainStage<BITS, MT, CT> &st, __amdgpu_buffer_rsrc_t ra,
                                                 __amdgpu_buffer_rsrc_t rb, const uint32_t (&voff_a)[MT],
                                                 const uint32_t (&voff_b)[Stream<BITS, CT>::kLoads], int chunk,
                                                 int a_stride) {
  const int soff_a = chunk * a_stride;
  const int soff_b = chunk * Stream<BITS, CT>::kFullChunkBytes;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    st.a[mt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)voff_a[mt], soff_a, 0));
#pragma unroll
  for (int l = 0; l < Stream<BITS, CT>::kLoads; ++l)
    st.b[l] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)voff_b[l], soff_b, POL));
}

// Copy a stage's weight bytes into LDS slot `slot` (byte address).
template <int BITS, int MT, int CT = 8>
__device__ __forceinline__ void stage_to_lds(const ChainStage<BITS, MT, CT> &st, char *slot,
                                             const uint32_t (&wr_off)[Stream<BITS, CT>::kLoads],
                                             const uint32_t (&wrap_off)[Stream<BITS, CT>::kLoads]) {
#pragma unroll
  for (int l = 0; l < Stream<BITS, CT>::kLoads; ++l) {
    *(u32x4 *)(slot + wr_off[l]) = st.b[l];
    *(uint32_t *)(slot + wrap_off[l]) = st.b[l][0];
  }
}

// The lane's words of a staged chunk: 2 or 3 dwords of each of the CT tiles.
// All CT reads are issued together so that their LDS latencies overlap.
template <int BITS, int CT = 8>
__device__ __forceinline__ void read_chain_chunk(const char *slot, uint32_t rd_off,
                                                 uint32_t (&w)[CT][BitsTraits<BITS>::kDwords]) {
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const uint32_t *q = (const uint32_t *)(slot + rd_off + t * Stream<BITS, CT>::kStride);
#pragma unroll
    for (int d = 0; d < BitsTraits<BITS>::kDwords; ++d) w[t][d] = q[d];
  }
}

template <int BITS, int MT, int CT = 8>
__device__ __forceinline__ void decode_chain_chunk(const uint32_t (&w)[CT][BitsTraits<BITS>::kDwords],
                                                   const ChainStage<BITS, MT, CT> &st, uint32_t shift,
                                                   const CbConst &cb, f32x4 (&acc)[MT][CT]) {
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const half8 bf = decode8<BITS>(w[t], shift, cb);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, st.a[mt]), bf, acc[mt][t], 0, 0, 0);
  }
}

// First float of split s's partial for (row block rb, column block nb) in the
// fragment layout [s][row block][block][MT * 8 * 256 floats].
__device__ __forceinline__ float *partial_frag(const MemberArgs &m, int s, int rb, int nb, int row_blocks, int mt) {
  return m.partials + (((int64_t)s * row_blocks + rb) * m.n_blocks + nb) * (int64_t)(mt * 8 * 256);
}

// The spread launch keeps partials for its left blocks only, in one buffer
// (member 0's partials): split s of left block lb (launch block own_blocks +
// lb) in row block rb at [s][row block][left block][8 * 256 floats].
__device__ __forceinline__ float *spread_partial(const LinearArgs &a, int s, int rb, int lb, int row_blocks) {
  return a.m[0].partials + (((int64_t)s * row_blocks + rb) * a.left_blocks + lb) * (int64_t)(8 * 256);
}

// Per-wave constants of the chain loop: buffer resources, lane offsets of
// the A loads, the 128-bit B loads and their LDS slots, and the lane's read
// offset and bit shift in a staged chunk.
template <int BITS, int MT, int CT = 8>
struct ChainCtx {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t voff_a[MT];
  int a_stride;                     // bytes from one chunk of Xr to the next (chunk-major: 64 M)
  uint32_t voff_b[Stream<BITS, CT>::kLoads], wr_off[Stream<BITS, CT>::kLoads], wrap_off[Stream<BITS, CT>::kLoads];
  uint32_t rd_off, shift;
  CbConst cb;
};

// `half`: which CT column tiles of the block's 8 the wave streams (CT = 4).
template <int BITS, int MT, int CT = 8>
__device__ __forceinline__ ChainCtx<BITS, MT, CT> chain_ctx(const MemberArgs &m, int M, int K, int nb, int row_base,
                                                           int lane, bool chunk_major, int half = 0) {
  using SB = Stream<BITS, CT>;
  ChainCtx<BITS, MT, CT> x;
  x.ra = make_rsrc(m.xr, (uint32_t)((uint64_t)M * K * 2));
  x.rb = make_rsrc(m.words + (int64_t)nb * m.block_stride, (uint32_t)(16u * K * BITS));
  const int c = lane & 15, g = lane >> 4;
  // chunk cc, row r of Xr at (cc * M + r) * 64 bytes (chunk-major) or at
  // r * 2K + 64 cc (row-major)
  x.a_stride = chunk_major ? 64 * M : 64;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = row_base + 16 * mt + c;
    x.voff_a[mt] = row < M ? (uint32_t)(row * (chunk_major ? 64 : 2 * K) + 16 * g) : kOutOfRange;
  }
  // 128-bit load l covers bytes [1024 l, 1024 l + 1024) of the wave's part
  // of a chunk: CT tiles of tile row 0, then CT of tile row 1 (in memory the
  // chunk is tile row 0's 8 tiles, then tile row 1's; the wave's tiles start
  // at tile CT * half of each). Lane bytes 16 lane .. +15 of a load belong to
  // one tile (tiles are 32b bytes, a multiple of 16), staged as tile tau of
  // the wave's 2 CT. Lanes past the end load the chunk's first bytes and dump
  // them.
#pragma unroll
  for (int l = 0; l < SB::kLoads; ++l) {
    const int off = 1024 * l + 16 * lane;
    const bool valid = off < SB::kChunkBytes;
    const int row = off / (CT * 32 * BITS), within = off % (CT * 32 * BITS);
    const int tau = row * CT + within / (32 * BITS), w = within % (32 * BITS);
    x.voff_b[l] = valid ? (uint32_t)(row * 256 * BITS + half * CT * 32 * BITS + within) : 0u;
    x.wr_off[l] = valid ? (uint32_t)(tau * SB::kStride + w) : (uint32_t)(2 * CT * SB::kStride);
    x.wrap_off[l] = valid ? (uint32_t)(tau * SB::kStride + 32 * BITS + (w == 0 ? 0 : 4)) : (uint32_t)(2 * CT * SB::kStride);
  }
  const int jseg = 2 * c + (g & 1);
  x.shift = 8u * (uint32_t)((BITS * jseg) & 3);
  x.rd_off = (uint32_t)((g >> 1) * CT * SB::kStride + 4 * ((BITS * jseg) >> 2));
  x.cb = cb_const();
  return x;
}

// No wait before the chain's first rotated-input loads.
struct NoWait {
  __device__ void operator()() const {}
};

// One K-split chain: chunks [c0, c1) of the block over all 8 column tiles and
// MT 16-row tiles, accumulated from zero in ascending chunk order. Chunk i of
// the chain uses register stage i % P and LDS slot i % 2 of the wave's
// region `wlds`; the next chunk is copied to LDS before chunk i is decoded.
// With `fused` the first P chunks' weight loads go out before ready(), which
// returns once the chain's part of Xr is written, and their Xr loads after.
template <int BITS, int MT, int P, int CT = 8, int POL = kStreamOnce, typename Ready = NoWait>
__device__ __forceinline__ void run_chain(f32x4 (&acc)[MT][CT], int c0, int c1, char *wlds,
                                          const ChainCtx<BITS, MT, CT> &x, bool fused = false, Ready ready = Ready{}) {
  using SB = Stream<BITS, CT>;
  static_assert(P % 2 == 0, "the chunk loop unrolls by P, a multiple of the 2 LDS slots");
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < CT; ++t) acc[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n = c1 - c0;
  const int last = c1 - 1;
  ChainStage<BITS, MT, CT> st[P];
  if (fused) {
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int l = 0; l < SB::kLoads; ++l)
        st[p].b[l] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   x.rb, (int)x.voff_b[l], min(c0 + p, last) * SB::kFullChunkBytes,
                                                   POL));
    __builtin_amdgcn_sched_barrier(0);
    ready();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        st[p].a[mt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    x.ra, (int)x.voff_a[mt], min(c0 + p, last) * x.a_stride, 0));
    __builtin_amdgcn_sched_barrier(0);
  } else {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      load_chain_stage<BITS, MT, CT, POL>(st[p], x.ra, x.rb, x.voff_a, x.voff_b, min(c0 + p, last), x.a_stride);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  stage_to_lds<BITS, MT, CT>(st[0], wlds, x.wr_off, x.wrap_off);
  // per chunk: read the staged chunk's words, stage the next chunk into the
  // other slot, decode and multiply, refill the register stage
  uint32_t w[CT][BitsTraits<BITS>::kDwords];
  int i = 0;
  for (; i + P < n; i += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      read_chain_chunk<BITS, CT>(wlds + (p % 2) * SB::kSlot, x.rd_off, w);
      __builtin_amdgcn_sched_barrier(0);
      stage_to_lds<BITS, MT, CT>(st[(p + 1) % P], wlds + ((p + 1) % 2) * SB::kSlot, x.wr_off, x.wrap_off);
      decode_chain_chunk<BITS, MT, CT>(w, st[p], x.shift, x.cb, acc);
      load_chain_stage<BITS, MT, CT, POL>(st[p], x.ra, x.rb, x.voff_a, x.voff_b, min(c0 + i + p + P, last), x.a_stride);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the last 1..P chunks, already loaded
  const int r = n - i;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (p < r) {
      read_chain_chunk<BITS, CT>(wlds + (p % 2) * SB::kSlot, x.rd_off, w);
      if (p + 1 < r) stage_to_lds<BITS, MT, CT>(st[(p + 1) % P], wlds + ((p + 1) % 2) * SB::kSlot, x.wr_off, x.wrap_off);
      decode_chain_chunk<BITS, MT, CT>(w, st[p], x.shift, x.cb, acc);
    }
  }
}

// ------------------------------------------------------------ linear, decode rows: spread launch
//
// Up to 16 rows, every member planned with the same S <= 15, one 16-wave
// workgroup per CU. Workgroup u owns launch block u (u < own_blocks): its
// waves 16-S .. 15 run the block's S chains and the workgroup folds them in
// split order in LDS, as a chained launch does. Its first 16 - S waves (the
// oldest, so the first to issue) are spare waves that share the splits of
// the launch blocks past own_blocks (the "left" blocks): spare wave k of
// workgroup u takes unit u*(16-S) + k, that is split unit % S of left block
// unit / S. Those splits meet through the workspace (partials and a counter,
// as in the exchanged launch); the workgroup whose spare wave arrives last
// adds them in split order while it folds its own block, and runs that
// block's epilogue as well. A launch of 272 blocks at S = 15 on 256 CUs thus
// gives every CU one block plus one split of the 16 left blocks: 16 busy
// waves, 4 per SIMD, the same work everywhere.

// ROWS: several 16-row blocks (row block and its bounds at run time; one
// row block keeps them compile-time constants, which the left blocks'
// partial addressing folds away)
template <int BITS, int POL, bool ROWS>
__device__ __forceinline__ void spread_body(const LinearArgs &a) {
  using SB = Stream<BITS>;
  constexpr int W = 16, NT = 64 * W;
  // 4 chunks in flight where a chunk is at most two 128-bit loads per lane,
  // 2 above that: 128 VGPRs per wave
  constexpr int P = SB::kLoads <= 2 ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // workgroup (row block rb, own block u): rows 16 rb .. 16 rb + Mr - 1
  const int rb = ROWS ? (int)blockIdx.x / a.own_blocks : 0;
  const int u = (int)blockIdx.x - rb * a.own_blocks;
  const int RB = ROWS ? a.row_blocks : 1;
  const int S = a.m[0].splits;                           // the same for every member
  const int spare = W - S;                               // waves 0 .. spare-1
  const int M = a.M, K = a.K, C = a.chunks;
  const int row_base = 16 * rb;
  const int Mr = ROWS ? min(16, M - row_base) : M;
  const int c = lane & 15, g = lane >> 4;

  // LDS: per-wave staging during the chains; afterwards the fold buffers
  // [S][16][128] and the two 16-row results (own block, left block)
  constexpr int kTile = 16 * kBlockCols * 4;
  constexpr int kFold = (W - 1) * kTile;
  constexpr int kStage = W * SB::kWave;
  constexpr int kLds = kStage > kFold + 2 * kTile ? kStage : kFold + 2 * kTile;
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  __shared__ int s_left[W];                              // left blocks this workgroup finishes
  __shared__ int s_nleft;
  __shared__ int s_clear;
  char *wlds = lds + wave * SB::kWave;
  if (threadIdx.x == 0) s_nleft = 0;
  const bool fused = a.x != nullptr;
  __syncthreads();
  if (fused) rot_produce<4>(a, wave, lane, true);

  // member j and block nb of launch block gb (members' blocks are consecutive)
  auto locate = [&](int gb, int &jj, int &nb) {
    jj = 0;
    if (a.n_members > 1 && gb >= a.m[1].wg_begin) jj = 1;
    if (a.n_members > 2 && gb >= a.m[2].wg_begin) jj = 2;
    nb = gb - a.m[jj].wg_begin;
  };

  int jo, nbo;
  locate(u, jo, nbo);
  const MemberArgs &mo = a.m[jo];
  f32x4 acc[1][8];
  if (wave >= spare) {
    const int sp = wave - spare;
    const ChainCtx<BITS, 1> x = chain_ctx<BITS, 1>(mo, M, K, nbo, row_base, lane, true);
    const int c0 = (int)(((int64_t)sp * C) / S), c1 = (int)(((int64_t)(sp + 1) * C) / S);
    run_chain<BITS, 1, P, 8, POL>(acc, c0, c1, wlds, x, fused,
                                  [&] { rot_wait<4>(a, jo, c0 >> 2, (c1 - 1) >> 2, lane, true); });
  } else {
    const int unit = u * spare + wave;
    if (unit < a.left_blocks * S) {
      const int gb = a.own_blocks + unit / S;
      const int sp = unit - (unit / S) * S;
      int jl, nbl;
      locate(gb, jl, nbl);
      const MemberArgs &ml = a.m[jl];
      const ChainCtx<BITS, 1> x = chain_ctx<BITS, 1>(ml, M, K, nbl, row_base, lane, true);
      const int c0 = (int)(((int64_t)sp * C) / S), c1 = (int)(((int64_t)(sp + 1) * C) / S);
      run_chain<BITS, 1, P, 8, POL>(acc, c0, c1, wlds, x, fused,
                                    [&] { rot_wait<4>(a, jl, c0 >> 2, (c1 - 1) >> 2, lane, true); });
      // the split's partial, agent scope, then the arrival (see the exchanged launch)
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(spread_partial(a, sp, rb, gb - a.own_blocks, RB), 8 * 1024);
      if (4 * g < Mr) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[0][t]), rp, t * 1024 + 16 * lane, 0,
                                                 kAgentScope);
      }
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      uint32_t *counter = ml.counters + (int64_t)rb * ml.n_blocks + nbl;
      uint32_t prev = 0;
      if (lane == 0) prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev == (uint32_t)(S - 1) && lane == 0) {
        __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_left[atomicAdd(&s_nleft, 1)] = gb;             // at most one per spare wave
      }
    }
  }
  const EpiCols eco = epi_cols(mo, nbo * kBlockCols, lane);
  __syncthreads();                                       // staging is free; the left list is final
  if (fused && threadIdx.x == 0) s_clear = rot_count_done(a);

  float *pbuf = (float *)lds;                            // [S][16][128]
  float *zown = (float *)(lds + kFold);                  // [16][128]
  float *zleft = (float *)(lds + kFold + kTile);         // [16][128]
  if (wave >= spare) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        pbuf[((wave - spare) * 16 + 4 * g + rr) * kBlockCols + 16 * t + c] = acc[0][t][rr];
  }
  const int nleft = s_nleft;
  __syncthreads();
  if (fused && s_clear) rot_clear(a);
  // Waves 0..7 fold the own block (P_0 + P_1 + ... in split order, 4 of its
  // 2048 values per thread); waves 8..15 meanwhile add up the first left
  // block's S partials in split order (fragment f = thread - 512: column
  // tile f / 64, lane f % 64), all S loads in flight. Later left blocks (only
  // when S is small) follow one at a time.
  auto left_sum = [&](int i, int f) {
    const int fl = f & 63, ft = f >> 6;
    const int fr0 = 4 * (fl >> 4);
    if (fr0 < Mr) {
      u32x4 v[15];
#pragma unroll
      for (int q = 0; q < 15; ++q) {
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(spread_partial(a, min(q, S - 1), rb, s_left[i] - a.own_blocks, RB), 8 * 1024);
        v[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, 16 * f, 0, kAgentScope));
      }
      f32x4 zv = __builtin_bit_cast(f32x4, v[0]);
#pragma unroll
      for (int q = 1; q < 15; ++q)
        if (q < S) zv = zv + __builtin_bit_cast(f32x4, v[q]);
#pragma unroll
      for (int q = 0; q < 4; ++q) zleft[(fr0 + q) * kBlockCols + 16 * ft + (fl & 15)] = zv[q];
    }
  };
  if (wave < 8) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = threadIdx.x + e * 512;
      float v = pbuf[idx];
      for (int sp = 1; sp < S; ++sp) v = v + pbuf[sp * 2048 + idx];
      zown[idx] = v;
    }
  } else if (nleft > 0) {
    left_sum(0, threadIdx.x - 512);
  }
  __syncthreads();
  // epilogues, 4 rows per wave: waves 0..3 the own block, 4..7 the left block
  if (wave < 4) {
    if (4 * wave < Mr)
      epilogue_rows_lds<1>(zown + 4 * wave * kBlockCols, kBlockCols, eco, lane, mo, nbo * kBlockCols,
                           row_base + 4 * wave, M);
  }
  for (int i = 0; i < nleft; ++i) {
    if (i > 0) {
      __syncthreads();                                   // zleft of the previous block is read
      if (wave >= 8) left_sum(i, threadIdx.x - 512);
      __syncthreads();
    }
    int jl, nbl;
    locate(s_left[i], jl, nbl);
    const MemberArgs &ml = a.m[jl];
    if (wave >= 4 && wave < 8 && 4 * (wave - 4) < Mr) {
      const int r4 = 4 * (wave - 4);
      const EpiCols ecl = epi_cols(ml, nbl * kBlockCols, lane);
      epilogue_rows_lds<1>(zleft + r4 * kBlockCols, kBlockCols, ecl, lane, ml, nbl * kBlockCols, row_base + r4, M);
    }
  }
}

// One 16-row block (streaming word loads), or several (normal policy: the
// grid reads each block's words once per row block).
template <int BITS>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
void linear_spread_kernel(const LinearArgs a) {
  spread_body<BITS, kStreamOnce, false>(a);
}

template <int BITS>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
void linear_spread_rows_kernel(const LinearArgs a) {
  spread_body<BITS, kStreamAgain, true>(a);
}

// ------------------------------------------------------------ linear, 16 and 32 rows per workgroup

// W = 8 (chained, 16 rows) keeps to 128 VGPRs so that two workgroups fit a CU.
// CT = 4 (exchanged, 16 rows, W = 8): the two waves 2i, 2i+1 share split i of
// the workgroup, each with 4 of the block's 8 column tiles: the same MFMA
// chains, two waves per SIMD where one wave per split would leave one.
template <int BITS, int MT, bool CHAINED, int W, int CT = 8, int POL = kStreamOnce>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(W == 8 ? 4 : 1)))
void linear_chain_kernel(const LinearArgs a) {
  static_assert(CT == 8 || (CT == 4 && !CHAINED && MT == 1), "column halves: exchanged 16-row tiles only");
  using SB = Stream<BITS, CT>;
  constexpr int SPW = W * CT / 8;                        // splits per workgroup and round
  constexpr int R = 16 * MT;
  constexpr int NT = W * 64;                             // threads
  const int lane = threadIdx.x & 63;
  // wave index as a scalar: everything derived from it (split, chunk,
  // buffer offsets) stays in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Exchanged: workgroups are dealt to the 8 XCDs in turn, each XCD taking a
  // contiguous range of (row block, block, split group), so a block's split
  // groups share an XCD and its L2 (the decode step at 16 / 1 rows 44.0-44.3
  // -> 43.3-43.6 / 39.8-40.1 -> 38.5-38.7 us, view B 18.2-18.3 -> 17.5-17.6
  // us; the same bytes, the exchange stays agent-scope)
  const int T = a.total_wgs, xcd = blockIdx.x & 7;
  const int bid = CHAINED ? (int)blockIdx.x : xcd * (T >> 3) + min(xcd, T & 7) + (int)(blockIdx.x >> 3);
  int j = 0;
  if (a.n_members > 1 && bid >= a.m[1].wg_begin) j = 1;
  if (a.n_members > 2 && bid >= a.m[2].wg_begin) j = 2;
  const MemberArgs &m = a.m[j];
  const int S = m.splits;
  const int groups = m.groups;
  const int local = bid - m.wg_begin;
  const int per_rb = m.n_blocks * groups;
  const int rb = local / per_rb;
  const int rem = local - rb * per_rb;
  const int nb = rem / groups;
  const int sg = rem - nb * groups;
  const int M = a.M, K = a.K, C = a.chunks;
  const int row_base = rb * R;
  const int col0 = nb * kBlockCols;

  // LDS: per-wave weight staging during the chunk loops; afterwards the
  // same bytes hold the chain fold buffers and the epilogue rows.
  constexpr int kStageBytes = W * SB::kWave;
  constexpr int kFoldBytes = (CHAINED ? W : 0) * R * kBlockCols * 4;
  constexpr int kRowBytes = R * kBlockCols * 4;
  constexpr int kLds = kStageBytes > kFoldBytes + kRowBytes ? kStageBytes : kFoldBytes + kRowBytes;
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  char *wlds = lds + wave * SB::kWave;

  const int sw = wave / (8 / CT), half = wave % (8 / CT);   // the wave's split in the workgroup, its columns
  // Xr chunk-major (the column-halves form, one row block) or row-major
  const bool cm = CT == 4 && a.xr_chunk_major != 0;
  const ChainCtx<BITS, MT, CT> x = chain_ctx<BITS, MT, CT>(m, M, K, nb, row_base, lane, cm, half);
  const int c = lane & 15, g = lane >> 4;
  // one row block (row_base == 0); the 8-wave chained form (weights of many
  // blocks, where a rotation launch costs little) would spill with the fused
  // prologue
  const bool fused = (W != 8 || CT == 4) && a.x != nullptr;
  __shared__ int s_clear;
  if (fused) rot_produce<4 * MT>(a, wave, lane, cm);

  const int s_first = CHAINED ? sw : SPW * sg + sw;
  const int rounds = CHAINED ? (S + SPW - 1) / SPW : 1;
  float zsum[CHAINED ? R * kBlockCols / NT : 1];

  for (int round = 0; round < rounds; ++round) {
    const int s = s_first + round * (CHAINED ? SPW : 0);
    const bool active = s < S;                           // uniform per wave
    f32x4 acc[MT][CT];
    if (CHAINED && round > 0) __syncthreads();           // fold buffers of the last round are read
    if (active) {
      // in 128 VGPRs (W = 8) only 2 chunks of more than two 128-bit loads fit
      constexpr int P = (W == 8 && SB::kLoads > 2) ? 2 : ChainDepth<MT>::P;
      const int c0 = (int)(((int64_t)s * C) / S), c1 = (int)(((int64_t)(s + 1) * C) / S);
      run_chain<BITS, MT, P, CT, POL>(acc, c0, c1, wlds, x, fused,
                             [&] { rot_wait<4 * MT>(a, j, c0 >> 2, (c1 - 1) >> 2, lane, cm); });
    }
    if constexpr (CHAINED) {
      // fold this round's chains into the running sum in split order
      float *pbuf = (float *)lds;                        // [W][R][128]
      __syncthreads();                                   // every wave is done with its staging
      if (active) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
              pbuf[(wave * R + 16 * mt + 4 * g + rr) * kBlockCols + 16 * t + c] = acc[mt][t][rr];
      }
      __syncthreads();
      const int in_round = min(W, S - round * W);
#pragma unroll
      for (int e = 0; e < R * kBlockCols / NT; ++e) {
        const int idx = threadIdx.x + e * NT;
        float v = round == 0 ? pbuf[idx] : zsum[e] + pbuf[idx];
        for (int w = 1; w < in_round; ++w) v = v + pbuf[w * R * kBlockCols + idx];
        zsum[e] = v;
      }
    } else {
      // Write this wave's split partial P_s in the MFMA fragment layout
      // [s][row block][block][mt][t][lane] x float4 (4 rows of one column),
      // with agent-scope 128-bit stores; fragments whose 4 rows all lie past
      // M are skipped (their rows are zero and never read).
      if (active) {
        const __amdgpu_buffer_rsrc_t rp = make_rsrc(partial_frag(m, s, rb, nb, a.row_blocks, MT), MT * 8 * 1024);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int t = 0; t < CT; ++t)
            if (row_base + 16 * mt + 4 * g < M)
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[mt][t]), rp,
                                                     (mt * 8 + half * CT + t) * 1024 + 16 * lane, 0, kAgentScope);
      }
    }
  }

  float *zrow = (float *)(lds + kFoldBytes);             // [R][128]
  const EpiCols ec = epi_cols(m, col0, lane);

  if constexpr (CHAINED) {
    // every wave is past the last round's fold barriers, hence its last poll
    if (fused && threadIdx.x == 0) s_clear = rot_count_done(a);
#pragma unroll
    for (int e = 0; e < R * kBlockCols / NT; ++e) zrow[threadIdx.x + e * NT] = zsum[e];
  } else {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);             // this wave's partial stores are complete
    __syncthreads();
    __shared__ int s_last;
    uint32_t *counter = m.counters + (int64_t)rb * m.n_blocks + nb;
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (fused) s_clear = rot_count_done(a);
      s_last = prev == (uint32_t)(groups - 1);
    }
    __syncthreads();
    if (fused && s_clear) rot_clear(a);
    if (!s_last) return;
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Sum the S partials in split order. Thread x owns the FB fragments x,
    // x + NT, ... (of MT * 512); the loads of all of them are issued together,
    // B splits at a time (clamped to the last split), before they are added:
    // one memory round trip per B splits.
    constexpr int FB = MT * 512 / NT;
    constexpr int B = FB <= 2 ? 16 : 8;
    f32x4 zv[FB];
    bool live[FB];
#pragma unroll
    for (int e = 0; e < FB; ++e) {
      const int fl = (threadIdx.x + e * NT) & 63, fmt = (threadIdx.x + e * NT) >> 9;
      live[e] = row_base + 16 * fmt + 4 * (fl >> 4) < M;
    }
    for (int s0 = 0; s0 < S; s0 += B) {
      u32x4 v[FB][B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(partial_frag(m, min(s0 + u, S - 1), rb, nb, a.row_blocks, MT), MT * 8 * 1024);
#pragma unroll
        for (int e = 0; e < FB; ++e)
          v[e][u] = live[e] ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                            rp, 16 * (threadIdx.x + e * NT), 0, kAgentScope))
                            : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int e = 0; e < FB; ++e)
#pragma unroll
        for (int u = 0; u < B; ++u)
          if (s0 + u < S) zv[e] = (s0 + u == 0) ? __builtin_bit_cast(f32x4, v[e][u]) : zv[e] + __builtin_bit_cast(f32x4, v[e][u]);
    }
#pragma unroll
    for (int e = 0; e < FB; ++e) {
      const int f = threadIdx.x + e * NT;                // fragment index: mt, t, lane
      const int fl = f & 63, ft = (f >> 6) & 7, fmt = f >> 9;
      const int fr0 = 16 * fmt + 4 * (fl >> 4);          // first of its 4 rows in the row block
      if (live[e]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) zrow[(fr0 + q) * kBlockCols + 16 * ft + (fl & 15)] = zv[e][q];
      }
    }
  }
  __syncthreads();
  if (CHAINED && fused && s_clear) rot_clear(a);
  // 4 rows per wave and pass
  for (int r4 = 4 * wave; r4 < R && row_base + r4 < M; r4 += 4 * W)
    epilogue_rows_lds<1>(zrow + r4 * kBlockCols, kBlockCols, ec, lane, m, col0, row_base + r4, M);
}

// ------------------------------------------------------------ linear, 128-row tiles
//
// Mid-M and prompt rows. A workgroup computes 128 rows x one 128-column block;
// its 4 waves form a 2 x 2 grid of 64 x 64 tiles (4 x 4 MFMA tiles each).
// Per 32-deep chunk the workgroup stages, with 128-bit loads, the rotated
// input tile (128 rows x 32 K fp16, rows padded to 80 bytes so ds_read_b128
// is conflict free) and the block's packed words (the padded tile layout of
// the decode-row kernel) into LDS, double-buffered with one barrier per
// chunk; global loads run 4 chunks ahead in registers. Each wave decodes its
// 4 column tiles from the staged words and issues 16 MFMAs. Chains, their
// fold in split order and the epilogue are those of every other tiling.

// RH row halves of 64 rows: 2 (the 128-row tile, 4 waves) or 1 (the 64-row
// tile, 2 waves).
template <int BITS, int RH = 2>
struct TileLds {
  static constexpr int kArow = 80;                         // bytes per staged A row
  static constexpr int kA = 64 * RH * kArow;
  static constexpr int kBuf = kA + Stream<BITS>::kSlot;    // one chunk: A tile + B words
  static constexpr int kWaves = 2 * RH;
  static constexpr int kPieces = (Stream<BITS>::kLoads + kWaves - 1) / kWaves;   // B loads per wave
};

template <int NB>
struct TileStage {
  u32x4 a[2];                                              // this wave's 2 A loads (32 rows)
  u32x4 b[NB];                                             // this wave's B loads
};

template <int NB>
__device__ __forceinline__ void load_tile_stage(TileStage<NB> &st, __amdgpu_buffer_rsrc_t ra,
                                                __amdgpu_buffer_rsrc_t rb, const uint32_t (&voff_a)[2], int a_step,
                                                const uint32_t (&voff_b)[NB], int chunk, int chunk_bytes) {
  st.a[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)voff_a[0], chunk * a_step, 0));
  st.a[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)voff_a[1], chunk * a_step, 0));
#pragma unroll
  for (int i = 0; i < NB; ++i)
    st.b[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)voff_b[i], chunk * chunk_bytes, 0));
}

template <int BITS, int RH, int NB>
__device__ __forceinline__ void tile_stage_to_lds(const TileStage<NB> &st, char *buf, const uint32_t (&a_wr)[2],
                                                  const uint32_t (&b_wr)[NB], const uint32_t (&b_wrap)[NB]) {
  *(u32x4 *)(buf + a_wr[0]) = st.a[0];
  *(u32x4 *)(buf + a_wr[1]) = st.a[1];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    *(u32x4 *)(buf + TileLds<BITS, RH>::kA + b_wr[i]) = st.b[i];
    *(uint32_t *)(buf + TileLds<BITS, RH>::kA + b_wrap[i]) = st.b[i][0];
  }
}

template <int BITS, int RH>
__device__ __forceinline__ void compute_tile_chunk(const char *buf, const uint32_t (&a_rd)[4], uint32_t b_rd,
                                                   uint32_t shift, const CbConst &cb, f32x4 (&acc)[4][4]) {
  constexpr int ND = BitsTraits<BITS>::kDwords;
  half8 af[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) af[mt] = __builtin_bit_cast(half8, *(const u32x4 *)(buf + a_rd[mt]));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t *q = (const uint32_t *)(buf + TileLds<BITS, RH>::kA + b_rd + i * Stream<BITS>::kStride);
    uint32_t w[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) w[d] = q[d];
    const half8 bf = decode8<BITS>(w, shift, cb);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      acc[mt][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt], bf, acc[mt][i], 0, 0, 0);
  }
}

template <int BITS, bool CHAINED, int RH>
__device__ __forceinline__ void tile_body(const LinearArgs &a) {
  using SB = Stream<BITS>;
  using TL = TileLds<BITS, RH>;
  constexpr int W = TL::kWaves;
  constexpr int NB = TL::kPieces;
  constexpr int R = 64 * RH;
  constexpr int RT = 4 * RH;                               // 16-row tiles of a workgroup
  // register stages (chunks in flight; even, for the two LDS buffers): 2
  // where a wave stages two word pieces (64-row tiles above 4 bits)
  constexpr int P = NB > 1 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = wave >> 1, wc = wave & 1;
  const int bid = blockIdx.x;
  int j = 0;
  if (a.n_members > 1 && bid >= a.m[1].wg_begin) j = 1;
  if (a.n_members > 2 && bid >= a.m[2].wg_begin) j = 2;
  const MemberArgs &m = a.m[j];
  const int S = m.splits;
  const int groups = m.groups;                             // 1 (chained) or S
  const int local = bid - m.wg_begin;
  const int per_rb = m.n_blocks * groups;
  const int rb = local / per_rb;
  const int rem = local - rb * per_rb;
  const int nb = rem / groups;
  const int sg = rem - nb * groups;
  const int M = a.M, K = a.K, C = a.chunks;
  const int row_base = rb * R;
  const int col0 = nb * kBlockCols;

  constexpr int kStage = 2 * TL::kBuf;
  constexpr int PR = 16 * W;                               // rows per epilogue pass
  constexpr int kEpi = PR * 132 * 4;
  __shared__ __attribute__((aligned(16))) char lds[kStage > kEpi ? kStage : kEpi];

  // Xr row-major or chunk-major (each chunk's M rows contiguous, 64 bytes a row)
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(m.xr, (uint32_t)((uint64_t)M * K * 2));
  const bool cm = a.xr_chunk_major != 0;
  const int a_step = cm ? 64 * M : 64;                       // bytes from one chunk to the next
  const __amdgpu_buffer_rsrc_t rbuf = make_rsrc(m.words + (int64_t)nb * m.block_stride, (uint32_t)(16u * K * BITS));
  const int c = lane & 15, g = lane >> 4;

  // staging: wave w loads A rows 32w .. 32w+31 (16 per 128-bit load, 4 lanes
  // a row) and the 1 KB pieces w, w + W, ... of the chunk's words (pieces
  // and lanes past the chunk load its first bytes into the dump)
  uint32_t voff_a[2], a_wr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 32 * wave + 16 * i + (lane >> 2);
    const int row = row_base + r;
    voff_a[i] = row < M ? (uint32_t)(row * (cm ? 64 : 2 * K) + 16 * (lane & 3)) : kOutOfRange;
    a_wr[i] = (uint32_t)(r * TL::kArow + 16 * (lane & 3));
  }
  uint32_t voff_b[NB], b_wr[NB], b_wrap[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int piece = wave + W * i;
    const int boff = 1024 * piece + 16 * lane;
    const bool bvalid = piece < SB::kLoads && boff < SB::kChunkBytes;
    const int tau_w = boff / (32 * BITS), w_in = boff % (32 * BITS);
    voff_b[i] = bvalid ? (uint32_t)boff : 0u;
    b_wr[i] = bvalid ? (uint32_t)(tau_w * SB::kStride + w_in) : (uint32_t)(16 * SB::kStride);
    b_wrap[i] =
        bvalid ? (uint32_t)(tau_w * SB::kStride + 32 * BITS + (w_in == 0 ? 0 : 4)) : (uint32_t)(16 * SB::kStride);
  }
  // reading: A fragments of m-tiles 4wr..4wr+3, B words of column tiles 4wc..4wc+3
  uint32_t a_rd[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) a_rd[mt] = (uint32_t)((64 * wr + 16 * mt + c) * TL::kArow + 16 * g);
  const int jseg = 2 * c + (g & 1);
  const uint32_t shift = 8u * (uint32_t)((BITS * jseg) & 3);
  const uint32_t b_rd = (uint32_t)(((g >> 1) * 8 + 4 * wc) * SB::kStride + 4 * ((BITS * jseg) >> 2));
  const CbConst cbc = cb_const();

  // chunk range: all splits (chained) or split sg
  const int s_begin = CHAINED ? 0 : sg;
  const int cb = (int)(((int64_t)s_begin * C) / S);
  const int ce = (int)(((int64_t)(CHAINED ? S : sg + 1) * C) / S);
  const int n = ce - cb;
  const int last = ce - 1;
  int s = s_begin;
  int bnd = (int)(((int64_t)(s + 1) * C) / S);             // end of the current chain

  f32x4 acc[4][4];
  f32x4 z[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[mt][i] = z[mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  TileStage<NB> st[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    load_tile_stage<NB>(st[p], ra, rbuf, voff_a, a_step, voff_b, min(cb + p, last), SB::kChunkBytes);
    __builtin_amdgcn_sched_barrier(0);
  }
  tile_stage_to_lds<BITS, RH, NB>(st[0], lds, a_wr, b_wr, b_wrap);

  // one step: chunk cc from LDS buffer `cur`; chunk cc+1 is staged into the
  // other buffer first; the register stage of chunk cc reloads chunk cc+P
  auto step = [&](int cc, char *cur, char *nxt, TileStage<NB> &mine, TileStage<NB> &next, bool has_next) {
    __syncthreads();
    if (has_next) tile_stage_to_lds<BITS, RH, NB>(next, nxt, a_wr, b_wr, b_wrap);
    load_tile_stage<NB>(mine, ra, rbuf, voff_a, a_step, voff_b, min(cc + P, last), SB::kChunkBytes);
    compute_tile_chunk<BITS, RH>(cur, a_rd, b_rd, shift, cbc, acc);
    if (cc + 1 == bnd) {                                   // chain s complete (uniform)
      if constexpr (CHAINED) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            z[mt][i] = (s == 0) ? acc[mt][i] : z[mt][i] + acc[mt][i];
            acc[mt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
      ++s;
      bnd = (int)(((int64_t)(s + 1) * C) / S);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  int i = 0;
  for (; i + P < n; i += P) {
#pragma unroll
    for (int p = 0; p < P; ++p)
      step(cb + i + p, lds + (p % 2) * TL::kBuf, lds + ((p + 1) % 2) * TL::kBuf, st[p], st[(p + 1) % P], true);
  }
  const int r = n - i;
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < r)
      step(cb + i + p, lds + (p % 2) * TL::kBuf, lds + ((p + 1) % 2) * TL::kBuf, st[p], st[(p + 1) % P], p + 1 < r);

  float *zbuf = (float *)lds;                              // [PR][132]: PR rows per epilogue pass
  const EpiCols ec = epi_cols(m, col0, lane);

  if constexpr (!CHAINED) {
    // split sg's partial in the fragment layout, then the counter exchange
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(partial_frag(m, sg, rb, nb, a.row_blocks, RT), RT * 8 * 1024);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2)
        if (row_base + 64 * wr + 16 * mt + 4 * g < M)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[mt][i2]), rp,
                                                 ((4 * wr + mt) * 8 + 4 * wc + i2) * 1024 + 16 * lane, 0,
                                                 kAgentScope);
    if (a.fold_launch) return;                             // the split-fold launch adds them (uniform)
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    __shared__ int s_last;
    uint32_t *counter = m.counters + (int64_t)rb * m.n_blocks + nb;
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (uint32_t)(groups - 1);
    }
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // z = P0 + P1 + ... in split order for this wave's own 16 fragments: one
    // split at a time with all 16 of its fragment loads in flight (one memory
    // round trip per split, not one per split and fragment). Fragments of
    // rows past M hold stale bytes (in bounds: whole 128-row blocks) that no
    // row of the epilogue uses.
    for (int sp = 0; sp < S; ++sp) {
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(partial_frag(m, sp, rb, nb, a.row_blocks, RT), RT * 8 * 1024);
      u32x4 v[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
          v[mt][i2] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rq, 16 * (((4 * wr + mt) * 8 + 4 * wc + i2) * 64 + lane), 0,
                                                    kAgentScope));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
          z[mt][i2] = sp == 0 ? __builtin_bit_cast(f32x4, v[mt][i2]) : z[mt][i2] + __builtin_bit_cast(f32x4, v[mt][i2]);
    }
  }

  // epilogue: the R rows in passes of PR through LDS (the rows of a pass
  // come from the waves whose 64-row half holds them); in each pass wave w
  // finishes rows 16w .. 16w + 15 of the pass
#pragma unroll
  for (int pass = 0; pass < R / PR; ++pass) {
    const int prow = row_base + PR * pass;
    if (prow >= M) break;                                  // uniform
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int tr = 64 * wr + 16 * mt - PR * pass;        // the tile's first row in the pass
      if (tr >= 0 && tr < PR) {                            // uniform
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
#pragma unroll
          for (int q = 0; q < 4; ++q) zbuf[(tr + 4 * g + q) * 132 + 16 * (4 * wc + i2) + c] = z[mt][i2][q];
      }
    }
    __syncthreads();
    if (prow + 16 * wave < M)
      epilogue_rows_lds<4>(zbuf + 16 * wave * 132, 132, ec, lane, m, col0, prow + 16 * wave, M);
  }
}

// Exchanged (one split per workgroup, about 165 VGPRs): three workgroups per
// CU, so that the down projection's 640 workgroups at 49-128 rows run in one
// round instead of 1.25 (-5 to -9 %); chained (about 230 VGPRs): two.
template <int BITS, bool CHAINED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(CHAINED ? 2 : 3, CHAINED ? 2 : 3)))
void linear_tile_kernel(const LinearArgs a) {
  tile_body<BITS, CHAINED, 2>(a);
}

// The same exchanged tiling in 64-row tiles of 2 waves (64 x 64 each): with
// the split-fold launch, the down projection's 40 blocks x 16 splits are 640
// tiles at up to 64 rows and 1280 at 65-128, 2.5 and 5 per CU, where the
// 128-row tiles left 128 CUs with three workgroups and 128 with two.
template <int BITS>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(3, 3)))
void linear_tile64_kernel(const LinearArgs a) {
  tile_body<BITS, false, 1>(a);
}

// ------------------------------------------------------------ linear, 128 x 256 tiles
//
// Prompt rows. A workgroup computes 128 rows x two adjacent 128-column blocks
// of one member; wave w owns all 128 rows of block w / 2, columns 64 (w % 2)
// .. 64 (w % 2) + 63: 8 x 4 MFMA tiles, one wave per SIMD, so that each
// decoded B operand feeds 8 MFMAs and each A operand 4. Per 32-deep chunk the
// rotated input tile (128 rows x 64 bytes) and the two blocks' words are
// copied from memory straight into an LDS ring (buffer loads with the LDS
// destination: no staging registers, no LDS store instructions), kStages - 1
// chunks ahead, one barrier per chunk. The input tile is stored as 8 MFMA
// operands of 1 KB, lane l's 16 bytes at 16 l, so the operand reads are
// linear and free of bank conflicts; each tile row of words gets a slot
// padded to an odd multiple of 128 bytes, so the two tile rows a wave reads
// fall in opposite halves of the banks. A wave decodes the next
// chunk's 4 B operands between this chunk's MFMAs and re-reads each A operand
// for the next chunk as soon as its 4 MFMAs are issued. Chains, their fold in
// split order and the epilogue are those of every other tiling.

template <int BITS>
struct WideLds {
  static constexpr int kA = 128 * 64;                        // input tile of one chunk
  static constexpr int kRowBytes = 256 * BITS;               // one tile row (8 tiles) of one block
  static constexpr int kRowCopies = (kRowBytes + 1023) / 1024;
  static constexpr int kRow = 1024 * kRowCopies + 128;       // its slot: whole 1 KB copies + 128 bytes
  static constexpr int kStage = kA + 4 * kRow;               // + 2 blocks x 2 tile rows
  static constexpr int kStages = 8;
  static constexpr int kRing = kStages * kStage;
  static constexpr int kZ = 2 * 128 * 132 * 4;               // epilogue: both blocks' Z, 132-float rows
  static constexpr int kBytes = kRing > kZ ? kRing : kZ;
  static constexpr int kCopies = 2 + kRowCopies;             // 1 KB copies per wave and chunk
};

// s_waitcnt operand: at most n vector memory operations outstanding.
__host__ __device__ constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier without a memory fence. LDS filled by buffer-to-LDS
// copies is ordered by explicit vmcnt waits before it; the compiler may not
// move memory operations across it.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane: lane l's bytes land at dst + 16 l; lanes past the
// buffer's num_records write zeros. Every lane of the wave takes part: a
// lane with nothing to copy gets kOutOfRange and writes zeros into padding,
// because under a lane-divergent branch the compiler has been seen to merge
// two copies and take M0 from one lane (wrong LDS address for the others).
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t r, char *dst, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, (int)voff, soff, 0, 0);
}

// +0 in four fresh accumulator registers. Opaque to the optimizer, which
// otherwise merges every cleared accumulator into one register and then
// copies all of them on every pass of the chunk loop.
__device__ __forceinline__ f32x4 opaque_zero4() {
  float e0, e1, e2, e3;
  asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(e0));
  asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(e1));
  asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(e2));
  asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(e3));
  return f32x4{e0, e1, e2, e3};
}

template <int BITS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void linear_wide_kernel(const LinearArgs a) {
  using WL = WideLds<BITS>;
  using TR = BitsTraits<BITS>;
  constexpr int NS = WL::kStages;
  constexpr int ND = TR::kDwords;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;

  // Workgroup -> tile. Workgroups are dealt to the 8 XCDs in turn; each XCD
  // takes a contiguous range of tiles, ordered by groups of 8 block pairs and
  // within a group by row block, so the workgroups that share an L2 at a time
  // share input rows and words.
  const int T = a.total_wgs;
  const int xcd = blockIdx.x & 7;
  const int tile = xcd * (T >> 3) + min(xcd, T & 7) + (int)(blockIdx.x >> 3);
  int j = 0;
  if (a.n_members > 1 && tile >= a.m[1].wg_begin) j = 1;
  if (a.n_members > 2 && tile >= a.m[2].wg_begin) j = 2;
  const MemberArgs &m = a.m[j];
  const int RB = a.row_blocks;
  const int pairs = (m.n_blocks + 1) >> 1;
  const int local = tile - m.wg_begin;
  const int pg = local / (8 * RB);
  const int in_g = local - pg * 8 * RB;
  const int gp = min(8, pairs - 8 * pg);
  const int rb = in_g / gp;
  const int pair = 8 * pg + (in_g - rb * gp);
  const int M = a.M, K = a.K, C = a.chunks;
  const int row_base = rb * 128;
  const int col0 = pair * 2 * kBlockCols;
  const int n_blk = min(2, m.n_blocks - 2 * pair);           // 1 or 2 blocks in this pair

  __shared__ __attribute__((aligned(16))) char lds[WL::kBytes];

  // copies: wave w moves input operands 2w + e (e = 0, 1; lane l brings row
  // 16 (2w + e) + l % 16, 16-byte column l / 16) and tile row slot w (block
  // w / 2, tile row w % 2) of every chunk
  const __amdgpu_buffer_rsrc_t ra =
      a.xr_chunk_major ? make_rsrc(m.xr + (int64_t)row_base * kChunk, (uint32_t)(C * M - row_base) * 64u)
                       : make_rsrc(m.xr + (int64_t)row_base * K, (uint32_t)min(M - row_base, 128) * (uint32_t)K * 2u);
  // Xr chunk-major (each chunk's M rows contiguous, 64 bytes a row) or row-major
  const int a_row = a.xr_chunk_major ? 64 : 2 * K;           // bytes from one row to the next
  const int a_step = a.xr_chunk_major ? 64 * M : 64;         // bytes from one chunk to the next
  uint32_t va[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int r = 16 * (2 * wave + e) + c;                   // operand 2w + e: rows 16 (2w + e) + l % 16
    va[e] = row_base + r < M ? (uint32_t)(r * a_row + 16 * g) : kOutOfRange;
  }
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(m.words + (int64_t)2 * pair * m.block_stride, (uint32_t)(n_blk * m.block_stride));
  const int qw = wave >> 1, hw = wave & 1;
  uint32_t vw[WL::kRowCopies];
#pragma unroll
  for (int e = 0; e < WL::kRowCopies; ++e) {
    const int b = 1024 * e + 16 * lane;
    vw[e] = b < WL::kRowBytes ? (uint32_t)(qw * m.block_stride + hw * WL::kRowBytes + b) : kOutOfRange;
  }
  auto issue_copies = [&](int chunk, char *stage) {
#pragma unroll
    for (int e = 0; e < 2; ++e) copy_to_lds(ra, stage + 1024 * (2 * wave + e), va[e], chunk * a_step);
#pragma unroll
    for (int e = 0; e < WL::kRowCopies; ++e)
      copy_to_lds(rw, stage + WL::kA + wave * WL::kRow + 1024 * e, vw[e], chunk * 512 * BITS);
  };

  // operand reads: A operand mt at 1 KB mt + 16 lane (linear: no bank
  // conflicts) and the lane's word dwords of column tiles 4 (w % 2) + t of
  // block w / 2
  const uint32_t a_rd = (uint32_t)(16 * lane);
  const BLane<BITS> bl = b_lane<BITS>(lane);
  uint32_t w_rd[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
    w_rd[d] = (uint32_t)(WL::kA + (2 * qw + (g >> 1)) * WL::kRow + hw * 128 * BITS) + bl.voff[d] -
              (uint32_t)((g >> 1) * WL::kRowBytes);
  const CbConst cbc = cb_const();

  auto stage_of = [&](int i) { return lds + (i & (NS - 1)) * WL::kStage; };
  auto read_a = [&](half8 (&af)[8], const char *st) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) af[mt] = __builtin_bit_cast(half8, *(const u32x4 *)(st + a_rd + 1024 * mt));
  };
  auto read_w = [&](uint32_t (&w)[4][ND], const char *st) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int d = 0; d < ND; ++d) w[t][d] = *(const uint32_t *)(st + w_rd[d] + 32 * BITS * t);
  };

  // z = P0 + P1 + ... in split order, starting from +0: an MFMA chain that
  // starts from +0 never ends in -0, so +0 + P0 is P0 bit for bit
  f32x4 acc[8][4], z[8][4];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t) z[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int last = C - 1;
  const int S = m.splits;

  // prologue: chunks 0 .. NS - 2 in flight; chunks 0 and 1 landed
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue_copies(min(p, last), stage_of(p));
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(WL::kCopies * (NS - 3)));
  ring_barrier();
  half8 af[8], bc[4], bn[4];
  uint32_t wa[4][ND], wb[4][ND];
  read_a(af, stage_of(0));
  read_w(wa, stage_of(0));
#pragma unroll
  for (int t = 0; t < 4; ++t) bc[t] = decode8<BITS>(wa[t], bl.shift, cbc);
  read_w(wa, stage_of(1));

  // one chunk: MFMAs of chunk cc (A in af, B in bc; FIRST: the chain's first
  // chunk, accumulating onto zero); meanwhile the words of chunk cc + 1 (wa)
  // become its B operands (bn), the words of chunk cc + 2 are read (wb) and
  // af is refilled with chunk cc + 1's A
  auto step = [&](int cc, auto first, half8 (&bc)[4], half8 (&bn)[4], uint32_t (&wa)[4][ND],
                  uint32_t (&wb)[4][ND]) {
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(WL::kCopies * (NS - 4)));   // this wave's copies of chunk cc + 2
    ring_barrier();                                         // everyone's; the stage of chunk cc - 1 is free
    issue_copies(min(cc + NS - 1, last), stage_of(cc + NS - 1));
    read_w(wb, stage_of(cc + 2));
    const char *nxt = stage_of(cc + 1);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt], bc[t], decltype(first)::value ? f32x4{0.f, 0.f, 0.f, 0.f}
                                                                                               : acc[mt][t], 0, 0, 0);
      af[mt] = __builtin_bit_cast(half8, *(const u32x4 *)(nxt + a_rd + 1024 * mt));
      if (mt & 1) bn[mt >> 1] = decode8<BITS>(wa[mt >> 1], bl.shift, cbc);
    }
    // issue order: each MFMA followed by about two VALU operations (the
    // decode of the next chunk), each A operand's reload after its 4 MFMAs
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
    }
  };
  using First = std::integral_constant<bool, true>;
  using Rest = std::integral_constant<bool, false>;
  // chain s covers chunks [s C / S, (s + 1) C / S), at least one chunk; its
  // sum is then added to z (accumulator registers read into the add
  // directly, so z stays in place)
  for (int sp = 0; sp < S; ++sp) {
    const int c0 = sp * C / S, c1 = (sp + 1) * C / S;      // S * C < 2^31
    step(c0, First{}, bc, bn, wa, wb);
    int cc = c0 + 1;
    for (; cc + 1 < c1; cc += 2) {
      step(cc, Rest{}, bn, bc, wb, wa);
      step(cc + 1, Rest{}, bc, bn, wa, wb);
    }
    if (cc < c1) {
      step(cc, Rest{}, bn, bc, wb, wa);
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bc[t] = bn[t];
#pragma unroll
        for (int d = 0; d < ND; ++d) wa[t][d] = wb[t][d];
      }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v;
          asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(acc[mt][t][q]));
          z[mt][t][q] = z[mt][t][q] + v;
        }
  }

  // epilogue: both blocks' Z through LDS once every copy has landed
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  float *zb = (float *)lds;                                  // [2][128][132]
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) zb[(qw * 128 + 16 * mt + 4 * g + q) * 132 + 64 * hw + 16 * t + c] = z[mt][t][q];
  const EpiCols ec0 = epi_cols(m, col0, lane);
  EpiCols ec1 = ec0;
  if (n_blk > 1) ec1 = epi_cols(m, col0 + kBlockCols, lane);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grp = wave + 4 * i;                            // 16-row group: block grp / 8, rows 16 (grp % 8) ..
    const int q = grp >> 3, r16 = 16 * (grp & 7);
    if (q < n_blk && row_base + r16 < M)
      epilogue_rows_lds<4>(zb + (q * 128 + r16) * 132, 132, q ? ec1 : ec0, lane, m, col0 + q * kBlockCols,
                           row_base + r16, M);
  }
}

// ------------------------------------------------------------ linear, 128-row block tiles
//
// Mid rows of wide weights and prompt rows of all but long-split weights
// (chained; the exchanged form only when forced). A workgroup of
// 4 waves computes 128 rows x one 128-column block; wave w owns all 128 rows
// of column tiles 2w, 2w + 1 (8 x 2 MFMA tiles), so each decoded B operand
// feeds 8 MFMAs, and two workgroups fit on a CU (two waves per SIMD).
// linear_block64_kernel is the same with 64 rows (4 x 2 MFMA tiles a wave)
// for launches of at most 64 rows, linear_block32_kernel with 32 rows (2 x 2)
// for launches of at most 32 rows. The operands reach LDS as in the
// 128 x 256 tiling: buffer-to-LDS copies into a 6-stage ring, input operands
// stored linearly, tile rows of words in padded slots. Chained: every split of the block, folded in split order (then,
// with left blocks, one split of a left block, its partial stored for the
// split-fold launch). Exchanged: one split per workgroup, its partial stored
// in the fragment layout; the block's last arriving workgroup adds the S
// partials in split order, resets the counter and finishes the rows.

template <int BITS, int RT = 8>
struct BlockLds {
  static constexpr int kAT = RT < 4 ? 4 : RT;                // input operand slots: one copy per wave at least
  static constexpr int kA = kAT * 16 * 64;                   // input tile of one chunk (RT * 16 rows used)
  static constexpr int kRowBytes = 256 * BITS;               // one tile row (8 tiles) of the block
  static constexpr int kRow = 2048 + 128;                    // its slot: two 1 KB halves (4 tiles each) + 128 bytes
  static constexpr int kStage = kA + 2 * kRow;
  static constexpr int kStages = 6;
  static constexpr int kRing = kStages * kStage;
  static constexpr int kZ = RT * 16 * 132 * 4;               // epilogue: the block's Z, 132-float rows
  static constexpr int kBytes = kRing > kZ ? kRing : kZ;
  static constexpr int kPiece = kRowBytes / 2;               // bytes of a half tile row (4 tiles, <= 1 KB)
  static constexpr int kCopies = kAT / 4 + 1;                // copies per wave and chunk: kAT / 4 input operands + a piece
};

// RT row tiles of 16 per workgroup: 8 (128 rows) or, chained, 4 (64 rows,
// for launches of at most 64 rows: half the MFMAs, the same bits per row)
// or 2 (32 rows, at most 32).
template <int BITS, bool CHAINED, int RT>
__device__ __forceinline__ void block_body(const LinearArgs &a) {
  static_assert(RT == 8 || ((RT == 4 || RT == 2) && CHAINED), "64- and 32-row workgroups: chained only");
  using BL = BlockLds<BITS, RT>;
  constexpr int R = 16 * RT;                                 // rows per workgroup
  constexpr int AE = BL::kAT / 4;                            // input operands each wave copies per chunk
  using TR = BitsTraits<BITS>;
  constexpr int NS = BL::kStages;
  constexpr int ND = TR::kDwords;
  constexpr int TN = 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;

  // Workgroup -> (member, row block, block, split): dealt to the 8 XCDs in
  // turn, each XCD taking a contiguous range ordered by groups of 8 blocks,
  // then row block, block and split.
  const int T = a.total_wgs;
  const int xcd = blockIdx.x & 7;
  const int tile = xcd * (T >> 3) + min(xcd, T & 7) + (int)(blockIdx.x >> 3);
  int j = 0;
  if (a.n_members > 1 && tile >= a.m[1].wg_begin) j = 1;
  if (a.n_members > 2 && tile >= a.m[2].wg_begin) j = 2;
  const MemberArgs &m = a.m[j];
  const int RB = a.row_blocks;
  const int groups = m.groups;                               // 1 (chained) or S
  const int local = tile - m.wg_begin;
  const int pg = local / (8 * RB * groups);
  const int in_g = local - pg * 8 * RB * groups;
  const int gp = min(8, m.n_blocks - 8 * pg);
  const int rb = in_g / (gp * groups);
  const int r2 = in_g - rb * gp * groups;
  const int nb = 8 * pg + r2 / groups;
  const int sg = r2 - (r2 / groups) * groups;
  const int M = a.M, K = a.K, C = a.chunks;
  const int S = m.splits;
  const int row_base = rb * R;
  const int col0 = nb * kBlockCols;

  __shared__ __attribute__((aligned(16))) char lds[BL::kBytes];

  // copies: wave w moves input operands AE w + e (lane l brings row
  // 16 (AE w + e) + l % 16, 16-byte column l / 16) and half w % 2 of tile
  // row w / 2 of every chunk; with 2 row tiles, waves 2 and 3 fill unused
  // operand slots with zeros (out-of-range copies, no memory read), so every
  // wave counts the same copies per chunk
  auto xr_rsrc = [&](const MemberArgs &mm) {
    return a.xr_chunk_major ? make_rsrc(mm.xr + (int64_t)row_base * kChunk, (uint32_t)(C * M - row_base) * 64u)
                            : make_rsrc(mm.xr + (int64_t)row_base * K, (uint32_t)min(M - row_base, R) * (uint32_t)K * 2u);
  };
  __amdgpu_buffer_rsrc_t ra = xr_rsrc(m);
  // Xr chunk-major (each chunk's M rows contiguous, 64 bytes a row) or row-major
  const int a_row = a.xr_chunk_major ? 64 : 2 * K;           // bytes from one row to the next
  const int a_step = a.xr_chunk_major ? 64 * M : 64;         // bytes from one chunk to the next
  uint32_t va[AE];
#pragma unroll
  for (int e = 0; e < AE; ++e) {
    const int r = 16 * (AE * wave + e) + c;
    va[e] = AE * wave + e < RT && row_base + r < M ? (uint32_t)(r * a_row + 16 * g) : kOutOfRange;
  }
  __amdgpu_buffer_rsrc_t rw = make_rsrc(m.words + (int64_t)nb * m.block_stride, (uint32_t)m.block_stride);
  const int hrow = wave >> 1, half = wave & 1;
  const uint32_t vw =
      16 * lane < BL::kPiece ? (uint32_t)(hrow * BL::kRowBytes + half * BL::kPiece + 16 * lane) : kOutOfRange;
  auto stage_of = [&](int i) { return lds + (int)((unsigned)i % NS) * BL::kStage; };
  auto issue_copies = [&](int chunk, char *stage) {
#pragma unroll
    for (int e = 0; e < AE; ++e) copy_to_lds(ra, stage + 1024 * (AE * wave + e), va[e], chunk * a_step);
    copy_to_lds(rw, stage + BL::kA + hrow * BL::kRow + half * 1024, vw, chunk * 512 * BITS);
  };

  // operand reads: A operand mt at 1 KB mt + 16 lane; the lane's word dwords
  // of column tiles 2w + t
  const int t0 = 2 * wave;
  const uint32_t a_rd = (uint32_t)(16 * lane);
  const BLane<BITS> bl = b_lane<BITS>(lane);
  uint32_t w_rd[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
    w_rd[d] = (uint32_t)(BL::kA + (g >> 1) * BL::kRow + (t0 >> 2) * 1024 + (t0 & 3) * 32 * BITS) + bl.voff[d] -
              (uint32_t)((g >> 1) * BL::kRowBytes);
  const CbConst cbc = cb_const();
  auto read_a = [&](half8 (&af)[RT], const char *st) {
#pragma unroll
    for (int mt = 0; mt < RT; ++mt) af[mt] = __builtin_bit_cast(half8, *(const u32x4 *)(st + a_rd + 1024 * mt));
  };
  auto read_w = [&](uint32_t (&w)[TN][ND], const char *st) {
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int d = 0; d < ND; ++d) w[t][d] = *(const uint32_t *)(st + w_rd[d] + 32 * BITS * t);
  };

  // chunk range: every split (chained) or split sg
  const int cbeg = CHAINED ? 0 : (int)(sg * C / S);
  const int cend = CHAINED ? C : (int)((sg + 1) * C / S);
  int last = cend - 1;

  // z = P0 + P1 + ... in split order, starting from +0: an MFMA chain that
  // starts from +0 never ends in -0, so +0 + P0 is P0 bit for bit
  f32x4 acc[RT][TN], z[RT][TN];
#pragma unroll
  for (int mt = 0; mt < RT; ++mt)
#pragma unroll
    for (int t = 0; t < TN; ++t) z[mt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue of a chunk range from c0: chunks c0 .. c0 + NS - 2 in flight;
  // c0 and c0 + 1 landed
  half8 af[RT], bc[TN], bn[TN];
  uint32_t wa[TN][ND], wb[TN][ND];
  auto prologue = [&](int c0) {
#pragma unroll
    for (int p = 0; p < NS - 1; ++p) issue_copies(min(c0 + p, last), stage_of(c0 + p));
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(BL::kCopies * (NS - 3)));
    ring_barrier();
    read_a(af, stage_of(c0));
    read_w(wa, stage_of(c0));
#pragma unroll
    for (int t = 0; t < TN; ++t) bc[t] = decode8<BITS>(wa[t], bl.shift, cbc);
    read_w(wa, stage_of(c0 + 1));
  };
  prologue(cbeg);

  // one chunk: MFMAs of chunk cc (A in af, B in bc; FIRST: the chain's first
  // chunk, accumulating onto zero); meanwhile the words of chunk cc + 1 (wa)
  // become its B operands (bn), the words of chunk cc + 2 are read (wb) and
  // af is refilled with chunk cc + 1's A
  auto step = [&](int cc, auto first, half8 (&bc)[TN], half8 (&bn)[TN], uint32_t (&wa)[TN][ND],
                  uint32_t (&wb)[TN][ND]) {
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(BL::kCopies * (NS - 4)));   // this wave's copies of chunk cc + 2
    ring_barrier();                                         // everyone's; the stage of chunk cc - 1 is free
    issue_copies(min(cc + NS - 1, last), stage_of(cc + NS - 1));
    read_w(wb, stage_of(cc + 2));
    const char *nxt = stage_of(cc + 1);
    constexpr int DQ = RT / TN;                              // row tiles per decoded B operand
#pragma unroll
    for (int mt = 0; mt < RT; ++mt) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
        acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt], bc[t], decltype(first)::value ? f32x4{0.f, 0.f, 0.f, 0.f}
                                                                                               : acc[mt][t], 0, 0, 0);
      af[mt] = __builtin_bit_cast(half8, *(const u32x4 *)(nxt + a_rd + 1024 * mt));
      if ((mt + 1) % DQ == 0) bn[mt / DQ] = decode8<BITS>(wa[mt / DQ], bl.shift, cbc);
    }
    if constexpr (CHAINED) {
      // issue order: the copies, the word reads, then per row tile its two
      // MFMAs, its next A read and a share of the decode (-5 % chained; the
      // exchanged form measured slightly slower with it)
      __builtin_amdgcn_sched_group_barrier(0x020, 3, 0);     // buffer-to-LDS copies
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);     // LDS reads
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
      }
    }
  };
  using First = std::integral_constant<bool, true>;
  using Rest = std::integral_constant<bool, false>;
  auto chain = [&](int c0, int c1) {
    step(c0, First{}, bc, bn, wa, wb);
    int cc = c0 + 1;
    for (; cc + 1 < c1; cc += 2) {
      step(cc, Rest{}, bn, bc, wb, wa);
      step(cc + 1, Rest{}, bc, bn, wa, wb);
    }
    if (cc < c1) {
      step(cc, Rest{}, bn, bc, wb, wa);
    } else {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        bc[t] = bn[t];
#pragma unroll
        for (int d = 0; d < ND; ++d) wa[t][d] = wb[t][d];
      }
    }
  };
  // z += the split's chain sum. The accumulators are left to the compiler:
  // in VGPRs (209-221 of the 256 two waves per SIMD allow) the fold is one
  // add per value instead of a read out of AGPRs and an add, about 0.4
  // fewer VALU instructions per MFMA (8192-row layer 5.26-5.29 -> 5.18 ms)
  auto fold = [&]() {
#pragma unroll
    for (int mt = 0; mt < RT; ++mt)
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) z[mt][t][e] = z[mt][t][e] + acc[mt][t][e];
  };

  if constexpr (CHAINED) {
    // chain s covers chunks [s C / S, (s + 1) C / S), at least one chunk
    for (int sp = 0; sp < S; ++sp) {
      chain(sp * C / S, (sp + 1) * C / S);                  // S * C < 2^31
      fold();
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  } else {
    chain(cbeg, cend);
    // split sg's partial in the fragment layout, then the counter exchange
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(partial_frag(m, sg, rb, nb, RB, 8), 8 * 8 * 1024);
#pragma unroll
    for (int mt = 0; mt < RT; ++mt)
#pragma unroll
      for (int t = 0; t < TN; ++t)
        if (row_base + 16 * mt + 4 * g < M) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[e]) : "a"(acc[mt][t][e]));
          __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                       __float_as_uint(v[2]), __float_as_uint(v[3])},
                                                 rp, (mt * 8 + t0 + t) * 1024 + 16 * lane, 0, kAgentScope);
        }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);                 // this wave's partial stores are complete
    __syncthreads();
    __shared__ int s_last;
    uint32_t *counter = m.counters + (int64_t)rb * m.n_blocks + nb;
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (uint32_t)(groups - 1);
    }
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // z = P0 + P1 + ... in split order for this wave's 16 fragments: two
    // splits at a time with all 32 fragment loads in flight (one memory round
    // trip per two splits). z starts from +0: +0 + P0 is P0 bit for bit (an
    // MFMA chain from +0 never ends in -0). Fragments of rows past M hold
    // stale bytes (in bounds: whole 128-row blocks) that no row of the
    // epilogue uses.
    for (int s0 = 0; s0 < S; s0 += 2) {
      u32x4 v[2][RT][TN];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(partial_frag(m, min(s0 + u, S - 1), rb, nb, RB, 8), 8 * 8 * 1024);
#pragma unroll
        for (int mt = 0; mt < RT; ++mt)
#pragma unroll
          for (int t = 0; t < TN; ++t)
            v[u][mt][t] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, 16 * ((mt * 8 + t0 + t) * 64 + lane), 0, kAgentScope));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (s0 + u < S)                                     // uniform
#pragma unroll
          for (int mt = 0; mt < RT; ++mt)
#pragma unroll
            for (int t = 0; t < TN; ++t) z[mt][t] = z[mt][t] + __builtin_bit_cast(f32x4, v[u][mt][t]);
    }
  }

  // epilogue: the block's Z through LDS
  float *zb = (float *)lds;                                  // [R][132]
#pragma unroll
  for (int mt = 0; mt < RT; ++mt)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) zb[(16 * mt + 4 * g + e) * 132 + 16 * (t0 + t) + c] = z[mt][t][e];
  const EpiCols ec = epi_cols(m, col0, lane);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < (RT + 3) / 4; ++i) {
    const int r16 = 16 * (wave + 4 * i);
    if (r16 < R && row_base + r16 < M) epilogue_rows_lds<4>(zb + r16 * 132, 132, ec, lane, m, col0, row_base + r16, M);
  }

  if constexpr (CHAINED) {
    // Left blocks (one row block, more blocks than workgroups): the launch
    // has a workgroup for each of its first own_blocks blocks only; the S
    // splits of each of the left_blocks blocks after them go one to a
    // workgroup, which after its own block runs that split's chain and
    // stores the partial ([split][left block of the member] x 8 KB per
    // 16-row tile, at the member's partials); the split-fold launch after
    // this one adds them in split order and finishes those blocks' rows.
    const int task = tile;
    if (a.left_blocks > 0 && task < a.left_blocks * S) {   // uniform
      const int lb = task / S, sp = task - lb * S;
      const int gb = a.own_blocks + lb;                      // the left block among the launch's blocks
      int j2 = 0;
      if (a.n_members > 1 && gb >= a.m[1].wg_begin) j2 = 1;
      if (a.n_members > 2 && gb >= a.m[2].wg_begin) j2 = 2;
      const MemberArgs &m2 = a.m[j2];
      const int nb2 = gb - m2.wg_begin;
      const int first_left = max(0, a.own_blocks - m2.wg_begin);   // the member's first left block
      const int c0 = (int)(((int64_t)sp * C) / S), c1 = (int)(((int64_t)(sp + 1) * C) / S);
      ra = xr_rsrc(m2);
      rw = make_rsrc(m2.words + (int64_t)nb2 * m2.block_stride, (uint32_t)m2.block_stride);
      last = c1 - 1;
      __syncthreads();                                       // the epilogue's LDS reads are done
      prologue(c0);
      chain(c0, c1);
      const __amdgpu_buffer_rsrc_t rp =
          make_rsrc(m2.partials + ((int64_t)sp * (m2.n_blocks - first_left) + (nb2 - first_left)) * (8 * 8 * 256),
                    8 * 8 * 1024);
#pragma unroll
      for (int mt = 0; mt < RT; ++mt)
#pragma unroll
        for (int t = 0; t < TN; ++t)
          if (16 * mt + 4 * g < M)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[mt][t]), rp,
                                                   (mt * 8 + t0 + t) * 1024 + 16 * lane, 0, 0);
    }
  }
}

template <int BITS, bool CHAINED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void linear_block_kernel(const LinearArgs a) {
  block_body<BITS, CHAINED, 8>(a);
}

template <int BITS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void linear_block64_kernel(const LinearArgs a) {
  block_body<BITS, true, 4>(a);
}

template <int BITS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void linear_block32_kernel(const LinearArgs a) {
  block_body<BITS, true, 2>(a);
}

// ------------------------------------------------------------ linear, opt-in single-chain prompt tiles
//
// Opt-in prompt arithmetic (not bit-equal to the other regimes): each
// output is one MFMA chain over all of K, with no K splits and no fold, so a
// wave can hold a 128 x 128 tile (8 x 8 MFMA tiles, 256 accumulators) and
// each decoded B operand feeds 8 MFMAs while each A operand feeds 8. A
// workgroup of 4 waves computes 128 rows x 4 adjacent blocks, wave w block w;
// the operands reach LDS as in the 128 x 256 tiling (buffer-to-LDS copies,
// input operands stored linearly, padded tile-row slots). The epilogue runs
// on the accumulators directly (a wave holds whole 128-column rows).

template <int BITS>
struct QuadLds {
  static constexpr int kA = 128 * 64;                        // input tile of one chunk
  static constexpr int kRowBytes = 256 * BITS;               // one tile row (8 tiles) of one block
  static constexpr int kRowCopies = (kRowBytes + 1023) / 1024;
  static constexpr int kRow = 1024 * kRowCopies + 128;       // its slot: whole 1 KB copies + 128 bytes
  static constexpr int kStage = kA + 8 * kRow;               // + 4 blocks x 2 tile rows
  static constexpr int kScratch = 4 * 4096;                  // epilogue: 4 KB of bf16 rows per wave
  static constexpr int kStages = (160 * 1024 - kScratch) / kStage < 8 ? (160 * 1024 - kScratch) / kStage : 8;
  static constexpr int kRing = kStages * kStage;
  static constexpr int kBytes = kRing + kScratch;
  static constexpr int kCopies = 2 + 2 * kRowCopies;         // per wave and chunk: 2 input operands + 2 tile rows
};

template <int BITS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void linear_quad_kernel(const LinearArgs a) {
  using QL = QuadLds<BITS>;
  using TR = BitsTraits<BITS>;
  constexpr int NS = QL::kStages;
  constexpr int ND = TR::kDwords;
  static_assert(NS >= 4, "ring too shallow");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;

  // workgroup -> (member, row block, quad of blocks), dealt to the 8 XCDs in
  // turn, each XCD a contiguous range ordered by groups of 4 quads, then row
  // block
  const int T = a.total_wgs;
  const int xcd = blockIdx.x & 7;
  const int tile = xcd * (T >> 3) + min(xcd, T & 7) + (int)(blockIdx.x >> 3);
  int j = 0;
  if (a.n_members > 1 && tile >= a.m[1].wg_begin) j = 1;
  if (a.n_members > 2 && tile >= a.m[2].wg_begin) j = 2;
  const MemberArgs &m = a.m[j];
  const int RB = a.row_blocks;
  const int quads = (m.n_blocks + 3) >> 2;
  const int local = tile - m.wg_begin;
  const int pg = local / (4 * RB);
  const int in_g = local - pg * 4 * RB;
  const int gp = min(4, quads - 4 * pg);
  const int rb = in_g / gp;
  const int quad = 4 * pg + (in_g - rb * gp);
  const int M = a.M, K = a.K, C = a.chunks;
  const int row_base = rb * 128;
  const int n_blk = min(4, m.n_blocks - 4 * quad);           // 1..4 blocks in this quad
  const int col0 = (4 * quad + wave) * kBlockCols;           // this wave's block

  __shared__ __attribute__((aligned(16))) char lds[QL::kBytes];

  // copies: wave w moves input operands 2w + e (lane l: row 16 (2w + e) + l % 16,
  // 16-byte column l / 16) and both tile rows of block w
  const __amdgpu_buffer_rsrc_t ra =
      a.xr_chunk_major ? make_rsrc(m.xr + (int64_t)row_base * kChunk, (uint32_t)(C * M - row_base) * 64u)
                       : make_rsrc(m.xr + (int64_t)row_base * K, (uint32_t)min(M - row_base, 128) * (uint32_t)K * 2u);
  // Xr chunk-major (each chunk's M rows contiguous, 64 bytes a row) or row-major
  const int a_row = a.xr_chunk_major ? 64 : 2 * K;           // bytes from one row to the next
  const int a_step = a.xr_chunk_major ? 64 * M : 64;         // bytes from one chunk to the next
  uint32_t va[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int r = 16 * (2 * wave + e) + c;
    va[e] = row_base + r < M ? (uint32_t)(r * a_row + 16 * g) : kOutOfRange;
  }
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(m.words + (int64_t)4 * quad * m.block_stride, (uint32_t)(n_blk * m.block_stride));
  uint32_t vw[2][QL::kRowCopies];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < QL::kRowCopies; ++e) {
      const int b = 1024 * e + 16 * lane;
      vw[h][e] = b < QL::kRowBytes ? (uint32_t)(wave * m.block_stride + h * QL::kRowBytes + b) : kOutOfRange;
    }
  auto stage_of = [&](int i) { return lds + (int)((unsigned)i % NS) * QL::kStage; };
  auto issue_copies = [&](int chunk, char *stage) {
#pragma unroll
    for (int e = 0; e < 2; ++e) copy_to_lds(ra, stage + 1024 * (2 * wave + e), va[e], chunk * a_step);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < QL::kRowCopies; ++e)
        copy_to_lds(rw, stage + QL::kA + (2 * wave + h) * QL::kRow + 1024 * e, vw[h][e], chunk * 512 * BITS);
  };

  // operand reads: A operand mt at 1 KB mt + 16 lane; the lane's word dwords
  // of column tile t of block w
  const uint32_t a_rd = (uint32_t)(16 * lane);
  const BLane<BITS> bl = b_lane<BITS>(lane);
  uint32_t w_rd[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d)
    w_rd[d] = (uint32_t)(QL::kA + (2 * wave + (g >> 1)) * QL::kRow) + bl.voff[d] - (uint32_t)((g >> 1) * QL::kRowBytes);
  const CbConst cbc = cb_const();
  auto read_w = [&](uint32_t (&w)[8][ND], const char *st) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int d = 0; d < ND; ++d) w[t][d] = *(const uint32_t *)(st + w_rd[d] + 32 * BITS * t);
  };

  f32x4 acc[8][8];
  const int last = C - 1;

  // prologue: chunks 0 .. NS - 2 in flight; chunks 0 and 1 landed
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue_copies(min(p, last), stage_of(p));
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(QL::kCopies * (NS - 3)));
  ring_barrier();
  half8 af[8], bc[8];
  uint32_t wa[8][ND];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) af[mt] = __builtin_bit_cast(half8, *(const u32x4 *)(stage_of(0) + a_rd + 1024 * mt));
  read_w(wa, stage_of(0));
#pragma unroll
  for (int t = 0; t < 8; ++t) bc[t] = decode8<BITS>(wa[t], bl.shift, cbc);
  read_w(wa, stage_of(1));

  // one chunk: column tile t's 8 MFMAs use bc[t], after which bc[t] is
  // refilled with chunk cc + 1's operand (from wa); chunk cc + 1's A goes to
  // an (read at the start, so it has the whole chunk to arrive) and the
  // words of chunk cc + 2 to wb
  half8 a2[8];
  uint32_t wb[8][ND];
  auto step = [&](int cc, auto first, half8 (&ac)[8], half8 (&an)[8], uint32_t (&wc)[8][ND], uint32_t (&wn)[8][ND]) {
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(QL::kCopies * (NS - 4)));   // this wave's copies of chunk cc + 2
    ring_barrier();                                         // everyone's; the stage of chunk cc - 1 is free
    issue_copies(min(cc + NS - 1, last), stage_of(cc + NS - 1));
    const char *nxt = stage_of(cc + 1);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) an[mt] = __builtin_bit_cast(half8, *(const u32x4 *)(nxt + a_rd + 1024 * mt));
    read_w(wn, stage_of(cc + 2));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac[mt], bc[t], decltype(first)::value ? f32x4{0.f, 0.f, 0.f, 0.f}
                                                                                               : acc[mt][t], 0, 0, 0);
      bc[t] = decode8<BITS>(wc[t], bl.shift, cbc);
    }
  };
  using First = std::integral_constant<bool, true>;
  using Rest = std::integral_constant<bool, false>;
  step(0, First{}, af, a2, wa, wb);
  int cc = 1;
  for (; cc + 1 < C; cc += 2) {
    step(cc, Rest{}, a2, af, wb, wa);
    step(cc + 1, Rest{}, af, a2, wa, wb);
  }
  if (cc < C) step(cc, Rest{}, a2, af, wb, wa);

  // epilogue straight from the accumulators: row tile mt of block w
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (wave < n_blk) {
    const EpiCols ec = epi_cols(m, col0, lane);
    uint16_t *scratch = (uint16_t *)(lds + QL::kRing + 4096 * wave);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      if (row_base + 16 * mt >= M) break;
      float z[8][4];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) z[t][e] = acc[mt][t][e];
      epilogue_rows<4>(z, ec, lane, m, col0, row_base + 16 * mt, M, scratch);
      wave_lds_sync();
    }
  }
}

// ------------------------------------------------------------ dispatch tables

typedef void (*LinearFn)(const LinearArgs);

// rows: row blocks of the launch (several: the normal policy on the 16- and
// 32-row forms' word loads)
template <int BITS, bool CHAINED>
constexpr LinearFn pick_kernel(int kernel, int rows) {
  return kernel == kChain16   ? (rows > 1 ? linear_chain_kernel<BITS, 1, CHAINED, 4, 8, kStreamAgain>
                                          : linear_chain_kernel<BITS, 1, CHAINED, 4>)
       : kernel == kChain32   ? (rows > 1 ? linear_chain_kernel<BITS, 2, CHAINED, 4, 8, kStreamAgain>
                                          : linear_chain_kernel<BITS, 2, CHAINED, 4>)
       : kernel == kNtile64   ? linear_ntile_kernel<BITS, 4, CHAINED>
                              : linear_tile_kernel<BITS, CHAINED>;
}

template <int BITS>
LinearFn pick_linear(int kernel, bool chained, int rows) {
  if (kernel == kSpread16) return rows > 1 ? linear_spread_rows_kernel<BITS> : linear_spread_kernel<BITS>;
  if (kernel == kChain16x8)
    return rows > 1 ? linear_chain_kernel<BITS, 1, true, 8, 8, kStreamAgain> : linear_chain_kernel<BITS, 1, true, 8>;
  if (kernel == kChain16H)
    return rows > 1 ? linear_chain_kernel<BITS, 1, false, 8, 4, kStreamAgain> : linear_chain_kernel<BITS, 1, false, 8, 4>;
  if (kernel == kWide128) return linear_wide_kernel<BITS>;
  if (kernel == kBlock128) return chained ? linear_block_kernel<BITS, true> : linear_block_kernel<BITS, false>;
  if (kernel == kBlock64) return linear_block64_kernel<BITS>;
  if (kernel == kBlock32) return linear_block32_kernel<BITS>;
  if (kernel == kTile64) return linear_tile64_kernel<BITS>;
  if (kernel == kQuad128) return linear_quad_kernel<BITS>;
  return chained ? pick_kernel<BITS, true>(kernel, rows) : pick_kernel<BITS, false>(kernel, rows);
}

// The kernel pick_linear returns, named as the compiler names that template
// instantiation (kStreamOnce = 2, kStreamAgain = 0): the dispatch registry of
// the tests and the compiler's resource records use these names. Kept beside
// pick_linear so that the two change together.
inline void linear_form_name(char *buf, size_t n, int bits, int kernel, bool chained, int rows) {
  const int pol = rows > 1 ? kStreamAgain : kStreamOnce;
  const char *ch = chained ? "true" : "false";
  switch (kernel) {
    case kSpread16:
      snprintf(buf, n, rows > 1 ? "linear_spread_rows_kernel<%d>" : "linear_spread_kernel<%d>", bits);
      return;
    case kChain16x8: snprintf(buf, n, "linear_chain_kernel<%d, 1, true, 8, 8, %d>", bits, pol); return;
    case kChain16H: snprintf(buf, n, "linear_chain_kernel<%d, 1, false, 8, 4, %d>", bits, pol); return;
    case kWide128: snprintf(buf, n, "linear_wide_kernel<%d>", bits); return;
    case kBlock128: snprintf(buf, n, "linear_block_kernel<%d, %s>", bits, ch); return;
    case kBlock64: snprintf(buf, n, "linear_block64_kernel<%d>", bits); return;
    case kBlock32: snprintf(buf, n, "linear_block32_kernel<%d>", bits); return;
    case kTile64: snprintf(buf, n, "linear_tile64_kernel<%d>", bits); return;
    case kQuad128: snprintf(buf, n, "linear_quad_kernel<%d>", bits); return;
    case kChain16: snprintf(buf, n, "linear_chain_kernel<%d, 1, %s, 4, 8, %d>", bits, ch, pol); return;
    case kChain32: snprintf(buf, n, "linear_chain_kernel<%d, 2, %s, 4, 8, %d>", bits, ch, pol); return;
    case kNtile64: snprintf(buf, n, "linear_ntile_kernel<%d, 4, %s>", bits, ch); return;
    default: snprintf(buf, n, "linear_tile_kernel<%d, %s>", bits, ch); return;
  }
}

// Launch of the linear kernel `kernel` at BITS bits per weight.
template <int BITS>
int launch_linear_t(const LinearArgs &a, int kernel, bool chained, void *stream) {
  const LinearFn fn = pick_linear<BITS>(kernel, chained, a.row_blocks);
  (void)hipGetLastError();   // report this launch's error, not an earlier one
  hipLaunchKernelGGL(fn, dim3((unsigned)a.total_wgs), dim3(threads_per_wg(kernel)), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace
}  // namespace exl3
