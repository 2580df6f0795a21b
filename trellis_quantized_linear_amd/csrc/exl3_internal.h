// Internal interface between the host library (exl3_api.cpp) and the HIP
// kernels (exl3_kernels.hip). Not installed; the public ABI is include/exl3.h.
#pragma once

#include <stdint.h>
#include <stddef.h>

namespace exl3 {

constexpr int kWaves = 4;                 // waves per workgroup, every plan
constexpr int kThreads = kWaves * 64;
constexpr int kMaxMembers = 3;
constexpr int kBlockCols = 128;
constexpr int kChunk = 32;                // K depth of one MFMA (16x16x32 f16)

// One member of a linear launch (a weight, a view or a group member).
struct MemberArgs {
  const uint8_t *words;       // first byte of this member's first block
  const uint16_t *scales;     // fp16[N]
  const uint16_t *svh;        // fp16[N]
  const uint16_t *xr;         // rotated input, fp16, slot order: [M][K], or [K/32][M][32] (chunk-major)
                              // for the spread launch and the 128-row tilings (LinearArgs::xr_chunk_major)
  const uint16_t *suh;        // fp16[K] input signs (read when the rotation is fused)
  uint16_t *y;                // bf16 [M][ldy]
  float *partials;            // [S][M][N] fp32, or null when chained
  uint32_t *counters;         // [row_blocks][n_blocks], or null when chained
  int64_t block_stride;       // bytes
  int64_t ldy;                // elements
  int32_t N;
  int32_t n_blocks;
  int32_t splits;             // S of the plan
  int32_t groups;             // workgroups per (row block, column block); 1 when chained
  int32_t wg_begin;           // first workgroup of this member in the grid (spread launch:
                              // the member's first block among the launch's blocks)
};

struct LinearArgs {
  MemberArgs m[kMaxMembers];
  int32_t n_members;
  int32_t M;
  int32_t K;
  int32_t chunks;             // K / 32
  int32_t row_blocks;         // ceil(M / (16 * m_tiles))
  int32_t total_wgs;
  int32_t own_blocks;         // spread launch: blocks owned by one workgroup each (= total_wgs)
  int32_t left_blocks;        // spread launch: blocks whose splits go to spare waves
  int32_t xr_chunk_major;     // 128-row tilings: Xr is chunk-major (else row-major)
  int32_t fold_launch;        // 128-row exchanged tiles: store the split partials only; a split-fold
                              // launch adds them and finishes the rows
  int32_t fold_tiles;         // split-fold launch: 16-row tiles per row block of the partials (8 or 4)
  // Fused input rotation (decode and 32-row launches): the launch itself
  // writes every member's Xr from x before its chains read it. sync[0]
  // counts finished workgroups; sync[1 + j * K/128 + k] says that member j's
  // 128-column chunk k of Xr is written. All of them are zero at rest: the
  // last workgroup to finish clears them.
  const uint16_t *x;          // bf16 [M][ldx], or null: Xr was written by a rotation launch
  int64_t ldx;
  uint32_t *sync;
  int32_t spin_limit;         // polls of an unwritten chunk's flag before a wave rotates it itself
};

// Workgroups (one wave each) of the split-fold launch: one per (member, row
// block, block, 16-row tile, group of 4 rows); fold_tiles 16-row tiles per
// row block (8 for 128-row partials, 4 for 64-row ones).
inline int64_t split_fold_wgs(const LinearArgs &a) {
  int64_t n = 0;
  for (int j = 0; j < a.n_members; ++j) n += (int64_t)a.row_blocks * a.m[j].n_blocks * a.fold_tiles * 4;
  return n;
}

// Words of the sync region of a fused launch.
inline int64_t fused_sync_words(int n_members, int64_t K) { return 1 + (int64_t)n_members * (K / 128); }
// Largest sync region a fused launch uses (flags of one workgroup's clear pass).
constexpr int64_t kMaxFusedFlags = 1024;

// Rotation launches of at least this many (4 rows, 128-chunk) items per
// member read X once for all members (a thousand rows at K = 5120).
constexpr int64_t kRotSharedItems = 10240;
// Rotation launches of at most this many pieces run one wave per workgroup.
constexpr int64_t kRotOneWaveItems = 4096;

struct RotArgs {
  const uint16_t *x;          // bf16 [M][ldx]
  const uint16_t *suh[kMaxMembers];
  uint16_t *xr[kMaxMembers];  // fp16 [M][K]
  int64_t ldx;
  int32_t M;
  int32_t K;
  int32_t n_members;
  int32_t natural_order;      // 1: natural K order (test hook), 0: MFMA slot order
  int32_t chunk_major;        // 1: Xr element (row, k) at ((k / 32) * M + row) * 32 + k % 32
                              // (the layout the spread launch reads), 0: row * K + k
  int32_t shared_x;           // 1: a wave per (4 rows, 128-chunk) rotates X for every member;
                              // 0: a wave per (member, 4 rows, 128-chunk)
};

struct DequantArgs {
  const uint8_t *words;
  uint16_t *out;              // fp16 [K][N]
  int64_t block_stride;
  int32_t K;
  int32_t N;
};

// Linear kernels.
enum LinearKernel {
  kChain16 = 0,     // 16 rows, 4 waves per workgroup, one split per wave
  kChain16x8 = 1,   // 16 rows, 8 waves per workgroup, all splits of a block (chained only)
  kChain32 = 2,     // 32 rows, 4 waves per workgroup, one split per wave
  kNtile64 = 3,     // 64 rows per workgroup, waves own column tiles
  kTile128 = 4,     // 128 rows per workgroup, 2 x 2 waves of 64 x 64
  kSpread16 = 5,    // 16 rows, 16 waves: one own block per workgroup + spare waves on left blocks
  kWide128 = 6,     // 128 rows x 2 blocks per workgroup, 4 waves of 128 x 64 (chained only)
  kBlock128 = 7,    // 128 rows x 1 block per workgroup, 4 waves of 128 x 32
  kQuad128 = 8,     // opt-in single-chain prompt tiles: 128 rows x 4 blocks, 4 waves of 128 x 128
  kChain16H = 9,    // 16 rows, 8 waves, exchanged: two waves per split, 4 column tiles each
  kBlock64 = 10,    // 64 rows x 1 block per workgroup, 4 waves of 64 x 32 (chained, one row block)
  kTile64 = 11,     // 64 rows per workgroup, 2 waves of 64 x 64 (exchanged, with the split-fold launch)
  kBlock32 = 12,    // 32 rows x 1 block per workgroup, 4 waves of 32 x 32 (chained, one row block)
};

inline int waves_per_wg(int kernel) {
  return kernel == kSpread16 ? 16 : (kernel == kChain16x8 || kernel == kChain16H) ? 8 : kernel == kTile64 ? 2 : kWaves;
}
inline int threads_per_wg(int kernel) { return 64 * waves_per_wg(kernel); }

// Arrivals per (row block, column block) of a launch: one when every split of
// a block runs in one workgroup; else ceil(S / W) workgroups for the 16- and
// 32-row tilings (one split per wave, W waves; two waves per split in the
// column-halves form) and S for the 64- and 128-row tilings (one split per
// workgroup).
inline int groups_per_block(int splits, int kernel, bool chained) {
  if (chained) return 1;
  if (kernel == kChain16H) return (splits + 3) / 4;
  return kernel <= kChain32 ? (splits + waves_per_wg(kernel) - 1) / waves_per_wg(kernel) : splits;
}

// Static scratch of exl3_linear_group_static: 64 MiB per device, the first
// 256 KiB of it the counter region.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;     // EXL3_STATIC_SCRATCH_BYTES
constexpr size_t kStaticCounterBytes = size_t(256) << 10;    // EXL3_STATIC_COUNTER_BYTES
constexpr int kMaxDevices = 64;

// The static scratch's device address on device `dev` (the current device):
// resolved with hipGetSymbolAddress on the first call for that device, which
// also zeroes its counter region on `stream`; cached afterwards. Returns a
// hipError_t as int.
int static_scratch(int dev, void *stream, void **ptr);

// The template instantiation a linear launch of this form runs, as the
// compiler names it (e.g. "linear_spread_kernel<4>").
void form_name(char *buf, size_t n, int bits, int kernel, bool chained, int rows);

// Launchers (exl3_kernels.hip). Each returns a hipError_t as int.
int launch_linear(const LinearArgs &a, int bits, int kernel, bool chained, void *stream);
// The linear launch at BITS bits per weight (exl3_linear_bits.hip, one
// translation unit per width).
template <int BITS>
int launch_linear_bits(const LinearArgs &a, int kernel, bool chained, void *stream);
int launch_rot(const RotArgs &a, void *stream);
// The split-fold launch after a linear launch with fold_launch set.
int launch_split_fold(const LinearArgs &a, void *stream);
int launch_dequant(const DequantArgs &a, int bits, void *stream);
int launch_codebook(const uint16_t *states, uint16_t *out, int64_t n, void *stream);
int launch_fill_zero(void *ptr, size_t bytes, void *stream);

}  // namespace exl3
