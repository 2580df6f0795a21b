// Host side of the EXL3 linear: argument checks, the K-split plan, column
// views, workspace layout and growth, regime choice and launches. The C ABI
// is declared in include/exl3.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>

#include "exl3.h"
#include "exl3_internal.h"

namespace {

using exl3::kBlockCols;
using exl3::kChunk;
using exl3::kMaxMembers;

thread_local int g_last_hip = 0;

// Test hooks (process-global; documented as not thread-safe).
struct TestHooks {
  int m_tiles = -1;
  int chained = -1;
  int splits = 0;
  bool mock = false;
  int64_t launches = 0;
  int64_t fills = 0;
  int64_t fill_bytes = 0;
  void *last_stream = nullptr;
  // the last linear launch's form (mock or real): bits, kernel, chained,
  // row blocks, rotation inside the launch
  int form_bits = 0, form_kernel = -1, form_rows = 0;
  bool form_chained = false, form_fused = false;
};
TestHooks g_hooks;

// Input rotation inside the linear launch at up to 32 rows (1: where the
// launch allows it, 0: always a rotation launch of its own; 0 by default, as
// the in-launch dependency costs more than the launch it removes on MI355X),
// and the polls a wave spends on an unwritten chunk of Xr before it rotates
// the chunk itself.
int g_fuse_rotation = 0;
constexpr int kDefaultSpinLimit = 1024;
int g_spin_limit = kDefaultSpinLimit;

// Prompt arithmetic above 128 rows: 0 bit-stable (every regime the same
// bits), 1 single-chain tiles (opt-in, faster, other bits). Process-global.
int g_prompt_mode = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int hip_fail(int err) {
  g_last_hip = err;
  return EXL3_EHIP;
}

int check_weight(const exl3_weight_t *w) {
  if (!w || !w->words || !w->scales || !w->suh || !w->svh) return EXL3_EINVAL;
  if (w->flags != 0) return EXL3_EINVAL;
  if (w->bits < 2 || w->bits > 8) return EXL3_EBITS;
  if (w->K <= 0 || w->N <= 0 || w->K % 128 != 0 || w->N % 128 != 0) return EXL3_EALIGN;
  // keep every in-kernel byte offset of a block inside 32 bits
  if (w->K > (int64_t(1) << 24) || w->N / kBlockCols > (int64_t(1) << 30)) return EXL3_EINVAL;
  if (w->block_stride < 16 * w->K * w->bits || w->block_stride % 4 != 0) return EXL3_EALIGN;
  if ((uintptr_t)w->words % 4 != 0) return EXL3_EALIGN;
  if ((uintptr_t)w->scales % 2 != 0 || (uintptr_t)w->suh % 2 != 0 || (uintptr_t)w->svh % 2 != 0)
    return EXL3_EALIGN;
  return EXL3_OK;
}

// The plan table. S depends on (K, N, bits) only, measured on MI355X at 1
// and 16 rows (one K split per wave, 256 CUs):
//  * a weight of at least EXL3_WIDE_BLOCKS blocks takes S_wide(K) = 15 when
//    that keeps at least 4 chunks (128 K) per split, else as many splits as
//    keep 4 chunks each; every such view plans alike. 15 chains fill 15 of a
//    16-wave workgroup, and the 16th wave of every workgroup takes a split of
//    the blocks that exceed one block per CU (the spread launch): a group of
//    272 blocks on 256 CUs then runs 16 waves on every CU;
//  * a narrower weight takes the smallest power of two with n_blocks * S >=
//    512 (about two splits per SIMD), at most 16 and keeping at least 4
//    chunks per split.
int32_t splits_for(int64_t K, int64_t N, int32_t bits) {
  (void)bits;
  const int64_t chunks = K / kChunk;
  const int64_t nb = N / kBlockCols;
  int32_t s = 1;
  if (nb >= EXL3_WIDE_BLOCKS) return (int32_t)std::max<int64_t>(1, std::min<int64_t>(15, chunks / 4));
  while (nb * s < 512 && s < 16 && chunks / (2 * s) >= 4) s *= 2;
  return s;
}

struct MemberPlan {
  const exl3_weight_t *w;
  int32_t splits;
  int32_t n_blocks;
};

struct Launch {
  int m_tiles;
  int kernel;               // exl3::LinearKernel
  bool chained;             // no exchange between workgroups (the spread launch exchanges left blocks only)
  bool exchange;            // partials and counters in the workspace
  int64_t row_blocks;
  int64_t own_blocks = 0;   // spread launch
  int64_t left_blocks = 0;  // spread launch
  bool can_fuse = false;    // the kernel can rotate the input itself (one row block of at most 32 rows)
  bool fold_launch = false; // 128-row exchanged tiles: the split partials are added by a launch of their own
  bool block_left = false;  // chained 128-row blocks, one row block: own_blocks workgroups, left blocks' splits
                            // one per workgroup after its own block, added by the split-fold launch
};

// CUs of the current device (256 on MI355X; 256 when no device answers).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Decode rows (up to 16): at or above this many blocks, one 8-wave workgroup
// per block (chained splits, two workgroups per CU) keeps every CU busy for
// several rounds without partials.
constexpr int64_t kChainedMinBlocks16 = 512;

// Above 16 rows the spread launch (where its block counts fit) runs one
// 16-row block after another in one grid, each as at 16 rows, up to this many
// rows (3-bit {gate, up}: 17-32 rows 57 us against 66 us for the chained
// 16-row form, 33-48 rows 82-84 against 85-91; at 49-64 rows 108 against 87
// for the 128-row block tiling).
constexpr int64_t kSpreadMaxRows = 48;

// Weights whose blocks exceed the CUs by a few (the 3-bit {gate, up} pair:
// 272 blocks on 256 CUs) leave the spread launch above this many rows for the
// chained block tiling with its left blocks (at 33, 40 and 48 rows 70-74 us
// on 128-row workgroups, split-fold launch included, against 73-79 us over
// three 16-row blocks; 64-row workgroups since, below); the same bits
// either way. At 17-32 rows the spread launch stays faster than the 32-row
// block tiling with left blocks (the MLP 88-89 against 90-93 us).
constexpr int64_t kSpreadMaxRowsLeft = 32;

// The chained 128-row block tiling can give the blocks past one per CU to
// the workgroups as single splits: one plan of at most 16 splits for every
// member, and no more left splits than CUs.
bool block_left_fits(const MemberPlan *mp, int n, int64_t blocks, int64_t ncu) {
  for (int j = 1; j < n; ++j)
    if (mp[j].splits != mp[0].splits) return false;
  return mp[0].splits <= 16 && blocks > ncu && (blocks - ncu) * mp[0].splits <= ncu;
}

// Mid-M rows (17..128) with the automatic tiling: the row tiling and
// whether the splits of a block fold inside one workgroup (chained) or
// exchange through the workspace, chosen from measurements on MI355X of the
// 27B's weights (gate/up at 3 bits, q/k/v, down, a 5120 x 8192 weight and
// the 6-bit head at 17..128 rows; every choice gives the same bits). The
// 8-wave chained 16-row form over ceil(M / 16) row blocks is the fastest
// wherever its workgroups fill the chip without too many rounds; the 64-row
// tiling never was.
struct MidChoice {
  int m_tiles;
  bool chained;
};

MidChoice mid_m_choice(int64_t blocks, bool long_chains, int64_t M) {
  const int64_t w16 = blocks * ((M + 15) / 16);            // workgroups of the chained 16-row form
  if (blocks >= 128) return w16 <= 1024 ? MidChoice{1, true} : MidChoice{8, true};
  if (!long_chains) return M <= 32 ? MidChoice{1, false} : MidChoice{1, true};
  // few blocks, long splits (down): the exchange keeps the CUs busy; from
  // 33 rows on the exchanged 2 x 2 tiles with the split-fold launch (down at
  // 49, 64, 80 and 96 rows 41-44 us against 45-53 us for the chained 16-row
  // form; in 64-row tiles, the MLP at 33 / 48 rows 99-103 -> 93-97 us
  // against the exchanged 16-row form over three row blocks; at 17-32 rows
  // the 32-row exchanged form stays, 0.5-3 us faster)
  if (M <= 32) return {2, false};
  return {8, false};
}

Launch choose_launch(const MemberPlan *mp, int n, int64_t M) {
  Launch L;
  bool all_single = true;
  int64_t blocks = 0;
  bool long_chains = false;
  for (int j = 0; j < n; ++j) {
    all_single = all_single && mp[j].splits == 1;
    blocks += mp[j].n_blocks;
    long_chains = long_chains || (mp[j].w->K / kChunk) > 16 * mp[j].splits;
  }
  // one plan S <= 15 for every member: the spread launch is possible
  int32_t s_uniform = mp[0].splits;
  for (int j = 1; j < n; ++j)
    if (mp[j].splits != s_uniform) s_uniform = 0;
  if (s_uniform > 15) s_uniform = 0;
  const int64_t ncu = cu_count();
  // the spread launch's blocks per 16-row block: one own block per CU and
  // left blocks that the spare waves can take, or 3/4 to 1 block per CU
  int64_t sp_own = 0, sp_left = 0;
  if (!all_single && s_uniform > 0 && blocks < kChainedMinBlocks16) {
    if (blocks > ncu && (blocks - ncu) * s_uniform <= ncu * (16 - s_uniform)) {
      sp_own = ncu;
      sp_left = blocks - ncu;
    } else if (4 * blocks >= 3 * ncu && blocks <= ncu) {
      sp_own = blocks;
    }
  }
  int mt = g_hooks.m_tiles;
  // 16: 128-row tiles two blocks wide. Automatic above 128 rows for long
  // splits (down): at the steady clock of a long prompt (these launches run
  // power-limited) the 8192-row down projection took 1260 us against 1333
  // on the block tiling (two workgroups of 128 rows x one block per CU),
  // which stays for the rest ({gate, up} 2913 against 2944 us, {q, k, v}
  // 711 against 709); the same bits either way.
  const bool wide = mt == 16 || (mt == -1 && M > 128 && long_chains);
  int mid_chained = -1;
  bool mid_spread = false;
  const bool left_fits = block_left_fits(mp, n, blocks, ncu);
  if (mt == 16) {
    mt = 8;
  } else if (mt == -1 && M > kSpreadMaxRowsLeft && M <= 128 && left_fits && !all_single) {
    mt = 8;
    mid_chained = 1;
  } else if (mt == -1 && M > 16 && M <= kSpreadMaxRows && sp_own > 0) {
    mt = 1;
    mid_spread = true;
  } else if (mt == -1 && M > 16 && M <= 128) {
    const MidChoice mc = mid_m_choice(blocks, long_chains, M);
    mt = mc.m_tiles;
    mid_chained = mc.chained ? 1 : 0;
  } else if (mt != 1 && mt != 2 && mt != 4 && mt != 8) {
    mt = M <= 16 ? 1 : 8;
  }
  L.m_tiles = mt;
  L.row_blocks = (M + 16 * mt - 1) / (16 * mt);
  L.exchange = false;
  bool spread = false;
  if (g_hooks.chained >= 0 && g_hooks.chained <= 3) {
    L.chained = g_hooks.chained == 1 || g_hooks.chained == 2;
    if (g_hooks.chained == 2 && mt == 1 && s_uniform > 0) {
      // forced: as many left blocks as the spare waves can take
      spread = true;
      L.left_blocks = blocks * (16 - s_uniform) / 16;
      L.own_blocks = blocks - L.left_blocks;
    }
  } else if (mid_spread) {
    L.chained = spread = true;
    L.own_blocks = sp_own;
    L.left_blocks = sp_left;
  } else if (mid_chained >= 0) {
    L.chained = mid_chained == 1 || all_single;
  } else if (mt == 1) {
    if (all_single || blocks >= kChainedMinBlocks16) {
      L.chained = true;
    } else if (L.row_blocks == 1 && sp_own > 0) {
      L.chained = spread = true;
      L.own_blocks = sp_own;
      L.left_blocks = sp_left;
    } else {
      L.chained = false;
    }
  } else {
    // Partials and counters only when the grid would otherwise be too small
    // to stream HBM: an exchange costs a few microseconds of serialized
    // memory round trips per block (stores, counter, the last arriver's
    // loads), which pays off below about one workgroup per CU. Prompt row
    // blocks and wide weights give enough workgroups by themselves.
    L.chained = all_single || M > 128 || L.row_blocks * blocks >= 256;
  }
  // 128-row tiles: the block tiling (4 waves of 128 x 32, operands copied
  // into an LDS ring), except exchanged splits of more than 16 chunks, which
  // run faster on the 2 x 2 tiling
  const bool quad = g_prompt_mode == 1 && M > 128 && g_hooks.m_tiles == -1 && g_hooks.chained != 0;
  // 16-row exchanged launches of at most one split chain per SIMD run each
  // chain on two waves (4 column tiles each): a lone wave per SIMD leaves
  // the decode's latency exposed
  int64_t chains = 0;
  for (int j = 0; j < n; ++j) chains += L.row_blocks * mp[j].n_blocks * mp[j].splits;
  const bool halves = mt == 1 && !L.chained &&
                      (g_hooks.chained == 3 || (g_hooks.chained == -1 && chains <= 4 * ncu));
  L.kernel = quad      ? exl3::kQuad128
           : spread    ? exl3::kSpread16
           : mt == 1 ? (L.chained ? exl3::kChain16x8 : halves ? exl3::kChain16H : exl3::kChain16)
           : mt == 2 ? exl3::kChain32
           : mt == 4 ? exl3::kNtile64
           : wide && L.chained ? exl3::kWide128
           : !L.chained && long_chains ? exl3::kTile128
                     : exl3::kBlock128;
  // Automatic chained 128-row block tiles of at most 64 rows run 64-row
  // workgroups: half the MFMAs, the same bits (3-bit {gate, up} pair: MLP at
  // 33-64 rows 112-129 -> 98-116 us; 6-bit head at 49 / 64 rows 406-411 /
  // 384-394 -> 358-361 / 328-345 us); of at most 32 rows 32-row workgroups
  // (the 6-bit head at 17 / 24 / 32 rows 329-336 / 301 / 290-294 ->
  // 297-303 / 275-278 / 263-269 us)
  if (L.kernel == exl3::kBlock128 && L.chained && M <= 64 && g_hooks.m_tiles == -1) {
    L.kernel = M <= 32 ? exl3::kBlock32 : exl3::kBlock64;
    L.m_tiles = M <= 32 ? 2 : 4;
  }
  L.exchange = !L.chained || (spread && L.left_blocks > 0);
  // The 2 x 2 tiling's exchange adds 64 KB partials: its last arriving
  // workgroup would make one memory round trip per split for the whole
  // block (the down projection at 128 rows: about 22 of its 71 us), while a
  // launch of 16-row tiles spreads the same additions over the chip. Plans
  // of up to 16 splits (every automatic plan).
  int32_t max_splits = 0;
  for (int j = 0; j < n; ++j) max_splits = std::max(max_splits, mp[j].splits);
  L.fold_launch = L.kernel == exl3::kTile128 && !L.chained && max_splits <= 16;
  // ... in 64-row tiles of 2 waves: the down projection's 640 128-row tiles
  // left 128 CUs with three workgroups and 128 with two (the launch 34 us,
  // its 2-workgroup CUs done at 26 us); 64-row tiles are 2.5 or 5 per CU,
  // and at up to 64 rows no wave computes masked rows
  if (L.fold_launch && g_hooks.m_tiles == -1) {
    L.kernel = exl3::kTile64;
    L.m_tiles = 4;
    L.row_blocks = (M + 63) / 64;
  }
  // The chained 128-row block tiling over one row block with a few more
  // blocks than CUs ({gate, up} at 33-128 rows: 272 blocks on 256 CUs): the
  // blocks past one per CU would run as second workgroups on a few CUs and
  // set the launch time; instead each CU's workgroup runs one split of one
  // of them after its own block, and the split-fold launch adds those
  // partials.
  if ((L.kernel == exl3::kBlock128 || L.kernel == exl3::kBlock64 || L.kernel == exl3::kBlock32) && L.chained &&
      L.row_blocks == 1 && left_fits) {
    L.block_left = true;
    L.own_blocks = ncu;
    L.left_blocks = blocks - ncu;
  }
  L.can_fuse = L.row_blocks == 1 &&
               (L.kernel == exl3::kSpread16 || L.kernel == exl3::kChain16 || L.kernel == exl3::kChain16H ||
                L.kernel == exl3::kChain32) &&
               exl3::fused_sync_words(n, mp[0].w->K) - 1 <= exl3::kMaxFusedFlags;
  return L;
}

struct Layout {
  size_t counters;          // uint32 words of the counter region used: split counters, then the sync words
  size_t sync_at;           // first sync word of a fused launch
  size_t xr_bytes[kMaxMembers];
  size_t part_bytes[kMaxMembers];
  size_t rest;              // bytes after the counter region
};

Layout layout_for(const MemberPlan *mp, int n, int64_t M, int64_t K, const Launch &L) {
  Layout lay{};
  int64_t first_block = 0;   // the member's first block among the launch's blocks
  for (int j = 0; j < n; ++j) {
    lay.xr_bytes[j] = align_up((size_t)M * K * 2);
    if (L.exchange && L.kernel == exl3::kSpread16) {
      // the spread launch: partials of the left blocks only, all members'
      // in member 0's buffer ([split][row block][left block][16 x 128])
      if (j == 0) lay.part_bytes[0] = align_up((size_t)mp[0].splits * L.row_blocks * L.left_blocks * 16 * 128 * 4);
      lay.counters += (size_t)L.row_blocks * mp[j].n_blocks;
    } else if (L.exchange) {
      // rows padded to whole row blocks (the fragment layout of the 16- and
      // 32-row tilings stores whole 16-row tiles)
      lay.part_bytes[j] = align_up((size_t)mp[j].splits * (L.row_blocks * 16 * L.m_tiles) * mp[j].w->N * 4);
      lay.counters += (size_t)L.row_blocks * mp[j].n_blocks;
    } else if (L.block_left) {
      // the member's left blocks (those past own_blocks): [split][left block] x 128 x 128 floats
      const int64_t left = std::max<int64_t>(0, std::min<int64_t>(mp[j].n_blocks, first_block + mp[j].n_blocks - L.own_blocks));
      lay.part_bytes[j] = align_up((size_t)mp[j].splits * left * 128 * 128 * 4);
    }
    first_block += mp[j].n_blocks;
    lay.rest += lay.xr_bytes[j] + lay.part_bytes[j];
  }
  lay.sync_at = lay.counters;
  if (L.can_fuse) lay.counters += (size_t)exl3::fused_sync_words(n, K);
  return lay;
}

int check_group(int32_t n, const exl3_weight_t *const *w, int64_t M, MemberPlan *mp) {
  if (n < 1 || n > kMaxMembers || !w) return EXL3_EGROUP;
  if (M < 0) return EXL3_EINVAL;
  for (int j = 0; j < n; ++j) {
    const int e = check_weight(w[j]);
    if (e != EXL3_OK) return e;
    if (j > 0 && (w[j]->K != w[0]->K || w[j]->bits != w[0]->bits)) return EXL3_EGROUP;
    mp[j].w = w[j];
    mp[j].splits = g_hooks.splits > 0 ? g_hooks.splits : splits_for(w[j]->K, w[j]->N, w[j]->bits);
    mp[j].n_blocks = (int32_t)(w[j]->N / kBlockCols);
    if (mp[j].splits > w[j]->K / kChunk) return EXL3_EINVAL;
  }
  // rotated input offsets of one member stay inside a 32-bit buffer range
  if (M > 0 && (uint64_t)M * w[0]->K * 2 >= (uint64_t(1) << 31)) return EXL3_EINVAL;
  return EXL3_OK;
}

// Sizes of one call at M rows: the counter region and what follows it.
void call_need(const MemberPlan *mp, int n, int64_t M, size_t *rest, size_t *counter_bytes) {
  const Launch L = choose_launch(mp, n, M);
  const Layout lay = layout_for(mp, n, M, mp[0].w->K, L);
  *counter_bytes = std::max(*counter_bytes, align_up(lay.counters * 4));
  *rest = std::max(*rest, lay.rest);
}

int issue_fill(void *ptr, size_t bytes, void *stream) {
  if (g_hooks.mock) {
    g_hooks.fills += 1;
    g_hooks.fill_bytes += (int64_t)bytes;
    g_hooks.last_stream = stream;
    return EXL3_OK;
  }
  const int e = exl3::launch_fill_zero(ptr, bytes, stream);
  return e ? hip_fail(e) : EXL3_OK;
}

}  // namespace

extern "C" {

int exl3_plan(int64_t K, int64_t N, int32_t bits, exl3_plan_t *out) {
  if (!out) return EXL3_EINVAL;
  if (bits < 2 || bits > 8) return EXL3_EBITS;
  if (K <= 0 || N <= 0 || K % 128 != 0 || N % 128 != 0) return EXL3_EALIGN;
  out->splits = splits_for(K, N, bits);
  out->waves = exl3::kWaves;
  out->chunks = K / kChunk;
  out->n_blocks = N / kBlockCols;
  return EXL3_OK;
}

int exl3_weight_columns(const exl3_weight_t *parent, int64_t col_from, int64_t n_cols, exl3_weight_t *view) {
  if (!parent || !view) return EXL3_EINVAL;
  const int e = check_weight(parent);
  if (e != EXL3_OK) return e;
  if (n_cols <= 0 || col_from < 0) return EXL3_EINVAL;
  if (col_from % kBlockCols != 0 || n_cols % kBlockCols != 0) return EXL3_EALIGN;
  if (col_from + n_cols > parent->N) return EXL3_ERANGE;
  exl3_weight_t v = *parent;
  v.words = (const uint8_t *)parent->words + (col_from / kBlockCols) * parent->block_stride;
  v.scales = (const uint16_t *)parent->scales + col_from;
  v.svh = (const uint16_t *)parent->svh + col_from;
  v.N = n_cols;
  *view = v;
  return EXL3_OK;
}

int exl3_workspace_need(int32_t n_members, const exl3_weight_t *const *w, int64_t M, size_t *bytes,
                        size_t *counter_bytes) {
  if (!bytes || !counter_bytes) return EXL3_EINVAL;
  MemberPlan mp[kMaxMembers];
  const int e = check_group(n_members, w, M, mp);
  if (e != EXL3_OK) return e;
  size_t rest = 0, cb = 0;
  // sizes grow with M while the launch form stays the same; the row counts
  // where the automatic choice changes form (16, 32, 48, 64, 96 and 128
  // rows; the 16- and 32-row forms also hold the rotation flags) and M
  // itself bound every smaller call. The counter region sits at a fixed
  // offset, so the largest counter need and the largest rest add up.
  const int64_t bounds[7] = {16, 32, 48, 64, 96, 128, M};
  int64_t probes[7];
  for (int i = 0; i < 7; ++i) probes[i] = std::min<int64_t>(M, bounds[i]);
  for (int64_t p : probes)
    if (p > 0) call_need(mp, n_members, p, &rest, &cb);
  *counter_bytes = cb;
  *bytes = cb + rest;
  return EXL3_OK;
}

int exl3_workspace_grow(exl3_workspace_t *ws, void *ptr, size_t bytes, size_t counter_bytes, void *stream) {
  if (!ws || !ptr) return EXL3_EINVAL;
  if ((uintptr_t)ptr % kAlign != 0 || counter_bytes % kAlign != 0) return EXL3_EALIGN;
  if (counter_bytes > bytes) return EXL3_EWORKSPACE;
  if (bytes <= ws->bytes && counter_bytes <= ws->counter_bytes) return EXL3_EWORKSPACE;
  const int e = issue_fill(ptr, counter_bytes, stream);
  if (e != EXL3_OK) return e;
  ws->ptr = ptr;
  ws->bytes = bytes;
  ws->counter_bytes = counter_bytes;
  return EXL3_OK;
}

int exl3_workspace_reset(const exl3_workspace_t *ws, void *stream) {
  if (!ws || !ws->ptr) return EXL3_EINVAL;
  return issue_fill(ws->ptr, ws->counter_bytes, stream);
}

}  // extern "C"

namespace {

enum Phase { kRotate = 1, kLinear = 2 };

// The whole call: checks, plans, workspace layout, then the rotation launch
// (phase kRotate) and the linear launch (phase kLinear; with the split-fold
// launch after it for 128-row exchanged tiles).
int run_group(int32_t n_members, const exl3_weight_t *const *w, const void *x, int64_t ldx, int64_t M,
              void *const *y, const int64_t *ldy, const exl3_workspace_t *ws, void *stream, int phases,
              bool static_scratch = false) {
  MemberPlan mp[kMaxMembers];
  int e = check_group(n_members, w, M, mp);
  if (e != EXL3_OK) return e;
  if ((phases & kLinear) && (!y || !ldy)) return EXL3_EINVAL;
  if (M == 0) return EXL3_OK;
  const int64_t K = w[0]->K;
  if (phases & kRotate) {
    if (!x || ldx < K) return EXL3_EINVAL;
    if ((uintptr_t)x % 2 != 0) return EXL3_EALIGN;
  }
  if (phases & kLinear) {
    for (int j = 0; j < n_members; ++j) {
      if (!y[j] || ldy[j] < w[j]->N) return EXL3_EINVAL;
      if ((uintptr_t)y[j] % 2 != 0) return EXL3_EALIGN;
    }
  }
  const Launch L = choose_launch(mp, n_members, M);
  const Layout lay = layout_for(mp, n_members, M, K, L);
  exl3_workspace_t sws{};
  if (static_scratch) {
    // the library's own scratch: refuse what it cannot hold, before any GPU call
    if (lay.counters * 4 > exl3::kStaticCounterBytes ||
        exl3::kStaticCounterBytes + lay.rest > exl3::kStaticScratchBytes)
      return EXL3_ESCRATCH;
    void *p = (void *)(uintptr_t)0x100000;           // mock mode: never dereferenced
    if (!g_hooks.mock) {
      int dev = 0;
      hipError_t he = hipGetDevice(&dev);
      if (he != hipSuccess) return hip_fail((int)he);
      const int se = exl3::static_scratch(dev, stream, &p);
      if (se != 0) return hip_fail(se);
    }
    sws = exl3_workspace_t{p, exl3::kStaticScratchBytes, exl3::kStaticCounterBytes};
    ws = &sws;
  }
  if (!ws || !ws->ptr) return EXL3_EWORKSPACE;
  if (lay.counters * 4 > ws->counter_bytes || ws->counter_bytes + lay.rest > ws->bytes) return EXL3_EWORKSPACE;

  exl3::RotArgs ra{};
  exl3::LinearArgs la{};
  uint8_t *base = (uint8_t *)ws->ptr;
  size_t off = ws->counter_bytes;
  size_t counter_off = 0;
  int64_t wg = 0;
  int64_t blocks_before = 0;
  for (int j = 0; j < n_members; ++j) {
    const exl3_weight_t *wj = w[j];
    uint16_t *xr = (uint16_t *)(base + off);
    off += lay.xr_bytes[j];
    ra.suh[j] = (const uint16_t *)wj->suh;
    ra.xr[j] = xr;
    exl3::MemberArgs &m = la.m[j];
    m.words = (const uint8_t *)wj->words;
    m.scales = (const uint16_t *)wj->scales;
    m.svh = (const uint16_t *)wj->svh;
    m.xr = xr;
    m.y = (phases & kLinear) ? (uint16_t *)y[j] : nullptr;
    m.ldy = (phases & kLinear) ? ldy[j] : 0;
    m.block_stride = wj->block_stride;
    m.N = (int32_t)wj->N;
    m.n_blocks = mp[j].n_blocks;
    m.splits = mp[j].splits;
    m.groups = exl3::groups_per_block(mp[j].splits, L.kernel, L.chained);
    m.wg_begin = (int32_t)(L.kernel == exl3::kSpread16 ? blocks_before : wg);
    blocks_before += mp[j].n_blocks;
    if (L.exchange) {
      m.partials = (float *)(base + off);
      off += lay.part_bytes[j];
      m.counters = (uint32_t *)base + counter_off;
      counter_off += (size_t)L.row_blocks * mp[j].n_blocks;
    } else if (L.block_left) {
      m.partials = (float *)(base + off);
      off += lay.part_bytes[j];
    }
    wg += L.kernel == exl3::kWide128   ? L.row_blocks * ((mp[j].n_blocks + 1) / 2)
        : L.kernel == exl3::kQuad128 ? L.row_blocks * ((mp[j].n_blocks + 3) / 4)
                                     : L.row_blocks * mp[j].n_blocks * m.groups;
  }
  if (L.kernel == exl3::kSpread16) wg = L.row_blocks * L.own_blocks;
  if (L.block_left) wg = L.own_blocks;
  if (wg >= (int64_t(1) << 31)) return EXL3_EINVAL;
  la.own_blocks = (int32_t)L.own_blocks;
  la.left_blocks = (int32_t)L.left_blocks;
  ra.x = (const uint16_t *)x;
  ra.ldx = ldx;
  ra.M = (int32_t)M;
  ra.K = (int32_t)K;
  ra.n_members = n_members;
  ra.natural_order = 0;
  // Xr layout. Row-major rows lie 2K bytes apart, so the 128 rows of one
  // chunk that every workgroup of a 128-row tiling loads at about the same
  // time fall on few memory channels; chunk-major puts them in one
  // contiguous 8 KB (the 3-bit {gate, up} pair at 128 rows: 121 -> 100 us).
  // The spread launch reads chunk-major too (its 16 rows as 8 whole lines);
  // the other 16- to 64-row launches measured as fast or faster row-major,
  // but for the column-halves launch below.
  // Chunk offsets are 32-bit: chunk-major needs 2 K M < 2^31, which every
  // accepted call meets (check_group).
  const bool tile_cm = (L.kernel == exl3::kTile128 || L.kernel == exl3::kBlock128 || L.kernel == exl3::kWide128 ||
                        L.kernel == exl3::kQuad128 || L.kernel == exl3::kBlock64 || L.kernel == exl3::kTile64 ||
                        L.kernel == exl3::kBlock32) &&
                       2 * K * M < (int64_t(1) << 31);
  // The 16-row column-halves launch ({q, k, v} at decode rows) reads its
  // 16 rows of a chunk as 8 whole lines instead of 16 half-used ones (the
  // decode step at 16 / 7 / 1 rows 0.1-0.3 us faster, the same bytes).
  const bool halves_cm = L.kernel == exl3::kChain16H && L.row_blocks == 1;
  ra.chunk_major = L.kernel == exl3::kSpread16 || tile_cm || halves_cm ? 1 : 0;
  la.xr_chunk_major = tile_cm || halves_cm ? 1 : 0;
  la.fold_launch = L.fold_launch ? 1 : 0;
  la.fold_tiles = L.kernel == exl3::kTile64 ? 4 : 8;       // partials of 64- or 128-row blocks
  la.n_members = n_members;
  la.M = (int32_t)M;
  la.K = (int32_t)K;
  la.chunks = (int32_t)(K / kChunk);
  la.row_blocks = (int32_t)L.row_blocks;
  la.total_wgs = (int32_t)wg;

  // both phases in one launch: the linear kernel rotates the input itself
  const bool fuse = phases == (kRotate | kLinear) && L.can_fuse && g_fuse_rotation == 1;
  if (fuse) {
    la.x = (const uint16_t *)x;
    la.ldx = ldx;
    la.sync = (uint32_t *)base + lay.sync_at;
    la.spin_limit = g_spin_limit;
    for (int j = 0; j < n_members; ++j) la.m[j].suh = (const uint16_t *)w[j]->suh;
    phases = kLinear;
  }
  if (phases & kLinear) {
    g_hooks.form_bits = w[0]->bits;
    g_hooks.form_kernel = L.kernel;
    g_hooks.form_chained = L.chained;
    g_hooks.form_rows = (int)L.row_blocks;
    g_hooks.form_fused = fuse;
  }
  if (g_hooks.mock) {
    g_hooks.launches += ((phases & kRotate) ? 1 : 0) + ((phases & kLinear) ? (L.fold_launch || L.block_left ? 2 : 1) : 0);
    g_hooks.last_stream = stream;
    return EXL3_OK;
  }
  if (phases & kRotate) {
    e = exl3::launch_rot(ra, stream);
    if (e) return hip_fail(e);
  }
  if (phases & kLinear) {
    e = exl3::launch_linear(la, w[0]->bits, L.kernel, L.chained, stream);
    if (e) return hip_fail(e);
    if (L.fold_launch) {
      e = exl3::launch_split_fold(la, stream);
      if (e) return hip_fail(e);
    }
    if (L.block_left) {
      // the split-fold launch over the left blocks only: each member that
      // has some, its pointers moved to its first left block
      exl3::LinearArgs fa = la;
      int nf = 0;
      int64_t first_block = 0;
      for (int j = 0; j < n_members; ++j) {
        const int64_t fl = std::max<int64_t>(0, L.own_blocks - first_block);
        if (fl < mp[j].n_blocks) {
          exl3::MemberArgs f = la.m[j];
          f.scales += fl * kBlockCols;
          f.svh += fl * kBlockCols;
          f.y += fl * kBlockCols;
          f.n_blocks = (int32_t)(mp[j].n_blocks - fl);
          fa.m[nf++] = f;
        }
        first_block += mp[j].n_blocks;
      }
      fa.n_members = nf;
      e = exl3::launch_split_fold(fa, stream);
      if (e) return hip_fail(e);
    }
  }
  return EXL3_OK;
}

}  // namespace

extern "C" {

int exl3_linear_group(int32_t n_members, const exl3_weight_t *const *w, const void *x, int64_t ldx, int64_t M,
                      void *const *y, const int64_t *ldy, const exl3_workspace_t *ws, void *stream) {
  return run_group(n_members, w, x, ldx, M, y, ldy, ws, stream, kRotate | kLinear);
}

int exl3_rotate(int32_t n_members, const exl3_weight_t *const *w, const void *x, int64_t ldx, int64_t M,
                const exl3_workspace_t *ws, void *stream) {
  return run_group(n_members, w, x, ldx, M, nullptr, nullptr, ws, stream, kRotate);
}

int exl3_linear_rotated(int32_t n_members, const exl3_weight_t *const *w, int64_t M, void *const *y,
                        const int64_t *ldy, const exl3_workspace_t *ws, void *stream) {
  return run_group(n_members, w, nullptr, 0, M, y, ldy, ws, stream, kLinear);
}



int exl3_linear_group_static(int32_t n_members, const exl3_weight_t *const *w, const void *x, int64_t ldx,
                             int64_t M, void *const *y, const int64_t *ldy, void *stream) {
  return run_group(n_members, w, x, ldx, M, y, ldy, nullptr, stream, kRotate | kLinear, true);
}

int exl3_linear(const exl3_weight_t *w, const void *x, int64_t ldx, int64_t M, void *y, int64_t ldy,
                const exl3_workspace_t *ws, void *stream) {
  const exl3_weight_t *ws_[1] = {w};
  void *ys[1] = {y};
  const int64_t ldys[1] = {ldy};
  return exl3_linear_group(1, ws_, x, ldx, M, ys, ldys, ws, stream);
}

const char *exl3_strerror(int code) {
  switch (code) {
    case EXL3_OK: return "ok";
    case EXL3_EINVAL: return "invalid argument (null pointer, negative size or leading dimension too small)";
    case EXL3_EALIGN: return "alignment: K and N must be multiples of 128, views whole 128-column blocks, pointers aligned";
    case EXL3_ERANGE: return "column view outside its parent";
    case EXL3_EBITS: return "bits per weight outside 2..8";
    case EXL3_EWORKSPACE: return "workspace missing or too small for this call";
    case EXL3_EGROUP: return "group must have 1..3 members of one K and one bit width";
    case EXL3_EHIP: return "a HIP launch failed (see exl3_last_hip_error)";
    case EXL3_ESCRATCH: return "the call needs more than the library's static scratch (64 MiB per device)";
    default: return "unknown error";
  }
}

int exl3_last_hip_error(void) { return g_last_hip; }

int exl3_test_dequant(const exl3_weight_t *w, void *out_fp16, void *stream) {
  const int e = check_weight(w);
  if (e != EXL3_OK) return e;
  if (!out_fp16) return EXL3_EINVAL;
  exl3::DequantArgs a{};
  a.words = (const uint8_t *)w->words;
  a.out = (uint16_t *)out_fp16;
  a.block_stride = w->block_stride;
  a.K = (int32_t)w->K;
  a.N = (int32_t)w->N;
  if (g_hooks.mock) { g_hooks.launches += 1; g_hooks.last_stream = stream; return EXL3_OK; }
  const int err = exl3::launch_dequant(a, w->bits, stream);
  return err ? hip_fail(err) : EXL3_OK;
}

int exl3_test_codebook(const void *states_u16, void *out_fp16, int64_t n, void *stream) {
  if (n < 0 || (n > 0 && (!states_u16 || !out_fp16))) return EXL3_EINVAL;
  if (n == 0) return EXL3_OK;
  if (g_hooks.mock) { g_hooks.launches += 1; g_hooks.last_stream = stream; return EXL3_OK; }
  const int err = exl3::launch_codebook((const uint16_t *)states_u16, (uint16_t *)out_fp16, n, stream);
  return err ? hip_fail(err) : EXL3_OK;
}

int exl3_test_rot_in(const exl3_weight_t *w, const void *x, int64_t ldx, int64_t M, void *xr_fp16, void *stream) {
  const int e = check_weight(w);
  if (e != EXL3_OK) return e;
  if (M < 0 || !xr_fp16 || !x || ldx < w->K) return EXL3_EINVAL;
  if ((uintptr_t)xr_fp16 % 16 != 0 || (uintptr_t)x % 2 != 0) return EXL3_EALIGN;
  if (M == 0) return EXL3_OK;
  if ((uint64_t)M * w->K * 2 >= (uint64_t(1) << 31)) return EXL3_EINVAL;
  exl3::RotArgs ra{};
  ra.x = (const uint16_t *)x;
  ra.ldx = ldx;
  ra.M = (int32_t)M;
  ra.K = (int32_t)w->K;
  ra.n_members = 1;
  ra.suh[0] = (const uint16_t *)w->suh;
  ra.xr[0] = (uint16_t *)xr_fp16;
  ra.natural_order = 1;
  ra.chunk_major = 0;
  if (g_hooks.mock) { g_hooks.launches += 1; g_hooks.last_stream = stream; return EXL3_OK; }
  const int err = exl3::launch_rot(ra, stream);
  return err ? hip_fail(err) : EXL3_OK;
}

int exl3_set_prompt_arithmetic(int32_t mode) {
  if (mode != 0 && mode != 1) return EXL3_EINVAL;
  g_prompt_mode = mode;
  return EXL3_OK;
}

int exl3_test_fuse_rotation(int32_t on, int32_t spin_limit) {
  if ((on != 0 && on != 1) || spin_limit < -1) return EXL3_EINVAL;
  g_fuse_rotation = on;
  g_spin_limit = spin_limit == -1 ? kDefaultSpinLimit : spin_limit;
  return EXL3_OK;
}

int exl3_test_force(int32_t m_tiles, int32_t chained, int32_t splits) {
  if (!(m_tiles == -1 || m_tiles == 1 || m_tiles == 2 || m_tiles == 4 || m_tiles == 8 || m_tiles == 16))
    return EXL3_EINVAL;
  if (chained < -1 || chained > 3 || splits < 0) return EXL3_EINVAL;
  g_hooks.m_tiles = m_tiles;
  g_hooks.chained = chained;
  g_hooks.splits = splits;
  return EXL3_OK;
}

int exl3_test_last_form(char *buf, int64_t n) {
  if (!buf || n < 2) return EXL3_EINVAL;
  if (g_hooks.form_kernel < 0) {
    buf[0] = 0;
    return EXL3_OK;
  }
  exl3::form_name(buf, (size_t)n, g_hooks.form_bits, g_hooks.form_kernel, g_hooks.form_chained, g_hooks.form_rows);
  if (g_hooks.form_fused) {
    const size_t len = strlen(buf);
    snprintf(buf + len, (size_t)n - len, " +rot");
  }
  return EXL3_OK;
}

int exl3_test_mock(int32_t on) {
  g_hooks.mock = on != 0;
  return EXL3_OK;
}

int exl3_test_mock_counts(int64_t *launches, int64_t *fills, int64_t *fill_bytes, void **last_stream) {
  if (launches) *launches = g_hooks.launches;
  if (fills) *fills = g_hooks.fills;
  if (fill_bytes) *fill_bytes = g_hooks.fill_bytes;
  if (last_stream) *last_stream = g_hooks.last_stream;
  g_hooks.launches = g_hooks.fills = g_hooks.fill_bytes = 0;
  g_hooks.last_stream = nullptr;
  return EXL3_OK;
}

}  // extern "C"
