// HIP kernels of the EXL3 trellis-quantized linear for gfx950 (MI355X), other
// than the linear kernels themselves (exl3_device.h, exl3_linear_bits.hip):
//
//   rot_kernel      Xr = fp16(FWHT128(X * suh) * 2^-4) for up to three members,
//                   X read once
//   dequant_kernel  test hook: the decoded weights, through the same decoder
//   codebook_kernel test hook: the codebook on arbitrary states
//   fill_zero       zeroes a grown counter region on the caller's stream
//   split_fold      adds the split partials of a 128-row exchanged launch
//                   and finishes its rows
//
// and the launchers, including the dispatch of a linear launch to its bit
// width's translation unit, and the static scratch of
// exl3_linear_group_static.
#include <hip/hip_runtime.h>

#include <mutex>

#include "exl3_device.h"

// Scratch of exl3_linear_group_static, for callers that cannot allocate: the
// split counters (zero at rest) in its first kStaticCounterBytes, then the
// rotated inputs and split partials of one call. Each device holds its own
// copy for the life of the process. Host code never uses this name as an
// address (it is a host-side stand-in there): the device address comes from
// hipGetSymbolAddress, per device, in static_scratch().
static __device__ __align__(256) unsigned char scratch[exl3::kStaticScratchBytes];

namespace exl3 {
namespace {

__global__ __launch_bounds__(kThreads) void rot_kernel(const RotArgs a) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int64_t item = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int kc = a.K >> 7;
  const int quads = (a.M + 3) >> 2;
  const int64_t per_member = (int64_t)quads * kc;
  // shared_x: item = (quad, chunk) and every member; else item = (member,
  // quad, chunk)
  const int n_items = a.shared_x ? 1 : a.n_members;
  if (item >= per_member * n_items) return;
  const int j0 = a.shared_x ? 0 : (int)(item / per_member);
  const int j1 = a.shared_x ? a.n_members : j0 + 1;
  const int64_t rem = item - (int64_t)j0 * per_member;
  const int quad = (int)(rem / kc);
  const int chunk = (int)(rem - (int64_t)quad * kc);
  const int row = 4 * quad + g;
  if (row >= a.M) return;                                // no cross-lane step below mixes rows
  const int k0 = chunk * 128 + 8 * c;
  const int64_t at = a.chunk_major ? ((int64_t)(k0 >> 5) * a.M + row) * 32 + (k0 & 31) : (int64_t)row * a.K + k0;
  const u32x4 xw = load8_u16(a.x + (int64_t)row * a.ldx + k0);
  for (int j = j0; j < j1; ++j) {                        // uniform; each member as if alone
    const uint16_t *suh = j == 0 ? a.suh[0] : (j == 1 ? a.suh[1] : a.suh[2]);
    uint16_t *xr = j == 0 ? a.xr[0] : (j == 1 ? a.xr[1] : a.xr[2]);
    *(u32x4 *)(xr + at) = rot_lane(xw, load8_u16(suh + k0), c, a.natural_order != 0);
  }
}

// ------------------------------------------------------------ split fold
//
// After a 128- or 64-row exchanged launch that only stored its split
// partials (LinearArgs::fold_launch; fold_tiles 16-row tiles per row block),
// and for the left blocks of the chained block tiling: one wave per
// (member, row block, block, 16-row tile, group of 4 rows) adds those rows'
// S partials in split order, z = P0, then z + P1,
// ... (the same fp32 additions, in the same order, as a linear launch's
// last arriving workgroup would make), and runs the epilogue of its 4
// rows. A 16-row tile is 512 fragments of 4 rows x 1 column, 8 KB per split
// in the fragment layout; the 128 fragments of rows 4q .. 4q + 3 are
// fragments t * 64 + 16 q + c (column tile t, column c); lane l loads
// column c = l % 16 of column tiles l / 16 and l / 16 + 4, every split's
// loads before the first addition. One-wave workgroups spread the loads
// over the CUs (the down projection's 320 tiles are 1280 waves).
__global__ __launch_bounds__(64) void split_fold_kernel(const LinearArgs a) {
  constexpr int kMaxSplits = 16;
  const int RB = a.row_blocks;
  int64_t local = blockIdx.x;
  int j = 0;
  const int TPB = a.fold_tiles;                            // 16-row tiles per row block
  while (j + 1 < a.n_members && local >= (int64_t)RB * a.m[j].n_blocks * TPB * 4) {
    local -= (int64_t)RB * a.m[j].n_blocks * TPB * 4;
    ++j;
  }
  const MemberArgs &m = a.m[j];
  const int per_rb = m.n_blocks * TPB * 4;
  const int rb = (int)(local / per_rb);
  const int rem = (int)(local - (int64_t)rb * per_rb);
  const int nb = rem / (TPB * 4), mt = (rem >> 2) % TPB, q = rem & 3;
  const int row0 = 16 * TPB * rb + 16 * mt + 4 * q;
  if (row0 >= a.M) return;                                 // uniform
  const int S = m.splits;
  const int lane = threadIdx.x;
  const int c = lane & 15, t0 = lane >> 4;
  const int col0 = nb * kBlockCols;

  u32x4 v[kMaxSplits][2];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s < S) {                                           // uniform
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(partial_frag(m, s, rb, nb, RB, TPB) + mt * 8 * 256, 8 * 1024);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        v[s][e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                rp, 16 * ((t0 + 4 * e) * 64 + 16 * q + c), 0, kAgentScope));
    }
  }
  f32x4 z[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) z[e] = __builtin_bit_cast(f32x4, v[0][e]);
#pragma unroll
  for (int s = 1; s < kMaxSplits; ++s)
    if (s < S)
#pragma unroll
      for (int e = 0; e < 2; ++e) z[e] = z[e] + __builtin_bit_cast(f32x4, v[s][e]);

  __shared__ __attribute__((aligned(16))) float zrow[4 * 132];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) zrow[r * 132 + 16 * (t0 + 4 * e) + c] = z[e][r];
  const EpiCols ec = epi_cols(m, col0, lane);
  __syncthreads();
  epilogue_rows_lds<1>(zrow, 132, ec, lane, m, col0, row0, a.M);
}

// ------------------------------------------------------------ test hooks

template <int BITS>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const DequantArgs a) {
  using T = BitsTraits<BITS>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int C = a.K / kChunk;
  const int nb = blockIdx.x / C;
  const int chunk = blockIdx.x - nb * C;
  const __amdgpu_buffer_rsrc_t rbuf = make_rsrc(a.words + (int64_t)nb * a.block_stride, (uint32_t)(16u * a.K * BITS));
  const BLane<BITS> bl = b_lane<BITS>(lane);
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t w[T::kDwords];
#pragma unroll
    for (int d = 0; d < T::kDwords; ++d)
      w[d] = __builtin_amdgcn_raw_buffer_load_b32(rbuf, (int)(bl.voff[d] + (2 * wave + i) * T::kTileBytes),
                                                  chunk * 512 * BITS, 0);
    const u32x4 v = __builtin_bit_cast(u32x4, decode8<BITS>(w, bl.shift, cb_const()));
    const int kbase = 16 * (2 * chunk + (g >> 1)) + 8 * (g & 1);
    const int n = nb * kBlockCols + 16 * (2 * wave + i) + c;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a.out[(int64_t)(kbase + r) * a.N + n] = (uint16_t)(v[r] & 0xFFFFu);
      a.out[(int64_t)(kbase + r + 4) * a.N + n] = (uint16_t)(v[r] >> 16);
    }
  }
}

__global__ void codebook_kernel(const uint16_t *states, uint16_t *out, int64_t n) {
  const int64_t pair = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i0 = 2 * pair;
  if (i0 >= n) return;
  const uint32_t s0 = states[i0];
  const uint32_t s1 = (i0 + 1 < n) ? states[i0 + 1] : 0u;
  const uint32_t w = codebook2(s0 | (s1 << 16), cb_const());
  out[i0] = (uint16_t)(w & 0xFFFFu);
  if (i0 + 1 < n) out[i0 + 1] = (uint16_t)(w >> 16);
}

__global__ void fill_zero_kernel(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

int launch_linear(const LinearArgs &a, int bits, int kernel, bool chained, void *stream) {
  if (kernel < kChain16 || kernel > kBlock32 ||
      ((kernel == kChain16x8 || kernel == kSpread16 || kernel == kWide128 || kernel == kQuad128 ||
        kernel == kBlock64 || kernel == kBlock32) && !chained) ||
      ((kernel == kChain16H || kernel == kTile64) && chained))
    return (int)hipErrorInvalidValue;
  switch (bits) {
    case 2: return launch_linear_bits<2>(a, kernel, chained, stream);
    case 3: return launch_linear_bits<3>(a, kernel, chained, stream);
    case 4: return launch_linear_bits<4>(a, kernel, chained, stream);
    case 5: return launch_linear_bits<5>(a, kernel, chained, stream);
    case 6: return launch_linear_bits<6>(a, kernel, chained, stream);
    case 7: return launch_linear_bits<7>(a, kernel, chained, stream);
    case 8: return launch_linear_bits<8>(a, kernel, chained, stream);
    default: return (int)hipErrorInvalidValue;
  }
}


void form_name(char *buf, size_t n, int bits, int kernel, bool chained, int rows) {
  linear_form_name(buf, n, bits, kernel, chained, rows);
}

int launch_rot(const RotArgs &a_in, void *stream) {
  // Prompt rows: X read once for all members (a layer's {q, k, v} at 8192
  // rows 504 -> 336 MB, the 8192-row layer 5.33-5.34 -> 5.29 ms). A few
  // rows: a wave per member, whose rotation launch waits on one X load per
  // wave either way (the decode step 45.1-45.9 us with it, 46.4-46.9 us
  // with X shared).
  RotArgs a = a_in;
  const int64_t per_member = (int64_t)((a.M + 3) / 4) * (a.K / 128);
  a.shared_x = a.n_members > 1 && per_member >= kRotSharedItems ? 1 : 0;
  const int64_t items = per_member * (a.shared_x ? 1 : a.n_members);
  // One-wave workgroups up to kRotOneWaveItems pieces (the decode step at 16
  // / 1 rows 43.4-43.6 -> 43.2-43.3 / 38.8-39.6 -> 38.2 us), 4-wave ones for
  // prompt rows.
  const int wpw = items <= kRotOneWaveItems ? 1 : kWaves;
  const int64_t wgs = (items + wpw - 1) / wpw;
  (void)hipGetLastError();
  hipLaunchKernelGGL(rot_kernel, dim3((unsigned)wgs), dim3(64 * wpw), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_split_fold(const LinearArgs &a, void *stream) {
  if (a.fold_tiles != 4 && a.fold_tiles != 8) return (int)hipErrorInvalidValue;
  const int64_t wgs = split_fold_wgs(a);
  for (int j = 0; j < a.n_members; ++j)
    if (a.m[j].splits < 1 || a.m[j].splits > 16) return (int)hipErrorInvalidValue;
  if (wgs <= 0 || wgs >= (int64_t(1) << 31)) return (int)hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(split_fold_kernel, dim3((unsigned)wgs), dim3(64), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_dequant(const DequantArgs &a, int bits, void *stream) {
  const unsigned wgs = (unsigned)((a.N / kBlockCols) * (a.K / kChunk));
  const dim3 grid(wgs), block(kThreads);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  switch (bits) {
    case 2: hipLaunchKernelGGL(dequant_kernel<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(dequant_kernel<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(dequant_kernel<4>, grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL(dequant_kernel<5>, grid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL(dequant_kernel<6>, grid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL(dequant_kernel<7>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(dequant_kernel<8>, grid, block, 0, s, a); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

int launch_codebook(const uint16_t *states, uint16_t *out, int64_t n, void *stream) {
  const int64_t pairs = (n + 1) / 2;
  const unsigned wgs = (unsigned)((pairs + 255) / 256);
  (void)hipGetLastError();
  hipLaunchKernelGGL(codebook_kernel, dim3(wgs), dim3(256), 0, (hipStream_t)stream, states, out, n);
  return (int)hipGetLastError();
}

int static_scratch(int dev, void *stream, void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr || ((uintptr_t)p & 255) != 0) return (int)hipErrorInvalidSymbol;
    // the counters must start at zero; afterwards every call's last arrivers
    // leave them at zero
    const int f = launch_fill_zero(p, kStaticCounterBytes, stream);
    if (f != 0) return f;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int launch_fill_zero(void *ptr, size_t bytes, void *stream) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return 0;
  int64_t wgs = (n + 255) / 256;
  if (wgs > 4096) wgs = 4096;
  (void)hipGetLastError();
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)wgs), dim3(256), 0, (hipStream_t)stream, (uint32_t *)ptr, n);
  return (int)hipGetLastError();
}

}  // namespace exl3
