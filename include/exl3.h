/*
 * exl3.h — C ABI of the EXL3 trellis-quantized linear on MI355X (gfx950).
 *
 *     Y = rot_out( dequant_trellis(W) . rot_in(X) )
 *
 * The operation is the EXL3 linear that the TensorFold pull requests about
 * serving EXL3 checkpoints describe: per 128-column block, decode K-bit
 * trellis codes of 16x16 tiles into fp16 weights, rotate the input by a sign
 * flip and a 128-point Hadamard, contract in fp32, reduce over K splits with
 * per-block counters that the last arriving workgroup resets, rotate the
 * output, for any row count with the same bits per row, for groups of up to
 * three same-K weights in one launch, and for column views of whole blocks.
 *
 * Conventions for every call:
 *   - Device pointers are plain addresses of device memory owned by the
 *     caller (for instance torch tensors' data_ptr()). The library never
 *     takes ownership, never frees, and keeps no pointer after returning.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every launch goes to that stream; no call synchronises the device.
 *   - Return value: EXL3_OK (0) or a negative EXL3_E* code. Errors are
 *     detected on the host before anything is launched, except EXL3_EHIP,
 *     which reports a failed HIP launch (exl3_last_hip_error() gives the HIP
 *     code). No C++ exception crosses this boundary.
 *   - Size: M * K * 2 < 2^31 per call (the rotated input of one member, fp16,
 *     stays under 2 GiB: the kernels address it with 32-bit offsets).
 *   - Arithmetic is fixed: the rotated input is fp16, weights are fp16, K
 *     sums are fp32 in one canonical order, outputs are bf16. Row m of Y is
 *     byte-identical for every row count M, every row regime, group
 *     membership and column view (TensorFold PR #1467, "The arithmetic";
 *     PR #1407, review item 1: a row gives the same bytes in a prompt call as
 *     in a decode call).
 *
 * Formats (all little-endian):
 *   packed words  block-major: the 16x16 tile at column block nb, tile row kt,
 *                 column tile t (0..7) starts at byte
 *                     nb*block_stride + (kt*8 + t)*32*bits.
 *                 A tile is a 256*bits-bit stream (bit j = bit j%8 of byte
 *                 j/8); weight i of the tile (K row i%16, column i/16) is the
 *                 codebook value of the 16-bit window at bits [i*bits,
 *                 i*bits+16), wrapping inside the tile. A dense weight has
 *                 block_stride = 16*K*bits bytes.
 *   codebook      cb(s) = ((40503*s + 31161) mod 2^16 AND 0x8FFF) OR 0x3000,
 *                 an fp16 bit pattern.
 *   X             bf16 [M][ldx], row-major, K used columns.
 *   scales, svh   fp16 [N] (per column of this weight or view).
 *   suh           fp16 [K].
 *   Y             bf16 [M][ldy], row-major, N written columns.
 */
#ifndef EXL3_H
#define EXL3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define EXL3_OK          0
#define EXL3_EINVAL     (-1)  /* null pointer, negative M, ldx < K, ldy < N, n_cols < 0,
                                 M * K * 2 >= 2^31 (one member's rotated input past 2 GiB) */
#define EXL3_EALIGN     (-2)  /* K or N not a multiple of 128, view not whole blocks,
                                 misaligned pointer (words and workspace: 4 bytes;
                                 fp16/bf16 arrays: 2 bytes), block_stride too small */
#define EXL3_ERANGE     (-3)  /* column view outside its parent */
#define EXL3_EBITS      (-4)  /* bits outside 2..8 */
#define EXL3_EWORKSPACE (-5)  /* workspace missing or too small for this call */
#define EXL3_EGROUP     (-6)  /* group of 0 or more than 3 members, or members
                                 that differ in K or bits */
#define EXL3_EHIP       (-7)  /* a HIP launch or call failed */
#define EXL3_ESCRATCH   (-8)  /* exl3_linear_group_static: the call needs more than
                                 the library's static scratch */

/* A quantized weight, or a column view of one. Plain descriptor of borrowed
 * device pointers: copying it copies no data. */
typedef struct exl3_weight {
  const void *words;     /* device: packed trellis words (layout above) */
  const void *scales;    /* device: fp16[N], per column, applied before rot_out */
  const void *suh;       /* device: fp16[K], input sign vector */
  const void *svh;       /* device: fp16[N], output sign vector */
  int64_t K;             /* input features, multiple of 128 */
  int64_t N;             /* output columns of this weight or view, multiple of 128 */
  int64_t block_stride;  /* bytes between consecutive 128-column blocks
                            (>= 16*K*bits; a view keeps its parent's) */
  int32_t bits;          /* bits per weight, 2..8 */
  int32_t flags;         /* reserved, must be 0 */
} exl3_weight_t;

/* A K-split plan. */
typedef struct exl3_plan {
  int32_t splits;        /* S: K sums are S chains added in split order */
  int32_t waves;         /* waves (64 lanes) per workgroup, fixed for all plans */
  int64_t chunks;        /* K / 32, MFMA depth steps */
  int64_t n_blocks;      /* N / 128 */
} exl3_plan_t;

/* Caller-owned device workspace. The first counter_bytes bytes hold the
 * split-K counters (uint32); they are zero whenever no call is running. The
 * rest holds the rotated input and split partials of one call at a time. */
typedef struct exl3_workspace {
  void *ptr;             /* device memory, 256-byte aligned */
  size_t bytes;          /* total size */
  size_t counter_bytes;  /* size of the counter region at the start (multiple of 256) */
} exl3_workspace_t;

/* exl3_plan — the K-split plan of a K x N weight at `bits` bits.
 * It depends on (K, N, bits) only, never on the row count, and every N of at
 * least EXL3_WIDE_BLOCKS blocks plans alike, so a column view that wide plans
 * as its whole parent does (TensorFold PR #1507, review and follow-up: a view
 * of at least 64 blocks takes the full head's plan; wide_blocks = 64).
 * Errors: EINVAL (out == NULL), EALIGN (K or N not a multiple of 128 or
 * zero), EBITS. */
#define EXL3_WIDE_BLOCKS 64
int exl3_plan(int64_t K, int64_t N, int32_t bits, exl3_plan_t *out);

/* exl3_weight_columns — a view of columns [col_from, col_from + n_cols) of
 * `parent`, made of whole 128-column blocks: its descriptor carries the
 * parent's block stride and points at the view's first block (PR #1507,
 * "What this changes").
 * It copies nothing and lives no longer than the parent's buffers.
 * Errors: EINVAL (NULL pointers, n_cols <= 0), EALIGN (col_from or n_cols
 * not a multiple of 128), ERANGE (outside the parent), and the parent's own
 * descriptor errors. */
int exl3_weight_columns(const exl3_weight_t *parent, int64_t col_from, int64_t n_cols,
                        exl3_weight_t *view);

/* exl3_workspace_need — bytes of workspace (and of its counter region) that
 * one call of exl3_linear_group with these members at M rows needs. The
 * counter region holds the split counters and, for calls of up to 32 rows,
 * the rotated-input chunk flags; all are zero between calls. Sizing a
 * workspace for the largest M it will see covers every smaller M under the
 * automatic launch choice (a launch forced through exl3_test_force may need
 * more: size under the same hooks).
 * Errors: as exl3_linear_group's argument checks. */
int exl3_workspace_need(int32_t n_members, const exl3_weight_t *const *w, int64_t M,
                        size_t *bytes, size_t *counter_bytes);

/* exl3_workspace_grow — adopt a new (larger) caller-allocated buffer and zero
 * its counter region once, on `stream`, with a fill kernel (so nothing is
 * allocated or memset inside a later linear call: PR #1475, "What this
 * changes": counters are zeroed on the call's stream only when they grow).
 * A buffer no larger than the current one is refused with EWORKSPACE and
 * nothing is launched. The old buffer may be freed by the caller once the
 * stream has passed all calls that used it.
 * Errors: EINVAL, EALIGN (ptr not 256-byte aligned), EWORKSPACE, EHIP. */
int exl3_workspace_grow(exl3_workspace_t *ws, void *ptr, size_t bytes, size_t counter_bytes,
                        void *stream);

/* exl3_workspace_reset — zero the counter region again on `stream` (only
 * needed after a launch failed and left counters in an unknown state). */
int exl3_workspace_reset(const exl3_workspace_t *ws, void *stream);

/* exl3_linear — Y[M x N] = rot_out(dequant(W) . rot_in(X)) for one weight or
 * view: the per-weight EXL3 linear of any row count (PR #1467, "What this
 * changes" and "The arithmetic": decode rows and 17-128-row forms with one
 * set of bits), its split-K partials met through counters that the last
 * arriving workgroup resets (PR #1475, "What this changes"). M == 0 returns
 * EXL3_OK and launches nothing. Two launches on `stream`: the input rotation,
 * then the linear (decode + MFMA + split-K exchange + epilogue); see
 * exl3_test_fuse_rotation for the one-launch form at up to 32 rows. Never allocates, memsets or synchronises, so it may be
 * captured in a HIP graph. Calls that run concurrently (other streams) must
 * use different workspaces.
 * Errors: EINVAL, EALIGN, EBITS, EWORKSPACE, EHIP. */
int exl3_linear(const exl3_weight_t *w, const void *x, int64_t ldx, int64_t M,
                void *y, int64_t ldy, const exl3_workspace_t *ws, void *stream);

/* exl3_linear_group — up to three members of one K and one bits over the same
 * X in one rotation launch and one linear launch (PR #1467, "What this
 * changes"). Each member keeps its own plan, suh, scales and svh, and
 * its output y[j] (ldy[j]) is byte-identical to exl3_linear of that member
 * alone. Errors: as exl3_linear, plus EGROUP. */
int exl3_linear_group(int32_t n_members, const exl3_weight_t *const *w, const void *x,
                      int64_t ldx, int64_t M, void *const *y, const int64_t *ldy,
                      const exl3_workspace_t *ws, void *stream);

/* exl3_rotate / exl3_linear_rotated — the two launches of exl3_linear_group,
 * callable one at a time (the pages keep the rotation, rot_in / rot_group,
 * and the linear as separate launches: PR #1467, "What this changes").
 * exl3_rotate writes the members' rotated inputs into the workspace;
 * exl3_linear_rotated then runs the linear on what the workspace holds. The
 * second call must name the same members and M as the exl3_rotate before it
 * on the same workspace (and stream); otherwise its output is meaningless
 * (it still stays inside the workspace and y). Together they produce exactly
 * the bytes of exl3_linear_group. Errors: as exl3_linear_group. */
int exl3_rotate(int32_t n_members, const exl3_weight_t *const *w, const void *x, int64_t ldx, int64_t M,
                const exl3_workspace_t *ws, void *stream);
int exl3_linear_rotated(int32_t n_members, const exl3_weight_t *const *w, int64_t M, void *const *y,
                        const int64_t *ldy, const exl3_workspace_t *ws, void *stream);

/* exl3_linear_group_static — exl3_linear_group without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Its
 * counters, rotated inputs and split partials live in a static scratch array
 * of the library: EXL3_STATIC_SCRATCH_BYTES per device (the first
 * EXL3_STATIC_COUNTER_BYTES of it the split counters), held by every device
 * the library runs on until the process ends. The first call on a device
 * resolves that device's copy of the array and zeroes its counter region on
 * `stream` (a fill kernel, no memset); afterwards each call leaves the
 * counters at zero, as exl3_linear_group does. The call allocates, frees and
 * synchronises nothing; it launches the same kernels as exl3_linear_group
 * and gives the same bytes. Every call on a device shares that device's
 * scratch: calls that overlap on one GPU (other streams, other threads) race
 * and must be ordered by the caller. A call that needs more scratch than the
 * array holds (for example prompt rows: M * K * 2 bytes of rotated input per
 * member) returns EXL3_ESCRATCH before anything is launched.
 * Errors: as exl3_linear_group, with ESCRATCH in place of EWORKSPACE. */
#define EXL3_STATIC_SCRATCH_BYTES (64u << 20)
#define EXL3_STATIC_COUNTER_BYTES (256u << 10)
int exl3_linear_group_static(int32_t n_members, const exl3_weight_t *const *w, const void *x,
                             int64_t ldx, int64_t M, void *const *y, const int64_t *ldy, void *stream);

/* exl3_strerror — static text for an error code. */
const char *exl3_strerror(int code);

/* exl3_last_hip_error — the HIP error code behind the last EXL3_EHIP of the
 * calling thread (0 if none). */
int exl3_last_hip_error(void);

/* ---- test hooks: not for production use; process-global, not thread-safe ---- */

/* exl3_test_dequant — the decoded, unscaled fp16 weights [K][N] (row-major,
 * natural K order) of `w`, written by the same device decode routine the
 * linear uses. Errors: descriptor errors, EINVAL (out NULL), EHIP. */
int exl3_test_dequant(const exl3_weight_t *w, void *out_fp16, void *stream);

/* exl3_test_codebook — out[i] = cb(states[i]) through the device codebook
 * routine; n may be odd. Errors: EINVAL, EHIP. */
int exl3_test_codebook(const void *states_u16, void *out_fp16, int64_t n, void *stream);

/* exl3_test_rot_in — the rotated input Xr [M][K] fp16 (natural K order) that
 * the input rotation of `w` produces; xr_fp16 must be 16-byte aligned.
 * Errors: as exl3_linear (EALIGN also for a misaligned xr_fp16), EHIP. */
int exl3_test_rot_in(const exl3_weight_t *w, const void *x, int64_t ldx, int64_t M,
                     void *xr_fp16, void *stream);

/* exl3_set_prompt_arithmetic — opt-in arithmetic for calls above 128 rows
 * (the pages' rejected 64-row prompt tiles, TensorFold PR #1475, kept here
 * as an explicit choice):
 *   mode 0 (default): every row count, group and view gives the same bits;
 *   mode 1: above 128 rows each output is one MFMA chain over all of K (no
 *           K splits), on 128 x 512 tiles — faster, but its bits differ from
 *           the other regimes' (still within the oracle tolerance). Calls of
 *           up to 128 rows are unaffected.
 * Process-global, not thread-safe; EXL3_EINVAL for another mode. */
int exl3_set_prompt_arithmetic(int32_t mode);

/* exl3_test_fuse_rotation — on = 1: exl3_linear and exl3_linear_group calls
 * of up to 32 rows (the 16- and 32-row launches of one row block) run as ONE
 * launch: its first workgroups write the rotated input into the workspace
 * and flag each 128-column chunk, and every chain waits for the flags of the
 * chunks it reads before reading them (the launch-gap removal the pages get
 * from programmatic dependent launch, PR #1467, "What this changes"; every
 * dependent read waits, as its merge review asks). on = 0 (default): a
 * rotation launch of its own; on MI355X the in-launch wait costs more than
 * the launch it removes. spin_limit: polls a wave makes of an unwritten
 * chunk's flag before it rotates that chunk itself (-1: the default, 1024; 0
 * makes every wave that finds a chunk unwritten rotate it itself, which
 * exercises that path). Neither setting changes bits. Errors: EINVAL. */
int exl3_test_fuse_rotation(int32_t on, int32_t spin_limit);

/* exl3_test_force — force the row tiling and launch shape (the analogue of
 * the pages' Linear.min_rows override, PR #1467 follow-up). Neither changes
 * the bits of a row:
 *   m_tiles: -1 automatic, else 1, 2, 4 or 8 16-row MFMA tiles per workgroup,
 *            or 16: 128-row tiles two 128-column blocks wide (chained
 *            launches only, else as 8; above 128 rows the automatic choice
 *            is 8, the 128-row block tiling);
 *   chained: -1 automatic, 0 one K split per workgroup with counter exchange,
 *            1 every split of a block in one workgroup, summed in order,
 *            2 the spread launch (16-row tiles, one S <= 15 for every
 *            member; otherwise as 1): a 16-wave workgroup per (16-row block,
 *            owned block), its spare waves taking splits of the remaining
 *            blocks (the automatic choice at up to 32 rows where the block
 *            counts fit, e.g. the {gate, up} pair; up to 48 rows where the
 *            128-row block tiling cannot give its blocks past one per CU
 *            to the workgroups as single splits),
 *            3 as 0, with each split on two waves of 4 column tiles (16-row
 *            tiles; the automatic choice when 16-row exchanged launches have
 *            at most one split chain per SIMD).
 * `splits` (0 = the plan's) overrides S and DOES change bits: it is the
 * planted control "another K split". */
int exl3_test_force(int32_t m_tiles, int32_t chained, int32_t splits);

/* exl3_test_last_form — the kernel form of the last linear launch the
 * library issued (or recorded, in mock mode), named as the compiler names
 * its template instantiation, e.g. "linear_spread_kernel<4>", followed by
 * " +rot" when the input rotation ran inside it; empty before any launch.
 * The pages' dispatch test and kernel contract are keyed by these forms
 * (PR #1467, author follow-up: "A dispatch test"). Errors: EINVAL (buf NULL
 * or n < 2). */
int exl3_test_last_form(char *buf, int64_t n);

/* exl3_test_mock — with on != 0, every later device operation (kernel launch,
 * counter fill) is recorded instead of issued, so host logic can be tested
 * without a GPU; exl3_test_mock_counts reads and clears the record. */
int exl3_test_mock(int32_t on);
int exl3_test_mock_counts(int64_t *launches, int64_t *fills, int64_t *fill_bytes,
                          void **last_stream);

#ifdef __cplusplus
}
#endif

#endif /* EXL3_H */
