"""Plain CPU oracle of the EXL3 trellis-quantized linear.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
It shares no code with the HIP library (no headers, tables or helpers); the
two meet only in the seeded input generators, which hold none of the method's
arithmetic.

It computes, in float64 unless a step fixes another precision,

    Y = rot_out( dequant_trellis(W) . rot_in(X) )

one step at a time, in the order the format defines them:

  1. decode: every 16x16 tile is a tail-biting bitstream of 256*b bits; weight
     i reads the 16-bit window starting at bit i*b (wrapping inside the tile)
     and a fixed codebook maps that 16-bit state to an fp16 weight;
  2. rot_in: X (bf16) times the input sign vector suh, then an unnormalised
     128-point Sylvester Hadamard per 128-chunk of K, times 2^-4, rounded to
     fp16 (round to nearest even);
  3. Z = Xr . W (float64 here; the GPU accumulates in fp32);
  4. Z times the per-column fp16 scale;
  5. per 128-column block: the same Hadamard, times 2^-3, times the output
     sign vector svh, rounded to bf16 (round to nearest even).

Sources.  The pages (TensorFold pull requests #1407, #1467, #1475 and #1507,
all about serving EXL3 checkpoints) name the format and its contract but
print neither the codebook nor the bit layout.  What they do fix, and where:

  * decoded weights are fp16 and K sums are fp32; a constant weight times
    rotated inputs of 4096 overflows fp16 sums but not fp32 ones
    (PR #1467, author follow-up on the kernel contract, gate 4);
  * the stress fill of the kernel contract: with unit scales, a stream of
    all set bits yields a single weight value whatever the width, whereas the
    alternating pattern 0xaaaa yields two values in turn at widths 3 and 5,
    since odd widths start their windows on odd bit positions (PR #1467,
    author follow-up, gate 4, after the width-matrix review);
  * per-column scales and a per-member input sign vector suh (PR #1467, gates
    and planted controls that swap one group member's scales or its suh);
  * a column view spans whole 128-column blocks and addresses them with the
    strides of the weight it is cut from (PR #1507, "What this changes");
  * planted NaN and both infinities reach the outputs (PR #1467, gate 1).

Everything else (16-bit state width, LSB-first bit order, the column-major
walk of a tile, the block-major layout, the codebook constants, where the
scale is applied, the Hadamard normalisation by 2^-4 and 2^-3, fp16 rotated
inputs and bf16 outputs) is the build's written reading of the format; each
function below states the reading it follows.
"""

from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# IEEE 754 binary16 / bfloat16 conversions, written from the format
# definitions (sign, biased exponent, fraction; round to nearest, ties to
# even).  They are pinned against numpy's float16 and torch's bfloat16 in the
# tests, and used for every rounding the oracle does.
# --------------------------------------------------------------------------


def fp16_to_f64(bits) -> np.ndarray:
    """binary16 bit patterns -> float64 values (exact)."""
    h = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((h >> 15) & 1, -1.0, 1.0)
    e = (h >> 10) & 0x1F
    f = h & 0x3FF
    mag = np.where(e == 0, np.ldexp(f.astype(np.float64), -24),
                   np.ldexp((1024 + f).astype(np.float64), (e - 25).astype(np.int64)))
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 values (exact)."""
    h = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((h >> 15) & 1, -1.0, 1.0)
    e = (h >> 7) & 0xFF
    f = h & 0x7F
    mag = np.where(e == 0, np.ldexp(f.astype(np.float64), -133),
                   np.ldexp((128 + f).astype(np.float64), (e - 134).astype(np.int64)))
    mag = np.where(e == 255, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def _round_to_format(x, frac_bits: int, emin: int, inf_bits: int, nan_bits: int) -> np.ndarray:
    """float64 -> bit pattern of a binary format with `frac_bits` fraction bits
    and smallest normal exponent `emin`, rounding to nearest, ties to even.

    With le = max(floor(log2|x|), emin) the rounding quantum is 2^(le-frac_bits)
    and r = rint(|x| / quantum) is the significand in quantum units.  The
    encoding is ((le - emin + 1) << frac_bits) + r - 2^frac_bits for normals,
    which equals ((le - emin) << frac_bits) + r and also covers subnormals
    (le == emin, r < 2^frac_bits) and a carry out of the fraction (r reaching
    2^(frac_bits+1) bumps the exponent field by one).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    finite = np.isfinite(a)
    a_safe = np.where(finite & (a > 0), a, 1.0)
    _, e2 = np.frexp(a_safe)                 # a = m * 2^e2, 0.5 <= m < 1
    lead = e2.astype(np.int64) - 1           # floor(log2 a)
    le = np.maximum(lead, emin)
    r = np.rint(np.ldexp(a_safe, (frac_bits - le).astype(np.int64)))   # ties to even
    enc = ((le - emin) << frac_bits) + r.astype(np.int64)
    enc = np.where(a == 0, 0, enc)
    enc = np.where(enc >= inf_bits, inf_bits, enc)        # overflow -> infinity
    enc = np.where(np.isinf(a), inf_bits, enc)
    enc = np.where(np.isnan(a), nan_bits, enc)
    sign = np.signbit(x) & ~np.isnan(x)
    enc = enc | np.where(sign, 0x8000, 0)
    return enc.astype(np.uint16)


def f64_to_fp16(x) -> np.ndarray:
    """float64 -> binary16 bits, round to nearest even (NaN -> 0x7E00)."""
    return _round_to_format(x, frac_bits=10, emin=-14, inf_bits=0x7C00, nan_bits=0x7E00)


def f64_to_bf16(x) -> np.ndarray:
    """float64 -> bfloat16 bits, round to nearest even (NaN -> 0x7FC0)."""
    return _round_to_format(x, frac_bits=7, emin=-126, inf_bits=0x7F80, nan_bits=0x7FC0)


# --------------------------------------------------------------------------
# Step 1: trellis decode.
# --------------------------------------------------------------------------

TILE = 16                 # tiles are 16x16 weights
BLOCK_COLS = 128          # a column block is 128 columns = 8 tiles
STATE_BITS = 16           # the decoder state is a 16-bit window of the stream

# Codebook constants.  The pages print no codebook, so this one is the
# build's own: an integer-only map from a 16-bit state to an fp16 bit pattern,
# cb(s) = ((A*s + B) mod 2^16 AND MASK) OR BASE.  A is odd, so s -> A*s+B is a
# bijection of the 16-bit states; the mask keeps the sign bit, the two low
# exponent bits and the fraction; BASE fixes the high exponent bits, so every
# weight lies in +-[2^-3, 2).  Exactly half the states are negative and the
# value multiset is symmetric about zero.
CB_MUL = 0x9E37
CB_ADD = 0x79B9
CB_MASK = 0x8FFF
CB_BASE = 0x3000


def codebook(states) -> np.ndarray:
    """16-bit trellis states -> fp16 weight bit patterns (unscaled)."""
    s = np.asarray(states, dtype=np.int64) & 0xFFFF
    t = (s * CB_MUL + CB_ADD) & 0xFFFF
    return ((t & CB_MASK) | CB_BASE).astype(np.uint16)


def tile_states(tile_bytes, bits: int) -> np.ndarray:
    """The 256 decoder states of each tile.

    `tile_bytes` is uint8 [..., 32*bits]: one tile's 256*bits-bit stream, bit j
    being bit (j mod 8) of byte floor(j/8) (LSB first; the same as bit j mod 16
    of little-endian 16-bit word floor(j/16)).  State i is the 16-bit window
    that starts at bit i*bits, read LSB first and wrapping around the end of the
    tile (tail-biting), so that storage is exactly `bits` bits per weight and
    windows start at odd offsets when `bits` is odd.
    """
    tb = np.asarray(tile_bytes, dtype=np.uint8)
    length = 256 * bits
    assert tb.shape[-1] * 8 == length
    stream = np.unpackbits(tb, axis=-1, bitorder="little")            # [..., 256*bits]
    pos = (np.arange(256)[:, None] * bits + np.arange(STATE_BITS)[None, :]) % length
    win = stream[..., pos].astype(np.int64)                           # [..., 256, 16]
    return (win << np.arange(STATE_BITS)).sum(axis=-1)               # [..., 256]


def packed_bytes(K: int, N: int, bits: int) -> int:
    """Bytes of packed trellis words for a K x N weight: exactly `bits` per weight."""
    return K * N * bits // 8


def block_bytes(K: int, bits: int) -> int:
    """Bytes of one 128-column block over all K: K/16 tile rows of 8 tiles."""
    return (K // TILE) * 8 * 32 * bits


def decode(words, K: int, N: int, bits: int, block_stride: int | None = None,
           offset: int = 0) -> np.ndarray:
    """Decode packed trellis words into the unscaled fp16 weight matrix W [K, N].

    Layout (block-major): the tile in 128-column block nb, tile row kt (K rows
    16kt..16kt+15) and column tile t (0..7) starts at byte
        offset + nb*block_stride + (kt*8 + t) * 32*bits.
    Inside a tile, weight i sits at K row i mod 16 and column floor(i/16): the
    stream walks down a column first.  A column view of whole blocks is the
    same call with `offset` moved by whole blocks and the parent's
    `block_stride` (a view addresses its blocks with the full weight's strides:
    PR #1507, "What this changes").
    """
    assert K % 128 == 0 and N % BLOCK_COLS == 0 and 1 <= bits <= 8
    if block_stride is None:
        block_stride = block_bytes(K, bits)
    buf = np.asarray(words, dtype=np.uint8).reshape(-1)
    nblk, kts, tb = N // BLOCK_COLS, K // TILE, 32 * bits
    i = np.arange(256)
    rows = np.broadcast_to(np.arange(kts)[:, None, None] * TILE + (i % TILE)[None, None, :], (kts, 8, 256))
    W = np.empty((K, N), dtype=np.uint16)
    for nb in range(nblk):                                   # one column block at a time
        starts = (offset + nb * block_stride
                  + (np.arange(kts)[:, None] * 8 + np.arange(8)[None, :]) * tb)      # [kts, 8]
        tiles = buf[starts[..., None] + np.arange(tb)]                              # [kts, 8, tb]
        w_tiles = codebook(tile_states(tiles, bits))                                 # [kts, 8, 256]
        cols = np.broadcast_to(nb * BLOCK_COLS + np.arange(8)[None, :, None] * TILE
                               + (i // TILE)[None, None, :], (kts, 8, 256))
        W[rows, cols] = w_tiles
    return W


# --------------------------------------------------------------------------
# Steps 2 and 5: the 128-point Hadamard rotations.
# --------------------------------------------------------------------------


def fwht128(v) -> np.ndarray:
    """Unnormalised 128-point Sylvester Hadamard transform (natural order) of
    every 128-chunk of the last axis, by butterflies in float64: for
    h = 1, 2, 4, ..., 64 each pair (i, i+h) with bit h of i clear becomes
    (a+b, a-b).  The result is v . H with H[i, j] = (-1)^popcount(i AND j)."""
    v = np.array(v, dtype=np.float64, copy=True)
    shape = v.shape
    assert shape[-1] % 128 == 0
    v = v.reshape(-1, 128)
    h = 1
    while h < 128:
        w = v.reshape(-1, 128 // (2 * h), 2, h)
        a = w[:, :, 0, :].copy()
        b = w[:, :, 1, :].copy()
        w[:, :, 0, :] = a + b
        w[:, :, 1, :] = a - b
        v = w.reshape(-1, 128)
        h *= 2
    return v.reshape(shape)


ROT_IN_SCALE = 2.0 ** -4      # 2^-4 * 2^-3 = 1/128 = (1/sqrt(128))^2
ROT_OUT_SCALE = 2.0 ** -3


def rot_in(x_bf16, suh_fp16, round_fp16: bool = True) -> np.ndarray:
    """Rotated input: Xr[m, c] = fp16( FWHT128(X[m, c] * suh[c]) * 2^-4 ) per
    128-chunk c of K.  Returns fp16 bits (or float64 values if not rounded)."""
    x = bf16_to_f64(x_bf16)
    with np.errstate(invalid="ignore", over="ignore"):
        xs = x * fp16_to_f64(suh_fp16)[None, :]
        xr = fwht128(xs) * ROT_IN_SCALE
    return f64_to_fp16(xr) if round_fp16 else xr


def linear(W_fp16, scales_fp16, suh_fp16, svh_fp16, x_bf16,
           exact: bool = False) -> np.ndarray:
    """Y = rot_out( (rot_in(X) . W) * scale ) for one weight or one view.

    W_fp16 [K, N] are the decoded (unscaled) weights; scales, svh are per
    column of this weight or view; suh is per K row.  Returns bf16 bits [M, N];
    with exact=True it skips both roundings (fp16 Xr, bf16 Y) and returns the
    float64 values, for the dense brute-force check.
    """
    W = fp16_to_f64(W_fp16)
    xr = rot_in(x_bf16, suh_fp16, round_fp16=not exact)
    xr = xr if exact else fp16_to_f64(xr)
    with np.errstate(invalid="ignore", over="ignore"):           # NaN/Inf propagate
        z = xr @ W                                                # step 3, float64
        zs = z * fp16_to_f64(scales_fp16)[None, :]                # step 4
        y = fwht128(zs) * ROT_OUT_SCALE * fp16_to_f64(svh_fp16)[None, :]   # step 5
    return y if exact else f64_to_bf16(y)


def linear_packed(words, K, N, bits, scales_fp16, suh_fp16, svh_fp16, x_bf16,
                  block_stride=None, offset=0, exact=False) -> np.ndarray:
    """Decode then apply: the whole path for one weight or column view."""
    W = decode(words, K, N, bits, block_stride=block_stride, offset=offset)
    return linear(W, scales_fp16, suh_fp16, svh_fp16, x_bf16, exact=exact)
