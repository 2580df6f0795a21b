"""Planted mistakes in the oracle must turn at least one pin red.

Each mutation replaces one oracle function (on the CPU, inside this test
process only) with a plausibly wrong variant: a dropped term, a wrong sign or
index, a transposed operand, a wrong constant or rounding.  The pins that
could see it are then run; the test passes only if one of them fails.
"""

import numpy as np
import pytest

import oracle_pins as P
from oracle import exl3_oracle as O

_orig = {name: getattr(O, name) for name in
         ("codebook", "tile_states", "decode", "fwht128", "rot_in", "linear", "f64_to_fp16", "f64_to_bf16",
          "_round_to_format", "fp16_to_f64")}


def _cb_even_multiplier(states):
    s = np.asarray(states, dtype=np.int64) & 0xFFFF
    t = (s * (O.CB_MUL + 1) + O.CB_ADD) & 0xFFFF
    return ((t & O.CB_MASK) | O.CB_BASE).astype(np.uint16)


def _cb_wrong_constant(states):
    s = np.asarray(states, dtype=np.int64) & 0xFFFF
    t = (s * (O.CB_MUL + 2) + O.CB_ADD) & 0xFFFF
    return ((t & O.CB_MASK) | O.CB_BASE).astype(np.uint16)


def _cb_xor_base(states):
    s = np.asarray(states, dtype=np.int64) & 0xFFFF
    t = (s * O.CB_MUL + O.CB_ADD) & 0xFFFF
    return ((t & 0x9FFF) ^ O.CB_BASE).astype(np.uint16)


def _states_msb_first(tile_bytes, bits):
    tb = np.asarray(tile_bytes, dtype=np.uint8)
    length = 256 * bits
    stream = np.unpackbits(tb, axis=-1, bitorder="big")
    pos = (np.arange(256)[:, None] * bits + np.arange(16)[None, :]) % length
    return (stream[..., pos].astype(np.int64) << np.arange(16)).sum(axis=-1)


def _states_no_wrap(tile_bytes, bits):
    tb = np.asarray(tile_bytes, dtype=np.uint8)
    length = 256 * bits
    stream = np.unpackbits(tb, axis=-1, bitorder="little")
    stream = np.concatenate([stream, np.zeros(stream.shape[:-1] + (16,), stream.dtype)], axis=-1)
    pos = np.arange(256)[:, None] * bits + np.arange(16)[None, :]
    return (stream[..., pos].astype(np.int64) << np.arange(16)).sum(axis=-1)


def _states_off_by_one(tile_bytes, bits):
    tb = np.asarray(tile_bytes, dtype=np.uint8)
    length = 256 * bits
    stream = np.unpackbits(tb, axis=-1, bitorder="little")
    pos = (np.arange(256)[:, None] * bits + 1 + np.arange(16)[None, :]) % length
    return (stream[..., pos].astype(np.int64) << np.arange(16)).sum(axis=-1)


def _states_stride_16(tile_bytes, bits):
    tb = np.asarray(tile_bytes, dtype=np.uint8)
    length = 256 * bits
    stream = np.unpackbits(tb, axis=-1, bitorder="little")
    pos = (np.arange(256)[:, None] * (bits + 1) + np.arange(16)[None, :]) % length
    return (stream[..., pos].astype(np.int64) << np.arange(16)).sum(axis=-1)


def _decode_row_major_tile(words, K, N, bits, block_stride=None, offset=0):
    W = _orig["decode"](words, K, N, bits, block_stride=block_stride, offset=offset)
    # weight i at (i // 16, i % 16) instead of (i % 16, i // 16): transpose every tile
    return W.reshape(K // 16, 16, N // 16, 16).transpose(0, 3, 2, 1).reshape(K, N)


def _decode_tiles_kt_inner(words, K, N, bits, block_stride=None, offset=0):
    # tiles ordered [nb][t][kt] instead of [nb][kt][t]
    W = _orig["decode"](words, K, N, bits, block_stride=block_stride, offset=offset)
    kts = K // 16
    nb = N // 128
    T = W.reshape(kts, 16, nb, 8, 16).transpose(2, 0, 3, 1, 4)        # [nb, kt, t, 16, 16]
    T = T.reshape(nb, kts * 8, 16, 16)
    idx = np.arange(kts * 8).reshape(kts, 8).T.reshape(-1)             # reinterpret order
    T = T[:, idx].reshape(nb, kts, 8, 16, 16).transpose(1, 3, 0, 2, 4)
    return T.reshape(K, N)


def _fwht_skip_level(v):
    v = np.array(v, dtype=np.float64, copy=True)
    shape = v.shape
    v = v.reshape(-1, 128)
    for h in (1, 2, 4, 8, 32, 64):          # level 16 dropped
        w = v.reshape(-1, 128 // (2 * h), 2, h)
        a, b = w[:, :, 0, :].copy(), w[:, :, 1, :].copy()
        w[:, :, 0, :], w[:, :, 1, :] = a + b, a - b
        v = w.reshape(-1, 128)
    return v.reshape(shape)


def _fwht_wrong_sign(v):
    v = np.array(v, dtype=np.float64, copy=True)
    shape = v.shape
    v = v.reshape(-1, 128)
    h = 1
    while h < 128:
        w = v.reshape(-1, 128 // (2 * h), 2, h)
        a, b = w[:, :, 0, :].copy(), w[:, :, 1, :].copy()
        w[:, :, 0, :], w[:, :, 1, :] = a + b, b - a
        v = w.reshape(-1, 128)
        h *= 2
    return v.reshape(shape)


def _rot_in_no_suh(x_bf16, suh_fp16, round_fp16=True):
    return _orig["rot_in"](x_bf16, np.full_like(suh_fp16, 0x3C00), round_fp16)


def _rot_in_wrong_scale(x_bf16, suh_fp16, round_fp16=True):
    x = O.bf16_to_f64(x_bf16) * O.fp16_to_f64(suh_fp16)[None, :]
    xr = O.fwht128(x) * 2.0 ** -3
    return O.f64_to_fp16(xr) if round_fp16 else xr


def _linear_transposed(W_fp16, scales, suh, svh, x, exact=False):
    return _orig["linear"](np.ascontiguousarray(W_fp16.T), scales, suh, svh, x, exact)


def _linear_scale_after_rotation(W_fp16, scales, suh, svh, x, exact=False):
    W = O.fp16_to_f64(W_fp16)
    xr = O.rot_in(x, suh, round_fp16=not exact)
    xr = xr if exact else O.fp16_to_f64(xr)
    y = O.fwht128(xr @ W) * O.ROT_OUT_SCALE * O.fp16_to_f64(scales)[None, :] * O.fp16_to_f64(svh)[None, :]
    return y if exact else O.f64_to_bf16(y)


def _linear_no_svh(W_fp16, scales, suh, svh, x, exact=False):
    return _orig["linear"](W_fp16, scales, suh, np.full_like(svh, 0x3C00), x, exact)


def _linear_no_out_rotation(W_fp16, scales, suh, svh, x, exact=False):
    W = O.fp16_to_f64(W_fp16)
    xr = O.rot_in(x, suh, round_fp16=not exact)
    xr = xr if exact else O.fp16_to_f64(xr)
    y = (xr @ W) * O.fp16_to_f64(scales)[None, :] * O.fp16_to_f64(svh)[None, :]
    return y if exact else O.f64_to_bf16(y)


def _round_half_away(x, frac_bits, emin, inf_bits, nan_bits):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    finite = np.isfinite(a)
    a_safe = np.where(finite & (a > 0), a, 1.0)
    _, e2 = np.frexp(a_safe)
    le = np.maximum(e2.astype(np.int64) - 1, emin)
    r = np.floor(np.ldexp(a_safe, (frac_bits - le).astype(np.int64)) + 0.5)
    enc = ((le - emin) << frac_bits) + r.astype(np.int64)
    enc = np.where(a == 0, 0, enc)
    enc = np.where(enc >= inf_bits, inf_bits, enc)
    enc = np.where(np.isinf(a), inf_bits, enc)
    enc = np.where(np.isnan(a), nan_bits, enc)
    return (enc | np.where(np.signbit(x) & ~np.isnan(x), 0x8000, 0)).astype(np.uint16)


def _round_truncate(x, frac_bits, emin, inf_bits, nan_bits):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    a_safe = np.where(np.isfinite(a) & (a > 0), a, 1.0)
    _, e2 = np.frexp(a_safe)
    le = np.maximum(e2.astype(np.int64) - 1, emin)
    r = np.floor(np.ldexp(a_safe, (frac_bits - le).astype(np.int64)))
    enc = ((le - emin) << frac_bits) + r.astype(np.int64)
    enc = np.where(a == 0, 0, enc)
    enc = np.where(enc >= inf_bits, inf_bits, enc)
    enc = np.where(np.isinf(a), inf_bits, enc)
    enc = np.where(np.isnan(a), nan_bits, enc)
    return (enc | np.where(np.signbit(x) & ~np.isnan(x), 0x8000, 0)).astype(np.uint16)


def _fp16_decode_wrong_bias(bits):
    return _orig["fp16_to_f64"](bits) * 2.0


MUTATIONS = {
    "codebook: even multiplier": ("codebook", _cb_even_multiplier),
    "codebook: wrong odd multiplier": ("codebook", _cb_wrong_constant),
    "codebook: xor instead of or": ("codebook", _cb_xor_base),
    "windows: MSB-first stream": ("tile_states", _states_msb_first),
    "windows: no tail-biting wrap": ("tile_states", _states_no_wrap),
    "windows: start off by one bit": ("tile_states", _states_off_by_one),
    "windows: wrong stride": ("tile_states", _states_stride_16),
    "decode: row-major tile walk": ("decode", _decode_row_major_tile),
    "decode: tiles kt-inner": ("decode", _decode_tiles_kt_inner),
    "fwht: level dropped": ("fwht128", _fwht_skip_level),
    "fwht: wrong butterfly sign": ("fwht128", _fwht_wrong_sign),
    "rot_in: suh dropped": ("rot_in", _rot_in_no_suh),
    "rot_in: 2^-3 instead of 2^-4": ("rot_in", _rot_in_wrong_scale),
    "linear: W transposed": ("linear", _linear_transposed),
    "linear: scale after rotation": ("linear", _linear_scale_after_rotation),
    "linear: svh dropped": ("linear", _linear_no_svh),
    "linear: output rotation dropped": ("linear", _linear_no_out_rotation),
    "rounding: ties away from zero": ("_round_to_format", _round_half_away),
    "rounding: truncation": ("_round_to_format", _round_truncate),
    "fp16 decode: wrong bias": ("fp16_to_f64", _fp16_decode_wrong_bias),
}


def _fails(check):
    try:
        check()
    except AssertionError:
        return True
    except Exception:          # a crash counts as red too
        return True
    return False


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_goes_red(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    red = [c.__name__ for c in P.ALL_CHECKS if _fails(c)]
    assert red, f"no pin caught the planted mistake '{name}'"
