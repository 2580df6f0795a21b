"""The opt-in prompt arithmetic (exl3_set_prompt_arithmetic(1)): above 128
rows each output is one MFMA chain over all of K. It is held to the oracle
tolerance like every other path, gives the same bits for a row whatever the
row count above 128, and leaves calls of up to 128 rows untouched. Its bits
differ from the bit-stable path's (the pages' reason for keeping such tiles
out of the default, TensorFold PR #1475 review), which the last test shows.
"""

import numpy as np
import pytest

import gpu_util as G
from oracle import exl3_oracle as O
from trellis_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu


def ex():
    import trellis_quantized_linear_amd.exl3 as m
    return m


@pytest.fixture(autouse=True)
def _mode():
    ex().lib()
    ex().exl3_test_force(-1, -1, 0)
    ex().exl3_set_prompt_arithmetic(1)
    yield
    ex().exl3_set_prompt_arithmetic(0)


@pytest.mark.parametrize("K,N,bits,M", [(256, 128, 4, 129), (640, 640, 2, 200), (1024, 1024, 3, 300),
                                        (384, 512, 5, 257), (512, 384, 6, 140), (256, 896, 7, 133),
                                        (512, 256, 8, 300)])
def test_single_chain_prompt_tiles_match_the_oracle(K, N, bits, M):
    """Every width, ragged row blocks, block counts that leave the last
    4-block tile partly empty; the whole output against the oracle."""
    L = G.layer("quad", f"{K}x{N}b{bits}", K, N, bits)
    x = G.xbits("quad", M, K, sigma=0.5)
    w = G.upload(L)
    y = G.run(w, G.dev_bf16(x), tag="single-chain prompt")
    ref = O.linear_packed(L.words, K, N, bits, L.scales, L.suh, L.svh, x)
    G.assert_close(G.host_u16(y), ref, what=f"single chain K={K} N={N} b={bits} M={M}")


def test_single_chain_rows_do_not_depend_on_row_count():
    K, N = 5120, 6144
    L = G.layer("quad", "q", K, N, 4)
    w = G.upload(L)
    x = G.xbits("quad-rows", 300, K, sigma=0.5)
    xd = G.dev_bf16(x)
    full = G.host_u16(G.run(w, xd, M=300, tag="300 rows"))
    part = G.host_u16(G.run(w, xd, M=129, tag="129 rows"))
    assert np.array_equal(part, full[:129])
    rows = np.array([0, 127, 128, 299])
    blocks = G.sample_blocks(N // 128, k=3, seed=5)
    G.assert_close(G.gpu_blocks(G.dev_u16(full).view(G.torch_mod().bfloat16), blocks, rows),
                   G.oracle_blocks(L, x, blocks, rows), what="single chain 27B q")


def test_group_and_small_calls():
    """A {gate, up} group at 256 rows equals each member alone; up to 128 rows
    the mode changes nothing (bitwise equal to mode 0)."""
    K = synth.HIDDEN
    layers = [G.layer("quad-group", n, K, 2048, 4) for n in ("gate", "up")]
    ws_ = [G.upload(L) for L in layers]
    xd = G.dev_bf16(G.xbits("quad-group", 256, K, sigma=0.5))
    ys = G.run_group(ws_, xd, tag="group")
    for w, y in zip(ws_, ys):
        assert np.array_equal(G.host_u16(y), G.host_u16(G.run(w, xd, tag="solo")))
    small = G.host_u16(G.run(ws_[0], xd[:128], M=128, tag="128 rows, mode 1"))
    ex().exl3_set_prompt_arithmetic(0)
    assert np.array_equal(small, G.host_u16(G.run(ws_[0], xd[:128], M=128, tag="128 rows, mode 0")))


def test_bits_differ_from_the_bit_stable_path():
    """Planted control: the single chain is another summation order, so some
    outputs move by a bf16 step against the default prompt path."""
    K, N, M = 5120, 1024, 256
    L = G.layer("quad", "k", K, N, 4)
    w = G.upload(L)
    xd = G.dev_bf16(G.xbits("quad-ctl", M, K, sigma=0.5))
    fast = G.host_u16(G.run(w, xd, tag="mode 1"))
    ex().exl3_set_prompt_arithmetic(0)
    stable = G.host_u16(G.run(w, xd, tag="mode 0"))
    assert not np.array_equal(fast, stable)
