"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bit-exact: the codebook on all 65,536 states, decoded weights at every width
(2..8 bits), the pages' fill patterns, and closed-form outputs whose every
intermediate is exact. Within the parity tolerance (max |Y - Y_oracle| <=
1e-2 max |Y_oracle|, NaN/Inf positions identical): the linear on the five
configurations of the 27B layer, at full size on sampled column blocks and
rows where the oracle cannot do the whole output in seconds.
"""

import numpy as np
import pytest

import gpu_util as G
from oracle import exl3_oracle as O
from trellis_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import trellis_quantized_linear_amd.exl3 as ex
    assert torch.cuda.is_available()
    ex.lib()
    ex.exl3_test_force(-1, -1, 0)
    yield
    ex.exl3_test_force(-1, -1, 0)


def ex():
    import trellis_quantized_linear_amd.exl3 as m
    return m


# ------------------------------------------------------------ bit-exact decode

def test_codebook_all_states():
    torch = G.torch_mod()
    states = np.arange(65536, dtype=np.uint16)
    s = G.dev_u16(states)
    out = torch.zeros_like(s)
    G.say("exl3_test_codebook n=65536")
    ex().exl3_test_codebook(s, out)
    assert np.array_equal(G.host_u16(out), O.codebook(states))
    # odd n: the last state is handled alone
    out3 = torch.zeros(3, dtype=torch.int16, device="cuda")
    ex().exl3_test_codebook(s[:3], out3)
    assert np.array_equal(G.host_u16(out3), O.codebook(states[:3]))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_dequant_bit_exact(bits):
    torch = G.torch_mod()
    L = G.layer("dequant", f"w{bits}", 256, 384, bits)
    w = G.upload(L)
    out = torch.zeros((256, 384), dtype=torch.int16, device="cuda")
    G.say(f"exl3_test_dequant K=256 N=384 bits={bits}")
    ex().exl3_test_dequant(w, out)
    assert np.array_equal(G.host_u16(out), O.decode(L.words, 256, 384, bits))


@pytest.mark.parametrize("K,N,bits", [(5120, 1024, 4), (5120, 512, 6), (17408, 256, 3)])
def test_dequant_bit_exact_large(K, N, bits):
    torch = G.torch_mod()
    L = G.layer("dequant-large", "w", K, N, bits)
    w = G.upload(L)
    out = torch.zeros((K, N), dtype=torch.int16, device="cuda")
    G.say(f"exl3_test_dequant K={K} N={N} bits={bits}")
    ex().exl3_test_dequant(w, out)
    assert np.array_equal(G.host_u16(out), O.decode(L.words, K, N, bits))


def test_dequant_of_a_view():
    torch = G.torch_mod()
    L = G.layer("dequant-view", "w", 512, 1024, 6)
    w = G.upload(L)
    v = w.columns(384, 512)
    out = torch.zeros((512, 512), dtype=torch.int16, device="cuda")
    G.say("exl3_test_dequant view [384, 896) of K=512 N=1024 bits=6")
    ex().exl3_test_dequant(v, out)
    ref = O.decode(L.words, 512, 512, 6, block_stride=O.block_bytes(512, 6), offset=3 * O.block_bytes(512, 6))
    assert np.array_equal(G.host_u16(out), ref)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_dequant_fills_from_the_pages(bits):
    """PR #1467 gate 4: all-ones states give one weight at every width; a
    0xaaaa fill gives two alternating weights at odd widths."""
    torch = G.torch_mod()
    K, N = 256, 128
    for fill in (0xFF, 0xAA, 0x00):
        L = synth.LayerInputs("fill", K, N, bits, np.full(O.packed_bytes(K, N, bits), fill, np.uint8),
                              np.full(N, 0x3C00, np.uint16), np.full(K, 0x3C00, np.uint16),
                              np.full(N, 0x3C00, np.uint16))
        w = G.upload(L)
        out = torch.zeros((K, N), dtype=torch.int16, device="cuda")
        G.say(f"exl3_test_dequant fill={fill:#x} bits={bits}")
        ex().exl3_test_dequant(w, out)
        got = G.host_u16(out)
        assert np.array_equal(got, O.decode(L.words, K, N, bits))
        n_distinct = np.unique(got).size
        assert n_distinct == (2 if (fill == 0xAA and bits % 2 == 1) else 1)


# ------------------------------------------------------------ rotation

@pytest.mark.parametrize("K,M", [(256, 3), (5120, 16), (17408, 5), (5120, 1101)])
def test_rot_in_vs_oracle(K, M):
    """fp32 butterflies then one fp16 rounding, against float64 then one fp16
    rounding: equal except where the fp32 sum lands across an fp16 rounding
    boundary, and then by one fp16 ulp (1101 rows: a ragged last 4-row
    piece)."""
    torch = G.torch_mod()
    L = G.layer("rot", "w", K, 128, 4)
    x = G.xbits("rot", M, K)
    w = G.upload(L)
    out = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    G.say(f"exl3_test_rot_in K={K} M={M}")
    ex().exl3_test_rot_in(w, G.dev_bf16(x), out)
    got = G.host_u16(out).astype(np.int64)
    ref = O.rot_in(x, L.suh).astype(np.int64)
    same_sign = ((got ^ ref) & 0x8000) == 0
    d = np.abs(got - ref)
    assert np.all((d == 0) | (same_sign & (d == 1))), "rotated input off by more than one fp16 ulp"
    assert (d != 0).mean() < 1e-3


# ------------------------------------------------------------ the linear, tiny configuration

@pytest.mark.parametrize("M", [1, 3, 16])
def test_linear_tiny_configuration(M):
    """K = N = 256, 4 bits, 2 column blocks, M = 1, 3, 16: the whole output."""
    L = G.layer("tiny", "w", 256, 256, 4)
    x = G.xbits("tiny", M, 256)
    w = G.upload(L)
    y = G.run(w, G.dev_bf16(x), tag="tiny")
    ref = O.linear_packed(L.words, 256, 256, 4, L.scales, L.suh, L.svh, x)
    G.assert_close(G.host_u16(y), ref, what=f"tiny M={M}")


@pytest.mark.parametrize("K,N,bits,M", [(128, 128, 4, 1), (128, 384, 3, 5), (384, 128, 5, 40), (640, 256, 2, 130),
                                        (1024, 640, 7, 17), (512, 256, 8, 300), (256, 128, 6, 129)])
def test_linear_small_shapes_whole_output(K, N, bits, M):
    """Small and ragged shapes (one block, one chunk group, ragged row blocks),
    whole output against the oracle."""
    L = G.layer("small", f"{K}x{N}b{bits}", K, N, bits)
    x = G.xbits("small", M, K)
    w = G.upload(L)
    y = G.run(w, G.dev_bf16(x), tag="small")
    ref = O.linear_packed(L.words, K, N, bits, L.scales, L.suh, L.svh, x)
    G.assert_close(G.host_u16(y), ref, what=f"K={K} N={N} b={bits} M={M}")


# ------------------------------------------------------------ the 27B configurations

C2_MEMBERS = [("q", synth.Q_COLS), ("k", synth.KV_COLS), ("v", synth.KV_COLS),
              ("gate", synth.INTERMEDIATE), ("up", synth.INTERMEDIATE)]


@pytest.mark.parametrize("M", [1, 7, 16])
@pytest.mark.parametrize("name,N", C2_MEMBERS)
def test_linear_decode_rows_27b(name, N, M):
    """27B decode-row members (K = 5120, 4 bits) at full size; the oracle on
    sampled column blocks (first, last, two random)."""
    L = G.layer("c2", name, synth.HIDDEN, N, 4)
    x = G.xbits("c2", M, synth.HIDDEN)
    w = G.upload(L)
    y = G.run(w, G.dev_bf16(x), tag=f"c2 {name}")
    blocks = G.sample_blocks(N // 128, seed=M)
    G.assert_close(G.gpu_blocks(y, blocks), G.oracle_blocks(L, x, blocks), what=f"c2 {name} M={M}")


@pytest.mark.parametrize("M", [17, 24, 32, 33, 48, 49, 64, 100, 128])
def test_linear_mid_rows_27b_mlp(M):
    """27B dense SwiGLU MLP at 3.5 bpw: gate/up 5120 -> 17408 at 3 bits, down
    17408 -> 5120 at 4 bits, mid-M rows."""
    for name, K, N, bits in (("gate", 5120, 17408, 3), ("down", 17408, 5120, 4)):
        L = G.layer("c3", name, K, N, bits)
        x = G.xbits("c3", M, K)
        w = G.upload(L)
        y = G.run(w, G.dev_bf16(x), tag=f"c3 {name}")
        blocks = G.sample_blocks(N // 128, k=3, seed=M)
        G.assert_close(G.gpu_blocks(y, blocks), G.oracle_blocks(L, x, blocks), what=f"c3 {name} M={M}")


@pytest.mark.parametrize("name,K,N", [("q", 5120, 6144), ("k", 5120, 1024), ("gate", 5120, 17408),
                                      ("down", 17408, 5120)])
def test_linear_prompt_8192_rows(name, K, N):
    """Prompt prefill of one 27B layer's linears: M = 8192 rows (64 row
    blocks of 128), 4 bits, X ~ N(0, 0.5); sampled rows x sampled blocks."""
    M = 8192
    L = G.layer("c4", name, K, N, 4)
    x = G.xbits("c4", M, K, sigma=0.5)
    w = G.upload(L)
    y = G.run(w, G.dev_bf16(x), tag=f"c4 {name}")
    rows = np.array([0, 1, 127, 128, 4095, 8000, 8191])
    blocks = G.sample_blocks(N // 128, k=3, seed=7)
    G.assert_close(G.gpu_blocks(y, blocks, rows), G.oracle_blocks(L, x, blocks, rows), what=f"c4 {name}")


def test_linear_head_6bit_views():
    """The 6-bit head 5120 -> 248,320 and its two span views at M = 16."""
    K, N, M = 5120, synth.VOCAB, 16
    L = G.layer("c5", "head", K, N, 6)
    x = G.xbits("c5", M, K)
    w = G.upload(L)
    xd = G.dev_bf16(x)
    a = w.columns(0, 98304)
    b = w.columns(240128, 8192)
    ya = G.run(a, xd, tag="c5 span A")
    yb = G.run(b, xd, tag="c5 span B")
    for y, base, nblk, what in ((ya, 0, 768, "span A"), (yb, 240128 // 128, 64, "span B")):
        blocks = G.sample_blocks(nblk, k=3, seed=nblk)
        G.assert_close(G.gpu_blocks(y, blocks), G.oracle_blocks(L, x, [base + b_ for b_ in blocks]), what=what)


# ------------------------------------------------------------ exact cases and special values

def test_constant_weights_closed_form_bit_exact():
    """All-ones states (one weight c at every width), scales 1, X nonzero only
    at K = 128j with small integers: every GPU intermediate is exact, so Y is
    exactly bf16(128 c svh[128b] sum_j x[m,128j] suh[128j]) in every regime."""
    torch = G.torch_mod()
    rng = np.random.default_rng(4)
    K, N, bits = 1024, 512, 5
    Lw = synth.LayerInputs("const", K, N, bits, np.full(O.packed_bytes(K, N, bits), 0xFF, np.uint8),
                           np.full(N, 0x3C00, np.uint16), synth.gen_signs(rng, K), synth.gen_signs(rng, N))
    w = G.upload(Lw)
    xv = np.zeros((20, K))
    xv[:, ::128] = rng.integers(-8, 9, size=(20, K // 128))
    x = O.f64_to_bf16(xv)
    ref = O.linear_packed(Lw.words, K, N, bits, Lw.scales, Lw.suh, Lw.svh, x)
    for mt in (1, 2, 4, 8):
        for chained in (0, 1):
            ex().exl3_test_force(mt, chained, 0)
            y = G.run(w, G.dev_bf16(x), tag=f"const m_tiles={mt} chained={chained}")
            got = O.bf16_to_f64(G.host_u16(y))
            assert np.array_equal(got, O.bf16_to_f64(ref)), (mt, chained)
    ex().exl3_test_force(-1, -1, 0)


def test_fp32_stress_rotated_inputs_of_4096():
    """PR #1467 gate 4: a constant weight times rotated inputs of 4096: fp16
    sums would overflow, fp32 ones stay in bound; the result is exact."""
    K, N, bits = 5120, 256, 4
    L = synth.LayerInputs("stress", K, N, bits, np.full(O.packed_bytes(K, N, bits), 0xFF, np.uint8),
                          np.full(N, 0x3C00, np.uint16), np.full(K, 0x3C00, np.uint16), np.full(N, 0x3C00, np.uint16))
    xv = np.zeros((4, K))
    xv[:, ::128] = 65536.0
    xv[1, ::256] = -65536.0
    x = O.f64_to_bf16(xv)
    w = G.upload(L)
    y = G.run(w, G.dev_bf16(x), tag="fp32 stress")
    ref = O.linear_packed(L.words, K, N, bits, L.scales, L.suh, L.svh, x)
    assert np.array_equal(O.bf16_to_f64(G.host_u16(y)), O.bf16_to_f64(ref))
    assert np.abs(O.bf16_to_f64(ref)).max() > 65504


def test_special_values_reach_the_outputs():
    """PR #1467 gate 1: planted NaN and both infinities reach the outputs, at
    the same positions as in the oracle."""
    K, N, bits, M = 512, 384, 4, 6
    L = G.layer("special", "w", K, N, bits)
    x = G.xbits("special", M, K)
    x[0, 3] = 0x7FC0
    x[1, 200] = 0x7F80
    x[2, 17] = 0xFF80
    L.scales[130] = 0x7C00      # +inf scale: its block
    L.svh[300] = 0x7E00         # NaN output sign: one column
    w = G.upload(L)
    y = G.run(w, G.dev_bf16(x), tag="special")
    ref = O.linear_packed(L.words, K, N, bits, L.scales, L.suh, L.svh, x)
    G.assert_close(G.host_u16(y), ref, what="special values")
    got = O.bf16_to_f64(G.host_u16(y))
    assert np.isnan(got[0]).all() and np.isnan(got[1]).all() and np.isnan(got[2]).all()
    assert np.isnan(got[3:, 300]).all()


def test_m_zero_leaves_output_untouched():
    torch = G.torch_mod()
    L = G.layer("empty", "w", 256, 256, 4)
    w = G.upload(L)
    y = G.empty_y(4, 256)
    before = G.host_u16(y).copy()
    x = G.dev_bf16(G.xbits("empty", 4, 256))
    ws = ex().Workspace().reserve([w], 4)
    ex().exl3_linear(w, x, y, ws, M=0)
    torch.cuda.synchronize()
    assert np.array_equal(G.host_u16(y), before)


def test_strided_x_and_y():
    """ldx > K and ldy > N: rows read and written with the given strides,
    untouched padding."""
    torch = G.torch_mod()
    K, N, M = 512, 256, 5
    L = G.layer("strided", "w", K, N, 4)
    x = G.xbits("strided", M, K)
    xpad = np.zeros((M, K + 64), np.uint16)
    xpad[:, :K] = x
    w = G.upload(L)
    xd = G.dev_bf16(xpad)
    ybig = torch.full((M, N + 128), 7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ws = ex().Workspace().reserve([w], M)
    G.say("exl3_linear strided ldx=576 ldy=384")
    ex().exl3_linear(w, xd, ybig, ws)
    yb = G.host_u16(ybig)
    G.assert_close(yb[:, :N], O.linear_packed(L.words, K, N, 4, L.scales, L.suh, L.svh, x), what="strided")
    assert np.all(yb[:, N:] == 7)


# ------------------------------------------------------------ widths x shapes sweep

SWEEP_KN = [(128, 128), (384, 640), (1024, 2048), (4096, 384), (16384, 256)]


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_width_and_shape_sweep_mid_rows(bits):
    """The width matrix (2..8 bits) over K, N in 128..16384 at mid-M rows
    (17..128; one row count per shape, rotating with the width), every
    launch the dispatcher picks there, sampled blocks against the oracle and
    two rows against single-row calls bit for bit."""
    rows_cycle = [17, 33, 64, 100, 128]
    for i, (K, N) in enumerate(SWEEP_KN):
        M = rows_cycle[(i + bits) % len(rows_cycle)]
        L = G.layer("sweep", f"{K}x{N}b{bits}", K, N, bits)
        x = G.xbits("sweep", M, K)
        w = G.upload(L)
        xd = G.dev_bf16(x)
        y = G.run(w, xd, tag=f"sweep b={bits}")
        blocks = G.sample_blocks(N // 128, k=2, seed=bits + i)
        G.assert_close(G.gpu_blocks(y, blocks), G.oracle_blocks(L, x, blocks), what=f"sweep K={K} N={N} b={bits} M={M}")
        full = G.host_u16(y)
        for r in (0, M - 1):
            one = G.host_u16(G.run(w, xd[r:r + 1], M=1, tag=f"sweep row {r}"))
            assert np.array_equal(one[0], full[r]), (K, N, bits, M, r)


def test_prompt_rows_at_the_size_limit():
    """Largest call: M K 2 < 2^31 bytes of rotated input per member (the
    library's 32-bit offsets), so at K = 5120 at most 209,715 rows; the
    128-row tilings read that input chunk-major up to the last chunk offset.
    X repeats 1024 seeded rows: sampled rows against the oracle, rows a
    multiple of 1024 apart byte-identical. One row more is refused
    (EXL3_EINVAL) before anything is launched."""
    torch = G.torch_mod()
    K, N, M = 5120, 128, 209715
    L = G.layer("size-limit", "w", K, N, 4)
    w = G.upload(L)
    base = G.xbits("size-limit", 1024, K)
    xd = G.dev_bf16(base).repeat((M + 1 + 1023) // 1024, 1)[:M + 1].contiguous()
    y = G.empty_y(M + 1, N)
    ws = ex().Workspace().reserve([w], M)
    G.say(f"exl3_linear K={K} N={N} M={M} (2KM = {2 * K * M}, limit {2 ** 31})")
    ex().exl3_linear(w, xd, y, ws, M=M)
    torch.cuda.synchronize()
    yh = G.host_u16(y)
    rows = [0, 1, 1023, 1024 * 100 + 7, M - 1]
    ref = G.oracle_blocks(L, base, [0], rows=[r % 1024 for r in rows])
    G.assert_close(yh[rows], ref, what=f"M={M}")
    for r in (5, 1000, M - 1):
        assert np.array_equal(yh[r], yh[r % 1024]), r
    last = yh[M].copy()
    with pytest.raises(ex().Exl3Error) as e:
        ex().exl3_linear(w, xd, y, ws, M=M + 1)
    assert e.value.code == ex().EXL3_EINVAL
    torch.cuda.synchronize()
    assert np.array_equal(G.host_u16(y)[M], last)
