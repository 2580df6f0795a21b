"""GPU self-consistency, bitwise: a row's bytes do not depend on how many rows
are in the call, on the row tiling or launch shape, on group membership or on
column views (TensorFold PR #1467 "The arithmetic" and its gate 3; PR #1407
review item 1; PR #1507 review: a wide view takes the full head's plan, so
its logits keep their bytes). Counters are zero whenever no call runs (PR #1475).

Planted controls (another K split, a member's scales swapped, a member's suh
swapped) must change bytes, which shows the comparisons can see a change.
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
def _hooks():
    ex().lib()
    ex().exl3_test_force(-1, -1, 0)
    yield
    ex().exl3_test_force(-1, -1, 0)


# weights covering each plan kind: narrow (S = 16), wide (S = 15), K = 17408, 3 and 6 bits
SHAPES = [("k", 5120, 1024, 4), ("q", 5120, 6144, 4), ("wide", 5120, 8192, 4), ("down", 17408, 5120, 4),
          ("gate3", 5120, 2048, 3), ("head6", 5120, 8192, 6)]


@pytest.mark.parametrize("name,K,N,bits", SHAPES)
def test_rows_identical_for_every_row_count(name, K, N, bits):
    L = G.layer("rows", name, K, N, bits)
    w = G.upload(L)
    x = G.xbits("rows", 128, K)
    xd = G.dev_bf16(x)
    full = G.host_u16(G.run(w, xd, M=128, tag=f"rows {name} M=128"))
    for M in (1, 2, 7, 15, 16, 17, 24, 32, 33, 48, 49, 64, 100, 127):
        y = G.host_u16(G.run(w, xd, M=M, tag=f"rows {name}"))
        assert np.array_equal(y[:M], full[:M]), (name, M)


@pytest.mark.parametrize("name,K,N,bits", SHAPES[:4])
def test_rows_identical_for_every_tiling_and_launch_shape(name, K, N, bits):
    """The min_rows analogue: force each row tiling (1, 2, 4, 8 MFMA row tiles
    per workgroup, and 128-row tiles two blocks wide) and each launch shape
    (one split per workgroup with counter exchange, every split in one
    workgroup, and at 16 rows the spread launch and the exchange with each
    split on two waves of 4 column tiles) at several row counts."""
    L = G.layer("tiling", name, K, N, bits)
    w = G.upload(L)
    x = G.xbits("tiling", 40, K)
    xd = G.dev_bf16(x)
    ref = G.host_u16(G.run(w, xd, M=40, tag="auto"))
    for mt in (1, 2, 4, 8, 16):
        for chained in ((0, 1, 2, 3) if mt == 1 else (0, 1)):
            ex().exl3_test_force(mt, chained, 0)
            for M in (1, 16, 17, 40):
                y = G.host_u16(G.run(w, xd, M=M, tag=f"forced m_tiles={mt} chained={chained}"))
                assert np.array_equal(y[:M], ref[:M]), (name, mt, chained, M)
    ex().exl3_test_force(-1, -1, 0)


@pytest.mark.parametrize("M", [1, 16])
def test_spread_launch_with_many_left_blocks(M):
    """The spread launch with 4 splits per block: 12 spare waves per workgroup,
    three quarters of the blocks finished by spare waves, several per
    workgroup; bitwise equal to the chained and the exchanged launch of the
    same plan."""
    L = G.layer("spread", "q", synth.HIDDEN, synth.Q_COLS, 4)
    w = G.upload(L)
    xd = G.dev_bf16(G.xbits("spread", M, synth.HIDDEN))
    out = {}
    for chained in (2, 1, 0):
        ex().exl3_test_force(1, chained, 4)
        out[chained] = G.host_u16(G.run(w, xd, tag=f"splits=4 chained={chained}"))
    ex().exl3_test_force(-1, -1, 0)
    assert np.array_equal(out[2], out[1]) and np.array_equal(out[2], out[0])


def test_gate_up_group_spread_equals_other_launches():
    """The {gate, up} group at 16 rows (272 blocks at S = 15: one block per CU
    and the 16 left blocks on spare waves) against the chained and the
    exchanged launch."""
    K = synth.HIDDEN
    ws_ = [G.upload(G.layer("spread-gu", n, K, synth.INTERMEDIATE, 4)) for n in ("gate", "up")]
    xd = G.dev_bf16(G.xbits("spread-gu", 16, K))
    auto = [G.host_u16(y) for y in G.run_group(ws_, xd, tag="gate+up auto")]
    for chained in (1, 0):
        ex().exl3_test_force(1, chained, 0)
        other = [G.host_u16(y) for y in G.run_group(ws_, xd, tag=f"gate+up chained={chained}")]
        ex().exl3_test_force(-1, -1, 0)
        assert all(np.array_equal(a, b) for a, b in zip(auto, other)), chained


def test_prompt_rows_equal_decode_rows():
    """A prompt of 300 rows (3 row blocks, ragged) against single-row calls."""
    K, N = 5120, 6144
    L = G.layer("prompt", "q", K, N, 4)
    w = G.upload(L)
    x = G.xbits("prompt", 300, K, sigma=0.5)
    xd = G.dev_bf16(x)
    full = G.host_u16(G.run(w, xd, M=300, tag="prompt 300"))
    for r in (0, 1, 127, 128, 200, 255, 256, 299):
        one = G.host_u16(G.run(w, xd[r:r + 1], M=1, tag=f"decode row {r}"))
        assert np.array_equal(one[0], full[r]), r
    # a 16-row window inside the prompt equals the same rows of the prompt
    win = G.host_u16(G.run(w, xd[128:144], M=16, tag="window"))
    assert np.array_equal(win, full[128:144])


@pytest.mark.parametrize("M", [1, 7, 16, 200, 1027])
def test_group_equals_each_member_alone(M):
    """PR #1467 exl3-midm: a {q, k, v} or {gate, up} group call gives, per
    member, the bytes of that member's solo call, at 1, 7, 16 and 200 prompt
    rows (two row blocks, the members' tiles side by side in one launch) and
    at 1027 rows, where the group's rotation launch reads each 4-row piece of
    X once for all members (a ragged last piece of 3 rows)."""
    K = synth.HIDDEN
    x = G.xbits("group", M, K)
    xd = G.dev_bf16(x)
    for names in (("q", "k", "v"), ("gate", "up")):
        cols = {"q": synth.Q_COLS, "k": synth.KV_COLS, "v": synth.KV_COLS,
                "gate": synth.INTERMEDIATE, "up": synth.INTERMEDIATE}
        layers = [G.layer("group", n, K, cols[n], 4) for n in names]
        ws_ = [G.upload(L) for L in layers]
        ys = G.run_group(ws_, xd, tag="+".join(names))
        for n, w, y in zip(names, ws_, ys):
            solo = G.host_u16(G.run(w, xd, tag=f"solo {n}"))
            assert np.array_equal(G.host_u16(y), solo), (names, n, M)


def test_group_planted_controls():
    """Planted controls: exchanging the scales (then the suh) of one group
    member for another's must change that member's bytes."""
    K, M = 5120, 7
    x = G.dev_bf16(G.xbits("control", M, K))
    a = G.layer("control", "a", K, 1024, 4)
    b = G.layer("control", "b", K, 1024, 4)
    wa, wb = G.upload(a), G.upload(b)
    ya, yb = [G.host_u16(t) for t in G.run_group([wa, wb], x, tag="control")]
    swapped = ex().Weight(wa.words, wb.scales, wa.suh, wa.svh, K, 1024, 4)
    assert not np.array_equal(G.host_u16(G.run_group([swapped, wb], x, tag="scales swapped")[0]), ya)
    swapped_suh = ex().Weight(wa.words, wa.scales, wb.suh, wa.svh, K, 1024, 4)
    assert not np.array_equal(G.host_u16(G.run_group([swapped_suh, wb], x, tag="suh swapped")[0]), ya)


def test_another_k_split_changes_bits():
    """Planted control 'another K split': forcing S away from the plan must
    change some bytes (so the bitwise tests can see a reduction-order change),
    while staying within the oracle tolerance."""
    K, N, M = 5120, 1024, 16
    L = G.layer("split", "k", K, N, 4)
    w = G.upload(L)
    x = G.xbits("split", M, K)
    xd = G.dev_bf16(x)
    base = G.host_u16(G.run(w, xd, tag="plan"))
    S = ex().exl3_plan(K, N, 4).splits
    other = 8 if S != 8 else 16
    ex().exl3_test_force(-1, -1, other)
    y = G.host_u16(G.run(w, xd, tag=f"forced S={other}"))
    ex().exl3_test_force(-1, -1, 0)
    assert not np.array_equal(y, base)
    G.assert_close(y, O.linear_packed(L.words, K, N, 4, L.scales, L.suh, L.svh, x), what="forced split")


def test_views_equal_full_head_columns():
    """PR #1507: span views of >= 64 blocks plan as the whole head, so their
    output is the head's output byte for byte; a 3-block view plans otherwise
    and is the control that goes red (against span B, over 128 rows). Full
    6-bit head 5120 -> 248,320, M = 16."""
    K, N, M = 5120, synth.VOCAB, 16
    L = G.layer("views", "head", K, N, 6)
    w = G.upload(L)
    xd = G.dev_bf16(G.xbits("views", M, K))
    full = G.host_u16(G.run(w, xd, tag="full head"))
    a = G.host_u16(G.run(w.columns(0, 98304), xd, tag="span A"))
    b = G.host_u16(G.run(w.columns(240128, 8192), xd, tag="span B"))
    assert np.array_equal(a, full[:, :98304])
    assert np.array_equal(b, full[:, 240128:])
    kept = b[:, 248032 - 240128:]
    assert kept.shape[1] == 288 and np.array_equal(kept, full[:, 248032:])
    # control: the 3-block tail plans otherwise; over 128 rows (49,152
    # outputs) some bf16 output moves with the summation order
    assert ex().exl3_plan(K, 384, 6).splits != ex().exl3_plan(K, N, 6).splits
    x128 = G.dev_bf16(G.xbits("views", 128, K))
    b128 = G.host_u16(G.run(w.columns(240128, 8192), x128, tag="span B, 128 rows"))
    tail3 = G.host_u16(G.run(w.columns(248320 - 384, 384), x128, tag="3-block tail, 128 rows"))
    assert not np.array_equal(tail3, b128[:, -384:])


def test_prompt_rows_of_an_odd_view_equal_full_head():
    """Prompt rows over a view that starts at an odd block and spans an odd
    number of blocks (65 of the 6-bit head, so it plans as the head does):
    the 128-row tiles two blocks wide pair other blocks than in the full
    head, and the last tile holds one block. 200 rows, bitwise against the
    full head's columns."""
    K, N, M = 5120, synth.VOCAB, 200
    L = G.layer("views", "head", K, N, 6)
    w = G.upload(L)
    xd = G.dev_bf16(G.xbits("views-prompt", M, K, sigma=0.5))
    full = G.host_u16(G.run(w, xd, tag="full head, 200 rows"))
    v = G.host_u16(G.run(w.columns(128, 65 * 128), xd, tag="65-block view from block 1, 200 rows"))
    assert ex().exl3_plan(K, 65 * 128, 6).splits == ex().exl3_plan(K, N, 6).splits
    assert np.array_equal(v, full[:, 128:128 + 65 * 128])


def test_counters_zero_at_rest_and_repeats_identical():
    """Counters are reset by each block's last arriver: zero after every call
    without any memset between calls; 200 repeats give identical bytes."""
    torch = G.torch_mod()
    K, N = 5120, 1024
    L = G.layer("repeat", "k", K, N, 4)
    w = G.upload(L)
    xd = G.dev_bf16(G.xbits("repeat", 16, K))
    ws = ex().Workspace().reserve([w], 128)
    first = None
    for it in range(200):
        y = G.empty_y(16, N)
        if it % 50 == 0:
            G.say(f"repeat {it}")
        ex().exl3_linear(w, xd, y, ws)
        if first is None:
            first = G.host_u16(y)
        elif it % 20 == 0 or it == 199:
            assert np.array_equal(G.host_u16(y), first), it
    torch.cuda.synchronize()
    assert int(ws.counters().abs().sum()) == 0
    # other row counts through the same workspace: still zero at rest
    for M in (1, 17, 64, 128):
        y = G.empty_y(M, N)
        ex().exl3_linear(w, G.dev_bf16(G.xbits("repeat", M, K)), y, ws)
        torch.cuda.synchronize()
        assert int(ws.counters().abs().sum()) == 0, M


def test_two_streams_equal_solo():
    """Concurrent == solo: two streams with their own workspaces."""
    torch = G.torch_mod()
    K = 5120
    La, Lb = G.layer("streams", "a", K, 1024, 4), G.layer("streams", "b", K, 6144, 4)
    wa, wb = G.upload(La), G.upload(Lb)
    xd = G.dev_bf16(G.xbits("streams", 16, K))
    solo_a = G.host_u16(G.run(wa, xd, tag="solo a"))
    solo_b = G.host_u16(G.run(wb, xd, tag="solo b"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1 = ex().Workspace().reserve([wa], 16, stream=s1)
    ws2 = ex().Workspace().reserve([wb], 16, stream=s2)
    torch.cuda.synchronize()
    ya, yb = G.empty_y(16, 1024), G.empty_y(16, 6144)
    G.say("two streams x 50")
    for _ in range(50):
        ex().exl3_linear(wa, xd, ya, ws1, stream=s1)
        ex().exl3_linear(wb, xd, yb, ws2, stream=s2)
    torch.cuda.synchronize()
    assert np.array_equal(G.host_u16(ya), solo_a) and np.array_equal(G.host_u16(yb), solo_b)


def test_split_exchange_stress():
    """Race check of the counter protocol: 2000 back-to-back calls of a narrow
    weight (the plan's 16 splits per block, exchange through partials) on one stream,
    bytes compared every 100 calls and counters zero at the end."""
    torch = G.torch_mod()
    K, N = 5120, 1024
    L = G.layer("stress", "k", K, N, 4)
    w = G.upload(L)
    xd = G.dev_bf16(G.xbits("stress", 16, K))
    ex().exl3_test_force(-1, 0, 0)
    ws = ex().Workspace().reserve([w], 16)
    ref = G.host_u16(G.run(w, xd, ws=ws, tag="stress ref"))
    ys = [G.empty_y(16, N) for _ in range(100)]
    for rep in range(20):
        G.say(f"stress batch {rep}")
        for y in ys:
            ex().exl3_linear(w, xd, y, ws)
        torch.cuda.synchronize()
        for y in ys:
            assert np.array_equal(G.host_u16(y), ref), rep
    ex().exl3_test_force(-1, -1, 0)
    assert int(ws.counters().abs().sum()) == 0


TWO_PHASE = [(1, (-1, -1, 0)), (16, (-1, -1, 0)), (16, (1, 2, 4)), (7, (1, 3, 0)), (16, (1, 0, 0)),
             (40, (-1, -1, 0)), (64, (-1, -1, 0)), (100, (-1, -1, 0)), (128, (-1, -1, 0)), (128, (8, 0, 0)),
             (200, (-1, -1, 0))]


@pytest.mark.parametrize("M,force", TWO_PHASE)
def test_two_phase_calls_equal_the_group_call(M, force):
    """exl3_rotate then exl3_linear_rotated give the bytes of one
    exl3_linear_group call: the rotation writes Xr in the layout the linear
    launch of that row count reads (chunk-major for the spread launch, forced
    here with 4 splits at 16 rows, for the exchanged column halves, forced at
    7 rows, and for the 128-row tilings at 100, 128 and 200 rows, chained and
    exchanged; row-major for the other 16- to 64-row launches, such as the
    exchanged 16-row form forced at 16 rows)."""
    torch = G.torch_mod()
    K = 5120
    layers = [G.layer("two-phase", n, K, N, 3) for n, N in (("gate", 2048), ("up", 2048), ("k", 1024))]
    ws_list = [G.upload(L) for L in layers]
    xd = G.dev_bf16(G.xbits("two-phase", M, K))
    ex().exl3_test_force(*force)
    ws = ex().Workspace().reserve(ws_list, M)
    one = [G.host_u16(y) for y in G.run_group(ws_list, xd, M=M, ws=ws, tag=f"group call {force}")]
    ys = [G.empty_y(M, L.N) for L in layers]
    G.say(f"exl3_rotate + exl3_linear_rotated M={M}")
    ex().exl3_rotate(ws_list, xd, ws, M=M)
    ex().exl3_linear_rotated(ws_list, ys, ws, M)
    torch.cuda.synchronize()
    for j, y in enumerate(ys):
        assert np.array_equal(G.host_u16(y), one[j]), (M, j)
    assert int(ws.counters().abs().sum()) == 0


def test_spread_launch_over_several_row_blocks():
    """The {gate, up} pair (272 blocks at S = 15) at 17-32 rows runs the
    spread launch once per 16-row block in one grid (the left blocks'
    partials and counters per row block), and forced at 40, 48 and 64 rows
    (where the automatic choice is the 128-row block tiling with its left
    blocks): byte for byte the automatic launch, the chained 16-row launch
    and the exchanged one, counters zero afterwards."""
    K = synth.HIDDEN
    ws_ = [G.upload(G.layer("spread-rb", n, K, synth.INTERMEDIATE, 3)) for n in ("gate", "up")]
    xd = G.dev_bf16(G.xbits("spread-rb", 64, K))
    ws = ex().Workspace().reserve(ws_, 64)
    for M in (17, 31, 32, 40, 48, 64):
        ex().exl3_test_force(*((1, 2, 0) if M > 32 else (-1, -1, 0)))
        ws.reserve(ws_, M)                                  # forced above 32 rows: that launch's workspace
        auto = [G.host_u16(y) for y in G.run_group(ws_, xd, M=M, ws=ws, tag="spread over row blocks")]
        ex().exl3_test_force(-1, -1, 0)
        assert int(ws.counters().abs().sum()) == 0, M
        for force in ((1, 1, 0), (1, 0, 0), (-1, -1, 0)):
            ex().exl3_test_force(*force)
            ws.reserve(ws_, M)
            other = [G.host_u16(y) for y in G.run_group(ws_, xd, M=M, ws=ws, tag=f"forced {force}")]
            ex().exl3_test_force(-1, -1, 0)
            assert all(np.array_equal(a, b) for a, b in zip(auto, other)), (M, force)


@pytest.mark.parametrize("what,K,Ns,bits,rows", [
    ("{gate, up} pair with left blocks", synth.HIDDEN, (synth.INTERMEDIATE, synth.INTERMEDIATE), 3, (33, 48, 64)),
    ("a 300-block weight, no left blocks", 1024, (300 * 128,), 6, (49, 64)),
    ("a 600-block weight at 17-32 rows", 1024, (600 * 128,), 6, (17, 24, 32))])
def test_64_row_block_tiling_equals_the_128_row_one(what, K, Ns, bits, rows):
    """Chained block tilings of at most 64 rows run 64-row workgroups, of at
    most 32 rows 32-row ones: with left blocks (the {gate, up} pair, 272
    blocks at 33-64 rows) and without (300 blocks of 8 splits at 49 and 64
    rows, two workgroups on some CUs; 600 blocks at 17-32 rows, where the
    16-row form over row blocks would exceed 1024 workgroups). Forced to
    128-row workgroups (the same left blocks and split-fold launch) they give
    the same bytes; sampled blocks (first, last, random, and the blocks past
    one per CU) against the oracle."""
    layers = [G.layer("block64", f"m{j}", K, N, bits) for j, N in enumerate(Ns)]
    ws_ = [G.upload(L) for L in layers]
    x = G.xbits("block64", max(rows), K)
    xd = G.dev_bf16(x)
    for M in rows:
        ys = G.run_group(ws_, xd, M=M, tag=f"{what}, 64-row workgroups")
        assert ex().exl3_test_last_form() == f"linear_block{32 if M <= 32 else 64}_kernel<{bits}>", M
        auto = [G.host_u16(y) for y in ys]
        ex().exl3_test_force(8, 1, 0)
        try:
            forced = [G.host_u16(y) for y in G.run_group(ws_, xd, M=M, tag=f"{what}, 128-row workgroups")]
            assert ex().exl3_test_last_form() == f"linear_block_kernel<{bits}, true>", M
        finally:
            ex().exl3_test_force(-1, -1, 0)
        assert all(np.array_equal(a, b) for a, b in zip(auto, forced)), M
        first = 0
        for j, (L, y) in enumerate(zip(layers, ys)):
            nb = L.N // 128
            blocks = sorted(set(G.sample_blocks(nb, k=3, seed=M + j)) | {b for b in range(nb) if 256 <= first + b < 320})
            first += nb
            G.assert_close(G.gpu_blocks(y, blocks), G.oracle_blocks(L, x[:M], blocks), what=f"{what} M={M} member {j}")


def test_split_fold_launch_equals_the_chained_fold():
    """Down-shaped weight (K 17408: long splits) at 100, 128 and 200 rows
    (two row blocks): the exchanged 2 x 2 tiling whose partials the
    split-fold launch adds gives the bytes of the chained 128-row block
    tiling (every split folded in one workgroup), in 128-row tiles (forced)
    and in the automatic 64-row tiles; with a forced plan of 17 splits the
    tiling folds in its last arriving workgroup instead, again byte for byte
    the chained form. Counters zero afterwards."""
    K, N = 17408, 1024
    L = G.layer("split-fold", "down", K, N, 4)
    w = G.upload(L)
    xd = G.dev_bf16(G.xbits("split-fold", 200, K))
    ws = ex().Workspace().reserve([w], 200)
    for M in (100, 128, 200):
        for S in (0, 17):
            ys = {}
            for chained in (0, 1):
                ex().exl3_test_force(8, chained, S)
                ws.reserve([w], M)
                ys[chained] = G.host_u16(G.run(w, xd, M=M, ws=ws, tag=f"split fold M={M} S={S} chained={chained}"))
                form = ex().exl3_test_last_form()
                ex().exl3_test_force(-1, -1, 0)
                assert form == ("linear_tile_kernel<4, false>" if chained == 0 else "linear_block_kernel<4, true>"), form
            assert np.array_equal(ys[0], ys[1]), (M, S)
            assert int(ws.counters().abs().sum()) == 0, (M, S)
            if S == 0 and M <= 128:
                # the automatic launch: the same tiling in 64-row tiles of 2 waves
                ws.reserve([w], M)
                y64 = G.host_u16(G.run(w, xd, M=M, ws=ws, tag=f"split fold M={M} automatic"))
                assert ex().exl3_test_last_form() == "linear_tile64_kernel<4>"
                assert np.array_equal(y64, ys[1]), M


@pytest.mark.parametrize("N", [384, 640, 1152])
def test_exchanged_launch_with_blocks_across_xcd_ranges(N):
    """Exchanged 16- and 32-row launches deal their workgroups to the XCDs
    in contiguous ranges; with 3, 5 or 9 blocks a block's split groups fall
    into two ranges. Every exchanged form (one split per wave, the column
    halves, 32-row tiles) gives the bytes of the chained form, at 1, 16 and
    17 rows, and leaves the counters at zero."""
    K = 5120
    L = G.layer("xcd-ranges", f"w{N}", K, N, 4)
    w = G.upload(L)
    xd = G.dev_bf16(G.xbits("xcd-ranges", 32, K))
    ws = ex().Workspace().reserve([w], 32)
    for M in (1, 16, 17):
        ys = {}
        for mt, chained in ((1, 1), (1, 0), (1, 3), (2, 0), (2, 1)):
            if M > 16 and mt == 1:
                continue
            ex().exl3_test_force(mt, chained, 0)
            ws.reserve([w], M)
            ys[(mt, chained)] = G.host_u16(G.run(w, xd, M=M, ws=ws, tag=f"N={N} M={M} m_tiles={mt} chained={chained}"))
            ex().exl3_test_force(-1, -1, 0)
        ref = ys[(1, 1)] if M <= 16 else ys[(2, 1)]
        for k, y in ys.items():
            assert np.array_equal(y[:M], ref[:M]), (N, M, k)
        assert int(ws.counters().abs().sum()) == 0, (N, M)
