"""Host logic of libexl3.so, on the CPU (no kernel runs here).

The library loads without a GPU; plan, views, workspace sizing and every
argument check are host code. With the mock driver on, launches and counter
fills are recorded instead of issued, so the launch/fill accounting of the
pages' host tests can be checked here (TensorFold PR #1475: counters zeroed
on the call's stream only when they grow; PR #1467: after reserve a call
allocates nothing and zeroes nothing).
"""

import ctypes
import os
import re

import pytest

import trellis_quantized_linear_amd.exl3 as ex
from trellis_quantized_linear_amd import synth


@pytest.fixture(scope="module")
def lib():
    return ex.lib()


@pytest.fixture(autouse=True)
def _reset_hooks(lib):
    ex.exl3_test_force(-1, -1, 0)
    ex.exl3_test_mock(False)
    ex.exl3_test_mock_counts()
    yield
    ex.exl3_test_force(-1, -1, 0)
    ex.exl3_test_mock(False)
    ex.exl3_test_mock_counts()


def fake_weight(K, N, bits, base=0x10000000, block_stride=None):
    """A descriptor with plausible (never dereferenced) device addresses."""
    bs = block_stride if block_stride is not None else 16 * K * bits
    d = ex.exl3_weight_t(base, base + 0x4000000, base + 0x8000000, base + 0xC000000, K, N, bs, bits, 0)
    return ex.Weight(None, None, None, None, K, N, bits, _desc=d)


def test_exports_every_declared_symbol(lib):
    text = open(ex.HEADER).read()
    names = sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(exl3_\w+)\s*\(", text, re.M)))
    assert len(names) == 21
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ex._SIGNATURES), set(names) ^ set(ex._SIGNATURES)


def test_plan_basic_and_m_independent(lib):
    p = ex.exl3_plan(5120, 6144, 4)
    assert p.waves == 4 and p.chunks == 160 and p.n_blocks == 48
    # the plan takes no row count: the same for every caller at any M
    assert ex.exl3_plan(5120, 6144, 4).splits == p.splits


def test_plan_wide_threshold_head_views(lib):
    """PR #1507: the 98,304-column span and the 64-block tail plan as the whole
    248,320-column head; a 3-block (384-column) tail does not ('expected 1,
    found 8' on the pages)."""
    head = ex.exl3_plan(5120, 248320, 6).splits
    assert ex.exl3_plan(5120, 98304, 6).splits == head
    assert ex.exl3_plan(5120, 8192, 6).splits == head
    assert ex.exl3_plan(5120, 64 * 128, 6).splits == head
    assert ex.exl3_plan(5120, 384, 6).splits != head
    assert ex.exl3_plan(5120, 63 * 128, 6).splits != head or head == 1


def test_plan_every_wide_n_equal(lib):
    for K in (256, 1024, 5120, 17408):
        s = {ex.exl3_plan(K, nb * 128, 4).splits for nb in (64, 65, 100, 136, 768, 1940, 4096)}
        assert len(s) == 1, (K, s)


def test_plan_table_fills_the_gpu(lib):
    """Narrow weights split until about two splits per SIMD (n_blocks * S >=
    512), at most 16 ways, keeping >= 4 chunks per split; wide ones take
    S_wide(K) = 15 (15 chains and a spare wave per 16-wave workgroup) unless
    that leaves fewer than 4 chunks per split."""
    for K, N in ((5120, 1024), (5120, 6144), (17408, 5120), (256, 256), (1024, 384)):
        p = ex.exl3_plan(K, N, 4)
        assert p.n_blocks < 64
        assert p.n_blocks * p.splits >= 512 or p.splits == 16 or p.chunks // (2 * p.splits) < 4
        assert p.chunks // p.splits >= 4 or p.splits == 1
    for K, want in ((128, 1), (1024, 8), (1920, 15), (5120, 15), (17408, 15)):
        p = ex.exl3_plan(K, 64 * 128, 4)
        assert p.splits == want, (K, p.splits)
        assert p.chunks // p.splits >= 4 or p.splits == 1
    assert ex.exl3_plan(5120, 248320, 6).splits == 15
    assert ex.exl3_plan(5120, 17408, 4).splits == 15
    assert ex.exl3_plan(5120, 1024, 4).splits == 16


def test_plan_errors(lib):
    out = ex.exl3_plan_t()
    assert lib.exl3_plan(5120, 6144, 1, ctypes.byref(out)) == ex.EXL3_EBITS
    assert lib.exl3_plan(5120, 6144, 9, ctypes.byref(out)) == ex.EXL3_EBITS
    assert lib.exl3_plan(5000, 6144, 4, ctypes.byref(out)) == ex.EXL3_EALIGN
    assert lib.exl3_plan(5120, 6100, 4, ctypes.byref(out)) == ex.EXL3_EALIGN
    assert lib.exl3_plan(0, 128, 4, ctypes.byref(out)) == ex.EXL3_EALIGN
    assert lib.exl3_plan(5120, 6144, 4, None) == ex.EXL3_EINVAL


def test_view_keeps_parent_strides_and_moves_to_first_block(lib):
    """PR #1507 host test: a view's descriptor carries the full weight's
    block stride, and its pointers start at the view's first 128-column
    block."""
    w = fake_weight(5120, 248320, 6)
    v = w.columns(240128, 8192)
    bs = 16 * 5120 * 6
    assert v.desc.block_stride == w.desc.block_stride == bs
    assert v.desc.words == w.desc.words + (240128 // 128) * bs
    assert v.desc.scales == w.desc.scales + 2 * 240128
    assert v.desc.svh == w.desc.svh + 2 * 240128
    assert v.desc.suh == w.desc.suh
    assert v.desc.K == 5120 and v.desc.N == 8192 and v.desc.bits == 6
    # a view of a view composes
    vv = v.columns(128, 256)
    assert vv.desc.words == w.desc.words + (240128 // 128 + 1) * bs and vv.desc.N == 256


def test_view_errors(lib):
    w = fake_weight(512, 1024, 4)
    out = ex.exl3_weight_t()
    f = lib.exl3_weight_columns
    assert f(ctypes.byref(w.desc), 64, 128, ctypes.byref(out)) == ex.EXL3_EALIGN
    assert f(ctypes.byref(w.desc), 0, 100, ctypes.byref(out)) == ex.EXL3_EALIGN
    assert f(ctypes.byref(w.desc), 896, 256, ctypes.byref(out)) == ex.EXL3_ERANGE
    assert f(ctypes.byref(w.desc), 0, 0, ctypes.byref(out)) == ex.EXL3_EINVAL
    assert f(ctypes.byref(w.desc), -128, 128, ctypes.byref(out)) == ex.EXL3_EINVAL
    assert f(None, 0, 128, ctypes.byref(out)) == ex.EXL3_EINVAL
    assert f(ctypes.byref(w.desc), 0, 1024, ctypes.byref(out)) == ex.EXL3_OK


def test_descriptor_errors(lib):
    ws = ex.exl3_workspace_t(0x20000000, 1 << 30, 1 << 20)
    x, y = 0x30000000, 0x40000000

    def call(d, M=4, ldx=None, ldy=None):
        return lib.exl3_linear(ctypes.byref(d), x, ldx or d.K, M, y, ldy or d.N, ctypes.byref(ws), None)

    ex.exl3_test_mock(True)
    good = fake_weight(512, 256, 4).desc
    assert call(good) == ex.EXL3_OK
    for field, val, code in (("bits", 1, ex.EXL3_EBITS), ("bits", 9, ex.EXL3_EBITS), ("K", 500, ex.EXL3_EALIGN),
                             ("N", 200, ex.EXL3_EALIGN), ("block_stride", 100, ex.EXL3_EALIGN),
                             ("words", 0x10000002, ex.EXL3_EALIGN), ("scales", 0x10000001, ex.EXL3_EALIGN),
                             ("words", 0, ex.EXL3_EINVAL), ("flags", 1, ex.EXL3_EINVAL)):
        d = fake_weight(512, 256, 4).desc
        setattr(d, field, val)
        assert call(d) == code, (field, val)
    assert call(good, M=-1) == ex.EXL3_EINVAL
    assert call(good, ldx=256) == ex.EXL3_EINVAL
    assert call(good, ldy=128) == ex.EXL3_EINVAL
    assert lib.exl3_linear(ctypes.byref(good), x + 1, 512, 4, y, 256, ctypes.byref(ws), None) == ex.EXL3_EALIGN
    assert lib.exl3_linear(ctypes.byref(good), None, 512, 4, y, 256, ctypes.byref(ws), None) == ex.EXL3_EINVAL
    assert lib.exl3_linear(ctypes.byref(good), x, 512, 4, None, 256, ctypes.byref(ws), None) == ex.EXL3_EINVAL
    assert lib.exl3_linear(ctypes.byref(good), x, 512, 4, y, 256, None, None) == ex.EXL3_EWORKSPACE
    launches, fills, _, _ = ex.exl3_test_mock_counts()
    assert launches == 2 and fills == 0      # only the one good call launched (rotation + linear)


def test_m_zero_launches_nothing(lib):
    ex.exl3_test_mock(True)
    d = fake_weight(512, 256, 4).desc
    ws = ex.exl3_workspace_t(0, 0, 0)        # not even a workspace is needed
    assert lib.exl3_linear(ctypes.byref(d), 0x30000000, 512, 0, 0x40000000, 256, ctypes.byref(ws), None) == 0
    assert ex.exl3_test_mock_counts()[:2] == (0, 0)


def test_group_errors(lib):
    ex.exl3_test_mock(True)
    a = fake_weight(5120, 6144, 4)
    b = fake_weight(5120, 1024, 4, base=0x50000000)
    c = fake_weight(5120, 1024, 3, base=0x60000000)
    d = fake_weight(4096, 1024, 4, base=0x70000000)
    need, _ = ex.exl3_workspace_need([a, b, b], 16)
    ws = ex.exl3_workspace_t(0x20000000, need + (1 << 20), 1 << 20)

    def group(members, M=16):
        arr = ex._wlist(members)
        ys = (ctypes.c_void_p * len(members))(*[0x80000000] * len(members))
        ld = (ctypes.c_int64 * len(members))(*[m.N for m in members])
        return lib.exl3_linear_group(len(members), arr, 0x30000000, 5120, M, ys, ld, ctypes.byref(ws), None)

    assert group([a, b, b]) == ex.EXL3_OK
    assert group([a, c]) == ex.EXL3_EGROUP          # different bits
    assert group([a, d]) == ex.EXL3_EGROUP          # different K
    assert group([a, b, b, b]) == ex.EXL3_EGROUP    # more than three
    assert lib.exl3_linear_group(0, None, 0x30000000, 5120, 16, None, None, ctypes.byref(ws), None) == ex.EXL3_EGROUP
    launches, fills, _, _ = ex.exl3_test_mock_counts()
    assert launches == 2 and fills == 0             # one rotation + one linear for the whole group


def test_workspace_zeroed_once_per_growth_on_the_given_stream(lib):
    """PR #1475 host test: one fill per growth, on the named stream, and none
    while the buffer is big enough; linear calls never fill."""
    ex.exl3_test_mock(True)
    w = fake_weight(5120, 1024, 4)
    need, cb = ex.exl3_workspace_need([w], 16)
    assert cb > 0 and need > cb
    ws = ex.exl3_workspace_t(0, 0, 0)
    stream = 0xABC000
    assert lib.exl3_workspace_grow(ctypes.byref(ws), 0x20000000, need, cb, stream) == ex.EXL3_OK
    launches, fills, fbytes, s = ex.exl3_test_mock_counts()
    assert (launches, fills, fbytes, s) == (0, 1, cb, stream)
    # the same size again is not a growth: refused, nothing issued
    assert lib.exl3_workspace_grow(ctypes.byref(ws), 0x21000000, need, cb, stream) == ex.EXL3_EWORKSPACE
    assert ex.exl3_test_mock_counts()[:2] == (0, 0)
    # steady state: every call at 1..16 rows launches two kernels, fills nothing
    for M in range(1, 17):
        assert lib.exl3_linear(ctypes.byref(w.desc), 0x30000000, 5120, M, 0x40000000, 1024, ctypes.byref(ws),
                               0x123000) == 0
    launches, fills, _, s = ex.exl3_test_mock_counts()
    assert launches == 32 and fills == 0 and s == 0x123000
    # a larger buffer grows once more, again on the named stream
    assert lib.exl3_workspace_grow(ctypes.byref(ws), 0x22000000, 2 * need, 2 * cb, 0xDEF000) == ex.EXL3_OK
    assert ex.exl3_test_mock_counts()[1:] == (1, 2 * cb, 0xDEF000)


def test_workspace_too_small_is_refused(lib):
    ex.exl3_test_mock(True)
    w = fake_weight(5120, 1024, 4)
    need, cb = ex.exl3_workspace_need([w], 16)
    ws = ex.exl3_workspace_t(0x20000000, need - 256, cb)
    assert lib.exl3_linear(ctypes.byref(w.desc), 0x30000000, 5120, 16, 0x40000000, 1024, ctypes.byref(ws),
                           None) == ex.EXL3_EWORKSPACE
    ws = ex.exl3_workspace_t(0x20000000, need, 0)
    assert lib.exl3_linear(ctypes.byref(w.desc), 0x30000000, 5120, 16, 0x40000000, 1024, ctypes.byref(ws),
                           None) == ex.EXL3_EWORKSPACE
    assert ex.exl3_test_mock_counts()[0] == 0


def test_workspace_for_max_rows_covers_smaller_calls(lib):
    """A workspace of exactly the size exl3_workspace_need reports for
    max_rows accepts every call of 1..max_rows rows, across the regime
    boundaries (decode, mid-M, prompt)."""
    ex.exl3_test_mock(True)
    shapes = [(5120, 1024), (5120, 6144), (5120, 17408), (17408, 5120), (5120, 248320), (256, 256)]
    for K, N in shapes:
        w = fake_weight(K, N, 4)
        for max_rows in (16, 100, 128, 300, 8192):
            need, cb = ex.exl3_workspace_need([w], max_rows)
            ws = ex.exl3_workspace_t(0x20000000, need, cb)
            for M in sorted({1, 7, 16, 17, 33, 64, 100, 128, 129, 256, max_rows}):
                if M > max_rows:
                    continue
                rc = lib.exl3_linear(ctypes.byref(w.desc), 0x30000000, K, M, 0x40000000, N, ctypes.byref(ws), None)
                assert rc == 0, (K, N, max_rows, M, rc)
    ex.exl3_test_mock_counts()


def test_group_workspace_for_max_rows_covers_smaller_calls(lib):
    """The same for groups, at every row count where the automatic choice
    changes form (the {gate, up} pair takes the spread launch up to 32 rows,
    over several 16-row blocks above 16, then the 128-row block tiling; the
    {q, k, v} group the 16-row forms, then 128-row tiles)."""
    ex.exl3_test_mock(True)
    groups = [[fake_weight(5120, 17408, b), fake_weight(5120, 17408, b, base=0x50000000)] for b in (3, 4)]
    groups.append([fake_weight(5120, 6144, 4), fake_weight(5120, 1024, 4, base=0x50000000),
                   fake_weight(5120, 1024, 4, base=0x60000000)])
    rows = (1, 7, 16, 17, 24, 32, 33, 40, 47, 48, 49, 64, 65, 96, 97, 100, 128, 129, 256)
    for ws_ in groups:
        n = len(ws_)
        arr = ex._wlist(ws_)
        ys = (ctypes.c_void_p * n)(*[0x80000000 + 0x10000000 * j for j in range(n)])
        ld = (ctypes.c_int64 * n)(*[w.N for w in ws_])
        for max_rows in (16, 32, 40, 48, 64, 100, 128, 300):
            need, cb = ex.exl3_workspace_need(ws_, max_rows)
            ws = ex.exl3_workspace_t(0x20000000, need, cb)
            for M in sorted(set(rows) | {max_rows}):
                if M > max_rows:
                    continue
                rc = lib.exl3_linear_group(n, arr, 0x30000000, 5120, M, ys, ld, ctypes.byref(ws), None)
                assert rc == 0, ([w.N for w in ws_], max_rows, M, rc)
    ex.exl3_test_mock_counts()


def test_workspace_grow_errors(lib):
    ws = ex.exl3_workspace_t(0, 0, 0)
    assert lib.exl3_workspace_grow(ctypes.byref(ws), 0x20000001, 1024, 256, None) == ex.EXL3_EALIGN
    assert lib.exl3_workspace_grow(ctypes.byref(ws), 0x20000000, 1024, 100, None) == ex.EXL3_EALIGN
    assert lib.exl3_workspace_grow(ctypes.byref(ws), 0x20000000, 256, 512, None) == ex.EXL3_EWORKSPACE
    assert lib.exl3_workspace_grow(None, 0x20000000, 1024, 256, None) == ex.EXL3_EINVAL
    assert lib.exl3_workspace_grow(ctypes.byref(ws), None, 1024, 256, None) == ex.EXL3_EINVAL


def test_rotate_and_linear_rotated_are_one_launch_each(lib):
    ex.exl3_test_mock(True)
    a = fake_weight(5120, 6144, 4)
    b = fake_weight(5120, 1024, 4, base=0x50000000)
    need, cb = ex.exl3_workspace_need([a, b], 16)
    ws = ex.exl3_workspace_t(0x20000000, need, cb)
    arr = ex._wlist([a, b])
    ys = (ctypes.c_void_p * 2)(0x80000000, 0x90000000)
    ld = (ctypes.c_int64 * 2)(6144, 1024)
    assert lib.exl3_rotate(2, arr, 0x30000000, 5120, 16, ctypes.byref(ws), 0x777000) == 0
    assert ex.exl3_test_mock_counts()[0] == 1
    assert lib.exl3_linear_rotated(2, arr, 16, ys, ld, ctypes.byref(ws), 0x777000) == 0
    launches, fills, _, s = ex.exl3_test_mock_counts()
    assert (launches, fills, s) == (1, 0, 0x777000)
    # each phase checks only what it uses
    assert lib.exl3_rotate(2, arr, None, 5120, 16, ctypes.byref(ws), None) == ex.EXL3_EINVAL
    assert lib.exl3_linear_rotated(2, arr, 16, None, ld, ctypes.byref(ws), None) == ex.EXL3_EINVAL
    assert lib.exl3_linear_rotated(2, arr, 16, ys, ld, None, None) == ex.EXL3_EWORKSPACE


def test_rotation_runs_inside_the_linear_launch_up_to_32_rows(lib):
    """Launch-gap removal (PR #1467, "What this changes": the rotations and
    decode-row linears chained without a gap), opt-in: with it on, a call
    whose launch is one row block of at most 32 rows (the 16-row forms; the
    32-row tiling, here forced at 17..32 rows, where the automatic choice
    takes two 16-row blocks) is one launch and everything else two; off (the
    default), two everywhere. The counter region holds the chunk flags either
    way (one word per member and 128 columns of K, plus a count)."""
    ex.exl3_test_mock(True)
    a = fake_weight(5120, 6144, 4)
    b = fake_weight(5120, 1024, 4, base=0x50000000)
    arr = ex._wlist([a, b, b])
    ys = (ctypes.c_void_p * 3)(0x80000000, 0x90000000, 0xA0000000)
    ld = (ctypes.c_int64 * 3)(6144, 1024, 1024)
    need, cb = ex.exl3_workspace_need([a, b, b], 300)
    ws = ex.exl3_workspace_t(0x20000000, need, cb)

    def launches(M):
        assert lib.exl3_linear_group(3, arr, 0x30000000, 5120, M, ys, ld, ctypes.byref(ws), None) == 0
        return ex.exl3_test_mock_counts()[0]

    for M in (1, 16, 32, 33):
        assert launches(M) == 2, M
    ex.exl3_test_fuse_rotation(True)
    try:
        for M in (1, 7, 16):
            assert launches(M) == 1, M
        for M in (17, 32, 33, 64, 128, 300):
            assert launches(M) == 2, M
        ex.exl3_test_force(2, -1, 0)
        for M in (17, 32):
            assert launches(M) == 1, M
        ex.exl3_test_force(-1, -1, 0)
        # the {gate, up} pair: one launch at 16 rows (spread launch, one row
        # block); at 17-32 rows the spread launch covers several row blocks
        # and keeps its rotation launch; at 33 and 48 rows the 64-row block
        # tiling with its left blocks (rotation, tiling, split fold)
        g = fake_weight(5120, 17408, 4, base=0x60000000)
        u = fake_weight(5120, 17408, 4, base=0x70000000)
        gu = ex._wlist([g, u])
        need2, cb2 = ex.exl3_workspace_need([g, u], 48)
        ws2 = ex.exl3_workspace_t(0x20000000, need2, cb2)
        ys2 = (ctypes.c_void_p * 2)(0x80000000, 0x90000000)
        ld2 = (ctypes.c_int64 * 2)(17408, 17408)
        for M, n in ((16, 1), (17, 2), (32, 2), (33, 3), (48, 3)):
            assert lib.exl3_linear_group(2, gu, 0x30000000, 5120, M, ys2, ld2, ctypes.byref(ws2), None) == 0
            assert ex.exl3_test_mock_counts()[0] == n, M
        # the two-phase calls never fuse
        assert lib.exl3_rotate(3, arr, 0x30000000, 5120, 16, ctypes.byref(ws), None) == 0
        assert lib.exl3_linear_rotated(3, arr, 16, ys, ld, ctypes.byref(ws), None) == 0
        assert ex.exl3_test_mock_counts()[0] == 2
    finally:
        ex.exl3_test_fuse_rotation(False)
    # flags: 3 members x 40 chunks + the count, on top of the split counters
    # of the 16-row exchanged launch (64 blocks, counters of one row block)
    _, cb16 = ex.exl3_workspace_need([a, b, b], 16)
    assert cb16 >= 4 * (64 + 1 + 3 * 40)
    assert lib.exl3_test_fuse_rotation(2, -1) == ex.EXL3_EINVAL
    assert lib.exl3_test_fuse_rotation(1, -2) == ex.EXL3_EINVAL
    assert lib.exl3_test_fuse_rotation(1, 0) == ex.EXL3_OK
    assert lib.exl3_test_fuse_rotation(0, -1) == ex.EXL3_OK


def test_strerror_covers_every_code(lib):
    for code in range(0, -8, -1):
        assert lib.exl3_strerror(code) != b"unknown error"
    assert lib.exl3_strerror(-99) == b"unknown error"


def test_test_force_validation(lib):
    assert lib.exl3_test_force(3, -1, 0) == ex.EXL3_EINVAL
    assert lib.exl3_test_force(-1, 4, 0) == ex.EXL3_EINVAL
    assert lib.exl3_test_force(1, 3, 0) == ex.EXL3_OK
    assert lib.exl3_test_force(-1, -1, -1) == ex.EXL3_EINVAL
    assert lib.exl3_test_force(8, 1, 4) == ex.EXL3_OK
    assert lib.exl3_test_force(16, 1, 0) == ex.EXL3_OK
    assert lib.exl3_test_force(32, 1, 0) == ex.EXL3_EINVAL
    assert lib.exl3_set_prompt_arithmetic(2) == ex.EXL3_EINVAL
    assert lib.exl3_set_prompt_arithmetic(0) == ex.EXL3_OK


def test_dispatch_sweep_reaches_only_built_forms(lib):
    """The pages' dispatch sweep (PR #1467 follow-up): K, N in 128..16384 at
    1..128 rows through the host dispatch; every call must be
    accepted (the kernel table covers every width x row tiling x launch
    shape), with a workspace sized by exl3_workspace_need."""
    ex.exl3_test_mock(True)
    for bits in (2, 3, 4, 5, 6, 7, 8):
        for K in (128, 512, 1408, 5120, 16384):
            for N in (128, 1024, 8192, 16384):
                w = fake_weight(K, N, bits)
                need, cb = ex.exl3_workspace_need([w], 128)
                ws = ex.exl3_workspace_t(0x20000000, need, cb)
                for M in (1, 16, 17, 48, 49, 128):
                    rc = lib.exl3_linear(ctypes.byref(w.desc), 0x30000000, K, M, 0x40000000, N, ctypes.byref(ws), None)
                    assert rc == 0, (bits, K, N, M, rc)
    ex.exl3_test_mock_counts()


def test_synth_is_seeded_and_shaped():
    a = synth.gen_layer("cfg", "q", 256, 384, 3)
    b = synth.gen_layer("cfg", "q", 256, 384, 3)
    assert (a.words == b.words).all() and (a.scales == b.scales).all()
    assert a.words.size == 256 * 384 * 3 // 8 and a.scales.size == 384 and a.suh.size == 256
    assert set(a.suh.tolist()) <= {0x3C00, 0xBC00}


def test_static_entry_checks_and_mock_launches(lib):
    """exl3_linear_group_static (the no-allocation variant): the same launches
    as exl3_linear_group in mock mode, no counter fill per call, and a call
    too large for the static scratch refused with ESCRATCH before any GPU
    call (8192 prompt rows of K = 5120: 80 MiB of rotated input)."""
    import ctypes
    K = 5120
    g, u = fake_weight(K, 17408, 4), fake_weight(K, 17408, 4, base=0x20000000)
    ws_arr = ex._wlist([g, u])
    ys = (ctypes.c_void_p * 2)(0x30000000, 0x38000000)
    ld = (ctypes.c_int64 * 2)(17408, 17408)
    ex.exl3_test_mock(True)
    for M in (16, 7, 1):
        assert lib.exl3_linear_group_static(2, ws_arr, 0x40000000, K, M, ys, ld, None) == ex.EXL3_OK
        launches, fills, _, _ = ex.exl3_test_mock_counts()
        assert (launches, fills) == (2, 0), M
    assert lib.exl3_linear_group_static(2, ws_arr, 0x40000000, K, 0, ys, ld, None) == ex.EXL3_OK
    assert ex.exl3_test_mock_counts()[0] == 0
    ex.exl3_test_mock(False)
    # refused on the host: nothing reaches a GPU (there is none here)
    assert lib.exl3_linear_group_static(2, ws_arr, 0x40000000, K, 8192, ys, ld, None) == ex.EXL3_ESCRATCH
    assert lib.exl3_linear_group_static(4, ws_arr, 0x40000000, K, 16, ys, ld, None) == ex.EXL3_EGROUP
    assert lib.exl3_linear_group_static(2, ws_arr, 0, K, 16, ys, ld, None) == ex.EXL3_EINVAL
    assert b"static scratch" in lib.exl3_strerror(ex.EXL3_ESCRATCH)


def test_split_fold_launch_after_the_exchanged_128_row_tiling(lib):
    """The down projection (K 17408, N 5120, 16 splits) at 33-128 rows runs the
    exchanged 2 x 2 tiling in 64-row tiles and a split-fold launch after it
    (three launches with the rotation); at 32 rows the exchanged 32-row form
    (two); a forced plan of more than 16 splits keeps the 128-row tiling and
    its own last-arriver fold."""
    ex.exl3_test_mock(True)
    w = fake_weight(17408, 5120, 4)
    need, cb = ex.exl3_workspace_need([w], 128)
    ws = ex.exl3_workspace_t(0x200000000, need, cb)

    def call(M):
        ex.exl3_test_mock_counts()
        assert lib.exl3_linear(ctypes.byref(w.desc), 0x300000000, 17408, M, 0x400000000, 5120, ctypes.byref(ws),
                               None) == ex.EXL3_OK
        return ex.exl3_test_mock_counts()[0], ex.exl3_test_last_form()

    for M in (33, 48, 49, 64, 96, 97, 100, 128):
        assert call(M) == (3, "linear_tile64_kernel<4>")
    assert call(32) == (2, "linear_chain_kernel<4, 2, false, 4, 8, 2>")
    ex.exl3_test_force(-1, -1, 17)
    need17, cb17 = ex.exl3_workspace_need([w], 128)
    ws = ex.exl3_workspace_t(0x200000000, need17, cb17)
    assert call(128) == (2, "linear_tile_kernel<4, false>")


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for two it exits with status 2 and a
    message naming the request, before it touches a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=root)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    assert "one GPU" in r.stdout + r.stderr and "2" in r.stdout + r.stderr
