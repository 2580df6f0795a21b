"""exl3_linear_group_static, the variant of exl3_linear_group for callers that
cannot allocate: its split counters, rotated inputs and partials live in the
library's static scratch. Through the C ABI it must give exactly the bytes of
exl3_linear_group with a caller workspace, on two calls in a row whose second
is smaller (the scratch keeps the first call's contents; the counters must be
back at zero), for the headline groups and a mid-row pair."""

import numpy as np
import pytest

import gpu_util as G
from trellis_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu

K = synth.HIDDEN


def ex():
    import trellis_quantized_linear_amd.exl3 as m
    return m


@pytest.fixture(autouse=True)
def _hooks():
    ex().lib()
    ex().exl3_test_force(-1, -1, 0)
    ex().exl3_test_fuse_rotation(False)
    yield


def _outputs(weights, Ns, xd, M, static):
    ys = [G.empty_y(M, N) for N in Ns]
    if static:
        G.say(f"exl3_linear_group_static members={Ns} M={M}")
        ex().exl3_linear_group_static(weights, xd, ys, M=M)
    else:
        ws = ex().Workspace().reserve(weights, M)
        G.say(f"exl3_linear_group members={Ns} M={M}")
        ex().exl3_linear_group(weights, xd, ys, ws, M=M)
    G.torch_mod().cuda.synchronize()
    return [G.host_u16(y) for y in ys]


CASES = [(("gate", "up"), (synth.INTERMEDIATE, synth.INTERMEDIATE), 4, (16, 7)),
         (("q", "k", "v"), (synth.Q_COLS, synth.KV_COLS, synth.KV_COLS), 4, (16, 1)),
         (("gate", "up"), (synth.INTERMEDIATE, synth.INTERMEDIATE), 3, (48, 17)),
         (("down",), (synth.HIDDEN,), 4, (128, 100))]


@pytest.mark.parametrize("names,Ns,bits,rows", CASES)
def test_static_scratch_equals_workspace_call(names, Ns, bits, rows):
    Kin = synth.INTERMEDIATE if names == ("down",) else K
    layers = [G.layer("no-alloc", n, Kin, N, bits) for n, N in zip(names, Ns)]
    weights = [G.upload(L) for L in layers]
    x = G.xbits("no-alloc", max(rows), Kin)
    xd = G.dev_bf16(x)
    for M in rows:                     # the second call is the smaller one
        want = _outputs(weights, Ns, xd, M, static=False)
        got = _outputs(weights, Ns, xd, M, static=True)
        for n, a, b in zip(names, got, want):
            assert np.array_equal(a, b), (n, M)
    # the same bytes again after the smaller call: the counters were left at zero
    M = rows[0]
    want = _outputs(weights, Ns, xd, M, static=False)
    got = _outputs(weights, Ns, xd, M, static=True)
    assert all(np.array_equal(a, b) for a, b in zip(got, want))
    # and against the oracle on a sampled block per member
    for L, y in zip(layers, got):
        blocks = G.sample_blocks(L.N // 128, k=2, seed=M)
        cols = np.concatenate([y[:, 128 * nb:128 * (nb + 1)] for nb in blocks], axis=1)
        G.assert_close(cols, G.oracle_blocks(L, x[:M], blocks), what=f"static {L.name} M={M}")


def test_static_scratch_refuses_calls_beyond_its_size():
    """Prompt rows need M K 2 bytes of rotated input per member: 8192 rows at
    K = 5120 is 80 MiB, past the 64 MiB scratch; refused before launching."""
    L = G.layer("no-alloc-big", "q", K, 1024, 4)
    w = G.upload(L)
    M = 8192
    xd = G.dev_bf16(np.zeros((M, K), np.uint16))
    y = G.empty_y(M, 1024)
    before = G.host_u16(y).copy()
    with pytest.raises(ex().Exl3Error) as e:
        ex().exl3_linear_group_static([w], xd, [y], M=M)
    assert e.value.code == ex().EXL3_ESCRATCH
    G.torch_mod().cuda.synchronize()
    assert np.array_equal(G.host_u16(y), before)
