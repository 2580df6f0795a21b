"""The input rotation inside the linear launch (up to 32 rows, opt-in),
bitwise against the two-launch form: the pages chain the rotation and the
decode-row linear without a launch gap and require that every dependent
launch waits before it reads what the rotation wrote (TensorFold PR #1467,
"What this changes" and the merge review). Here the linear launch's first workgroups
write Xr and flag each 128-column chunk; every chain polls the flags of the
chunks it reads, and after a bounded number of polls rotates a missing chunk
itself. Checked:

* fused == two launches, byte for byte, for every decode launch form that
  fuses (spread, exchanged 16 rows with one or two waves per split, 32 rows
  chained and exchanged), groups of
  one to three members, three widths, and a chain that spans more than 64
  chunks (one split over K = 17408);
* the fallback (spin limit 0: a wave that finds a chunk unflagged rotates it
  itself) gives the same bytes;
* flags and counters are zero after every call;
* calls whose inputs alternate (eagerly, and as graph replays with X
  rewritten in place between replays) each get their own input's result, so
  no call reads a flag or an Xr chunk left by the one before.
"""

import numpy as np
import pytest

import gpu_util as G

pytestmark = pytest.mark.gpu


def ex():
    import trellis_quantized_linear_amd.exl3 as m
    return m


@pytest.fixture(autouse=True)
def _hooks():
    ex().lib()
    ex().exl3_test_force(-1, -1, 0)
    ex().exl3_test_fuse_rotation(True, -1)
    yield
    ex().exl3_test_force(-1, -1, 0)
    ex().exl3_test_fuse_rotation(False, -1)


def _group(config, K, Ns, bits):
    layers = [G.layer(config, f"m{j}", K, N, bits) for j, N in enumerate(Ns)]
    return layers, [G.upload(L) for L in layers]


def _run(ws_list, xd, M, ws, tag):
    ys = G.run_group(ws_list, xd, M=M, ws=ws, tag=tag)
    return [G.host_u16(y) for y in ys]


# (label, K, member widths, bits, rows, forced (m_tiles, chained, splits))
CASES = [
    ("q/k/v exchanged 16 rows", 5120, (6144, 1024, 1024), 4, (1, 7, 16), (-1, -1, 0)),
    ("gate/up spread", 5120, (17408, 17408), 4, (1, 16), (-1, -1, 0)),
    ("spread, many left blocks", 5120, (8192, 8192), 3, (5,), (1, 2, 0)),
    ("32 rows exchanged", 5120, (1024, 2048), 6, (17, 32), (-1, -1, 0)),
    ("32 rows chained", 5120, (1024,), 4, (24, 32), (2, 1, 0)),
    ("16 rows exchanged, one split over K=17408", 17408, (1024,), 4, (3, 16), (1, 0, 1)),
    ("16 rows exchanged, 2 bits", 1024, (512, 256, 384), 2, (2, 15), (1, 0, 0)),
    ("16 rows, column halves, 6 bits", 5120, (1024, 2048), 6, (4, 16), (1, 3, 0)),
]


@pytest.mark.parametrize("label,K,Ns,bits,rows,force", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_two_launches(label, K, Ns, bits, rows, force):
    torch = G.torch_mod()
    _, ws_list = _group("fused-" + label, K, Ns, bits)
    ex().exl3_test_force(*force)
    ws = ex().Workspace().reserve(ws_list, max(rows))
    for M in rows:
        xd = G.dev_bf16(G.xbits("fused", M, K))
        ex().exl3_test_fuse_rotation(False)
        two = _run(ws_list, xd, M, ws, f"{label}: two launches")
        ex().exl3_test_fuse_rotation(True, -1)
        one = _run(ws_list, xd, M, ws, f"{label}: fused")
        ex().exl3_test_fuse_rotation(True, 0)
        helped = _run(ws_list, xd, M, ws, f"{label}: fused, spin limit 0")
        torch.cuda.synchronize()
        for j in range(len(ws_list)):
            assert np.array_equal(one[j], two[j]), (label, M, j)
            assert np.array_equal(helped[j], two[j]), (label, M, j, "fallback")
        assert int(ws.counters().abs().sum()) == 0, (label, M)


def test_fused_launch_matches_the_oracle_at_a_ragged_row_count():
    """Fused path against the oracle directly (sampled blocks), 13 rows of the
    q/k/v group, with an input whose rows are an unaligned strided view."""
    torch = G.torch_mod()
    from oracle import exl3_oracle as O
    K, Ns, M = 5120, (6144, 1024, 1024), 13
    layers, ws_list = _group("fused-oracle", K, Ns, 4)
    x = G.xbits("fused-oracle", M, K)
    big = torch.zeros((M, K + 8), dtype=torch.int16, device="cuda")
    big[:, 3:3 + K] = torch.from_numpy(x.view(np.int16).copy()).to("cuda")
    xd = big.view(torch.bfloat16)[:, 3:3 + K]                # row stride K + 8, 6-byte offset
    ws = ex().Workspace().reserve(ws_list, M)
    ys = G.run_group(ws_list, xd, M=M, ws=ws, tag="fused, strided x")
    torch.cuda.synchronize()
    for L, y in zip(layers, ys):
        blocks = G.sample_blocks(L.N // 128, k=3, seed=L.N)
        G.assert_close(G.gpu_blocks(y, blocks), G.oracle_blocks(L, x, blocks), what=f"fused N={L.N}")
    assert int(ws.counters().abs().sum()) == 0


def test_alternating_inputs_each_get_their_own_result():
    """Back-to-back fused calls on one workspace with inputs A, B, A, B, ...:
    a flag or an Xr chunk left over from the call before would hand a call
    the other input's rotation."""
    torch = G.torch_mod()
    K, Ns, M = 5120, (17408, 17408), 16
    _, ws_list = _group("fused-alt", K, Ns, 4)
    ws = ex().Workspace().reserve(ws_list, M)
    xa = G.dev_bf16(G.xbits("fused-alt", M, K, tag="a"))
    xb = G.dev_bf16(G.xbits("fused-alt", M, K, tag="b"))
    ex().exl3_test_fuse_rotation(False)
    ref_a = _run(ws_list, xa, M, ws, "ref a")
    ref_b = _run(ws_list, xb, M, ws, "ref b")
    assert not np.array_equal(ref_a[0], ref_b[0])
    ex().exl3_test_fuse_rotation(True, -1)
    outs = [[G.empty_y(M, N) for N in Ns] for _ in range(40)]
    G.say("40 alternating fused calls")
    for i, ys in enumerate(outs):
        ex().exl3_linear_group(ws_list, xa if i % 2 == 0 else xb, ys, ws, M=M)
    torch.cuda.synchronize()
    for i, ys in enumerate(outs):
        ref = ref_a if i % 2 == 0 else ref_b
        for j, y in enumerate(ys):
            assert np.array_equal(G.host_u16(y), ref[j]), (i, j)
    assert int(ws.counters().abs().sum()) == 0


def test_graph_replays_with_input_rewritten_in_place():
    """A captured fused call replayed four times, X overwritten in place
    (by a copy kernel) before each replay, eager work and a synchronisation
    between replays; each replay equals the eager call on its input."""
    torch = G.torch_mod()
    K, Ns, M = 5120, (6144, 1024, 1024), 16
    _, ws_list = _group("fused-graph", K, Ns, 4)
    ws = ex().Workspace().reserve(ws_list, M)
    inputs = [G.dev_bf16(G.xbits("fused-graph", M, K, tag=f"x{i}")) for i in range(3)]
    refs = [_run(ws_list, xi, M, ws, f"eager {i}") for i, xi in enumerate(inputs)]
    x = inputs[0].clone()
    ys = [G.empty_y(M, N) for N in Ns]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ex().exl3_linear_group(ws_list, x, ys, ws, M=M)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    G.say("capture the fused call")
    with torch.cuda.graph(g):
        ex().exl3_linear_group(ws_list, x, ys, ws, M=M)
    torch.cuda.synchronize()
    for rep, i in enumerate((1, 2, 0, 1)):
        x.copy_(inputs[i])
        _ = (inputs[i].float() * 2).sum()                 # unrelated eager work between replays
        G.say(f"replay {rep} with input {i}")
        g.replay()
        torch.cuda.synchronize()
        for j, y in enumerate(ys):
            assert np.array_equal(G.host_u16(y), refs[i][j]), (rep, i, j)
    assert int(ws.counters().abs().sum()) == 0
