"""GPU parity of the default group launch against the oracle, on the launches
the benchmark times (TensorFold PR #1467, "The arithmetic": a group member's
output is its own single-weight launch's, which the oracle defines).

* The 27B decode-row groups {q, k, v} and {gate, up} (K = 5120, 4 bits) at 1,
  7 and 16 rows through exl3_linear_group with the automatic launch choice:
  the rotation of two or three members in one launch, then the
  column-halves exchanged launch ({q, k, v}) or the spread launch ({gate,
  up}: one block per CU, the blocks past one per CU finished by the
  workgroups' spare waves through the workspace). Every such left block is
  compared with the oracle, beside the first, last and a random block of
  each member.
* The 3-bit {gate, up} pair of the 3.5 bpw MLP at 17, 24 and 32 rows: the
  spread launch over several 16-row blocks in one grid; at 33, 48, 49, 100
  and 128 rows the chained block tiling (64-row workgroups up to 64 rows,
  128-row ones above) with one workgroup per CU, the
  blocks past one per CU split one chain to a workgroup and finished by the
  split-fold launch (every such block against the oracle, and rows 0 and
  M - 1 byte for byte against one-row calls).
* The same pair at 40 rows at widths 2 and 4-8 (the 64-row block tiling
  with its left blocks at every width).
* A stress of the relaxed split-K exchange on that headline launch and on
  the {q, k, v} group's exchanged launch: 10^4 group calls each at 16 rows,
  bytes compared every 100 calls, counters zero at the end (PR #1475, "What
  this changes": the last arriver resets its counter).
"""

import numpy as np
import pytest

import gpu_util as G
from trellis_quantized_linear_amd import synth

pytestmark = pytest.mark.gpu

K = synth.HIDDEN
COLS = {"q": synth.Q_COLS, "k": synth.KV_COLS, "v": synth.KV_COLS,
        "gate": synth.INTERMEDIATE, "up": synth.INTERMEDIATE}


def ex():
    import trellis_quantized_linear_amd.exl3 as m
    return m


@pytest.fixture(autouse=True)
def _hooks():
    ex().lib()
    ex().exl3_test_force(-1, -1, 0)
    ex().exl3_test_fuse_rotation(False)
    yield
    ex().exl3_test_force(-1, -1, 0)


def cu_count():
    return G.torch_mod().cuda.get_device_properties(0).multi_processor_count


def left_blocks(n_blocks_list):
    """Per member, the blocks of a spread launch past one block per CU (the
    launch's blocks are the members' blocks in member order)."""
    ncu = cu_count()
    out, first = [], 0
    for nb in n_blocks_list:
        out.append([b for b in range(nb) if first + b >= ncu])
        first += nb
    return out


def check_group(names, M, bits, config, rows_tag):
    layers = [G.layer(config, n, K, COLS[n], bits) for n in names]
    ws_ = [G.upload(L) for L in layers]
    x = G.xbits(config, M, K, tag=rows_tag)
    ys = G.run_group(ws_, G.dev_bf16(x), tag=f"{'+'.join(names)} {bits}-bit M={M}")
    lefts = left_blocks([L.N // 128 for L in layers])
    total = sum(L.N // 128 for L in layers)
    for j, (n, L, y) in enumerate(zip(names, layers, ys)):
        nb = L.N // 128
        blocks = sorted(set(G.sample_blocks(nb, k=3, seed=M + j)) | set(lefts[j]))
        if lefts[j]:
            G.say(f"{n}: blocks {lefts[j][0]}..{lefts[j][-1]} are left blocks ({total} blocks, {cu_count()} CUs)")
        G.assert_close(G.gpu_blocks(y, blocks), G.oracle_blocks(L, x, blocks), what=f"group {n} M={M} b={bits}")


@pytest.mark.parametrize("M", [1, 7, 16])
def test_qkv_group_default_launch_vs_oracle(M):
    check_group(("q", "k", "v"), M, 4, "group-oracle", "x")


@pytest.mark.parametrize("M", [1, 7, 16])
def test_gate_up_group_spread_launch_vs_oracle(M):
    """Includes every left block of the spread launch (on 256 CUs: up's
    blocks 120..135)."""
    check_group(("gate", "up"), M, 4, "group-oracle", "x")


@pytest.mark.parametrize("M", [17, 24, 32])
def test_gate_up_3bit_spread_over_row_blocks_vs_oracle(M):
    """The 3.5 bpw MLP's {gate, up} pair at mid rows: the spread launch once
    per 16-row block in one grid, left blocks per row block."""
    check_group(("gate", "up"), M, 3, "group-oracle-c3", "x")


@pytest.mark.parametrize("M", [33, 48, 49, 64, 65, 100, 128])
def test_gate_up_3bit_block_tiling_left_blocks_vs_oracle(M):
    """The 3.5 bpw MLP's {gate, up} pair at 33-128 rows (64-row workgroups up
    to 64 rows, 128-row ones above): 256 block workgroups,
    the 16 left blocks' splits one per workgroup after its own block."""
    check_group(("gate", "up"), M, 3, "group-oracle-c3", "x")
    layers = [G.layer("group-oracle-c3", n, K, COLS[n], 3) for n in ("gate", "up")]
    ws_ = [G.upload(L) for L in layers]
    xd = G.dev_bf16(G.xbits("group-oracle-c3", M, K, tag="x"))
    full = [G.host_u16(y) for y in G.run_group(ws_, xd, M=M, tag=f"left blocks M={M}")]
    for r in sorted({0, M - 1}):
        one = [G.host_u16(y) for y in G.run_group(ws_, xd[r:r + 1], M=1, tag=f"row {r} alone")]
        for j in range(2):
            assert np.array_equal(one[j][0], full[j][r]), (M, r, j)


@pytest.mark.parametrize("bits", [2, 4, 5, 6, 7, 8])
def test_gate_up_block_tiling_left_blocks_every_width_vs_oracle(bits):
    """The {gate, up} pair at 40 rows at the other widths: the same launch
    (chained 64-row blocks, the left blocks' splits after each workgroup's
    own block, the split-fold launch), every left block and sampled blocks
    against the oracle."""
    check_group(("gate", "up"), 40, bits, "group-oracle-w", "x")
    assert ex().exl3_test_last_form() == f"linear_block64_kernel<{bits}>"


@pytest.mark.parametrize("names,form", [(("gate", "up"), "linear_spread_kernel<4>"),
                                        (("q", "k", "v"), "linear_chain_kernel<4, 1, false, 8, 4, 2>")])
def test_decode_group_exchange_stress(names, form):
    """10^4 calls of each decode-row group launch at M = 16: {gate, up} (the
    headline spread launch, its left blocks exchanged) and {q, k, v} (the
    exchanged column halves, a block's split groups dealt to one XCD's
    range), bytes compared with the first call every 100 calls (stops at the
    first mismatch), split counters zero at the end."""
    torch = G.torch_mod()
    layers = [G.layer("stress-gu" if len(names) == 2 else "stress-qkv", n, K, COLS[n], 4) for n in names]
    ws_ = [G.upload(L) for L in layers]
    xd = G.dev_bf16(G.xbits("stress-gu" if len(names) == 2 else "stress-qkv", 16, K))
    ws = ex().Workspace().reserve(ws_, 16)
    ref = G.run_group(ws_, xd, ws=ws, tag="stress reference")
    torch.cuda.synchronize()
    assert ex().exl3_test_last_form() == form
    ys = [[G.empty_y(16, L.N) for L in layers] for _ in range(100)]
    for batch in range(100):
        if batch % 20 == 0:
            G.say(f"stress batch {batch} of 100 (100 group calls each)")
        for y in ys:
            ex().exl3_linear_group(ws_, xd, y, ws)
        torch.cuda.synchronize()
        for i, y in enumerate(ys):
            for a, b in zip(y, ref):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (batch, i)
    assert int(ws.counters().abs().sum()) == 0
