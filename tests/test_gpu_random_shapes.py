"""Seeded random shapes through the group call. K, the members' widths, the
row count and the bit width are drawn per case so that the launch choices'
thresholds are crossed from either side: decode rows (1-16), mid rows
(17-128) and prompt rows (129-400); one to three members; weights of a few
blocks, of more than 64 blocks (the wide plan) and groups of more blocks
than CUs (the spread launch and the 128-row block tiling with their left
blocks). Each case: every member against the oracle on sampled column
blocks (first, last, a random one and every block past one per CU of the
launch), on all rows; and the group's bytes equal to each member's own
call (a group member's bytes are its own launch's: PR #1467, "The
arithmetic")."""

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
    ex().exl3_test_fuse_rotation(False)
    yield


def _cases():
    rng = np.random.default_rng(20261202)
    out = []
    for i in range(20):
        regime = i % 4
        M = int(rng.integers(1, 17) if regime == 0 else rng.integers(17, 49) if regime == 1
                else rng.integers(49, 129) if regime == 2 else rng.integers(129, 401))
        if i % 5 == 0:
            # more blocks than CUs: two wide members of the same K
            K = 128 * int(rng.integers(16, 33))
            blocks = (int(rng.integers(120, 150)), int(rng.integers(120, 150)))
        else:
            K = 128 * int(rng.integers(1, 33))
            n_mem = int(rng.integers(1, 4))
            blocks = tuple(int(rng.integers(1, 100)) for _ in range(n_mem))
        bits = int(rng.integers(2, 9))
        out.append((i, K, blocks, M, bits))
    # forms the draws above miss: the spread launch over several row blocks,
    # and a long-split weight (K 12,288: 24 chunks a split) at 24 rows (32-row
    # exchanged), 100 rows (2 x 2 exchanged tiles and the split-fold launch)
    # and 300 rows (the 128 x 256 tiling)
    out += [(20, 5120, (136, 136), 24, 3), (21, 12288, (40,), 24, 4), (22, 12288, (40,), 100, 5),
            (23, 12288, (40,), 300, 4)]
    return out


CASES = _cases()


def cu_count():
    return G.torch_mod().cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("i,K,blocks,M,bits", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_group_vs_oracle_and_solo(i, K, blocks, M, bits):
    config = f"random-{i}"
    layers = [G.layer(config, f"m{j}", K, 128 * nb, bits) for j, nb in enumerate(blocks)]
    ws_ = [G.upload(L) for L in layers]
    x = G.xbits(config, M, K)
    xd = G.dev_bf16(x)
    G.say(f"case {i}: K={K} blocks={blocks} M={M} bits={bits}")
    ys = G.run_group(ws_, xd, tag=f"case {i}")
    form = ex().exl3_test_last_form()
    G.say(f"case {i}: {form}")
    ncu, first = cu_count(), 0
    for j, (L, w, y) in enumerate(zip(layers, ws_, ys)):
        nb = L.N // 128
        left = [b for b in range(nb) if first + b >= ncu]
        first += nb
        pick = sorted(set(G.sample_blocks(nb, k=3, seed=i + j)) | set(left))
        G.assert_close(G.gpu_blocks(y, pick), G.oracle_blocks(L, x, pick), what=f"case {i} member {j}")
        solo = G.host_u16(G.run(w, xd, tag=f"case {i} member {j} alone"))
        assert np.array_equal(G.host_u16(y), solo), (i, j)
