"""Registry of the kernel contract: every linear kernel form that the
library's dispatch can reach, with the gate shapes that run it on the GPU
(against the oracle, and byte for byte against one-row calls) and the
occupancy its launch was designed for.

The pages require the same of their kernels (TensorFold PR #1467, "Receipt",
"Kernel contract": every launch registered in gates 1-4, with a resource
record; author follow-up, "A dispatch test": a host-side sweep of the
dispatch over K and N up to 16384 must find each reachable form among the
registered ones, each run by some gate shape). Here a form is a kernel template instantiation, named as the
compiler names it (exl3_test_last_form, the build's resource records).

A gate is (K, [N of each member], M, mode): mode "" is the automatic
dispatch, "prompt1" the opt-in prompt arithmetic (exl3_set_prompt_arithmetic
(1)), "rot" the input rotation inside the linear launch
(exl3_test_fuse_rotation). The dispatch does not depend on the bit width, so
every form is registered at every width the library accepts.
"""

from __future__ import annotations

WIDTHS = tuple(range(2, 9))
LDS_PER_CU = 160 * 1024

# form template ({b}: bits) -> (waves per SIMD the launch is built for, gates)
FORMS = {
    # 16 rows, every split of a block in one 8-wave workgroup, two per CU
    "linear_chain_kernel<{b}, 1, true, 8, 8, 2>": (4, [(128, [128], 1, ""), (256, [65536], 16, "")]),
    "linear_chain_kernel<{b}, 1, true, 8, 8, 0>": (4, [(128, [128], 17, ""), (256, [65536], 17, "")]),
    # 16 rows exchanged, each split on two waves of 4 column tiles
    "linear_chain_kernel<{b}, 1, false, 8, 4, 2>": (4, [(256, [128], 1, ""), (5120, [1024, 1024], 16, "")]),
    "linear_chain_kernel<{b}, 1, false, 8, 4, 0>": (4, [(256, [128], 17, "")]),
    "linear_chain_kernel<{b}, 1, false, 8, 4, 2> +rot": (4, [(256, [128], 1, "rot")]),
    # 16 rows exchanged, one split per wave
    "linear_chain_kernel<{b}, 1, false, 4, 8, 2>": (1, [(1024, [20480], 1, "")]),
    "linear_chain_kernel<{b}, 1, false, 4, 8, 0>": (1, [(1024, [8320], 17, "")]),
    "linear_chain_kernel<{b}, 1, false, 4, 8, 2> +rot": (1, [(1024, [20480], 1, "rot")]),
    # 32 rows exchanged (long splits)
    "linear_chain_kernel<{b}, 2, false, 4, 8, 2>": (1, [(16384, [128], 17, "")]),
    "linear_chain_kernel<{b}, 2, false, 4, 8, 2> +rot": (1, [(16384, [128], 17, "rot")]),
    # the spread launch: one 16-wave workgroup per CU, spare waves on the left blocks
    "linear_spread_kernel<{b}>": (4, [(256, [34816], 1, ""), (256, [17408, 17408], 16, "")]),
    "linear_spread_kernel<{b}> +rot": (4, [(256, [34816], 7, "rot")]),
    "linear_spread_rows_kernel<{b}>": (4, [(256, [34816], 17, ""), (256, [17408, 17408], 32, ""), (256, [24576], 48, "")]),
    # 128-row tilings
    "linear_block_kernel<{b}, true>": (2, [(256, [34816], 65, ""), (256, [17408, 17408], 100, ""), (128, [128], 129, ""),
                                          (256, [384], 300, ""), (256, [1024, 256, 256], 200, "")]),
    # 64-row block tiling: a few more blocks than CUs at 33-64 rows (left blocks as single splits)
    "linear_block64_kernel<{b}>": (2, [(256, [34816], 33, ""), (256, [17408, 17408], 64, "")]),
    # 32-row block tiling: chained block tiles at 17-32 rows (many blocks: the head)
    "linear_block32_kernel<{b}>": (2, [(128, [248320], 17, ""), (256, [131072], 32, ""), (128, [65536, 65536], 24, "")]),
    # exchanged 2 x 2 tiles of 64 rows (2 waves), partials added by the split-fold launch; the
    # 128-row form (4 waves) is reached only through exl3_test_force now
    "linear_tile64_kernel<{b}>": (3, [(16384, [128], 97, ""), (16384, [128, 256], 64, ""), (17408, [5120], 49, ""),
                                     (17408, [5120], 128, "")]),
    # prompt rows of long-split weights (down): 128 rows x 2 blocks (the last pair of an odd count: 1)
    "linear_wide_kernel<{b}>": (1, [(16384, [128], 129, ""), (16384, [384], 300, ""), (17408, [256, 128], 200, "")]),
    # opt-in single-chain prompt tiles (other bits than the rest, by design)
    "linear_quad_kernel<{b}>": (1, [(128, [128], 129, "prompt1"), (256, [640], 300, "prompt1")]),
}


def registered(forms=None):
    """{form name at a width: (bits, waves per SIMD, gates)} for every width."""
    forms = FORMS if forms is None else forms
    out = {}
    for tmpl, (waves, gates) in forms.items():
        for b in WIDTHS:
            out[tmpl.format(b=b)] = (b, waves, gates)
    return out


def waves_per_workgroup(form: str) -> int:
    """Waves of one workgroup of a form (its launch's block size)."""
    if form.startswith("linear_spread"):
        return 16
    if form.startswith("linear_chain_kernel"):
        return int(form.split("<")[1].split(",")[3])
    return 4
