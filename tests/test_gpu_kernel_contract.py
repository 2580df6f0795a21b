"""The kernel contract's GPU gates (TensorFold PR #1467, "Receipt", "Kernel
contract", gates 1-4, and the author follow-up's dispatch test): every form
of the registry, at every width 2..8, runs its gate shapes through the
library, and

* the launch is the registered form (exl3_test_last_form after the real
  launch),
* sampled column blocks match the oracle within the parity tolerance (the
  first and last block, and for a spread launch its first and last left
  block),
* rows 0 and M - 1 are byte-identical to one-row calls (the decode-row
  launch), except for the opt-in prompt arithmetic, whose rows are compared
  with the same rows of a longer call of that arithmetic instead,
* a form with the rotation inside the launch gives the bytes of the same
  call with a rotation launch of its own.
"""

import numpy as np
import pytest

import gpu_util as G
import kernel_contract as KC

pytestmark = pytest.mark.gpu


def ex():
    import trellis_quantized_linear_amd.exl3 as m
    return m


@pytest.fixture(autouse=True)
def _modes():
    ex().lib()
    ex().exl3_test_force(-1, -1, 0)
    ex().exl3_set_prompt_arithmetic(0)
    ex().exl3_test_fuse_rotation(False)
    yield
    ex().exl3_set_prompt_arithmetic(0)
    ex().exl3_test_fuse_rotation(False)


def _set_mode(mode):
    ex().exl3_set_prompt_arithmetic(1 if mode == "prompt1" else 0)
    ex().exl3_test_fuse_rotation(mode == "rot")


def _call(weights, xd, M, mode):
    _set_mode(mode)
    try:
        ys = G.run_group(weights, xd, M=M, tag=f"mode={mode or 'auto'}")
        G.torch_mod().cuda.synchronize()
        form = ex().exl3_test_last_form()
    finally:
        _set_mode("")
    return [G.host_u16(y) for y in ys], form


def _left_blocks(Ns):
    ncu = G.torch_mod().cuda.get_device_properties(0).multi_processor_count
    out, first = [], 0
    for N in Ns:
        nb = N // 128
        out.append([b for b in range(nb) if first + b >= ncu])
        first += nb
    return out


@pytest.mark.parametrize("bits", KC.WIDTHS)
@pytest.mark.parametrize("tmpl", list(KC.FORMS))
def test_registered_form_gates(tmpl, bits):
    form = tmpl.format(b=bits)
    _, gates = KC.FORMS[tmpl]
    for gi, (K, Ns, M, mode) in enumerate(gates):
        tag = f"{form} gate {gi}"
        layers = [G.layer("contract", f"{tmpl}/{bits}/{gi}/{j}", K, N, bits) for j, N in enumerate(Ns)]
        weights = [G.upload(L) for L in layers]
        Mx = M + 71 if mode == "prompt1" else M
        x = G.xbits("contract", Mx, K, sigma=0.5 if M > 128 else 1.0, tag=f"{tmpl}/{bits}/{gi}")
        xd = G.dev_bf16(x)
        G.say(f"{tag}: K={K} N={Ns} M={M} bits={bits} mode={mode or 'auto'}")
        ys, got_form = _call(weights, xd, M, mode)
        assert got_form == form, (tag, got_form)
        lefts = _left_blocks(Ns) if form.startswith("linear_spread") else [[] for _ in Ns]
        for j, (L, y) in enumerate(zip(layers, ys)):
            nb = L.N // 128
            blocks = sorted({0, nb - 1} | ({lefts[j][0], lefts[j][-1]} if lefts[j] else set()))
            cols = np.concatenate([y[:, 128 * b:128 * (b + 1)] for b in blocks], axis=1)
            G.assert_close(cols, G.oracle_blocks(L, x[:M], blocks), what=f"{tag} member {j}")
        if mode == "prompt1":
            # the opt-in arithmetic's rows do not depend on the row count above 128
            longer, _ = _call(weights, xd, Mx, mode)
            for j in range(len(Ns)):
                assert np.array_equal(longer[j][:M], ys[j]), (tag, j)
        else:
            for r in sorted({0, M - 1}):
                one, _ = _call(weights, xd[r:r + 1], 1, "")
                for j in range(len(Ns)):
                    assert np.array_equal(one[j][0], ys[j][r]), (tag, j, r)
        if mode == "rot":
            two, _ = _call(weights, xd, M, "")
            for j in range(len(Ns)):
                assert np.array_equal(two[j], ys[j]), (tag, j)
