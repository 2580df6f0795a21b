"""Float64 error report (the "changed reduction order keeps native error no
worse" criterion of the pages' review of the mid-M path, PR #1475 review
thread): for several shapes and K-split counts, the GPU's Y is compared with
the exact result (float64 everywhere: no fp16 rounding of the rotated input,
no bf16 rounding of Y) and its RMS and worst-column RMS error are set beside
those of the oracle's own Y (fp16 Xr, float64 accumulation, bf16 Y). The
GPU's fp32 MFMA chains, in any split plan, must stay within a few percent of
the oracle's error, which the two roundings dominate.
"""

import numpy as np
import pytest

import gpu_util as G
from oracle import exl3_oracle as O

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


def _errors(y, exact):
    d = y - exact
    scale = np.sqrt(np.mean(exact ** 2))
    rms = np.sqrt(np.mean(d ** 2)) / scale
    col = np.sqrt(np.mean(d ** 2, axis=0)) / scale
    return rms, float(col.max())


# (K, N, bits, M, splits to force besides the plan's)
CASES = [(5120, 1024, 4, 16, (2, 4, 8)), (17408, 512, 4, 8, (4, 15)), (5120, 2048, 3, 64, (2, 8)),
         (5120, 768, 6, 100, (4,))]


@pytest.mark.parametrize("K,N,bits,M,others", CASES)
def test_error_no_worse_than_the_oracle_in_any_plan(K, N, bits, M, others):
    L = G.layer("errors", f"{K}x{N}b{bits}", K, N, bits)
    x = G.xbits("errors", M, K)
    w = G.upload(L)
    xd = G.dev_bf16(x)
    exact = O.linear_packed(L.words, K, N, bits, L.scales, L.suh, L.svh, x, exact=True)
    ref = O.bf16_to_f64(O.linear_packed(L.words, K, N, bits, L.scales, L.suh, L.svh, x))
    o_rms, o_col = _errors(ref, exact)
    plan = ex().exl3_plan(K, N, bits).splits
    for s in (0,) + tuple(others):
        ex().exl3_test_force(-1, -1, s)
        y = O.bf16_to_f64(G.host_u16(G.run(w, xd, tag=f"error report S={s or plan}")))
        g_rms, g_col = _errors(y, exact)
        G.say(f"K={K} N={N} b={bits} M={M} S={s or plan}: RMS err GPU {g_rms:.3e} vs oracle {o_rms:.3e}; "
              f"worst column {g_col:.3e} vs {o_col:.3e}")
        assert g_rms <= 1.05 * o_rms, (s, g_rms, o_rms)
        assert g_col <= 1.25 * o_col, (s, g_col, o_col)
    ex().exl3_test_force(-1, -1, 0)
