"""Float64 error report: the pages' rule for the mid-M path that a new
summation order may not raise the error against float64 (PR #1467, review
item 1, "Fixed plans"), checked at 16 rows and again at 128 rows.

For several shapes, every K-split count tried (the plan's and forced others)
runs at 16 and at 128 rows. Each GPU Y is compared with the exact result
(float64 everywhere: no fp16 rounding of the rotated input, no bf16 rounding
of Y); its RMS error and worst-column RMS error are set beside those of the
oracle's own Y (fp16 Xr, float64 accumulation, bf16 Y), which is the best
any fp32 summation order can reach up to the two roundings.

Why a tolerance of 1e-3 (relative) and not zero: an fp32 sum and a float64
sum round to different bf16 values only where the exact value sits within
about 1e-6 (relative) of a bf16 rounding boundary, and there both roundings
are half an ulp from it, so such a flip moves a squared error by a few parts
per million of an ulp squared. Measured, the GPU's figures equal the
oracle's to four digits in every plan at both row counts; 1e-3 is that
agreement, far below the change one dropped tile or wrong sign makes (it
moves Y by more than a tenth of its largest value).
"""

import numpy as np
import pytest

import gpu_util as G
from oracle import exl3_oracle as O

pytestmark = pytest.mark.gpu

NO_WORSE = 1e-3


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
    return float(rms), float(col.max())


# (K, N, bits, splits to force besides the plan's)
CASES = [(5120, 1024, 4, (2, 4, 8)), (17408, 512, 4, (4, 15)), (5120, 2048, 3, (2, 8)), (5120, 768, 6, (4,))]


@pytest.mark.parametrize("K,N,bits,others", CASES)
def test_error_no_worse_at_16_and_128_rows_in_any_plan(K, N, bits, others):
    L = G.layer("errors", f"{K}x{N}b{bits}", K, N, bits)
    w = G.upload(L)
    plan = ex().exl3_plan(K, N, bits).splits
    for M in (16, 128):
        x = G.xbits("errors", M, K)
        xd = G.dev_bf16(x)
        exact = O.linear_packed(L.words, K, N, bits, L.scales, L.suh, L.svh, x, exact=True)
        ref = O.bf16_to_f64(O.linear_packed(L.words, K, N, bits, L.scales, L.suh, L.svh, x))
        o_rms, o_col = _errors(ref, exact)
        by_plan = {}
        for s in (0,) + tuple(others):
            ex().exl3_test_force(-1, -1, s)
            y = O.bf16_to_f64(G.host_u16(G.run(w, xd, tag=f"error report S={s or plan} M={M}")))
            by_plan[s or plan] = _errors(y, exact)
        ex().exl3_test_force(-1, -1, 0)
        p_rms, p_col = by_plan[plan]
        for s, (g_rms, g_col) in by_plan.items():
            G.say(f"K={K} N={N} b={bits} M={M} S={s}{' (plan)' if s == plan else ''}: RMS err {g_rms:.5e} "
                  f"(oracle {o_rms:.5e}), worst column {g_col:.5e} (oracle {o_col:.5e})")
            # the GPU's fp32 order against the float64 sum: no worse
            assert g_rms <= o_rms * (1 + NO_WORSE), (M, s, g_rms, o_rms)
            assert g_col <= o_col * (1 + NO_WORSE), (M, s, g_col, o_col)
            # a changed K split against the plan's order: no worse either
            assert g_rms <= p_rms * (1 + NO_WORSE), (M, s, g_rms, p_rms)
            assert g_col <= p_col * (1 + NO_WORSE), (M, s, g_col, p_col)
