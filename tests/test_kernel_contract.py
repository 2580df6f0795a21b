"""The kernel contract on the CPU (no kernel runs): the dispatch sweep, the
registry's gate shapes, and the compiler's resource records of every
registered form (TensorFold PR #1467, author follow-up, "A dispatch test";
"Receipt", "Kernel contract", gate 5: every launch carries a resource
record).

* The sweep calls the library's dispatch (mock mode: launches are recorded,
  not issued) over K, N in 128..16384 (and the 27B's 17408 and
  248,320), 1 to 128 rows and the prompt rows 129, 200, 300 and 8192, for
  single weights and for groups of two and three members, in the default
  mode, the opt-in prompt arithmetic and with the in-launch rotation. It
  fails when it reaches a form the registry lacks; the planted control removes
  one registration and must see the sweep fail on it.
* Every registered gate shape, at every width, must reach its form.
* The build's resource records (kernel_resources.json, from the compiler's
  -Rpass-analysis=kernel-resource-usage remarks) must cover every registered
  form: no scratch, no spilled registers, the occupancy the launch was built
  for, and LDS for that many workgroups per CU.
"""

import ctypes
import itertools
import json
import os

import pytest

import kernel_contract as KC
import trellis_quantized_linear_amd.exl3 as ex
from trellis_quantized_linear_amd import _build

KS = [128, 256, 384, 512, 640, 1024, 2048, 4096, 5120, 8192, 16384, 17408]
NS = [128, 256, 384, 512, 1024, 2048, 4096, 5120, 6144, 8192, 16384, 17408, 24576, 34816, 65536, 248320]
MS = list(range(1, 129)) + [129, 200, 300, 8192]
GROUP_MS = [1, 7, 16, 17, 24, 32, 33, 48, 49, 64, 65, 96, 97, 100, 128, 129, 300]


@pytest.fixture(scope="module")
def lib():
    return ex.lib()


@pytest.fixture(autouse=True)
def _modes(lib):
    ex.exl3_test_force(-1, -1, 0)
    ex.exl3_set_prompt_arithmetic(0)
    ex.exl3_test_fuse_rotation(False)
    ex.exl3_test_mock(True)
    yield
    ex.exl3_test_mock(False)
    ex.exl3_test_mock_counts()
    ex.exl3_set_prompt_arithmetic(0)
    ex.exl3_test_fuse_rotation(False)


def _desc(K, N, bits, j):
    base = 0x10000000 * (j + 1)
    return ex.exl3_weight_t(base, base + 0x4000000, base + 0x8000000, base + 0xC000000, K, N, 16 * K * bits, bits, 0)


_WS = ex.exl3_workspace_t(0x800000000, 1 << 44, 1 << 28)


def dispatch_form(lib, K, Ns, M, bits=4, mode=""):
    """The form the dispatch picks for this call (mock mode), or None if the
    call is refused."""
    ex.exl3_set_prompt_arithmetic(1 if mode == "prompt1" else 0)
    ex.exl3_test_fuse_rotation(mode == "rot")
    descs = [_desc(K, N, bits, j) for j, N in enumerate(Ns)]
    n = len(descs)
    arr = (ex.W_P * n)(*[ctypes.pointer(d) for d in descs])
    ys = (ctypes.c_void_p * n)(*[0x900000000 + j * 0x40000000 for j in range(n)])
    ld = (ctypes.c_int64 * n)(*Ns)
    rc = lib.exl3_linear_group(n, arr, 0xA00000000, K, M, ys, ld, ctypes.byref(_WS), None)
    ex.exl3_set_prompt_arithmetic(0)
    ex.exl3_test_fuse_rotation(False)
    return ex.exl3_test_last_form() if rc == ex.EXL3_OK else None


def sweep(lib):
    """{form reached: first call that reached it}, at 4 bits (the dispatch
    does not depend on the width; the form names carry it)."""
    seen = {}

    def note(form, what):
        if form and form not in seen:
            seen[form] = what

    for K, N in itertools.product(KS, NS):
        for M in MS:
            note(dispatch_form(lib, K, [N], M), (K, [N], M, ""))
        for M in (129, 300, 8192):
            note(dispatch_form(lib, K, [N], M, mode="prompt1"), (K, [N], M, "prompt1"))
        for M in range(1, 33):
            note(dispatch_form(lib, K, [N], M, mode="rot"), (K, [N], M, "rot"))
    for K in KS:
        for n in (2, 3):
            for Ns in itertools.combinations_with_replacement(NS[:13], n):
                for M in GROUP_MS:
                    note(dispatch_form(lib, K, list(Ns), M), (K, list(Ns), M, ""))
                for M in (1, 16, 17, 32):
                    note(dispatch_form(lib, K, list(Ns), M, mode="rot"), (K, list(Ns), M, "rot"))
    return seen


def unregistered(seen, forms=None):
    reg = KC.registered(forms)
    return {f: what for f, what in seen.items() if f not in reg}


@pytest.fixture(scope="module")
def swept(lib):
    ex.exl3_test_mock(True)
    s = sweep(lib)
    ex.exl3_test_mock(False)
    return s


def test_every_reachable_form_is_registered(swept):
    missing = unregistered(swept)
    assert not missing, "unregistered: " + "; ".join(f"{f} ({w})" for f, w in missing.items())
    # and the sweep reaches every registered form at 4 bits (no dead registrations)
    reg4 = {f for f, (b, _, _) in KC.registered().items() if b == 4}
    assert reg4 == set(swept), reg4 ^ set(swept)


def test_planted_control_an_unregistered_form_fails_the_sweep(swept):
    """Remove the 3-bit-style control of the pages: drop one registration
    (the spread launch over row blocks) and the sweep must name it."""
    forms = dict(KC.FORMS)
    del forms["linear_spread_rows_kernel<{b}>"]
    missing = unregistered(swept, forms)
    assert set(missing) == {"linear_spread_rows_kernel<4>"}, missing


def test_every_gate_reaches_its_form_at_every_width(lib):
    for form, (bits, _, gates) in KC.registered().items():
        for K, Ns, M, mode in gates:
            got = dispatch_form(lib, K, Ns, M, bits=bits, mode=mode)
            assert got == form, (form, (K, Ns, M, mode), got)


def test_resource_records_of_every_registered_form():
    path = _build.RESOURCES
    assert os.path.exists(path), f"{path} is written by the build; build the library first"
    rec = json.load(open(path))
    problems = []
    for form, (bits, waves, _) in KC.registered().items():
        name = form.replace(" +rot", "")
        r = rec.get(name)
        if r is None:
            problems.append(f"{name}: no resource record")
            continue
        if r["scratch"] != 0 or r["vgpr_spill"] != 0 or r["sgpr_spill"] != 0:
            problems.append(f"{name}: spills (scratch {r['scratch']} B/lane, {r['vgpr_spill']} VGPRs, "
                            f"{r['sgpr_spill']} SGPRs)")
        if r["occupancy"] < waves:
            problems.append(f"{name}: occupancy {r['occupancy']} waves/SIMD < {waves} it is built for")
        wgs_per_cu = max(1, waves * 4 // KC.waves_per_workgroup(name))
        if r["lds"] * wgs_per_cu > KC.LDS_PER_CU:
            problems.append(f"{name}: {r['lds']} B of LDS x {wgs_per_cu} workgroups per CU > {KC.LDS_PER_CU}")
    # every other kernel of the library: no scratch either
    for name, r in rec.items():
        if r["scratch"] != 0 or r["vgpr_spill"] != 0 or r["sgpr_spill"] != 0:
            problems.append(f"{name}: spills")
    assert not problems, "\n".join(problems)
