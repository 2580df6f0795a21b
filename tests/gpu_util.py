"""Helpers shared by the GPU tests: upload seeded inputs, run the library,
run the oracle on sampled column blocks, compare.

Every GPU step prints (and flushes) what it is about to run, so a run that
dies names its case.
"""

from __future__ import annotations

import numpy as np

from oracle import exl3_oracle as O
from trellis_quantized_linear_amd import synth


def torch_mod():
    import torch
    return torch


def say(*a):
    print("[gpu]", *a, flush=True)


def dev_u16(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).to("cuda")


def dev_bf16(a):
    return dev_u16(a).view(torch_mod().bfloat16)


def host_u16(t):
    return t.contiguous().view(torch_mod().int16).cpu().numpy().view(np.uint16)


def upload(layer):
    import trellis_quantized_linear_amd.exl3 as ex
    return ex.Weight.from_host(layer, "cuda")


def empty_y(M, N):
    torch = torch_mod()
    return torch.full((M, N), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def run(w, x_dev, M=None, ws=None, stream=None, tag=""):
    """One exl3_linear call; returns the bf16 output tensor."""
    import trellis_quantized_linear_amd.exl3 as ex
    M = x_dev.shape[0] if M is None else M
    y = empty_y(max(M, 1), w.N)
    if ws is None:
        ws = ex.Workspace().reserve([w], max(M, 1))
    say(f"exl3_linear {tag} K={w.K} N={w.N} bits={w.bits} M={M}")
    ex.exl3_linear(w, x_dev, y, ws, stream=stream, M=M)
    return y


def run_group(ws_list, x_dev, M=None, ws=None, tag=""):
    import trellis_quantized_linear_amd.exl3 as ex
    M = x_dev.shape[0] if M is None else M
    ys = [empty_y(M, w.N) for w in ws_list]
    if ws is None:
        ws = ex.Workspace().reserve(ws_list, M)
    say(f"exl3_linear_group {tag} members={[w.N for w in ws_list]} M={M}")
    ex.exl3_linear_group(ws_list, x_dev, ys, ws, M=M)
    return ys


def oracle_blocks(layer, x_bits, blocks, rows=None):
    """Oracle Y (bf16 bits) of the listed 128-column blocks, [M, 128*len]."""
    bs = O.block_bytes(layer.K, layer.bits)
    xs = x_bits if rows is None else x_bits[rows]
    out = []
    for nb in blocks:
        cols = slice(128 * nb, 128 * (nb + 1))
        out.append(O.linear_packed(layer.words, layer.K, 128, layer.bits, layer.scales[cols], layer.suh,
                                   layer.svh[cols], xs, block_stride=bs, offset=nb * bs))
    return np.concatenate(out, axis=1)


def gpu_blocks(y_dev, blocks, rows=None):
    y = host_u16(y_dev)
    if rows is not None:
        y = y[rows]
    return np.concatenate([y[:, 128 * nb:128 * (nb + 1)] for nb in blocks], axis=1)


def assert_close(got_bits, ref_bits, rel=1e-2, what=""):
    """Y within rel * max|Y_oracle| element by element (the parity bar),
    with NaN positions identical and infinities identical."""
    g = O.bf16_to_f64(got_bits)
    r = O.bf16_to_f64(ref_bits)
    assert np.array_equal(np.isnan(g), np.isnan(r)), f"{what}: NaN positions differ"
    fin = np.isfinite(r)
    assert np.array_equal(np.isinf(g), np.isinf(r)) and np.array_equal(g[np.isinf(r)], r[np.isinf(r)]), \
        f"{what}: infinities differ"
    if not fin.any():
        return 0.0
    scale = np.max(np.abs(r[fin]))
    err = np.max(np.abs(g[fin] - r[fin]))
    say(f"{what}: max|Y-oracle| = {err:.3e} ({err / max(scale, 1e-300):.2e} of max|Y|)")
    assert err <= rel * scale, f"{what}: error {err} > {rel} * {scale}"
    return err / max(scale, 1e-300)


def sample_blocks(n_blocks, k=4, seed=0):
    rng = np.random.default_rng(seed)
    pick = {0, n_blocks - 1}
    while len(pick) < min(k, n_blocks):
        pick.add(int(rng.integers(0, n_blocks)))
    return sorted(pick)


def layer(config, name, K, N, bits):
    return synth.gen_layer(config, name, K, N, bits)


def xbits(config, M, K, sigma=1.0, tag="x"):
    return synth.gen_x(synth.rng_for(config, tag, M, K), M, K, sigma)
