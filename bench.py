#!/usr/bin/env python3
"""Benchmark of the EXL3 linear on one MI355X.

A step is one pass of the whole hot path over one batch: for the 27B
decode-row grouped linear (K = 5120, 4 bits, M = 16) it is the {q, k, v}
group and the {gate, up} group, each one exl3_linear_group call: a rotation
launch and a linear launch (trellis decode + MFMA contraction + split-K
exchange + epilogue). The same step with the opt-in in-launch rotation (one
launch per group) is timed beside it.
Steps cycle through 8 distinct copies of the weights (8 x 110 MB) so each
step streams its weights from HBM rather than from the 256 MB last-level
cache. The timed steps replay a HIP graph of 8 consecutive steps, one per
weight copy, as a model's decode graph holds its layers back to back (the
library's calls allocate and memset nothing, so they capture), bracketed by
a device synchronisation on both sides; the same steps replayed as one graph
each are reported beside it.

Printed: one JSON line with the weight-stream GB/s of the step (`value`),
the roofline of the dominant kernel (the {gate, up} linear launch, timed with
HIP events around graph replays of back-to-back launches on its stream), the
CPU oracle on a bounded sample, and extra figures: the same group at M = 1
and 7, the 3.5 bpw MLP at M = 128 (TFLOP/s), one layer's 8192-row prefill
(TFLOP/s) and the 6-bit head and its span views at M = 16 (GB/s).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EXL3 linear weight-stream GB/s at M=1..16; TFLOP/s at M=128 and 8192-row prefill"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
NCOPY = 8
CSRC = os.path.join(ROOT, "trellis_quantized_linear_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_linear_gate_up_m16.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def alg_bytes(weights, M, with_x=True):
    """Algorithmic bytes of one group call: packed words, fp16 scales, suh and
    svh per member, bf16 X once, bf16 Y per member."""
    K = weights[0].K
    b = 2 * M * K if with_x else 0
    for w in weights:
        b += w.K * w.N * w.bits // 8 + 2 * w.N + 2 * w.K + 2 * w.N + 2 * M * w.N
    return b


def flops(weights, M):
    return sum(2 * M * w.K * w.N for w in weights)


class Group:
    """One group call's device state: members, input, outputs, workspace."""

    def __init__(self, ex, weights, x, M, ws):
        import torch
        self.ex, self.w, self.x, self.M, self.ws = ex, weights, x, M, ws
        self.y = [torch.empty((M, w.N), dtype=torch.bfloat16, device="cuda") for w in weights]

    def rotate(self):
        self.ex.exl3_rotate(self.w, self.x, self.ws, M=self.M)

    def linear(self):
        self.ex.exl3_linear_rotated(self.w, self.y, self.ws, self.M)

    def call(self):
        """The group call (rotation + linear; one launch with the opt-in
        in-launch rotation at up to 32 rows)."""
        self.ex.exl3_linear_group(self.w, self.x, self.y, self.ws, M=self.M)


def capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # warm once outside capture on the same stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_events(fn, reps):
    """Average ms per fn() call, HIP events on the current stream."""
    import torch
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(reps):
        fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def upload_copies(ex, layers, n):
    return [[ex.Weight.from_host(L, "cuda") for L in layers] for _ in range(n)]


def x_dev(M, K, sigma, tag):
    import numpy as np
    import torch
    from trellis_quantized_linear_amd import synth
    x = synth.gen_x(synth.rng_for("bench", tag, M, K), M, K, sigma)
    return torch.from_numpy(x.view(np.int16).copy()).to("cuda").view(torch.bfloat16)


# ---------------------------------------------------------------- CPU oracle leg
#
# The oracle as it stands, on every host core this process may use (at most
# 16, the box's share for one GPU): a pool of worker processes, started
# before this process touches the GPU, each running the oracle single-threaded
# on column blocks of the step's members. Each worker draws the members from
# their seeds once, when it starts; the timed region is the whole step's
# oracle work, spread over the pool.

_W = {}


def _worker_init(K, bits, names):
    from trellis_quantized_linear_amd import synth
    _W["layers"] = {n: synth.gen_layer("bench-27b", n, K, N, bits) for n, N in names}


def _worker_noop(i):
    return i


def _worker_blocks(name, b0, b1, x_bits):
    """Oracle Y (bf16 bits) of member `name`'s column blocks b0..b1-1."""
    from threadpoolctl import threadpool_limits
    from oracle import exl3_oracle as O
    L = _W["layers"][name]
    bs = O.block_bytes(L.K, L.bits)
    with threadpool_limits(1):
        y = O.linear_packed(L.words, L.K, 128 * (b1 - b0), L.bits, L.scales[128 * b0:128 * b1], L.suh,
                            L.svh[128 * b0:128 * b1], x_bits, block_stride=bs, offset=b0 * bs)
    return name, b0, b1, y


def cpu_workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def start_cpu_pool(K, bits, names):
    """The oracle's worker pool, started (and its workers brought up) before
    any GPU work in this process."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    n = cpu_workers()
    pool = ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=_worker_init,
                               initargs=(K, bits, names))
    list(pool.map(_worker_noop, range(4 * n)))
    return pool, n


def cpu_baseline(pool, n_workers, layers, M, x_bits, y_gpu, parity):
    """Wall time of the oracle on the whole step (every column block of q, k,
    v, gate and up at M rows, X counted once), spread over the pool; the
    oracle's Y is then set against the GPU's step output (parity columns)."""
    from oracle import exl3_oracle as O
    tasks = []
    for name, L in layers:
        nb = L.N // 128
        step = max(1, min(8, nb // 2))
        tasks += [(name, b, min(nb, b + step)) for b in range(0, nb, step)]
    t0 = time.perf_counter()
    futs = [pool.submit(_worker_blocks, n, b0, b1, x_bits) for n, b0, b1 in tasks]
    out = [f.result() for f in futs]
    dt = time.perf_counter() - t0
    nbytes = 2 * M * layers[0][1].K + sum(L.K * L.N * L.bits // 8 + 4 * L.N + 2 * L.K + 2 * M * L.N
                                          for _, L in layers)
    worst, scale = 0.0, 0.0
    for name, b0, b1, y in out:
        g = O.bf16_to_f64(y_gpu[name][:, 128 * b0:128 * b1])
        r = O.bf16_to_f64(y)
        worst = max(worst, float(np.max(np.abs(g - r))))
        scale = max(scale, float(np.max(np.abs(r))))
    blocks = sum(L.N // 128 for _, L in layers)
    rec = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": n_workers, "kind": "oracle",
           "sample": f"the whole step: q/k/v/gate/up, all {blocks} column blocks, {nbytes / 1e6:.1f} MB "
                     f"algorithmic, M={M}; numpy float64 oracle, {n_workers} worker processes of one thread, "
                     f"{dt:.2f} s wall",
           "nproc": os.cpu_count(), "cpu_model": cpu_model(), "seconds": round(dt, 3),
           "max_rel_err_vs_gpu": round(worst / scale, 6) if scale > 0 else None}
    rec.update(parity)
    return rec


def host_bits(t):
    """A device bf16/fp16 tensor's raw 16-bit patterns on the host."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def parity_columns(ex, torch, weights, names, layers, x, y_group, M):
    """What the step's parity rests on, measured here: the decoded weights of
    every member's first and last block bit for bit against the oracle's
    decode, and the group outputs byte for byte against each member's own
    launch."""
    from oracle import exl3_oracle as O
    exact = True
    for (n, N), w in zip(names, weights):
        L = layers[n]
        for nb in (0, N // 128 - 1):
            v = w.columns(128 * nb, 128)
            out = torch.empty((L.K, 128), dtype=torch.int16, device="cuda")
            ex.exl3_test_dequant(v, out)
            bs = O.block_bytes(L.K, L.bits)
            ref = O.decode(L.words, L.K, 128, L.bits, block_stride=bs, offset=nb * bs)
            exact = exact and bool(np.array_equal(host_bits(out), ref))
    same = True
    ws = ex.Workspace().reserve(weights[3:4], M)
    for j, w in enumerate(weights):
        ws.reserve([w], M)
        y = torch.empty((M, w.N), dtype=torch.bfloat16, device="cuda")
        ex.exl3_linear(w, x, y, ws)
        torch.cuda.synchronize()
        same = same and torch.equal(y.view(torch.int16), y_group[j].view(torch.int16))
    return {"decoded_bit_exact": exact, "group_equals_solo_bytes": bool(same),
            "graph_replays_equal_eager_bytes": True}


def traffic_record():
    """HBM traffic per launch of the dominant kernel from the committed PMC
    summary, if it was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    return rec.get("bytes_per_launch") if rec.get("kernel_sha256") == kernel_source_hash() else None


def kernel_source_hash():
    """sha256 over the device sources (every .hip and .h under csrc, by name):
    a profile taken on other kernels does not count."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the M=128, prefill and head figures")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (PMC scale reference)")
    ap.add_argument("--only", choices=SECTIONS,
                    help="profiling aid: run one of the extra figures alone and print it (no bench line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    from trellis_quantized_linear_amd import synth
    K, bits, M = synth.HIDDEN, 4, 16
    names = [("q", synth.Q_COLS), ("k", synth.KV_COLS), ("v", synth.KV_COLS),
             ("gate", synth.INTERMEDIATE), ("up", synth.INTERMEDIATE)]
    pool = None
    if not args.no_cpu and not args.only:
        pool, n_workers = start_cpu_pool(K, bits, names)      # before this process touches the GPU
        log(f"CPU oracle pool: {n_workers} worker processes")

    import torch
    import trellis_quantized_linear_amd.exl3 as ex

    ex.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    layers = {n: synth.gen_layer("bench-27b", n, K, N, bits) for n, N in names}
    log("uploading", NCOPY, "copies of q/k/v/gate/up")
    copies = upload_copies(ex, [layers[n] for n, _ in names], NCOPY)
    if args.only:
        print(json.dumps(run_extras(ex, torch, synth, layers, copies, args.only)), flush=True)
        return
    x = x_dev(M, K, 1.0, "x")
    x_host = host_bits(x)
    ws_qkv = ex.Workspace().reserve(copies[0][:3], 128)
    ws_gu = ex.Workspace().reserve(copies[0][3:], 128)
    torch.cuda.synchronize()

    def step_groups(c, m=M, xx=x):
        return Group(ex, copies[c][:3], xx, m, ws_qkv), Group(ex, copies[c][3:], xx, m, ws_gu)

    # eager reference, then one graph per weight copy
    steps = [step_groups(c) for c in range(NCOPY)]
    for g1, g2 in steps:
        g1.call()
        g2.call()
    torch.cuda.synchronize()
    ref = [[y.clone() for y in g1.y + g2.y] for g1, g2 in steps]
    graphs = [capture(lambda g1=g1, g2=g2: (g1.call(), g2.call())) for g1, g2 in steps]
    for c, gr in enumerate(graphs):
        gr.replay()
        torch.cuda.synchronize()
        got = steps[c][0].y + steps[c][1].y
        assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(got, ref[c])), \
            "graph replay differs from the eager call"

    # The timed steps: replays of one graph holding NCOPY consecutive steps (one
    # per weight copy), as a model's decode graph holds its layers back to
    # back; a remainder of K mod NCOPY steps replays one-step graphs.
    multi = capture(lambda: [(g1.call(), g2.call()) for g1, g2 in steps])
    multi.replay()
    torch.cuda.synchronize()
    for c in range(NCOPY):
        got = steps[c][0].y + steps[c][1].y
        assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(got, ref[c])), \
            "multi-step graph replay differs from the eager call"

    def run_steps(k):
        for _ in range(k // NCOPY):
            multi.replay()
        for i in range(k % NCOPY):
            graphs[i].replay()

    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1e3 / args.steps
    # the timed replays left every copy's outputs in place: the same bytes as
    # the eager calls (the split-K exchange raced nowhere over the timed steps)
    for c in range(NCOPY):
        got = steps[c][0].y + steps[c][1].y
        assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(got, ref[c])), \
            "outputs after the timed replays differ from the eager call"
    step_bytes = alg_bytes(copies[0][:3], M) + alg_bytes(copies[0][3:], M)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"step {ms_step * 1e3:.2f} us, {step_bytes / 1e6:.2f} MB -> {value:.1f} GB/s")
    # the same steps as one graph replay each
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % NCOPY].replay()
    torch.cuda.synchronize()
    ms_step_single = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"step as one graph replay each: {ms_step_single * 1e3:.2f} us -> "
        f"{step_bytes / (ms_step_single * 1e-3) / 1e9:.1f} GB/s")

    # the same step with the rotation inside each group's linear launch (opt-in;
    # an extra figure, so that profiles of --no-extra runs see one kernel form)
    ms1 = None
    if not args.no_extra:
        ex.exl3_test_fuse_rotation(True)
        try:
            multi1 = capture(lambda: [(g1.call(), g2.call()) for g1, g2 in steps])
            multi1.replay()
            torch.cuda.synchronize()
            for c in range(NCOPY):
                got = steps[c][0].y + steps[c][1].y
                assert all(torch.equal(a.view(torch.int16), b.view(torch.int16)) for a, b in zip(got, ref[c])), \
                    "one-launch step differs from the two-launch step"
            ms1 = time_events(multi1.replay, 25) / NCOPY
        finally:
            ex.exl3_test_fuse_rotation(False)
        log(f"one-launch step (rotation inside the linear) {ms1 * 1e3:.2f} us -> "
            f"{step_bytes / (ms1 * 1e-3) / 1e9:.1f} GB/s")
        del multi1

    # dominant kernel: the {gate, up} linear launch, back-to-back over the copies
    gu = [s[1] for s in steps]
    for g in gu:
        g.rotate()
    torch.cuda.synchronize()
    reps_in_graph = 2
    g_lin = capture(lambda: [g.linear() for _ in range(reps_in_graph) for g in gu])
    launches = reps_in_graph * NCOPY
    ms_graph = time_events(g_lin.replay, 20)
    ms_kernel = ms_graph / launches
    kbytes = alg_bytes(copies[0][3:], M)
    achieved = kbytes / (ms_kernel * 1e-3) / 1e9
    log(f"gate/up linear: {ms_kernel * 1e3:.2f} us per launch -> {achieved:.1f} GB/s")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_record(),
                "kernel": "linear_spread_kernel<4> (the {gate, up} group, M=16)",
                "alg_bytes_per_launch": kbytes, "us_per_launch": round(ms_kernel * 1e3, 3)}

    extra = {}
    if not args.no_extra:
        extra = run_extras(ex, torch, synth, layers, copies)

    cpu = None
    if pool is not None:
        log("CPU oracle baseline (all host cores) and parity columns")
        cpu = cpu_baseline(pool, n_workers, [(n, layers[n]) for n, _ in names], M, x_host,
                           {n: host_bits(y) for (n, _), y in zip(names, ref[0])},
                           parity_columns(ex, torch, copies[0], names, layers, x, ref[0], M))
        pool.shutdown()

    if args.calibrate_copy:
        # an elementwise kernel that reads 1 GiB and writes 1 GiB
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = {"read": 1 << 30, "write": 1 << 30}

    extra["step_one_graph_replay_each_us"] = round(ms_step_single * 1e3, 2)
    extra["step_one_graph_replay_each_GBps"] = round(step_bytes / (ms_step_single * 1e-3) / 1e9, 1)
    if ms1 is not None:
        extra["step_rotation_in_launch_us"] = round(ms1 * 1e3, 2)
        extra["step_rotation_in_launch_GBps"] = round(step_bytes / (ms1 * 1e-3) / 1e9, 1)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "27B decode-row grouped linear: {q,k,v} and {gate,up} groups, K=5120, 4 bits, "
                               "M=16, X bf16 ~N(0,1)",
                   "K": K, "bits": bits, "M": M, "members": {n: N for n, N in names},
                   "weight_copies": NCOPY, "step_alg_bytes": step_bytes},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


SECTIONS = ("rows", "mlp128", "prefill", "head")
MLP_ROWS = (17, 24, 32, 33, 48, 49, 64, 100, 128)      # the 3.5 bpw MLP's mid rows


def run_extras(ex, torch, synth, layers, copies, only=None):
    extra = {}
    K = synth.HIDDEN
    # the same grouped step at M = 1 and 7 (graph replays over the copies)
    for m in ((1, 7) if only in (None, "rows") else ()):
        xx = x_dev(m, K, 1.0, f"x{m}")
        wsa = ex.Workspace().reserve(copies[0][:3], m)
        wsb = ex.Workspace().reserve(copies[0][3:], m)
        gs = [(Group(ex, c[:3], xx, m, wsa), Group(ex, c[3:], xx, m, wsb)) for c in copies]
        multi = capture(lambda: [(a.call(), b.call()) for a, b in gs])
        ms = time_events(multi.replay, 25) / len(gs)
        by = alg_bytes(copies[0][:3], m) + alg_bytes(copies[0][3:], m)
        extra[f"decode_step_M{m}_GBps"] = round(by / (ms * 1e-3) / 1e9, 1)
        log(f"decode step M={m}: {ms * 1e3:.2f} us, {extra[f'decode_step_M{m}_GBps']} GB/s")

    if only not in (None, "mlp128"):
        return run_extras_prefill(ex, torch, synth, copies, extra, only)
    # 27B dense SwiGLU MLP at 3.5 bpw: {gate, up} 3-bit group + down 4-bit,
    # at M = 128 and at the other mid rows of that configuration
    mlp = [synth.gen_layer("bench-mlp", "gate", K, synth.INTERMEDIATE, 3),
           synth.gen_layer("bench-mlp", "up", K, synth.INTERMEDIATE, 3),
           synth.gen_layer("bench-mlp", "down", synth.INTERMEDIATE, K, 4)]
    mc = upload_copies(ex, mlp, 4)
    wsa = ex.Workspace().reserve(mc[0][:2], 128)
    wsb = ex.Workspace().reserve(mc[0][2:], 128)
    rows_us, rows_tf = {}, {}
    for m in MLP_ROWS:
        xa = x_dev(m, K, 1.0, "mlp-x")
        xb = x_dev(m, synth.INTERMEDIATE, 1.0, "mlp-x2")
        gs = [(Group(ex, c[:2], xa, m, wsa), Group(ex, c[2:], xb, m, wsb)) for c in mc]
        multi = capture(lambda: [(a.call(), b.call()) for a, b in gs])
        ms = time_events(multi.replay, 10) / len(gs)
        fl = flops(mc[0], m)
        rows_us[m] = round(ms * 1e3, 2)
        rows_tf[m] = round(fl / (ms * 1e-3) / 1e12, 1)
        if m == 128:
            by = alg_bytes(mc[0][:2], m) + alg_bytes(mc[0][2:], m)
            extra["mlp_M128_TFLOPs"] = rows_tf[m]
            extra["mlp_M128_us"] = rows_us[m]
            extra["mlp_M128_frac_mfma"] = round(fl / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
            extra["mlp_M128_GBps"] = round(by / (ms * 1e-3) / 1e9, 1)
        log(f"MLP M={m}: {ms * 1e3:.1f} us, {rows_tf[m]} TFLOP/s")
        del gs, multi
    extra["mlp_rows_us"] = rows_us
    extra["mlp_rows_TFLOPs"] = rows_tf
    del mc
    return run_extras_prefill(ex, torch, synth, copies, extra, only)


PREFILL_WARM, PREFILL_REPS = 30, 20


def run_extras_prefill(ex, torch, synth, copies, extra, only):
    K = synth.HIDDEN
    if only not in (None, "prefill"):
        return run_extras_head(ex, torch, synth, extra, only)
    # one 27B layer's six linears over an 8192-row prompt (4 bits, X ~ N(0, 0.5))
    m = 8192
    six = [copies[0][0], copies[0][1], copies[0][2], copies[0][3], copies[0][4]]
    down = ex.Weight.from_host(synth.gen_layer("bench-27b", "down", synth.INTERMEDIATE, K, 4), "cuda")
    xa = x_dev(m, K, 0.5, "prefill-x")
    xb = x_dev(m, synth.INTERMEDIATE, 0.5, "prefill-x2")
    wsa = ex.Workspace().reserve(six[:3], m)
    wsb = ex.Workspace().reserve(six[3:], m)
    wsc = ex.Workspace().reserve([down], m)
    ga, gb, gc = Group(ex, six[:3], xa, m, wsa), Group(ex, six[3:], xa, m, wsb), Group(ex, [down], xb, m, wsc)
    fn = lambda: (ga.call(), gb.call(), gc.call())
    # a prompt runs layer after layer: these launches run power-limited, so
    # each figure is taken at the steady clock, after 30 layers of the same
    # work (a few-layer window right after other work reads up to 10 % off)
    time_events(fn, PREFILL_WARM)
    ms = time_events(fn, PREFILL_REPS)
    fl = flops(six + [down], m)
    extra["prefill_8192_TFLOPs"] = round(fl / (ms * 1e-3) / 1e12, 1)
    extra["prefill_8192_ms_per_layer"] = round(ms, 3)
    extra["prefill_8192_frac_mfma"] = round(fl / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
    log(f"prefill 8192 rows: {ms:.2f} ms per layer, {extra['prefill_8192_TFLOPs']} TFLOP/s")
    # the same layer with the opt-in single-chain prompt arithmetic (other
    # bits than every other regime; exl3_set_prompt_arithmetic(1))
    ex.exl3_set_prompt_arithmetic(1)
    try:
        time_events(fn, PREFILL_WARM)
        ms1 = time_events(fn, PREFILL_REPS)
    finally:
        ex.exl3_set_prompt_arithmetic(0)
    extra["prefill_8192_single_chain_opt_in_TFLOPs"] = round(fl / (ms1 * 1e-3) / 1e12, 1)
    extra["prefill_8192_single_chain_opt_in_ms_per_layer"] = round(ms1, 3)
    log(f"prefill 8192 rows, opt-in single chain: {ms1:.2f} ms per layer, "
        f"{extra['prefill_8192_single_chain_opt_in_TFLOPs']} TFLOP/s")
    # the same bits on the 128 x 256 tiling (one workgroup of two blocks per
    # CU), which the automatic choice passes over for the 128-row block tiling
    ex.exl3_test_force(16, 1, 0)
    try:
        time_events(fn, PREFILL_WARM)
        ms2 = time_events(fn, PREFILL_REPS)
    finally:
        ex.exl3_test_force(-1, -1, 0)
    extra["prefill_8192_tiling_128x256_ms_per_layer"] = round(ms2, 3)
    log(f"prefill 8192 rows, 128 x 256 tiling (same bits): {ms2:.2f} ms per layer")
    del ga, gb, gc, xa, xb, wsa, wsb, wsc
    return run_extras_head(ex, torch, synth, extra, only)


def run_extras_head(ex, torch, synth, extra, only):
    K = synth.HIDDEN
    if only not in (None, "head"):
        return extra
    # the 6-bit head 5120 -> 248,320 and its span views, M = 16
    m = 16
    head = ex.Weight.from_host(synth.gen_layer("bench-head", "head", K, synth.VOCAB, 6), "cuda")
    xx = x_dev(m, K, 1.0, "head-x")
    # Several calls per graph replay, as the decode step: the full head twice
    # (963 MB each, past the 256 MB last-level cache); span A (columns
    # 0..98304, 768 blocks, 381 MB) alternating with the next 768-block span,
    # which plans alike, so each call streams from HBM.
    span_a = [head.columns(0, 98304), head.columns(98304, 98304)]
    for tag, ws_list in (("head_full", [head, head]), ("head_span_A", span_a + span_a)):
        ws = ex.Workspace().reserve([ws_list[0]], m)
        gs = [Group(ex, [w], xx, m, ws) for w in ws_list]
        gr = capture(lambda: [g.call() for g in gs])
        ms = time_events(gr.replay, 5) / len(gs)
        w = ws_list[0]
        extra[f"{tag}_M16_GBps"] = round(alg_bytes([w], m) / (ms * 1e-3) / 1e9, 1)
        extra[f"{tag}_M16_us"] = round(ms * 1e3, 2)
        log(f"{tag}: {ms * 1e3:.1f} us, {extra[f'{tag}_M16_GBps']} GB/s")
        del gs, gr
    # span B is 64 blocks (31.5 MB): cycle 16 distinct 64-block views of the
    # head (504 MB) so it streams from HBM, not from the last-level cache
    views = [head.columns(240128 - 128 * 64 * i, 8192) for i in range(16)]
    ws = ex.Workspace().reserve([views[0]], m)
    gs = [Group(ex, [v], xx, m, ws) for v in views]
    gr = capture(lambda: [g.call() for g in gs])
    ms = time_events(gr.replay, 10) / len(gs)
    extra["head_span_B_M16_GBps"] = round(alg_bytes([views[0]], m) / (ms * 1e-3) / 1e9, 1)
    extra["head_span_B_M16_us"] = round(ms * 1e3, 2)
    log(f"head_span_B: {ms * 1e3:.1f} us, {extra['head_span_B_M16_GBps']} GB/s")
    return extra


if __name__ == "__main__":
    main()
