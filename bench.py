"""Benchmark of the sliced-integer (Matryoshka-nested) matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]

One step is one decode pass (batch 1) through the Gemma-2-9B MLP matrices
(up/gate 3584 -> 14336, down 14336 -> 3584, per-channel scales, 0.1% x10
outlier weights) at each slice precision r = 8, 4, 2: the nine products in
one mixed-precision GEMV launch (mq_gemv_mixed).  Weights rotate over
>= 1 GiB of distinct copies per r so that the 256 MB last-level cache cannot
serve them.  `value` is the effective HBM bandwidth over the step:
algorithmic bytes (packed plane + fp32 alpha/zero + bf16 x + fp32 y) per
second.

The same JSON line also carries:
  roofline      the step's kernel against 8 TB/s, its duration measured live
                with HIP events on the launch stream over the timed region
                (single-r launches are timed afterwards for reference);
  rows          the other steps of the path measured in the same run: pack,
                small-batch GEMM (Mistral shapes, g128), prefill GEMM
                (M = 2048), the 32-layer Mix'n'Match stack and the
                Extra-Precision sparse addition (r = 2, Gemma MLP);
  cpu_baseline  the float64 CPU oracle on the same workload (host cores).

Only one GPU is used; --gpus above 1 exits with a message.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s (GEMV) & TFLOP/s (GEMM) of sliced-int matmul at r=8/4/2"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 1 << 30
RS = (8, 4, 2)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_gemma9b_mlp.md")
GEMV_SOURCE = os.path.join(ROOT, "nested_int_matmul_amd", "csrc", "gemv.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def linear_bytes(n, k, r, group, m):
    """Algorithmic bytes of one product: packed plane, fp32 alpha and zero,
    bf16 activations, fp32 outputs."""
    g = k // group
    return n * k * r // 8 + 8 * n * g + 2 * m * k + 4 * m * n


class Timer:
    """HIP events on the given stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e


# --------------------------------------------------------------------------- main step

def setup_gemma(torch, mq, inputs, dev):
    mats = []
    for i, name in enumerate(("up", "gate", "down")):
        n, k = inputs.GEMMA9B_MLP[name]
        w = inputs.device_gaussian_weights("gemma9b_mlp", n, k, dev, matrix=i, outlier_frac=1e-3)
        codes, alpha, zero = mq.quantize(w, k)
        del w
        xb = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=i)
        x = torch.from_numpy(xb.view("int16")).to(dev)
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        mats.append(dict(name=name, N=n, K=k, codes=codes, alpha=alpha, zero=zero, x=x, y=y))
    planes = {}
    for r in RS:
        base = [mq.pack(m["codes"], r) for m in mats]
        mlp_bytes = sum(linear_bytes(m["N"], m["K"], r, m["K"], 1) for m in mats)
        ncopy = max(2, -(-ROTATE_BYTES // mlp_bytes))
        planes[r] = [base] + [[p.clone() for p in base] for _ in range(ncopy - 1)]
    for m in mats:
        del m["codes"]
    torch.cuda.synchronize()
    return mats, planes


def gemma_problems(mq, mats, plane_set):
    return [dict(packed=p, alpha=m["alpha"], zero=m["zero"], x=m["x"], y=m["y"], N=m["N"],
                 K=m["K"], group=m["K"]) for m, p in zip(mats, plane_set)]


def run_main(torch, mq, inputs, dev, steps, warmup):
    mats, planes = setup_gemma(torch, mq, inputs, dev)
    stream = torch.cuda.current_stream()
    T = Timer(torch, stream)
    # one launch per step: the nine products (three matrices at r = 8, 4, 2)
    # through mq_gemv_mixed; prepared plans keep argument marshalling out of
    # the timed loop.  Plan c uses weight copy c (mod the copies of each r).
    ncopy = max(len(planes[r]) for r in RS)
    rs = [r for r in RS for _ in mats]
    plans = []
    for c in range(ncopy):
        probs = []
        for r in RS:
            probs += gemma_problems(mq, mats, planes[r][c % len(planes[r])])
        plans.append(mq.GemvGroupedPlan(probs, rs, 1, stream))
    step_bytes = sum(linear_bytes(m["N"], m["K"], r, m["K"], 1) for m in mats for r in RS)

    def step(i):
        plans[i % ncopy]()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = T.event()
    for j in range(steps):
        step(warmup + j)
    t1 = T.event()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    # spread of single steps: 50 more steps, each between its own two events
    # (the events add their own cost to each reading)
    pairs = []
    for j in range(50):
        a = T.event()
        step(warmup + steps + j)
        pairs.append((a, T.event()))
    torch.cuda.synchronize()
    one = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
    spread = {"p10": round(one[4], 2), "median": round(one[25], 2), "p90": round(one[44], 2),
              "n": 50, "how": "each step between its own two HIP events"}
    # for reference: each r alone (three products per launch), back to back
    # (replayed from a graph: see time_loop)
    per_r_us = {}
    side = torch.cuda.Stream()
    for r in RS:
        single = [mq.GemvGroupedPlan(gemma_problems(mq, mats, ps), r, 1, side)
                  for ps in planes[r]]
        per_r_us[r] = time_loop(torch, lambda i: single[i % len(single)](), max(steps, 50),
                                stream=side)
    # and each matrix alone at each r (one product per launch)
    per_matrix_us = {}
    for r in RS:
        per_matrix_us[f"r{r}"] = {}
        for j, m in enumerate(mats):
            alone = [mq.GemvGroupedPlan(gemma_problems(mq, [m], [ps[j]]), r, 1, side)
                     for ps in planes[r]]
            per_matrix_us[f"r{r}"][m["name"]] = round(
                time_loop(torch, lambda i: alone[i % len(alone)](), 50, stream=side), 2)
    return dict(total_ms=total_ms, step_bytes=step_bytes, per_r_us=per_r_us, mats=mats,
                spread=spread, per_matrix_us=per_matrix_us)


# --------------------------------------------------------------------------- roofline

def traffic_for(source_sha, kernel):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy of known size), if recorded for the
    current kernel source; None otherwise."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip().strip("-* ")] = v.strip().strip("`")
    if rec.get("gemv.hip sha256") != source_sha:
        return None
    v = rec.get(f"traffic bytes per launch {kernel}")
    return float(v) if v else None


def sha256(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


# --------------------------------------------------------------------------- extra rows

def time_loop(torch, fn, iters, warmup=3, stream=None, reps=3):
    """GPU microseconds per call of fn(i), i = 0 .. iters - 1: the calls are
    captured once into a HIP graph on `stream` (a new stream if None) and the
    graph is replayed `reps` times between two events, so that the host's
    per-call argument checks and marshalling (several microseconds in the
    Python binding) do not pace kernels that are only 10-20 us long.  The
    library's entry points launch kernels only (no allocation, copy, memset
    or synchronization), so each call captures as plain kernel nodes."""
    s = stream if stream is not None else torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(warmup):
            fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(iters):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) * 1e3 / (reps * iters)  # us


def time_queued(torch, fn, iters, warmup=3):
    """GPU microseconds per call of fn(i) for launches long enough (hundreds of
    microseconds) that the host queues them far ahead of the GPU: iters calls
    back to back on the current stream between two events.  The prefill rows
    use it: replayed from a HIP graph, the 220-310 us prefill launches measured
    about 30 us slower per call than the same launches queued this way, while
    the short decode and small-batch launches (and the Mix'n'Match stack) time
    the same either way."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(iters):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / iters  # us


def row_pack(torch, mq, inputs, dev):
    """a1: slice-and-pack of the Gemma down matrix (reads N*K, writes N*K*r/8)."""
    n, k = inputs.GEMMA9B_MLP["down"]
    w = inputs.device_gaussian_weights("gemma9b_mlp", n, k, dev, matrix=2, outlier_frac=1e-3)
    codes, _, _ = mq.quantize(w, k)
    del w
    copies = [codes] + [codes.clone() for _ in range(6)]
    pack = {}
    for r in RS:
        outs = [torch.empty((n, k * r // 8), dtype=torch.uint8, device=dev) for _ in copies]
        us = time_loop(torch, lambda i: mq.pack(copies[i % 7], r, out=outs[i % 7]), 21)
        b = n * k * (1 + r / 8)
        pack[f"r{r}"] = {"us": round(us, 2), "GB/s": round(b / us / 1e3, 1)}
    del copies, codes
    return pack


def row_small(torch, mq, inputs, dev):
    """a3: small-batch GEMM, Mistral shapes, group 128."""
    small = {}
    for (N2, K2) in inputs.MISTRAL_SMALL_SHAPES:
        w = inputs.device_gaussian_weights("mistral_small", N2, K2, dev, matrix=N2 // 4096)
        c2, a2, z2 = mq.quantize(w, 128)
        del w
        for r in (4, 2, 6, 3):
            pl = mq.pack(c2, r)
            b1 = linear_bytes(N2, K2, r, 128, 0)
            nc = max(2, -(-ROTATE_BYTES // b1))
            pls = [pl] + [pl.clone() for _ in range(nc - 1)]
            for M2 in (16, 64):
                xb = inputs.activations_bf16("mistral_small", M2, K2, heavy_channels=8)
                x2 = torch.from_numpy(xb.view("int16")).to(dev)
                y2 = torch.empty((M2, N2), dtype=torch.float32, device=dev)
                ws2 = torch.empty(max(1, mq.gemm_workspace_bytes(M2, N2, K2, 128)),
                                  dtype=torch.uint8, device=dev)
                us = time_loop(torch, lambda i: mq.gemm(pls[i % nc], r, a2, z2, 128, N2, K2, x2,
                                                        out=y2, workspace=ws2), 40)
                b = linear_bytes(N2, K2, r, 128, M2)
                small[f"M{M2}_N{N2}_K{K2}_r{r}"] = {
                    "us": round(us, 2), "GB/s": round(b / us / 1e3, 1),
                    "TFLOP/s": round(2 * M2 * N2 * K2 / us / 1e6, 2)}
            del pls, pl
        del c2, a2, z2
    return small


def row_prefill(torch, mq, inputs, dev):
    """a4: prefill GEMM, group 128."""
    M, K, N = inputs.PREFILL_SHAPE
    w = inputs.device_gaussian_weights("prefill", N, K, dev)
    c5, a5, z5 = mq.quantize(w, 128)
    del w
    xb = inputs.activations_bf16("prefill", M, K)
    x5 = torch.from_numpy(xb.view("int16")).to(dev)
    y5 = torch.empty((M, N), dtype=torch.float32, device=dev)
    pre = {}
    ws5 = torch.empty(max(1, mq.gemm_workspace_bytes(M, N, K, 128)), dtype=torch.uint8,
                      device=dev)
    for r in (4, 2, 8, 6, 3):
        pl = mq.pack(c5, r)
        us = time_queued(torch, lambda i: mq.gemm(pl, r, a5, z5, 128, N, K, x5, out=y5,
                                                  workspace=ws5), 30)
        tf = 2 * M * N * K / us / 1e6
        pre[f"r{r}"] = {"us": round(us, 1), "TFLOP/s": round(tf, 1),
                        "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    del c5, a5, z5
    # the same weights with per-channel scales (no group transitions), r = 4
    w = inputs.device_gaussian_weights("prefill", N, K, dev)
    c5, a5, z5 = mq.quantize(w, K)
    del w
    pl = mq.pack(c5, 4)
    us = time_queued(torch, lambda i: mq.gemm(pl, 4, a5, z5, K, N, K, x5, out=y5,
                                              workspace=ws5), 30)
    tf = 2 * M * N * K / us / 1e6
    pre["r4_per_channel"] = {"us": round(us, 1), "TFLOP/s": round(tf, 1),
                             "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    return pre


def row_prefill_down(torch, mq, inputs, dev):
    """a4, the 4096-wide down projection of the same layer (K = 14336): 128
    output tiles at M = 2048, so the kernel splits K over workgroups."""
    M, K, N = inputs.PREFILL_SHAPE
    w = inputs.device_gaussian_weights("prefill", K, N, dev, matrix=1)
    c6, a6, z6 = mq.quantize(w, 128)
    del w
    xb = inputs.activations_bf16("prefill", M, N, matrix=1)
    x6 = torch.from_numpy(xb.view("int16")).to(dev)
    y6 = torch.empty((M, K), dtype=torch.float32, device=dev)
    ws6 = torch.empty(mq.gemm_workspace_bytes(M, K, N, 128), dtype=torch.uint8, device=dev)
    down = {}
    for r in (4, 2, 8):
        pl = mq.pack(c6, r)
        us = time_queued(torch, lambda i: mq.gemm(pl, r, a6, z6, 128, K, N, x6, out=y6,
                                                  workspace=ws6), 30)
        tf = 2 * M * N * K / us / 1e6
        down[f"r{r}"] = {"us": round(us, 1), "TFLOP/s": round(tf, 1),
                         "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    del c6, a6, z6, x6, y6, ws6
    return down


def row_tiny(torch, mq, inputs, dev):
    """The tiny linear (K = 512 -> N = 256, per-channel) at M = 1 and 4: the
    parity configuration, launch-bound; microseconds per call."""
    n, k = 256, 512
    w = torch.from_numpy(inputs.gaussian_weights("tiny_linear", n, k)).to(dev)
    codes, alpha, zero = mq.quantize(w, k)
    out = {}
    for r in RS:
        pl = mq.pack(codes, r)
        for m in (1, 4):
            x = torch.from_numpy(inputs.activations_bf16("tiny_linear", m, k).view("int16")).to(dev)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            us = time_loop(torch, lambda i: mq.gemv(pl, r, alpha, zero, k, n, k, x, out=y), 50)
            out[f"r{r}_M{m}"] = round(us, 2)
    return out


def row_decode_split(torch, mq, inputs, dev):
    """f1: the Gemma-2-9B MLP decode at the split precisions r = 6 and 3, each
    r alone (three products per launch), rotating over weight copies."""
    mats = []
    for i, name in enumerate(("up", "gate", "down")):
        n, k = inputs.GEMMA9B_MLP[name]
        w = inputs.device_gaussian_weights("gemma9b_mlp", n, k, dev, matrix=i, outlier_frac=1e-3)
        codes, alpha, zero = mq.quantize(w, k)
        del w
        xb = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=i)
        x = torch.from_numpy(xb.view("int16")).to(dev)
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        mats.append(dict(name=name, N=n, K=k, codes=codes, alpha=alpha, zero=zero, x=x, y=y))
    out = {}
    side = torch.cuda.Stream()
    for r in (6, 3):
        base = [mq.pack(m["codes"], r) for m in mats]
        b = sum(linear_bytes(m["N"], m["K"], r, m["K"], 1) for m in mats)
        ncopy = max(2, -(-ROTATE_BYTES // b))
        sets = [base] + [[p.clone() for p in base] for _ in range(ncopy - 1)]
        plans = [mq.GemvGroupedPlan(gemma_problems(mq, mats, ps), r, 1, side) for ps in sets]
        us = time_loop(torch, lambda i: plans[i % ncopy](), 50, stream=side)
        out[f"r{r}"] = {"us": round(us, 2), "bytes": b, "GB/s": round(b / us / 1e3, 1),
                        "frac_of_hbm_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
        del plans, sets, base
    del mats
    return out


def row_mid_m(torch, mq, inputs, dev):
    """a4 between small batch and prefill: the 4096-wide down projection
    (K = 14336), group 128, r = 4, at M = 128, 256, 512 and 1024 (the kernel
    splits K over workgroups where the output tiles are few)."""
    _, K, N = inputs.PREFILL_SHAPE
    w = inputs.device_gaussian_weights("prefill", K, N, dev, matrix=1)
    c, a, z = mq.quantize(w, 128)
    del w
    r = 4
    pl = mq.pack(c, r)
    out = {}
    for M in (128, 256, 512, 1024):
        xb = inputs.activations_bf16("prefill", M, N, matrix=1)
        x = torch.from_numpy(xb.view("int16")).to(dev)
        y = torch.empty((M, K), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, mq.gemm_workspace_bytes(M, K, N, 128)), dtype=torch.uint8,
                         device=dev)
        us = time_loop(torch, lambda i: mq.gemm(pl, r, a, z, 128, K, N, x, out=y, workspace=ws),
                       20)
        tf = 2 * M * N * K / us / 1e6
        out[f"M{M}_r{r}"] = {"us": round(us, 1), "TFLOP/s": round(tf, 1),
                             "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    del c, a, z, pl
    return out


# name -> (function, what it measures); run in this order
ROWS = {
    "gemv_tiny_linear": (row_tiny, "parity configuration: 512 -> 256, M = 1, 4"),
    "pack_gemma_down": (row_pack, "a1 slice-and-pack"),
    "gemm_mistral_small": (row_small, "a3 small-batch GEMM"),
    "gemm_prefill_M2048": (row_prefill, "a4 prefill GEMM"),
    "gemm_prefill_down_M2048": (row_prefill_down, "a4 prefill down projection"),
    "gemm_down_mid_M": (row_mid_m, "a4 down projection at M = 128 to 1024"),
    "gemv_gemma9b_mlp_r6_r3": (row_decode_split, "f1 decode at r = 6, 3"),
    "mixnmatch_mistral7b_32l": (lambda t, m, i, d: run_stack(t, m, i, d), "a5 Mix'n'Match stack"),
    "extra_precision_gemma_r2": (lambda t, m, i, d: run_extra(t, m, i, d), "f2 Extra-Precision"),
    "bitplanes_gemma9b_mlp": (lambda t, m, i, d: run_bitplanes(t, m, i, d), "f3 bit-planes"),
    "mlp_decode_gemma9b": (lambda t, m, i, d: run_mlp(t, m, i, d), "f4 decode MLP block"),
}


def run_rows(torch, mq, inputs, dev, only=None):
    rows = {}
    for name, (fn, what) in ROWS.items():
        if only is not None and name not in only:
            continue
        log(f"row {name}: {what}")
        rows[name] = fn(torch, mq, inputs, dev)
        torch.cuda.synchronize()
    return rows


def run_extra(torch, mq, inputs, dev, r=2):
    mats = []
    nnz_total, codes_total = 0, 0
    for i, name in enumerate(("up", "gate", "down")):
        n, k = inputs.GEMMA9B_MLP[name]
        w = inputs.device_gaussian_weights("gemma9b_mlp", n, k, dev, matrix=i, outlier_frac=1e-3)
        codes, alpha, zero = mq.quantize(w, k)
        del w
        row_ptr, col_idx = mq.overflow_lists(codes, r)
        xb = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=i)
        x = torch.from_numpy(xb.view("int16")).to(dev)
        y = torch.zeros((1, n), dtype=torch.float32, device=dev)
        mats.append((row_ptr, col_idx, alpha, n, k, x, y))
        nnz_total += col_idx.numel()
        codes_total += n * k
        del codes
    torch.cuda.synchronize()

    # the three matrices' sparse additions in one launch
    probs = [dict(row_ptr=row_ptr, col_idx=col_idx, alpha=alpha, x=x, y=y, N=n, K=k, group=k)
             for row_ptr, col_idx, alpha, n, k, x, y in mats]

    def apply_all(i):
        mq.overflow_apply_grouped(probs, r, 1)

    us = time_loop(torch, apply_all, 50)
    # 16-bit column indices and a 32-bit row pointer per row
    list_bits = 16.0 * nnz_total + 32.0 * sum(m[3] + 1 for m in mats)
    return {"r": r, "apply_us_3_matrices": round(us, 2), "overflow_codes": nnz_total,
            "overflow_fraction": round(nnz_total / codes_total, 6),
            "effective_bits": round(r + list_bits / codes_total, 4)}


def run_bitplanes(torch, mq, inputs, dev):
    """NEXT-3: one bit-plane copy of the Gemma MLP codes served at several r
    (and unclamped at r = 2); planes read = (r + 1)/8 of the codes (8/8 at
    r = 8).  One launch per matrix, three per MLP."""
    mats = []
    for i, name in enumerate(("up", "gate", "down")):
        n, k = inputs.GEMMA9B_MLP[name]
        w = inputs.device_gaussian_weights("gemma9b_mlp", n, k, dev, matrix=i, outlier_frac=1e-3)
        codes, alpha, zero = mq.quantize(w, k)
        del w
        xb = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=i)
        x = torch.from_numpy(xb.view("int16")).to(dev)
        y = torch.empty((1, n), dtype=torch.float32, device=dev)
        mats.append(dict(codes=codes, alpha=alpha, zero=zero, N=n, K=k, x=x, y=y))
    out = {}
    down = mats[2]
    pl_out = torch.empty((8, down["N"], down["K"] // 8), dtype=torch.uint8, device=dev)
    us = time_loop(torch, lambda i: mq.pack_bitplanes(down["codes"], out=pl_out), 20)
    out["pack_down_us"] = round(us, 2)
    out["pack_down_GB/s"] = round(2 * down["N"] * down["K"] / us / 1e3, 1)
    del pl_out
    one = sum(m["N"] * m["K"] for m in mats)
    ncopy = max(2, -(-ROTATE_BYTES // one))
    planes = [[mq.pack_bitplanes(m["codes"]) for m in mats] for _ in range(ncopy)]
    for m in mats:
        del m["codes"]
    torch.cuda.synchronize()
    for r, extra in ((2, False), (2, True), (3, False), (4, False), (6, False), (8, False)):
        def run(i):
            for j, m in enumerate(mats):
                mq.gemv_bitplanes(planes[i % ncopy][j], r, m["alpha"], m["zero"], m["K"], m["N"],
                                  m["K"], m["x"], extra=extra, out=m["y"])
        us = time_loop(torch, run, 50)
        b = sum(min(r + 1, 8) * m["N"] * m["K"] // 8 + 8 * m["N"] + 2 * m["K"] + 4 * m["N"]
                for m in mats)
        out[f"r{r}" + ("_extra" if extra else "")] = {
            "us_3_launches": round(us, 2), "bytes": b, "GB/s": round(b / us / 1e3, 1),
            "frac_of_hbm_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
    return out


def run_mlp(torch, mq, inputs, dev):
    """NEXT-4: the Gemma-2-9B decode MLP block (up and gate paired in one
    launch writing bf16(u * gelu(g)), then down), batch 1, at r = 8, 4, 2."""
    mats = {}
    for i, name in enumerate(("up", "gate", "down")):
        n, k = inputs.GEMMA9B_MLP[name]
        w = inputs.device_gaussian_weights("gemma9b_mlp", n, k, dev, matrix=i, outlier_frac=1e-3)
        codes, alpha, zero = mq.quantize(w, k)
        del w
        mats[name] = dict(codes=codes, alpha=alpha, zero=zero, N=n, K=k, group=k)
    F, H = mats["up"]["N"], mats["up"]["K"]
    xb = inputs.activations_bf16("gemma9b_mlp", 1, H, matrix=0)
    x = torch.from_numpy(xb.view("int16")).to(dev)
    y = torch.empty((1, H), dtype=torch.float32, device=dev)
    ws = torch.empty(mq.mlp_workspace_bytes(1, F), dtype=torch.uint8, device=dev)
    out = {}
    for r in RS:
        one = sum(m["N"] * m["K"] * r // 8 for m in mats.values())
        ncopy = max(2, -(-ROTATE_BYTES // one))
        copies = [{nm: dict(m, packed=mq.pack(m["codes"], r)) for nm, m in mats.items()}
                  for _ in range(ncopy)]

        def run(i):
            c = copies[i % ncopy]
            mq.mlp_decode(c["up"], c["gate"], c["down"], r, x, act="gelu_tanh", workspace=ws,
                          out=y)

        us = time_loop(torch, run, 50)
        b = sum(linear_bytes(m["N"], m["K"], r, m["K"], 1) for m in mats.values())
        out[f"r{r}"] = {"us": round(us, 2), "bytes": b, "GB/s": round(b / us / 1e3, 1),
                        "frac_of_hbm_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
        del copies
    return out


def run_stack(torch, mq, inputs, dev, n_layers=32):
    rs = inputs.mixnmatch_pattern(n_layers)
    layers = []
    codes_bytes = 0
    meta_bytes = 0
    for li, r in enumerate(rs):
        L = {"r": r}
        for mi, name in enumerate(mq.LAYER_LINEARS):
            n, k = inputs.MISTRAL_LAYER[name]
            w = inputs.device_gaussian_weights("mistral_stack", n, k, dev, layer=li, matrix=mi)
            codes, a, z = mq.quantize(w, k)
            del w
            L[name] = {"packed": mq.pack(codes, r), "alpha": a, "zero": z, "N": n, "K": k,
                       "group": k}
            del codes
            codes_bytes += n * k * r // 8
            meta_bytes += 8 * n
        layers.append(L)
    arr = mq.make_layers(layers)
    H = inputs.MISTRAL_LAYER["q"][0]
    ws = torch.empty(mq.mixnmatch_workspace_bytes(arr, 1), dtype=torch.uint8, device=dev)
    xb = inputs.activations_bf16("mistral_stack", 1, H)
    x = torch.from_numpy(xb.view("int16")).to(dev)
    h = torch.empty((1, H), dtype=torch.float32, device=dev)

    def fwd(i):
        mq.mixnmatch_forward(arr, x, ws, out=h)

    us = time_loop(torch, fwd, 10, warmup=2)
    b = codes_bytes + meta_bytes
    out = {"us_per_token": round(us, 1), "GB/s": round(b / us / 1e3, 1),
           "codes_GB": round(codes_bytes / 1e9, 3), "layers": n_layers,
           "r_pattern": "".join(str(r) for r in rs), "avg_bits": sum(rs) / len(rs)}
    del layers, arr, ws
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------- measured peaks

class Peaks:
    """The probes of libmq_peaks.so (include/mq_peaks.h): the achievable HBM
    read rate for a given byte count (rotating over >= 1 GiB of buffers, the
    best of a few grid sizes), the dense bf16 matrix-core rate, and the
    per-launch cadence of an empty kernel, timed with HIP events on the
    launch stream."""

    def __init__(self, torch, dev):
        import ctypes

        from nested_int_matmul_amd import build as _b

        self.torch, self.dev = torch, dev
        L = ctypes.CDLL(_b.PEAKS_LIB)
        vp = ctypes.c_void_p
        L.mqp_stream_read.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, vp, vp]
        L.mqp_mfma_loop.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
        L.mqp_mfma_loop_flops.restype = ctypes.c_double
        L.mqp_mfma_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        L.mqp_empty.argtypes = [vp]
        self.L, self.vp = L, vp
        self.stream = torch.cuda.current_stream()
        self.sp = vp(self.stream.cuda_stream)

    def _time(self, fn, n):
        torch = self.torch
        for i in range(3):
            fn(i)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for i in range(n):
            fn(i)
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n  # us per launch

    def hbm_read(self, nbytes):
        """Best GB/s reading nbytes per launch, rotating buffers."""
        torch = self.torch
        nbytes = (nbytes + 4095) // 4096 * 4096
        ncopy = max(2, -(-ROTATE_BYTES // nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=self.dev) for _ in range(ncopy)]
        sink = torch.empty(16384, dtype=torch.int32, device=self.dev)
        best = 0.0
        for blocks in (1024, 2048, 4096, 8192, 16384):
            def fn(i):
                assert self.L.mqp_stream_read(self.vp(bufs[i % ncopy].data_ptr()), nbytes, blocks,
                                              self.vp(sink.data_ptr()), self.sp) == 0
            us = self._time(fn, 30)
            best = max(best, nbytes / us / 1e3)
        del bufs
        return best

    def mfma_tflops(self):
        torch = self.torch
        blocks, iters = 1024, 2000
        out = torch.empty(blocks * 256, dtype=torch.float32, device=self.dev)

        def fn(i):
            assert self.L.mqp_mfma_loop(self.vp(out.data_ptr()), blocks, iters, self.sp) == 0

        us = self._time(fn, 10)
        return self.L.mqp_mfma_loop_flops(blocks, iters) / us / 1e6

    def empty_launch_us(self):
        return self._time(lambda i: self.L.mqp_empty(self.sp), 200)


def measured_peaks(torch, dev, sizes):
    P = Peaks(torch, dev)
    out = {"hbm_read_GBs": {str(k): round(P.hbm_read(b), 1) for k, b in sizes.items()},
           "bf16_mfma_TFLOPs": round(P.mfma_tflops(), 1),
           "empty_launch_us": round(P.empty_launch_us(), 3)}
    return out


# --------------------------------------------------------------------------- CPU baseline

def cpu_baseline(inputs):
    """The float64 oracle on the host: slice -> dequantize -> product for the
    three Gemma MLP matrices at r = 8, 4, 2 (the same work as one GPU step)
    on seeded numpy inputs of the same law."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    data = []
    for i, name in enumerate(("up", "gate", "down")):
        n, k = inputs.GEMMA9B_MLP[name]
        w = inputs.gaussian_weights("gemma9b_mlp", n, k, matrix=i, outlier_frac=1e-3)
        q, a, z = oracle.quantize_minmax(w, k)
        del w
        xb = inputs.activations_bf16("gemma9b_mlp", 1, k, matrix=i)
        data.append((q, a, z, k, xb, n))
    # whole steps, repeated until about 10 s of CPU work
    t0 = time.perf_counter()
    nbytes = 0
    reps = 0
    while reps < 8 and (reps == 0 or time.perf_counter() - t0 < 10.0):
        for r in RS:
            for q, a, z, k, xb, n in data:
                y = oracle.linear(xb, q, a, z, k, r)
                assert np.all(np.isfinite(y))
                nbytes += linear_bytes(n, k, r, k, 1)
        reps += 1
    dt = time.perf_counter() - t0
    # the same oracle on one thread: the tiny linear (K = 512 -> N = 256) at
    # every r and M = 1, 4, and the Gemma down matrix at r = 4 once
    one_thread = None
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            tq, ta, tz = oracle.quantize_minmax(inputs.gaussian_weights("tiny_linear", 256, 512), 512)
            tiny = {}
            for r in RS:
                for m in (1, 4):
                    tx = inputs.activations_bf16("tiny_linear", m, 512)
                    n_calls, t1 = 0, time.perf_counter()
                    while n_calls == 0 or time.perf_counter() - t1 < 0.3:
                        oracle.linear(tx, tq, ta, tz, 512, r)
                        n_calls += 1
                    tiny[f"r{r}_M{m}"] = round((time.perf_counter() - t1) / n_calls * 1e6, 1)
            q, a, z, k, xb, n = data[2]
            t1 = time.perf_counter()
            oracle.linear(xb, q, a, z, k, 4)
            dd = time.perf_counter() - t1
            one_thread = {"cores": 1, "tiny_linear_us_per_call": tiny,
                          "gemma_down_r4_s": round(dd, 3),
                          "gemma_down_r4_GBs": round(linear_bytes(n, k, 4, k, 1) / dd / 1e9, 4)}
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"{reps} full steps: the 3 Gemma-2-9B MLP matrices at r=8,4,2, batch 1, "
                       f"float64 numpy oracle, {dt:.1f} s"),
            "one_thread": one_thread}


# --------------------------------------------------------------------------- entry

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-rows", action="store_true", help="skip the extra per-row timings")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--rows", default=None,
                    help="comma-separated subset of the extra rows (default: all): " +
                         ", ".join(ROWS))
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for rocprofv3)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: this build runs on one GPU only (asked for {max(args.gpus, world)}); "
              "the multi-GPU sharding is a design note, not a measured path.", flush=True)
        sys.exit(2)

    import torch

    import nested_int_matmul_amd as mq
    from nested_int_matmul_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", flush=True)
        sys.exit(2)
    mq.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log("main step: Gemma-2-9B MLP decode, r = 8/4/2")
    res = run_main(torch, mq, inputs, dev, args.steps, args.warmup)
    ms_per_step = res["total_ms"] / args.steps
    value = res["step_bytes"] * args.steps / (res["total_ms"] * 1e-3) / 1e9

    # the step is one launch of the skinny kernel: its average duration over
    # the timed region (HIP events on the launch stream) is the kernel time
    launch_us = res["total_ms"] * 1e3 / args.steps
    achieved = res["step_bytes"] / (launch_us * 1e-6) / 1e9
    traffic = traffic_for(sha256(GEMV_SOURCE), "mixed")
    # measured ceilings: HBM read rate over the same byte counts (the step,
    # and one MLP at each r), the bf16 matrix-core rate, the launch cadence
    mlp_bytes = {r: sum(linear_bytes(m["N"], m["K"], r, m["K"], 1) for m in res["mats"])
                 for r in RS}
    log("measured peaks: HBM read, bf16 MFMA, empty launch")
    peaks = measured_peaks(torch, dev, {"step": res["step_bytes"],
                                        **{f"mlp_r{r}": b for r, b in mlp_bytes.items()}})
    read_step = peaks["hbm_read_GBs"]["step"]
    per_r = {}
    for r, us in res["per_r_us"].items():
        a = mlp_bytes[r] / us / 1e3
        per_r[f"r{r}"] = {"launch_us": round(us, 3), "bytes": mlp_bytes[r],
                          "achieved": round(a, 1), "frac": round(a / HBM_PEAK_GBS, 4),
                          "frac_of_measured_read":
                              round(a / peaks["hbm_read_GBs"][f"mlp_r{r}"], 4)}
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "mq::skinny_kernel<false, false> (9 products, r = 8/4/2, one launch)",
                "launch_us": round(launch_us, 3), "bytes_per_launch": res["step_bytes"],
                "measured_read_peak": read_step,
                "frac_of_measured_read": round(achieved / read_step, 4),
                "per_r_single_mlp_launch": per_r,
                "per_matrix_launch_us": res["per_matrix_us"],
                "step_spread_us": res["spread"],
                "measured_peaks": peaks}
    del res

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    rows = None
    if not args.no_rows:
        only = None if args.rows is None else set(args.rows.split(","))
        if only is not None and not only <= set(ROWS):
            print(f"bench.py: unknown rows {sorted(only - set(ROWS))}", flush=True)
            sys.exit(2)
        rows = run_rows(torch, mq, inputs, dev, only)
    cpu = None
    if not args.no_cpu:
        log("CPU baseline: float64 oracle")
        cpu = cpu_baseline(inputs)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gemma2_9b_mlp_decode", "M": 1,
                   "matrices": "up/gate 3584->14336, down 14336->3584",
                   "r": list(RS), "scales": "per-channel fp32 alpha,z",
                   "weights": "N(0,0.02), 0.1% x10 outliers", "rotation_bytes": ROTATE_BYTES},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
