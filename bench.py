#!/usr/bin/env python3
"""Throughput of the CQ matrix product on one MI355X.

Headline workload: HBM-resident streaming matvec, CQ2 W 65536 x 16384
(285,212,672 bytes of packed indices + fp16 norms), batch 1, fp32
activations N(0,1).  One step = cq_rotate_matvec(W, x) (the rotation and the product),
with the step's W taken in turn from three copies of the matrix so that no copy is
re-read while still resident in the 256 MB Infinity Cache.

  value       = packed bytes per step / wall time per step        (GB/s)
  roofline    = one cq_rotate_matvec call (the table-lookup kernel and the
                small kernel that adds the K-slice partial sums): packed bytes /
                mean call time (HIP events on the launch stream) against the
                8 TB/s HBM peak; traffic = HBM bytes per call from the committed
                rocprofv3 FETCH_SIZE/WRITE_SIZE summary
  cpu_baseline= the float64 oracle (dense dequantisation + product) on row
                slices of the same matrix, timed on this host

The same JSON line carries secondary figures under "secondary": the other
widths and batch 8 at the same shape, the CQ-W2A8 integer product (int8
activations and code book) at the same shape, the 4096 x 16384 x 16384 GEMM on the
matrix cores (TFLOP/s), the 16384 x 16384 encoder (GB/s of fp32 input) and
the Needle-shaped decode sweep (27 layers of 512-wide CQ2 matrices plus the
8192 x 512 CQ4 logits, per token, eager and replayed from a HIP graph), and
the tied-embedding row gather (2048 ids from the 8192 x 512 CQ4 matrix).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only matvec|w2a8|decode|gemm|encode|all]
       python bench.py --calibrate-copy      (counter calibration run)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROWS, COLS = 65536, 16384
GEMM_M, GEMM_N, GEMM_K = 4096, 16384, 16384
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "matvec_cq2_65536x16384_traffic.md")
MATVEC_SRC = os.path.join(ROOT, "hadamard_rotated_codebook_amd", "csrc", "matvec.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _events(torch, n):
    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def bench_matvec(torch, cq, cq_inputs, master, bits, batch, steps, warmup, gen, fused=True, w2a8=False,
                 read_ceiling=False):
    """One step = the rotation and the product of one batch: cq_rotate_matvec
    (fused=True), cq_rotate_acts + cq_matvec, or the int8 product
    cq_matvec_w2a8 (w2a8=True).  Three copies of the matrix take turns, so no
    step finds its matrix in the 256 MB Infinity Cache."""
    rows, cols = master.shape
    levels = cq_inputs.codebook(bits)
    W0 = cq.cq_quantize(master, bits, levels)
    mats = [W0] + [cq.CQMatrix(bits, rows, cols, W0.blob.clone(), levels) for _ in range(2)]
    x = torch.randn((batch, cols), generator=gen, device=master.device)
    xr = torch.empty((batch, cols), device=master.device)
    y = torch.empty((batch, rows), device=master.device)
    ws = torch.empty(max(cq.cq_workspace_bytes(cq.OP_ROTATE_MATVEC, mats[0], batch), 16), dtype=torch.uint8,
                     device=master.device)

    def step(i, ev=None):
        if w2a8:
            if ev is not None:
                ev[0].record()
            cq.cq_matvec_w2a8(mats[i % 3], x, out=y)
        elif fused:
            if ev is not None:
                ev[0].record()
            cq.cq_rotate_matvec(mats[i % 3], x, out=y, workspace=ws)
        else:
            cq.cq_rotate_acts(x, out=xr)
            if ev is not None:
                ev[0].record()
            cq.cq_matvec(mats[i % 3], xr, out=y, workspace=ws)
        if ev is not None:
            ev[1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # the step rate, with nothing else in the stream (event records between
    # the calls would add their own gaps) ...
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    # ... and, in a second pass, the product call alone between events
    ev = _events(torch, steps)
    for i in range(steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) / 1e3 for a, b in ev)
    nbytes = W0.blob.numel()
    res = {"bits": bits, "batch": batch, "bytes": nbytes, "step_s": wall, "kernel_s": sum(times) / steps,
           "kernel_median_s": times[steps // 2], "flop": 2.0 * rows * cols * batch,
           "call": "cq_matvec_w2a8" if w2a8 else ("cq_rotate_matvec" if fused else "cq_rotate_acts + cq_matvec")}
    if read_ceiling:
        res["read_ceiling"] = bench_read_ceiling(torch, cq, [W.blob for W in mats], steps, warmup)
    del mats, W0
    return res


def bench_read_ceiling(torch, cq, bufs, steps, warmup):
    """The streaming-read ceiling on the same bytes: cq_read_probe (16-byte
    loads with the nt streaming hint, 32 KB contiguous tiles per workgroup) over the same three
    copies of the matrix in turn, timed between HIP events."""
    sink = torch.empty(2048 * 256, dtype=torch.int32, device=bufs[0].device)
    for i in range(warmup):
        cq.cq_read_probe(bufs[i % 3], sink)
    torch.cuda.synchronize()
    ev = _events(torch, steps)
    for i in range(steps):
        ev[i][0].record()
        cq.cq_read_probe(bufs[i % 3], sink)
        ev[i][1].record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) / 1e3 for a, b in ev)
    nbytes = bufs[0].numel()
    return {"bytes": nbytes, "median_s": t[steps // 2], "gbs": nbytes / t[steps // 2] / 1e9,
            "frac_hbm_peak": nbytes / t[steps // 2] / 1e9 / HBM_PEAK_GBS,
            "probe": "cq_read_probe: 2048 workgroups x 256 threads, 16-byte nt loads, 8 in flight per thread"}


def bench_needle_decode(torch, cq, cq_inputs, steps, gen):
    """One decode token of a Needle-shaped model at batch 1: per layer one
    activation feeds Q 512x512, K and V 256x512 and gate 512x512, another
    feeds out 512x512 (all CQ2), then the 8192x512 CQ4 tied logits.  Two
    ways: one cq_rotate_matvec call per product (136 calls a token), and the
    shared-activation call for Q/K/V/gate (cq_rotate_multi_matvec) plus one
    call for out (55 calls a token).  Each eager and replayed from a HIP
    graph.  Weights are seeded N(0, 0.02^2) masters encoded on the GPU."""
    dev = torch.device("cuda:0")
    shapes = [512, 256, 256, 512, 512]
    mats, xs, ys = [], [], []
    for layer in range(27):
        for rows in shapes:
            w = torch.randn((rows, 512), generator=gen, device=dev).mul_(0.02)
            mats.append(cq.cq_quantize(w, 2, cq_inputs.codebook(2)))
            ys.append(torch.empty((1, rows), device=dev))
        xs += [torch.randn((1, 512), generator=gen, device=dev) for _ in range(2)]
    w = torch.randn((8192, 512), generator=gen, device=dev).mul_(0.02)
    logits = cq.cq_quantize(w, 4, cq_inputs.codebook(4))
    xl, yl = torch.randn((1, 512), generator=gen, device=dev), torch.empty((1, 8192), device=dev)
    need = max(cq.cq_workspace_bytes(cq.OP_ROTATE_MATVEC, m, 1) for m in mats + [logits])
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def per_call():
        for layer in range(27):
            for t in range(5):
                x = xs[2 * layer + (1 if t == 4 else 0)]
                cq.cq_rotate_matvec(mats[5 * layer + t], x, out=ys[5 * layer + t], workspace=ws)
        cq.cq_rotate_matvec(logits, xl, out=yl, workspace=ws)

    def shared():
        for layer in range(27):
            cq.cq_rotate_multi_matvec(mats[5 * layer:5 * layer + 4], xs[2 * layer], outs=ys[5 * layer:5 * layer + 4],
                                      workspace=ws)
            cq.cq_rotate_matvec(mats[5 * layer + 4], xs[2 * layer + 1], out=ys[5 * layer + 4], workspace=ws)
        cq.cq_rotate_matvec(logits, xl, out=yl, workspace=ws)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        eager = (time.perf_counter() - t0) / steps
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        graph = (time.perf_counter() - t0) / steps
        del g
        return eager, graph

    nbytes = sum(m.blob.numel() for m in mats) + logits.blob.numel()
    out = {"bytes_per_token": nbytes}
    for name, fn, calls in (("per_call", per_call, 136), ("shared_activation", shared, 55)):
        eager, graph = timed(fn)
        out[name] = {"calls_per_token": calls, "eager_us_per_token": eager * 1e6, "graph_us_per_token": graph * 1e6,
                     "graph_gbs": nbytes / graph / 1e9}
    return out


def bench_gather(torch, cq, cq_inputs, gen, steps=50):
    """The tied-embedding lookup of a Needle-shaped decode: 2048 token ids
    gathered from the 8192 x 512 CQ4 matrix as fp32 rows (cq_gather_rows)."""
    dev = torch.device("cuda:0")
    w = torch.randn((8192, 512), generator=gen, device=dev).mul_(0.02)
    W = cq.cq_quantize(w, 4, cq_inputs.codebook(4))
    ids = torch.randint(0, 8192, (2048,), generator=gen, device=dev)
    out = torch.empty((2048, 512), device=dev)
    for _ in range(5):
        cq.cq_gather_rows(W, ids, out=out)
    torch.cuda.synchronize()
    ev = _events(torch, steps)
    for i in range(steps):
        ev[i][0].record()
        cq.cq_gather_rows(W, ids, out=out)
        ev[i][1].record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) / 1e3 for a, b in ev)[steps // 2]
    row_bytes = W.blob.numel() // 8192
    moved = 2048 * (row_bytes + 512 * 4)  # packed row + norms read, fp32 row written
    return {"rows": 2048, "cols": 512, "bits": 4, "kernel_median_s": t, "rows_per_s": 2048 / t,
            "gbs": moved / t / 1e9}


def bench_small_and_prefill(torch, cq, cq_inputs, gen, steps=100):
    """The single 512 x 512 CQ2 matvec (batch 1, one cq_rotate_matvec call,
    eager and replayed from a HIP graph) and the Needle-shaped prefill: 2048
    tokens x 512 of fp16 activations rotated to bf16 once (cq_rotate_acts),
    then cq_gemm through the 512 x 512 and 256 x 512 CQ2 projections and the
    8192 x 512 CQ4 logits, each timed per call from HIP graph replays."""
    dev = torch.device("cuda:0")
    out = {}
    w = torch.randn((512, 512), generator=gen, device=dev).mul_(0.02)
    W = cq.cq_quantize(w, 2, cq_inputs.codebook(2))
    x = torch.randn((1, 512), generator=gen, device=dev)
    y = torch.empty((1, 512), device=dev)

    def eager_median(fn, n):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        ev = _events(torch, n)
        for i in range(n):
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) / 1e3 for a, b in ev)[n // 2]

    def graph_per_call(fn, calls=20, replays=10):
        # launch gaps of the host removed: the calls replayed from a HIP graph
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                fn()
        g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(replays):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        del g
        return t0.elapsed_time(t1) / 1e3 / (calls * replays)

    t_eager = eager_median(lambda: cq.cq_rotate_matvec(W, x, out=y), steps)
    t_graph = graph_per_call(lambda: cq.cq_rotate_matvec(W, x, out=y))
    nb = W.blob.numel()
    out["matvec_cq2_512x512_b1"] = {"bytes": nb, "eager_median_s": t_eager, "graph_s_per_call": t_graph,
                                    "graph_gbs": nb / t_graph / 1e9}
    # prefill
    X = torch.randn((2048, 512), generator=gen, device=dev).half()
    mats = {"q_512x512_cq2": (2, 512), "kv_256x512_cq2": (2, 256), "logits_8192x512_cq4": (4, 8192)}
    Ws = {k: cq.cq_quantize(torch.randn((r, 512), generator=gen, device=dev).mul_(0.02), b, cq_inputs.codebook(b))
          for k, (b, r) in mats.items()}
    xr = torch.empty((2048, 512), dtype=torch.bfloat16, device=dev)
    t_rot = graph_per_call(lambda: cq.cq_rotate_acts(X, torch.bfloat16, out=xr))
    pre = {"rotate_2048x512_s": t_rot}
    for k, Wk in Ws.items():
        C = torch.empty((2048, Wk.rows), device=dev)
        t = graph_per_call(lambda: cq.cq_gemm(Wk, xr, out=C))
        pre[k] = {"s": t, "tflops": 2.0 * 2048 * Wk.rows * 512 / t / 1e12}
    out["needle_prefill_2048_tokens"] = pre
    return out


def bench_kv_attention(torch, cq, cq_inputs, gen, steps=50):
    """One layer's decode attention over a CQ-quantised KV cache, Needle 2
    shape: a 256-token window of keys and values (4 KV heads of 64, the ring
    full) at kv_bits 2, 3 and 4; a step appends the new token's key and value
    (cq_quantize_rows), scores 8 query heads (cq_kv_scores), softmax (torch),
    and the weighted values (cq_matvec_t); the fused step is one cq_kv_append
    (both appends in one launch) and one cq_kv_attention.  Per step from HIP
    graph replays."""
    dev = torch.device("cuda:0")
    out = {}
    for bits in (2, 3, 4):
        lv = cq_inputs.codebook(bits)
        K = cq.cq_quantize(torch.randn((256, 256), generator=gen, device=dev), bits, lv)
        V = cq.cq_quantize(torch.randn((256, 256), generator=gen, device=dev), bits, lv)
        kn = torch.randn((steps, 256), generator=gen, device=dev)
        vn = torch.randn((steps, 256), generator=gen, device=dev)
        q = torch.randn((8, 64), generator=gen, device=dev)
        s = torch.empty((8, 256), device=dev)
        o = torch.empty((8, 256), device=dev)
        ws = torch.empty(cq.cq_kv_scores_workspace_bytes(K, 8, 4, 64) + 256, dtype=torch.uint8, device=dev)
        wt = cq.workspace_for(cq.cq_workspace_bytes(cq.OP_MATVEC_T, V, 8), dev)

        of = torch.empty((8, 64), device=dev)

        def step(i):
            cq.cq_quantize_rows(K, kn[i:i + 1], i % 256)
            cq.cq_quantize_rows(V, vn[i:i + 1], i % 256)
            cq.cq_kv_scores(K, q, 4, out=s, workspace=ws)
            p = torch.softmax(s * 0.125, dim=1)
            cq.cq_matvec_t(V, p, out=o, workspace=wt)

        def fused(i):
            cq.cq_kv_append(K, V, kn[i:i + 1], vn[i:i + 1], i % 256)
            cq.cq_kv_attention(K, V, q, 4, scale=0.125, out=of)

        res = {"cache_bytes": 2 * K.blob.numel()}
        for name, fn in (("graph_us_per_step", step), ("fused_graph_us_per_step", fused)):
            for i in range(5):
                fn(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    fn(i)
            g.replay()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(5):
                g.replay()
            t1.record()
            torch.cuda.synchronize()
            res[name] = t0.elapsed_time(t1) * 1e3 / (5 * steps)
            del g
        out[f"kv{bits}"] = res
    return out


def bench_gemm(torch, cq, cq_inputs, master, bits, m, steps, warmup, gen):
    rows, cols = master.shape
    levels = cq_inputs.codebook(bits)
    W = cq.cq_quantize(master, bits, levels)
    X = torch.randn((m, cols), generator=gen, device=master.device).to(torch.bfloat16)
    xr = cq.cq_rotate_acts(X, torch.bfloat16)
    C = torch.empty((m, rows), device=master.device)
    for _ in range(warmup):
        cq.cq_gemm(W, xr, out=C)
    torch.cuda.synchronize()
    ev = _events(torch, steps)
    for i in range(steps):
        ev[i][0].record()
        cq.cq_gemm(W, xr, out=C)
        ev[i][1].record()
    torch.cuda.synchronize()
    kern = sum(a.elapsed_time(b) for a, b in ev) / steps / 1e3
    flop = 2.0 * m * rows * cols
    return {"bits": bits, "m": m, "n": rows, "k": cols, "kernel_s": kern, "tflops": flop / kern / 1e12,
            "frac_bf16_peak": flop / kern / 1e12 / BF16_PEAK_TFLOPS}


def bench_encode(torch, cq, cq_inputs, master, bits, steps, warmup):
    levels = cq_inputs.codebook(bits)
    out = torch.empty(cq.cq_blob_bytes(bits, *master.shape), dtype=torch.uint8, device=master.device)
    for _ in range(warmup):
        cq.cq_quantize(master, bits, levels, out=out)
    torch.cuda.synchronize()
    ev = _events(torch, steps)
    for i in range(steps):
        ev[i][0].record()
        cq.cq_quantize(master, bits, levels, out=out)
        ev[i][1].record()
    torch.cuda.synchronize()
    kern = sum(a.elapsed_time(b) for a, b in ev) / steps / 1e3
    nbytes = master.numel() * 4
    return {"bits": bits, "rows": master.shape[0], "cols": master.shape[1], "kernel_s": kern,
            "input_gbs": nbytes / kern / 1e9, "frac_hbm_peak": nbytes / kern / 1e9 / HBM_PEAK_GBS}


def cpu_baseline(seconds=12.0, rows_per_slice=256):
    """The oracle as it stands, on row slices of the headline matrix."""
    import numpy as np
    import cq_inputs
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    levels = cq_inputs.codebook(2)
    x = cq_inputs.activations(4, 0, 1, COLS)
    done_bytes, spent, s = 0, 0.0, 0
    while spent < seconds:
        r0 = (s * rows_per_slice) % ROWS
        w = cq_inputs.master(4, 0, ROWS, COLS, r0, r0 + rows_per_slice)
        blob = oracle.quantize(w, 2, levels)  # input preparation, not timed
        t0 = time.perf_counter()
        oracle.matvec(blob, 2, rows_per_slice, COLS, x, levels)
        spent += time.perf_counter() - t0
        done_bytes += blob.size
        s += 1
    return {"value": done_bytes / spent / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{s} slices of {rows_per_slice} rows x {COLS} cols of the CQ2 matrix "
                      f"(float64 dense dequantisation + product), {spent:.1f} s of CPU work"}


def stored_traffic():
    """HBM bytes per cq_matvec call from the committed rocprofv3 counter summary
    ("key: value" lines), if it was taken on the current kernel source; else None."""
    try:
        fields = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith(("#", "|", " ")):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        src = hashlib.sha256(open(MATVEC_SRC, "rb").read()).hexdigest()
        if fields.get("matvec_source_sha256") != src:
            return None
        return int(fields["traffic_bytes_per_call"])
    except (OSError, ValueError, KeyError):
        return None


def calibrate_copy(torch, repeats=5, nbytes=1 << 30):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE
    and WRITE_SIZE counters: each launch reads and writes exactly nbytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(repeats):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
                      "launches": repeats}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--only", choices=["all", "matvec", "batch8", "w2a8", "decode", "gemm", "encode"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; there is no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    import cq_inputs
    import hadamard_rotated_codebook_amd as cq

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261202)
    result = {}
    secondary = {}

    if args.only in ("all", "matvec", "batch8", "w2a8"):
        log("generating the 65536 x 16384 fp32 master on the GPU")
        master = torch.randn((ROWS, COLS), generator=gen, device=dev).mul_(0.02)
    if args.only in ("all", "matvec"):
        head = bench_matvec(torch, cq, cq_inputs, master, 2, 1, args.steps, args.warmup, gen, read_ceiling=True)
        log(f"CQ2 b1: step {head['step_s']*1e6:.1f} us, matvec kernel {head['kernel_s']*1e6:.1f} us; "
            f"read ceiling {head['read_ceiling']['gbs']:.0f} GB/s")
        result["head"] = head
        if args.only == "all":
            two = bench_matvec(torch, cq, cq_inputs, master, 2, 1, args.steps, args.warmup, gen, fused=False)
            two["gbs"] = two["bytes"] / two["step_s"] / 1e9
            secondary["matvec_cq2_b1_two_calls"] = two
            log(f"CQ2 b1 as rotate + matvec: step {two['step_s']*1e6:.1f} us, matvec {two['kernel_s']*1e6:.1f} us")
    if args.only in ("all", "batch8"):
        legs = ([(3, 1), (4, 1), (5, 1), (1, 1)] if args.only == "all" else []) + [(2, 8), (4, 8), (1, 8)]
        for bits, batch in legs:
            r = bench_matvec(torch, cq, cq_inputs, master, bits, batch, max(args.steps // 3, 20),
                             args.warmup, gen)
            key = f"matvec_cq{ {5: 't', 1: 'b'}.get(bits, bits) }_b{batch}"
            # rates from the median call: a stall of the launching thread
            # shows up in the events of the call it delays
            r["gbs"] = r["bytes"] / r["kernel_median_s"] / 1e9
            r["frac_hbm_peak"] = r["gbs"] / HBM_PEAK_GBS
            if batch > 1:
                r["tflops"] = r["flop"] / r["kernel_median_s"] / 1e12  # fp16 matrix cores, fp32 sums
            secondary[key] = r
            log(key, f"{r['kernel_median_s']*1e6:.1f} us (median)", f"{r['gbs']:.0f} GB/s")
    if args.only in ("all", "w2a8"):
        # the pages' deployment numerics: int8 activations and code book
        for bits, batch in [(2, 1), (4, 1), (1, 1), (2, 2)]:
            r = bench_matvec(torch, cq, cq_inputs, master, bits, batch, max(args.steps // 3, 20),
                             args.warmup, gen, w2a8=True)
            key = f"matvec_w2a8_cq{ {1: 'b'}.get(bits, bits) }_b{batch}"
            r["gbs"] = r["bytes"] / r["kernel_median_s"] / 1e9
            r["frac_hbm_peak"] = r["gbs"] / HBM_PEAK_GBS
            secondary[key] = r
            log(key, f"{r['kernel_median_s']*1e6:.1f} us (median)", f"{r['gbs']:.0f} GB/s")
    if args.only in ("all", "matvec", "batch8", "w2a8"):
        del master
        torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        r = bench_needle_decode(torch, cq, cq_inputs, 50, gen)
        secondary["needle_decode_token"] = r
        for k in ("per_call", "shared_activation"):
            log(f"needle decode token, {k}: {r[k]['eager_us_per_token']:.0f} us eager, "
                f"{r[k]['graph_us_per_token']:.0f} us graph")
        r = bench_gather(torch, cq, cq_inputs, gen)
        secondary["gather_cq4_8192x512_2048_rows"] = r
        log(f"gather 2048 rows of 8192x512 CQ4: {r['kernel_median_s']*1e6:.1f} us, {r['gbs']:.0f} GB/s")
        r = bench_kv_attention(torch, cq, cq_inputs, gen)
        secondary["kv_attention_step_needle2"] = r
        log("kv attention step: " + ", ".join(f"{k} {v['graph_us_per_step']:.1f} us" for k, v in r.items())
            + "; fused (cq_kv_append + cq_kv_attention): "
            + ", ".join(f"{k} {v['fused_graph_us_per_step']:.1f} us" for k, v in r.items()))
        r = bench_small_and_prefill(torch, cq, cq_inputs, gen)
        secondary.update(r)
        s5 = r["matvec_cq2_512x512_b1"]
        log(f"matvec 512x512 CQ2 b1: {s5['eager_median_s']*1e6:.1f} us eager, {s5['graph_s_per_call']*1e6:.2f} us "
            f"per call in a graph")
        p = r["needle_prefill_2048_tokens"]
        log("prefill 2048 tokens: rotate " + f"{p['rotate_2048x512_s']*1e6:.1f} us; " +
            ", ".join(f"{k} {v['s']*1e6:.1f} us ({v['tflops']:.0f} TFLOP/s)" for k, v in p.items() if k != "rotate_2048x512_s"))

    if args.only in ("all", "gemm", "encode"):
        log("generating the 16384 x 16384 fp32 master on the GPU")
        master = torch.randn((GEMM_N, GEMM_K), generator=gen, device=dev).mul_(0.02)
        if args.only in ("all", "encode"):
            for bits in (4, 3):
                r = bench_encode(torch, cq, cq_inputs, master, bits, 10, 2)
                secondary[f"encode_cq{bits}_16384x16384"] = r
                log(f"encode cq{bits}: {r['kernel_s']*1e3:.3f} ms, {r['input_gbs']:.0f} GB/s")
        if args.only in ("all", "gemm"):
            for bits in (4, 3):
                r = bench_gemm(torch, cq, cq_inputs, master, bits, GEMM_M, 20, 10, gen)
                secondary[f"gemm_cq{bits}_4096x16384x16384"] = r
                log(f"gemm cq{bits}: {r['kernel_s']*1e3:.3f} ms, {r['tflops']:.1f} TFLOP/s")
        del master
        torch.cuda.empty_cache()

    line = {"metric": "CQ2 batch-1 matvec GB/s of packed weights (% HBM peak); CQ GEMM TFLOP/s",
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f32 activations, f16 lookup-table entries, f32 accumulation",
            "data": "synthetic: seeded N(0,0.02^2) master encoded on the GPU; activations N(0,1)"}
    if "head" in result:
        h = result["head"]
        line["value"] = h["bytes"] / h["step_s"] / 1e9
        line["ms_per_step"] = h["step_s"] * 1e3
        line["config"] = {"workload": "HBM-resident CQ2 matvec, W 65536x16384, batch 1, fp32 activations",
                          "rows": ROWS, "cols": COLS, "bits": 2, "batch": 1, "packed_bytes": h["bytes"]}
        ach = h["bytes"] / h["kernel_s"] / 1e9
        line["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": ach / HBM_PEAK_GBS, "traffic": stored_traffic(),
                            "kernel": "cq_rotate_matvec call: matvec_kernel<2, true, 2> (nt code loads) + combine_kernel",
                            "kernel_us": h["kernel_s"] * 1e6, "algorithmic_bytes": h["bytes"],
                            "read_ceiling_gbs": h["read_ceiling"]["gbs"],
                            "frac_of_read_ceiling": ach / h["read_ceiling"]["gbs"]}
    else:
        line["value"] = None
        line["ms_per_step"] = None
        line["config"] = {"workload": f"partial run (--only {args.only})"}
    if secondary:
        line["secondary"] = secondary
    # the pages' own figures, for context only: they print no GPU or kernel
    # throughput for this path
    line["pages_context"] = {
        "needle2_archive": "13,737,807 bytes in 405 tensors (CQ2 at 2.125 bpw, CQ4 at 4.125 bpw, fp16, raw)",
        "decode_rate": "about 500 tokens/s for a whole Needle model on a Raspberry Pi 5 CPU, int8 activations "
                       "(a relayed product claim)"}
    if not args.no_cpu_baseline and args.only in ("all", "matvec"):
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
