"""Benchmark of the ternary x int8 GEMM hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input at
M=16384, N=3456, K=1280 (the "500m" throughput shape):
    forward  C  = A x W          int8 x ternary (2-bit packed) -> int32
    dX       dX = dC x W^T       same stored W
    dW       dW = A^T x dC       int8 x int8 -> int32, contraction over M
Inputs are resident in HBM before the timed region.  W steps run untimed, then
K steps are timed between HIP events on the stream the kernels run on, with a
device synchronisation on both sides; each kernel is also bracketed by its own
events to give its average launch duration.  One JSON line goes to stdout;
its "value" is the metric, the forward's TOPS at this shape (its average
launch time inside the step), and "step" gives the rate of the whole step.

Work is counted as 2*M*N*K ops per product (zero weights included: the method
computes densely).  Peaks are AMD's published MI355X figures.
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

METRIC = "ternary x int8 GEMM TOPS at 16384x3456x1280; % of int8 MFMA peak"
PEAK_INT8_OPS = 5.0e15      # dense int8 MFMA, ops/s
PEAK_HBM_BPS = 8.0e12       # HBM3E, bytes/s
RIDGE = PEAK_INT8_OPS / PEAK_HBM_BPS
PROFILES = os.path.join(ROOT, "profiles")


def kernel_work(name, M, N, K):
    """(ops, algorithmic HBM bytes) of one launch: each operand read once, output written once."""
    ops = 2 * M * N * K
    if name == "fwd":
        byts = M * K + N * (K // 4) + 4 * M * N
    elif name == "dx":
        byts = M * N + N * (K // 4) + 4 * M * K
    else:
        byts = M * K + M * N + 4 * K * N
    return ops, byts


PREP_KERNELS = ("pack", "quantize_rows", "quantize_cols")


def source_digest(kernel=None):
    """sha256 of the source file that holds a kernel (the GEMM kernels'
    file unless the kernel is one of the packer / quantizer's)."""
    name = "prep.hip" if kernel in PREP_KERNELS else "ternary_gemm.hip"
    src = os.path.join(ROOT, "ternary_weight_int8_amd", "csrc", name)
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic(kernel, workload_tag):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload_tag}_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != source_digest(kernel):
        return None
    try:
        return int(float(fields["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_threads():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit():
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(A, Wp, dC, K, rows):
    """The oracle as it stands, on the first `rows` rows of the same batch."""
    import oracle  # CPU baseline leg only

    threads = cpu_threads()
    a, g = np.ascontiguousarray(A[:rows]), np.ascontiguousarray(dC[:rows])
    N = Wp.shape[0]
    t0 = time.perf_counter()
    oracle.fwd(a, Wp, threads=threads)
    oracle.dx(g, Wp, K, threads=threads)
    oracle.dw(a, g, threads=threads)
    dt = time.perf_counter() - t0
    ops = 3 * 2 * rows * N * K
    return {
        "value": ops / dt / 1e12,
        "unit": "TOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": f"forward + dX + dW on the first {rows} of the 16384 rows "
                  f"({rows}x{N}x{K} each, same inputs), {dt:.1f} s",
    }


def scaled_outputs(B, synth, torch, stream, Ad, Wd, dCd, M, N, K, seed, steps):
    """Average launch time of each product with a scaled bf16 output (row and
    column scales fused into the stores), on the step's inputs; not part of
    the step's metric.  Bytes: inputs, scale vectors and the bf16 output."""
    dev = Ad.device
    rs_m = torch.from_numpy(synth.positive_scales(seed, synth.STREAM_ROW_SCALE, M)).to(dev)
    rs_k = torch.from_numpy(synth.positive_scales(seed, synth.STREAM_ROW_SCALE, K)).to(dev)
    cs_n = torch.from_numpy(synth.positive_scales(seed, synth.STREAM_COL_SCALE, N)).to(dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((K, N), dtype=torch.bfloat16, device=dev)
    runs = {
        "fwd_bf16": (lambda: B.ternary_gemm_s8_scaled(Ad, Wd, rs_m, synth.W_SCALE, torch.bfloat16,
                                                      Y=Y, stream=stream),
                     M * K + N * (K // 4) + 4 * M + 2 * M * N),
        "dx_bf16": (lambda: B.ternary_gemm_s8_dx_scaled(dCd, Wd, K, rs_m, synth.W_SCALE, torch.bfloat16,
                                                        dX=dX, stream=stream),
                    M * N + N * (K // 4) + 4 * M + 2 * M * K),
        "dw_bf16": (lambda: B.ternary_gemm_s8_dw_scaled(Ad, dCd, rs_k, cs_n, torch.bfloat16, dW=dW,
                                                        stream=stream),
                    M * K + M * N + 4 * (K + N) + 2 * K * N),
    }
    out = {}
    ops = 2 * M * N * K
    for name, (fn, byts) in runs.items():
        for _ in range(3):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(steps):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        t = ev[0].elapsed_time(ev[-1]) / steps / 1e3
        out[name] = {"avg_us": t * 1e6, "tops": ops / t / 1e12, "mfma_frac": ops / t / PEAK_INT8_OPS,
                     "gbps": byts / t / 1e9, "hbm_frac": byts / t / PEAK_HBM_BPS,
                     "algorithmic_bytes": byts, "ops": ops}
    return out


SKINNY = [(27, 16384, 16384), (1, 16384, 16384), (27, 3456, 1280)]


def skinny_rows(B, synth, torch, stream, seed, steps, op):
    """The forward ("fwd") or dX ("dx") with few rows (the skinny kernels, M
    <= 32; 27 is the pages' backward batch), bound by reading the packed
    weights.  Successive launches read different copies of the weights, more
    than 512 MB of them in all, so that each launch streams its weights from
    HBM (past the 256 MB memory-side cache), as a pass over many layers
    would.  Bytes: packed weights, the int8 rows, the int32 output.  dX runs
    with a workspace (the contraction split across workgroups where that
    applies, two kernels per call); the one-pass call is timed beside it.
    `graph_us` replays the same `steps` calls from one captured HIP graph:
    the device-bound time per call, where the eager loop is bound by the
    host's launch rate (the smallest shape)."""
    out = {}
    dev = torch.device("cuda:0")

    def timed(call, Xd, Ws, O, copies):
        first = torch.empty_like(O)
        call(Xd, Ws[0], first, stream)
        for i in range(3):
            call(Xd, Ws[i % copies], O, stream)
        torch.cuda.synchronize()
        if not torch.equal(first, O):
            raise RuntimeError(f"skinny {op}: copies of the same weights gave different results")
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(steps):
            call(Xd, Ws[(i + 3) % copies], O, stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps / 1e3, first

    def graph_timed(call, Xd, Ws, O, copies, first):
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                call(Xd, Ws[(i + 3) % copies], O, side)
        O.zero_()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        if not torch.equal(first, O):
            raise RuntimeError(f"skinny {op}: the graph replay differs from the eager calls")
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            ev0.record(stream)
            g.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        if not torch.equal(first, O):
            raise RuntimeError(f"skinny {op}: the second graph replay differs from the eager calls")
        del g
        return ev0.elapsed_time(ev1) / steps / 1e3

    for (M, N, K) in SKINNY:
        one_pass = None
        if op == "fwd":
            X, Wp = synth.fwd_inputs(seed, M, N, K, 3)
            call = lambda Xd, W, O, s: B.ternary_gemm_s8(Xd, W, C=O, stream=s)
            shape, byts = (M, N), N * (K // 4) + M * K + 4 * M * N
        else:
            X, Wp = synth.dx_inputs(seed, M, N, K, 3)
            nws = B.ternary_gemm_dx_workspace(M, N, K)
            ws = torch.empty(nws, dtype=torch.uint8, device=dev)   # empty: no query per call
            call = lambda Xd, W, O, s: B.ternary_gemm_s8_dx_ws(Xd, W, K, workspace=ws, dX=O, stream=s)
            one_pass = lambda Xd, W, O, s: B.ternary_gemm_s8_dx(Xd, W, K, dX=O, stream=s)
            shape, byts = (M, K), N * (K // 4) + M * N + 4 * M * K
        copies = max(2, -(-(512 << 20) // (N * K // 4)))
        Xd = torch.from_numpy(X).to(dev)
        Ws = torch.from_numpy(Wp).to(dev).unsqueeze(0).repeat(copies, 1, 1)
        O = torch.empty(shape, dtype=torch.int32, device=dev)
        t, first = timed(call, Xd, Ws, O, copies)
        tg = graph_timed(call, Xd, Ws, O, copies, first)
        ops = 2 * M * N * K
        row = {"avg_us": t * 1e6, "gbps": byts / t / 1e9, "hbm_frac": byts / t / PEAK_HBM_BPS,
               "tops": ops / t / 1e12, "algorithmic_bytes": byts, "ops": ops, "weight_copies": copies,
               "graph_us": tg * 1e6}
        if one_pass is not None:
            t1, first1 = timed(one_pass, Xd, Ws, O, copies)
            if not torch.equal(first, first1):
                raise RuntimeError(f"skinny dX {M}x{N}x{K}: the workspace and one-pass calls differ")
            row["workspace_bytes"] = nws
            row["kernels_per_call"] = 2 if nws else 1
            row["one_pass_us"] = t1 * 1e6
        out[f"{M}x{N}x{K}"] = row
        del Ws, Xd, O, first
        torch.cuda.empty_cache()
    head = out["27x16384x16384"]
    kernel = "skinny" if op == "fwd" else "skinny_dx_split"
    out["roofline"] = {"bound": "hbm", "achieved": head["gbps"], "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                       "frac": head["hbm_frac"], "kernel": kernel, "workload": "27x16384x16384",
                       "traffic": recorded_traffic(kernel, "27x16384x16384")}
    return out


def floors(B, torch, stream, M, N, steps):
    """The bounds the forward's time is compared with, measured by the probe
    library (csrc/roofline.hip) with HIP events on `stream`: a write-only
    pass over an int32 buffer of the forward's output size (M x N), and
    MFMA-only loops of each int8 shape, 8 waves per CU."""
    import ctypes
    from ternary_weight_int8_amd import build as hb
    if not os.path.exists(hb.PROBE_LIB):
        raise RuntimeError(f"{hb.PROBE_LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(hb.PROBE_LIB)
    L.tgemm_roofline_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
    L.tgemm_roofline_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p]
    cus, _ = B.machine()
    s = stream.cuda_stream

    def timed(fn, reps):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3   # seconds per launch

    out = {}
    buf = torch.empty(M * N, dtype=torch.int32, device=stream.device)
    t = timed(lambda: L.tgemm_roofline_fill(buf.data_ptr(), M * N, 1, s), steps)
    out["store_floor"] = {"bytes": M * N * 4, "us": t * 1e6, "tbs": M * N * 4 / t / 1e12,
                          "note": "one write-only pass over the forward's int32 output size"}
    del buf
    mo = torch.empty(cus * 512, dtype=torch.int32, device=stream.device)
    macs = ctypes.c_int64(0)
    for shape, iters in ((16, 8000), (32, 4000)):
        t = timed(lambda: L.tgemm_roofline_mfma(mo.data_ptr(), shape, iters, cus, ctypes.byref(macs), s),
                  max(steps // 2, 1))
        ops = 2 * macs.value
        out[f"mfma_{shape}"] = {"tops": ops / t / 1e12, "frac": ops / t / PEAK_INT8_OPS,
                                "instruction": {16: "v_mfma_i32_16x16x64_i8",
                                                32: "v_mfma_i32_32x32x32_i8"}[shape],
                                "note": "MFMAs only, independent accumulators, 2 waves per SIMD"}
    return out


def backward_rows(B, synth, torch, stream, seed, steps):
    """dX and dW of the pages' backward batch (1782 rows, N = 3456, K = 1280),
    warm inputs, each over `steps` launches, eagerly and replayed from one
    captured HIP graph (checked against the eager result).  Ops 2 MNK;
    bytes as the step's."""
    dev = torch.device("cuda:0")
    M, N, K = 1782, 3456, 1280
    A, Wp = synth.fwd_inputs(seed, M, N, K, 3)
    dC = synth.uniform_int8(seed, synth.STREAM_DC, M, N)
    Ad, Wd, dCd = (torch.from_numpy(x).to(dev) for x in (A, Wp, dC))
    cases = {"dx": (lambda O, s: B.ternary_gemm_s8_dx(dCd, Wd, K, dX=O, stream=s), (M, K)),
             "dw": (lambda O, s: B.ternary_gemm_s8_dw(Ad, dCd, dW=O, stream=s), (K, N))}
    out = {"workload": f"{M}x{N}x{K}"}
    for name, (call, shape) in cases.items():
        O = torch.empty(shape, dtype=torch.int32, device=dev)
        for _ in range(3):
            call(O, stream)
        torch.cuda.synchronize()
        first = O.clone()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(steps):
            call(O, stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        t = ev0.elapsed_time(ev1) / steps / 1e3
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(steps):
                call(O, side)
        O.zero_()
        with torch.cuda.stream(stream):
            ev0.record(stream)
            g.replay()
            ev1.record(stream)
        torch.cuda.synchronize()
        if not torch.equal(O, first):
            raise RuntimeError(f"backward {name}: the graph replay differs from the eager calls")
        tg = ev0.elapsed_time(ev1) / steps / 1e3
        del g
        ops = 2 * M * N * K
        byts = kernel_work(name, M, N, K)[1]
        out[name] = {"avg_us": t * 1e6, "graph_us": tg * 1e6, "tops": ops / tg / 1e12,
                     "mfma_frac": ops / tg / PEAK_INT8_OPS, "gbps": byts / tg / 1e9,
                     "kernel": int(B.plan(name, M, N, K).kernel)}
    return out


def prep_steps(B, synth, torch, stream, seed, steps):
    """The steps before the product, each timed over `steps` launches on
    inputs cycled through enough copies (more than 256 MB in all) that every
    launch reads its input from HBM: packing ternary weights at 16384 x 16384
    (the skinny workload's weights), and quantizing bf16 activations of the
    step's shape (16384 x 1280) per row and per column.  Bytes: input read
    once, outputs written once."""
    dev = torch.device("cuda:0")
    out = {}
    cases = [
        ("pack", "16384x16384", lambda: synth.ternary_int8(seed, 16384, 16384),
         lambda x, o: B.ternary_pack_weights(x, Wpacked=o[0], stream=stream),
         lambda x: (torch.empty((x.shape[0], x.shape[1] // 4), dtype=torch.uint8, device=dev),),
         lambda R, C: R * C + R * C // 4),
        ("quantize_rows", "16384x1280", lambda: synth.float_inputs(seed, synth.STREAM_X, 16384, 1280, "bf16"),
         lambda x, o: B.ternary_quantize_rows(x, Q=o[0], scale=o[1], stream=stream),
         lambda x: (torch.empty(x.shape, dtype=torch.int8, device=dev),
                    torch.empty((x.shape[0],), dtype=torch.float32, device=dev)),
         lambda R, C: 2 * R * C + R * C + 4 * R),
        ("quantize_cols", "16384x1280", lambda: synth.float_inputs(seed, synth.STREAM_X, 16384, 1280, "bf16"),
         lambda x, o: B.ternary_quantize_cols(x, Q=o[0], scale=o[1], stream=stream),
         lambda x: (torch.empty(x.shape, dtype=torch.int8, device=dev),
                    torch.empty((x.shape[1],), dtype=torch.float32, device=dev)),
         lambda R, C: 2 * R * C + R * C + 4 * C),
    ]
    for name, tag, make, run, outs, nbytes in cases:
        x = torch.from_numpy(make()).to(dev)
        if x.dtype == torch.uint16:
            x = x.view(torch.bfloat16)
        R, C = x.shape
        copies = max(2, -(-(512 << 20) // (x.numel() * x.element_size())))
        xs = x.unsqueeze(0).repeat(copies, 1, 1)
        o = outs(x)
        for i in range(3):
            run(xs[i % copies], o)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(steps):
            run(xs[(i + 3) % copies], o)
        ev1.record(stream)
        torch.cuda.synchronize()
        t = ev0.elapsed_time(ev1) / steps / 1e3
        byts = nbytes(R, C)
        out[name] = {"workload": tag, "avg_us": t * 1e6, "gbps": byts / t / 1e9,
                     "algorithmic_bytes": byts, "input_copies": copies,
                     "roofline": {"bound": "hbm", "achieved": byts / t / 1e9, "peak": PEAK_HBM_BPS / 1e9,
                                  "unit": "GB/s", "frac": byts / t / PEAK_HBM_BPS,
                                  "traffic": recorded_traffic(name, tag)}}
        del x, xs, o
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-rows", type=int, default=16384,
                    help="rows of the batch the CPU oracle baseline runs on (0: skip)")
    ap.add_argument("--only", choices=["fwd", "dx", "dw"], default=None,
                    help="time a single product instead of the whole step (for profiling)")
    ap.add_argument("--scaled-steps", type=int, default=20,
                    help="after the timed step, time each product's scaled bf16 output "
                         "(the dequantizing epilogue) over this many launches (0: skip)")
    ap.add_argument("--skinny-steps", type=int, default=50,
                    help="after the timed step, time the few-row forward and dX (27 and 1 rows, "
                         "cold weights) over this many launches each (0: skip)")
    ap.add_argument("--backward-steps", type=int, default=50,
                    help="after the timed step, time dX and dW at the pages' backward batch "
                         "(1782 x 3456 x 1280) over this many launches each (0: skip)")
    ap.add_argument("--prep-steps", type=int, default=50,
                    help="after the timed step, time the packer and the quantizers over this many "
                         "launches each (0: skip)")
    ap.add_argument("--floor-steps", type=int, default=10,
                    help="after the timed step, measure the store floor for the forward's output size "
                         "and the MFMA-only rate with the probe kernels, over this many launches (0: skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before timing, run one plain device-to-device copy of this many MiB "
                         "(a known-size reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(each GPU would run these kernels on its own shard of the batch).", file=sys.stderr)
        sys.exit(2)

    import torch
    from ternary_weight_int8_amd import binding as B
    from ternary_weight_int8_amd import synth

    B.lib()  # fail loudly now if the library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    c = synth.CONFIGS["large"]
    M, N, K = c["M"], c["N"], c["K"]
    A, Wp = synth.fwd_inputs(args.seed, M, N, K, c["alphabet"])
    dC = synth.uniform_int8(args.seed, synth.STREAM_DC, M, N)

    Ad = torch.from_numpy(A).to(dev)
    Wd = torch.from_numpy(Wp).to(dev)
    dCd = torch.from_numpy(dC).to(dev)
    Cd = torch.empty((M, N), dtype=torch.int32, device=dev)
    dXd = torch.empty((M, K), dtype=torch.int32, device=dev)
    dWd = torch.empty((K, N), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    launches = {
        "fwd": lambda: B.ternary_gemm_s8(Ad, Wd, C=Cd, stream=stream),
        "dx": lambda: B.ternary_gemm_s8_dx(dCd, Wd, K, dX=dXd, stream=stream),
        "dw": lambda: B.ternary_gemm_s8_dw(Ad, dCd, dW=dWd, stream=stream),
    }
    names = [args.only] if args.only else ["fwd", "dx", "dw"]

    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        for n in names:
            launches[n]()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(args.steps)]
    t_wall = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, n in enumerate(names):
            launches[n]()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall

    total_ms = ev[0][0].elapsed_time(ev[-1][-1])
    per = {n: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
           for i, n in enumerate(names)}
    ms_per_step = total_ms / args.steps

    tag = f"{M}x{N}x{K}"
    kernels = {}
    for n in names:
        ops, byts = kernel_work(n, M, N, K)
        t = per[n] / 1e3
        kernels[n] = {
            "avg_us": per[n] * 1e3,
            "tops": ops / t / 1e12,
            "mfma_frac": ops / t / PEAK_INT8_OPS,
            "gbps": byts / t / 1e9,
            "hbm_frac": byts / t / PEAK_HBM_BPS,
            "bound": "hbm" if ops / byts < RIDGE else "mfma",
            "algorithmic_bytes": byts,
            "ops": ops,
        }
    kernels["fwd_context"] = {"pages_rtx4090_fwd_tops": 171,
                              "note": "the pages' forward at this shape on another vendor's GPU"}

    # The metric is the forward's: its TOPS at this shape, measured inside the
    # step.  At nominal peaks the forward is HBM-bound (583 ops per byte
    # against a ridge of 625), so its roofline is the HBM one, with the MFMA
    # fraction beside it.
    head = "fwd" if "fwd" in names else names[0]
    d = kernels[head]
    if d["bound"] == "hbm":
        roof = {"bound": "hbm", "achieved": d["gbps"], "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                "frac": d["hbm_frac"]}
    else:
        roof = {"bound": "mfma", "achieved": d["tops"], "peak": PEAK_INT8_OPS / 1e12,
                "unit": "TFLOP/s", "frac": d["mfma_frac"]}
    roof["mfma_frac"] = d["mfma_frac"]
    roof["kernel"] = head
    roof["traffic"] = recorded_traffic(head, tag)

    total_ops = sum(kernel_work(n, M, N, K)[0] for n in names)
    value = d["tops"]
    step = {"products": names, "tops": total_ops * args.steps / (total_ms / 1e3) / 1e12,
            "ms": ms_per_step,
            "note": "all products of one step (forward, dX, dW) over the step's time"}

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "wall_ms_per_step": t_wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": (f"ternary x int8 GEMM forward at M={M} N={N} K={K}, timed inside a step of "
                         + " + ".join({"fwd": "forward", "dx": "dX", "dw": "dW"}[n] for n in names)),
            "M": M, "N": N, "K": K, "seed": args.seed,
            "A": "int8 uniform [-128,127]", "W": "2-bit codes uniform over {0,1,2}",
            "dC": "int8 uniform [-128,127]",
        },
        "roofline": roof,
        "step": step,
        "kernels": kernels,
    }
    if args.scaled_steps > 0 and not args.only:
        line["scaled_outputs"] = scaled_outputs(B, synth, torch, stream, Ad, Wd, dCd, M, N, K,
                                                args.seed, args.scaled_steps)
    if args.skinny_steps > 0 and not args.only:
        line["skinny_forward"] = skinny_rows(B, synth, torch, stream, args.seed, args.skinny_steps, "fwd")
        line["skinny_dx"] = skinny_rows(B, synth, torch, stream, args.seed, args.skinny_steps, "dx")
    if args.backward_steps > 0 and not args.only:
        line["backward_1782"] = backward_rows(B, synth, torch, stream, args.seed, args.backward_steps)
    if args.prep_steps > 0 and not args.only:
        line["prep"] = prep_steps(B, synth, torch, stream, args.seed, args.prep_steps)
    if args.floor_steps > 0 and not args.only:
        line["floors"] = floors(B, torch, stream, M, N, args.floor_steps)
    if args.cpu_rows > 0 and int(os.environ.get("RANK", "0")) == 0:
        line["cpu_baseline"] = cpu_baseline(A, Wp, dC, K, min(args.cpu_rows, M))
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
