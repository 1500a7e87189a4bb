#!/usr/bin/env python3
"""Throughput of the binary linear / conv2d forward on one MI355X.

One step = one forward pass over one batch of synthetic input with the
weights already packed (the layers pack weights once, ahead of the forward):
activation sign+pack, then the binary contraction with its fused scale and
output-cast epilogue. The default workload is the largest one: the
16384 x 8192 x 8192 binary linear layer whose bf16 activations are signed and
packed inside each step, with fp32 output.

Prints ONE JSON line: binary TOPS (2*M*N*K per second; for conv M = batch*Ho*Wo,
N = out channels, K = C*k*k), the dominant kernel's roofline (average
duration from HIP events recorded around it on its own stream inside the
timed region) and the CPU oracle's throughput on the host as a baseline.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--path auto|xor|mfma]
"""
import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0           # HBM3E, MI355X
PEAK_MFMA_I8_TOPS = 5000.0      # dense int8 MFMA, MI355X
PEAK_MFMA_F4_TOPS = 10100.0     # dense fp4 MFMA, MI355X
PEAK_MFMA_BF16_TFLOPS = 2500.0  # dense bf16 / fp16 MFMA, MI355X
# XOR path: 256 CUs x 64 lanes x 2.4 GHz lane-ops; one v_xor_b32 + one v_bcnt_u32_b32
# cover 32 MACs = 64 binary ops, i.e. 32 binary ops per lane-op.
PEAK_VALU_BINARY_TOPS = 256 * 64 * 2.4e9 * 32 / 1e12

DEFAULT_WORKLOAD = "linear_16384x8192x8192_bf16"
# Codec workloads: one HBM-bound kernel over one workload's activation (no contraction).
#   name -> (kernel kind, workload whose x it reads, shift dtype or None)
CODEC_WORKLOADS = {
    "pack_linear_16384x8192_bf16": ("pack", "linear_16384x8192x8192_bf16", None),
    "pack_shift_linear_16384x8192_bf16": ("pack_shift", "linear_16384x8192x8192_bf16", "f32"),
    "pack_nchw_128x128x28x28_f16": ("pack_nchw", "conv_down_s2_f16", None),
    "pack_nchw_32x256x14x14_f32": ("pack_nchw", "conv_resnet18_s3_f32", None),
    "pack_shift_nchw_128x128x28x28_f16": ("pack_nchw", "conv_down_s2_f16", "f16"),
    "abs_mean_16384x8192_bf16": ("abs_mean", "linear_16384x8192x8192_bf16", None),
    # one-pass prologue: the shifted pack and the lazy scale's sum of |x| from one read of x
    "prologue_linear_16384x8192_bf16": ("prologue", "linear_16384x8192x8192_bf16", "f32"),
    "prologue_nchw_128x128x28x28_f16": ("prologue_nchw", "conv_down_s2_f16", "f16"),
}
# W8A8 conv workloads (the blog's quantized im2col + GEMM): name -> (conv workload, amax_x, amax_w)
W8A8_WORKLOADS = {
    "w8a8_conv_128x128x28x28_s2_f16": ("conv_down_s2_f16", 4.0, 3.0),
    "w8a8_conv_128x128x28x28_d2_f16": ("conv_dil2_f16", 4.0, 3.0),
}
# straight-through linear backward (grad_input with clip mask and grad_scale_a, grad_weight):
# name -> linear workload whose x, W and output shape it differentiates
BWD_WORKLOADS = {
    "bwd_linear_2048x4096x4096_f16": "linear_2048x4096x4096_f16",
    "bwd_linear_16384x8192x8192_bf16": "linear_16384x8192x8192_bf16",
}
# straight-through conv backward (grad_input through columns + col2im with the clip mask and
# grad_scale_a, grad_weight against the unfolded input with its int8 codes): name -> conv workload
BWD_CONV_WORKLOADS = {
    "bwd_conv_128x128x28x28_s2_f16": "conv_down_s2_f16",
    "bwd_conv_128x128x28x28_d2_f16": "conv_dil2_f16",
}
PACK_WORKLOAD = "pack_linear_16384x8192_bf16"
# kernel kinds: source file, kernel function name, roofline peak and arithmetic type
KERNEL_SOURCES = {"mfma": "gemm_mfma.hip", "mfma_fp4": "gemm_mfma.hip", "xor": "gemm_xor.hip",
                  "w8a8": "w8a8.hip", "bwd": "backward.hip",
                  "pack": "pack.hip", "pack_shift": "pack.hip", "pack_nchw": "pack.hip",
                  "abs_mean": "pack.hip", "prologue": "pack.hip", "prologue_nchw": "pack.hip"}
KERNEL_NAMES = {"mfma": "mfma_kernel", "mfma_fp4": "mfma_kernel", "xor": "xor_kernel",
                "w8a8": "w8a8_conv_kernel", "bwd": "bwd_gemm_kernel",
                "pack": "pack_rows_kernel", "pack_shift": "pack_rows_shift_kernel",
                "pack_nchw": "pack_nchw_flat_kernel", "abs_mean": "abs_sum_kernel",
                "prologue": "pack_rows_shift_kernel", "prologue_nchw": "pack_nchw_flat_kernel"}
PEAKS = {"mfma": PEAK_MFMA_I8_TOPS, "mfma_fp4": PEAK_MFMA_F4_TOPS, "xor": PEAK_VALU_BINARY_TOPS,
         "w8a8": PEAK_MFMA_I8_TOPS, "bwd": PEAK_MFMA_BF16_TFLOPS}
DTYPES = {"mfma": "i8", "mfma_fp4": "fp4(e2m1)", "xor": "u32", "w8a8": "i8"}
CODEC_KINDS = ("pack", "pack_shift", "pack_nchw", "abs_mean", "prologue", "prologue_nchw")


def kernel_kind(name):
    """Kind of a demangled kernel name from a rocprofv3 counter file (None: not ours)."""
    if "bwd_gemm_kernel<" in name:
        # template arguments <bf16, A transposed, grad_input epilogue, ...>: the roofline line of
        # the backward is the grad_input contraction
        return "bwd" if re.search(r"bwd_gemm_kernel<\w+, false, true[,>]", name) else None
    for kind in CODEC_KINDS + ("xor", "w8a8"):
        if KERNEL_NAMES[kind] + "<" in name or KERNEL_NAMES[kind] + "(" in name:
            return kind
    if "mfma_kernel<" in name:
        # the tile's seventh template argument is the fp4 flag
        m = re.search(r"Tile<(?:\d+, ){6}(true|false)", name)
        return "mfma_fp4" if m and m.group(1) == "true" else "mfma"
    return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def src_sha(kind):
    """Hash of the kernel's source file with comments and blank lines removed, so that a
    traffic record survives comment edits but not code changes."""
    path = os.path.join(ROOT, "convolution_bnn_pack_amd", "csrc", KERNEL_SOURCES[kind])
    code = []
    for line in open(path).read().splitlines():
        line = line.split("//", 1)[0].rstrip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def traffic_for(kind, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when absent or
    when the kernel source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kind}|{workload}")
    if not rec or rec.get("src_sha") != src_sha(kind):
        return None
    return rec.get("bytes_per_launch")


def pmc_summary(args):
    """Scaled HBM traffic per launch from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE).

    Each counter is read in KiB per dispatch. The copy-calibration kernel in the same file
    moved a known number of bytes (read = write = copy size); the ratio known/counted is the
    scale applied to the workload kernel's reading. Writes profiles/traffic.json."""
    import csv
    import statistics

    def read(path, counter):
        vals, order = {}, {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            order.setdefault(r["Kernel_Name"], []).append(int(r["Dispatch_Id"]))
        return vals, order

    wl = args.workload
    kind = CODEC_WORKLOADS[wl][0] if wl in CODEC_WORKLOADS else None
    out = {}
    for counter, path in (("FETCH_SIZE", args.pmc_summary[0]), ("WRITE_SIZE", args.pmc_summary[1])):
        vals, order = read(path, counter)
        # the five calibration copies are the last copy dispatches of the run (copies made
        # while setting up the workload, e.g. of the activation, come earlier)
        copy = sorted((d, v) for k, vs in vals.items() if args.copy_kernel in k
                      for d, v in zip(order[k], vs))[-5:]
        if not copy:
            raise SystemExit(f"no {args.copy_kernel} kernel in {path}")
        copy_kib = statistics.median(v for _, v in copy)
        scale = (args.copy_mib << 20) / 1024.0 / copy_kib if args.copy_mib else 1.0
        for k in ([kind] if kind else ["mfma", "mfma_fp4", "xor", "w8a8", "bwd"]):
            # the workload's kernel is the instantiation launched most often (the parity spot
            # check adds single launches of other output types); a codec workload names its
            # kernel (kinds that share a kernel function, e.g. the one-pass prologue, differ by
            # instantiation only)
            def is_k(name):
                if kind:
                    return KERNEL_NAMES[k] + "<" in name or KERNEL_NAMES[k] + "(" in name
                return kernel_kind(name) == k
            cands = [(len(vs), name) for name, vs in vals.items() if is_k(name)]
            if not cands:
                continue
            _, name = max(cands)
            rec = out.setdefault(k, {"kernel": KERNEL_NAMES[k], "launches": len(vals[name])})
            rec[counter.lower() + "_kib_median"] = statistics.median(vals[name])
            rec[counter.lower() + "_scale"] = scale
    path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    for k, rec in out.items():
        if "fetch_size_kib_median" not in rec or "write_size_kib_median" not in rec:
            continue
        fetch = rec["fetch_size_kib_median"] * 1024 * rec["fetch_size_scale"]
        write = rec["write_size_kib_median"] * 1024 * rec["write_size_scale"]
        db[f"{k}|{wl}"] = {"kernel": KERNEL_NAMES[k],
            "bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
            "write_bytes": round(write), "fetch_scale": round(rec["fetch_size_scale"], 4),
            "write_scale": round(rec["write_size_scale"], 4), "src_sha": src_sha(k),
            "launches_measured": rec["launches"]}
    os.makedirs(os.path.dirname(path), exist_ok=True)
    json.dump(db, open(path, "w"), indent=1, sort_keys=True)
    print(json.dumps(db, indent=1, sort_keys=True))


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None where it is not readable."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, x, w):
    """The oracle as it stands on the host cores: the whole workload when it takes under
    about 30 s, else a row / image sample sized for ~15 s, scaled to binary TOPS."""
    import oracle
    cores = oracle.num_threads()
    if wl.kind == "linear":
        # a probe of a few hundred rows: a handful of rows is too short to time with 16 threads
        probe = max(1, min(wl.m, 256))
        t0 = time.perf_counter()
        oracle.linear_acc(x, w, rows=range(probe))
        t_probe = time.perf_counter() - t0
        rows = wl.m if t_probe / probe * wl.m < 30 else max(probe, int(15 / (t_probe / probe)))
        t0 = time.perf_counter()
        acc = oracle.linear_acc(x, w, rows=None if rows == wl.m else range(rows))
        oracle.scale(acc, 1.0, 1.0)
        dt = time.perf_counter() - t0
        ops = 2.0 * rows * wl.n * wl.k
        sample = "whole workload" if rows == wl.m else f"first {rows} of {wl.m} rows"
    else:
        t0 = time.perf_counter()
        oracle.conv2d_acc(x, w, wl.stride, wl.padding, wl.dilation, images=[0])
        t_img = time.perf_counter() - t0
        imgs = wl.batch if t_img * wl.batch < 30 else max(1, int(15 / t_img))
        t0 = time.perf_counter()
        acc = oracle.conv2d_acc(x, w, wl.stride, wl.padding, wl.dilation,
                                images=None if imgs == wl.batch else range(imgs))
        oracle.scale(acc, 1.0, 1.0)
        dt = time.perf_counter() - t0
        m, n, k = wl.gemm_mnk()
        ops = 2.0 * (m // wl.batch) * imgs * n * k
        sample = "whole workload" if imgs == wl.batch else f"first {imgs} of {wl.batch} images"
    return {"value": round(ops / dt / 1e12, 6), "unit": "binary TOPS", "cores": cores,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{sample} ({dt:.2f} s, sign + contraction + scale)"}


# Shapes of the path table (--path-table): linear (m, n, k) and conv
# (batch, c, h, w, out_channels, kernel, stride, padding, dilation).
PATH_TABLE_LINEAR = [(64, 256, 512), (128, 256, 1024), (256, 256, 1024), (256, 512, 2048),
                     (512, 512, 2048), (512, 1024, 2048), (1024, 1024, 1024), (1024, 1024, 4096),
                     (1024, 2048, 4096), (2048, 2048, 2048), (2048, 4096, 4096), (4096, 4096, 4096),
                     (8192, 8192, 8192), (64, 4096, 4096), (16, 8192, 8192)]
PATH_TABLE_CONV = [(1, 64, 14, 14, 64, 3, 1, 1, 1), (8, 64, 28, 28, 64, 3, 1, 1, 1),
                   (32, 256, 14, 14, 256, 3, 1, 1, 1), (128, 128, 28, 28, 256, 3, 2, 1, 1),
                   (128, 128, 28, 28, 256, 3, 1, 2, 2), (16, 512, 7, 7, 512, 3, 1, 1, 1),
                   (64, 64, 56, 56, 64, 3, 1, 1, 1), (8, 256, 14, 14, 256, 1, 1, 0, 1)]


def path_table():
    """Kernel time of the three contraction paths (XOR, int8 MFMA, fp4 MFMA) over linear and conv
    shapes on random packed words (f16 output; HIP events around a graph of 50 back-to-back
    launches), and the path AUTO picks; prints a markdown table."""
    import torch

    import convolution_bnn_pack_amd as bnn

    dev = torch.device("cuda:0")
    lib = bnn.lib
    gen = torch.Generator(device=dev).manual_seed(0)

    def words(*shape):
        return torch.randint(-2 ** 31, 2 ** 31 - 1, shape, dtype=torch.int32, device=dev, generator=gen)

    def time_call(f, reps=50):
        for _ in range(3):
            assert f() == 0
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                f()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    paths = [("XOR", bnn.PATH_XOR), ("int8", bnn.PATH_MFMA), ("fp4", bnn.PATH_MFMA_FP4)]
    names = {bnn.PATH_XOR: "XOR", bnn.PATH_MFMA: "int8", bnn.PATH_MFMA_FP4: "fp4"}
    print("| layer | MACs | XOR us | int8 us | fp4 us | AUTO | fastest |")
    print("|---|---|---|---|---|---|---|")
    for shape in PATH_TABLE_LINEAR + PATH_TABLE_CONV:
        if len(shape) == 3:
            m, n, k = shape
            xp, wp = words(m, k // 32), words(n, k // 32)
            out = torch.empty((m, n), dtype=torch.float16, device=dev)
            label, macs = f"linear {m}x{n}x{k}", m * n * k
            auto = lib.bnn_gemm_auto_path(m, n, k)

            def call(path):
                return lambda: lib.bnn_gemm(xp.data_ptr(), bnn.U32_PACKED, wp.data_ptr(), m, n, k, 1.0, 1.0,
                                            path, out.data_ptr(), bnn.F16, None, 0,
                                            torch.cuda.current_stream().cuda_stream)
        else:
            b, c, h, w, o, ks, st, pd, dl = shape
            ho = (h + 2 * pd - dl * (ks - 1) - 1) // st + 1
            wo = (w + 2 * pd - dl * (ks - 1) - 1) // st + 1
            cw = (c + 31) // 32
            xp, wp = words(b, h, w, cw), words(o, ks, ks, cw)
            out = torch.empty((b, o, ho, wo), dtype=torch.float16, device=dev)
            label = f"conv {b}x{c}x{h}x{w}->{o}, {ks}x{ks} s{st} p{pd} d{dl}"
            macs = b * ho * wo * o * c * ks * ks
            auto = lib.bnn_conv2d_auto_path(b, c, h, w, o, ks, st, pd, dl)

            def call(path):
                return lambda: lib.bnn_conv2d(xp.data_ptr(), bnn.U32_PACKED, b, c, h, w, wp.data_ptr(), o, 1.0,
                                              1.0, ks, st, pd, dl, path, out.data_ptr(), bnn.F16, None, 0,
                                              torch.cuda.current_stream().cuda_stream)
        t = {name: time_call(call(code)) for name, code in paths}
        best = min(t, key=t.get)
        print(f"| {label} | {macs:.3g} | {t['XOR']:.1f} | {t['int8']:.1f} | {t['fp4']:.1f} | "
              f"{names.get(auto, auto)} | {best} |", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--path", default="auto", choices=["auto", "xor", "mfma", "mfma_fp4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the workload, run 5 plain device copies of this many MiB "
                         "(reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE run, "
                         "WRITE_SIZE run; each also holding the copy-calibration kernel) into HBM "
                         "bytes per launch of the workload's dominant kernel in profiles/traffic.json")
    ap.add_argument("--copy-kernel", default="copyBuffer",
                    help="substring naming the copy kernel in the counter files")
    ap.add_argument("--path-table", action="store_true",
                    help="time the three contraction paths over a set of linear and conv shapes "
                         "and print a markdown table (nothing else runs)")
    args = ap.parse_args()
    if args.path_table:
        path_table()
        return
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the binary forward has no "
              f"cross-GPU exchange here; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import convolution_bnn_pack_amd as bnn
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pack_only = args.workload in CODEC_WORKLOADS
    w8a8 = args.workload in W8A8_WORKLOADS
    bwd = args.workload in BWD_WORKLOADS
    bwd_conv = args.workload in BWD_CONV_WORKLOADS
    codec_kind, base, shift_dt = CODEC_WORKLOADS.get(args.workload, (None, None, None))
    if w8a8:
        base, amax_x, amax_w = W8A8_WORKLOADS[args.workload]
    if bwd:
        base = BWD_WORKLOADS[args.workload]
    if bwd_conv:
        base = BWD_CONV_WORKLOADS[args.workload]
    wl = synth.WORKLOADS[base if (pack_only or w8a8 or bwd or bwd_conv) else args.workload]
    log(f"workload {args.workload}: generating inputs")
    x, w, sa, sw = synth.make_inputs(wl, draw_weight=not pack_only)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    xd = x.to(dev)
    lib = bnn.lib
    xcode = bnn._DT[xd.dtype]

    def cur_stream():
        # read at call time: under graph capture the current stream is the capture stream
        return torch.cuda.current_stream().cuda_stream

    if pack_only:
        # enough copies of the activation, used in turn, that every pass reads HBM rather than
        # the 256 MB last-level cache
        xbytes = xd.numel() * xd.element_size()
        ncopy = max(2, -(-(640 << 20) // xbytes))
        xs = [xd] + [xd.clone() for _ in range(ncopy - 1)]
        path_used = None
        if wl.kind == "linear":
            words = wl.m * wl.k // 32
            xp = torch.empty((wl.m, wl.k // 32), dtype=torch.int32, device=dev)
        else:
            words = wl.batch * wl.h * wl.w * wl.c // 32
            xp = torch.empty((wl.batch, wl.h, wl.w, wl.c // 32), dtype=torch.int32, device=dev)
        bias = None
        if shift_dt:
            nb = wl.k if wl.kind == "linear" else wl.c
            bias = synth.make_shift(nb, shift_dt, wl.seed + 50).to(dev)
            bcode = bnn._DT[bias.dtype]
        if codec_kind == "pack":
            fn = lambda i: lib.bnn_pack_sign(xs[i % ncopy].data_ptr(), xcode, wl.m, wl.k,
                                             xp.data_ptr(), cur_stream())
        elif codec_kind == "pack_shift":
            fn = lambda i: lib.bnn_pack_sign_shift(xs[i % ncopy].data_ptr(), xcode, wl.m, wl.k,
                                                   bias.data_ptr(), bcode, bias.numel(),
                                                   xp.data_ptr(), cur_stream())
        elif codec_kind == "pack_nchw" and bias is None:
            fn = lambda i: lib.bnn_pack_sign_nchw(xs[i % ncopy].data_ptr(), xcode, wl.batch, wl.c,
                                                  wl.h, wl.w, xp.data_ptr(), cur_stream())
        elif codec_kind == "pack_nchw":
            fn = lambda i: lib.bnn_pack_sign_nchw_shift(xs[i % ncopy].data_ptr(), xcode, wl.batch,
                                                        wl.c, wl.h, wl.w, bias.data_ptr(), bcode,
                                                        xp.data_ptr(), cur_stream())
        elif codec_kind == "prologue":
            scale_out = torch.empty((), dtype=torch.float64, device=dev)
            ws = torch.empty(lib.bnn_pack_sign_shift_abs_mean_workspace_bytes(wl.m, wl.k),
                             dtype=torch.uint8, device=dev)
            fn = lambda i: lib.bnn_pack_sign_shift_abs_mean(
                xs[i % ncopy].data_ptr(), xcode, wl.m, wl.k, bias.data_ptr(), bcode, bias.numel(), 2.0,
                xp.data_ptr(), scale_out.data_ptr(), ws.data_ptr(), ws.numel(), cur_stream())
        elif codec_kind == "prologue_nchw":
            scale_out = torch.empty((), dtype=torch.float64, device=dev)
            ws = torch.empty(lib.bnn_pack_sign_nchw_shift_abs_mean_workspace_bytes(
                xcode, wl.batch, wl.c, wl.h, wl.w), dtype=torch.uint8, device=dev)
            fn = lambda i: lib.bnn_pack_sign_nchw_shift_abs_mean(
                xs[i % ncopy].data_ptr(), xcode, wl.batch, wl.c, wl.h, wl.w, bias.data_ptr(), bcode, 2.0,
                xp.data_ptr(), scale_out.data_ptr(), ws.data_ptr(), ws.numel(), cur_stream())
        else:
            count = xd.numel()
            scale_out = torch.empty((), dtype=torch.float64, device=dev)
            ws = torch.empty(lib.bnn_abs_mean_workspace_bytes(count), dtype=torch.uint8, device=dev)
            words = 0
            fn = lambda i: lib.bnn_abs_mean_scale(xs[i % ncopy].data_ptr(), xcode, count, 2.0,
                                                  scale_out.data_ptr(), ws.data_ptr(), ws.numel(),
                                                  cur_stream())
        # algorithmic bytes: the activation read once, the packed words written once, the shift
        # vector read once (abs-mean: its partial sums, written and read once, and the result)
        bytes_per = xbytes + words * 4
        if bias is not None:
            bytes_per += bias.numel() * bias.element_size()
        if codec_kind in ("abs_mean", "prologue", "prologue_nchw"):
            bytes_per += 2 * ws.numel() + 8
        kernels = {"pack": [fn]}
        step_fns = kernels["pack"]
    elif bwd:
        # step: grad_input (GEMM with the clip mask and the grad_scale_a sums in its epilogue, then
        # the one-workgroup grad_scale_a reduction) and grad_weight; W is the layer's float weight
        # in the gradient's dtype
        m, n, k = wl.gemm_mnk()
        ops = 2 * 2.0 * m * n * k
        gdt = wl.x_dtype
        gcpu = synth.make_grad(m, n, gdt, wl.seed + 70)
        w = w.to(x.dtype).contiguous()
        gd, wd = gcpu.to(dev), w.to(dev)
        gi = torch.empty((m, k), dtype=torch.float32, device=dev)
        gsa = torch.empty((), dtype=torch.float64, device=dev)
        gw = torch.empty((n, k), dtype=torch.float32, device=dev)
        ws = torch.empty(lib.bnn_linear_grad_input_workspace_bytes(m, k), dtype=torch.uint8, device=dev)
        pack = lambda i: lib.bnn_linear_grad_input(gd.data_ptr(), wd.data_ptr(), xd.data_ptr(), xcode,
                                                   m, n, k, sa, sw, gi.data_ptr(), gsa.data_ptr(),
                                                   ws.data_ptr(), ws.numel(), cur_stream())
        core = lambda i: lib.bnn_linear_grad_weight(gd.data_ptr(), xd.data_ptr(), xcode, m, n, k, sa,
                                                    gw.data_ptr(), cur_stream())
        # the page's backward ends with the int8 codes of grad_weight: the step runs the
        # contraction + amax + coder call; the contraction alone is timed for the roofline
        gq = torch.empty((n, k), dtype=torch.int8, device=dev)
        gamax = torch.empty((), dtype=torch.float32, device=dev)
        qws = torch.empty(lib.bnn_linear_grad_weight_i8_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
        core_q = lambda i: lib.bnn_linear_grad_weight_i8(gd.data_ptr(), xd.data_ptr(), xcode, m, n, k, sa,
                                                         gw.data_ptr(), gq.data_ptr(), gamax.data_ptr(),
                                                         qws.data_ptr(), qws.numel(), cur_stream())
        path_used = None
        kernels = {"pack": [pack], "core": [core], "core_q": [core_q]}
        step_fns = [pack, core_q]
    elif bwd_conv:
        # step: grad_input (g to [O][pixels], the column contraction, col2im with the clip mask and
        # grad_scale_a) and grad_weight with its int8 codes (im2col of x, the contraction, amax,
        # coder); W is the layer's float weight in the gradient's dtype
        m, n, k = wl.gemm_mnk()            # m = batch*Ho*Wo, n = O, k = C*kh*kw
        ops = 2 * 2.0 * m * n * k
        w = w.to(x.dtype).contiguous()
        ho, wo = wl.out_shape()[2:]
        gcpu = synth.make_grad(wl.batch * wl.o * ho * wo, 1, wl.x_dtype, wl.seed + 70).view(
            wl.batch, wl.o, ho, wo)
        gd, wd = gcpu.to(dev), w.to(dev)
        geo = (wl.batch, wl.c, wl.h, wl.w, wl.o, wl.ks, wl.ks, wl.stride, wl.stride, wl.padding,
               wl.padding, wl.dilation, wl.dilation)
        gi = torch.empty((wl.batch, wl.c, wl.h, wl.w), dtype=torch.float32, device=dev)
        gsa = torch.empty((), dtype=torch.float64, device=dev)
        gw = torch.empty((wl.o, wl.c, wl.ks, wl.ks), dtype=torch.float32, device=dev)
        gq = torch.empty((wl.o, wl.c, wl.ks, wl.ks), dtype=torch.int8, device=dev)
        gamax = torch.empty((), dtype=torch.float32, device=dev)
        wsi = torch.empty(lib.bnn_conv2d_grad_input_workspace_bytes(*geo), dtype=torch.uint8, device=dev)
        wsw = torch.empty(lib.bnn_conv2d_grad_weight_workspace_bytes(*geo), dtype=torch.uint8, device=dev)
        pack = lambda i: lib.bnn_conv2d_grad_input(gd.data_ptr(), wd.data_ptr(), xd.data_ptr(), xcode,
                                                   *geo, sa, sw, gi.data_ptr(), gsa.data_ptr(),
                                                   wsi.data_ptr(), wsi.numel(), cur_stream())
        core = lambda i: lib.bnn_conv2d_grad_weight(gd.data_ptr(), xd.data_ptr(), xcode, *geo, sa,
                                                    gw.data_ptr(), gq.data_ptr(), gamax.data_ptr(),
                                                    wsw.data_ptr(), wsw.numel(), cur_stream())
        path_used = None
        kernels = {"pack": [pack], "core": [core]}
        step_fns = [pack, core]
    elif w8a8:
        # step: activation codes (NCHW -> NHWC int8), then the int8 conv; weight codes are made
        # once ahead, as the layer's weights are
        wq = bnn.quant_i8_weight(w.to(dev), amax_w)
        m, n, k = wl.gemm_mnk()
        ops = 2.0 * m * n * k
        out = torch.empty(wl.out_shape(), dtype=tdt[wl.out_dtype], device=dev)
        ocode = bnn._DT[out.dtype]
        xp = torch.empty((wl.batch, wl.h, wl.w, wl.c), dtype=torch.int8, device=dev)
        pack = lambda i: lib.bnn_quant_i8_nhwc(xd.data_ptr(), xcode, wl.batch, wl.c, wl.h, wl.w,
                                               amax_x, xp.data_ptr(), cur_stream())
        core = lambda i: lib.bnn_w8a8_conv2d(xp.data_ptr(), wl.batch, wl.c, wl.h, wl.w, wq.data_ptr(),
                                             wl.o, amax_x, amax_w, wl.ks, wl.ks, wl.stride, wl.stride,
                                             wl.padding, wl.padding, wl.dilation, wl.dilation,
                                             out.data_ptr(), ocode, cur_stream())
        path_used = None
        kernels = {"pack": [pack], "core": [core]}
        step_fns = [pack, core]
    else:
        wp = bnn.w_pack(w.to(dev))
        m, n, k = wl.gemm_mnk()
        ops = 2.0 * m * n * k
        path = bnn._PATHS[args.path]
        out = torch.empty(wl.out_shape(), dtype=tdt[wl.out_dtype], device=dev)
        ocode = bnn._DT[out.dtype]
        if wl.kind == "linear":
            xp = torch.empty((wl.m, wl.k // 32), dtype=torch.int32, device=dev)
            pack = lambda i: lib.bnn_pack_sign(xd.data_ptr(), xcode, wl.m, wl.k, xp.data_ptr(),
                                               cur_stream())
            core = lambda i: lib.bnn_gemm(xp.data_ptr(), bnn.U32_PACKED, wp.data_ptr(), wl.m, wl.n,
                                          wl.k, sa, sw, path, out.data_ptr(), ocode, None, 0,
                                          cur_stream())
            path_used = path if path else bnn.gemm_auto_path(wl.m, wl.n, wl.k)
        else:
            xp = torch.empty((wl.batch, wl.h, wl.w, wl.c // 32), dtype=torch.int32, device=dev)
            pack = lambda i: lib.bnn_pack_sign_nchw(xd.data_ptr(), xcode, wl.batch, wl.c, wl.h, wl.w,
                                                    xp.data_ptr(), cur_stream())
            core = lambda i: lib.bnn_conv2d(xp.data_ptr(), bnn.U32_PACKED, wl.batch, wl.c, wl.h,
                                            wl.w, wp.data_ptr(), wl.o, sa, sw, wl.ks, wl.stride,
                                            wl.padding, wl.dilation, path, out.data_ptr(), ocode,
                                            None, 0, cur_stream())
            path_used = path if path else bnn.conv2d_auto_path(wl.batch, wl.c, wl.h, wl.w, wl.o,
                                                               wl.ks, wl.stride, wl.padding,
                                                               wl.dilation)
        kernels = {"pack": [pack], "core": [core]}
        step_fns = [pack, core]

    # parity spot check before timing (int32 accumulators of sampled rows / images vs the oracle)
    parity = None
    if bwd:
        import oracle
        rows = sorted({0, 1, m // 2, m - 1})
        if pack(0) != 0 or core(0) != 0:
            raise RuntimeError("libbnn call failed")
        torch.cuda.synchronize()
        ref, _ = oracle.linear_grad_input(gcpu[rows], w, x[rows], sa, sw)
        got = gi[rows].cpu().double()
        # fp32 sums of n exact products: within n * 2^-24 * sum|g| * scale_w, plus the scale rounding
        bound = ((n + 1) * sw * gcpu[rows].double().abs().sum(1, keepdim=True) + ref.abs()) * 2.0 ** -24
        ok_in = bool(((got - ref).abs() <= bound).all())
        cols = sorted({0, n // 2, n - 1})
        refw = oracle.linear_grad_weight(gcpu[:, cols].contiguous(), x, sa)
        gotw = gw[cols].cpu().double()
        boundw = ((m + 1) * sa * gcpu[:, cols].double().abs().sum(0).unsqueeze(1) + refw.abs()) * 2.0 ** -24
        parity = ok_in and bool(((gotw - refw).abs() <= boundw).all())
        if core_q(0) != 0:
            raise RuntimeError("libbnn call failed")
        torch.cuda.synchronize()
        # codes (a property of the kernel's own outputs at any size): amax is the max of the fp32
        # gradient and each sampled code is the half-even rounding of gradient / (amax / 127), clamped
        amax_v = float(gamax.cpu())
        step = torch.tensor(amax_v, dtype=torch.float32) / 127.0
        want_q = torch.round(gw[cols].cpu() / step).clamp(-127, 127).to(torch.int8)
        parity = parity and amax_v == float(gw.abs().max().cpu())
        parity = parity and bool(torch.equal(gq[cols].cpu(), want_q))
        log(f"parity spot check vs oracle (within the fp32 summation bound): {parity}")
    elif bwd_conv:
        import oracle
        # two images end to end (grad_input of those images, the weight gradient summed over
        # them), recomputed on the device for the same two images: exact sums bound as in the tests
        imgs = [0, wl.batch - 1]
        g2, x2 = gcpu[imgs].contiguous(), x[imgs].contiguous()
        ref_i, ref_sa, ref_w = oracle.conv2d_grad(g2, w, x2, wl.stride, wl.padding, wl.dilation, sa, sw)
        gi2, _ = bnn.conv2d_grad_input(g2.to(dev), wd, x2.to(dev), sa, sw, wl.stride, wl.padding,
                                       wl.dilation)
        gw2 = bnn.conv2d_grad_weight(g2.to(dev), x2.to(dev), wl.ks, sa, wl.stride, wl.padding,
                                     wl.dilation)
        torch.cuda.synchronize()
        t_in = wl.o * wl.ks * wl.ks + 2
        ho, wo = wl.out_shape()[2:]
        t_w = 2 * ho * wo + 2
        abs_in, _, _ = oracle.conv2d_grad(g2.abs(), torch.ones_like(w), torch.zeros_like(x2),
                                          wl.stride, wl.padding, wl.dilation, sa, sw)
        _, _, abs_w = oracle.conv2d_grad(g2.abs(), torch.ones_like(w), torch.ones_like(x2),
                                         wl.stride, wl.padding, wl.dilation, sa, sw)
        U = 2.0 ** -24
        ok_i = bool(((gi2.cpu().double() - ref_i).abs() <= t_in * U * abs_in + U * ref_i.abs()).all())
        ok_w = bool(((gw2.cpu().double() - ref_w).abs() <= t_w * U * abs_w + U * ref_w.abs()).all())
        parity = ok_i and ok_w
        log(f"parity spot check vs oracle (within the fp32 summation bound): {parity}")
    elif w8a8:
        import oracle
        imgs = sorted({0, wl.batch - 1})
        ref = oracle.w8a8_conv2d_acc(x, w, wl.stride, wl.padding, wl.dilation, amax_x, amax_w,
                                     images=imgs)
        if pack(0) != 0:
            raise RuntimeError("libbnn call failed")
        got = bnn.w8a8_conv2d(xp, wq, amax_x, amax_w, wl.ks, wl.stride, wl.padding, wl.dilation,
                              out_dtype=torch.int32)[imgs].cpu()
        parity = bool(torch.equal(got, ref))
        log(f"parity spot check vs oracle: {parity}")
    elif not pack_only:
        import oracle
        if wl.kind == "linear":
            rows = sorted({0, 1, wl.m // 2, wl.m - 1})
            ref = oracle.linear_acc(x, w, rows=rows)
            got = bnn.gemm(xd, wp, 1.0, 1.0, path=args.path, out_dtype=torch.int32)[rows].cpu()
        else:
            imgs = sorted({0, wl.batch - 1})
            ref = oracle.conv2d_acc(x, w, wl.stride, wl.padding, wl.dilation, images=imgs)
            got = bnn.conv2d(xd, wp, 1.0, 1.0, wl.ks, wl.stride, wl.padding, wl.dilation,
                             path=args.path, out_dtype=torch.int32)[imgs].cpu()
        parity = bool(torch.equal(got, ref))
        log(f"parity spot check vs oracle: {parity}")

    def run(fns, i):
        for f in fns:
            if f(i) != 0:
                raise RuntimeError("libbnn call failed")

    # Steps are replayed from a HIP graph so that host-side launch cost (Python + ctypes)
    # does not leak into the GPU timeline: the captured kernels are exactly the eager ones.
    def capture(fns, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                run(fns, i)
        return g

    for i in range(args.warmup):
        run(step_fns, i)
    torch.cuda.synchronize()
    step_graph = capture(step_fns, args.steps)
    step_graph.replay()                      # one untimed replay: graph upload and warm caches
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps (one graph replay)")
    t0 = time.perf_counter()
    step_graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-kernel average launch duration: a graph of back-to-back launches of one kernel,
    # bracketed by HIP events on the stream it runs on
    reps = max(20, min(200, args.steps))
    kern_ms = {}
    for name, fns in kernels.items():
        g = capture(fns, reps)
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        kern_ms[name] = e0.elapsed_time(e1) / reps
        del g

    if pack_only:
        # the abs-mean step is two launches (partial sums, then the final one-workgroup sum):
        # its timed average covers both, so the roofline figure is a lower bound for the first
        dom_ms = kern_ms["pack"]
        achieved = bytes_per / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic_for(codec_kind, args.workload),
                "kernel": KERNEL_NAMES[codec_kind], "kernel_ms": round(dom_ms, 5)}
        value = bytes_per / (ms_per_step * 1e-3) / 1e9
        metric, unit = {"abs_mean": ("abs-mean scale bandwidth", "GB/s"),
                        "prologue": ("one-pass prologue bandwidth", "GB/s"),
                        "prologue_nchw": ("one-pass prologue bandwidth", "GB/s")}.get(
            codec_kind, ("sign+pack bandwidth", "GB/s"))
        dtype = "f64" if codec_kind == "abs_mean" else "u32"
    elif bwd_conv:
        # each entry point runs one 2*M*N*K-flop contraction plus its layout kernels; the roofline
        # line is the slower call's contraction measured as part of that call (an upper bound on
        # the contraction's own time)
        kind = "bwd"
        name, dom_ms = max((("grad_input", kern_ms["pack"]), ("grad_weight", kern_ms["core"])),
                           key=lambda t: t[1])
        achieved = ops / 2 / (dom_ms * 1e-3) / 1e12
        peak = PEAKS[kind]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None,
                "kernel": f"{name} call (transpose + bwd_gemm_kernel + layout kernels)",
                "kernel_ms": round(dom_ms, 5),
                "grad_input_call_ms": round(kern_ms["pack"], 5),
                "grad_weight_i8_call_ms": round(kern_ms["core"], 5)}
        value = ops / (ms_per_step * 1e-3) / 1e12
        metric, unit = "conv backward TFLOP/s (2 contractions of 2*M*N*K)", "TFLOP/s"
        dtype = wl.x_dtype
    elif bwd:
        # both launches are 2*M*N*K-flop contractions; the slower one is the roofline kernel
        kind = "bwd"
        name, dom_ms = max((("grad_input", kern_ms["pack"]), ("grad_weight", kern_ms["core"])),
                           key=lambda t: t[1])
        achieved = ops / 2 / (dom_ms * 1e-3) / 1e12
        peak = PEAKS[kind]
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic_for(kind, args.workload),
                "kernel": f"{KERNEL_NAMES[kind]} ({name})", "kernel_ms": round(dom_ms, 5),
                "traffic_kernel": "grad_input",
                "grad_input_ms": round(kern_ms["pack"], 5), "grad_weight_ms": round(kern_ms["core"], 5),
                "grad_weight_int8_codes_ms": round(kern_ms["core_q"] - kern_ms["core"], 5)}
        value = ops / (ms_per_step * 1e-3) / 1e12
        metric, unit = "backward TFLOP/s (2 contractions of 2*M*N*K)", "TFLOP/s"
        dtype = wl.x_dtype
    else:
        dom_ms = kern_ms["core"]
        kind = "w8a8" if w8a8 else {bnn.PATH_XOR: "xor", bnn.PATH_MFMA: "mfma",
                                    bnn.PATH_MFMA_FP4: "mfma_fp4"}[path_used]
        achieved = ops / (dom_ms * 1e-3) / 1e12
        peak = PEAKS[kind]
        roof = {"bound": "alu" if kind == "xor" else "mfma", "achieved": round(achieved, 2),
                "peak": round(peak, 1), "unit": "TOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic_for(kind, args.workload), "kernel": KERNEL_NAMES[kind],
                "kernel_ms": round(dom_ms, 5), "pack_kernel_ms": round(kern_ms["pack"], 5)}
        value = ops / (ms_per_step * 1e-3) / 1e12
        metric, unit = ("int8 TOPS (2*M*N*K/s)", "TOPS") if w8a8 else ("binary TOPS (2*M*N*K/s)", "TOPS")
        dtype = DTYPES[kind]

    result = {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": args.workload, "parallelism": "none (1 GPU)",
                   "timing": "HIP graph of the timed steps, replayed once untimed then once timed"},
        "roofline": roof,
    }
    if bwd_conv:
        result["config"].update({"m": m, "n": n, "k": k, "dtype": wl.x_dtype,
                                 "outputs": "grad_input fp32 NCHW, grad_scale_a f64, grad_weight fp32 OIHW and its int8 codes + amax"})
        result["parity_spot_check"] = parity
    elif bwd:
        result["config"].update({"m": m, "n": n, "k": k, "dtype": wl.x_dtype,
                                 "outputs": "grad_input fp32 [m, k], grad_scale_a f64, grad_weight fp32 [n, k] and its int8 codes + amax"})
        result["parity_spot_check"] = parity
    elif not pack_only:
        m, n, k = wl.gemm_mnk()
        result["config"].update({"m": m, "n": n, "k": k, "x_dtype": wl.x_dtype,
                                 "out_dtype": wl.out_dtype,
                                 "path": kind})
        result["parity_spot_check"] = parity
    if args.copy_mib:
        # plain device copies of a known size, for scaling the traffic counters
        n = args.copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n
        del src, dst
    if not args.no_cpu_baseline and bwd_conv:
        import oracle
        nimg = 2
        log(f"cpu baseline (oracle on host cores, both gradients of {nimg} images)")
        t0 = time.perf_counter()
        oracle.conv2d_grad(gcpu[:nimg].contiguous(), w, x[:nimg].contiguous(), wl.stride, wl.padding,
                           wl.dilation, sa, sw)
        dt_cpu = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(ops * nimg / wl.batch / dt_cpu / 1e12, 6),
                                  "unit": "TFLOP/s", "cores": oracle.num_threads(),
                                  "cpu_model": cpu_model(), "kind": "oracle",
                                  "sample": f"both gradients of the first {nimg} of {wl.batch} images ({dt_cpu:.2f} s)"}
    elif not args.no_cpu_baseline and bwd:
        import oracle
        rows = min(m, 4096)         # about 2-10 s of host work at the layer sizes
        log(f"cpu baseline (oracle on host cores, grad_input of {rows} rows)")
        t0 = time.perf_counter()
        oracle.linear_grad_input(gcpu[:rows].contiguous(), w, x[:rows].contiguous(), sa, sw)
        dt_cpu = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(2.0 * rows * n * k / dt_cpu / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                                  "sample": f"grad_input of the first {rows} of {m} rows ({dt_cpu:.2f} s)"}
    elif not args.no_cpu_baseline and w8a8:
        import oracle
        log("cpu baseline (oracle on host cores, one image)")
        t0 = time.perf_counter()
        oracle.w8a8_conv2d_acc(x, w, wl.stride, wl.padding, wl.dilation, amax_x, amax_w, images=[0])
        dt_cpu = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(ops / wl.batch / dt_cpu / 1e12, 6), "unit": "int8 TOPS",
                                  "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
                                  "sample": f"first 1 of {wl.batch} images ({dt_cpu:.2f} s, quantize + contraction)"}
    elif not args.no_cpu_baseline and not pack_only:
        log("cpu baseline (oracle on host cores)")
        del xd, xp
        result["cpu_baseline"] = cpu_baseline(wl, x, w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
