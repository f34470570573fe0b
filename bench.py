#!/usr/bin/env python3
"""Benchmark of the Quant Experts (QE) linear hot path on one MI355X.

Workload (one step): the seven decoder-layer linears of a Qwen2VL-72B-shaped layer
(q 8192->8192, k/v 8192->1024, o 8192->8192, gate/up 8192->29568, down 29568->8192),
W4A6, T = 4096 prefill tokens (3200 image-like + 896 text-like, synthetic), shared
expert rank 32, 8 routed experts of rank 32, router d_in x 8.  Every linear runs the
whole hot path: the prologue (route pass: router and shared-expert projections and
the per-token max |x/s|; route finish: argmin routing, u, s_x; expert-sorted pass:
A6 codes, stable bucketing and the selected routed expert's input v) and the
int8-MFMA main GEMM with the dequantization and the shared/routed low-rank terms
fused into its epilogue.  Inputs are resident in HBM before the timed region.

Prints one JSON line.  `value` is tokens/s of the whole layer (T / step time).
`roofline` is the dominant kernel, the main GEMM: one launch per group of linears that read
the same input (q+k+v, o, gate+up, down; 128-token tiles), timed with HIP events around each
of its launches on the stream it is launched on.

`--copy-calibration` only times a 1 GiB device copy (the reference kernel for the
HBM byte counters) and exits.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0    # MI355X dense int8 MFMA, tera-ops/s
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # HBM3E
METRIC = "QE-linear tokens/s + % int8-MFMA/HBM roofline, 72B shapes W4A6 (1 GPU)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048,
                    help="tokens of the workload the C oracle runs on every host core")
    ap.add_argument("--cpu-sample-tokens-1t", type=int, default=64,
                    help="tokens the C oracle runs on one host thread")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ceiling", action="store_true",
                    help="time the int8 and bf16 MFMA ceilings of this part at the 72B layer's GEMM shapes: the "
                         "library's main GEMM, torch's int8 and bf16 matrix products (hipBLASLt) and the MFMA "
                         "probe loops; prints one JSON line and exits")
    ap.add_argument("--decode-only", action="store_true",
                    help="run only the decode lines (Qwen2VL-72B up + down, T = 8, W3A16 and W4A6), print them "
                         "as one JSON line and exit (the workload of the decode traffic counters)")
    ap.add_argument("--mfma-counters", metavar="DIR",
                    help="summarize a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_I8 "
                         "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE GRBM_COUNT --kernel-trace "
                         "--output-format csv run (its output directory) per kernel and exit")
    ap.add_argument("--write-traffic", nargs=4, metavar="DIR",
                    help="rocprofv3 CSV directories: bench FETCH_SIZE, bench WRITE_SIZE, copy FETCH_SIZE, "
                         "copy WRITE_SIZE; writes the GEMM traffic summary under profiles/ and exits")
    return ap.parse_args()


def gemm_source_hash():
    h = hashlib.sha256()
    for f in ("k_gemm_w4.hip", "qe_dma.h", "qe_internal.h"):
        with open(os.path.join(ROOT, "quantized_linear_moe_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(per_launch_alg_bytes):
    """HBM bytes per GEMM launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel source (else None)."""
    p = os.path.join(ROOT, "profiles", "gemm_w4_qwen2vl72b_traffic.json")
    try:
        with open(p) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_hash") != gemm_source_hash():
        return None
    return d.get("hbm_bytes_per_launch", {}).get("total")


TRAFFIC_KERNEL = "gemm_w4_group_kernel"


def mfma_counters(d, n_simd=1024, n_xcd=8):
    """Matrix-core utilization and effective clock per kernel from one rocprofv3 counter run
    (CSV output).  Per dispatch: GRBM_GUI_ACTIVE is summed over the 8 XCDs, so
    clock = GRBM_GUI_ACTIVE / 8 / duration; MFMA busy = sum of SQ_VALU_MFMA_BUSY_CYCLES over
    the 1024 SIMDs / (GRBM_GUI_ACTIVE / 8 * 1024) (rocprofv3's MfmaUtil); int8 / bf16 ops =
    SQ_INSTS_VALU_MFMA_MOPS_* * 512.  Dispatches shorter than 100 us are left out (their
    GRBM counts include the dispatch overhead around the kernel)."""
    import csv
    import glob
    import collections
    cc = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    kt = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not cc or not kt:
        raise SystemExit(f"no counter_collection.csv / kernel_trace.csv under {d}")
    dur = {}
    with open(kt[0]) as fh:
        for r in csv.DictReader(fh):
            dur[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    disp = collections.defaultdict(dict)
    with open(cc[0]) as fh:
        for r in csv.DictReader(fh):
            v = disp[r["Dispatch_Id"]]
            v[r["Counter_Name"]] = v.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            v["kernel"] = r["Kernel_Name"]
    groups = collections.defaultdict(list)
    for did, v in disp.items():
        if did in dur and dur[did] >= 100_000:
            v["ns"] = dur[did]
            groups[v["kernel"].split("(")[0][:72]].append(v)
    print(f"{'kernel':72s} {'n':>4s} {'avg_us':>9s} {'clock_GHz':>9s} {'mfma_busy':>9s} {'int8_TOP/s':>10s} "
          f"{'bf16_TFLOP/s':>12s}")
    for name, vs in sorted(groups.items(), key=lambda kv: -sum(v["ns"] for v in kv[1])):
        ns = sum(v["ns"] for v in vs)
        gui = sum(v.get("GRBM_GUI_ACTIVE", 0.0) for v in vs)
        busy = sum(v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for v in vs)
        i8 = sum(v.get("SQ_INSTS_VALU_MFMA_MOPS_I8", 0.0) for v in vs) * 512
        bf = sum(v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for v in vs) * 512
        clock = gui / n_xcd / ns
        util = busy / (gui / n_xcd * n_simd) if gui else 0.0
        print(f"{name:72s} {len(vs):4d} {ns / len(vs) / 1e3:9.1f} {clock:9.3f} {util:9.3f} {i8 / ns / 1e3:10.1f} "
              f"{bf / ns / 1e3:12.1f}")


def write_traffic(d_bench_fetch, d_bench_write, d_copy_fetch, d_copy_write):
    """Write profiles/gemm_w4_qwen2vl72b_traffic.json from four rocprofv3 --pmc runs (CSV output
    directories): FETCH_SIZE and WRITE_SIZE of this benchmark (--steps 2 --warmup 1
    --no-cpu-baseline --no-extras), then of --copy-calibration.  The counters of the dominant
    GEMM are averaged over its dispatches and scaled by what they read for the 1 GiB copy."""
    import csv
    import glob

    def rows(d):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {d}")
        with open(f[0]) as fh:
            return list(csv.DictReader(fh))

    def mean_kib(d, counter, match):
        vals = [float(r["Counter_Value"]) for r in rows(d)
                if r["Counter_Name"] == counter and match(r["Kernel_Name"])]
        if not vals:
            raise SystemExit(f"no {counter} rows for the kernel under {d}")
        return sum(vals) / len(vals), len(vals)

    is_gemm = lambda k: TRAFFIC_KERNEL in k
    is_copy = lambda k: "copyBuffer" in k
    g_fetch, n_fetch = mean_kib(d_bench_fetch, "FETCH_SIZE", is_gemm)
    g_write, n_write = mean_kib(d_bench_write, "WRITE_SIZE", is_gemm)
    c_fetch, _ = mean_kib(d_copy_fetch, "FETCH_SIZE", is_copy)
    c_write, _ = mean_kib(d_copy_write, "WRITE_SIZE", is_copy)
    copy_bytes = 1 << 30
    f_fetch, f_write = copy_bytes / (c_fetch * 1024), copy_bytes / (c_write * 1024)
    fetch, write = g_fetch * 1024 * f_fetch, g_write * 1024 * f_write
    cmd = "rocprofv3 --pmc {c} --output-format csv -d {d} -o p -- python3 bench.py {a}"
    bench_args = "--steps 2 --warmup 1 --no-cpu-baseline --no-extras"
    out = {
        "kernel": TRAFFIC_KERNEL,
        "workload": "Qwen2VL-72B layer linears, W4A6, T=4096: the grouped main-GEMM launches q+k+v, o, gate+up and "
                    "down, averaged over them",
        "kernel_source_hash": gemm_source_hash(),
        "commands": [cmd.format(c="FETCH_SIZE", d=d_bench_fetch, a=bench_args),
                     cmd.format(c="WRITE_SIZE", d=d_bench_write, a=bench_args),
                     cmd.format(c="FETCH_SIZE", d=d_copy_fetch, a="--copy-calibration"),
                     cmd.format(c="WRITE_SIZE", d=d_copy_write, a="--copy-calibration")],
        "gemm_dispatches_averaged": {"FETCH_SIZE": n_fetch, "WRITE_SIZE": n_write},
        "gemm_FETCH_SIZE_KiB": round(g_fetch, 1),
        "gemm_WRITE_SIZE_KiB": round(g_write, 1),
        "copy_calibration": {"bytes_read": copy_bytes, "bytes_written": copy_bytes,
                             "FETCH_SIZE_KiB": round(c_fetch, 1), "WRITE_SIZE_KiB": round(c_write, 1),
                             "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)},
        "hbm_bytes_per_launch": {"fetch": round(fetch), "write": round(write), "total": round(fetch + write)},
        "note": "FETCH_SIZE counts L2 misses going to the fabric, so hits in the 256 MB Infinity Cache are "
                "included; each of the 8 XCDs streams the weights through its own L2.",
    }
    path = os.path.join(ROOT, "profiles", "gemm_w4_qwen2vl72b_traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(path, out["hbm_bytes_per_launch"])


def copy_calibration():
    import torch
    n = 1 << 28  # 1 GiB of float32, four times the Infinity Cache
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "ms": round(ms, 4),
                      "gbs_read_plus_write": round(8 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def ceiling(reps=20):
    """The int8 (and bf16) matrix-core rate this part reaches at the Qwen2VL-72B layer's GEMM shapes
    (T = 4096 tokens; q 8192x8192, gate/up 8192x29568, down 29568x8192), by three independent routes:
    the library's main GEMM (prologue first, then qe_wq_gemm timed alone), torch's int8 product
    torch._int_mm and torch's bf16 linear (both hipBLASLt) on the same shapes, and the MFMA probe
    loops.  Median of `reps` event-timed launches each, on torch's current stream (the one every
    launch here uses).  Run under rocprofv3 --pmc for the matrix-core busy cycles and the clock."""
    import torch
    import synth
    import quantized_linear_moe_amd as qe
    from quantized_linear_moe_amd import libqe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def med_ms(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    cfg = synth.get_config("qwen2vl_72b")
    T = cfg.T
    rows = []
    for name in ("q", "gate", "down"):
        spec = next(l for l in cfg.linears if l.name == name)
        params = synth.gen_linear(cfg, spec)
        layer = qe.QELinear.from_params(params, cfg.w_bits, cfg.a_bits, device=dev)
        x = synth.gen_activations(cfg, spec.stream).to(dev)
        ws = layer.workspace(T)
        codes = torch.empty(T, spec.d_in, dtype=torch.int8, device=dev)
        s_x = torch.empty(T, dtype=torch.float32, device=dev)
        u = torch.empty(T, libqe.rank_pad(cfg.r_shared), dtype=torch.bfloat16, device=dev)
        v = torch.empty(T, libqe.rank_pad(cfg.r_routed), dtype=torch.bfloat16, device=dev)
        e = torch.empty(T, dtype=torch.int32, device=dev)
        perm = torch.empty(T, dtype=torch.int32, device=dev)
        y = torch.empty(T, spec.d_out, dtype=torch.float32, device=dev)
        libqe.qe_linear_prologue(layer.lin, x, codes, s_x, u, v, e, ws, perm=perm)
        t_qe = med_ms(lambda: libqe.qe_wq_gemm(layer.lin, codes, s_x, None, T, u, v, e, y, None, ws, perm=perm))
        ops = 2.0 * T * spec.d_in * spec.d_out
        row = {"shape": f"{T}x{spec.d_in}x{spec.d_out}", "linear": name,
               "qe_gemm_us": round(t_qe * 1e3, 1), "qe_gemm_tops": round(ops / (t_qe * 1e-3) / 1e12, 1)}
        # torch int8 product: codes [T, d_in] times an int8 matrix of the same shape as the weights
        wq = torch.randint(-7, 8, (spec.d_out, spec.d_in), dtype=torch.int8, device=dev)
        for lay, b in (("nt", wq.t()), ("nn", wq.t().contiguous())):
            try:
                t_i = med_ms(lambda: torch._int_mm(codes, b))
                row[f"torch_int_mm_{lay}_us"] = round(t_i * 1e3, 1)
                row[f"torch_int_mm_{lay}_tops"] = round(ops / (t_i * 1e-3) / 1e12, 1)
            except RuntimeError as ex:  # not every layout is supported by the library
                row[f"torch_int_mm_{lay}_error"] = str(ex).splitlines()[0][:160]
        del wq
        wb = torch.from_numpy(params["W_f"]).to(torch.bfloat16).to(dev)
        xb = x.to(torch.bfloat16)
        t_b = med_ms(lambda: torch.nn.functional.linear(xb, wb))
        row["torch_bf16_linear_us"] = round(t_b * 1e3, 1)
        row["torch_bf16_linear_tflops"] = round(ops / (t_b * 1e-3) / 1e12, 1)
        rows.append(row)
        log(f"ceiling {name}: {row}")
        del layer, x, ws, codes, s_x, u, v, e, perm, y, wb, xb, params
        torch.cuda.empty_cache()
    peaks = measured_peaks(torch, libqe, dev)
    print(json.dumps({"ceiling_qwen2vl72b_T4096": rows, "probes": peaks,
                      "spec": {"int8_tops": PEAK_INT8_TOPS, "bf16_tflops": PEAK_BF16_TFLOPS}}), flush=True)


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.ceiling:
        ceiling()
        return
    if args.mfma_counters:
        mfma_counters(args.mfma_counters)
        return
    if args.decode_only:
        import torch
        import synth
        import quantized_linear_moe_amd as qe
        from quantized_linear_moe_amd import libqe
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        print(json.dumps({"decode_qwen2vl72b_up_down_w3a16_T8": decode_line(torch, synth, qe, libqe, dev, 3, 16),
                          "decode_qwen2vl72b_up_down_w4a6_T8": decode_line(torch, synth, qe, libqe, dev, 4, 6)}),
              flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the QE linear on exactly one GPU; multi-GPU runs are not part of this "
              f"benchmark (got --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import quantized_linear_moe_amd as qe
    from quantized_linear_moe_amd import libqe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.get_config("qwen2vl_72b")
    T = cfg.T
    want_cpu = not args.no_cpu_baseline

    # ------------------------------------------------------------ inputs (untimed)
    t_setup = time.time()
    xs_cpu = {s: synth.gen_activations(cfg, s) for s in cfg.streams()}
    xs = {s: t.to(dev) for s, t in xs_cpu.items()}
    layers, host_params = [], []
    for spec in cfg.linears:
        params = synth.gen_linear(cfg, spec)
        layer = qe.QELinear.from_params(params, cfg.w_bits, cfg.a_bits, device=dev)
        if want_cpu:
            host_params.append(params)  # the CPU-baseline leg quantizes W_f with the oracle
        else:
            del params["W_f"]
        layers.append((spec, layer))
        log(f"prepared {spec.name} {spec.d_in}->{spec.d_out}")
    # one workspace per linear: the linears that read the same input (q/k/v, gate/up) share one
    # route pass, which leaves each linear's partial sums in that linear's workspace
    wss = [torch.empty(libqe.qe_workspace_bytes(l.lin, T), dtype=torch.uint8, device=dev) for _, l in layers]
    groups = []  # indices of consecutive linears that read the same activation stream
    for i, (spec, _) in enumerate(layers):
        if groups and layers[groups[-1][0]][0].stream == spec.stream:
            groups[-1].append(i)
        else:
            groups.append([i])
    gi_of = {g[0]: k for k, g in enumerate(groups)}
    bufs = []
    for spec, layer in layers:
        bufs.append(dict(
            codes=torch.empty(T, spec.d_in, dtype=torch.int8, device=dev),
            s_x=torch.empty(T, dtype=torch.float32, device=dev),
            u=torch.empty(T, libqe.rank_pad(cfg.r_shared), dtype=torch.bfloat16, device=dev),
            v=torch.empty(T, libqe.rank_pad(cfg.r_routed), dtype=torch.bfloat16, device=dev),
            e=torch.empty(T, dtype=torch.int32, device=dev),
            perm=torch.empty(T, dtype=torch.int32, device=dev),
            y=torch.empty(T, spec.d_out, dtype=torch.float32, device=dev)))
    # reading 1 GiB (four times the 256 MB Infinity Cache) evicts it with clean lines
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s")

    # One step: every linear's prologue (route, bucket, quantize, adapter inputs) then its
    # GEMM, in layer order on one stream.  (Running the next prologue on a second stream
    # under the GEMM was measured slower: the GEMM occupies every CU and the prologue
    # kernels only get the gaps.)
    def step(ev=None):
        for g in groups:
            x = xs[layers[g[0]][0].stream]
            if len(g) == 1:
                b = bufs[g[0]]
                libqe.qe_linear_prologue(layers[g[0]][1].lin, x, b["codes"], b["s_x"], b["u"], b["v"], b["e"],
                                         wss[g[0]], perm=b["perm"])
            else:
                bb = [bufs[i] for i in g]
                libqe.qe_group_prologue([layers[i][1].lin for i in g], x, [b["codes"] for b in bb],
                                        [b["s_x"] for b in bb], [b["u"] for b in bb], [b["v"] for b in bb],
                                        [b["e"] for b in bb], [wss[i] for i in g], perm=[b["perm"] for b in bb])
            bb = [bufs[i] for i in g]
            if ev is not None:
                ev[gi_of[g[0]]][0].record()
            libqe.qe_group_gemm([layers[i][1].lin for i in g], [b["codes"] for b in bb], [b["s_x"] for b in bb], T,
                                [b["u"] for b in bb], [b["v"] for b in bb], [b["e"] for b in bb],
                                [b["y"] for b in bb], [wss[i] for i in g], perm=[b["perm"] for b in bb])
            if ev is not None:
                ev[gi_of[g[0]]][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev_t = lambda: torch.cuda.Event(enable_timing=True)
    K = args.steps
    evs = [[(ev_t(), ev_t()) for _ in groups] for _ in range(K)]
    marks = [ev_t() for _ in range(K + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks[0].record()
    for k in range(K):
        step(evs[k])
        marks[k + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = marks[0].elapsed_time(marks[K]) / K
    step_ms = np.array([marks[k].elapsed_time(marks[k + 1]) for k in range(K)])
    gemm_ms = np.array([[a.elapsed_time(b) for (a, b) in evs[k]] for k in range(K)])  # [K, groups]
    gemm_ms_step = float(gemm_ms.sum(axis=1).mean())

    # cold steps: the Infinity Cache flushed before each (timed alone, not part of `value`)
    cold = []
    for _ in range(min(K, 20)):
        flush.sum()
        a, b = ev_t(), ev_t()
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush

    # the composite entry points on the same inputs (must match the split prologue + GEMM)
    def composite():
        for g in groups:
            libqe.qe_group_forward([layers[i][1].lin for i in g], xs[layers[g[0]][0].stream],
                                   [bufs[i]["y"] for i in g], [bufs[i]["e"] for i in g], [wss[i] for i in g])
    for _ in range(2):
        composite()
    torch.cuda.synchronize()
    s2, e2 = ev_t(), ev_t()
    s2.record()
    for _ in range(K):
        composite()
    e2.record()
    torch.cuda.synchronize()
    ms_step_fwd = s2.elapsed_time(e2) / K

    # the same composite step captured once in a HIP graph and replayed K times (a serving loop's
    # form: one launch of the whole step); every replay must reproduce the eager outputs bit for bit
    ref_y = [bufs[i]["y"].clone() for i in range(len(layers))]
    g_step = graph_of(torch, composite)
    s3, e3 = ev_t(), ev_t()
    s3.record()
    for _ in range(K):
        g_step.replay()
    e3.record()
    torch.cuda.synchronize()
    ms_step_graph = s3.elapsed_time(e3) / K
    graph_equal = all(torch.equal(bufs[i]["y"], ref_y[i]) for i in range(len(layers)))
    del g_step, ref_y

    # ------------------------------------------------------------ accounting
    int_ops = adapter_flops = alg_bytes = 0.0
    per_linear, per_group = [], []
    gpu_routes = []
    ops_lin = []
    for i, (spec, layer) in enumerate(layers):
        e_host = bufs[i]["e"].cpu().numpy()
        gpu_routes.append(e_host)
        n_distinct = int(np.unique(e_host).size)
        im, am, ab = libqe.qe_linear_cost(layer.lin, T, n_distinct, 2)
        int_ops += 2 * im
        adapter_flops += 2 * am
        alg_bytes += ab
        ops_lin.append(2 * im)
        per_linear.append(dict(name=spec.name, d_in=spec.d_in, d_out=spec.d_out,
                               expert_histogram=np.bincount(e_host, minlength=cfg.n_routed).tolist()))
    for k, g in enumerate(groups):
        ops = sum(ops_lin[i] for i in g)
        per_group.append(dict(linears=",".join(layers[i][0].name for i in g),
                              gemm_us=round(float(gemm_ms[:, k].mean()) * 1e3, 2),
                              gemm_tops=round(ops / (gemm_ms[:, k].mean() * 1e-3) / 1e12, 1)))
    # every group's main products run as one launch of the grouped GEMM kernel (128-token tiles)
    big_ops = sum(ops_lin)
    big_ms = float(gemm_ms.sum(axis=1).mean())  # per step
    achieved = big_ops / (big_ms * 1e-3) / 1e12
    big = groups
    t_roof = max(int_ops / (PEAK_INT8_TOPS * 1e12) + adapter_flops / (PEAK_BF16_TFLOPS * 1e12),
                 alg_bytes / (PEAK_HBM_GBS * 1e9))
    traffic = load_traffic(None)

    result = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "qwen2vl_72b layer linears (q,k,v,o,gate,up,down), W4A6 prefill, T=4096, "
                        "shared rank 32, 8 routed experts rank 32, router d_in x 8",
            "T": T, "w_bits": 4, "a_bits": 6, "r_shared": 32, "n_routed": 8, "r_routed": 32,
        },
        "step_ms": {"median": round(float(np.median(step_ms)), 4), "p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4),
                    "cold_median": round(float(np.median(cold)), 4),
                    "cold_p10": round(float(np.percentile(cold, 10)), 4),
                    "cold_p90": round(float(np.percentile(cold, 90)), 4), "cold_steps": len(cold),
                    "note": "per-step HIP events over the K timed steps (warm: inputs and weights as the previous "
                            "step left the caches); cold: the Infinity Cache flushed by reading 1 GiB before each "
                            "step"},
        "roofline": {
            "scope": "dominant kernel only: the main GEMM's launches (one per group of linears that read the same "
                     "input: q+k+v, o, gate+up, down); the whole step is in layer_roofline",
            "kernel": "gemm_w4_group_kernel (int8 MFMA main GEMM, 128-token tiles, fused dequant/SE/RE epilogue)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_INT8_TOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": traffic,
            "launches_per_step": len(big),
            "avg_launch_us": round(big_ms / len(big) * 1e3, 2),
            "ops_per_launch": round(big_ops / len(big)),
        },
        "layer_roofline": {
            "t_roof_ms": round(t_roof * 1e3, 4),
            "frac": round(t_roof / (ms_step * 1e-3), 4),
            "int_tops": round(int_ops / 1e12, 3), "adapter_tflop": round(adapter_flops / 1e12, 4),
            "alg_gbytes": round(alg_bytes / 1e9, 3),
        },
        "breakdown": {"gemm_ms_per_step": round(gemm_ms_step, 4),
                      "prologue_ms_per_step": round(ms_step - gemm_ms_step, 4),
                      "ms_per_step_composite_entry": round(ms_step_fwd, 4),
                      "ms_per_step_composite_graph": round(ms_step_graph, 4),
                      "graph_replays_bit_equal": bool(graph_equal),
                      "wall_s_timed_region": round(wall, 3),
                      "per_group": per_group, "per_linear": per_linear},
    }

    peaks = measured_peaks(torch, libqe, dev)
    result["measured_peaks"] = peaks

    if not args.no_extras:
        result["extras"] = extras(torch, synth, qe, libqe, dev, peaks)

    if want_cpu:
        result["cpu_baseline"] = cpu_baseline(torch, cfg, xs_cpu, host_params, gpu_routes, args.cpu_sample_tokens,
                                              args.cpu_sample_tokens_1t)

    print(json.dumps(result), flush=True)


def measured_peaks(torch, libqe, dev):
    """Rates this device sustains, from the library's probe kernels timed with events on the
    stream they run on: an int8 MFMA loop (the main GEMM's instruction, 2048 workgroups, about
    25 ms) on small constant operands, the highest rate the power-limited matrix cores sustain,
    and on operands in the main GEMM's value ranges; the same for the bf16 MFMA (the weight-only
    GEMM's instruction); and a 1 GiB streaming copy.  Median of five runs each."""
    def median_ms(fn, reps=5):
        fn()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    blocks, iters = 2048, 30000
    sink = torch.empty(blocks * 256 * 4, dtype=torch.int32, device=dev)
    rates = []
    for operands in (0, 1):
        ops = libqe.qe_probe_mfma_i8(sink, blocks, iters, operands)
        t = median_ms(lambda: libqe.qe_probe_mfma_i8(sink, blocks, iters, operands))
        rates.append(ops / (t * 1e-3) / 1e12)
    sink_f = torch.empty(blocks * 256 * 4, dtype=torch.float32, device=dev)
    for operands in (0, 1):
        flops = libqe.qe_probe_mfma_bf16(sink_f, blocks, iters, operands)
        t = median_ms(lambda: libqe.qe_probe_mfma_bf16(sink_f, blocks, iters, operands))
        rates.append(flops / (t * 1e-3) / 1e12)
    del sink_f
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t_copy = median_ms(lambda: libqe.qe_probe_copy(src, dst, nbytes))
    del sink, src, dst
    torch.cuda.empty_cache()
    return {"int8_mfma_tops": round(rates[0], 1),
            "int8_mfma_tops_gemm_operands": round(rates[1], 1),
            "bf16_mfma_tflops": round(rates[2], 1),
            "bf16_mfma_tflops_gemm_operands": round(rates[3], 1),
            "copy_gbs": round(2 * nbytes / (t_copy * 1e-3) / 1e9, 1),
            "method": "qe_probe_mfma_i8 (2048 workgroups x 4 waves x 240000 MFMA 16x16x64 i8; small "
                      "constant operands, then operands in the A6 x W4 code ranges), qe_probe_mfma_bf16 (the same "
                      "on MFMA 16x16x32 bf16; operands in the A16 x W3 ranges) and qe_probe_copy "
                      "(1 GiB read + 1 GiB write), median of 5"}


def graph_of(torch, fn):
    """fn (launches only: no allocation, copy or synchronization inside) captured once in a HIP
    graph after warm-up calls on a side stream; returns the graph, replayed by the caller."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def layer_throughput(torch, synth, qe, libqe, dev, name, steps=10):
    """The composite entry point over every linear of a configuration, one stream, inputs resident:
    tokens/s, the int8 rate of the whole step and its fraction of the spec roofline."""
    cfg = synth.get_config(name)
    T = cfg.T
    xs = {s: synth.gen_activations(cfg, s).to(dev) for s in cfg.streams()}
    layers = []
    for spec in cfg.linears:
        params = synth.gen_linear(cfg, spec)
        layers.append((spec, qe.QELinear.from_params(params, cfg.w_bits, cfg.a_bits, device=dev)))
        del params
    wss = [torch.empty(max(libqe.qe_workspace_bytes(l.lin, T), 256), dtype=torch.uint8, device=dev) for _, l in layers]
    ys = [torch.empty(T, spec.d_out, dtype=torch.float32, device=dev) for spec, _ in layers]
    es = [torch.empty(T, dtype=torch.int32, device=dev) for _ in layers]
    groups = []  # consecutive linears that read the same input share one route pass
    for i, (spec, _) in enumerate(layers):
        if groups and layers[groups[-1][0]][0].stream == spec.stream:
            groups[-1].append(i)
        else:
            groups.append([i])

    def run():
        for g in groups:
            libqe.qe_group_forward([layers[i][1].lin for i in g], xs[layers[g[0]][0].stream], [ys[i] for i in g],
                                   [es[i] for i in g], [wss[i] for i in g])

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        run()
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / steps * 1e-3
    ref_y = [y.clone() for y in ys]
    g = graph_of(torch, run)  # the same step as one HIP graph, replayed
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    t_graph = a.elapsed_time(b) / steps * 1e-3
    graph_equal = all(torch.equal(y, r) for y, r in zip(ys, ref_y))
    del g, ref_y
    int_ops = adapter_flops = alg = 0.0
    for i, (spec, layer) in enumerate(layers):
        im, am, ab = libqe.qe_linear_cost(layer.lin, T, int(torch.unique(es[i]).numel()), 2)
        int_ops, adapter_flops, alg = int_ops + 2 * im, adapter_flops + 2 * am, alg + ab
    t_roof = max(int_ops / (PEAK_INT8_TOPS * 1e12) + adapter_flops / (PEAK_BF16_TFLOPS * 1e12),
                 alg / (PEAK_HBM_GBS * 1e9))
    del layers, wss, xs, ys, es
    torch.cuda.empty_cache()
    return {"linears": [f"{s.name} {s.d_in}->{s.d_out}" for s in cfg.linears], "T": T,
            "w_bits": cfg.w_bits, "a_bits": cfg.a_bits, "us_per_step": round(t * 1e6, 2),
            "us_per_step_graph": round(t_graph * 1e6, 2), "graph_replays_bit_equal": bool(graph_equal),
            "tokens_per_s": round(T / t, 1), "int8_tops": round(int_ops / t / 1e12, 1),
            "layer_roofline_frac": round(t_roof / t, 4)}


TABLE8_NPU = {(3584, 3584): {"W4A6": 3.56, "W4A8": 3.50, "W3A16": 4.10},
              (3584, 18944): {"W4A6": 3.60, "W4A8": 3.59, "W3A16": 4.50},
              (18944, 3584): {"W4A6": 3.84, "W4A8": 3.77, "W3A16": 4.50}}


def table8(torch, synth, qe, libqe, dev, reps=20):
    """The listing's Table 8 workload on this GPU: each Qwen2VL-7B linear shape at s = 128 as a
    QE linear (W4A6, W4A8, W3A16: the composite entry point, inputs resident) against the same
    linear in bf16 through torch (hipBLASLt), warm.  The pages' column is an analytical NPU
    model's speedup over fp16, given for context."""
    import dataclasses

    def med_us(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)) * 1e3

    base = synth.get_config("qwen2vl_7b_s128")
    rows = []
    for spec in base.linears:
        x = synth.gen_activations(base, spec.stream).to(dev)
        W = None
        for wb, ab in ((4, 6), (4, 8), (3, 16)):
            cfg = dataclasses.replace(base, w_bits=wb, a_bits=ab)
            params = synth.gen_linear(cfg, spec)
            if W is None:
                W = torch.from_numpy(params["W_f"]).to(torch.bfloat16).to(dev)
                xb = x.to(torch.bfloat16)
                t_bf16 = med_us(lambda: torch.nn.functional.linear(xb, W))
            layer = qe.QELinear.from_params(params, wb, ab, device=dev)
            del params
            ws = layer.workspace(base.T)
            y = torch.empty(base.T, spec.d_out, dtype=torch.float32, device=dev)
            t_qe = med_us(lambda: libqe.qe_linear_forward(layer.lin, x, y, None, ws))
            key = f"W{wb}A{ab}"
            bf16_roof_us = max(2.0 * spec.d_in * spec.d_out / (PEAK_HBM_GBS * 1e3),
                               2.0 * base.T * spec.d_in * spec.d_out / (PEAK_BF16_TFLOPS * 1e6))
            rows.append({"shape": f"{spec.d_in}x{spec.d_out}", "bits": key, "qe_us": round(t_qe, 2),
                         "bf16_torch_us": round(t_bf16, 2), "speedup_vs_bf16": round(t_bf16 / t_qe, 3),
                         "bf16_roofline_us": round(bf16_roof_us, 2),
                         "speedup_vs_bf16_roofline": round(bf16_roof_us / t_qe, 3),
                         "npu_speedup_pages": TABLE8_NPU[(spec.d_in, spec.d_out)][key]})
            del layer, ws, y
        del W, x
        torch.cuda.empty_cache()
    return {"T": base.T, "rows": rows,
            "note": "bf16_roofline_us = max(bf16 weight bytes / 8 TB/s, flops / 2.5 PFLOP/s)"}


def decode_line(torch, synth, qe, libqe, dev, w_bits, a_bits, copy_gbs=None, y_bf16=False):
    """Qwen2VL-72B MLP up + down at T = 8 through the composite entry point, cold (the Infinity
    Cache flushed before every iteration) and warm; y float32, or bf16 with y_bf16."""
    import dataclasses
    cfg = dataclasses.replace(synth.get_config("qwen2vl_72b_decode"), w_bits=w_bits, a_bits=a_bits)
    layers = []
    for spec in cfg.linears:
        params = synth.gen_linear(cfg, spec)
        layers.append((spec, qe.QELinear.from_params(params, cfg.w_bits, cfg.a_bits, device=dev)))
        del params
    xs = {s: synth.gen_activations(cfg, s).to(dev) for s in cfg.streams()}
    T = cfg.T
    wss = [l.workspace(T) for _, l in layers]
    for _, l in layers:
        l.lin.y_dtype = libqe.QE_BF16 if y_bf16 else libqe.QE_F32
    ydt = torch.bfloat16 if y_bf16 else torch.float32
    ys = [torch.empty(T, s.d_out, dtype=ydt, device=dev) for s, _ in layers]
    es = [torch.empty(T, dtype=torch.int32, device=dev) for _ in layers]
    # Reading 1 GiB (four times the 256 MB Infinity Cache) evicts it with clean lines; a write
    # flush would leave dirty lines whose write-back lands inside the timed region.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def run():
        for i, (spec, layer) in enumerate(layers):
            libqe.qe_linear_forward(layer.lin, xs[spec.stream], ys[i], es[i], wss[i])

    for _ in range(3):
        run()
    cold, warm = [], []
    for it in range(30):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    for it in range(30):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        warm.append(a.elapsed_time(b))
    alg = 0.0
    for i, (spec, layer) in enumerate(layers):
        nd = int(torch.unique(es[i]).numel())
        alg += libqe.qe_linear_cost(layer.lin, T, nd, 2)[2]
    # the read-only streaming rate of the same byte count, cold: the measured counterpart of a
    # path whose traffic is almost all weight reads
    nb = int(alg) // 16 * 16
    buf = torch.ones(nb // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(libqe.qe_probe_read_sink_bytes() // 4, dtype=torch.int32, device=dev)
    reads = []
    for it in range(10):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        libqe.qe_probe_read(buf, nb, sink)
        b.record()
        torch.cuda.synchronize()
        reads.append(a.elapsed_time(b))
    read_gbs = nb / (float(np.median(reads)) * 1e-3) / 1e9
    del buf, sink
    t_cold = float(np.median(cold)) * 1e-3
    res = {
        "us_cold_median": round(t_cold * 1e6, 2), "us_cold_p10": round(float(np.percentile(cold, 10)) * 1e3, 2),
        "us_cold_p90": round(float(np.percentile(cold, 90)) * 1e3, 2),
        "us_warm_median": round(float(np.median(warm)) * 1e3, 2),
        "tokens_per_s": round(T / t_cold, 1), "alg_mbytes": round(alg / 1e6, 2),
        "achieved_gbs": round(alg / t_cold / 1e9, 1), "hbm_frac": round(alg / t_cold / 1e9 / PEAK_HBM_GBS, 4),
        "read_probe_gbs_same_bytes_cold": round(read_gbs, 1),
        "frac_of_measured_read": round(alg / t_cold / 1e9 / read_gbs, 4),
        "hbm_frac_of_measured_copy": round(alg / t_cold / 1e9 / copy_gbs, 4) if copy_gbs else None,
        "note": "Infinity Cache flushed by reading 1 GiB before every cold iteration; hbm_frac is against the "
                "8 TB/s spec, frac_of_measured_read against qe_probe_read streaming the same number of bytes "
                "cold, hbm_frac_of_measured_copy against a 1 GiB read + write copy",
    }
    del layers, wss, flush
    torch.cuda.empty_cache()
    return res


def sweeps(torch, synth, qe, libqe, dev, reps=10):
    """Variants the pages study: the number of routed experts N_r (Table 6: 2, 4, 8, 16) on the
    Qwen2VL-72B q projection (8192 -> 8192, W4A6, T = 4096, the composite entry point), with
    top-2 routing at N_r = 8, and the top-k size k of the calibration statistic on the
    InternVL2-8B down input (T = 4096)."""
    import dataclasses

    def med_us(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)) * 1e3

    out = {"n_routed_qwen2vl72b_q_w4a6_T4096": [], "topk_k_internvl2_8b_down_T4096": []}
    base = synth.get_config("qwen2vl_72b")
    spec = next(l for l in base.linears if l.name == "q")
    x = synth.gen_activations(base, spec.stream).to(dev)
    for n_r in (2, 4, 8, 16):
        cfg = dataclasses.replace(base, n_routed=n_r)
        layer = qe.QELinear.from_params(synth.gen_linear(cfg, spec), cfg.w_bits, cfg.a_bits, device=dev)
        ws = layer.workspace(base.T)
        y = torch.empty(base.T, spec.d_out, dtype=torch.float32, device=dev)
        t = med_us(lambda: libqe.qe_linear_forward(layer.lin, x, y, None, ws))
        row = {"n_routed": n_r, "us": round(t, 2), "tokens_per_s": round(base.T / t * 1e6, 1)}
        if n_r == 8:  # top-2 routing on the same linear: both routed corrections in the GEMM epilogue
            ws2 = torch.empty(libqe.qe_top2_workspace_bytes(layer.lin, base.T), dtype=torch.uint8, device=dev)
            t2 = med_us(lambda: libqe.qe_linear_forward_top2(layer.lin, x, y, None, None, ws2))
            row.update(top2_us=round(t2, 2), top2_tokens_per_s=round(base.T / t2 * 1e6, 1))
            del ws2
        out["n_routed_qwen2vl72b_q_w4a6_T4096"].append(row)
        del layer, ws, y
    del x
    cfg = synth.get_config("internvl2_8b")
    spec = next(l for l in cfg.linears if l.name == "down")
    x = synth.gen_activations(cfg, spec.stream).to(dev)
    w = torch.rand(spec.d_in, dtype=torch.float32, device=dev) + 0.5
    hist = torch.zeros(spec.d_in, dtype=torch.int32, device=dev)
    for k in (4, 8, 16, 32, 64):
        topk = torch.empty(cfg.T, k, dtype=torch.int32, device=dev)
        t = med_us(lambda: libqe.qe_channel_topk(x, w, k, topk, hist))
        out["topk_k_internvl2_8b_down_T4096"].append({"k": k, "us": round(t, 2)})
    torch.cuda.empty_cache()
    return out


def prefill_w3a16(torch, synth, qe, libqe, dev, bf16_measured, reps=5):
    """Weight-only prefill: the Qwen2VL-72B MLP up and down projections at W3A16 over the 4096
    prefill tokens (the pages' weight-only setting), composite entry point, inputs resident;
    rates against the bf16 spec peak and the rate the bf16 MFMA probe sustains on operands in
    this GEMM's ranges."""
    import dataclasses
    base = synth.get_config("qwen2vl_72b")
    cfg = dataclasses.replace(synth.get_config("qwen2vl_72b_decode"), T=base.T)
    rows, total = [], 0.0
    for spec in cfg.linears:
        x = synth.gen_activations(base, spec.stream).to(dev)
        layer = qe.QELinear.from_params(synth.gen_linear(cfg, spec), 3, 16, device=dev)
        ws = layer.workspace(base.T)
        y = torch.empty(base.T, spec.d_out, dtype=torch.float32, device=dev)
        for _ in range(2):
            libqe.qe_linear_forward(layer.lin, x, y, None, ws)
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            libqe.qe_linear_forward(layer.lin, x, y, None, ws)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        t = float(np.median(ts)) * 1e-3
        flops = 2.0 * base.T * spec.d_in * spec.d_out
        rows.append({"linear": f"{spec.name} {spec.d_in}->{spec.d_out}", "us": round(t * 1e6, 1),
                     "bf16_tflops": round(flops / t / 1e12, 1),
                     "frac_of_bf16_peak": round(flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "frac_of_bf16_measured": round(flops / t / 1e12 / bf16_measured, 4)})
        total += t
        del layer, ws, y, x
        torch.cuda.empty_cache()
    return {"T": base.T, "rows": rows, "tokens_per_s_up_down": round(base.T / total, 1)}


def extras(torch, synth, qe, libqe, dev, peaks):
    out = {}
    copy_gbs = peaks["copy_gbs"]
    out["prefill_qwen2vl72b_up_down_w3a16_T4096"] = prefill_w3a16(torch, synth, qe, libqe, dev,
                                                                   peaks["bf16_mfma_tflops_gemm_operands"])
    out["sweeps"] = sweeps(torch, synth, qe, libqe, dev)
    out["table8_qwen2vl7b_s128"] = table8(torch, synth, qe, libqe, dev)
    # ---- the other configurations: a small single linear (latency), a 2B layer, an 8B layer
    out["linear_tiny_w4a8_T64"] = layer_throughput(torch, synth, qe, libqe, dev, "tiny", steps=50)
    out["layer_qwen2vl2b_w4a6_T2048"] = layer_throughput(torch, synth, qe, libqe, dev, "qwen2vl_2b")
    out["layer_internvl2_8b_w4a8_T4096"] = layer_throughput(torch, synth, qe, libqe, dev, "internvl2_8b")
    # ---- decode: Qwen2VL-72B MLP up/down, T=8 (HBM-bound weight streaming): W3A16 (the
    # configuration's own), and W4A6 (quantized activations: few-token split-K main product)
    out["decode_qwen2vl72b_up_down_w3a16_T8"] = decode_line(torch, synth, qe, libqe, dev, 3, 16, copy_gbs)
    out["decode_qwen2vl72b_up_down_w4a6_T8"] = decode_line(torch, synth, qe, libqe, dev, 4, 6, copy_gbs)
    out["decode_qwen2vl72b_up_down_w3a16_T8_bf16y"] = decode_line(torch, synth, qe, libqe, dev, 3, 16, copy_gbs,
                                                                  y_bf16=True)
    out["decode_qwen2vl72b_up_down_w4a6_T8_bf16y"] = decode_line(torch, synth, qe, libqe, dev, 4, 6, copy_gbs,
                                                                 y_bf16=True)

    # ---- calibration statistic: InternVL2-8B down input, k = 32 (HBM / ALU bound)
    cfg = synth.get_config("internvl2_8b")
    spec = next(l for l in cfg.linears if l.name == "down")
    lp = synth.gen_linear(cfg, spec)
    W = torch.from_numpy(lp["W_f"]).to(dev)
    w = torch.empty(spec.d_in, dtype=torch.float32, device=dev)
    libqe.qe_colmean_abs(W, w)
    x = synth.gen_activations(cfg, spec.stream).to(dev)
    hist = torch.zeros(spec.d_in, dtype=torch.int32, device=dev)
    topk = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device=dev)
    for _ in range(3):
        libqe.qe_channel_topk(x, w, cfg.k, topk, hist)
    ts = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        libqe.qe_channel_topk(x, w, cfg.k, topk, hist)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    t = float(np.median(ts)) * 1e-3
    nbytes = x.numel() * 2 + spec.d_in * 4 * 2 + cfg.T * cfg.k * 4
    out["topk_internvl2_8b_down_T4096_k32"] = {
        "us_median": round(t * 1e6, 2), "tokens_per_s": round(cfg.T / t, 1),
        "achieved_gbs": round(nbytes / t / 1e9, 1), "hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)}

    # ---- the rest of the statistic on the same top-k lists: frequency partition (host),
    # co-occurrence counts of the N_r * k token-dependent channels (GPU), NPMI spectral
    # clustering (host); the 65536-token line repeats the 4096 tokens sixteen times
    n_r = cfg.n_routed
    hist.zero_()
    libqe.qe_channel_topk(x, w, cfg.k, topk, hist)
    h = hist.cpu().numpy().view(np.uint32)
    t0 = time.perf_counter()
    _, dep, slot = libqe.qe_partition_channels(h, cfg.k, n_r)
    t_part = time.perf_counter() - t0
    slot_d = torch.from_numpy(slot).to(dev)
    n_dep = len(dep)
    cooc = torch.zeros(n_dep, n_dep, dtype=torch.int32, device=dev)
    cws = torch.empty(libqe.qe_cooccur_workspace_bytes(16 * cfg.T, n_dep), dtype=torch.uint8, device=dev)
    for T_c, tk in ((cfg.T, topk), (16 * cfg.T, topk.repeat(16, 1).contiguous())):
        for _ in range(3):
            libqe.qe_cooccur(tk, slot_d, n_dep, cooc, cws)
        ts = []
        for _ in range(20):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            libqe.qe_cooccur(tk, slot_d, n_dep, cooc, cws)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        t = float(np.median(ts)) * 1e-3
        nbytes = T_c * cfg.k * 4 + spec.d_in * 4 + 2 * n_dep * n_dep * 4
        out[f"cooccur_internvl2_8b_down_T{T_c}_k{cfg.k}_C{n_dep}"] = {
            "us_median": round(t * 1e6, 2), "tokens_per_s": round(T_c / t, 1),
            "achieved_gbs": round(nbytes / t / 1e9, 1), "hbm_frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)}
    cooc.zero_()
    libqe.qe_cooccur(topk, slot_d, n_dep, cooc, cws)
    c = cooc.cpu().numpy().view(np.uint32)
    t0 = time.perf_counter()
    labels = libqe.qe_cluster_channels(c, cfg.T, n_r, 0.2)
    t_clu = time.perf_counter() - t0
    out["partition_cluster_host_internvl2_8b_down"] = {
        "partition_ms": round(t_part * 1e3, 3), "cluster_ms": round(t_clu * 1e3, 2), "channels": n_dep,
        "cluster_sizes": np.bincount(labels, minlength=n_r).tolist(), "note": "host C++, one thread"}

    # ---- expert construction on the same linear and clusters: whitening weights from the
    # calibration tokens, then the SE (rank 32) and the 8 REs (rank 32 each) from the weight
    # quantization error by randomized truncated SVD (k = 40 columns, 2 power iterations)
    W_f = W
    s_d = torch.from_numpy(lp["s"]).to(dev)
    r_s = r_r = 32
    k_sv, q_it = 40, 2
    cr = torch.empty(spec.d_in, device=dev)
    rws = torch.empty(libqe.qe_channel_rms_workspace_bytes(cfg.T, spec.d_in), dtype=torch.uint8, device=dev)
    gen = torch.Generator(device=dev).manual_seed(1)
    omegas = torch.randn(1 + n_r, spec.d_out, k_sv, device=dev, generator=gen)
    bws = torch.empty(libqe.qe_build_experts_workspace_bytes(spec.d_out, spec.d_in, k_sv, 32), dtype=torch.uint8,
                      device=dev)
    ts, tr = [], []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        libqe.qe_channel_rms(x, cr, rws)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ex = libqe.qe_build_experts(W_f, s_d, cfg.w_bits, cr, dep, labels, n_r, r_s, r_r, omegas, q_it, bws)
        ts.append(time.perf_counter() - t1)
        tr.append(t1 - t0)
    # the default construction: covariance whitening over the same calibration tokens (passes over E
    # and over a float32 copy of x; test matrices [1 + N_r][T][k])
    om_c = torch.randn(1 + n_r, cfg.T, k_sv, device=dev, generator=torch.Generator(device=dev).manual_seed(2))
    cws = torch.empty(libqe.qe_build_experts_cov_workspace_bytes(spec.d_out, spec.d_in, cfg.T, k_sv, 32),
                      dtype=torch.uint8, device=dev)
    tc = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        exc = libqe.qe_build_experts_cov(W_f, s_d, cfg.w_bits, x, dep, labels, n_r, r_s, r_r, om_c, q_it, cws)
        tc.append(time.perf_counter() - t0)
    del cws, om_c
    out["expert_build_cov_internvl2_8b_down"] = {
        "d_in": spec.d_in, "d_out": spec.d_out, "calibration_tokens": cfg.T, "r_shared": r_s, "n_routed": n_r,
        "r_routed": r_r, "k_columns": k_sv, "power_iters": q_it, "build_ms": round(float(np.median(tc)) * 1e3, 1),
        "passes_per_fit": {"E": 2 * q_it + 2, "X": 2 * q_it + 2},
        "sigma_shared_top": [round(float(v), 3) for v in exc["sigma_s"][:4]],
        "note": "covariance whitening (the default reading): the SE and each RE minimize the residual times the "
                "calibration tokens; randomized subspace iteration on E X^T by passes over E and a float32 copy of x"}
    # router: targets on the calibration tokens from the residual after the SE, then the ridge fit
    E1 = torch.empty(spec.d_out, spec.d_in, device=dev)
    libqe.qe_quant_error(W_f, s_d, cfg.w_bits, E1)
    libqe.qe_sub_lowrank(E1, torch.from_numpy(ex["A_s"]).to(dev), torch.from_numpy(ex["B_s"]).to(dev))
    A_r = torch.from_numpy(ex["A_r"]).to(dev)
    B_r = torch.from_numpy(ex["B_r"]).to(dev)
    tgt = torch.empty(cfg.T, n_r, device=dev)
    tws = torch.empty(libqe.qe_router_targets_workspace_bytes(spec.d_out, spec.d_in, n_r, r_r), dtype=torch.uint8,
                      device=dev)
    fws = torch.empty(libqe.qe_router_fit_workspace_bytes(cfg.T, spec.d_in, n_r), dtype=torch.uint8, device=dev)
    t_tg, t_fit = [], []
    for _ in range(2):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        libqe.qe_router_targets(E1, x, A_r, B_r, tgt, tws)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        R_fit, iters = libqe.qe_router_fit(x, tgt, 1e-2, 500, 1e-5, fws)
        t_fit.append(time.perf_counter() - t1)
        t_tg.append(t1 - t0)
    pred = (x.float() @ torch.from_numpy(R_fit).to(dev)).argmin(1)
    agree = float((pred == tgt.argmin(1)).float().mean())
    del E1, A_r, B_r, fws, tws
    fits = 1 + n_r
    out["expert_build_internvl2_8b_down"] = {
        "d_in": spec.d_in, "d_out": spec.d_out, "w_bits": cfg.w_bits, "r_shared": r_s, "n_routed": n_r,
        "r_routed": r_r, "k_columns": k_sv, "power_iters": q_it,
        "channel_rms_ms": round(float(np.median(tr)) * 1e3, 3), "build_ms": round(float(np.median(ts)) * 1e3, 1),
        "ms_per_fit": round(float(np.median(ts)) * 1e3 / fits, 1),
        "passes_over_E_per_fit": 2 * q_it + 2,
        "router_targets_ms": round(float(np.median(t_tg)) * 1e3, 1),
        "router_fit_ms": round(float(np.median(t_fit)) * 1e3, 1), "router_fit_cg_iters": iters,
        "router_ridge": 1e-2, "router_argmin_agreement_on_calibration": round(agree, 4),
        "sigma_shared_top": [round(float(v), 5) for v in ex["sigma_s"][:4]],
        "note": "wall clock of the synchronous entry point: GPU passes over E (float32), Gram matrices (float64) "
                "and k x k products on the GPU, k x k eigenproblems on the host between them"}
    return out


def cpu_baseline(torch, cfg, xs_cpu, host_params, gpu_routes, n_tok, n_tok_1t):
    """The plain C oracle (OpenMP over tokens) as it stands, on a bounded sample of the same
    workload: n_tok of the T tokens through all seven linears on every host thread, and n_tok_1t
    tokens on one thread (its weight quantization is done beforehand and not timed, as the GPU's
    weight packing is not).  The numpy oracle is timed on the same sample beside it.  The
    oracle's router also runs on all T tokens of every linear: near-tie tokens (the two smallest
    scores closer than 1e-4 of their magnitude) are counted, and so are tokens whose GPU route
    differs from the oracle's (allowed only at near-ties)."""
    from oracle import qe_oracle as O
    from oracle import qe_ref as C
    rng = np.random.default_rng(7)
    toks = np.sort(rng.choice(cfg.T, n_tok, replace=False))
    f32 = lambda t: None if t is None else t.float().numpy()
    n_all = C.num_threads()
    t_all = t_one = t_np = 0.0
    routes = []
    for li, (spec, params) in enumerate(zip(cfg.linears, host_params)):
        qw, s_w = C.quant_weights(params["W_f"], params["s"], cfg.w_bits)
        del params["W_f"]
        ad = dict(A_s=f32(params["A_s"]), B_s=f32(params["B_s"]), A_r=f32(params["A_r"]), B_r=f32(params["B_r"]),
                  R=f32(params["R"]))
        x_all = xs_cpu[spec.stream].float().numpy()
        x = x_all[toks]
        C.set_threads(n_all)
        t0 = time.perf_counter()
        C.qe_linear(x, True, params["s"], qw, s_w, cfg.a_bits, **ad)
        t_all += time.perf_counter() - t0
        C.set_threads(1)
        t0 = time.perf_counter()
        C.qe_linear(x[:n_tok_1t], True, params["s"], qw, s_w, cfg.a_bits, **ad)
        t_one += time.perf_counter() - t0
        C.set_threads(n_all)
        t0 = time.perf_counter()
        O.qe_linear(x, True, params["s"], qw, s_w, cfg.a_bits, **ad)
        t_np += time.perf_counter() - t0
        r = C.route(x_all, ad["R"])
        near = r["margin"] < 1e-4 * r["margin_scale"]
        differ = gpu_routes[li] != r["expert"]
        routes.append({"linear": spec.name, "near_tie_tokens": int(near.sum()), "routes_differing": int(differ.sum()),
                       "routes_differing_away_from_near_ties": int((differ & ~near).sum()),
                       "oracle_expert_histogram": np.bincount(r["expert"], minlength=cfg.n_routed).tolist()})
        log(f"oracle {spec.name}: all-core {t_all:.2f}s cumulative; routes {routes[-1]}")
        del qw, x_all
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), "unknown")
    except OSError:  # pragma: no cover
        model = "unknown"
    return {"value": round(n_tok / t_all, 2), "unit": "tokens/s", "cores": int(n_all), "kind": "oracle",
            "sample": f"{n_tok} of {cfg.T} tokens through all 7 linears of the same layer on {n_all} threads "
                      f"({t_all:.1f} s of oracle time); weight quantization untimed",
            "implementation": "plain C oracle (oracle/qe_ref.c: loops in index order, int64 / double sums, "
                              "gcc -O3 -march=x86-64-v3 -fopenmp over tokens)",
            "cpu_model": model,
            "one_thread": {"value": round(n_tok_1t / t_one, 3), "unit": "tokens/s",
                           "sample": f"{n_tok_1t} tokens through all 7 linears ({t_one:.1f} s)"},
            "numpy_oracle": {"value": round(n_tok / t_np, 2), "unit": "tokens/s",
                             "sample": f"the same {n_tok} tokens ({t_np:.1f} s; BLAS float64 products)"},
            "routing_vs_oracle_all_tokens": routes}


if __name__ == "__main__":
    main()
