#!/usr/bin/env python3
"""Benchmark of the bitmap SpMM hot path on one MI355X.

A step is one call of usw_spmm on the OPT-13B FFN-up layer (M=20480,
K=5120, 50% magnitude pruning, N=16 activations): it streams the encoded
weight (bitmaps, offsets, values) and X from HBM, rebuilds the tiles and
writes Y.  The weight is encoded once (offline, not timed) and copied into
enough independent device buffers (>= 5, > 512 MB in total) that the timed
loop, which rotates through them, reads from HBM rather than from the 256 MB
Infinity Cache.

Prints one JSON line: effective TFLOP/s (2*M*K*N per step) with the GB/s of
algorithmic traffic (bitmaps + offsets + values + X + Y), the kernel's
roofline fraction against 8 TB/s, a dense fp16 torch.matmul of the same
shape under the same rotation, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import hashlib

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBPS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "effective TFLOP/s + HBM GB/s, bitmap SpMM M=20480 K=5120 s=50% N=16"


def algorithmic_bytes(M, K, N, nnz, ngt, value_bytes=2.0, y_bytes=2, scales=False):
    """Bytes read and written once: bitmaps, offsets, values, (scales), X, Y."""
    b = 8 * (M * K // 64) + 4 * (ngt + 1) + value_bytes * nnz + 2 * N * K + y_bytes * N * M
    if scales:
        b += 2 * M
    return b


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-dense", action="store_true", help="skip the dense fp16 baseline")
    p.add_argument("--splits", type=int, default=0)
    p.add_argument("--M", type=int, default=20480)
    p.add_argument("--K", type=int, default=5120)
    p.add_argument("--N", type=int, default=16)
    p.add_argument("--sparsity", type=float, default=0.5)
    p.add_argument("--dtype", default="f16", choices=["f16", "i4", "i2"],
                   help="value type: fp16, INT4, or 2-bit (union format only)")
    p.add_argument("--format", default="tca", choices=["tca", "union", "cbc", "encode", "encode_union", "encode_cbc"],
                   help="tca: TCA-BME bitmaps (usw_spmm); union: IE-BME union-mask INT4 or 2-bit, LT shape and"
                        " area grid from --lt and --areas (usw_union_spmm; fp16 becomes INT4); cbc: Tiled-CBC spMspV with dynamic pruning"
                        " (usw_cbc_spmspv; implies --N 1 and fp16); encode: the on-device TCA-BME encoder"
                        " (usw_encode_device_index + usw_encode_device_values) of the weight, not the SpMM;"
                        " encode_union: the on-device IE-BME encoder, INT4 or 2-bit (64x64 LTs, 2x2 areas); encode_cbc: the"
                        " on-device Tiled-CBC encoder")
    p.add_argument("--lt", type=int, default=64, choices=[64, 32, 16],
                   help="union: LT height (LTs of 64, 32 or 16 rows by 64 columns)")
    p.add_argument("--areas", default="2x2",
                   help="union: the R_A x C_A area grid of an LT, e.g. 2x2, 4x1, 1x8")
    p.add_argument("--reorder", action="store_true",
                   help="union with --lt 16: bitmap-aware row reordering of every LT before encoding"
                        " (usw_union_reorder, then usw_union_encode_reordered)")
    p.add_argument("--dp", type=float, default=0.5,
                   help="cbc: fraction of activations below the pruning threshold (tau is that quantile of |x|)")
    p.add_argument("--cpu-reps", type=int, default=5)
    p.add_argument("--rotation", type=int, default=0,
                   help="number of encoded copies the steps rotate over (default: enough for > 512 MB, so reads come"
                        " from HBM; 1 keeps a layer resident in the 256 MB Infinity Cache, which is not the"
                        " measured configuration)")
    p.add_argument("--eager", action="store_true",
                   help="launch each timed step from Python with its own pair of HIP events instead of replaying"
                        " the steps from a HIP graph")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain device copy of known size (for scaling the FETCH_SIZE and WRITE_SIZE counters)")
    return p.parse_args()


# Sources that make up each kernel: a measured traffic figure is only used
# while they are unchanged.
KERNEL_SOURCES = {
    "decode": ["unstructured_sparse_weight_amd/csrc/usw_spmm.hip", "unstructured_sparse_weight_amd/csrc/usw_decode_common.h",
               "unstructured_sparse_weight_amd/csrc/usw_device.h"],
    "union": ["unstructured_sparse_weight_amd/csrc/usw_union.hip", "unstructured_sparse_weight_amd/csrc/usw_decode_common.h",
              "unstructured_sparse_weight_amd/csrc/usw_device.h"],
    "cbc": ["unstructured_sparse_weight_amd/csrc/usw_cbc.hip", "unstructured_sparse_weight_amd/csrc/usw_device.h"],
    "prefill": ["unstructured_sparse_weight_amd/csrc/usw_prefill.hip", "unstructured_sparse_weight_amd/csrc/usw_device.h"],
}


def kernel_hash(kind):
    """Hash of the kernel's code: its sources without // comments and blank
    lines, so that comment edits do not invalidate a measurement."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(name, kind):
    """HBM bytes per launch from profiles/traffic_<name>.md (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's readings), or None when there is no
    such summary or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sources_sha256_16") != kernel_hash(kind):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def format_stats(h, M, K, kept, union, cbc):
    """Storage figures of the encoding: compression ratio (dense fp16 bytes
    over stored bytes), payload-to-metadata ratio (value bytes over index
    bytes) and the realized sparsity of the mask."""
    if cbc:
        index = h.bitmaps.nbytes + h.tile_offsets.nbytes + h.colinfo.nbytes
        payload = 2 * h.nnz_padded
    else:
        index = h.bitmaps.nbytes + h.offsets.nbytes + (h.rowmap.nbytes if union and h.rowmap is not None else 0)
        payload = h.values_bytes + (h.scales.nbytes if h.scales is not None else 0)
    return {"cr": round(2.0 * M * K / (index + payload), 4), "pmr": round(payload / index, 4),
            "realized_sparsity": round(1.0 - kept / (M * K), 6), "stored_bytes": int(index + payload)}


def probe_same_bytes(L, nbytes, dev, stream, steps):
    """Per-launch time of the library's streaming-read probe over nbytes,
    timed as the SpMM is: a HIP graph of `steps` launches, each on the next
    of enough buffers (> 768 MB together) that reads come from HBM, one
    untimed replay, then HIP events around one replay."""
    import torch
    nb = (int(nbytes) + 15) // 16 * 16
    R = max(2, -(-(768 << 20) // nb))
    bufs = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(R)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    cap = torch.cuda.Stream(dev)
    cap_sp = ctypes.c_void_p(cap.cuda_stream)
    for b in bufs:
        if L.usw_probe_read(b.data_ptr(), nb, sink.data_ptr(), cap_sp) != 0:
            raise RuntimeError("usw_probe_read failed")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for i in range(steps):
            L.usw_probe_read(bufs[i % R].data_ptr(), nb, sink.data_ptr(), cap_sp)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del graph, bufs, sink
    return us


def calibrate_copy(args):
    """A plain copy of 1 GiB (read 1 GiB, write 1 GiB), rotating over two
    buffer pairs so that it streams from HBM."""
    import torch
    n = 1 << 30
    dev = torch.device("cuda:0")
    bufs = [(torch.ones(n, dtype=torch.uint8, device=dev), torch.empty(n, dtype=torch.uint8, device=dev))
            for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        src, dst = bufs[i % 2]
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "launches": args.steps}), flush=True)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path shards without communication along M); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import unstructured_sparse_weight_amd as usw
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args)
        return
    if args.format in ("encode", "encode_union", "encode_cbc"):
        encode_bench(args)
        return
    dev = torch.device("cuda:0")
    union = args.format == "union"
    cbc = args.format == "cbc"
    if union and args.dtype not in ("i4", "i2"):
        args.dtype = "i4"
    if not union and args.dtype == "i2":
        raise SystemExit("2-bit values exist in the union format only (--format union --dtype i2)")
    try:
        areas = tuple(int(v) for v in args.areas.lower().split("x"))
        assert len(areas) == 2
    except (ValueError, AssertionError):
        raise SystemExit("--areas takes R_AxC_A, e.g. 2x2 or 4x1")
    if cbc:
        args.dtype, args.N = "f16", 1
    M, K, N, s = args.M, args.K, args.N, args.sparsity
    # Kernel family as usw_spmm picks it: fp16 with more than 128 tokens runs
    # the prefill kernels, everything else the decode kernels (in passes of
    # up to 64 tokens).  The synthetic inputs follow the prefill workload's
    # recipe from 33 tokens on.
    prefill = args.dtype == "f16" and N > 128
    layer_id = {(20480, 5120): 2, (11008, 4096): 0, (4096, 11008): 1}.get((M, K), 0)
    cfg_id = 5 if args.dtype in ("i4", "i2") else (4 if N > 32 else 2)

    log(f"[bench] generating W {M}x{K} (magnitude pruning s={s}) and X [{N}][{K}]")
    W, mask, X = wl.config_case(cfg_id, M, K, N, s, layer_id=layer_id)
    t = time.time()
    tau = 0.0
    if cbc:
        h = usw.cbc_encode_host(W, mask)
        xa = np.abs(X[0].astype(np.float32))
        tau = float(np.quantile(xa, args.dp)) if args.dp > 0 else 0.0
        active = xa >= np.float32(tau)
        log(f"[bench] host Tiled-CBC encode {time.time() - t:.2f} s, nnz={h.nnz} padded={h.nnz_padded};"
            f" tau={tau:.4f} keeps {int(active.sum())} of {K} columns")
        # Per GTile: tile offset and 16 ColInfo words; per active column:
        # its 4 bitmap words and its padded run; x and y once.
        runs = ((h.colinfo & 0xFFFF).astype(np.int64) + 7) // 8 * 8
        act_cols = np.tile(active.reshape(-1, 16), (M // 256, 1)).reshape(-1)
        alg = (h.tile_offsets.nbytes + h.colinfo.nbytes + 2 * K + 2 * M
               + int((32 + 2 * runs[act_cols]).sum()))
    elif union:
        lt = (args.lt, 64)
        perms = None
        if args.reorder:
            if args.lt != 16:
                raise SystemExit("--reorder needs --lt 16 (the solver takes LTs of at most 20 rows)")
            perms, before, after = usw.union_reorder(W, mask, lt, areas)
            log(f"[bench] row reordering {time.time() - t:.2f} s: active union entries {int(before.sum())}"
                f" -> {int(after.sum())} ({100.0 * (1 - after.sum() / max(before.sum(), 1)):.2f}% fewer)")
            t = time.time()
        h = usw.union_encode_host(W, mask, lt, areas, args.dtype, perm=perms)
        kept = int(mask.sum())
        log(f"[bench] host union encode {time.time() - t:.2f} s, payload={h.payload} for nnz={kept}"
            f" ({h.payload / max(kept, 1):.3f} stored per kept weight)")
        # Union words, offsets, INT4 payload, scales, row maps, X and Y, each
        # moved once.
        alg = (h.bitmaps.nbytes + h.offsets.nbytes + h.values_bytes + 2 * M + 2 * N * K + 2 * N * M
               + (h.rowmap.nbytes if h.rowmap is not None else 0))
    else:
        h = usw.encode_host(W, mask, (64, 64), args.dtype)
        log(f"[bench] host encode {time.time() - t:.2f} s, nnz={h.nnz}")
        ngt = (M // 64) * (K // 64)
        vbytes = 2.0 if args.dtype == "f16" else 0.5
        alg = algorithmic_bytes(M, K, N, h.nnz, ngt, vbytes, 2, args.dtype == "i4")
    enc_bytes = h.bitmaps.nbytes + (h.tile_offsets.nbytes + h.colinfo.nbytes if cbc else h.offsets.nbytes) + h.values.nbytes
    R = args.rotation if args.rotation > 0 else max(5, math.ceil(600e6 / enc_bytes))
    to_dev = usw.cbc_to_device if cbc else (usw.union_to_device if union else usw.to_device)
    encs = [to_dev(h, dev) for _ in range(R)]
    xs = [torch.from_numpy(X).to(dev) for _ in range(R)]
    ys = [torch.empty((N, M), dtype=torch.float16, device=dev) for _ in range(R)]

    L = usw.lib()
    fmts = [e.fmt() for e in encs]
    if cbc:
        wsb = usw.cbc_workspace_bytes(encs[0], args.splits)[0]
    elif union:
        wsb = usw.union_workspace_bytes(encs[0], N, args.splits)[0]
    else:
        wsb = usw.spmm_workspace_bytes(encs[0], N, args.splits)
    ws = torch.zeros(max(wsb, 256), dtype=torch.uint8, device=dev)   # counter region starts at zero
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(i, on=sp):
        j = i % R
        if cbc:
            st = L.usw_cbc_spmspv(ctypes.byref(fmts[j]), xs[j].data_ptr(), ys[j].data_ptr(), 1, tau, args.splits,
                                  ws.data_ptr(), wsb, on)
        elif union:
            st = L.usw_union_spmm(ctypes.byref(fmts[j]), xs[j].data_ptr(), ys[j].data_ptr(), 1, N, args.splits,
                                  ws.data_ptr(), wsb, on)
        else:
            st = L.usw_spmm_ex(ctypes.byref(fmts[j]), xs[j].data_ptr(), ys[j].data_ptr(), 1, N, args.splits,
                               ws.data_ptr(), wsb, on)
        if st != 0:
            raise RuntimeError(f"spmm failed: {st}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    if args.eager:
        # Timed region: K steps launched one by one from Python, bracketed by
        # device synchronisation; a pair of HIP events on the launch stream
        # around each launch (these include any wait for the host's launch).
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(args.warmup + i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kern_ms = [a.elapsed_time(b) for a, b in ev]
        kern_avg_ms = float(np.mean(kern_ms))
        kern_med_ms = float(np.median(kern_ms))
    else:
        # The K timed steps are captured once in a HIP graph (each a usw_spmm
        # launch on the next rotated copy; the library allocates and clears
        # nothing, so the graph holds exactly the K kernels).  Timed region:
        # one replay on the launch stream, bracketed by device
        # synchronisation and a pair of HIP events, so the host's launch cost
        # does not leave the GPU idle between steps.  The graph is replayed
        # once untimed first.
        cap = torch.cuda.Stream(dev)
        cap_sp = ctypes.c_void_p(cap.cuda_stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                step(args.warmup + i, cap_sp)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kern_avg_ms = e0.elapsed_time(e1) / args.steps
        kern_med_ms = kern_avg_ms
    ms_step = (t1 - t0) * 1e3 / args.steps

    # Streaming-read ceiling: the library's plain read kernel over 1 GiB
    # (more than the 256 MB Infinity Cache), same stream, HIP events.
    probe = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 12, dtype=torch.int32, device=dev)
    for _ in range(3):
        L.usw_probe_read(probe.data_ptr(), probe.numel(), sink.data_ptr(), sp)
    pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a_, b_ in pe:
        a_.record(stream)
        st = L.usw_probe_read(probe.data_ptr(), probe.numel(), sink.data_ptr(), sp)
        b_.record(stream)
        if st != 0:
            raise RuntimeError(f"usw_probe_read failed: {st}")
    torch.cuda.synchronize()
    stream_gbps = probe.numel() / (float(np.median([a_.elapsed_time(b_) for a_, b_ in pe])) * 1e-3) / 1e9
    del probe, sink
    same_us = probe_same_bytes(L, alg, dev, stream, args.steps) if not args.eager else None

    flops = 2.0 * M * K * N
    value = flops / (ms_step * 1e-3) / 1e12
    gbps_step = alg / (ms_step * 1e-3) / 1e9
    achieved = alg / (kern_avg_ms * 1e-3) / 1e9
    log(f"[bench] step {ms_step * 1e3:.2f} us, kernel avg {kern_avg_ms * 1e3:.2f} us (median {kern_med_ms * 1e3:.2f}),"
        f" {achieved:.0f} GB/s algorithmic, {flops / (kern_avg_ms * 1e-3) / 1e12:.1f} eff TFLOP/s;"
        f" streaming-read ceiling {stream_gbps:.0f} GB/s"
        + (f"; a plain read of the same {alg / 1e6:.1f} MB: {same_us:.2f} us" if same_us else ""))

    # Dense fp16 baseline of the same shape and rotation (hipBLASLt through
    # torch.matmul); its output also serves as a sanity check of the timed
    # sparse result (the oracle comparison proper lives in the tests).
    dense = None
    if not args.no_dense and args.dtype == "f16":
        Wd = np.where(mask, W, np.float16(0))
        dense = [torch.from_numpy(Wd).to(dev) for _ in range(max(3, math.ceil(600e6 / Wd.nbytes)))]
        Rd = len(dense)
        yd = torch.empty((N, M), dtype=torch.float16, device=dev)
        for i in range(10):
            torch.matmul(xs[i % R], dense[i % Rd].t(), out=yd)
        torch.cuda.synchronize()
        evd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
        for i in range(50):
            evd[i][0].record(stream)
            torch.matmul(xs[i % R], dense[i % Rd].t(), out=yd)
            evd[i][1].record(stream)
        torch.cuda.synchronize()
        dms = float(np.mean([a.elapsed_time(b) for a, b in evd]))
        dbytes = 2 * M * K + 2 * N * K + 2 * N * M
        yref = (xs[0].float() @ dense[0].float().t())
        err = float((ys[0].float() - yref).abs().max() / (yref.abs().max() + 1e-30))
        dense = {"kernel_avg_us": round(dms * 1e3, 2), "eff_tflops": round(flops / (dms * 1e-3) / 1e12, 2),
                 "gbps": round(dbytes / (dms * 1e-3) / 1e9, 1), "hbm_frac": round(dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                 "speedup_sparse_vs_dense": round(dms / kern_avg_ms, 3), "max_rel_dev_vs_fp32": err}
        log(f"[bench] dense fp16 torch.matmul {dms * 1e3:.2f} us ({dense['gbps']} GB/s); sparse/dense speedup {dense['speedup_sparse_vs_dense']}")

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(W, mask, X, M, K, N, args.dtype, args.cpu_reps, union, cbc, tau,
                           lt=(args.lt, 64), perms=perms if union else None, areas=areas)

    if cbc:
        kname = "cbc_spmspv_kernel"
    elif union:
        if areas != (2, 2) or args.lt == 32 or (args.lt == 64 and args.reorder):
            kname = "union_grid_decode_kernel"
        else:
            kname = "union16_decode_kernel" if args.lt == 16 else "union_decode_kernel"
    elif prefill:
        kname = "prefill_ws_kernel" if N > 256 else "prefill_kernel"
    else:
        # fp16 values at most 55% dense with N <= 16 take the workgroup-
        # cooperative kernel, the rest the per-wave one.
        if args.dtype == "f16" and N <= 16 and s >= 0.45:
            kname = "decode_ring_kernel"
        else:
            kname = "decode_f16_kernel" if args.dtype == "f16" else "decode_i4_kernel"
    if prefill:
        # Compute-bound: the matrix cores run the dense 64x64 tiles rebuilt
        # from the bitmaps, 2*M*K*N flops per launch.
        tf = flops / (kern_avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tf, 1), "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4), "traffic": None, "kernel": kname,
                    "kernel_avg_us": round(kern_avg_ms * 1e3, 3), "alg_flops_per_launch": int(flops),
                    "alg_bytes_per_launch": int(alg)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": kname,
                    "kernel_avg_us": round(kern_avg_ms * 1e3, 3), "alg_bytes_per_launch": int(alg),
                    "streaming_read_ceiling": round(stream_gbps, 1),
                    "frac_of_streaming_ceiling": round(achieved / stream_gbps, 4),
                    "plain_read_same_bytes_us": round(same_us, 3) if same_us else None}
    if (M, K) == (20480, 5120):
        workload = f"opt13b_ffn_up_{M}x{K}_s{s}_N{N}"
        if union:
            # the union layouts and payloads are separate measurements
            workload += (f"_{args.dtype}" if args.dtype != "i4" else "") + (f"_lt{args.lt}" if args.lt != 64 else "") + \
                (f"_a{areas[0]}x{areas[1]}" if areas != (2, 2) else "") + ("_reordered" if args.reorder else "")
    elif prefill and (M, K) in ((11008, 4096), (4096, 11008)):
        workload = f"llama7b_prefill_{M}x{K}_s{s}_N{N}"
    else:
        workload = f"spmm_{M}x{K}_s{s}_N{N}"
    if args.splits == 0:
        roofline["traffic"] = measured_traffic(f"{kname}_{workload}" + (f"_dp{args.dp}" if cbc else ""),
                                               "cbc" if cbc else ("union" if union else
                                                                  ("prefill" if prefill else "decode")))
    roofline["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    out = {
        "metric": METRIC if (M, K, N, s, args.dtype) == (20480, 5120, 16, 0.5, "f16") else
        f"effective TFLOP/s + HBM GB/s, bitmap SpMM M={M} K={K} s={int(s * 100)}% N={N} {args.dtype}",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded N(0,0.02) weights, magnitude pruning, N(0,1) activations)",
        "config": {"workload": workload,
                   "format": "tiled_cbc_spmspv" if cbc else (
                       (f"ie_bme_union_{areas[0]}x{areas[1]}_lt{args.lt}" + ("_reordered" if args.reorder else "")) if union
                       else "tca_bme"),
                   "M": M, "K": K, "N": N, "sparsity": s, "values": args.dtype,
                   **({"localTile": f"{args.lt}x64", "areas": f"{areas[0]}x{areas[1]}"} if union
                      else {"gTile": "256x16"} if cbc else {"groupTile": "64x64"}),
                   "rotation_copies": R, "splits": args.splits or "auto",
                   "launch": "eager" if args.eager else "hip_graph"},
        "gbps": round(gbps_step, 1),
        "hbm_frac": round(gbps_step / HBM_PEAK_GBPS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense_fp16": dense,
        "nnz": int(mask.sum()) if union else int(h.nnz),
    }
    if union:
        out["union_payload"] = int(h.payload)
        out["union_encoded_bytes"] = int(h.bitmaps.nbytes + h.offsets.nbytes + h.values_bytes + 2 * M
                                         + (h.rowmap.nbytes if h.rowmap is not None else 0))
    if cbc:
        out["config"]["dynamic_sparsity"] = args.dp
        out["config"]["tau"] = tau
    out["format_stats"] = format_stats(h, M, K, int(mask.sum()), union, cbc)
    print(json.dumps(out), flush=True)


def encode_bench(args):
    """Throughput of an on-device encoder on one layer (default FFN-up
    20480 x 5120, 50% magnitude pruning, with a mask): TCA-BME (--format
    encode) or IE-BME INT4 with 64x64 LTs and 2x2 areas (--format
    encode_union).  A step is one *_encode_device_index call (bitmaps or
    union words, counts, scan, INT4 scales) and one *_encode_device_values
    call, given the NNZ (payload) that an untimed first run read back (the
    work per step is the same).  Algorithmic bytes: W and the
    mask read once, bitmaps, offsets, values and scales written once.  W and
    mask rotate over copies of more than 512 MB in total so that reads come
    from HBM."""
    import torch
    import unstructured_sparse_weight_amd as usw
    import workloads as wl
    import oracle.tca_bme as ob

    dev = torch.device("cuda:0")
    M, K, s = args.M, args.K, args.sparsity
    union = args.format == "encode_union"
    cbc = args.format == "encode_cbc"
    if union and args.dtype not in ("i4", "i2"):
        args.dtype = "i4"
    if not union and args.dtype == "i2":
        raise SystemExit("2-bit values exist in the union format only (--format encode_union --dtype i2)")
    if cbc:
        args.dtype = "f16"
    vt = {"f16": usw.USW_VAL_F16, "i4": usw.USW_VAL_I4, "i2": usw.USW_VAL_I2}[args.dtype]
    W, mask, _ = wl.config_case(2 if args.dtype == "f16" else 5, M, K, 1, s, layer_id=2)
    in_bytes = W.nbytes + mask.nbytes
    R = args.rotation if args.rotation > 0 else max(2, math.ceil(600e6 / in_bytes))
    Ws = [torch.from_numpy(W).to(dev) for _ in range(R)]
    ms = [torch.from_numpy(mask.view(np.uint8)).to(dev) for _ in range(R)]
    if union:
        enc_fn = lambda w, m: usw.union_encode_device(w, m, (64, 64), (2, 2), args.dtype)  # noqa: E731
    elif cbc:
        enc_fn = lambda w, m: usw.cbc_encode_device(w, m)  # noqa: E731
    else:
        enc_fn = lambda w, m: usw.encode_device(w, m, (64, 64), args.dtype)  # noqa: E731
    first = enc_fn(Ws[0], ms[0])
    torch.cuda.synchronize()
    nnz = first.payload if union else (first.nnz_padded if cbc else first.nnz)
    ngt = (M // 256) * (K // 16) if cbc else (M // 64) * (K // 64)
    outs = [enc_fn(Ws[0], ms[0]) for _ in range(R)]
    L = usw.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step(i, ev=None):
        j = i % R
        o = outs[j]
        sc = o.scales.data_ptr() if getattr(o, "scales", None) is not None else None
        if ev:
            ev[0].record(stream)
        if cbc:
            st = L.usw_cbc_encode_device_index(Ws[j].data_ptr(), ms[j].data_ptr(), M, K, o.bitmaps.data_ptr(),
                                               o.tile_offsets.data_ptr(), o.colinfo.data_ptr(), sp)
        elif union:
            geo = (M, K, 64, 64, 2, 2, vt)
            st = L.usw_union_encode_device_index(Ws[j].data_ptr(), ms[j].data_ptr(), *geo, o.bitmaps.data_ptr(),
                                                 o.offsets.data_ptr(), sc, sp)
        else:
            st = L.usw_encode_device_index(Ws[j].data_ptr(), ms[j].data_ptr(), M, K, 64, 64, vt,
                                           o.bitmaps.data_ptr(), o.offsets.data_ptr(), sc, sp)
        if ev:
            ev[1].record(stream)
        if cbc:
            st = st or L.usw_cbc_encode_device_values(Ws[j].data_ptr(), M, K, o.bitmaps.data_ptr(),
                                                      o.tile_offsets.data_ptr(), o.colinfo.data_ptr(), nnz,
                                                      o.values.data_ptr(), o.values.numel() * 2, sp)
        elif union:
            st = st or L.usw_union_encode_device_values(Ws[j].data_ptr(), ms[j].data_ptr(), *geo, o.bitmaps.data_ptr(),
                                                        o.offsets.data_ptr(), sc, nnz, o.values.data_ptr(),
                                                        o.values.numel(), sp)
        else:
            st = st or L.usw_encode_device_values(Ws[j].data_ptr(), M, K, 64, 64, vt, o.bitmaps.data_ptr(),
                                                  o.offsets.data_ptr(), sc, nnz, o.values.data_ptr(),
                                                  o.values.numel(), sp)
        if ev:
            ev[2].record(stream)
        if st != 0:
            raise RuntimeError(f"device encode failed: {st}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    idx_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    val_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_step = (t1 - t0) * 1e3 / args.steps
    offs_of = (lambda e: e.tile_offsets) if cbc else (lambda e: e.offsets)  # noqa: E731
    for o in outs:      # every rotated copy holds the same encoding as the first
        if not (torch.equal(o.bitmaps, first.bitmaps) and torch.equal(offs_of(o), offs_of(first))
                and torch.equal(o.values, first.values)):
            raise RuntimeError("device encode is not deterministic")
    vbytes = 2 * nnz if args.dtype == "f16" else (nnz + 1) // 2 if args.dtype == "i4" else (nnz + 3) // 4
    words = first.bitmaps.numel() * 8
    out_bytes = words + 4 * (ngt + 1) + vbytes + (2 * M if args.dtype != "f16" else 0) + (64 * ngt if cbc else 0)
    alg = in_bytes + out_bytes
    enc_ms = idx_ms + val_ms
    achieved = alg / (enc_ms * 1e-3) / 1e9
    log(f"[bench] device encode: index pass {idx_ms * 1e3:.1f} us, values pass {val_ms * 1e3:.1f} us,"
        f" {achieved:.0f} GB/s algorithmic; step {ms_step * 1e3:.1f} us")

    # Host encoder (the library's multithreaded C++) and the oracle encoder,
    # each on the whole layer once, for context.
    import oracle.ie_bme as ou
    t = time.perf_counter()
    if union:
        usw.union_encode_host(W, mask, (64, 64), (2, 2), args.dtype)
    elif cbc:
        usw.cbc_encode_host(W, mask)
    else:
        usw.encode_host(W, mask, (64, 64), args.dtype)
    host_s = time.perf_counter() - t
    cpu = None
    if not args.no_cpu:
        t = time.perf_counter()
        if union:
            ou.encode_union(W, mask, 64, 64, 2, 2, ob.VAL_I4 if args.dtype == "i4" else ob.VAL_I2)
        elif cbc:
            import oracle.tiled_cbc as oc
            oc.encode_cbc(W, mask)
        else:
            (ob.encode if args.dtype == "f16" else ob.encode_i4)(W, mask)
        oracle_s = time.perf_counter() - t
        cpu = {"value": round(alg / oracle_s / 1e9, 3), "unit": "GB/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "sample": f"whole layer {M}x{K}: oracle encoder once ({oracle_s:.1f} s)",
               "seconds_per_step": round(oracle_s, 3)}
    fmt_name = "ie_bme_union_2x2" if union else ("tiled_cbc" if cbc else "tca_bme")
    workload = f"encode_{fmt_name}_{M}x{K}_s{s}_{args.dtype}"
    out = {
        "metric": f"device encode GB/s (algorithmic), {fmt_name} M={M} K={K} s={int(s * 100)}% {args.dtype}",
        "value": round(achieved, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded N(0,0.02) weights, magnitude pruning)",
        "config": {"workload": workload, "format": fmt_name, "M": M, "K": K, "sparsity": s, "values": args.dtype,
                   "tile": "256x16" if cbc else "64x64", "rotation_copies": R, "launch": "eager"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "encode (index + scan + scales, then values)",
                     "index_call_avg_us": round(idx_ms * 1e3, 2), "values_call_avg_us": round(val_ms * 1e3, 2),
                     "alg_bytes_per_launch": int(alg)},
        "cpu_baseline": cpu,
        "host_encoder_seconds": round(host_s, 3),
        "nnz": int(nnz),
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(W, mask, X, M, K, N, dtype, reps, union=False, cbc=False, tau=0.0, lt=(64, 64), perms=None,
                 areas=(2, 2)):
    """The oracle as it stands (decode + fp64 product) on the host cores."""
    import oracle.tca_bme as ob
    import oracle.ie_bme as ou
    import oracle.tiled_cbc as oc
    t = time.perf_counter()
    if cbc:
        enc = oc.encode_cbc(W, mask)
        product = lambda e, Xm: oc.spmspv(e, Xm[0], tau)  # noqa: E731
    elif union:
        vt = ob.VAL_I2 if dtype == "i2" else ob.VAL_I4
        if perms is not None:
            enc = ou.encode_union_reordered(W, mask, perms, lt[0], lt[1], areas[0], areas[1], vt)
        else:
            enc = ou.encode_union(W, mask, lt[0], lt[1], areas[0], areas[1], vt)
        product = ou.spmm_union
    else:
        enc = ob.encode(W, mask) if dtype == "f16" else ob.encode_i4(W, mask)
        product = ob.spmm
    t_enc = time.perf_counter() - t
    times = []
    for _ in range(reps):
        t = time.perf_counter()
        Y = product(enc, X)
        times.append(time.perf_counter() - t)
        del Y
    best = min(times)
    # One more run with the BLAS pool held to a single thread.
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t = time.perf_counter()
            Y = product(enc, X)
            single = time.perf_counter() - t
            del Y
    except ImportError:
        pass
    cores = len(os.sched_getaffinity(0))
    threads = os.environ.get("OMP_NUM_THREADS")
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(2.0 * M * K * N / best / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "blas_threads": int(threads) if threads and threads.isdigit() else cores, "kind": "oracle",
            "sample": f"whole layer {M}x{K}, N={N}: decode + fp64 matmul, best of {reps} ({sum(times):.1f} s total);"
                      f" oracle encode {t_enc:.1f} s excluded",
            "seconds_per_step": round(best, 3),
            "single_thread_seconds_per_step": round(single, 3) if single is not None else None,
            "cpu_model": model}


if __name__ == "__main__":
    main()
