#!/usr/bin/env python3
"""Benchmark of the N:M hot path on one MI355X.

One step = the whole path over one batch of synthetic input: for each weight
matrix of the workload, nm_mask, nm_compress (mask + values + metadata),
nm_decompress and nm_spmm (Y = W_sparse X).  Inputs are resident in HBM before
the timed region.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload llama_mlp]

`value` is the whole step's effective throughput: dense-equivalent product
flops (2 R K T per matrix) divided by the step time.  Per-kernel figures,
the roofline of the dominant kernel, the dense GEMM on the same shapes and the
CPU oracle timed on the host are reported alongside.

The SR-STE passes of a training step on the same weights (nm_prune, the
forward's masked weight, and nm_srste_grad, the backward's gradient) are timed
in a separate pass after the step, each launch after a cache-clearing fill, and
reported under "srste" with their HBM roofline; they are not part of `value`.
So is the transposable-mask path under "transposable": nm_tprune (greedy
transposable mask applied), nm_compress_t (the compressed transpose) and the
backward product W^T dY through nm_spmm; and one round of the channel-
permutation search (nm_perm_gains) under "permutation".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "2:4 spmm effective TFLOP/s + mask/compress GB/s (% of MI355X roofline)"
METRIC_I8 = "2:4 int8 spmm effective TOP/s + mask/compress GB/s (% of MI355X roofline)"
METRIC_FP8 = "2:4 fp8 spmm effective TFLOP/s + mask/compress GB/s (% of MI355X roofline)"
PEAK_HBM_GBS = 8000.0
# fp32 VALU operations: the 157.3 TFLOP/s fp32 vector peak counts an FMA as two flops,
# i.e. 256 CUs x 128 fp32 lanes per clock x 2.4 GHz = 78.6 T operations per second
PEAK_VALU_TOPS = 78.64
# dense matrix-core peaks (TFLOP/s; TOP/s for int8)
PEAK_MFMA_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3, "i8": 5033.2, "fp8": 5033.2}
# workload name -> (synthetic matrices, N:M pattern)
WORKLOADS = {
    "llama_mlp": (["llama_up", "llama_down"], (2, 4)),
    "llama_mlp_i8": (["llama_up_i8", "llama_down_i8"], (2, 4)),
    "llama_mlp_fp8": (["llama_up_fp8", "llama_down_fp8"], (2, 4)),
    "bert_ffn": (["bert_ffn"], (2, 4)),
    "resnet_conv3x3": (["resnet_conv3x3"], (2, 4)),
    "sweep_f16_2_4": (["sweep_f16"], (2, 4)),
    "sweep_f16_1_2": (["sweep_f16"], (1, 2)),
    "sweep_f16_4_8": (["sweep_f16"], (4, 8)),
    "toy_f32": (["toy_f32"], (2, 4)),
    "sweep_f32_2_4": (["sweep_f32"], (2, 4)),
}


def meta_bits(m: int) -> int:
    return {2: 1, 4: 2, 8: 3}[m]


def algorithmic_bytes(R, K, T, n, m, s, ys):
    """Bytes each kernel must move at minimum (one read of inputs, one write of outputs):
    elements of s bytes, products of ys bytes (int32 for int8, bf16 for fp8)."""
    e = R * K
    kept = e * n // m
    meta = R * ((K // m * n * meta_bits(m) + 31) // 32) * 4
    return {
        "mask_compress": e * s + e + kept * s + meta,  # one pass: W in; mask, values, meta out
        "mask": e * s + e,
        "compress": e * s + kept * s + meta,
        "decompress": kept * s + meta + e * s,
        "spmm": kept * s + meta + K * T * s + R * T * ys,
    }


def profiled_traffic(workload: str, kernel: str = "spmm_kernel", source: str = "nm_spmm.hip"):
    """HBM bytes per dispatch of the kernels whose name contains `kernel`, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy-kernel calibration),
    or None when that summary is missing or was taken on a different version of `source`."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    src = os.path.join(ROOT, "masking_sparse_gemm_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != prof.get("sources_sha256", {}).get(source):
            return None
    per = [v["read_bytes"] + v["write_bytes"] for k, v in prof["per_dispatch_bytes"].items()
           if kernel in k]
    return sum(per) / len(per) if per else None


def srste_cpu_sample(mats, n, m, budget_s: float = 3.0):
    """The oracle's SR-STE forward weight + gradient on leading rows of each matrix,
    one thread, for about budget_s seconds: elements per second."""
    import oracle

    oracle.lib()
    done, elems = {}, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        progressed = False
        for w in mats:
            r0 = done.get(w["name"], 0)
            r1 = min(w["R"], r0 + 64)
            if r1 <= r0:
                continue
            Wsl, Gsl = np.ascontiguousarray(w["W"][r0:r1]), np.ascontiguousarray(w["G"][r0:r1])
            oracle.prune(Wsl, w["dtype"], n, m)
            oracle.srste_grad(Wsl, Gsl, w["dtype"], n, m, 2e-4)
            done[w["name"]] = r1
            elems += (r1 - r0) * w["K"]
            progressed = True
        if not progressed:
            break
    dt = time.perf_counter() - t0
    return {"value": round(elems / dt / 1e6, 2), "unit": "Melem/s (forward weight + gradient)",
            "cores": 1, "kind": "oracle", "seconds": round(dt, 2),
            "sample": ", ".join(f"{k}: rows 0..{v}" for k, v in done.items())}


def cpu_baseline(mats, n, m, threads: int, budget_s: float = 12.0):
    """The oracle as it stands, on the host: mask + compress + decompress + product of a
    bounded slice of rows of every matrix, rows spread over `threads` threads."""
    import oracle

    oracle.lib()
    F = 0.0
    rows_done = {}
    t0 = time.perf_counter()
    block = 4  # rows per thread per round
    rounds = 0
    while True:
        for w in mats:
            r0 = rows_done.get(w["name"], 0)
            r1 = min(w["R"], r0 + block * threads)
            if r1 <= r0:
                continue
            Wsl = np.ascontiguousarray(w["W"][r0:r1])
            R = r1 - r0

            def work(k, Wsl=Wsl, R=R, w=w):
                a = k * R // threads
                b = (k + 1) * R // threads
                if b <= a:
                    return
                part = np.ascontiguousarray(Wsl[a:b])
                oracle.mask(part, w["dtype"], n, m)
                vals, meta = oracle.compress(part, w["dtype"], n, m)
                oracle.decompress(vals, meta, w["dtype"], b - a, w["K"], n, m)
                Y = np.empty((b - a, w["T"]), dtype=np.float64)
                oracle.spmm_rows(vals, meta, b - a, w["K"], n, m, w["X"], w["dtype"], 0, b - a, Y)

            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(work, range(threads)))
            rows_done[w["name"]] = r1
            F += 2.0 * R * w["K"] * w["T"]
        rounds += 1
        if time.perf_counter() - t0 >= budget_s or all(rows_done.get(w["name"], 0) >= w["R"]
                                                       for w in mats):
            break
    dt = time.perf_counter() - t0
    sample = ", ".join(f"{k}: rows 0..{v} of {next(w['R'] for w in mats if w['name'] == k)}"
                       for k, v in rows_done.items())
    unit = "TOP/s" if mats[0]["dtype"] == "i8" else "TFLOP/s"
    return {"value": F / dt / 1e12, "unit": unit, "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"mask+compress+decompress+product of {sample} (fp64 product, all T columns)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama_mlp", choices=sorted(WORKLOADS))
    ap.add_argument("--layout", default="blocked", choices=["blocked", "rows"],
                    help="storage layout of the compressed weight (include/nm.h)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense GEMM baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one 512 MiB device-to-device copy (a kernel of known traffic "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the kernels shard by rows of W with no exchange, but bench.py measures one GPU)",
              file=sys.stderr)
        return 2

    import torch

    import masking_sparse_gemm_amd as nm
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    names, (n, m) = WORKLOADS[args.workload]

    # ---- inputs, resident in HBM before timing ----
    mats = []
    for name in names:
        w = synth.WORKLOADS[name]
        W, X = w.W(), w.X()
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32,
               "i8": torch.int8, "fp8": torch.float8_e4m3fn}[w.dtype]
        # int8 products are exact int32; fp8 products are written as bf16
        ydt = {"i8": torch.int32, "fp8": torch.bfloat16}.get(w.dtype, tdt)

        def to_dev(a, tdt=tdt):
            if a.dtype in (np.float32, np.int8):
                return torch.from_numpy(a).to(dev)
            if a.dtype == np.uint8:  # fp8 codes
                return torch.from_numpy(a).to(dev).view(tdt)
            return torch.from_numpy(a.view(np.int16)).view(tdt).to(dev)

        s = {"f32": 4, "i8": 1, "fp8": 1}.get(w.dtype, 2)
        ys = {"i8": 4, "fp8": 2}.get(w.dtype, s)
        # the SR-STE gradient (16/32-bit float weights only)
        G = w.G() if w.dtype in ("f32", "f16", "bf16") else W
        d = dict(name=name, R=w.R, K=w.K, T=w.T, dtype=w.dtype, s=s, ys=ys, W=W, X=X, G=G,
                 Wd=to_dev(W), Xd=to_dev(X), Gd=to_dev(G))
        vshape, mshape = nm.compressed_shapes(w.R, w.K, n, m, args.layout)
        d["vals"] = torch.empty(vshape, dtype=tdt, device=dev)
        d["meta"] = torch.empty(mshape, dtype=torch.int32, device=dev)
        d["mask"] = torch.empty((w.R, w.K), dtype=torch.bool, device=dev)
        d["dec"] = torch.empty((w.R, w.K), dtype=tdt, device=dev)
        d["Y"] = torch.empty((w.R, w.T), dtype=ydt, device=dev)
        d["pruned"] = torch.empty((w.R, w.K), dtype=tdt, device=dev)
        d["grad"] = torch.empty((w.R, w.K), dtype=tdt, device=dev)
        # transposable-mask path: pruned weight, compressed transpose, backward product
        d["tpruned"] = torch.empty((w.R, w.K), dtype=tdt, device=dev)
        vts, mts = nm.compressed_shapes(w.K, w.R, n, m, args.layout)
        d["vals_t"] = torch.empty(vts, dtype=tdt, device=dev)
        d["meta_t"] = torch.empty(mts, dtype=torch.int32, device=dev)
        d["dX"] = torch.empty((w.K, w.T), dtype=ydt, device=dev)
        mats.append(d)
    dtype = mats[0]["dtype"]
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    L = nm.lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    DT = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3, "fp8": 5}[dtype]
    YDT = {"i8": 4, "fp8": 2}.get(dtype, DT)  # int32 for int8, bf16 for fp8
    # SR-STE and transposable masks train 16/32-bit float weights
    float_path = dtype in ("f32", "f16", "bf16")
    LAY = nm.LAYOUTS[args.layout]
    # the step: mask and compressed pair from one pass over W, decompress, product
    kinds = ["mask_compress", "decompress", "spmm"]

    def launch(d, kind):
        if kind == "mask_compress":
            rc = L.nm_mask_compress(d["Wd"].data_ptr(), DT, d["R"], d["K"], n, m, LAY,
                                    d["mask"].data_ptr(), d["vals"].data_ptr(),
                                    d["meta"].data_ptr(), sp)
        elif kind == "mask":
            rc = L.nm_mask(d["Wd"].data_ptr(), DT, d["R"], d["K"], n, m, d["mask"].data_ptr(), sp)
        elif kind == "compress":
            rc = L.nm_compress(d["Wd"].data_ptr(), DT, d["R"], d["K"], n, m, LAY,
                               d["vals"].data_ptr(), d["meta"].data_ptr(), sp)
        elif kind == "decompress":
            rc = L.nm_decompress(d["vals"].data_ptr(), d["meta"].data_ptr(), DT, d["R"], d["K"],
                                 n, m, LAY, d["dec"].data_ptr(), sp)
        elif kind == "spmm":
            rc = L.nm_spmm(d["vals"].data_ptr(), d["meta"].data_ptr(), d["R"], d["K"], n, m, LAY,
                           d["Xd"].data_ptr(), d["T"], DT, d["Y"].data_ptr(), YDT, sp)
        elif kind == "tprune":
            rc = L.nm_tprune(d["Wd"].data_ptr(), DT, d["R"], d["K"], n, m, d["tpruned"].data_ptr(),
                             sp)
        elif kind == "compress_t":
            rc = L.nm_compress_t(d["tpruned"].data_ptr(), DT, d["R"], d["K"], n, m, LAY,
                                 d["vals_t"].data_ptr(), d["meta_t"].data_ptr(), sp)
        elif kind == "spmm_t":  # dX = W^T dY, with the forward output Y standing in for dY
            rc = L.nm_spmm(d["vals_t"].data_ptr(), d["meta_t"].data_ptr(), d["K"], d["R"], n, m,
                           LAY, d["Y"].data_ptr(), d["T"], DT, d["dX"].data_ptr(), DT, sp)
        elif kind == "prune":
            rc = L.nm_prune(d["Wd"].data_ptr(), DT, d["R"], d["K"], n, m, d["pruned"].data_ptr(), sp)
        else:
            rc = L.nm_srste_grad(d["Wd"].data_ptr(), d["Gd"].data_ptr(), DT, d["R"], d["K"], n, m,
                                 nm.SRSTE_DECAY, d["grad"].data_ptr(), sp)
        if rc != 0:
            raise RuntimeError(f"{kind} failed: {nm.status_str(rc)}")

    def step(events=None, kinds=kinds):
        for d in mats:
            for kind in kinds:
                if events is not None:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    launch(d, kind)
                    e1.record(stream)
                    events.append((d["name"], kind, e0, e1))
                else:
                    launch(d, kind)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, synchronised on both sides ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # ---- per-kernel durations, HIP events on the launch stream (separate pass) ----
    events = []
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    per = {}
    for name, kind, e0, e1 in events:
        per.setdefault((name, kind), []).append(e0.elapsed_time(e1))

    F_eff = sum(2.0 * d["R"] * d["K"] * d["T"] for d in mats)
    F_alg = F_eff * n / m
    value = F_eff / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    tot = {k: [0.0, 0.0] for k in kinds}  # [seconds per step, algorithmic bytes per step]
    for d in mats:
        ab = algorithmic_bytes(d["R"], d["K"], d["T"], n, m, d["s"], d["ys"])
        for kind in kinds:
            samples = per[(d["name"], kind)]
            t = float(np.mean(samples)) * 1e-3
            entry = {"us": round(t * 1e6, 2), "us_median": round(float(np.median(samples)) * 1e3, 2),
                     "us_min": round(float(np.min(samples)) * 1e3, 2), "alg_bytes": ab[kind],
                     "gbps": round(ab[kind] / t / 1e9, 1)}
            if kind == "spmm":
                f_alg = 2.0 * d["R"] * d["K"] * d["T"] * n / m
                entry["eff_tflops"] = round(2.0 * d["R"] * d["K"] * d["T"] / t / 1e12, 1)
                entry["alg_tflops"] = round(f_alg / t / 1e12, 1)
            else:
                entry["frac_hbm"] = round(ab[kind] / t / 1e9 / PEAK_HBM_GBS, 3)
            kernels[f"{d['name']}.{kind}"] = entry
            tot[kind][0] += t
            tot[kind][1] += ab[kind]

    spmm_t = tot["spmm"][0]
    achieved = F_alg / spmm_t / 1e12
    peak = PEAK_MFMA_TFLOPS[dtype]
    roofline = {"bound": "mfma",
                "kernel": ("nm_spmm (structured-sparse matrix cores)"
                           if n * 2 == m and dtype != "f32" else
                           "nm_spmm (dense matrix cores on expanded tiles)"),
                "achieved": round(achieved, 1), "peak": peak,
                "unit": "TOP/s" if dtype == "i8" else "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None,
                "alg_bytes_per_launch": sum(algorithmic_bytes(d["R"], d["K"], d["T"], n, m, d["s"],
                                                              d["ys"])["spmm"] for d in mats) / len(mats),
                "note": "achieved = algorithmic flops 2*R*(K*N/M)*T per launch / mean launch time; "
                        "traffic = profiled HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, "
                        "calibrated on a copy kernel)"}
    traffic = profiled_traffic(args.workload)
    if traffic is not None:
        roofline["traffic"] = round(traffic)

    mc_bytes, mc_time = tot["mask_compress"][1], tot["mask_compress"][0]
    mask_compress = {"gbps": round(mc_bytes / mc_time / 1e9, 1),
                     "frac_hbm": round(mc_bytes / mc_time / 1e9 / PEAK_HBM_GBS, 3),
                     "how": "nm_mask_compress: one pass writes the mask and the compressed pair"}
    # the two separate passes (nm_mask, nm_compress), for reference; not part of the step
    sep = {k: [0.0, 0.0] for k in ("mask", "compress")}
    sep_events = []
    for _ in range(args.steps):
        step(sep_events, kinds=["mask", "compress"])
    torch.cuda.synchronize()
    sep_per = {}
    for name, kind, e0, e1 in sep_events:
        sep_per.setdefault((name, kind), []).append(e0.elapsed_time(e1) * 1e-3)
    for d in mats:
        ab = algorithmic_bytes(d["R"], d["K"], d["T"], n, m, d["s"], d["ys"])
        for kind in ("mask", "compress"):
            t = float(np.mean(sep_per[(d["name"], kind)]))
            sep[kind][0] += t
            sep[kind][1] += ab[kind]
    for kind in ("mask", "compress"):
        mask_compress[f"separate_{kind}_gbps"] = round(sep[kind][1] / sep[kind][0] / 1e9, 1)
        mask_compress[f"separate_{kind}_frac_hbm"] = round(sep[kind][1] / sep[kind][0] / 1e9
                                                           / PEAK_HBM_GBS, 3)

    dense = None
    if not args.no_dense:
        # hipBLASLt through torch.matmul on the decompressed weight, same dtype and shapes
        ts = []
        for d in mats:
            A, B = d["dec"], d["Xd"]
            # int8: torch._int_mm (int8 x int8 -> int32); fp8: torch._scaled_mm (unit scales,
            # X column-major as it requires, bf16 out), where this PyTorch build has them
            if d["dtype"] == "i8":
                mm = torch._int_mm
            elif d["dtype"] == "fp8":
                one = torch.ones((), dtype=torch.float32, device=dev)
                B = B.t().contiguous().t()

                def mm(A, B, one=one):
                    return torch._scaled_mm(A, B, one, one, out_dtype=torch.bfloat16)
            else:
                mm = torch.matmul
            try:
                for _ in range(3):
                    mm(A, B)
            except (RuntimeError, AttributeError):
                continue
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                mm(A, B)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / args.steps * 1e-3)
        if ts:
            dense_t = sum(ts)
            dense = {"tflops": round(F_eff / dense_t / 1e12, 1), "us_total": round(dense_t * 1e6, 1),
                     "spmm_speedup": round(dense_t / spmm_t, 3),
                     "how": {"i8": "torch._int_mm", "fp8": "torch._scaled_mm (bf16 out)"}.get(
                         dtype, "torch.matmul (hipBLASLt)")
                            + " on the decompressed weight, same dtype"}

    srste = transposable = None
    if float_path:
        # ---- SR-STE passes on the same weights (not part of the step) ----
        # Each timed launch starts cold: a 512 MiB read (twice the 256 MB Infinity Cache) runs
        # before it, outside its events, so its inputs come from HBM as in a training step,
        # where the forward and the backward of a layer are far apart.  A read, not a fill:
        # a fill would leave dirty lines whose write-back competes with the timed kernel.
        sr_kinds = ["prune", "srste_grad"]
        flush = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            step(kinds=sr_kinds)
        torch.cuda.synchronize()
        sr_per = {}
        for _ in range(args.steps):
            for d in mats:
                for kind in sr_kinds:
                    flush.view(torch.int64).sum()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    launch(d, kind)
                    e1.record(stream)
                    sr_per.setdefault((d["name"], kind), []).append((e0, e1))
        torch.cuda.synchronize()
        sr_per = {k: [a.elapsed_time(b) * 1e-3 for a, b in v] for k, v in sr_per.items()}
        del flush
        srste = {"decay": nm.SRSTE_DECAY, "kernels": {}}
        sr_tot = {k: [0.0, 0.0] for k in sr_kinds}
        for d in mats:
            e = d["R"] * d["K"]
            ab = {"prune": 2 * e * d["s"], "srste_grad": 3 * e * d["s"]}
            for kind in sr_kinds:
                t = float(np.mean(sr_per[(d["name"], kind)]))
                srste["kernels"][f"{d['name']}.{kind}"] = {
                    "us": round(t * 1e6, 2), "alg_bytes": ab[kind], "gbps": round(ab[kind] / t / 1e9, 1),
                    "frac_hbm": round(ab[kind] / t / 1e9 / PEAK_HBM_GBS, 3)}
                sr_tot[kind][0] += t
                sr_tot[kind][1] += ab[kind]
        g_t, g_b = sr_tot["srste_grad"]
        srste["roofline"] = {"bound": "hbm", "kernel": "nm_srste_grad", "achieved": round(g_b / g_t / 1e9, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(g_b / g_t / 1e9 / PEAK_HBM_GBS, 3),
                             "alg_bytes_per_elem": 3 * mats[0]["s"], "traffic": None}
        g_traffic = profiled_traffic(args.workload, "srste_unit_kernel<2, 2, 4, true>"
                                     if dtype == "bf16" else "srste_unit_kernel", "nm_srste.hip")
        if g_traffic is not None:
            srste["roofline"]["traffic"] = round(g_traffic)
        srste["prune_frac_hbm"] = round(sr_tot["prune"][1] / sr_tot["prune"][0] / 1e9 / PEAK_HBM_GBS, 3)
        srste["step_us"] = round((g_t + sr_tot["prune"][0]) * 1e6, 1)

        # ---- transposable-mask path on the same weights (not part of the step) ----
        # tprune and compress_t are timed cold, like the SR-STE passes; the backward product
        # in the step's manner (its operands fit the Infinity Cache only in part).
        tr_kinds = ["tprune", "compress_t", "spmm_t"]
        flush = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            step(kinds=tr_kinds)
        torch.cuda.synchronize()
        tr_ev = {}
        for _ in range(args.steps):
            for d in mats:
                for kind in tr_kinds:
                    if kind != "spmm_t":
                        flush.view(torch.int64).sum()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    launch(d, kind)
                    e1.record(stream)
                    tr_ev.setdefault((d["name"], kind), []).append((e0, e1))
        torch.cuda.synchronize()
        del flush
        transposable = {"kernels": {}}
        for d in mats:
            e = d["R"] * d["K"]
            kept = e * n // m
            meta_t = d["K"] * ((d["R"] // m * n * meta_bits(m) + 31) // 32) * 4
            for kind in tr_kinds:
                t = float(np.mean([a.elapsed_time(b) for a, b in tr_ev[(d["name"], kind)]])) * 1e-3
                entry = {"us": round(t * 1e6, 2)}
                if kind == "spmm_t":
                    entry["eff_tflops"] = round(2.0 * e * d["T"] / t / 1e12, 1)
                    entry["alg_tflops"] = round(2.0 * kept * d["T"] / t / 1e12, 1)
                else:
                    ab = 2 * e * d["s"] if kind == "tprune" else e * d["s"] + kept * d["s"] + meta_t
                    entry.update(alg_bytes=ab, gbps=round(ab / t / 1e9, 1),
                                 frac_hbm=round(ab / t / 1e9 / PEAK_HBM_GBS, 3))
                transposable["kernels"][f"{d['name']}.{kind}"] = entry

    # ---- channel permutation: one round of swap-gain evaluation per matrix ----
    # (compute-bound: pairs of column groups x rows x M^2 swaps, each two max and four adds)
    permutation = {"kernels": {}}
    for d in mats:
        K, G = d["K"], d["K"] // m
        nbytes = int(L.nm_perm_workspace_bytes(d["R"], K, n, m))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        pv = torch.arange(K, dtype=torch.int32, device=dev)
        gain = torch.empty((G, G), dtype=torch.float32, device=dev)
        pick = torch.empty((G, G), dtype=torch.int32, device=dev)

        def gains_launch(d=d, K=K, ws=ws, pv=pv, gain=gain, pick=pick, nbytes=nbytes):
            rc = L.nm_perm_gains(d["Wd"].data_ptr(), DT, d["R"], K, n, m, pv.data_ptr(),
                                 gain.data_ptr(), pick.data_ptr(), ws.data_ptr(), nbytes, sp)
            if rc != 0:
                raise RuntimeError(f"nm_perm_gains failed: {nm.status_str(rc)}")

        gains_launch()
        torch.cuda.synchronize()
        reps = max(2, min(args.steps, 5))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            gains_launch()
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps * 1e-3
        evals = G * (G - 1) // 2 * d["R"] * m * m
        ops = evals * 7  # per swap and row: two adds and two max (the kept sums), one add,
        #                   one subtract (the base) and one accumulate
        permutation["kernels"][f"{d['name']}.perm_gains"] = {
            "ms": round(t * 1e3, 3), "pairs": G * (G - 1) // 2, "swap_row_evals": evals,
            "gops": round(ops / t / 1e9, 1), "frac_alu": round(ops / t / 1e12 / PEAK_VALU_TOPS, 3)}
        del ws, gain, pick
    permutation["roofline"] = {
        "bound": "alu", "unit": "T op/s", "peak": PEAK_VALU_TOPS,
        "note": "7 fp32 VALU operations per swap and row; peak = the fp32 vector peak "
                "157.3 TFLOP/s counted as operations (an FMA is two flops): 78.6 T op/s"}

    cpu = None
    if not args.no_cpu:
        if float_path:
            srste["cpu_baseline"] = srste_cpu_sample(mats, n, m)
        threads = max(1, min(16, os.cpu_count() or 1))
        cpu = cpu_baseline(mats, n, m, threads)

    w0 = mats[0]
    out = {
        "metric": {"i8": METRIC_I8, "fp8": METRIC_FP8}.get(dtype, METRIC),
        "value": round(value, 2),
        "unit": "TOP/s" if dtype == "i8" else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "matrices": [f"{d['name']} {d['R']}x{d['K']} X {d['K']}x{d['T']}" for d in mats],
                   "pattern": f"{n}:{m}", "layout": args.layout, "global_batch": w0["T"],
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "spmm_eff_tflops": round(F_eff / spmm_t / 1e12, 1),
        "mask_compress": mask_compress,
        "dense_gemm": dense,
        "kernels": kernels,
        "srste": srste,
        "transposable": transposable,
        "permutation": permutation,
        "context": "pages: up to 2x dense math throughput on A100 sparse Tensor Cores (not a target)",
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
