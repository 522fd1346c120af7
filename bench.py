#!/usr/bin/env python3
"""Benchmark of the N:M hot path on one MI355X.

One step = the whole path over one batch of synthetic input: for each weight
matrix of the workload, nm_mask, nm_compress (mask + values + metadata),
nm_decompress and nm_spmm (Y = W_sparse X).  Inputs are resident in HBM before
the timed region.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 100] [--workload llama_mlp]

`value` is the whole step's effective throughput: dense-equivalent product
flops (2 R K T per matrix) divided by the step time.  Per-kernel figures,
the roofline of the dominant kernel, the dense GEMM on the same shapes and the
CPU oracle timed on the host are reported alongside.

Each step kernel is also timed cold beside the in-step (warm) timing: launched on copies
of its buffers in rotation, enough copies that 512 MiB of other traffic (twice the 256 MB
Infinity Cache) separates two launches on one copy, rounds of the rotation between two
events.  The fp16 N:M sweep (4096 x 4096 weights, 8192 activation columns; 1:2, 2:4, 4:8
and mask-only) is timed warm (back to back) and cold the same way under "sweep_f16",
with its product's roofline and the dense GEMM.  The matrix cores' own rate on the
workload's values and the vector ALU's rate (libnm_probe) are reported under
"matrix_core_ceiling" and in the permutation roofline.

The SR-STE passes of a training step on the same weights (nm_prune, the
forward's masked weight, and nm_srste_grad, the backward's gradient) are timed
in a separate pass after the step, each launch after a 512 MiB read, and
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
# Vector-ALU peak in lane operations: the published fp32 vector rate, 157.3 TFLOP/s, is
# 256 CUs x 128 FMA lanes per clock x 2 flops x 2.4 GHz, i.e. 78.6 T lane-op/s.  The VALU
# probe (libnm_probe) shows plain, unpacked v_add_f32 and v_fma_f32 retiring 112-114 lanes
# per clock per CU, so this rate needs no packed math (which the library is compiled without);
# v_max_f32 retires at half that rate, so a kernel heavy in max/min stays below it.
PEAK_VALU_LANE_TOPS = 78.64
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


class HipTimer:
    """Kernel timing with HIP events created with hipEventDisableSystemFence, through the HIP
    runtime this process already loaded (PyTorch's).  Recording such an event does not make
    the queue flush caches to system scope, which costs a few microseconds per record with
    default events and inflates the time of short kernels; the interval between two records
    on the launch stream is then the kernels' own time, as a profiler's kernel trace shows."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, stream_handle: int):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        import ctypes

        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.stream = ctypes.c_void_p(stream_handle)
        self.pool = []

    def event(self):
        e = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.pool.append(e)
        return e

    def record(self, e):
        if self.hip.hipEventRecord(e, self.stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, e0, e1) -> float:
        self.hip.hipEventSynchronize(e1)
        out = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(out), e0, e1) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def close(self):
        for e in self.pool:
            self.hip.hipEventDestroy(e)
        self.pool = []


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


SPMM_SOURCES = ("nm_spmm.hip", "nm_spmm_sk.hip", "nm_mfma.h")


def profile_matches(prof: dict, sources) -> bool:
    """True when every source file in `sources` is byte-identical to the one the committed
    profile `prof` was taken on (its "sources_sha256" table)."""
    for source in sources:
        src = os.path.join(ROOT, "masking_sparse_gemm_amd", "csrc", source)
        with open(src, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != prof.get("sources_sha256", {}).get(source):
                return False
    return True


def profiled_traffic(workload: str, kernel: str = "spmm_kernel", sources=SPMM_SOURCES):
    """HBM bytes per dispatch of the kernels whose key contains `kernel`, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy-kernel calibration),
    or None when that summary is missing or was taken on a different version of any of
    `sources`."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    if not profile_matches(prof, sources):
        return None
    per = [v["read_bytes"] + v["write_bytes"] for k, v in prof["per_dispatch_bytes"].items()
           if kernel in k]
    return sum(per) / len(per) if per else None


def profiled_valu(workload: str, kernel: str = "gains_kernel", sources=("nm_perm.hip",)):
    """Wave-level VALU instructions per dispatch of `kernel` (SQ_INSTS_VALU) from the committed
    rocprofv3 summary, keyed by matrix name, or {} when that summary is missing or was taken
    on a different version of any of `sources`."""
    path = os.path.join(ROOT, "profiles", f"{workload}_valu.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        prof = json.load(f)
    if not profile_matches(prof, sources) or kernel not in prof.get("kernel", ""):
        return {}
    return dict(prof.get("valu_insts_per_dispatch", {}))


def cpu_info():
    """Host CPU model and the cores this process may run on (the box allots 16 per GPU)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:
        visible = os.cpu_count() or 1
    return model, visible


def cpu_one_core(mats, n, m, rows: int = 64):
    """The oracle on one thread: mask + compress, decompress and the fp64 product of the first
    `rows` rows of every matrix (all T columns), each phase timed, scaled to the workload."""
    import oracle

    oracle.lib()
    F = F_all = B_mc = 0.0
    t_mc = t_rest = t_mm = 0.0
    for w in mats:
        part = np.ascontiguousarray(w["W"][:rows])
        r = part.shape[0]
        ta = time.perf_counter()
        oracle.mask(part, w["dtype"], n, m)
        vals, meta = oracle.compress(part, w["dtype"], n, m)
        tb = time.perf_counter()
        oracle.decompress(vals, meta, w["dtype"], r, w["K"], n, m)
        tc = time.perf_counter()
        Y = np.empty((r, w["T"]), dtype=np.float64)
        oracle.spmm_rows(vals, meta, r, w["K"], n, m, w["X"], w["dtype"], 0, r, Y)
        td = time.perf_counter()
        t_mc += tb - ta
        t_rest += tc - tb
        t_mm += td - tc
        B_mc += algorithmic_bytes(r, w["K"], w["T"], n, m, w["s"], w["ys"])["mask_compress"]
        F += 2.0 * r * w["K"] * w["T"]
        F_all += 2.0 * w["R"] * w["K"] * w["T"]
    dt = t_mc + t_rest + t_mm
    rate = F / dt
    unit = "TOP/s" if mats[0]["dtype"] == "i8" else "TFLOP/s"
    return {"value": rate / 1e12, "unit": unit, "cores": 1, "seconds": round(dt, 2),
            "sample": f"rows 0..{rows} of each matrix, all T columns",
            "extrapolated_step_s": round(F_all / rate, 1),
            "note": "one step of the whole workload on one core, extrapolated from the sample",
            "phases": {"mask_compress_gbps": round(B_mc / t_mc / 1e9, 3),
                       "product_" + unit.replace("/", "_per_"): round(F / t_mm / 1e12, 5)}}


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
    """The oracle as it stands, on the host: mask + compress, decompress and the product of a
    bounded slice of rows of every matrix, rows spread over `threads` threads.  Each phase
    runs over all threads before the next starts, so their rates are reported apart as well
    (mask + compress in GB/s of its algorithmic bytes, the product in TFLOP/s)."""
    import oracle

    oracle.lib()
    F = 0.0
    B_mc = B_dec = 0.0
    t_mc = t_dec = t_mm = 0.0
    rows_done = {}
    t0 = time.perf_counter()
    block = 4  # rows per thread per round
    while True:
        for w in mats:
            r0 = rows_done.get(w["name"], 0)
            r1 = min(w["R"], r0 + block * threads)
            if r1 <= r0:
                continue
            Wsl = np.ascontiguousarray(w["W"][r0:r1])
            R = r1 - r0
            parts = [None] * threads

            def split(k, R=R):
                return k * R // threads, (k + 1) * R // threads

            def mask_compress(k, Wsl=Wsl, w=w):
                a, b = split(k)
                if b > a:
                    part = np.ascontiguousarray(Wsl[a:b])
                    oracle.mask(part, w["dtype"], n, m)
                    parts[k] = oracle.compress(part, w["dtype"], n, m)

            def decompress(k, w=w):
                a, b = split(k)
                if b > a:
                    oracle.decompress(parts[k][0], parts[k][1], w["dtype"], b - a, w["K"], n, m)

            def product(k, w=w):
                a, b = split(k)
                if b > a:
                    Y = np.empty((b - a, w["T"]), dtype=np.float64)
                    oracle.spmm_rows(parts[k][0], parts[k][1], b - a, w["K"], n, m, w["X"],
                                     w["dtype"], 0, b - a, Y)

            ab = algorithmic_bytes(R, w["K"], w["T"], n, m, w["s"], w["ys"])
            with ThreadPoolExecutor(max_workers=threads) as ex:
                ta = time.perf_counter()
                list(ex.map(mask_compress, range(threads)))
                tb = time.perf_counter()
                list(ex.map(decompress, range(threads)))
                tc = time.perf_counter()
                list(ex.map(product, range(threads)))
                td = time.perf_counter()
            t_mc += tb - ta
            t_dec += tc - tb
            t_mm += td - tc
            B_mc += ab["mask_compress"]
            B_dec += ab["decompress"]
            rows_done[w["name"]] = r1
            F += 2.0 * R * w["K"] * w["T"]
        if time.perf_counter() - t0 >= budget_s or all(rows_done.get(w["name"], 0) >= w["R"]
                                                       for w in mats):
            break
    dt = time.perf_counter() - t0
    sample = ", ".join(f"{k}: rows 0..{v} of {next(w['R'] for w in mats if w['name'] == k)}"
                       for k, v in rows_done.items())
    unit = "TOP/s" if mats[0]["dtype"] == "i8" else "TFLOP/s"
    return {"value": F / dt / 1e12, "unit": unit, "cores": threads, "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"mask+compress+decompress+product of {sample} (fp64 product, all T columns)",
            "phases": {"mask_compress_gbps": round(B_mc / t_mc / 1e9, 3),
                       "decompress_gbps": round(B_dec / t_dec / 1e9, 3),
                       "product_" + unit.replace("/", "_per_"): round(F / t_mm / 1e12, 5)}}


def bf16_sample(a: np.ndarray, dtype: str, count: int = 1 << 20) -> np.ndarray:
    """bf16 bit patterns of (up to) the first `count` values of a workload array."""
    a = a.reshape(-1)[:count]
    if dtype == "bf16":
        return a.view(np.uint16)
    if dtype == "f16":
        a = a.view(np.float16).astype(np.float32)
    elif dtype in ("i8",):
        a = a.astype(np.float32)
    elif dtype != "f32":
        a = np.zeros(1, dtype=np.float32)
    return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def matrix_core_ceiling(torch, dev, stream, hipt, w_vals, x_vals, waves_per_simd: int = 2):
    """What the matrix cores sustain alone (libnm_probe): the 2:4 structured-sparse bf16
    instruction and the dense bf16 one in register-only loops, on three kinds of operands:
    zeros, small integers, and values drawn from the workload's own weights and
    activations.  Returns effective (dense-equivalent) TFLOP/s per instruction and kind,
    and the shader clock the loop ran at (s_memtime over the 100 MHz s_memrealtime)."""
    import masking_sparse_gemm_amd as nm

    P = nm.probe_lib()
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    per_lane = 24
    n_ops = 4 * 64 * per_lane
    rng = np.random.default_rng(7)
    kinds = {
        "zeros": np.zeros(n_ops, dtype=np.uint16),
        "small_integers": (np.array(rng.integers(-3, 4, n_ops), dtype=np.float32)
                           .view(np.uint32) >> 16).astype(np.uint16),
    }
    # the workload's values: A lanes from W, B lanes from X (bf16 bit patterns)
    ops = np.empty((4, 64, per_lane), dtype=np.uint16)
    ops[:, :, :8] = rng.choice(w_vals, size=(4, 64, 8))
    ops[:, :, 8:] = rng.choice(x_vals, size=(4, 64, 16))
    kinds["workload"] = ops.reshape(-1)
    clocks = torch.zeros(4 * cus * waves_per_simd, dtype=torch.int64, device=dev)
    sink = torch.zeros(cus * waves_per_simd * 256, dtype=torch.float32, device=dev)
    out = {"waves_per_simd": waves_per_simd, "cus": cus}
    for kname, arr in kinds.items():
        dops = torch.from_numpy(arr.view(np.int16)).to(dev)
        for inst, kind, flops in (("smfmac_32x32x32_bf16", 0, 65536), ("mfma_32x32x16_bf16", 1, 32768)):
            iters = 4000
            for _ in range(3):  # warm-up (clock ramp)
                P.nm_probe_matrix_core(kind, dops.data_ptr(), cus, waves_per_simd, iters,
                                       clocks.data_ptr(), sink.data_ptr(), stream.cuda_stream)
            best = None
            for _ in range(3):  # the best of three launches: what the instruction sustains
                e0, e1 = hipt.event(), hipt.event()
                hipt.record(e0)
                rc = P.nm_probe_matrix_core(kind, dops.data_ptr(), cus, waves_per_simd, iters,
                                            clocks.data_ptr(), sink.data_ptr(), stream.cuda_stream)
                hipt.record(e1)
                torch.cuda.synchronize()
                if rc != 0:
                    raise RuntimeError(f"nm_probe_matrix_core failed ({rc})")
                t = hipt.ms(e0, e1) * 1e-3
                c = clocks.view(-1, 4).cpu().numpy().astype(np.float64)
                mhz = float(np.median((c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1)
                                      * 100.0))
                if best is None or t < best[0]:
                    best = (t, mhz)
            t, mhz = best
            insts = cus * waves_per_simd * 4 * iters * 16
            out[f"{inst}.{kname}"] = {"eff_tflops": round(insts * flops / t / 1e12, 1),
                                      "clock_mhz": round(mhz, 0), "ms": round(t * 1e3, 3)}
    return out


def hbm_copy(torch, dev, stream, hipt, nbytes: int = 1 << 30, reps: int = 10):
    """What HBM sustains for a pass that reads and writes each byte once: a plain 16-byte
    non-temporal copy kernel (libnm_probe) over 1 GiB, far past the 256 MB Infinity Cache."""
    import masking_sparse_gemm_amd as nm

    P = nm.probe_lib()
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    for _ in range(3):
        if P.nm_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream.cuda_stream) != 0:
            raise RuntimeError("nm_probe_copy failed")
    e0, e1 = hipt.event(), hipt.event()
    hipt.record(e0)
    for _ in range(reps):
        P.nm_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream.cuda_stream)
    hipt.record(e1)
    torch.cuda.synchronize()
    t = hipt.ms(e0, e1) * 1e-3 / reps
    # the runtime's own device-to-device copy of the same buffers, for comparison
    for _ in range(3):
        dst.copy_(src)
    e2, e3 = hipt.event(), hipt.event()
    hipt.record(e2)
    for _ in range(reps):
        dst.copy_(src)
    hipt.record(e3)
    torch.cuda.synchronize()
    t_rt = hipt.ms(e2, e3) * 1e-3 / reps
    del src, dst
    gbps, gbps_rt = 2.0 * nbytes / t / 1e9, 2.0 * nbytes / t_rt / 1e9
    return {"gbps": round(max(gbps, gbps_rt), 1),
            "frac_hbm": round(max(gbps, gbps_rt) / PEAK_HBM_GBS, 3),
            "probe_gbps": round(gbps, 1), "runtime_copy_gbps": round(gbps_rt, 1),
            "how": "1 GiB device-to-device copies, read + write bytes: a 16-byte non-temporal "
                   "copy kernel (libnm_probe) and the runtime's copy (torch copy_); gbps is "
                   "the faster"}


def valu_ceiling(torch, dev, stream, hipt):
    """What the vector ALU sustains alone (libnm_probe): plain (unpacked) v_add_f32,
    v_max_f32 and v_fma_f32 in register-only loops, 1 to 8 waves per SIMD.  Returns, per
    instruction, the best rate in T lane-op/s (wave instructions x 64 lanes / s), the lanes
    retired per clock per CU at the measured shader clock, and that clock."""
    import masking_sparse_gemm_amd as nm

    P = nm.probe_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {"cus": cus}
    clocks = torch.zeros(4 * cus * 8, dtype=torch.int64, device=dev)
    sink = torch.zeros(cus * 8 * 256, dtype=torch.float32, device=dev)
    iters = 20000
    for name, op in (("v_add_f32", 0), ("v_max_f32", 1), ("v_fma_f32", 2)):
        best = None
        for wps in (1, 2, 4, 8):
            P.nm_probe_valu(op, cus, wps, iters, clocks.data_ptr(), sink.data_ptr(), stream.cuda_stream)
            e0, e1 = hipt.event(), hipt.event()
            hipt.record(e0)
            rc = P.nm_probe_valu(op, cus, wps, iters, clocks.data_ptr(), sink.data_ptr(),
                                 stream.cuda_stream)
            hipt.record(e1)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"nm_probe_valu failed ({rc})")
            t = hipt.ms(e0, e1) * 1e-3
            lane_ops = cus * wps * 4 * iters * 64 * 64.0
            c = clocks[: 4 * cus * wps].view(-1, 4).cpu().numpy().astype(np.float64)
            mhz = float(np.median((c[:, 1] - c[:, 0]) / np.maximum(c[:, 3] - c[:, 2], 1) * 100.0))
            r = {"waves_per_simd": wps, "lane_tops": round(lane_ops / t / 1e12, 2),
                 "lanes_per_clock_per_cu": round(lane_ops / t / (mhz * 1e6) / cus, 1),
                 "clock_mhz": round(mhz, 0), "ms": round(t * 1e3, 3)}
            if best is None or r["lane_tops"] > best["lane_tops"]:
                best = r
        out[name] = best
    return out


def load_path_ceiling(nm, mats, stream, hipt, launch, reps):
    """What the product's direct global -> LDS loads take alone (libnm_probe's load-path
    probe: the same loads, ring, waits, barriers and tile mapping as the 2:4 product on its
    256 x 128 tiles, with idle waves in place of the matrix work), timed as `reps` launches
    back to back on each matrix's own inputs, beside the product timed the same way."""
    import torch

    P = nm.probe_lib()
    sp = stream.cuda_stream
    out = {"us": {}, "spmm_us": {}}
    for d in mats:
        def probe(d=d):
            rc = P.nm_probe_load_path(d["vals"].data_ptr(), d["meta"].data_ptr(),
                                      d["Xd"].data_ptr(), d["R"], d["K"], d["T"], sp)
            if rc != 0:
                raise RuntimeError(f"nm_probe_load_path failed ({rc})")
        for name, fn in (("us", probe), ("spmm_us", lambda d=d: launch(d, "spmm"))):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = hipt.event(), hipt.event()
            hipt.record(e0)
            for _ in range(reps):
                fn()
            hipt.record(e1)
            torch.cuda.synchronize()
            out[name][d["name"]] = round(hipt.ms(e0, e1) / reps * 1e3, 2)
    out["how"] = ("the product's direct loads alone (libnm_probe): X rows, compressed values and "
                  "metadata of every 64-wide K step into the same 4-stage LDS ring with the same "
                  "waits, barriers and XCD tile mapping, idle waves in place of the matrix work; "
                  "launches back to back, the product timed the same way beside it (spmm_us); "
                  "alg_tflops = the product's algorithmic flops over the probe's time")
    return out


def sweep_f16_block(torch, nm, synth, L, dev, stream, hipt, args, cold_times):
    """The fp16 N:M sweep: W 4096 x 4096 ~Laplace(0, 0.05), X 4096 x 8192 ~N(0, 1).  For each
    of 1:2, 2:4 and 4:8: the fused mask + compress pass, the mask alone, decompress and the
    product, warm (back to back on one buffer set) and cold (rotating buffer copies, so
    every launch reads from HBM), the dense GEMM (hipBLASLt) on the decompressed weight, and
    the product's matrix-core roofline."""
    w = synth.WORKLOADS["sweep_f16"]
    R, K, T = w.R, w.K, w.T
    W, X = w.W(), w.X()
    f16 = torch.float16
    Wd = torch.from_numpy(W.view(np.int16)).view(f16).to(dev)
    Xd = torch.from_numpy(X.view(np.int16)).view(f16).to(dev)
    mask = torch.empty((R, K), dtype=torch.bool, device=dev)
    dec = torch.empty((R, K), dtype=f16, device=dev)
    Y = torch.empty((R, T), dtype=f16, device=dev)
    sp = stream.cuda_stream
    LAY = nm.LAYOUTS[args.layout]
    out = {"matrix": f"{R}x{K} X {K}x{T}", "dtype": "f16", "layout": args.layout, "patterns": {}}
    reps = args.steps
    for (n, m) in w.patterns:
        vshape, mshape = nm.compressed_shapes(R, K, n, m, args.layout)
        vals = torch.empty(vshape, dtype=f16, device=dev)
        meta = torch.empty(mshape, dtype=torch.int32, device=dev)
        d = {"name": f"{n}:{m}", "R": R, "K": K, "T": T, "Wd": Wd, "mask": mask, "vals": vals,
             "meta": meta, "dec": dec, "Xd": Xd, "Y": Y}

        def launch(d, kind, n=n, m=m):
            if kind == "mask_compress":
                rc = L.nm_mask_compress(d["Wd"].data_ptr(), 1, R, K, n, m, LAY,
                                        d["mask"].data_ptr(), d["vals"].data_ptr(),
                                        d["meta"].data_ptr(), sp)
            elif kind == "mask":
                rc = L.nm_mask(d["Wd"].data_ptr(), 1, R, K, n, m, d["mask"].data_ptr(), sp)
            elif kind == "decompress":
                rc = L.nm_decompress(d["vals"].data_ptr(), d["meta"].data_ptr(), 1, R, K, n, m,
                                     LAY, d["dec"].data_ptr(), sp)
            else:
                rc = L.nm_spmm(d["vals"].data_ptr(), d["meta"].data_ptr(), R, K, n, m, LAY,
                               d["Xd"].data_ptr(), T, 1, d["Y"].data_ptr(), 1, sp)
            if rc != 0:
                raise RuntimeError(f"sweep {kind} {n}:{m} failed: {nm.status_str(rc)}")

        kinds = ["mask_compress", "mask", "decompress", "spmm"]
        for _ in range(max(2, args.warmup)):
            for k in kinds:
                launch(d, k)
        torch.cuda.synchronize()
        # warm: `reps` launches of one kernel back to back between two events (its inputs stay
        # in the Infinity Cache); the per-launch mean includes the gaps between launches
        warm = {}
        for k in kinds:
            e0, e1 = hipt.event(), hipt.event()
            hipt.record(e0)
            for _ in range(reps):
                launch(d, k)
            hipt.record(e1)
            warm[k] = [hipt.ms(e0, e1) / reps]
        cold = {k[1]: v for k, v in cold_times([d], kinds, launch, reps).items()}
        ab = algorithmic_bytes(R, K, T, n, m, 2, 2)
        entry = {}
        for k in kinds:
            t, tc = float(np.mean(warm[k])) * 1e-3, float(np.mean(cold[k])) * 1e-3
            e = {"us": round(t * 1e6, 2), "us_cold": round(tc * 1e6, 2), "alg_bytes": ab[k]}
            if k == "spmm":
                f_eff = 2.0 * R * K * T
                e.update(eff_tflops=round(f_eff / t / 1e12, 1),
                         eff_tflops_cold=round(f_eff / tc / 1e12, 1),
                         alg_tflops=round(f_eff * n / m / t / 1e12, 1),
                         frac_mfma=round(f_eff * n / m / t / 1e12 / PEAK_MFMA_TFLOPS["f16"], 4),
                         frac_mfma_cold=round(f_eff * n / m / tc / 1e12 / PEAK_MFMA_TFLOPS["f16"], 4))
                tr = profiled_traffic("sweep_f16", f"{n}:{m} spmm ")
                e["traffic"] = None if tr is None else round(tr)
                e["traffic_over_alg"] = None if tr is None else round(tr / ab[k], 2)
            else:
                e.update(gbps=round(ab[k] / t / 1e9, 1), frac_hbm=round(ab[k] / t / 1e9 / PEAK_HBM_GBS, 3),
                         gbps_cold=round(ab[k] / tc / 1e9, 1),
                         frac_hbm_cold=round(ab[k] / tc / 1e9 / PEAK_HBM_GBS, 3))
            entry[k] = e
        if not args.no_dense:
            for _ in range(3):
                torch.matmul(dec, Xd)
            torch.cuda.synchronize()
            e0, e1 = hipt.event(), hipt.event()
            hipt.record(e0)
            for _ in range(reps):
                torch.matmul(dec, Xd)
            hipt.record(e1)
            torch.cuda.synchronize()
            td = hipt.ms(e0, e1) / reps * 1e-3
            entry["dense_gemm"] = {"us": round(td * 1e6, 2),
                                   "eff_tflops": round(2.0 * R * K * T / td / 1e12, 1),
                                   "how": "torch.matmul (hipBLASLt) on the decompressed weight"}
            entry["spmm_speedup"] = round(td / (float(np.mean(warm["spmm"])) * 1e-3), 3)
        out["patterns"][f"{n}:{m}"] = entry
        del vals, meta
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 100 untimed steps (~35 ms of GPU work on the LLaMA pair) bring the device to its steady
    # clock; after 5, the timed steps still ran ~13% slower than after 100 or 300
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="llama_mlp", choices=sorted(WORKLOADS))
    ap.add_argument("--layout", default="blocked", choices=["blocked", "rows"],
                    help="storage layout of the compressed weight (include/nm.h)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense GEMM baseline")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the fp16 N:M sweep block (1:2, 2:4, 4:8 on 4096 x 4096 x 8192)")
    ap.add_argument("--product-only", action="store_true",
                    help="time only nm_spmm on the workload's matrices (for profiling runs)")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="run only the rate probes (libnm_probe): matrix cores, vector ALU, "
                         "HBM copy and the product's load path")
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
    hipt = HipTimer(sp)
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
                    e0 = hipt.event()
                    e1 = hipt.event()
                    hipt.record(e0)
                    launch(d, kind)
                    hipt.record(e1)
                    events.append((d["name"], kind, e0, e1))
                else:
                    launch(d, kind)

    if args.ceiling_only:
        w_vals, x_vals = bf16_sample(mats[0]["W"], dtype), bf16_sample(mats[0]["X"], dtype)
        out = {"matrix_core_ceiling": matrix_core_ceiling(torch, dev, stream, hipt, w_vals, x_vals),
               "valu_ceiling": valu_ceiling(torch, dev, stream, hipt),
               "hbm_copy": hbm_copy(torch, dev, stream, hipt)}
        if dtype in ("bf16", "f16") and (n, m) == (2, 4) and args.layout == "blocked" and \
                all(d["T"] % 8 == 0 and d["K"] % 64 == 0 for d in mats):
            for d in mats:
                launch(d, "mask_compress")
            lp = load_path_ceiling(nm, mats, stream, hipt, launch, args.steps)
            f_alg = sum(2.0 * d["R"] * d["K"] * d["T"] for d in mats) * n / m
            lp["alg_tflops"] = round(f_alg / (sum(lp["us"].values()) * 1e-6) / 1e12, 1)
            lp["frac_of_peak"] = round(lp["alg_tflops"] / PEAK_MFMA_TFLOPS[dtype], 4)
            out["load_path_ceiling"] = lp
        print(json.dumps(out), flush=True)
        return 0

    if args.product_only:
        # the compressed pairs once, then only the products: the launches a profiler sees
        for d in mats:
            launch(d, "mask_compress")
        for _ in range(args.warmup):
            step(kinds=["spmm"])
        torch.cuda.synchronize()
        ev = []
        for _ in range(args.steps):
            step(ev, kinds=["spmm"])
        torch.cuda.synchronize()
        res = {}
        for name, kind, e0, e1 in ev:
            res.setdefault(name, []).append(hipt.ms(e0, e1) * 1e3)
        out = {}
        for d in mats:
            t = float(np.mean(res[d["name"]]))
            out[d["name"]] = {"us": round(t, 2), "us_min": round(float(np.min(res[d["name"]])), 2),
                              "eff_tflops": round(2.0 * d["R"] * d["K"] * d["T"] / t / 1e6, 1)}
        print(json.dumps({"workload": args.workload, "pattern": f"{n}:{m}", "layout": args.layout,
                          "spmm": out}), flush=True)
        return 0

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
        per.setdefault((name, kind), []).append(hipt.ms(e0, e1))

    # ---- the same kernels cold.  Each (matrix, kernel) is launched on copies of the buffers
    # it touches, in rotation, with enough copies that at least 512 MiB of other traffic
    # (twice the 256 MB Infinity Cache) separates two launches on one copy, so every launch
    # finds its inputs in HBM; `steps` rounds of the rotation run between two events.
    touch = {"mask_compress": (["Wd"], ["mask", "vals", "meta"]), "mask": (["Wd"], ["mask"]),
             "compress": (["Wd"], ["vals", "meta"]), "decompress": (["vals", "meta"], ["dec"]),
             "spmm": (["vals", "meta", "Xd"], ["Y"])}
    cold_bytes = 1 << 29

    def cold_times(mat_list, kind_list, launch_fn, reps):
        res = {}
        for d in mat_list:
            for kind in kind_list:
                ins, outs = touch[kind]
                nbytes = sum(d[k].numel() * d[k].element_size() for k in ins + outs)
                sets = -(-cold_bytes // nbytes) + 1
                copies = [d] + [dict(d, **{k: d[k].clone() for k in ins},
                                     **{k: torch.empty_like(d[k]) for k in outs})
                                for _ in range(sets - 1)]
                for c in copies:  # one untimed round: the first round starts cold as well
                    launch_fn(c, kind)
                e0, e1 = hipt.event(), hipt.event()
                hipt.record(e0)
                for _ in range(reps):
                    for c in copies:
                        launch_fn(c, kind)
                hipt.record(e1)
                torch.cuda.synchronize()
                res[(d["name"], kind)] = [hipt.ms(e0, e1) / (reps * len(copies))]
                del copies
        return res

    per_cold = cold_times(mats, kinds, launch, args.steps)

    F_eff = sum(2.0 * d["R"] * d["K"] * d["T"] for d in mats)
    F_alg = F_eff * n / m
    value = F_eff / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    tot = {k: [0.0, 0.0] for k in kinds}  # [seconds per step, algorithmic bytes per step]
    tot_cold = {k: 0.0 for k in kinds}
    for d in mats:
        ab = algorithmic_bytes(d["R"], d["K"], d["T"], n, m, d["s"], d["ys"])
        for kind in kinds:
            samples = per[(d["name"], kind)]
            t = float(np.mean(samples)) * 1e-3
            tc = float(np.mean(per_cold[(d["name"], kind)])) * 1e-3
            entry = {"us": round(t * 1e6, 2), "us_median": round(float(np.median(samples)) * 1e3, 2),
                     "us_min": round(float(np.min(samples)) * 1e3, 2), "us_cold": round(tc * 1e6, 2),
                     "alg_bytes": ab[kind], "gbps": round(ab[kind] / t / 1e9, 1)}
            if kind == "spmm":
                f_alg = 2.0 * d["R"] * d["K"] * d["T"] * n / m
                entry["eff_tflops"] = round(2.0 * d["R"] * d["K"] * d["T"] / t / 1e12, 1)
                entry["alg_tflops"] = round(f_alg / t / 1e12, 1)
                entry["eff_tflops_cold"] = round(2.0 * d["R"] * d["K"] * d["T"] / tc / 1e12, 1)
            else:
                entry["frac_hbm"] = round(ab[kind] / t / 1e9 / PEAK_HBM_GBS, 3)
                entry["frac_hbm_cold"] = round(ab[kind] / tc / 1e9 / PEAK_HBM_GBS, 3)
            kernels[f"{d['name']}.{kind}"] = entry
            tot[kind][0] += t
            tot[kind][1] += ab[kind]
            tot_cold[kind] += tc

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
        roofline["traffic_over_alg"] = round(traffic / roofline["alg_bytes_per_launch"], 2)

    mc_bytes, mc_time = tot["mask_compress"][1], tot["mask_compress"][0]
    mask_compress = {"gbps": round(mc_bytes / mc_time / 1e9, 1),
                     "frac_hbm": round(mc_bytes / mc_time / 1e9 / PEAK_HBM_GBS, 3),
                     "gbps_cold": round(mc_bytes / tot_cold["mask_compress"] / 1e9, 1),
                     "frac_hbm_cold": round(mc_bytes / tot_cold["mask_compress"] / 1e9
                                            / PEAK_HBM_GBS, 3),
                     "how": "nm_mask_compress: one pass writes the mask and the compressed pair"}
    # the two separate passes (nm_mask, nm_compress), for reference; not part of the step
    sep = {k: [0.0, 0.0] for k in ("mask", "compress")}
    sep_events = []
    for _ in range(args.steps):
        step(sep_events, kinds=["mask", "compress"])
    torch.cuda.synchronize()
    sep_per = {}
    for name, kind, e0, e1 in sep_events:
        sep_per.setdefault((name, kind), []).append(hipt.ms(e0, e1) * 1e-3)
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
        # the product timed as the dense GEMM is below: `steps` launches back to back on one
        # matrix between two events, so the ratio compares like with like
        spmm_b = 0.0
        for d in mats:
            launch(d, "spmm")
            torch.cuda.synchronize()
            e0, e1 = hipt.event(), hipt.event()
            hipt.record(e0)
            for _ in range(args.steps):
                launch(d, "spmm")
            hipt.record(e1)
            torch.cuda.synchronize()
            spmm_b += hipt.ms(e0, e1) / args.steps * 1e-3
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
            e0, e1 = hipt.event(), hipt.event()
            hipt.record(e0)
            for _ in range(args.steps):
                mm(A, B)
            hipt.record(e1)
            torch.cuda.synchronize()
            ts.append(hipt.ms(e0, e1) / args.steps * 1e-3)
        if ts:
            dense_t = sum(ts)
            dense = {"tflops": round(F_eff / dense_t / 1e12, 1), "us_total": round(dense_t * 1e6, 1),
                     "spmm_us_total": round(spmm_b * 1e6, 1),
                     "spmm_speedup": round(dense_t / spmm_b, 3),
                     "spmm_speedup_in_step": round(dense_t / spmm_t, 3),
                     "how": {"i8": "torch._int_mm", "fp8": "torch._scaled_mm (bf16 out)"}.get(
                         dtype, "torch.matmul (hipBLASLt)")
                            + " on the decompressed weight, same dtype"}

    # ---- what HBM sustains for a plain copy on this device (libnm_probe) ----
    copy_rate = hbm_copy(torch, dev, stream, hipt)
    mask_compress["frac_of_copy"] = round(mask_compress["gbps"] / copy_rate["gbps"], 3)

    # ---- the matrix cores' own rate on this workload's values (libnm_probe) ----
    ceiling = None
    if dtype in ("bf16", "f16"):
        ceiling = matrix_core_ceiling(torch, dev, stream, hipt, bf16_sample(mats[0]["W"], dtype),
                                      bf16_sample(mats[0]["X"], dtype))
        c = ceiling["smfmac_32x32x32_bf16.workload"]
        roofline["ceiling"] = {
            "alg_tflops": round(c["eff_tflops"] / 2, 1), "clock_mhz": c["clock_mhz"],
            "how": "v_smfmac_f32_32x32x32_bf16 alone in a register loop on operands drawn from "
                   "this workload's W and X (libnm_probe); the device lowers its clock under "
                   "such load (zeros: %d MHz)" % ceiling["smfmac_32x32x32_bf16.zeros"]["clock_mhz"]}
        roofline["frac_of_ceiling"] = round(achieved / (c["eff_tflops"] / 2), 4)

    # ---- the product's direct loads alone (libnm_probe): its load-path bound ----
    if dtype in ("bf16", "f16") and (n, m) == (2, 4) and args.layout == "blocked" and \
            all(d["T"] % 8 == 0 and d["K"] % 64 == 0 for d in mats):
        lp = load_path_ceiling(nm, mats, stream, hipt, launch, args.steps)
        lp["alg_tflops"] = round(F_alg / (sum(lp["us"].values()) * 1e-6) / 1e12, 1)
        lp["frac_of_peak"] = round(lp["alg_tflops"] / peak, 4)
        roofline["load_path_ceiling"] = lp
        roofline["frac_of_load_path"] = round(sum(lp["us"].values())
                                              / sum(lp["spmm_us"].values()), 4)

    # ---- the fp16 N:M sweep: 4096 x 4096 weights, 8192 activation columns ----
    sweep = None
    if args.workload == "llama_mlp" and not args.no_sweep:
        sweep = sweep_f16_block(torch, nm, synth, L, dev, stream, hipt, args, cold_times)

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
                    e0 = hipt.event()
                    e1 = hipt.event()
                    hipt.record(e0)
                    launch(d, kind)
                    hipt.record(e1)
                    sr_per.setdefault((d["name"], kind), []).append((e0, e1))
        torch.cuda.synchronize()
        sr_per = {k: [hipt.ms(a, b) * 1e-3 for a, b in v] for k, v in sr_per.items()}
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
                    "frac_hbm": round(ab[kind] / t / 1e9 / PEAK_HBM_GBS, 3),
                    "frac_of_copy": round(ab[kind] / t / 1e9 / copy_rate["gbps"], 3)}
                sr_tot[kind][0] += t
                sr_tot[kind][1] += ab[kind]
        g_t, g_b = sr_tot["srste_grad"]
        srste["roofline"] = {"bound": "hbm", "kernel": "nm_srste_grad", "achieved": round(g_b / g_t / 1e9, 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(g_b / g_t / 1e9 / PEAK_HBM_GBS, 3),
                             "alg_bytes_per_elem": 3 * mats[0]["s"], "traffic": None}
        g_traffic = profiled_traffic(args.workload, "srste_unit_kernel<2, 2, 4, true>"
                                     if dtype == "bf16" else "srste_unit_kernel", ("nm_srste.hip",))
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
                    e0 = hipt.event()
                    e1 = hipt.event()
                    hipt.record(e0)
                    launch(d, kind)
                    hipt.record(e1)
                    tr_ev.setdefault((d["name"], kind), []).append((e0, e1))
        torch.cuda.synchronize()
        del flush
        transposable = {"kernels": {}}
        for d in mats:
            e = d["R"] * d["K"]
            kept = e * n // m
            meta_t = d["K"] * ((d["R"] // m * n * meta_bits(m) + 31) // 32) * 4
            for kind in tr_kinds:
                t = float(np.mean([hipt.ms(a, b) for a, b in tr_ev[(d["name"], kind)]])) * 1e-3
                entry = {"us": round(t * 1e6, 2)}
                if kind == "spmm_t":
                    entry["eff_tflops"] = round(2.0 * e * d["T"] / t / 1e12, 1)
                    entry["alg_tflops"] = round(2.0 * kept * d["T"] / t / 1e12, 1)
                else:
                    ab = 2 * e * d["s"] if kind == "tprune" else e * d["s"] + kept * d["s"] + meta_t
                    entry.update(alg_bytes=ab, gbps=round(ab / t / 1e9, 1),
                                 frac_hbm=round(ab / t / 1e9 / PEAK_HBM_GBS, 3),
                                 frac_of_copy=round(ab / t / 1e9 / copy_rate["gbps"], 3))
                transposable["kernels"][f"{d['name']}.{kind}"] = entry

    # ---- channel permutation: one round of swap-gain evaluation per matrix ----
    # (compute-bound: pairs of column groups x rows x M^2 swaps, each two max and four adds)
    permutation = {"kernels": {}}
    valu = profiled_valu(args.workload)
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
        e0, e1 = hipt.event(), hipt.event()
        hipt.record(e0)
        for _ in range(reps):
            gains_launch()
        hipt.record(e1)
        torch.cuda.synchronize()
        t = hipt.ms(e0, e1) / reps * 1e-3
        evals = G * (G - 1) // 2 * d["R"] * m * m
        entry = {"ms": round(t * 1e3, 3), "pairs": G * (G - 1) // 2, "swap_row_evals": evals,
                 "swap_row_evals_per_s": round(evals / t / 1e9, 1)}
        # issued VALU instructions per launch, counted by rocprofv3 (SQ_INSTS_VALU) on the
        # same kernel and shape; each is 64 lane-operations
        insts = valu.get(d["name"])
        if insts is not None:
            lane_ops = insts * 64.0
            entry.update(valu_insts=insts, lane_tops=round(lane_ops / t / 1e12, 2),
                         frac_alu=round(lane_ops / t / 1e12 / PEAK_VALU_LANE_TOPS, 3))
        permutation["kernels"][f"{d['name']}.perm_gains"] = entry
        del ws, gain, pick
    vc = valu_ceiling(torch, dev, stream, hipt)
    permutation["roofline"] = {
        "bound": "alu", "unit": "T lane-op/s", "peak": PEAK_VALU_LANE_TOPS,
        "measured_ceiling": {k: vc[k] for k in ("v_add_f32", "v_max_f32", "v_fma_f32")},
        "note": "achieved = SQ_INSTS_VALU of the launch (committed rocprofv3 profile of the same "
                "kernel, shape and source) x 64 lanes / launch time; peak = the fp32 vector "
                "peak in lane operations (157.3 TFLOP/s / 2 flops per FMA); measured_ceiling = "
                "unpacked 32-bit VALU instructions alone in register loops (libnm_probe)"}

    cpu = None
    if not args.no_cpu:
        if float_path:
            srste["cpu_baseline"] = srste_cpu_sample(mats, n, m)
        model, visible = cpu_info()
        threads = max(1, min(16, visible))  # the host share of one GPU on the box is 16 cores
        cpu = cpu_baseline(mats, n, m, threads)
        cpu.update(cpu_model=model, cores_visible=visible,
                   one_core=cpu_one_core(mats, n, m))

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
        "matrix_core_ceiling": ceiling,
        "hbm_copy": copy_rate,
        "sweep_f16": sweep,
        "spmm_eff_tflops": round(F_eff / spmm_t / 1e12, 1),
        "mask_compress": mask_compress,
        "dense_gemm": dense,
        "kernels": kernels,
        "srste": srste,
        "transposable": transposable,
        "permutation": permutation,
        "context": "pages: up to 2x dense math throughput on A100 sparse Tensor Cores (not a target)",
    }
    hipt.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
