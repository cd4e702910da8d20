"""Benchmark of the block-scaled FP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-extra] [--calibrate-copy]

A step is one pass of the whole quantize/dequantize path over the
8192 x 8192 bf16 tensor ~ N(0, 0.02^2) (seed 0):
    NVFP4 quantize (tensor-amax kernel + quantize kernel),
    NVFP4 dequantize -> bf16,
    MXFP4 quantize, MXFP4 dequantize -> bf16.
The step is captured once as a HIP graph and replayed K times between two
HIP events (the timed region).  NVFP4 works on one copy of the input and
MXFP4 on another, so between two reads of the same input ~500 MB of other
traffic passes through the 256 MB MALL; nothing is flushed.  Inputs are
resident in HBM before timing.

Per-op rows (`breakdown`) time each entry point over a graph of 24
back-to-back launches cycling through three buffer sets (each set is evicted
from the MALL before it is reused), so they match the profiler's kernel
durations.

value = algorithmic bytes of the four ops per step / step time (GB/s).
Algorithmic bytes count every input byte once and every output byte once:
  quantize: 2 B per bf16 element in, 1/2 B codes + 1 B per block scale out
            (+ 4 B tensor scale for NVFP4); dequantize: the mirror.
The NVFP4 tensor-amax pass re-reads the input; that is implementation cost,
not algorithmic bytes.

One JSON line on stdout.  `roofline` is for the op with the largest launch
time in the breakdown, timed with HIP events on the stream it runs on (for
NVFP4 quantize that launch is the entry point's two kernels).
`cpu_baseline` is the CPU oracle (single thread) on one full step of the same
input.  `extra` reports the other workloads measured in the same run: MXFP4
quantize of the 16384 x 7168 activation, the 4096 x 14336 NVFP4 scale
search, and the 128 x 8192 x 8192 MXFP4 GEMM.
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import mxfp4_block_amax_amd as fp4  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP4_DENSE_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA, published
FP16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 MFMA, published
METRIC = "quantize GB/s (bytes in+out) and % of HBM peak; Gelem/s, NVFP4 & MXFP4"


# ---------------------------------------------------------------------------
# algorithmic byte accounting ("NVFP4 / MXFP4 format" page, section 8: T/2
# payload bytes, one byte per block, 4 bytes of tensor scale for NVFP4)
# ---------------------------------------------------------------------------
def fp4_bytes(elements: int, block: int, global_bytes: int) -> int:
    return elements // 2 + elements // block + global_bytes


def quantize_bytes(elements: int, in_bytes_per_elem: int, fmt: str) -> int:
    block, gb = (32, 0) if fmt == "mx" else (16, 4)
    return elements * in_bytes_per_elem + fp4_bytes(elements, block, gb)


def gemm_bytes(M: int, N: int, K: int, out_bytes: int = 2) -> int:
    return fp4_bytes(M * K, 32, 0) + fp4_bytes(N * K, 32, 0) + M * N * out_bytes


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


# ---------------------------------------------------------------------------
# measured HBM traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated against a
# device copy of known size), valid only for the kernel sources it was taken on
# ---------------------------------------------------------------------------
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "roundtrip_8192x8192_bf16_hbm_traffic.md")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "mxfp4_block_amax_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """Per-launch HBM bytes by entry point, or None if the kernels changed."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            for line in f:
                if line.startswith("traffic_record:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("source_sha256_16") == kernel_source_hash():
                        return rec["per_launch_bytes"]
    except (OSError, ValueError, KeyError):
        pass
    return None


VALU_PROFILE = os.path.join(ROOT, "profiles", "valu_issue_arithmetic_kernels.md")


def measured_valu_issue():
    """VALU issue of the arithmetic-bound kernels (percent of one wave64
    instruction per SIMD every two cycles at 2.4 GHz), by extra-workload
    name, from the committed SQ-counter profile; None if the kernels changed."""
    try:
        with open(VALU_PROFILE) as f:
            for line in f:
                if line.startswith("valu_record:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("source_sha256_16") == kernel_source_hash():
                        return rec["pct_of_peak"]
    except (OSError, ValueError, KeyError):
        pass
    return None


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
def capture(fn) -> "torch.cuda.CUDAGraph":
    """A HIP graph of fn()'s launches (the library's kernels record no memset
    nodes; every buffer is preallocated)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps: int) -> float:
    """Mean milliseconds per replay, HIP events on the replay stream."""
    g.replay()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def time_rotating(fns, launches: int = 24, reps: int = 5) -> float:
    """Mean milliseconds per launch of an op over `launches` back-to-back
    launches that cycle through the given buffer sets (each fn is the op on
    one set; enough sets that a set is evicted from the 256 MB MALL before it
    is used again), captured in one graph."""
    def run():
        for i in range(launches):
            fns[i % len(fns)]()
    return time_graph(capture(run), reps) / launches


# ---------------------------------------------------------------------------
# the step
# ---------------------------------------------------------------------------
NSETS = 3  # buffer sets rotated by the per-op timing


class RoundTrip:
    """Buffers for NVFP4 + MXFP4 quantize/dequantize of one [R, C] tensor,
    NSETS copies of everything."""

    def __init__(self, x_cpu: torch.Tensor):
        R, C = x_cpu.shape
        dev = torch.device("cuda")
        self.shape = (R, C)
        self.sets = []
        for _ in range(NSETS):
            b = {
                "x": x_cpu.to(dev),
                "nv": (torch.empty(R, C // 2, dtype=torch.uint8, device=dev),
                       torch.empty(R, C // 16, dtype=torch.uint8, device=dev),
                       torch.empty(1, dtype=torch.float32, device=dev)),
                "mx": (torch.empty(R, C // 2, dtype=torch.uint8, device=dev),
                       torch.empty(R, C // 32, dtype=torch.uint8, device=dev)),
                "y_nv": torch.empty(R, C, dtype=torch.bfloat16, device=dev),
                "y_mx": torch.empty(R, C, dtype=torch.bfloat16, device=dev),
                "ws": fp4.new_workspace(R, C, dev),
                "status": torch.zeros(1, dtype=torch.int32, device=dev),
            }
            self.sets.append(b)
        n = R * C
        self.elements = n
        self.bytes = {
            "nvfp4_quantize": quantize_bytes(n, 2, "nv"),
            "nvfp4_dequantize": quantize_bytes(n, 2, "nv"),
            "mxfp4_quantize": quantize_bytes(n, 2, "mx"),
            "mxfp4_dequantize": quantize_bytes(n, 2, "mx"),
        }

    def op(self, tag, i):
        b = self.sets[i]
        if tag == "nvfp4_quantize":
            return lambda: fp4.quantize_nvfp4(b["x"], check=False, out=b["nv"], status=b["status"],
                                              workspace=b["ws"])
        if tag == "nvfp4_dequantize":
            return lambda: fp4.dequantize(fp4.NVFP4, b["nv"][0], b["nv"][1], b["nv"][2], out=b["y_nv"])
        if tag == "mxfp4_quantize":
            return lambda: fp4.quantize_mxfp4(b["x"], check=False, out=b["mx"], status=b["status"])
        if tag == "mxfp4_dequantize":
            return lambda: fp4.dequantize(fp4.MXFP4, b["mx"][0], b["mx"][1], None, out=b["y_mx"])
        raise KeyError(tag)

    def step(self):
        # NVFP4 on set 0's input, MXFP4 on set 1's: between two reads of the
        # same input ~500 MB of other traffic passes through the MALL
        self.op("nvfp4_quantize", 0)()
        self.op("nvfp4_dequantize", 0)()
        self.op("mxfp4_quantize", 1)()
        self.op("mxfp4_dequantize", 1)()


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_cpu: torch.Tensor, step_bytes: int):
    """The oracle (plain C) on one full step of the same input, its rows split
    over the host's threads (at most 16); the C calls release the GIL.  The
    NVFP4 tensor scale is the largest of the slices' (it is monotone in the
    amax)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    xo = workloads.bf16_bits(x_cpu).reshape(x_cpu.shape[0], -1)
    nt = max(1, min(16, len(os.sched_getaffinity(0))))
    parts = [p.reshape(-1) for p in np.array_split(xo, nt) if p.size]
    def one_step(pool):
        sgs = list(pool.map(oracle.nv_global_scale, parts))
        sg = max(v for v, _ in sgs)

        def nv(part):
            p, s, _ = oracle.nv_quantize_with_scale(part, sg)
            oracle.dequantize(oracle.NV, p, s, sg, out_bf16=True)

        def mx(part):
            p, s, _ = oracle.mx_quantize(part)
            oracle.dequantize(oracle.MX, p, s, out_bf16=True)
        list(pool.map(nv, parts))
        list(pool.map(mx, parts))

    # whole steps until the threads have done at least ~10 s of CPU work (at
    # most 8 steps)
    steps = 0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(nt) as pool:
        while True:
            one_step(pool)
            steps += 1
            dt = time.perf_counter() - t0
            if dt * len(parts) >= 10.0 or steps >= 8:
                break
    return {"value": round(steps * step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": len(parts),
            "kind": "oracle", "cpu": _cpu_model(),
            "sample": f"{steps} full step(s) (NVFP4 + MXFP4 quantize and dequantize) of the "
                      f"{x_cpu.shape[0]}x{x_cpu.shape[1]} bf16 input, rows split over "
                      f"{len(parts)} threads; {dt:.2f} s wall"}


def _rate(b: int, ms: float, elements: int = None):
    d = {"us": round(ms * 1e3, 2), "GB/s": round(b / ms / 1e6, 1),
         "pct_hbm_peak": round(100 * b / ms / 1e6 / HBM_PEAK_GBS, 1)}
    if elements:
        d["Gelem/s"] = round(elements / ms / 1e6, 1)
    return d


def extra_workloads():
    out = {}
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    # NVFP4 quantize of the same-shape weight with seed 1: amax 235 * 2^-11,
    # a generic tensor scale, so the one-pass kernel takes the
    # reciprocal-correction divide (seed 0's amax is 21 * 11 * 2^-11)
    xw_cpu = workloads.nvfp4_weight(8192, 8192, seed=1)
    xs = [xw_cpu.cuda() for _ in range(3)]
    outs = [fp4.quantize_nvfp4(x) for x in xs]
    wss = [fp4.new_workspace(8192, 8192, "cuda") for _ in range(3)]
    ms = time_rotating([lambda x=x, o=o, w=w: fp4.quantize_nvfp4(x, check=False, out=o, status=st,
                                                                 workspace=w)
                        for x, o, w in zip(xs, outs, wss)])
    out["nvfp4_quantize_8192x8192_bf16_seed1"] = _rate(quantize_bytes(xw_cpu.numel(), 2, "nv"), ms,
                                                      xw_cpu.numel())
    del xs, outs, wss
    # MXFP4 activation quantize, 16384 x 7168 bf16: two 235 MB input copies
    xa_cpu = workloads.mxfp4_activation()
    xs = [xa_cpu.cuda() for _ in range(2)]
    outs = [fp4.quantize_mxfp4(x) for x in xs]
    ms = time_rotating([lambda x=x, o=o: fp4.quantize_mxfp4(x, check=False, out=o, status=st)
                        for x, o in zip(xs, outs)])
    out["mxfp4_activation_quantize_16384x7168_bf16"] = _rate(quantize_bytes(xa_cpu.numel(), 2, "mx"),
                                                             ms, xa_cpu.numel())
    del xs, outs
    # NVFP4 MSE scale search, 4096 x 14336 bf16 ~ Laplace(0, 0.01), 64 candidates
    xs_cpu = workloads.scale_search_input()
    xs = [xs_cpu.cuda() for _ in range(3)]
    res = [fp4.scale_search(x) for x in xs]
    ws = fp4.new_workspace(*xs_cpu.shape, "cuda")
    ms = time_rotating([lambda x=x, r=r: fp4.scale_search(x, check=False, out=r, status=st, workspace=ws)
                        for x, r in zip(xs, res)], launches=6)
    d = _rate(quantize_bytes(xs_cpu.numel(), 2, "nv"), ms, xs_cpu.numel())
    d["candidate_element_evals_per_s"] = f"{xs_cpu.numel() * 64 / ms / 1e-3:.3e}"
    out["nvfp4_scale_search_4096x14336_bf16"] = d
    # the same search over c in [0.5, 1.5] (amax may map to 4), and over every
    # E4M3 code
    ms = time_rotating([lambda x=x, r=r: fp4.scale_search(x, 64, 0.5, 1.5, check=False, out=r,
                                                          status=st, workspace=ws)
                        for x, r in zip(xs, res)], launches=6)
    out["nvfp4_scale_search_c0.5-1.5_4096x14336_bf16"] = _rate(
        quantize_bytes(xs_cpu.numel(), 2, "nv"), ms, xs_cpu.numel())
    ms = time_rotating([lambda x=x, r=r: fp4.scale_search_exhaustive(x, check=False, out=r,
                                                                     status=st, workspace=ws)
                        for x, r in zip(xs, res)], launches=3, reps=3)
    d = _rate(quantize_bytes(xs_cpu.numel(), 2, "nv"), ms, xs_cpu.numel())
    d["candidate_element_evals_per_s"] = f"{xs_cpu.numel() * 126 / ms / 1e-3:.3e}"
    out["nvfp4_scale_search_all_codes_4096x14336_bf16"] = d
    del xs, res
    # MXFP4 quantize of the 8192 x 8192 weight under the ceil rule and the
    # three-exponent squared-error search
    xw_cpu = workloads.nvfp4_weight()
    xs = [xw_cpu.cuda() for _ in range(3)]
    outs = [fp4.quantize_mxfp4(x) for x in xs]
    for rule in ("ceil", "mse"):
        ms = time_rotating([lambda x=x, o=o, rule=rule: fp4.quantize_mxfp4_rule(x, rule, check=False, out=o,
                                                                    status=st)
                            for x, o in zip(xs, outs)])
        out[f"mxfp4_quantize_rule_{rule}_8192x8192_bf16"] = _rate(
            quantize_bytes(xw_cpu.numel(), 2, "mx"), ms, xw_cpu.numel())
    # stochastic rounding of the same weight: MXFP4 (one pass) and NVFP4
    # (tensor amax, then quantize)
    ms = time_rotating([lambda x=x, o=o: fp4.quantize_sr(fp4.MXFP4, x, 0x5EED, check=False, out=o,
                                                         status=st)
                        for x, o in zip(xs, outs)])
    out["mxfp4_quantize_stochastic_8192x8192_bf16"] = _rate(
        quantize_bytes(xw_cpu.numel(), 2, "mx"), ms, xw_cpu.numel())
    nouts = [fp4.quantize_nvfp4(x) for x in xs]
    wss = [fp4.new_workspace(8192, 8192, "cuda") for _ in range(3)]
    ms = time_rotating([lambda x=x, o=o, w=w: fp4.quantize_sr(fp4.NVFP4, x, 0x5EED, check=False,
                                                              out=o, status=st, workspace=w)
                        for x, o, w in zip(xs, nouts, wss)])
    out["nvfp4_quantize_stochastic_8192x8192_bf16"] = _rate(
        quantize_bytes(xw_cpu.numel(), 2, "nv"), ms, xw_cpu.numel())
    del xs, outs, nouts, wss
    # MXFP4 GEMM 128 x 8192 x 8192: operands quantized on the GPU; eight
    # copies of B (36 MB each) rotate so B comes from HBM
    M, N, K = 128, 8192, 8192
    a, bt = workloads.gemm_operands(M, N, K)
    ac, asc = fp4.quantize_mxfp4(a.cuda())
    bq = [fp4.quantize_mxfp4(bt.cuda()) for _ in range(8)]
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    ms = time_rotating([lambda b=b: fp4.gemm_mxfp4(ac, asc, b[0], b[1], out=c) for b in bq])
    d = _rate(gemm_bytes(M, N, K), ms)
    tf = gemm_flops(M, N, K) / ms / 1e9
    d.update({"TFLOP/s": round(tf, 1), "pct_fp4_mfma_peak": round(100 * tf / FP4_DENSE_PEAK_TFLOPS, 2)})
    # the same product split over K (fp32 partials in a workspace, then a
    # fixed-order reduction)
    ws = torch.empty(fp4.gemm_splitk_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    ms2 = time_rotating([lambda b=b: fp4.gemm_mxfp4_splitk(ac, asc, b[0], b[1], out=c, workspace=ws)
                         for b in bq])
    d["split_k_us"] = round(ms2 * 1e3, 2)
    out["mxfp4_gemm_128x8192x8192_bf16out"] = d
    # the same product on packed operands (MFMA operand order): B packed once
    # (a weight), A packed per call (pack_a_us, timed on its own)
    bps = [fp4.pack_mxfp4_operand(*b) for b in bq]
    pa = fp4.pack_mxfp4_operand(ac, asc)
    ms = time_rotating([lambda b=b: fp4.gemm_mxfp4_packed(pa, b, M, N, K, out=c) for b in bps])
    d = _rate(gemm_bytes(M, N, K), ms)
    tf = gemm_flops(M, N, K) / ms / 1e9
    d.update({"TFLOP/s": round(tf, 1), "pct_fp4_mfma_peak": round(100 * tf / FP4_DENSE_PEAK_TFLOPS, 2)})
    ms2 = time_rotating([lambda: fp4.pack_mxfp4_operand(ac, asc, out=pa)])
    d["pack_a_us"] = round(ms2 * 1e3, 2)
    out["mxfp4_gemm_packed_128x8192x8192_bf16out"] = d
    del bps
    # K = 16384, beyond the staged kernel's scale capacity: the split-K path
    # against the entry point's register-fed fallback
    K2 = 16384
    a2, bt2 = workloads.gemm_operands(M, N, K2)
    ac2, asc2 = fp4.quantize_mxfp4(a2.cuda())
    bq2 = [fp4.quantize_mxfp4(bt2.cuda()) for _ in range(4)]
    ws2 = torch.empty(fp4.gemm_splitk_workspace_bytes(M, N, K2), dtype=torch.uint8, device="cuda")
    ms = time_rotating([lambda b=b: fp4.gemm_mxfp4_splitk(ac2, asc2, b[0], b[1], out=c, workspace=ws2)
                        for b in bq2])
    d = _rate(gemm_bytes(M, N, K2), ms)
    tf = gemm_flops(M, N, K2) / ms / 1e9
    d.update({"TFLOP/s": round(tf, 1), "pct_fp4_mfma_peak": round(100 * tf / FP4_DENSE_PEAK_TFLOPS, 2)})
    ms2 = time_rotating([lambda b=b: fp4.gemm_mxfp4(ac2, asc2, b[0], b[1], out=c) for b in bq2])
    d["unsplit_us"] = round(ms2 * 1e3, 2)
    out["mxfp4_gemm_splitk_128x8192x16384_bf16out"] = d
    del bq2, ws2
    # W4A4 linear: bf16 activations quantized in the GEMM's launch (grid
    # barrier), against the two launches of quantize then GEMM
    xa = a.to(torch.bfloat16).cuda()
    ws = fp4.new_workspace(M, K, "cuda")
    aq = (torch.empty(M, K // 2, dtype=torch.uint8, device="cuda"),
          torch.empty(M, K // 32, dtype=torch.uint8, device="cuda"))
    ms = time_rotating([lambda b=b: fp4.linear_mxfp4(xa, b[0], b[1], out=c, a_out=aq, status=st,
                                                     workspace=ws, check=False) for b in bq])
    lin_bytes = (M * K * 2 + M * K // 2 + M * K // 32 + N * K // 2 + N * K // 32 + M * N * 2)
    d = _rate(lin_bytes, ms)
    ms2 = time_rotating([lambda b=b: fp4.linear_mxfp4(xa, b[0], b[1], out=c, a_out=aq, status=st,
                                                      workspace=ws, check=False, one_launch=False)
                         for b in bq])
    d["two_launches_us"] = round(ms2 * 1e3, 2)
    out["mxfp4_linear_w4a4_128x8192x8192_bf16"] = d
    # the same linear on a packed weight: activations quantized straight into
    # the packed layout, then the packed GEMM (two launches)
    bps = [fp4.pack_mxfp4_operand(*b) for b in bq]
    apk = torch.empty(fp4.packed_operand_bytes(M, K), dtype=torch.uint8, device="cuda")
    ms = time_rotating([lambda b=b: fp4.linear_mxfp4_packed(xa, b, N, out=c, a_out=apk, status=st,
                                                            check=False) for b in bps])
    out["mxfp4_linear_w4a4_packed_128x8192x8192_bf16"] = _rate(lin_bytes, ms)
    del bps
    # NVFP4 x NVFP4 GEMM, same shape: operands NVFP4-quantized on the GPU,
    # eight copies of B rotate
    an = fp4.quantize_nvfp4(a.cuda())
    bn = [fp4.quantize_nvfp4(bt.cuda()) for _ in range(8)]
    ms = time_rotating([lambda b=b: fp4.gemm_nvfp4(an[0], an[1], an[2], b[0], b[1], b[2], out=c)
                        for b in bn])
    nv_bytes = M * K // 2 + M * K // 16 + N * K // 2 + N * K // 16 + 8 + M * N * 2
    d = _rate(nv_bytes, ms)
    tf = gemm_flops(M, N, K) / ms / 1e9
    d.update({"TFLOP/s": round(tf, 1),
              "pct_fp16_mfma_peak": round(100 * tf / FP16_DENSE_PEAK_TFLOPS, 2)})
    out["nvfp4_gemm_128x8192x8192_bf16out"] = d
    # the same product on packed NVFP4 operands (each B packed once)
    bnp = [fp4.pack_nvfp4_operand(b[0], b[1]) for b in bn]
    anp = fp4.pack_nvfp4_operand(an[0], an[1])
    ms = time_rotating([lambda b=b, bb=bb: fp4.gemm_nvfp4_packed(anp, an[2], bb, b[2], M, N, K, out=c)
                        for b, bb in zip(bn, bnp)])
    d = _rate(nv_bytes, ms)
    tf = gemm_flops(M, N, K) / ms / 1e9
    d.update({"TFLOP/s": round(tf, 1),
              "pct_fp16_mfma_peak": round(100 * tf / FP16_DENSE_PEAK_TFLOPS, 2)})
    ms2 = time_rotating([lambda: fp4.pack_nvfp4_operand(an[0], an[1], out=anp)])
    d["pack_a_us"] = round(ms2 * 1e3, 2)
    out["nvfp4_gemm_packed_128x8192x8192_bf16out"] = d
    # NVFP4 W4A4 linear on a packed weight: bf16 activations quantized
    # straight into the packed layout (amax pass, encode), then the packed GEMM
    wsn = fp4.new_workspace(M, K, "cuda")
    apn = (torch.empty(fp4.nv_packed_operand_bytes(M, K), dtype=torch.uint8, device="cuda"),
           torch.empty(1, dtype=torch.float32, device="cuda"))
    ms = time_rotating([lambda b=b, bb=bb: fp4.linear_nvfp4_packed(xa, bb, b[2], N, out=c, a_out=apn,
                                                                   status=st, workspace=wsn,
                                                                   check=False)
                        for b, bb in zip(bn, bnp)])
    nv_lin_bytes = (M * K * 2 + M * K // 2 + M * K // 16 + N * K // 2 + N * K // 16 + M * N * 2)
    out["nvfp4_linear_w4a4_packed_128x8192x8192_bf16"] = _rate(nv_lin_bytes, ms)
    del bnp
    if int(st.item()) != 0:
        raise RuntimeError(f"a timed call raised status flags {int(st.item())}")
    # arithmetic-bound workloads: their profiled VALU issue (SQ counters)
    valu = measured_valu_issue()
    if valu:
        for k, pct in valu.items():
            if k in out:
                out[k]["valu_issue_pct_of_peak_profiled"] = pct
    return out


def calibrate_copy(iters: int = 5):
    """A plain device copy of known size, for scaling HBM byte counters."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(iters):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read": n, "bytes_written": n, "iters": iters}


def copy_ceiling(iters: int = 20):
    """Measured device-to-device copy rate (bytes read + written per second)
    of a 256 MiB buffer, alternating two source/destination pairs so that
    neither is served from the 256 MB MALL: a practical HBM ceiling beside
    the published peak."""
    n = 256 << 20
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i) for i in range(4)]
    for i in range(2):
        bufs[2 * i + 1].copy_(bufs[2 * i])
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(iters):
        bufs[2 * (i & 1) + 1].copy_(bufs[2 * (i & 1)])
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / iters
    gbs = 2 * n / (ms * 1e-3) / 1e9
    return {"GB/s": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
            "method": "torch copy_ of 256 MiB, two buffer pairs alternating, HIP events; "
                      "bytes read + written"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the quantize path runs on one device and this "
              "build launches no multi-GPU work; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)

    x_cpu = workloads.nvfp4_weight()
    rt = RoundTrip(x_cpu)
    step_bytes = sum(rt.bytes.values())

    # correctness gate on the benchmark's own buffers before timing
    for i in range(NSETS):
        b = rt.sets[i]
        fp4.quantize_nvfp4(b["x"], out=b["nv"], workspace=b["ws"])
        fp4.quantize_mxfp4(b["x"], out=b["mx"])

    # the timed region: K replays of the graph-captured step
    step_graph = capture(rt.step)
    for _ in range(args.warmup):
        step_graph.replay()
    torch.cuda.synchronize()
    s_ev = torch.cuda.Event(enable_timing=True)
    e_ev = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s_ev.record()
    for _ in range(args.steps):
        step_graph.replay()
    e_ev.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    ms_per_step = max(wall_s * 1e3, s_ev.elapsed_time(e_ev)) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # per-op launch durations: back-to-back launches rotating NSETS buffer sets
    breakdown = {}
    for tag in rt.bytes:
        ms = time_rotating([rt.op(tag, i) for i in range(NSETS)])
        breakdown[tag] = _rate(rt.bytes[tag], ms, rt.elements)
        breakdown[tag]["bytes"] = rt.bytes[tag]

    # every call of the timed region reported its conditions here
    for b in rt.sets:
        if int(b["status"].item()) != 0:
            raise RuntimeError(f"a timed call raised status flags {int(b['status'].item())}")

    dom = max(breakdown, key=lambda t: breakdown[t]["us"])
    kernel_names = {"nvfp4_quantize": "nv_resident_kernel<64, exact> (one pass, tensor held on chip; "
                                      "this tensor's s_g = 11 * 2^-18 takes the two-operation divide)",
                    "nvfp4_dequantize": "dequant_kernel<1, bf16 out>",
                    "mxfp4_quantize": "mx_quantize_kernel<bf16 in>",
                    "mxfp4_dequantize": "dequant_kernel<0, bf16 out>"}
    traffic = measured_traffic()
    roofline = {"bound": "hbm", "kernel": kernel_names[dom],
                "achieved": breakdown[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(breakdown[dom]["GB/s"] / HBM_PEAK_GBS, 4),
                "traffic": traffic[dom] if traffic else None,
                "algorithmic_bytes_per_launch": rt.bytes[dom],
                "avg_launch_us": breakdown[dom]["us"]}
    if traffic:
        roofline["traffic_GB/s"] = round(traffic[dom] / (breakdown[dom]["us"] * 1e3), 1)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "nvfp4_mxfp4_roundtrip_8192x8192_bf16",
                   "shape": [8192, 8192], "input": "bf16 N(0, 0.02^2), seed 0",
                   "ops": list(rt.bytes), "step_bytes": step_bytes,
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
                   "Gelem/s_per_op": round(4 * rt.elements / (ms_per_step * 1e-3) / 1e9, 1),
                   "timing": "HIP graph of one step replayed K times; per-op rows from graphs "
                             "of back-to-back launches over 3 rotating buffer sets"},
        "breakdown": breakdown,
        "roofline": roofline,
        "copy_ceiling": copy_ceiling(),
    }
    if not args.no_extra:
        line["extra"] = extra_workloads()
    if args.calibrate_copy:
        line["copy_calibration"] = calibrate_copy()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x_cpu, step_bytes)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
