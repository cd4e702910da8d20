"""Per-phase timeline of the one-pass NVFP4 quantize (a profiling aid).

Loads libfp4_phase.so (build it first: python -m mxfp4_block_amax_amd.build
--phase-clock), runs the one-pass quantize on an 8192 x 8192 bf16 weight
(workloads.nvfp4_weight) several times, and prints, over the calls after the
first two, the phase boundaries of every workgroup relative to the earliest
workgroup start of its call (the device's 100 MHz constant clock, 10 ns
steps): the minimum, median and maximum over workgroups, averaged over calls;
the phases' per-workgroup durations; whether the load phase's spread stays
with the workgroups from call to call, and its median per XCD.  Then the
mean duration of one call, from HIP events around a graph of 24
back-to-back launches on three buffer sets.

    python -m mxfp4_block_amax_amd.phase_timeline [--seed S] [--calls N] [--lib PATH]
"""
import argparse
import ctypes
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import mxfp4_block_amax_amd as fp4  # noqa: E402
import workloads  # noqa: E402

# slot of each stamp in a workgroup's row, in the order the kernel passes them
PHASES = [("start", 0), ("loaded", 1), ("barrier seen", 7), ("barrier", 2), ("s_g, window", 5),
          ("table per code", 6), ("table", 3), ("done", 4)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--calls", type=int, default=12)
    ap.add_argument("--lib", default=os.path.join(HERE, "libfp4_phase.so"),
                    help="a build of the library with the phase clock")
    args = ap.parse_args()
    lib_path = args.lib
    if not os.path.exists(lib_path):
        raise SystemExit(f"{lib_path} is not built: python -m mxfp4_block_amax_amd.build --phase-clock")
    fp4.LIB_PATH = lib_path
    L = fp4.lib()
    L.fp4_debug_phase_clock.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.fp4_debug_phase_clock.restype = ctypes.c_int

    x = workloads.nvfp4_weight(seed=args.seed)
    xs = [x.cuda() for _ in range(3)]
    outs = [fp4.quantize_nvfp4(t) for t in xs]
    wss = [fp4.new_workspace(*x.shape, "cuda") for _ in range(3)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rel = []
    for it in range(args.calls):
        i = it % 3
        fp4.quantize_nvfp4(xs[i], check=False, out=outs[i], workspace=wss[i])
        torch.cuda.synchronize()
        buf = np.zeros(cus * 8, np.uint64)
        if L.fp4_debug_phase_clock(buf.ctypes.data, buf.size) != 0:
            raise SystemExit("reading the phase clock failed")
        t = buf.reshape(cus, 8)[:, [slot for _, slot in PHASES]].astype(np.int64)
        if it >= 2:
            rel.append((t - t[:, 0].min()) * 10 / 1000.0)  # us
    r = np.stack(rel)  # [call, workgroup, stamp]

    def run():
        for k in range(24):
            i = k % 3
            fp4.quantize_nvfp4(xs[i], check=False, out=outs[i], workspace=wss[i])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(5):
        g.replay()
    e.record()
    torch.cuda.synchronize()

    print(f"one-pass NVFP4 quantize, 8192 x 8192 bf16 (seed {args.seed}), {cus} workgroups, "
          f"{r.shape[0]} calls")
    print("| boundary | min us | median us | max us |")
    print("|---|---|---|---|")
    for k, (name, _) in enumerate(PHASES):
        v = r[:, :, k]
        print(f"| {name} | {v.min(axis=1).mean():.2f} | {np.median(v, axis=1).mean():.2f} | "
              f"{v.max(axis=1).mean():.2f} |")
    print("| per workgroup | median us | max us | |")
    for k in range(len(PHASES) - 1):
        d = r[:, :, k + 1] - r[:, :, k]
        name = f"{PHASES[k][0]} -> {PHASES[k + 1][0]}"
        print(f"| {name} | {np.median(d):.2f} | {d.max(axis=1).mean():.2f} | |")
    # Is the spread of the load phase a property of the workgroup (the same
    # ones slow on every call) or of the call?  Workgroup w runs on XCD w % 8.
    load = r[:, :, 1] - r[:, :, 0]
    end = r[:, :, 1]
    cc = [np.corrcoef(end[i], end[i + 1])[0, 1] for i in range(end.shape[0] - 1)]
    print(f"loads end, correlation over workgroups between consecutive calls: "
          f"{np.mean(cc):.2f} (1: the same workgroups late every call)")
    xcd = np.arange(r.shape[1]) % 8
    print("| XCD | median loads end us | max loads end us | median load us |")
    print("|---|---|---|---|")
    for x in range(8):
        ex = end[:, xcd == x]
        print(f"| {x} | {np.median(ex):.2f} | {ex.max(axis=1).mean():.2f} | "
              f"{np.median(load[:, xcd == x]):.2f} |")
    print(f"call duration (events, 24-launch graph): {s.elapsed_time(e) / 120 * 1000:.2f} us")


if __name__ == "__main__":
    main()
