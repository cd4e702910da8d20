"""Helpers for the GPU parity tests: move seeded inputs to the device, hand
the same bytes to the oracle, and announce each case before its GPU step."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import workloads


def announce(msg: str):
    """Name the case about to run on the GPU (flushed, so a fault names it)."""
    print(f"[gpu case] {msg}", file=sys.stderr, flush=True)


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().to("cuda")


def oracle_view(t: torch.Tensor) -> np.ndarray:
    """The tensor's bytes in the oracle's input form (float32 or bf16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return workloads.bf16_bits(t).reshape(-1)
    assert t.dtype == torch.float32
    return t.numpy().reshape(-1)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().reshape(-1)


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got).reshape(-1)
    want = np.asarray(want).reshape(-1)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)[0]
    if bad.size:
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} of {got.size} differ; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")


def assert_float_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    """Bit-exact, except that any NaN matches any NaN (payloads are free)."""
    g = np.asarray(got)
    w = np.asarray(want)
    if g.dtype == np.uint16:  # bf16 bit patterns
        gn = (g & 0x7FFF) > 0x7F80
        wn = (w & 0x7FFF) > 0x7F80
    else:
        gn, wn = np.isnan(g), np.isnan(w)
        g, w = f32_bits(g), f32_bits(w)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    assert_bytes_equal(np.where(gn, 0, g), np.where(wn, 0, w), what)


def oracle_threads() -> int:
    """Host threads for splitting an oracle call (at most 16: the GPU host's
    CPU share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_split(fn, x: np.ndarray, unit: int, nparts: int = None):
    """fn over contiguous slices of the flat array x, each a multiple of
    `unit` elements (whole blocks), run on host threads (the oracle's C calls
    release the GIL); returns the per-slice results in order."""
    n = x.size
    assert n % unit == 0
    nparts = nparts or 4 * oracle_threads()
    per = max(1, (n // unit + nparts - 1) // nparts) * unit
    parts = [x[i:i + per] for i in range(0, n, per)]
    with ThreadPoolExecutor(oracle_threads()) as pool:
        return list(pool.map(fn, parts))
