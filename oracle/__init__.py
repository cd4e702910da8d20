"""CPU oracle for block-scaled FP4 quantization (MXFP4 / NVFP4).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``mxfp4_block_amax_amd``) never imports it, and it imports nothing from
the product path; the two share only the seeded input generators in
``workloads``.

The arithmetic lives in ``fp4_oracle.c`` (plain C, one definition per step,
each citing the page it follows); this module marshals numpy arrays into it.
The block-scaled GEMM reference is in ``oracle.gemm``.

bf16 tensors are passed as their uint16 bit patterns (numpy has no bf16).
"""
import ctypes
import os

import numpy as np

from . import build as _build

FLAG_NONFINITE = 1
FLAG_SCALE_UNDERFLOW = 2
DT_F32 = 0
DT_BF16 = 1
MX = 0
NV = 1

_lib = None


def lib():
    """Load liboracle.so, compiling it first if it is missing or stale."""
    global _lib
    if _lib is not None:
        return _lib
    if (not os.path.exists(_build.LIB)
            or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    P, I64, I, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    sig = {
        "or_e2m1_value": (D, [I]),
        "or_e2m1_round": (I, [F]),
        "or_e2m1_round_array": (None, [P, I64, P]),
        "or_pack": (None, [P, I64, P]),
        "or_unpack": (None, [P, I64, P]),
        "or_e4m3_value": (D, [I]),
        "or_e4m3_nearest": (I, [D, D]),
        "or_f32_to_bf16": (ctypes.c_uint16, [F]),
        "or_mx_exponent": (I, [D]),
        "or_mx_quantize": (I, [P, I, I64, P, P]),
        "or_mx_exponent_ceil": (I, [D]),
        "or_block_loss32_pow2": (F, [P, I]),
        "or_mx_quantize_rule": (I, [P, I, I64, I, P, P]),
        "or_scale_search_all": (I, [P, I, I64, F, P, P, P]),
        "or_padded_storage_bytes": (I64, [I64, I64, I, I64]),
        "or_mx_quantize_padded": (I, [P, I, I64, I64, P, P]),
        "or_nv_quantize_padded": (I, [P, I, I64, I64, P, P, P]),
        "or_dequantize_padded": (I, [I, P, P, F, I64, I64, I, P]),
        "or_nv_global_scale": (I, [P, I, I64, P]),
        "or_nv_quantize": (I, [P, I, I64, F, P, P]),
        "or_dequantize": (None, [I, P, P, F, I64, I, P]),
        "or_block_loss_f32": (F, [P, F]),
        "or_candidate_c": (F, [I, I, F, F]),
        "or_scale_search": (I, [P, I, I64, F, I, F, F, P, P, P]),
        "or_ideal_roundtrip": (None, [P, I64, I, P]),
        "or_ideal_code": (I, [F, F]),
        "or_storage_bytes": (I64, [I64, I, I64]),
        "or_sr_bits": (ctypes.c_uint32, [ctypes.c_uint64, I64]),
        "or_e2m1_round_sr": (I, [F, ctypes.c_uint32]),
        "or_mx_quantize_sr": (I, [P, I, I64, ctypes.c_uint64, P, P]),
        "or_nv_quantize_sr": (I, [P, I, I64, F, ctypes.c_uint64, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x: np.ndarray):
    """Return (contiguous array, dtype code).  float32 or uint16 (bf16 bits)."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, DT_F32
    if x.dtype == np.uint16:
        return x, DT_BF16
    raise TypeError(f"oracle input must be float32 or uint16 (bf16 bits), got {x.dtype}")


# ---- scalar definitions ---------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().or_e2m1_value(int(code))


def e2m1_round(q: float) -> int:
    """Code of RoundE2M1(q) for an fp32 value q (-1 if q is not finite)."""
    return lib().or_e2m1_round(float(np.float32(q)))


def e2m1_round_array(q: np.ndarray) -> np.ndarray:
    """RoundE2M1 codes of an fp32 array (255 where the input is not finite)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(q.size, np.uint8)
    lib().or_e2m1_round_array(_ptr(q), q.size, _ptr(out))
    return out.reshape(q.shape)


def e4m3_value(code: int) -> float:
    return lib().or_e4m3_value(int(code))


def e4m3_nearest(num: float, den: float) -> int:
    return lib().or_e4m3_nearest(float(num), float(den))


def f32_to_bf16_bits(v: float) -> int:
    return lib().or_f32_to_bf16(float(np.float32(v)))


def mx_exponent(amax: float) -> int:
    return lib().or_mx_exponent(float(amax))


def candidate_c(k: int, n: int = 64, c_lo: float = 0.5, c_hi: float = 1.0) -> float:
    return lib().or_candidate_c(k, n, float(np.float32(c_lo)), float(np.float32(c_hi)))


def block_loss(xb: np.ndarray, alpha: float) -> float:
    xb = np.ascontiguousarray(xb, dtype=np.float32)
    assert xb.size == 16
    return lib().or_block_loss_f32(_ptr(xb), float(np.float32(alpha)))


def storage_bytes(elements: int, block: int, global_bytes: int) -> int:
    return lib().or_storage_bytes(elements, block, global_bytes)


def padded_storage_bytes(rows: int, cols: int, block: int, global_bytes: int) -> int:
    return lib().or_padded_storage_bytes(rows, cols, block, global_bytes)


def _padded_cols(cols: int, block: int) -> int:
    return (cols + block - 1) // block * block


def mx_quantize_padded(x: np.ndarray, rows: int, cols: int):
    """MXFP4 quantize of a [rows, cols] matrix, rows zero-padded to whole
    blocks.  Returns (packed [rows * pc / 2], scales [rows * pc / 32], flags)."""
    x, dt = _as_input(x)
    assert x.size == rows * cols
    pc = _padded_cols(cols, 32)
    packed = np.empty(rows * pc // 2, np.uint8)
    scales = np.empty(rows * pc // 32, np.uint8)
    flags = lib().or_mx_quantize_padded(_ptr(x), dt, rows, cols, _ptr(packed), _ptr(scales))
    assert flags >= 0
    return packed, scales, flags


def nv_quantize_padded(x: np.ndarray, rows: int, cols: int):
    """NVFP4 quantize, rows zero-padded to whole 16-blocks.  Returns
    (packed, scales, s_g, flags)."""
    x, dt = _as_input(x)
    assert x.size == rows * cols
    pc = _padded_cols(cols, 16)
    packed = np.zeros(rows * pc // 2, np.uint8)
    scales = np.zeros(rows * pc // 16, np.uint8)
    sg = np.zeros(1, np.float32)
    flags = lib().or_nv_quantize_padded(_ptr(x), dt, rows, cols, _ptr(packed), _ptr(scales), _ptr(sg))
    assert flags >= 0
    return packed, scales, sg[0], flags


def dequantize_padded(fmt: int, packed: np.ndarray, scales: np.ndarray, rows: int, cols: int,
                      s_g=1.0, out_bf16=False):
    """Dequantize a row-padded layout and crop to [rows, cols]."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    y = np.empty(rows * cols, np.uint16 if out_bf16 else np.float32)
    r = lib().or_dequantize_padded(int(fmt), _ptr(packed), _ptr(scales), float(np.float32(s_g)),
                                   rows, cols, DT_BF16 if out_bf16 else DT_F32, _ptr(y))
    assert r == 0
    return y


def pack(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    if codes.size % 2:
        raise ValueError("packing requires an even number of codes")
    out = np.empty(codes.size // 2, np.uint8)
    lib().or_pack(_ptr(codes), codes.size, _ptr(out))
    return out


def unpack(packed: np.ndarray) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty(packed.size * 2, np.uint8)
    lib().or_unpack(_ptr(packed), packed.size, _ptr(out))
    return out


# ---- tensor operations ----------------------------------------------------
# All take a flat view: blocks run along the last dimension and the number of
# elements per row is a multiple of the block, so the flat order of blocks,
# codes and scales equals the row-major order.

def mx_quantize(x: np.ndarray):
    """MXFP4 quantize.  Returns (packed uint8[n/2], scales uint8[n/32], flags)."""
    x, dt = _as_input(x)
    n = x.size
    if n % 32:
        raise ValueError("MXFP4 needs complete 32-element blocks")
    packed = np.empty(n // 2, np.uint8)
    scales = np.empty(n // 32, np.uint8)
    flags = lib().or_mx_quantize(_ptr(x), dt, n, _ptr(packed), _ptr(scales))
    return packed, scales, flags


MX_RULES = {"ocp": 0, "ceil": 1, "mse": 2}


def mx_exponent_ceil(amax: float) -> int:
    """Ceil-rule MX exponent: the smallest e with 6 * 2^e >= amax."""
    return lib().or_mx_exponent_ceil(float(amax))


def mx_block_loss32(xb: np.ndarray, e: int) -> float:
    xb = np.ascontiguousarray(xb, dtype=np.float32)
    assert xb.size == 32
    return float(lib().or_block_loss32_pow2(_ptr(xb), int(e)))


def mx_quantize_rule(x: np.ndarray, rule: str):
    """MXFP4 quantize with exponent rule "ocp" (floor), "ceil" or "mse"
    (search over e0 - 1, e0, e0 + 1).  Returns (packed, scales, flags)."""
    x, dt = _as_input(x)
    n = x.size
    if n % 32:
        raise ValueError("MXFP4 needs complete 32-element blocks")
    packed = np.empty(n // 2, np.uint8)
    scales = np.empty(n // 32, np.uint8)
    flags = lib().or_mx_quantize_rule(_ptr(x), dt, n, MX_RULES[rule], _ptr(packed), _ptr(scales))
    return packed, scales, flags


def nv_global_scale(x: np.ndarray):
    """NVFP4 tensor scale s_g.  Returns (s_g as np.float32, flags)."""
    x, dt = _as_input(x)
    out = np.zeros(1, np.float32)
    flags = lib().or_nv_global_scale(_ptr(x), dt, x.size, _ptr(out))
    return out[0], flags


def nv_quantize_with_scale(x: np.ndarray, s_g):
    """NVFP4 quantize of whole 16-blocks given the tensor scale s_g."""
    x, dt = _as_input(x)
    n = x.size
    if n % 16:
        raise ValueError("NVFP4 needs complete 16-element blocks")
    packed = np.empty(n // 2, np.uint8)
    scales = np.empty(n // 16, np.uint8)
    flags = lib().or_nv_quantize(_ptr(x), dt, n, float(np.float32(s_g)), _ptr(packed), _ptr(scales))
    return packed, scales, flags


def nv_quantize(x: np.ndarray):
    """NVFP4 quantize.  Returns (packed, scales, s_g, flags)."""
    s_g, f1 = nv_global_scale(x)
    if f1:
        n = np.asarray(x).size
        return (np.zeros(n // 2, np.uint8), np.zeros(n // 16, np.uint8), s_g, f1)
    packed, scales, f2 = nv_quantize_with_scale(x, s_g)
    return packed, scales, s_g, f1 | f2


# ---- stochastic rounding ----------------------------------------------------

def sr_bits(seed: int, i: int) -> int:
    """The 24 random bits element i draws (SplitMix64 on the counter)."""
    return int(lib().or_sr_bits(int(seed) & (2**64 - 1), int(i)))


def e2m1_round_sr(q: float, r24: int) -> int:
    """Stochastic E2M1 code of fp32 q given 24 random bits."""
    return lib().or_e2m1_round_sr(float(np.float32(q)), int(r24))


def mx_quantize_sr(x: np.ndarray, seed: int):
    """MXFP4 quantize (OCP floor scale) with stochastic element rounding."""
    x, dt = _as_input(x)
    n = x.size
    if n % 32:
        raise ValueError("MXFP4 needs complete 32-element blocks")
    packed = np.empty(n // 2, np.uint8)
    scales = np.empty(n // 32, np.uint8)
    flags = lib().or_mx_quantize_sr(_ptr(x), dt, n, int(seed) & (2**64 - 1), _ptr(packed),
                                    _ptr(scales))
    return packed, scales, flags


def nv_quantize_sr(x: np.ndarray, seed: int):
    """NVFP4 quantize with stochastic element rounding (block scales and
    s_g as the deterministic encoder).  Returns (packed, scales, s_g, flags)."""
    s_g, f1 = nv_global_scale(x)
    x, dt = _as_input(x)
    n = x.size
    if n % 16:
        raise ValueError("NVFP4 needs complete 16-element blocks")
    if f1:
        return (np.zeros(n // 2, np.uint8), np.zeros(n // 16, np.uint8), s_g, f1)
    packed = np.empty(n // 2, np.uint8)
    scales = np.empty(n // 16, np.uint8)
    f2 = lib().or_nv_quantize_sr(_ptr(x), dt, n, float(s_g), int(seed) & (2**64 - 1),
                                 _ptr(packed), _ptr(scales))
    return packed, scales, s_g, f2


def dequantize(fmt: int, packed: np.ndarray, scales: np.ndarray, s_g=1.0, out_bf16=False):
    """Dequantize; returns float32 values, or uint16 bf16 bits if out_bf16."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n = packed.size * 2
    y = np.empty(n, np.uint16 if out_bf16 else np.float32)
    lib().or_dequantize(int(fmt), _ptr(packed), _ptr(scales), float(np.float32(s_g)), n,
                        DT_BF16 if out_bf16 else DT_F32, _ptr(y))
    return y


def scale_search_with_scale(x: np.ndarray, s_g, ncand=64, c_lo=0.5, c_hi=1.0, want_loss=False):
    x, dt = _as_input(x)
    n = x.size
    if n % 16:
        raise ValueError("scale search needs complete 16-element blocks")
    packed = np.empty(n // 2, np.uint8)
    scales = np.empty(n // 16, np.uint8)
    loss = np.empty(n // 16, np.float32) if want_loss else None
    flags = lib().or_scale_search(_ptr(x), dt, n, float(np.float32(s_g)), int(ncand),
                                  float(np.float32(c_lo)), float(np.float32(c_hi)),
                                  _ptr(packed), _ptr(scales),
                                  _ptr(loss) if want_loss else None)
    if want_loss:
        return packed, scales, flags, loss
    return packed, scales, flags


def scale_search(x: np.ndarray, ncand=64, c_lo=0.5, c_hi=1.0):
    """MSE-optimal NVFP4 scale search.  Returns (packed, scales, s_g, flags)."""
    s_g, f1 = nv_global_scale(x)
    if f1:
        n = np.asarray(x).size
        return (np.zeros(n // 2, np.uint8), np.zeros(n // 16, np.uint8), s_g, f1)
    packed, scales, f2 = scale_search_with_scale(x, s_g, ncand, c_lo, c_hi)
    return packed, scales, s_g, f1 | f2


def scale_search_all_with_scale(x: np.ndarray, s_g, want_loss=False):
    """Brute-force NVFP4 scale search over every E4M3 code, given s_g."""
    x, dt = _as_input(x)
    n = x.size
    if n % 16:
        raise ValueError("scale search needs complete 16-element blocks")
    packed = np.empty(n // 2, np.uint8)
    scales = np.empty(n // 16, np.uint8)
    loss = np.empty(n // 16, np.float32) if want_loss else None
    flags = lib().or_scale_search_all(_ptr(x), dt, n, float(np.float32(s_g)), _ptr(packed),
                                      _ptr(scales), _ptr(loss) if want_loss else None)
    if want_loss:
        return packed, scales, flags, loss
    return packed, scales, flags


def scale_search_all(x: np.ndarray):
    """Brute-force NVFP4 scale search.  Returns (packed, scales, s_g, flags)."""
    s_g, f1 = nv_global_scale(x)
    if f1:
        n = np.asarray(x).size
        return (np.zeros(n // 2, np.uint8), np.zeros(n // 16, np.uint8), s_g, f1)
    packed, scales, f2 = scale_search_all_with_scale(x, s_g)
    return packed, scales, s_g, f1 | f2


def ideal_roundtrip(x: np.ndarray, block: int) -> np.ndarray:
    """Ideal-scale (amax/6, unencoded) reconstruction; test-only teaching mode."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size % block:
        raise ValueError("complete blocks required")
    y = np.empty_like(x)
    lib().or_ideal_roundtrip(_ptr(x), x.size, int(block), _ptr(y))
    return y


def ideal_code(x: float, alpha: float) -> int:
    return lib().or_ideal_code(float(np.float32(x)), float(np.float32(alpha)))
