"""Block-scaled FP4 (MXFP4 / NVFP4) quantization for AMD MI355X (gfx950).

Thin Python binding over ``libfp4.so`` (C ABI in ``include/fp4.h``): argument
marshalling only.  Every step of the method runs in the library's HIP
kernels; PyTorch provides device memory and the current stream.  If the
library is not built, every call raises; there is no fallback.

Functions mirror the C entry points:

    quantize_mxfp4(x)                       -> (codes, scales)
    quantize_nvfp4(x)                       -> (codes, scales, global_scale)
    dequantize(fmt, codes, scales, s_g, out_dtype)
    scale_search(x, n_candidates, c_lo, c_hi) -> (codes, scales, global_scale)
    gemm_mxfp4(a_codes, a_scales, bt_codes, bt_scales, out_dtype)

Inputs are contiguous CUDA (HIP) tensors of dtype float32 or bfloat16 whose
last dimension is a multiple of the block (32 for MXFP4, 16 for NVFP4).
codes have shape [..., K/2] (uint8, two E2M1 codes per byte, even element in
the low nibble); scales [..., K/block] (uint8: E8M0 for MXFP4, E4M3FN for
NVFP4); global_scale is a 1-element float32 tensor (NVFP4 s_g).

With ``check=True`` (the default) a call synchronises the stream, reads the
device status word and raises ValueError for non-finite input or a scale
that underflows, as the format page's reference contract does.  Pass
``check=False`` to keep calls asynchronous (benchmarks).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4.so")

MXFP4 = 0
NVFP4 = 1
F32 = 0
BF16 = 1
FLAG_NONFINITE = 1
FLAG_SCALE_UNDERFLOW = 2
FLAG_BARRIER_TIMEOUT = 4

EXPORTS = ("fp4_quantize_mxfp4", "fp4_quantize_mxfp4_rule", "fp4_quantize_nvfp4",
           "fp4_dequantize", "fp4_scale_search", "fp4_scale_search_exhaustive",
           "fp4_gemm_mxfp4", "fp4_gemm_mxfp4_splitk", "fp4_gemm_splitk_workspace_bytes",
           "fp4_gemm_nvfp4", "fp4_linear_mxfp4", "fp4_quantize_padded",
           "fp4_dequantize_padded", "fp4_padded_storage_bytes", "fp4_quantize_sr",
           "fp4_debug_quantize_nvfp4_spin", "fp4_debug_linear_mxfp4_spin",
           "fp4_packed_operand_bytes", "fp4_pack_mxfp4_operand",
           "fp4_gemm_mxfp4_packed", "fp4_quantize_mxfp4_packed", "fp4_linear_mxfp4_packed",
           "fp4_nv_packed_operand_bytes", "fp4_pack_nvfp4_operand", "fp4_gemm_nvfp4_packed",
           "fp4_quantize_nvfp4_packed", "fp4_linear_nvfp4_packed",
           "fp4_quantize_nvfp4_noalloc", "fp4_workspace_bytes", "fp4_status_str")

# fp4_mx_rule: the MXFP4 block-exponent rules
MX_RULES = {"ocp": 0, "ceil": 1, "mse": 2}

_lib = None


class Fp4Error(RuntimeError):
    """A libfp4 entry point returned a non-OK status."""


def lib() -> ctypes.CDLL:
    """Load the in-tree libfp4.so (built by ``mxfp4_block_amax_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise Fp4Error(f"{LIB_PATH} is not built; run python -m mxfp4_block_amax_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, F, S = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                         ctypes.c_size_t)
    I = ctypes.c_int
    L.fp4_quantize_mxfp4.argtypes = [P, I, I64, I64, I32, P, P, P, P]
    L.fp4_quantize_mxfp4_rule.argtypes = [P, I, I64, I64, I32, I, P, P, P, P]
    L.fp4_scale_search_exhaustive.argtypes = [P, I, I64, I64, I32, P, P, P, P, S, P, P]
    L.fp4_quantize_nvfp4.argtypes = [P, I, I64, I64, I32, P, P, P, P, S, P, P]
    L.fp4_quantize_nvfp4_noalloc.argtypes = [P, I, I64, I64, I32, P, P, P, P, P]
    L.fp4_dequantize.argtypes = [I, P, P, P, I64, I64, I32, P, I, P]
    L.fp4_scale_search.argtypes = [P, I, I64, I64, I32, I32, F, F, P, P, P, P, S, P, P]
    L.fp4_gemm_mxfp4.argtypes = [P, P, P, P, I64, I64, I64, P, I, P]
    L.fp4_gemm_nvfp4.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, I, P]
    L.fp4_gemm_mxfp4_splitk.argtypes = [P, P, P, P, I64, I64, I64, P, I, P, S, P]
    L.fp4_gemm_splitk_workspace_bytes.argtypes = [I64, I64, I64]
    L.fp4_gemm_splitk_workspace_bytes.restype = S
    L.fp4_quantize_padded.argtypes = [I, P, I, I64, I64, P, P, P, P, S, P, P]
    L.fp4_dequantize_padded.argtypes = [I, P, P, P, I64, I64, P, I, P]
    L.fp4_quantize_sr.argtypes = [I, P, I, I64, I64, I32, ctypes.c_uint64, P, P, P, P, S, P, P]
    L.fp4_padded_storage_bytes.argtypes = [I, I64, I64]
    L.fp4_padded_storage_bytes.restype = I64
    L.fp4_linear_mxfp4.argtypes = [P, I, I64, I64, P, P, I64, P, P, P, I, I, P, S, P, P]
    L.fp4_packed_operand_bytes.argtypes = [I64, I64]
    L.fp4_packed_operand_bytes.restype = I64
    L.fp4_pack_mxfp4_operand.argtypes = [P, P, I64, I64, P, S, P]
    L.fp4_gemm_mxfp4_packed.argtypes = [P, P, I64, I64, I64, P, I, P]
    L.fp4_nv_packed_operand_bytes.argtypes = [I64, I64]
    L.fp4_nv_packed_operand_bytes.restype = I64
    L.fp4_pack_nvfp4_operand.argtypes = [P, P, I64, I64, P, S, P]
    L.fp4_gemm_nvfp4_packed.argtypes = [P, P, P, P, I64, I64, I64, P, I, P]
    L.fp4_quantize_nvfp4_packed.argtypes = [P, I, I64, I64, P, S, P, P, S, P, P]
    L.fp4_linear_nvfp4_packed.argtypes = [P, I, I64, I64, P, P, I64, P, S, P, P, I, P, S, P, P]
    L.fp4_quantize_mxfp4_packed.argtypes = [P, I, I64, I64, P, S, P, P]
    L.fp4_linear_mxfp4_packed.argtypes = [P, I, I64, I64, P, I64, P, S, P, I, P, P]
    L.fp4_debug_quantize_nvfp4_spin.argtypes = [P, I, I64, I64, I32, P, P, P, P, S, P, P,
                                                ctypes.c_uint32]
    L.fp4_debug_linear_mxfp4_spin.argtypes = [P, I, I64, I64, P, P, I64, P, P, P, I, I, P, S, P, P,
                                              ctypes.c_uint32]
    L.fp4_workspace_bytes.argtypes = [I, I64, I64]
    L.fp4_workspace_bytes.restype = S
    L.fp4_status_str.argtypes = [I]
    L.fp4_status_str.restype = ctypes.c_char_p
    for name in ("fp4_quantize_mxfp4", "fp4_quantize_mxfp4_rule", "fp4_quantize_nvfp4",
                 "fp4_quantize_nvfp4_noalloc",
                 "fp4_dequantize", "fp4_scale_search", "fp4_scale_search_exhaustive",
                 "fp4_gemm_mxfp4", "fp4_gemm_mxfp4_splitk", "fp4_gemm_nvfp4",
                 "fp4_linear_mxfp4", "fp4_quantize_padded", "fp4_dequantize_padded",
                 "fp4_quantize_sr"):
        getattr(L, name).restype = I
    _lib = L
    return L


def status_str(code: int) -> str:
    return lib().fp4_status_str(int(code)).decode()


def _ok(code: int):
    if code != 0:
        raise Fp4Error(f"libfp4 status {code}: {status_str(code)}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype_code(dt) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {dt}; use torch.float32 or torch.bfloat16")


def _rows_cols(x: torch.Tensor):
    if not x.is_cuda:
        raise TypeError("expected a device tensor")
    if not x.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if x.dim() < 1 or x.numel() == 0:
        raise ValueError("expected a non-empty tensor")
    cols = x.shape[-1]
    return x.numel() // cols, cols


def _raise_flags(flags: int):
    if flags & FLAG_NONFINITE:
        raise ValueError("finite input required (NaN or Inf found)")
    if flags & FLAG_SCALE_UNDERFLOW:
        raise ValueError("a nonzero scale rounded to zero (tensor, block scale or alpha underflow)")
    # FLAG_BARRIER_TIMEOUT is information only: a workgroup took the grid
    # barrier's fallback and the outputs are exact


def _finish(status: torch.Tensor, check: bool):
    if check:
        _raise_flags(int(status.item()))


BARRIER_SPIN_LIMIT_DEFAULT = 2048  # polls of the grid barrier before its fallback


def _spin(spin_limit) -> int:
    """A grid-barrier poll limit for the debug entry points (0 .. 2^32 - 1)."""
    v = int(spin_limit)
    if not 0 <= v < 2 ** 32:
        raise ValueError("spin_limit must fit in 32 unsigned bits")
    return v


def workspace_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(lib().fp4_workspace_bytes(int(fmt), int(rows), int(cols)))


def new_workspace(rows: int, cols: int, device) -> torch.Tensor:
    """A zero-filled NVFP4 / scale-search workspace.  Reuse it across calls
    (the library keeps a barrier epoch in it); calls sharing one must be
    stream-ordered."""
    return torch.zeros(max(workspace_bytes(NVFP4, rows, cols), 16), dtype=torch.uint8, device=device)


def quantize_mxfp4(x: torch.Tensor, check: bool = True, out=None, status=None):
    rows, cols = _rows_cols(x)
    if out is None:
        codes = torch.empty(*x.shape[:-1], cols // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*x.shape[:-1], max(cols // 32, 1), dtype=torch.uint8, device=x.device)
    else:
        codes, scales = out
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_quantize_mxfp4(_ptr(x), _dtype_code(x.dtype), rows, cols, 32, _ptr(codes),
                                 _ptr(scales), _ptr(status), _stream(x)))
    _finish(status, check)
    return codes, scales


def quantize_mxfp4_rule(x: torch.Tensor, rule: str = "ocp", check: bool = True, out=None,
                       status=None):
    """MXFP4 quantize with block-exponent rule "ocp" (floor), "ceil" or "mse"."""
    rows, cols = _rows_cols(x)
    if rule not in MX_RULES:
        raise ValueError(f"unknown MX rule {rule!r}; one of {sorted(MX_RULES)}")
    if out is None:
        codes = torch.empty(*x.shape[:-1], cols // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*x.shape[:-1], max(cols // 32, 1), dtype=torch.uint8, device=x.device)
    else:
        codes, scales = out
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_quantize_mxfp4_rule(_ptr(x), _dtype_code(x.dtype), rows, cols, 32,
                                      MX_RULES[rule], _ptr(codes), _ptr(scales), _ptr(status),
                                      _stream(x)))
    _finish(status, check)
    return codes, scales


def quantize_nvfp4(x: torch.Tensor, check: bool = True, out=None, status=None, workspace=None,
                   spin_limit=None):
    """NVFP4 quantize; returns (codes, scales, s_g).  spin_limit (tests of the
    grid barrier's fallback) calls fp4_debug_quantize_nvfp4_spin with that
    poll limit instead of fp4_quantize_nvfp4."""
    rows, cols = _rows_cols(x)
    if out is None:
        codes = torch.empty(*x.shape[:-1], cols // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*x.shape[:-1], max(cols // 16, 1), dtype=torch.uint8, device=x.device)
        s_g = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        codes, scales, s_g = out
    if workspace is None:
        workspace = new_workspace(rows, cols, x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    args = (_ptr(x), _dtype_code(x.dtype), rows, cols, 16, _ptr(codes), _ptr(scales), _ptr(s_g),
            _ptr(workspace), workspace.numel(), _ptr(status), _stream(x))
    if spin_limit is None:
        _ok(lib().fp4_quantize_nvfp4(*args))
    else:
        _ok(lib().fp4_debug_quantize_nvfp4_spin(*args, _spin(spin_limit)))
    _finish(status, check)
    return codes, scales, s_g


NOALLOC_SCRATCH_BYTES = 20480


def quantize_nvfp4_noalloc(x: torch.Tensor, check: bool = True, out=None, status=None):
    """NVFP4 quantize through the entry point that allocates nothing (its
    workspace is the library's fixed per-GPU scratch).  Same results as
    quantize_nvfp4.  Calls that overlap in time on one GPU race on the
    scratch; keep them on one stream."""
    rows, cols = _rows_cols(x)
    if out is None:
        codes = torch.empty(*x.shape[:-1], cols // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*x.shape[:-1], max(cols // 16, 1), dtype=torch.uint8, device=x.device)
        s_g = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        codes, scales, s_g = out
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_quantize_nvfp4_noalloc(_ptr(x), _dtype_code(x.dtype), rows, cols, 16,
                                         _ptr(codes), _ptr(scales), _ptr(s_g), _ptr(status),
                                         _stream(x)))
    _finish(status, check)
    return codes, scales, s_g


def quantize_sr(fmt: int, x: torch.Tensor, seed: int, check: bool = True, out=None, status=None,
                workspace=None):
    """Quantize with stochastic element rounding (MXFP4 or NVFP4).  Returns
    (codes, scales) for MXFP4, (codes, scales, s_g) for NVFP4."""
    rows, cols = _rows_cols(x)
    block = 32 if fmt == MXFP4 else 16
    if out is None:
        codes = torch.empty(*x.shape[:-1], cols // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*x.shape[:-1], max(cols // block, 1), dtype=torch.uint8,
                             device=x.device)
        s_g = torch.empty(1, dtype=torch.float32, device=x.device) if fmt == NVFP4 else None
    else:
        codes, scales, s_g = out if fmt == NVFP4 else (*out, None)
    if fmt == NVFP4 and workspace is None:
        workspace = new_workspace(rows, cols, x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_quantize_sr(int(fmt), _ptr(x), _dtype_code(x.dtype), rows, cols, block,
                              int(seed) & (2**64 - 1), _ptr(codes), _ptr(scales), _ptr(s_g),
                              _ptr(workspace), workspace.numel() if workspace is not None else 0,
                              _ptr(status), _stream(x)))
    _finish(status, check)
    return (codes, scales, s_g) if fmt == NVFP4 else (codes, scales)


def dequantize(fmt: int, codes: torch.Tensor, scales: torch.Tensor, global_scale=None,
               out_dtype=torch.bfloat16, out=None):
    rows, half = _rows_cols(codes)
    cols = half * 2
    block = 32 if fmt == MXFP4 else 16
    y = out if out is not None else torch.empty(*codes.shape[:-1], cols, dtype=out_dtype,
                                                device=codes.device)
    _ok(lib().fp4_dequantize(int(fmt), _ptr(codes), _ptr(scales), _ptr(global_scale), rows, cols,
                             block, _ptr(y), _dtype_code(y.dtype), _stream(codes)))
    return y


def scale_search(x: torch.Tensor, n_candidates: int = 64, c_lo: float = 0.5, c_hi: float = 1.0,
                 check: bool = True, out=None, status=None, workspace=None):
    rows, cols = _rows_cols(x)
    if out is None:
        codes = torch.empty(*x.shape[:-1], cols // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*x.shape[:-1], max(cols // 16, 1), dtype=torch.uint8, device=x.device)
        s_g = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        codes, scales, s_g = out
    if workspace is None:
        workspace = new_workspace(rows, cols, x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_scale_search(_ptr(x), _dtype_code(x.dtype), rows, cols, 16, int(n_candidates),
                               float(c_lo), float(c_hi), _ptr(codes), _ptr(scales), _ptr(s_g),
                               _ptr(workspace), workspace.numel(), _ptr(status), _stream(x)))
    _finish(status, check)
    return codes, scales, s_g


def scale_search_exhaustive(x: torch.Tensor, check: bool = True, out=None, status=None,
                            workspace=None):
    """NVFP4 scale search over every E4M3 code."""
    rows, cols = _rows_cols(x)
    if out is None:
        codes = torch.empty(*x.shape[:-1], cols // 2, dtype=torch.uint8, device=x.device)
        scales = torch.empty(*x.shape[:-1], max(cols // 16, 1), dtype=torch.uint8, device=x.device)
        s_g = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        codes, scales, s_g = out
    if workspace is None:
        workspace = new_workspace(rows, cols, x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_scale_search_exhaustive(_ptr(x), _dtype_code(x.dtype), rows, cols, 16,
                                          _ptr(codes), _ptr(scales), _ptr(s_g), _ptr(workspace),
                                          workspace.numel(), _ptr(status), _stream(x)))
    _finish(status, check)
    return codes, scales, s_g


def gemm_mxfp4(a_codes: torch.Tensor, a_scales: torch.Tensor, bt_codes: torch.Tensor,
               bt_scales: torch.Tensor, out_dtype=torch.bfloat16, out=None):
    """C [M, N] = A [M, K] @ B [K, N] with A and Bt = B^T [N, K] in MXFP4."""
    M, kh = _rows_cols(a_codes)
    N, kh2 = _rows_cols(bt_codes)
    if kh != kh2:
        raise ValueError("A and Bt must share K")
    K = 2 * kh
    c = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=a_codes.device)
    _ok(lib().fp4_gemm_mxfp4(_ptr(a_codes), _ptr(a_scales), _ptr(bt_codes), _ptr(bt_scales), M, N,
                             K, _ptr(c), _dtype_code(c.dtype), _stream(a_codes)))
    return c


def packed_operand_bytes(rows: int, K: int) -> int:
    return int(lib().fp4_packed_operand_bytes(int(rows), int(K)))


def _check_u8(t: torch.Tensor, numel: int, what: str, device):
    """t must be a contiguous uint8 tensor on `device` with `numel` elements
    (checked here because the C call takes no size for it)."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8:
        raise TypeError(f"{what} must be a uint8 tensor")
    if t.device != torch.device(device) or not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous on {device}")
    if t.numel() != numel:
        raise ValueError(f"{what} has {t.numel()} elements, needs {numel}")


def _check_global_scale(t: torch.Tensor, what: str, device):
    """A tensor scale: a float32 tensor on `device` with at least one element."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
        raise TypeError(f"{what} must be a float32 tensor")
    if t.device != torch.device(device) or t.numel() < 1:
        raise ValueError(f"{what} must hold at least one element on {device}")


def pack_mxfp4_operand(codes: torch.Tensor, scales: torch.Tensor, out=None) -> torch.Tensor:
    """An MXFP4 operand [rows, K] (codes [rows, K/2], scales [rows, K/32]) in
    MFMA operand order, one uint8 buffer, for gemm_mxfp4_packed."""
    rows, kh = _rows_cols(codes)
    n = packed_operand_bytes(rows, 2 * kh)
    if n == 0:
        raise ValueError("packing needs K a positive multiple of 512")
    _check_u8(scales, rows * (2 * kh) // 32, "scales", codes.device)
    packed = out if out is not None else torch.empty(n, dtype=torch.uint8, device=codes.device)
    _ok(lib().fp4_pack_mxfp4_operand(_ptr(codes), _ptr(scales), rows, 2 * kh, _ptr(packed),
                                     packed.numel(), _stream(codes)))
    return packed


def gemm_mxfp4_packed(a_packed: torch.Tensor, bt_packed: torch.Tensor, M: int, N: int, K: int,
                      out_dtype=torch.bfloat16, out=None):
    """C [M, N] = A @ B from packed A [M, K] and packed Bt [N, K]."""
    if a_packed.numel() < packed_operand_bytes(M, K) or bt_packed.numel() < packed_operand_bytes(N, K):
        raise ValueError("packed operand smaller than its shape")
    c = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=a_packed.device)
    _ok(lib().fp4_gemm_mxfp4_packed(_ptr(a_packed), _ptr(bt_packed), int(M), int(N), int(K),
                                    _ptr(c), _dtype_code(c.dtype), _stream(a_packed)))
    return c


def quantize_mxfp4_packed(x: torch.Tensor, check: bool = True, out=None, status=None):
    """MXFP4 quantize (floor rule) of x [rows, cols] written in MFMA operand
    order: the bytes pack_mxfp4_operand(*quantize_mxfp4(x)) would give."""
    rows, cols = _rows_cols(x)
    n = packed_operand_bytes(rows, cols)
    if n == 0:
        raise ValueError("the packed layout needs cols a positive multiple of 512")
    packed = out if out is not None else torch.empty(n, dtype=torch.uint8, device=x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_quantize_mxfp4_packed(_ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(packed),
                                        packed.numel(), _ptr(status), _stream(x)))
    _finish(status, check)
    return packed


def linear_mxfp4_packed(x: torch.Tensor, bt_packed: torch.Tensor, N: int,
                        out_dtype=torch.bfloat16, out=None, a_out=None, status=None,
                        check: bool = True):
    """W4A4 linear on a packed weight: x [M, K] quantized into packed A, then
    the packed GEMM.  Returns (C [M, N], a_packed)."""
    M, K = _rows_cols(x)
    n = packed_operand_bytes(M, K)
    a_packed = a_out if a_out is not None else torch.empty(max(n, 16), dtype=torch.uint8,
                                                           device=x.device)
    c = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_linear_mxfp4_packed(_ptr(x), _dtype_code(x.dtype), M, K, _ptr(bt_packed), int(N),
                                      _ptr(a_packed), a_packed.numel(), _ptr(c),
                                      _dtype_code(c.dtype), _ptr(status), _stream(x)))
    _finish(status, check)
    return c, a_packed


def gemm_splitk_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().fp4_gemm_splitk_workspace_bytes(int(M), int(N), int(K)))


def gemm_mxfp4_splitk(a_codes: torch.Tensor, a_scales: torch.Tensor, bt_codes: torch.Tensor,
                      bt_scales: torch.Tensor, out_dtype=torch.bfloat16, out=None, workspace=None):
    """The MXFP4 GEMM split over K (fp32 partials in `workspace`, then a
    fixed-order reduction); for short A."""
    M, kh = _rows_cols(a_codes)
    N, kh2 = _rows_cols(bt_codes)
    if kh != kh2:
        raise ValueError("A and Bt must share K")
    K = 2 * kh
    c = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=a_codes.device)
    if workspace is None:
        need = gemm_splitk_workspace_bytes(M, N, K)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a_codes.device)
    _ok(lib().fp4_gemm_mxfp4_splitk(_ptr(a_codes), _ptr(a_scales), _ptr(bt_codes),
                                    _ptr(bt_scales), M, N, K, _ptr(c), _dtype_code(c.dtype),
                                    _ptr(workspace), workspace.numel(), _stream(a_codes)))
    return c


def gemm_nvfp4(a_codes: torch.Tensor, a_scales: torch.Tensor, a_global_scale: torch.Tensor,
               bt_codes: torch.Tensor, bt_scales: torch.Tensor, bt_global_scale: torch.Tensor,
               out_dtype=torch.bfloat16, out=None):
    """C [M, N] = A [M, K] @ B [K, N] with A and Bt = B^T [N, K] in NVFP4."""
    M, kh = _rows_cols(a_codes)
    N, kh2 = _rows_cols(bt_codes)
    if kh != kh2:
        raise ValueError("A and Bt must share K")
    K = 2 * kh
    c = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=a_codes.device)
    _ok(lib().fp4_gemm_nvfp4(_ptr(a_codes), _ptr(a_scales), _ptr(a_global_scale), _ptr(bt_codes),
                             _ptr(bt_scales), _ptr(bt_global_scale), M, N, K, _ptr(c),
                             _dtype_code(c.dtype), _stream(a_codes)))
    return c


def nv_packed_operand_bytes(rows: int, K: int) -> int:
    return int(lib().fp4_nv_packed_operand_bytes(int(rows), int(K)))


def pack_nvfp4_operand(codes: torch.Tensor, scales: torch.Tensor, out=None) -> torch.Tensor:
    """An NVFP4 operand [rows, K] (codes [rows, K/2], E4M3 scales [rows, K/16])
    in MFMA operand order, one uint8 buffer, for gemm_nvfp4_packed."""
    rows, kh = _rows_cols(codes)
    n = nv_packed_operand_bytes(rows, 2 * kh)
    if n == 0:
        raise ValueError("packing needs K a positive multiple of 512")
    _check_u8(scales, rows * (2 * kh) // 16, "scales", codes.device)
    packed = out if out is not None else torch.empty(n, dtype=torch.uint8, device=codes.device)
    _ok(lib().fp4_pack_nvfp4_operand(_ptr(codes), _ptr(scales), rows, 2 * kh, _ptr(packed),
                                     packed.numel(), _stream(codes)))
    return packed


def gemm_nvfp4_packed(a_packed: torch.Tensor, a_global_scale: torch.Tensor,
                      bt_packed: torch.Tensor, bt_global_scale: torch.Tensor, M: int, N: int,
                      K: int, out_dtype=torch.bfloat16, out=None):
    """C [M, N] = A @ B from packed NVFP4 A [M, K] and Bt [N, K] with their
    tensor scales."""
    if (a_packed.numel() < nv_packed_operand_bytes(M, K)
            or bt_packed.numel() < nv_packed_operand_bytes(N, K)):
        raise ValueError("packed operand smaller than its shape")
    _check_global_scale(a_global_scale, "a_global_scale", a_packed.device)
    _check_global_scale(bt_global_scale, "bt_global_scale", a_packed.device)
    c = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=a_packed.device)
    _ok(lib().fp4_gemm_nvfp4_packed(_ptr(a_packed), _ptr(a_global_scale), _ptr(bt_packed),
                                    _ptr(bt_global_scale), int(M), int(N), int(K), _ptr(c),
                                    _dtype_code(c.dtype), _stream(a_packed)))
    return c


def quantize_nvfp4_packed(x: torch.Tensor, check: bool = True, out=None, status=None,
                          workspace=None):
    """NVFP4 quantize of x [rows, cols] written in the packed NVFP4 layout:
    returns (packed, s_g), the bytes pack_nvfp4_operand(*quantize_nvfp4(x)[:2])
    would give and the tensor scale."""
    rows, cols = _rows_cols(x)
    n = nv_packed_operand_bytes(rows, cols)
    if n == 0:
        raise ValueError("the packed layout needs cols a positive multiple of 512")
    if out is None:
        packed = torch.empty(n, dtype=torch.uint8, device=x.device)
        s_g = torch.empty(1, dtype=torch.float32, device=x.device)
    else:
        packed, s_g = out
    if workspace is None:
        workspace = new_workspace(rows, cols, x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_quantize_nvfp4_packed(_ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(packed),
                                        packed.numel(), _ptr(s_g), _ptr(workspace),
                                        workspace.numel(), _ptr(status), _stream(x)))
    _finish(status, check)
    return packed, s_g


def linear_nvfp4_packed(x: torch.Tensor, bt_packed: torch.Tensor, bt_global_scale: torch.Tensor,
                        N: int, out_dtype=torch.bfloat16, out=None, a_out=None, status=None,
                        workspace=None, check: bool = True):
    """NVFP4 W4A4 linear on a packed weight: x [M, K] quantized to NVFP4 in
    the packed layout, times Bt [N, K] (packed, with its tensor scale).
    Returns (C [M, N], (a_packed, a_s_g))."""
    M, K = _rows_cols(x)
    _check_global_scale(bt_global_scale, "bt_global_scale", x.device)
    if a_out is None:
        a_out = (torch.empty(nv_packed_operand_bytes(M, K), dtype=torch.uint8, device=x.device),
                 torch.empty(1, dtype=torch.float32, device=x.device))
    a_packed, a_sg = a_out
    _check_global_scale(a_sg, "a_out[1]", x.device)
    c = out if out is not None else torch.empty(M, int(N), dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = new_workspace(M, K, x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_linear_nvfp4_packed(_ptr(x), _dtype_code(x.dtype), M, K, _ptr(bt_packed),
                                      _ptr(bt_global_scale), int(N), _ptr(a_packed),
                                      a_packed.numel(), _ptr(a_sg), _ptr(c), _dtype_code(c.dtype),
                                      _ptr(workspace), workspace.numel(), _ptr(status),
                                      _stream(x)))
    _finish(status, check)
    return c, a_out


def linear_mxfp4(x: torch.Tensor, bt_codes: torch.Tensor, bt_scales: torch.Tensor,
                 out_dtype=torch.bfloat16, out=None, a_out=None, status=None, workspace=None,
                 check: bool = True, one_launch: bool = True, spin_limit=None):
    """W4A4 linear: x [M, K] (fp32/bf16) quantized to MXFP4, times B with
    Bt = B^T [N, K] in MXFP4.  Returns (C [M, N], (a_codes, a_scales)).
    one_launch: quantize and multiply in one kernel when the grid fits.
    spin_limit (tests of the grid barrier's fallback): through
    fp4_debug_linear_mxfp4_spin with that poll limit."""
    M, K = _rows_cols(x)
    N, kh = _rows_cols(bt_codes)
    if 2 * kh != K:
        raise ValueError("x and Bt must share K")
    if a_out is None:
        a_codes = torch.empty(M, K // 2, dtype=torch.uint8, device=x.device)
        a_scales = torch.empty(M, K // 32, dtype=torch.uint8, device=x.device)
    else:
        a_codes, a_scales = a_out
    c = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=x.device)
    if workspace is None:
        workspace = new_workspace(M, K, x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    args = (_ptr(x), _dtype_code(x.dtype), M, K, _ptr(bt_codes), _ptr(bt_scales), N,
            _ptr(a_codes), _ptr(a_scales), _ptr(c), _dtype_code(c.dtype), 0 if one_launch else 1,
            _ptr(workspace), workspace.numel(), _ptr(status), _stream(x))
    if spin_limit is None:
        _ok(lib().fp4_linear_mxfp4(*args))
    else:
        _ok(lib().fp4_debug_linear_mxfp4_spin(*args, _spin(spin_limit)))
    _finish(status, check)
    return c, (a_codes, a_scales)


def _padded_cols(cols: int, fmt: int) -> int:
    block = 32 if fmt == MXFP4 else 16
    return (cols + block - 1) // block * block


def quantize_padded(fmt: int, x: torch.Tensor, check: bool = True, status=None, workspace=None):
    """Quantize a [rows, cols] tensor, rows zero-padded to whole blocks.
    Returns (codes [rows, pcols/2], scales [rows, pcols/block], s_g or None)."""
    rows, cols = _rows_cols(x)
    pc = _padded_cols(cols, fmt)
    block = 32 if fmt == MXFP4 else 16
    codes = torch.empty(rows, pc // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, pc // block, dtype=torch.uint8, device=x.device)
    s_g = torch.empty(1, dtype=torch.float32, device=x.device) if fmt == NVFP4 else None
    if fmt == NVFP4 and workspace is None:
        workspace = new_workspace(rows, pc, x.device)
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=x.device)
    _ok(lib().fp4_quantize_padded(int(fmt), _ptr(x), _dtype_code(x.dtype), rows, cols, _ptr(codes),
                                  _ptr(scales), _ptr(s_g), _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _ptr(status),
                                  _stream(x)))
    _finish(status, check)
    return codes, scales, s_g


def dequantize_padded(fmt: int, codes: torch.Tensor, scales: torch.Tensor, cols: int,
                      global_scale=None, out_dtype=torch.bfloat16):
    """Decode a row-padded layout to [rows, cols]."""
    rows = codes.shape[0]
    y = torch.empty(rows, cols, dtype=out_dtype, device=codes.device)
    _ok(lib().fp4_dequantize_padded(int(fmt), _ptr(codes), _ptr(scales), _ptr(global_scale), rows,
                                    cols, _ptr(y), _dtype_code(out_dtype), _stream(codes)))
    return y


def padded_storage_bytes(fmt: int, rows: int, cols: int) -> int:
    return int(lib().fp4_padded_storage_bytes(int(fmt), int(rows), int(cols)))

