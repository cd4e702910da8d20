"""Seeded synthetic inputs for the block-scaled FP4 workloads.

This module holds only random-number generation and dtype casts: none of the
quantization method's arithmetic.  It is the one module that both the CPU
oracle's tests and the GPU path's tests and benchmark use, so that both sides
see the same input bytes.

All generators draw from explicit ``torch.Generator`` objects on the CPU in
fp32 and round once to bf16 (round-to-nearest-even) where the workload is
bf16.  Shapes, distributions and seeds:

* ``tiny_roundtrip``: fp32 [1, 4096] ~ N(0, 1), seed 0, every 512th element
  multiplied by 20 (the Ultralytics "FP4" glossary's block-size snippet).
* ``nvfp4_weight``: bf16 [8192, 8192] ~ N(0, 0.02^2), seed 0.
* ``mxfp4_activation``: bf16 [16384, 7168] = 0.5 * Student-t(nu = 3), seed 0;
  72 columns (1% of 7168, the first 72 of a seed-1 permutation) times 50.
* ``scale_search_input``: bf16 [4096, 14336] ~ Laplace(0, b = 0.01), seed 0.
* ``gemm_operands``: A fp32 [128, 8192] ~ N(0, 1), seed 0; B [K=8192, N=8192]
  ~ N(0, 0.02^2), seed 1, returned transposed and contiguous as Bt [N, K].

Every generator takes the shape as arguments so tests can draw smaller
instances with the same recipe.
"""
import numpy as np
import torch

_CHUNK_ROWS = 1024


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 CPU tensor (numpy has no bf16 type)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def tiny_roundtrip(n: int = 4096, seed: int = 0) -> torch.Tensor:
    g = _gen(seed)
    x = torch.randn(n, generator=g, dtype=torch.float32)
    x[::512] *= 20
    return x.reshape(1, n)


def nvfp4_weight(rows: int = 8192, cols: int = 8192, seed: int = 0, std: float = 0.02) -> torch.Tensor:
    g = _gen(seed)
    out = torch.empty(rows, cols, dtype=torch.bfloat16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        out[r0:r1] = (torch.randn(r1 - r0, cols, generator=g) * std).to(torch.bfloat16)
    return out


def _student_t3(shape, g: torch.Generator) -> torch.Tensor:
    # Student-t with 3 degrees of freedom: Z / sqrt(V / 3), V ~ chi^2(3),
    # the chi-square drawn as a sum of three squared standard normals.  The
    # quotient is taken in float64 with numpy's IEEE divide and square root
    # and rounded once to float32: torch's float32 CPU kernels for it give
    # different last bits on different host CPUs, and the input must be the
    # same bytes wherever it is generated.
    z = torch.randn(shape, generator=g).numpy().astype(np.float64)
    v = np.zeros(shape)
    for _ in range(3):
        w = torch.randn(shape, generator=g).numpy().astype(np.float64)
        v += w * w
    return torch.from_numpy((z / np.sqrt(v / 3.0)).astype(np.float32))


def outlier_columns(cols: int, frac: float = 0.01, seed: int = 1) -> torch.Tensor:
    k = int(round(frac * cols))
    return torch.randperm(cols, generator=_gen(seed))[:k]


def mxfp4_activation(rows: int = 16384, cols: int = 7168, seed: int = 0, scale: float = 0.5,
                     outlier_mult: float = 50.0) -> torch.Tensor:
    g = _gen(seed)
    oc = outlier_columns(cols)
    out = torch.empty(rows, cols, dtype=torch.bfloat16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        x = _student_t3((r1 - r0, cols), g) * scale
        x[:, oc] *= outlier_mult
        out[r0:r1] = x.to(torch.bfloat16)
    return out


def _laplace(shape, b: float, g: torch.Generator) -> torch.Tensor:
    # Laplace(0, b) as b * (E1 - E2) with E = -log(1 - U), U ~ U[0, 1):
    # never infinite because 1 - U > 0.
    e1 = -torch.log1p(-torch.rand(shape, generator=g))
    e2 = -torch.log1p(-torch.rand(shape, generator=g))
    return b * (e1 - e2)


def scale_search_input(rows: int = 4096, cols: int = 14336, seed: int = 0, b: float = 0.01) -> torch.Tensor:
    g = _gen(seed)
    out = torch.empty(rows, cols, dtype=torch.bfloat16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        out[r0:r1] = _laplace((r1 - r0, cols), b, g).to(torch.bfloat16)
    return out


def gemm_operands(M: int = 128, N: int = 8192, K: int = 8192, seed_a: int = 0, seed_b: int = 1,
                  std_b: float = 0.02):
    """Returns (A [M, K] fp32, Bt [N, K] fp32 contiguous)."""
    a = torch.randn(M, K, generator=_gen(seed_a))
    b = torch.randn(K, N, generator=_gen(seed_b)) * std_b
    return a.contiguous(), b.t().contiguous()


WORKLOADS = {
    "tiny_roundtrip_4096_f32": dict(shape=(1, 4096), dtype="f32"),
    "nvfp4_weight_8192x8192_bf16": dict(shape=(8192, 8192), dtype="bf16"),
    "mxfp4_activation_16384x7168_bf16": dict(shape=(16384, 7168), dtype="bf16"),
    "nvfp4_scale_search_4096x14336_bf16": dict(shape=(4096, 14336), dtype="bf16"),
    "mxfp4_gemm_128x8192x8192": dict(shape=(128, 8192, 8192), dtype="mxfp4"),
}
