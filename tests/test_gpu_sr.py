"""GPU parity for stochastic rounding (Ultralytics glossary "FP4", section
"Inferenza e addestramento FP4"), bit-exact against the oracle on the same
inputs and seeds: MXFP4 and NVFP4, fp32 and bf16, every bf16 value at every
E8M0 exponent, quotients placed one fp32 step either side of each element's
own decision threshold, tensors at extreme magnitudes, ragged shapes and the
full-size workloads."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import workloads
from tests._gpu import announce, assert_bytes_equal, dev, f32_bits, host_u8, oracle_view
from tests._sr_cases import (SEED_ZERO_BITS_AT_16, mean_within_bounds, neighbour_values,
                             threshold_blocks, tiny_quotient_cases, tiny_quotient_tensor)
from tests.test_gpu_quantize import _mx_fp32_midpoint_tensor, _mx_sweep_tensor

pytestmark = pytest.mark.gpu

SEEDS = [0, 1, 0x123456789ABCDEF0, 2**64 - 1]


def check_sr(fmt: int, x: torch.Tensor, seed: int, what: str):
    name = "mxfp4" if fmt == fp4.MXFP4 else "nvfp4"
    announce(f"{name} stochastic quantize {what} {tuple(x.shape)} {x.dtype} seed={seed:#x}")
    got = fp4.quantize_sr(fmt, dev(x), seed)
    torch.cuda.synchronize()
    xv = oracle_view(x)
    if fmt == fp4.MXFP4:
        p, s, flags = oracle.mx_quantize_sr(xv, seed)
    else:
        p, s, sg, flags = oracle.nv_quantize_sr(xv, seed)
        assert f32_bits(got[2].cpu().numpy())[0] == f32_bits([sg])[0], f"{what}: s_g"
    assert flags == 0
    assert_bytes_equal(host_u8(got[1]), s, f"{what}: {name} SR scales")
    assert_bytes_equal(host_u8(got[0]), p, f"{what}: {name} SR codes")
    return got


# ---- quotients on both sides of each element's own threshold -----------------

@pytest.mark.parametrize("fmt", [fp4.MXFP4, fp4.NVFP4])
@pytest.mark.parametrize("seed", [3, 2**63 + 11])
def test_quotients_at_each_elements_threshold(fmt, seed):
    block = 32 if fmt == fp4.MXFP4 else 16
    lead = 16 if fmt == fp4.NVFP4 else 0  # NVFP4: a leading 2688 block fixes s_g = 1
    x, want = threshold_blocks(block, 96, seed, offset=lead)
    if lead:
        x = np.concatenate([np.full(lead, 2688.0, np.float32), x])
    t = torch.from_numpy(x).reshape(1, -1)
    # the oracle takes the expected decisions (an independent restatement of
    # the threshold rule), then the GPU must match the oracle byte for byte
    xv = oracle_view(t)
    if fmt == fp4.MXFP4:
        p, s, _ = oracle.mx_quantize_sr(xv, seed)
    else:
        p, s, sg, _ = oracle.nv_quantize_sr(xv, seed)
        assert float(sg) == 1.0
    assert np.array_equal(oracle.unpack(p)[lead:], want)
    check_sr(fmt, t, seed, "threshold quotients")


def test_tiny_quotients_with_zero_random_bits():
    """Quotients far below 2^-25 (down to the fp32 subnormals and the tie at
    2^-150) at an element whose random bits are zero: they round up exactly
    when the fp32 quotient is nonzero, on both sides."""
    for value, nv_code, mx_code in tiny_quotient_cases():
        codes = check_sr(fp4.NVFP4, torch.from_numpy(tiny_quotient_tensor(16, value)).reshape(1, -1),
                         SEED_ZERO_BITS_AT_16, f"tiny quotient {value!r}")[0]
        assert oracle.unpack(host_u8(codes))[16] == nv_code
        codes = check_sr(fp4.MXFP4, torch.from_numpy(tiny_quotient_tensor(32, value)).reshape(1, -1),
                         SEED_ZERO_BITS_AT_16, f"tiny quotient {value!r}")[0]
        assert oracle.unpack(host_u8(codes))[16] == mx_code


# ---- exhaustive and adversarial value sets -------------------------------------

@pytest.mark.parametrize("seed", SEEDS[:2])
def test_mx_every_bf16_value_at_every_exponent(seed):
    check_sr(fp4.MXFP4, _mx_sweep_tensor(), seed, "exhaustive bf16 x E8M0 sweep")


def test_mx_fp32_midpoints_and_subnormals():
    for seed in SEEDS:
        check_sr(fp4.MXFP4, _mx_fp32_midpoint_tensor(), seed, "fp32 midpoints")


def test_nv_grid_values_zeros_and_ties():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -5.0, -0.0, 0.0, 1e-30,
            -1e-30, 2.0]
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0,
            -0.0]
    x = np.concatenate([np.full(16, 2688.0), mids, grid, np.zeros(16), [-0.0] * 16,
                        [0.3, 0.6, 0.9, 1.2, 1.8, 2.4, 3.6, 0.0] * 2]).astype(np.float32)
    t = torch.from_numpy(x).reshape(1, -1)
    for seed in SEEDS:
        codes = check_sr(fp4.NVFP4, t, seed, "ties/zeros/grid fp32")[0]
        check_sr(fp4.NVFP4, t.to(torch.bfloat16), seed, "ties/zeros/grid bf16")
        # grid values never move (the scale of that block is 1)
        c = oracle.unpack(host_u8(codes))[32:48]
        assert np.array_equal(c, oracle.e2m1_round_array(np.array(grid, np.float32)))


@pytest.mark.parametrize("scale_exp", [-140, -126, -100, -64, 0, 64, 110])
def test_nv_extreme_tensor_scales(scale_exp):
    g = torch.Generator().manual_seed(scale_exp + 2000)
    x = torch.randn(64, 256, generator=g) * torch.rand(64, 256, generator=g) ** 4
    x = (x * 2.0 ** scale_exp).to(torch.float32)
    if oracle.nv_quantize_sr(x.numpy().reshape(-1), 5)[3]:
        pytest.skip("oracle reports underflow for this magnitude (covered by the status test)")
    check_sr(fp4.NVFP4, x, 5, f"magnitude 2^{scale_exp}")


@pytest.mark.parametrize("fmt", [fp4.MXFP4, fp4.NVFP4])
def test_ragged_shapes_both_dtypes(fmt):
    g = torch.Generator().manual_seed(17)
    shapes = [(1, 32), (3, 96), (7, 4128), (129, 160), (257, 1056)]
    for rows, cols in shapes:
        x = torch.randn(rows, cols, generator=g) * torch.rand(rows, cols, generator=g) ** 2 * 10
        for seed in (SEEDS[0], SEEDS[2]):
            check_sr(fmt, x, seed, f"ragged fp32 {rows}x{cols}")
            check_sr(fmt, x.to(torch.bfloat16), seed, f"ragged bf16 {rows}x{cols}")


# ---- the workloads at full size --------------------------------------------------

def test_mx_activation_16384x7168_full():
    check_sr(fp4.MXFP4, workloads.mxfp4_activation(), 0x5EED, "activation 16384x7168")


def test_nv_weight_8192_full():
    check_sr(fp4.NVFP4, workloads.nvfp4_weight(), 0x5EED, "weight 8192x8192")


# ---- contract ------------------------------------------------------------------------

def test_same_seed_repeats_and_another_seed_differs():
    x = dev(workloads.nvfp4_weight(512, 2048, seed=3))
    announce("stochastic determinism 512x2048")
    for fmt in (fp4.MXFP4, fp4.NVFP4):
        a = fp4.quantize_sr(fmt, x, 42)
        b = fp4.quantize_sr(fmt, x, 42)
        c = fp4.quantize_sr(fmt, x, 43)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        assert torch.equal(a[1], c[1]) and not torch.equal(a[0], c[0])
        # scales equal those of the deterministic encoder
        d = fp4.quantize_mxfp4(x) if fmt == fp4.MXFP4 else fp4.quantize_nvfp4(x)
        assert torch.equal(a[1], d[1])


def test_unbiased_on_average_over_seeds():
    """Averaged over 256 seeds the dequantized tensor is consistent with
    expectation x, while nearest rounding is several times further off (the
    oracle pins the rule; this checks the device path end to end through the
    dequantizer)."""
    g = torch.Generator().manual_seed(23)
    x = torch.randn(8, 512, generator=g)
    xd = dev(x)
    announce("stochastic mean over 256 seeds 8x512")
    acc = torch.zeros_like(xd, dtype=torch.float64)
    for sd in range(256):
        codes, scales = fp4.quantize_sr(fp4.MXFP4, xd, 10_000 + sd)
        acc += fp4.dequantize(fp4.MXFP4, codes, scales, out_dtype=torch.float32).double()
    mean = (acc / 256).cpu().numpy().reshape(-1)
    xv = x.numpy().reshape(-1).astype(np.float64)
    _, s_det = fp4.quantize_mxfp4(xd)
    scale = np.repeat(np.ldexp(1.0, host_u8(s_det).astype(np.int64) - 127), 32)
    lo, hi = neighbour_values((xv / scale).astype(np.float32), scale)
    assert mean_within_bounds(xv, lo, hi, mean, 256)
    det = fp4.dequantize(fp4.MXFP4, *fp4.quantize_mxfp4(xd), out_dtype=torch.float32)
    det = det.double().cpu().numpy().reshape(-1)
    assert np.abs(det - xv).mean() > 3 * np.abs(mean - xv).mean()


def test_flags_and_errors():
    announce("stochastic status flags")
    x = torch.zeros(2, 64, dtype=torch.float32)
    x[1, 5] = float("nan")
    for fmt in (fp4.MXFP4, fp4.NVFP4):
        with pytest.raises(ValueError):
            fp4.quantize_sr(fmt, dev(x), 1)
    blk = torch.tensor([2688.0] * 16 + [1e-10] * 16).reshape(1, 32)
    with pytest.raises(ValueError):
        fp4.quantize_sr(fp4.NVFP4, dev(blk), 1)
    z = torch.zeros(4, 64, dtype=torch.bfloat16)
    codes, scales, sg = fp4.quantize_sr(fp4.NVFP4, dev(z), 9)
    assert float(sg.item()) == 1.0 and bool((scales == 0x38).all()) and bool((codes == 0).all())
