"""GPU parity for the encoder variants, bit-exact against the oracle: the
MXFP4 ceil rule and three-exponent search ("NVFP4 / MXFP4 format" page,
section 5), the NVFP4 search over c in [0.5, 1.5] (the scale-choice section
of the "FP4, FP8 and INT8/INT4" page) and the brute-force search over every
E4M3 code (format page, section 4)."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import workloads
from tests._gpu import (announce, assert_bytes_equal, dev, f32_bits, host_u8, oracle_split,
                        oracle_view)
from tests.test_gpu_dequant_search import _search_check
from tests.test_gpu_quantize import _mx_fp32_midpoint_tensor, _mx_sweep_tensor

pytestmark = pytest.mark.gpu


def check_mx_rule(x: torch.Tensor, rule: str, what: str):
    announce(f"mxfp4 quantize rule={rule} {what} {tuple(x.shape)} {x.dtype}")
    codes, scales = fp4.quantize_mxfp4_rule(dev(x), rule)
    torch.cuda.synchronize()
    p, s, flags = oracle.mx_quantize_rule(oracle_view(x), rule)
    assert flags == 0
    assert_bytes_equal(host_u8(scales), s, f"{what}: MX {rule} scales")
    assert_bytes_equal(host_u8(codes), p, f"{what}: MX {rule} codes")


@pytest.mark.parametrize("rule", ["ocp", "ceil", "mse"])
def test_mx_rule_every_bf16_value_at_every_exponent(rule):
    check_mx_rule(_mx_sweep_tensor(), rule, "exhaustive bf16 x E8M0 sweep")


@pytest.mark.parametrize("rule", ["ceil", "mse"])
def test_mx_rule_fp32_midpoints_and_subnormals(rule):
    check_mx_rule(_mx_fp32_midpoint_tensor(), rule, "fp32 midpoints")


@pytest.mark.parametrize("rule", ["ceil", "mse"])
def test_mx_rule_activation_workload(rule):
    check_mx_rule(workloads.mxfp4_activation(), rule, "activation 16384x7168")


def test_mx_rule_page_blocks_and_ragged_sizes():
    def block(vals, fill=0.0):
        b = torch.full((1, 32), fill)
        b[0, : len(vals)] = torch.tensor(vals)
        return b
    x = torch.cat([block([7.0]), block([7.5]), block([4.0], 0.2), block([0.0]), block([6.0]),
                   block([1e-39, -3e-40]), block([3e38])])
    for rule in ("ceil", "mse"):
        check_mx_rule(x, rule, "page blocks")
        check_mx_rule(x.to(torch.bfloat16), rule, "page blocks bf16")
    codes, scales = fp4.quantize_mxfp4_rule(dev(x), "ceil")
    assert int(scales[0, 0]) - 127 == 1                 # max 7 -> scale 2
    codes, scales = fp4.quantize_mxfp4_rule(dev(x), "mse")
    assert [int(v) - 127 for v in scales.reshape(-1)[:3].tolist()] == [0, 1, -1]
    g = torch.Generator().manual_seed(41)
    for rows, cols in [(1, 32), (3, 96), (7, 4128), (129, 160)]:
        y = torch.randn(rows, cols, generator=g) * torch.rand(rows, cols, generator=g) ** 4
        for rule in ("ceil", "mse"):
            check_mx_rule(y, rule, f"ragged {rows}x{cols}")
            check_mx_rule(y.to(torch.bfloat16), rule, f"ragged {rows}x{cols} bf16")


def test_mx_rule_flags_nonfinite():
    x = torch.zeros(2, 64)
    x[1, 5] = float("nan")
    for rule in ("ceil", "mse"):
        with pytest.raises(ValueError):
            fp4.quantize_mxfp4_rule(dev(x), rule)


# ---- NVFP4 search, wider range ------------------------------------------------

def test_search_range_to_1_5_small_full_compare():
    x = workloads.scale_search_input(64, 1024, seed=5)
    _search_check(x, "laplace 64x1024 c=[0.5,1.5]", c_hi=1.5)
    block = torch.tensor([1.0, 2.0, 3.0, 4.0] * 4 + [2688.0] * 16).reshape(1, 32)
    codes, scales, sg = fp4.scale_search(dev(block), 64, 0.5, 1.5)
    assert float(sg) == 1.0 and int(scales[0, 0]) == 0x38   # the max maps to 4


def test_search_range_to_1_5_full_size_every_block():
    _search_check(workloads.scale_search_input(), "laplace 4096x14336 c=[0.5,1.5] (every block)",
                  c_hi=1.5)


# ---- brute force over every E4M3 code -----------------------------------------

def check_search_all(x: torch.Tensor, what: str):
    announce(f"exhaustive scale search {what} {tuple(x.shape)} {x.dtype}")
    codes, scales, sg = fp4.scale_search_exhaustive(dev(x))
    torch.cuda.synchronize()
    xo = oracle_view(x)
    s_g, f1 = oracle.nv_global_scale(xo)
    assert f1 == 0
    assert f32_bits(sg.cpu().numpy())[0] == f32_bits([s_g])[0]
    res = oracle_split(lambda part: oracle.scale_search_all_with_scale(part, s_g), xo, 16)
    assert all(r[2] == 0 for r in res)
    assert_bytes_equal(host_u8(scales), np.concatenate([r[1] for r in res]), f"{what}: scales")
    assert_bytes_equal(host_u8(codes), np.concatenate([r[0] for r in res]), f"{what}: codes")


def test_exhaustive_search_page_block():
    x = torch.tensor([2688.0] * 16 + [0.4] * 15 + [3.6]).reshape(1, 32)
    check_search_all(x, "page block")
    check_search_all(x.to(torch.bfloat16), "page block bf16")
    codes, scales, sg = fp4.scale_search_exhaustive(dev(x))
    assert oracle.e4m3_value(int(scales[0, 1])) == 0.875


def test_exhaustive_search_laplace_and_heavy_tails():
    check_search_all(workloads.scale_search_input(256, 1024, seed=7), "laplace 256x1024")
    g = torch.Generator().manual_seed(43)
    y = torch.randn(48, 512, generator=g) * torch.rand(48, 512, generator=g) ** 3
    check_search_all(y, "heavy-tailed fp32 48x512")
    check_search_all((y * 2.0 ** -120).to(torch.float32), "tiny magnitudes 2^-120")
    check_search_all((y * 2.0 ** 100).to(torch.float32), "large magnitudes 2^100")
    z = y.clone()
    z[3] = 0.0
    check_search_all(z.to(torch.bfloat16), "zero blocks bf16")


def test_exhaustive_search_full_size_every_block():
    check_search_all(workloads.scale_search_input(), "laplace 4096x14336 (every block)")


def test_search_exact_loss_ties_go_to_the_smaller_code():
    """Blocks [A, 0 x 15] for every bf16 A in [4, 16) behind a 2688 block
    (s_g = 1): the clipped and the unclipped neighbour codes often give
    bit-equal losses (two- and three-way ties), and the smaller code must
    win, as in the oracle's increasing-order search; the kernel walks codes
    downward with an early stop."""
    A = (np.arange(0x4080, 0x4180, dtype=np.uint32) << 16).view(np.float32)
    blocks = np.zeros((A.size, 16), np.float32)
    blocks[:, 0] = A
    x = torch.from_numpy(np.concatenate([np.full(16, 2688.0, np.float32), blocks.reshape(-1)]))
    x = x.reshape(1, -1).to(torch.bfloat16)
    _search_check(x, "exact loss ties, c in [0.5, 1]")
    _search_check(x, "exact loss ties, c in [0.5, 1.5]", c_hi=1.5)
