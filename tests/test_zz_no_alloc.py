"""GPU test of fp4_quantize_nvfp4_noalloc, the NVFP4 quantize entry point that
allocates nothing (its workspace is the library's fixed per-GPU scratch):
through the C ABI, its codes, scale bytes, tensor scale and status must equal
those of fp4_quantize_nvfp4 with a caller workspace, bit for bit, call after
call, with inputs that shrink and grow between calls (the scratch keeps the
previous call's grid-barrier state)."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import workloads
from tests._gpu import announce, assert_bytes_equal, dev, f32_bits, host_u8, oracle_view

pytestmark = pytest.mark.gpu


def _both(x: torch.Tensor, what: str):
    announce(f"nvfp4 noalloc vs workspace entry point: {what} {tuple(x.shape)} {x.dtype}")
    xd = dev(x)
    st_a = torch.zeros(1, dtype=torch.int32, device="cuda")
    st_b = torch.zeros(1, dtype=torch.int32, device="cuda")
    a = fp4.quantize_nvfp4_noalloc(xd, check=False, status=st_a)
    b = fp4.quantize_nvfp4(xd, check=False, status=st_b)
    torch.cuda.synchronize()
    assert int(st_a.item()) == 0, f"{what}: noalloc status {int(st_a.item())}"
    assert int(st_b.item()) == 0, f"{what}: workspace status {int(st_b.item())}"
    assert f32_bits(a[2].cpu().numpy())[0] == f32_bits(b[2].cpu().numpy())[0], f"{what}: s_g"
    assert_bytes_equal(host_u8(a[1]), host_u8(b[1]), f"{what}: scale bytes")
    assert_bytes_equal(host_u8(a[0]), host_u8(b[0]), f"{what}: codes")
    return a


def test_noalloc_equals_workspace_entry_point_shrinking_inputs():
    # 1: the 8192 x 8192 bf16 weight (one-pass kernel, one workgroup per CU)
    _both(workloads.nvfp4_weight(), "weight 8192x8192 bf16")
    # 2: a smaller bf16 tensor right after (one-pass kernel on fewer
    #    workgroups, the scratch's barrier slots left by call 1)
    x = workloads.nvfp4_weight(1000, 2048, seed=3)
    a = _both(x, "weight 1000x2048 bf16")
    p, s, sg, flags = oracle.nv_quantize(oracle_view(x))
    assert flags == 0
    assert f32_bits(a[2].cpu().numpy())[0] == f32_bits([sg])[0]
    assert_bytes_equal(host_u8(a[1]), s, "1000x2048 vs oracle: scale bytes")
    assert_bytes_equal(host_u8(a[0]), p, "1000x2048 vs oracle: codes")
    # 3: fp32 input (two-pass path: tensor-amax partials in the scratch)
    _both(workloads.tiny_roundtrip(), "tiny 4096 fp32")
    # 4: large again, then ragged small, back to back on one stream
    _both(workloads.nvfp4_weight(4096, 8192, seed=5), "weight 4096x8192 bf16")
    _both(workloads.nvfp4_weight(3, 48, seed=6), "3x48 bf16")


def test_noalloc_stream_ordered_calls_without_sync():
    # several calls queued on one stream before any synchronisation: each
    # call's barrier state follows the previous one's in stream order
    xs = [workloads.nvfp4_weight(r, c, seed=10 + i) for i, (r, c) in
          enumerate([(2048, 4096), (512, 512), (2048, 4096), (64, 8192)])]
    announce("nvfp4 noalloc: four calls queued on one stream")
    outs = [fp4.quantize_nvfp4_noalloc(dev(x), check=False) for x in xs]
    torch.cuda.synchronize()
    for i, (x, o) in enumerate(zip(xs, outs)):
        ref = fp4.quantize_nvfp4(dev(x))
        torch.cuda.synchronize()
        assert f32_bits(o[2].cpu().numpy())[0] == f32_bits(ref[2].cpu().numpy())[0], i
        assert_bytes_equal(host_u8(o[1]), host_u8(ref[1]), f"call {i}: scale bytes")
        assert_bytes_equal(host_u8(o[0]), host_u8(ref[0]), f"call {i}: codes")


def test_noalloc_reports_data_errors():
    # the status contract is fp4_quantize_nvfp4's: non-finite input is flagged
    x = workloads.nvfp4_weight(256, 256, seed=7)
    x[17, 33] = float("nan")
    announce("nvfp4 noalloc: NaN input flagged")
    with pytest.raises(ValueError):
        fp4.quantize_nvfp4_noalloc(dev(x))
    # and the next call is unaffected
    _both(workloads.nvfp4_weight(256, 256, seed=8), "256x256 bf16 after a flagged call")
