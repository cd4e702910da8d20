"""The grid barrier's bounded wait, forced from the host.  With the poll
limit at zero, the one-pass NVFP4 quantize (bf16 input, the resident kernel)
and the one-launch MXFP4 linear either find every workgroup already arrived at
their first poll (then their results are the exact ones) or give up: they set
FLAG_BARRIER_TIMEOUT in the status word and end normally, with unspecified
outputs, and a checked call raises.  With the default limit back, a fresh
workspace, or the same one zeroed again, gives bit-exact results."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import workloads
from tests._gpu import announce, assert_bytes_equal, dev, f32_bits, host_u8, oracle_view

pytestmark = pytest.mark.gpu


def _with_poll_limit(polls, fn):
    prev = fp4.debug_barrier_spin_limit(polls)
    try:
        return fn()
    finally:
        fp4.debug_barrier_spin_limit(prev)


def _status(device):
    return torch.zeros(1, dtype=torch.int32, device=device)


def _timed_out(st) -> bool:
    f = int(st.item())
    assert f & ~fp4.FLAG_BARRIER_TIMEOUT == 0, f"unexpected flags {f:#x}"
    return f != 0


def test_nv_resident_quantize_times_out_and_recovers():
    x = workloads.nvfp4_weight()  # 8192 x 8192 bf16: the resident kernel, 256 workgroups
    p, s, sg, flags = oracle.nv_quantize(oracle_view(x))
    assert flags == 0
    xd = dev(x)

    def exact(got, what):
        codes, scales, s_g = got
        torch.cuda.synchronize()
        assert f32_bits(s_g.cpu().numpy())[0] == f32_bits([sg])[0], f"{what}: s_g"
        assert_bytes_equal(host_u8(scales), s, f"{what}: NV scales")
        assert_bytes_equal(host_u8(codes), p, f"{what}: NV codes")

    ws = fp4.new_workspace(*x.shape, xd.device)
    st = _status(xd.device)
    announce("nvfp4 quantize 8192x8192 bf16, poll limit 0, unchecked")
    got = _with_poll_limit(0, lambda: fp4.quantize_nvfp4(xd, check=False, status=st, workspace=ws))
    torch.cuda.synchronize()
    timed_out = _timed_out(st)
    print(f"barrier timeout: {timed_out}", flush=True)
    if not timed_out:
        exact(got, "poll limit 0, every workgroup on time")

    announce("nvfp4 quantize 8192x8192 bf16, poll limit 0, checked")
    ws2 = fp4.new_workspace(*x.shape, xd.device)
    try:
        got = _with_poll_limit(0, lambda: fp4.quantize_nvfp4(xd, workspace=ws2))
    except fp4.Fp4Error as e:
        assert "timed out" in str(e)
    else:
        exact(got, "checked call, poll limit 0, every workgroup on time")

    announce("nvfp4 quantize 8192x8192 bf16, default limit, fresh and re-zeroed workspaces")
    assert fp4.debug_barrier_spin_limit(fp4.BARRIER_SPIN_LIMIT_DEFAULT) == fp4.BARRIER_SPIN_LIMIT_DEFAULT
    exact(fp4.quantize_nvfp4(xd, workspace=fp4.new_workspace(*x.shape, xd.device)), "fresh workspace")
    ws.zero_()
    exact(fp4.quantize_nvfp4(xd, workspace=ws), "re-zeroed workspace")
    exact(fp4.quantize_nvfp4(xd, workspace=ws), "re-zeroed workspace, second call")


def test_one_launch_linear_times_out_and_recovers():
    M, N, K = 128, 8192, 8192
    a, bt = workloads.gemm_operands(M, N, K, seed_a=0, seed_b=1)
    bp, bsc, f2 = oracle.mx_quantize(bt.numpy())
    ap, asc, f1 = oracle.mx_quantize(oracle_view(a))
    assert f1 == 0 and f2 == 0
    xd = dev(a)
    bt_d = dev(torch.from_numpy(bp.reshape(N, K // 2)))
    bs_d = dev(torch.from_numpy(bsc.reshape(N, K // 32)))
    announce(f"linear mxfp4 {M}x{N}x{K} two launches (no barrier)")
    want, _ = fp4.linear_mxfp4(xd, bt_d, bs_d, torch.float32, one_launch=False)
    torch.cuda.synchronize()
    want = want.cpu()

    def exact(got, what):
        c, (ac, asd) = got
        torch.cuda.synchronize()
        assert_bytes_equal(host_u8(asd), asc, f"{what}: A scales")
        assert_bytes_equal(host_u8(ac), ap, f"{what}: A codes")
        assert torch.equal(c.cpu(), want), f"{what}: C"

    ws = fp4.new_workspace(M, K, xd.device)
    st = _status(xd.device)
    announce(f"linear mxfp4 {M}x{N}x{K} one launch, poll limit 0")
    got = _with_poll_limit(0, lambda: fp4.linear_mxfp4(xd, bt_d, bs_d, torch.float32, status=st,
                                                       workspace=ws, check=False))
    torch.cuda.synchronize()
    timed_out = _timed_out(st)
    print(f"barrier timeout: {timed_out}", flush=True)
    if not timed_out:
        exact(got, "poll limit 0, every workgroup on time")

    announce(f"linear mxfp4 {M}x{N}x{K} one launch, default limit, re-zeroed workspace")
    ws.zero_()
    exact(fp4.linear_mxfp4(xd, bt_d, bs_d, torch.float32, workspace=ws), "re-zeroed workspace")
    exact(fp4.linear_mxfp4(xd, bt_d, bs_d, torch.float32, workspace=ws), "second call")
    assert np.isfinite(want.numpy()).all()
