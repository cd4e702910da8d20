"""The grid barrier's bounded wait and its fallback.  The one-pass NVFP4
quantize (bf16 input, the resident kernel) and the one-launch MXFP4 linear
meet at a grid barrier; a workgroup that stops waiting (poll limit reached,
e.g. because another kernel holds CUs) finishes by a fallback that gives the
same result: the NVFP4 kernel reads the missing slices' amax itself, the
linear quantizes all of A itself.  FLAG_BARRIER_TIMEOUT only records that it
happened.  Forced from the host (the debug entry points with poll limit 0:
every kernel still exits normally), and by two calls running at once on two
streams, the results must be bit-exact; calls after a fallback must be too
(the barrier's epoch rules keep stale slots from matching)."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import workloads
from tests._gpu import announce, assert_bytes_equal, dev, f32_bits, host_u8, oracle_view

pytestmark = pytest.mark.gpu


def _status(device):
    return torch.zeros(1, dtype=torch.int32, device=device)


def _flags_ok(st) -> bool:
    """Only the informational timeout bit may be set; returns whether it is."""
    f = int(st.item())
    assert f & ~fp4.FLAG_BARRIER_TIMEOUT == 0, f"unexpected flags {f:#x}"
    return f != 0


def _nv_reference(x):
    p, s, sg, flags = oracle.nv_quantize(oracle_view(x))
    assert flags == 0
    return p, s, sg


def _nv_exact(got, ref, what):
    p, s, sg = ref
    codes, scales, s_g = got
    torch.cuda.synchronize()
    assert f32_bits(s_g.cpu().numpy())[0] == f32_bits([sg])[0], f"{what}: s_g"
    assert_bytes_equal(host_u8(scales), s, f"{what}: NV scales")
    assert_bytes_equal(host_u8(codes), p, f"{what}: NV codes")


def test_nv_resident_quantize_fallback_is_exact():
    x = workloads.nvfp4_weight()  # 8192 x 8192 bf16: the resident kernel, 256 workgroups
    ref = _nv_reference(x)
    xd = dev(x)
    ws = fp4.new_workspace(*x.shape, xd.device)
    timeouts = 0
    for i in range(3):
        st = _status(xd.device)
        announce(f"nvfp4 quantize 8192x8192 bf16, poll limit 0, call {i}")
        got = fp4.quantize_nvfp4(xd, check=False, status=st, workspace=ws, spin_limit=0)
        torch.cuda.synchronize()
        timeouts += _flags_ok(st)
        _nv_exact(got, ref, f"poll limit 0, call {i}")
    print(f"calls that took the fallback: {timeouts} of 3", flush=True)
    # the same workspace, not re-zeroed, with the default limit: the epoch
    # rules keep the slots left by the fallbacks from matching
    announce("nvfp4 quantize 8192x8192 bf16, default limit after fallbacks")
    for i in range(2):
        st = _status(xd.device)
        got = fp4.quantize_nvfp4(xd, check=False, status=st, workspace=ws)
        torch.cuda.synchronize()
        _flags_ok(st)
        _nv_exact(got, ref, f"default limit, call {i}")
    # a different tensor through the same workspace, fallback then not
    x2 = workloads.nvfp4_weight(seed=1)
    ref2 = _nv_reference(x2)
    x2d = dev(x2)
    announce("nvfp4 quantize 8192x8192 bf16 seed 1, poll limit 0 then default, same workspace")
    _nv_exact(fp4.quantize_nvfp4(x2d, workspace=ws, spin_limit=0), ref2, "seed 1, limit 0")
    _nv_exact(fp4.quantize_nvfp4(xd, workspace=ws), ref, "seed 0 after seed 1")
    _nv_exact(fp4.quantize_nvfp4(x2d, workspace=ws), ref2, "seed 1 after seed 0")


def test_nv_resident_quantize_two_streams_at_once():
    # Two one-pass quantizes enqueued on two streams, each with its own
    # workspace: they may share the CUs, so neither grid need be resident as a
    # whole.  Both must be exact.
    xa, xb = workloads.nvfp4_weight(), workloads.nvfp4_weight(seed=1)
    refs = [_nv_reference(xa), _nv_reference(xb)]
    xs = [dev(xa), dev(xb)]
    wss = [fp4.new_workspace(*xa.shape, "cuda") for _ in range(2)]
    outs = [fp4.quantize_nvfp4(x, workspace=w) for x, w in zip(xs, wss)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    timeouts = 0
    for rep in range(4):
        sts = [_status("cuda") for _ in range(2)]
        announce(f"nvfp4 quantize 8192x8192 bf16 on two streams, round {rep}")
        for k in range(2):
            streams[k].wait_stream(torch.cuda.current_stream())  # the zeroed status words
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                fp4.quantize_nvfp4(xs[k], check=False, out=outs[k], status=sts[k], workspace=wss[k])
        torch.cuda.synchronize()
        for k in range(2):
            timeouts += _flags_ok(sts[k])
            _nv_exact(outs[k], refs[k], f"stream {k}, round {rep}")
    print(f"calls that took the fallback: {timeouts} of 8", flush=True)


def _linear_setup(M, N, K):
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
    return xd, bt_d, bs_d, ap, asc, want.cpu()


def test_one_launch_linear_fallback_is_exact():
    M, N, K = 128, 8192, 8192
    xd, bt_d, bs_d, ap, asc, want = _linear_setup(M, N, K)

    def exact(got, what):
        c, (ac, asd) = got
        torch.cuda.synchronize()
        assert_bytes_equal(host_u8(asd), asc, f"{what}: A scales")
        assert_bytes_equal(host_u8(ac), ap, f"{what}: A codes")
        assert torch.equal(c.cpu(), want), f"{what}: C"

    ws = fp4.new_workspace(M, K, xd.device)
    timeouts = 0
    for i in range(2):
        st = _status(xd.device)
        announce(f"linear mxfp4 {M}x{N}x{K} one launch, poll limit 0, call {i}")
        got = fp4.linear_mxfp4(xd, bt_d, bs_d, torch.float32, status=st, workspace=ws,
                               check=False, spin_limit=0)
        torch.cuda.synchronize()
        timeouts += _flags_ok(st)
        exact(got, f"poll limit 0, call {i}")
    print(f"calls that took the fallback: {timeouts} of 2", flush=True)
    announce(f"linear mxfp4 {M}x{N}x{K} one launch, default limit, same workspace")
    exact(fp4.linear_mxfp4(xd, bt_d, bs_d, torch.float32, workspace=ws), "default limit")
    exact(fp4.linear_mxfp4(xd, bt_d, bs_d, torch.float32, workspace=ws), "second call")
    assert np.isfinite(want.numpy()).all()


def test_one_launch_linear_two_streams_at_once():
    M, N, K = 128, 8192, 8192
    xd, bt_d, bs_d, ap, asc, want = _linear_setup(M, N, K)
    wss = [fp4.new_workspace(M, K, "cuda") for _ in range(2)]
    outs = [(torch.empty(M, N, dtype=torch.float32, device="cuda"),
             (torch.empty(M, K // 2, dtype=torch.uint8, device="cuda"),
              torch.empty(M, K // 32, dtype=torch.uint8, device="cuda"))) for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for rep in range(3):
        sts = [_status("cuda") for _ in range(2)]
        announce(f"linear mxfp4 {M}x{N}x{K} one launch on two streams, round {rep}")
        for k in range(2):
            streams[k].wait_stream(torch.cuda.current_stream())  # the zeroed status words
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                fp4.linear_mxfp4(xd, bt_d, bs_d, out=outs[k][0], a_out=outs[k][1], status=sts[k],
                                 workspace=wss[k], check=False)
        torch.cuda.synchronize()
        for k in range(2):
            _flags_ok(sts[k])
            c, (ac, asd) = outs[k]
            assert_bytes_equal(host_u8(asd), asc, f"stream {k}: A scales")
            assert_bytes_equal(host_u8(ac), ap, f"stream {k}: A codes")
            assert torch.equal(c.cpu(), want), f"stream {k}, round {rep}: C"
