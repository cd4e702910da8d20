"""GPU parity: MXFP4 and NVFP4 quantization, bit-exact against the oracle on
codes, scale bytes and the tensor scale, on the five workloads' inputs and on
adversarial tensors (ties, signed zero, subnormals, saturation, zero blocks,
extreme tensor scales) and ragged sizes."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
import workloads
from tests._gpu import announce, assert_bytes_equal, dev, f32_bits, host_u8, oracle_view

pytestmark = pytest.mark.gpu


def check_mx(x: torch.Tensor, what: str):
    announce(f"mxfp4 quantize {what} {tuple(x.shape)} {x.dtype}")
    codes, scales = fp4.quantize_mxfp4(dev(x))
    torch.cuda.synchronize()
    p, s, flags = oracle.mx_quantize(oracle_view(x))
    assert flags == 0
    assert_bytes_equal(host_u8(scales), s, f"{what}: MX scales")
    assert_bytes_equal(host_u8(codes), p, f"{what}: MX codes")


def check_nv(x: torch.Tensor, what: str):
    announce(f"nvfp4 quantize {what} {tuple(x.shape)} {x.dtype}")
    codes, scales, s_g = fp4.quantize_nvfp4(dev(x))
    torch.cuda.synchronize()
    p, s, sg, flags = oracle.nv_quantize(oracle_view(x))
    assert flags == 0
    assert f32_bits(s_g.cpu().numpy())[0] == f32_bits([sg])[0], f"{what}: s_g"
    assert_bytes_equal(host_u8(scales), s, f"{what}: NV scales")
    assert_bytes_equal(host_u8(codes), p, f"{what}: NV codes")


# ---- the workloads' inputs -------------------------------------------------

def test_tiny_roundtrip_input_both_formats():
    x = workloads.tiny_roundtrip()
    check_mx(x, "tiny 4096 fp32")
    check_nv(x, "tiny 4096 fp32")


def test_nvfp4_weight_8192_full():
    x = workloads.nvfp4_weight()
    check_nv(x, "weight 8192x8192 bf16")
    check_mx(x, "weight 8192x8192 bf16")


def test_mxfp4_activation_16384x7168_full():
    check_mx(workloads.mxfp4_activation(), "activation 16384x7168 bf16")


def test_nv_one_pass_per_workgroup_ranges():
    # The one-pass kernel at 8192 x 8192 holds, in workgroup w of 256, the
    # 4096-element pieces p with p % 256 == w.  Each workgroup's pieces get
    # their own scale 2^-(w % 13) (a different range of block amaxes, so a
    # different part of the scale table) and every sixteenth workgroup's are
    # all zero (no nonzero block at all); the tensor amax stays in workgroup 0.
    x = workloads.nvfp4_weight().float().reshape(-1, 4096)
    w = torch.arange(x.shape[0]) % 256
    scale = torch.pow(2.0, -(w % 13).double()).float()
    scale[w % 16 == 5] = 0.0
    x = (x * scale[:, None]).reshape(8192, 8192)
    x[0, 0] = 0.2  # above every other magnitude (N(0, 0.02^2) data)
    check_nv(x.to(torch.bfloat16), "per-workgroup magnitude ranges 8192x8192 bf16")


# ---- exhaustive conversion sweep --------------------------------------------

def _mx_sweep_tensor() -> torch.Tensor:
    """bf16 values at every E8M0 exponent: for each block exponent e, blocks
    hold an anchor just below 2^(e+3) (so the exponent is e) and 31 other
    values, both signs: every bf16 pattern in the seven binades that can
    round to a nonzero code (all patterns for e <= -120, where subnormal
    quotients occur), and a sample of the smaller ones."""
    allbits = np.arange(0, 0x7F80, dtype=np.uint32)  # finite non-negative bf16
    blocks = []
    for byte in range(0, 253):
        e = byte - 127
        if e == -127:
            anchor_bits = (2 << 7) | 0x7F   # just below 2^-124: floor(log2) = -125
        else:
            anchor_bits = ((e + 2 + 127) << 7) | 0x7F
        vals = allbits[allbits <= anchor_bits]
        lo = ((e - 4 + 127) << 7) if e > -120 else 0
        vals = np.concatenate([vals[vals >= lo], vals[vals < lo][::97]])
        vals = vals | np.where(np.arange(vals.size) % 2 == 1, 0x8000, 0).astype(np.uint32)
        vals = np.concatenate([vals, np.zeros((-vals.size) % 31, np.uint32)]).reshape(-1, 31)
        anchor = np.full((vals.shape[0], 1), anchor_bits, np.uint32)
        blocks.append(np.concatenate([anchor, vals], axis=1))
    b = np.concatenate(blocks).astype(np.uint16)
    b = np.concatenate([b, np.zeros(((-b.shape[0]) % 16, 32), np.uint16)])
    return torch.from_numpy(b.reshape(-1, 512).view(np.int16)).view(torch.bfloat16)


def test_mx_every_bf16_value_at_every_exponent():
    check_mx(_mx_sweep_tensor(), "exhaustive bf16 x E8M0 sweep")


def _mx_fp32_midpoint_tensor() -> torch.Tensor:
    """fp32 values on and one ulp around every E2M1 decision point, at several
    block exponents, plus signed zeros and subnormals."""
    pts = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 0.5, 1.0, 4.0], np.float32)
    rows = []
    for e in (-127, -126, -100, -3, 0, 5, 60, 125):
        s = np.float32(2.0 ** e)
        anchor = np.float32(np.nextafter(np.float32(8.0), np.float32(0)) * s) if e > -127 else np.float32(2.0 ** -125)
        vals = []
        for p in pts:
            v = np.float32(p * s)
            vals += [np.nextafter(v, np.float32(0)), v, np.nextafter(v, np.float32(np.inf))]
        vals = np.array(vals, np.float32)
        vals = np.concatenate([vals, -vals, [0.0, -0.0, 1e-45, -1e-45, 1e-40]]).astype(np.float32)
        vals = np.concatenate([vals, np.zeros((-vals.size) % 31, np.float32)]).reshape(-1, 31)
        rows.append(np.concatenate([np.full((vals.shape[0], 1), anchor, np.float32), vals], 1))
    x = torch.from_numpy(np.concatenate(rows).reshape(-1))
    return x[: (x.numel() // 32) * 32].reshape(-1, 32)


def test_mx_fp32_every_midpoint_and_subnormal():
    check_mx(_mx_fp32_midpoint_tensor(), "fp32 midpoints")


# ---- adversarial NVFP4 ------------------------------------------------------

def test_nv_ties_signed_zero_and_zero_blocks():
    # a 2688 block fixes s_g = 1; a block with amax 6 has s_b = 1 (0x38), so
    # alpha = 1 and the elements below sit exactly on E2M1 midpoints
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -5.0, -0.0, 0.0, 1e-30,
            -1e-30, 2.0]
    x = np.concatenate([np.full(16, 2688.0), mids, np.zeros(16), [-0.0] * 16,
                        [0.3, 0.6, 0.9, 1.2, 1.8, 2.4, 3.6, 0.0] * 2, [0.4] * 15 + [3.6]])
    check_nv(torch.tensor(x, dtype=torch.float32).reshape(1, -1), "ties/zeros fp32")
    check_nv(torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).reshape(1, -1), "ties/zeros bf16")


def test_nv_block_scale_ties():
    # block amaxes placed exactly on E4M3 midpoints times 6 s_g (s_g = 1)
    rng = np.random.default_rng(0)
    blocks = [np.full(16, 2688.0, np.float32)]
    e4 = [oracle.e4m3_value(c) for c in range(127)]
    for c in range(1, 126):   # the 0|1 tie rounds to code 0: an underflow, tested below
        m = (e4[c] + e4[c + 1]) / 2 * 6.0
        b = rng.uniform(-m, m, 16).astype(np.float32)
        b[3] = np.float32(m)
        blocks.append(b)
    x = torch.from_numpy(np.concatenate(blocks)).reshape(1, -1)
    check_nv(x, "E4M3 midpoint amaxes")
    # amax 6 * 2^-10 sits halfway between codes 0 and 1: even code 0, so the
    # nonzero block's scale underflows, on both sides
    tie0 = np.concatenate([np.full(16, 2688.0, np.float32), np.full(16, 6 * 2.0 ** -10, np.float32)])
    assert oracle.nv_quantize(tie0)[3] & oracle.FLAG_SCALE_UNDERFLOW
    announce("nvfp4 quantize E4M3 0|1 tie underflow")
    with pytest.raises(ValueError):
        fp4.quantize_nvfp4(dev(torch.from_numpy(tie0).reshape(1, -1)))


@pytest.mark.parametrize("scale_exp", [-140, -130, -126, -120, -100, -64, -20, 0, 20, 64, 100, 110])
def test_nv_extreme_tensor_scales(scale_exp):
    # tensors at every magnitude, including subnormal s_g and subnormal alpha
    g = torch.Generator().manual_seed(scale_exp + 1000)
    x = torch.randn(64, 256, generator=g) * torch.rand(64, 256, generator=g) ** 4
    x = (x * 2.0 ** scale_exp).to(torch.float32)
    p, s, sg, flags = oracle.nv_quantize(x.numpy().reshape(-1))
    if flags:
        pytest.skip("oracle reports underflow for this magnitude (covered by the status test)")
    check_nv(x, f"magnitude 2^{scale_exp}")


def test_nv_bf16_subnormals_and_ragged_sizes():
    g = torch.Generator().manual_seed(5)
    for rows, cols in [(1, 16), (3, 48), (5, 1040), (7, 4112), (129, 80)]:
        x = torch.randn(rows, cols, generator=g) * 0.02
        x[0, : min(cols, 8)] = torch.tensor([1e-39, -1e-39, 3e-40, 0.0, -0.0, 1e-38, 2e-38, -5e-39][: min(cols, 8)])
        check_nv(x.to(torch.bfloat16), f"ragged {rows}x{cols}")
        if cols % 32 == 0:
            check_mx(x.to(torch.bfloat16), f"ragged {rows}x{cols}")


def test_mx_ragged_fp32_and_bf16():
    g = torch.Generator().manual_seed(6)
    for rows, cols in [(1, 32), (3, 96), (11, 4128), (257, 160)]:
        x = torch.randn(rows, cols, generator=g) * torch.rand(rows, cols, generator=g) * 100
        check_mx(x, f"ragged fp32 {rows}x{cols}")
        check_mx(x.to(torch.bfloat16), f"ragged bf16 {rows}x{cols}")


# ---- status flags -------------------------------------------------------------

def test_status_flags_match_the_contract():
    announce("status flags")
    x = torch.zeros(2, 64, dtype=torch.float32)
    x[1, 5] = float("nan")
    with pytest.raises(ValueError):
        fp4.quantize_mxfp4(dev(x))
    with pytest.raises(ValueError):
        fp4.quantize_nvfp4(dev(x))
    tiny = torch.full((1, 16), 1e-42, dtype=torch.float32)       # s_g underflows
    with pytest.raises(ValueError):
        fp4.quantize_nvfp4(dev(tiny))
    blk = torch.tensor([2688.0] * 16 + [1e-10] * 16).reshape(1, 32)  # block scale underflows
    with pytest.raises(ValueError):
        fp4.quantize_nvfp4(dev(blk))
    z = torch.zeros(4, 64, dtype=torch.bfloat16)                  # all-zero tensor is fine
    codes, scales, sg = fp4.quantize_nvfp4(dev(z))
    assert float(sg.item()) == 1.0 and bool((scales == 0x38).all()) and bool((codes == 0).all())


def test_deterministic_repeat():
    x = dev(workloads.nvfp4_weight(1024, 4096, seed=3))
    announce("determinism nvfp4/mxfp4 1024x4096")
    a = fp4.quantize_nvfp4(x)
    b = fp4.quantize_nvfp4(x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    c = fp4.quantize_mxfp4(x)
    d = fp4.quantize_mxfp4(x)
    for u, v in zip(c, d):
        assert torch.equal(u, v)



# ---- one-pass (tensor on chip) and two-pass NVFP4 paths ------------------------

def test_nv_bf16_beyond_on_chip_capacity_takes_two_passes():
    # 10240 x 8192 bf16 (168 MB) exceeds what the CUs hold at once, so this
    # runs the tensor-amax + quantize kernels; 8192 x 8192 above runs the
    # one-pass kernel
    x = workloads.nvfp4_weight(10240, 8192, seed=7)
    check_nv(x, "weight 10240x8192 bf16")


def test_nv_bf16_largest_one_pass_with_ragged_tail():
    # just below the on-chip capacity: 64 chunks per lane, the last grid step
    # partly outside the tensor (clamped loads, predicated stores)
    for i, (r, c) in enumerate([(8191, 8192), (8192, 8176)]):
        check_nv(workloads.nvfp4_weight(r, c, seed=40 + i), f"weight {r}x{c} bf16")


def test_nv_workspace_reused_across_sizes_and_graph_replays():
    # the barrier epoch lives in the workspace: reuse it across calls of
    # different grid sizes (stale slots from larger grids must never match)
    # and across replays of a captured graph, with eager work in between
    ws = fp4.new_workspace(8192, 8192, "cuda")
    shapes = [(8192, 8192), (64, 1024), (4096, 8192), (3, 48), (8192, 8192), (1024, 4096)]
    for i, (r, c) in enumerate(shapes):
        x = workloads.nvfp4_weight(r, c, seed=20 + i)
        announce(f"nvfp4 quantize shared workspace call {i} {r}x{c}")
        codes, scales, s_g = fp4.quantize_nvfp4(dev(x), workspace=ws)
        torch.cuda.synchronize()
        p, s, sg, flags = oracle.nv_quantize(oracle_view(x))
        assert flags == 0
        assert f32_bits(s_g.cpu().numpy())[0] == f32_bits([sg])[0]
        assert_bytes_equal(host_u8(scales), s, f"call {i}: NV scales")
        assert_bytes_equal(host_u8(codes), p, f"call {i}: NV codes")

    x = dev(workloads.nvfp4_weight(2048, 4096, seed=31))
    p, s, sg, flags = oracle.nv_quantize(oracle_view(x))
    codes = torch.empty(2048, 2048, dtype=torch.uint8, device="cuda")
    scales = torch.empty(2048, 256, dtype=torch.uint8, device="cuda")
    s_g = torch.empty(1, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    announce("nvfp4 quantize graph capture 2048x4096")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the graph
        fp4.quantize_nvfp4(x, check=False, out=(codes, scales, s_g), status=status, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fp4.quantize_nvfp4(x, check=False, out=(codes, scales, s_g), status=status, workspace=ws)
    for rep in range(4):
        codes.zero_()
        scales.zero_()
        y = fp4.quantize_nvfp4(x, workspace=ws)      # eager call on the same workspace
        torch.cuda.synchronize()
        announce(f"nvfp4 graph replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert_bytes_equal(host_u8(scales), s, f"replay {rep}: NV scales")
        assert_bytes_equal(host_u8(codes), p, f"replay {rep}: NV codes")
        assert torch.equal(y[0], codes) and torch.equal(y[1], scales)


# ---- the one-multiply quotient and its guard ------------------------------------

def _bf16(v) -> np.ndarray:
    """Round float64 values to bf16 (nearest even) and return them as float32."""
    f = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _product_errs_cases(max_cases=6):
    """bf16 tensors (one row: [tensor-amax block | test block]) in which the
    plain product x * RN32(1/alpha) would give a wrong E2M1 code for some
    element of the test block: found by search over tensor amaxes A (which
    fix s_g) and block codes c (alpha = RN32(s_g E4M3(c)))."""
    from tests.test_fast_quotient_rule import all_bf16_finite, codes_both_ways
    xs = all_bf16_finite()
    xs = xs[xs > 0]
    cases = []
    rng = np.random.default_rng(21)
    e4 = np.array([oracle.e4m3_value(c) for c in range(127)], np.float64)
    for A in _bf16(rng.uniform(1.0, 4096.0, 4000)):
        s_g = np.float32(np.float64(A) / 2688.0)
        for c in range(96, 127):
            alpha = np.float32(s_g * np.float32(e4[c]))
            x = xs[(xs >= 0.2 * alpha) & (xs <= 5.5 * alpha)]
            cd, cm = codes_both_ways(x, alpha)
            bad = x[cd != cm]
            if bad.size == 0:
                continue
            ag = _bf16([6.0 * np.float64(s_g) * e4[c]])[0]
            if not (ag > bad.max()) or ag >= A:
                continue
            block = np.concatenate([[ag], bad[:15]]).astype(np.float32)
            block = np.concatenate([block, np.zeros(16 - block.size, np.float32)])
            row = np.concatenate([[A], np.zeros(15, np.float32), block]).astype(np.float32)
            t = torch.from_numpy(row).reshape(1, 32).to(torch.bfloat16)
            p, s, sg, flags = oracle.nv_quantize(oracle_view(t))
            if flags or s[1] != c:
                continue
            cases.append((t, c, bad[:15]))
            break
        if len(cases) >= max_cases:
            break
    return cases


def test_nv_one_multiply_quotient_guard():
    from tests.test_fast_quotient_rule import codes_both_ways
    cases = _product_errs_cases()
    assert len(cases) >= 3, "search found too few sensitive tensors"
    for i, (t, c, bad) in enumerate(cases):
        # sensitivity: the unguarded product disagrees with the oracle here
        p, s, sg, flags = oracle.nv_quantize(oracle_view(t))
        alpha = np.float32(np.float32(sg) * np.float32(oracle.e4m3_value(c)))
        cd, cm = codes_both_ways(bad, alpha)
        assert (cd != cm).any()
        check_nv(t, f"one-multiply guard case {i} (code {c})")


# ---- every form of the one-pass kernel's quantize loop ---------------------------

def _one_pass_form(A: float) -> str:
    """Which loop the one-pass kernel runs for a bf16 tensor of amax A (the
    kernel decides from s_g alone): restated from the rules it follows."""
    sg = np.float32(np.float64(A) / 2688.0)
    alphas = [np.float32(sg * np.float32(oracle.e4m3_value(c))) for c in range(1, 127)]
    if any(0 < a < 2.0 ** -90 for a in alphas):
        return "compact"
    if sg >= 2.0 ** -126 and (sg.view(np.uint32) & 0xFFF) == 0:
        return "short"
    return "full"


@pytest.mark.parametrize("M,exp,form", [(168, -4, "short"), (231, 20, "short"), (129, -4, "full"),
                                        (131, -4, "full"), (131, -90, "compact"),
                                        (168, -100, "compact")])
def test_nv_one_pass_forms(M, exp, form):
    # amax significand M: 168 = 21 * 8 and 231 = 21 * 11 make s_g short;
    # 129 = 3 * 43 and the prime 131 make it a repeating fraction; the tiny
    # amaxes need operand scaling for the smallest codes
    A = float(M) * 2.0 ** exp
    assert _one_pass_form(A) == form
    g = torch.Generator().manual_seed(M + exp)
    for rows, cols in [(2048, 4096), (1000, 4112)]:   # exact cover, and ragged
        x = torch.randn(rows, cols, generator=g) * (A / 8)
        x = x.clamp(-A, A)
        x[rows // 2, cols // 3] = -A
        check_nv(x.to(torch.bfloat16), f"one-pass form {form} amax {A!r} {rows}x{cols}")


def _bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _amax_sweep_tensor(A: float, seed: int, rows: int, cols: int) -> torch.Tensor:
    """bf16 blocks whose amaxes run through every bf16 magnitude that gets a
    nonzero block scale under the tensor scale of amax A (A itself a bf16
    value), repeated to fill rows x cols, with a zero block in every 64; the
    other elements of a block are smaller, of random sign."""
    a_bits = int(np.float32(A).view(np.uint32)) >> 16
    assert _bf16_value(np.array([a_bits]))[0] == np.float32(A)
    sg = np.float64(np.float32(np.float64(A) / 2688.0))
    # E4M3 code >= 1 exactly when amax / (6 s_g) > 2^-10 (the tie goes to 0)
    thr = 6.0 * sg * 2.0 ** -10
    lo = int(np.float32(thr).view(np.uint32)) >> 16
    while np.float64(_bf16_value(np.array([lo]))[0]) <= thr:
        lo += 1
    pats = np.arange(lo, a_bits + 1, dtype=np.uint32)
    nblk = rows * cols // 16
    rng = np.random.default_rng(seed)
    amax = _bf16_value(pats[np.arange(nblk) % len(pats)]).astype(np.float64)
    amax[rng.permutation(nblk)[: nblk // 64]] = 0.0
    amax[0] = np.float64(np.float32(A))  # the tensor amax is present
    x = rng.uniform(0.0, 1.0, (nblk, 16)) * amax[:, None]
    x[np.arange(nblk), rng.integers(0, 16, nblk)] = amax
    x *= np.where(rng.random((nblk, 16)) < 0.5, -1.0, 1.0)
    # fp32 first (exact for the amaxes), then RNE to bf16: never above a
    # block's amax, which is a bf16 value
    return torch.from_numpy(x.astype(np.float32).reshape(rows, cols)).to(torch.bfloat16)


@pytest.mark.parametrize("M,exp", [(231, -11), (235, -11), (131, -100), (3, -121), (255, 119)])
def test_nv_every_block_amax_under_one_tensor_scale(M, exp):
    # every reachable block amax, so every code guess and its two-threshold
    # settlement runs against the oracle; tensor scales: short (231), generic
    # (235), operands scaled (tiny), subnormal s_g, and near the bf16 maximum
    A = float(M) * 2.0 ** exp
    for rows, cols in [(2048, 4096), (333, 1040)]:   # exact cover, and ragged
        x = _amax_sweep_tensor(A, M + exp + rows, rows, cols)
        check_nv(x, f"every block amax under amax {A!r} ({_one_pass_form(A)}) {rows}x{cols}")


# ---- hazard values of the one-pass kernel's per-code reciprocal --------------------

def _hazard_tensor(A: float) -> torch.Tensor:
    """One bf16 row: a block holding the tensor amax A (it fixes s_g), then,
    for every E4M3 code c whose block amax a bf16 value can reach, a block with
    that amax and, over two blocks, the bf16 values nearest to m alpha_c and
    their bf16 neighbours for the seven E2M1 decision points m (alpha_c =
    RN32(s_g E4M3(c))), both signs: the inputs whose product with an inexact
    reciprocal may round to the wrong side of a decision point."""
    s_g = np.float32(np.float64(np.float32(A)) / 2688.0)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    blocks = [np.concatenate([[A], np.zeros(15)])]
    for c in range(1, 127):
        alpha = np.float64(np.float32(s_g * np.float32(oracle.e4m3_value(c))))
        ag = _bf16([6.0 * np.float64(s_g) * oracle.e4m3_value(c)])[0]
        if not (0 < ag <= A):
            continue
        near = _bf16(mids * alpha).view(np.uint32)
        vals = np.concatenate([near - 0x10000, near, near + 0x10000]).view(np.float32)
        vals = vals[(vals > 0) & (vals < ag)]
        vals = np.concatenate([vals, -vals])[:30]
        pad = np.zeros(31 - vals.size, np.float32)
        two = np.concatenate([[ag], vals, pad]).astype(np.float64)
        blocks.append(two[:16])
        blocks.append(np.concatenate([[ag], two[16:31]]))
    row = np.concatenate(blocks).astype(np.float32)
    return torch.from_numpy(row).reshape(1, -1).to(torch.bfloat16)


@pytest.mark.parametrize("exp", [-6, -20, 3])
def test_nv_hazard_values_every_code_every_bf16_significand(exp):
    # every one of the 128 bf16 significands of the tensor amax, so every
    # distinct s_g significand a bf16 tensor can have, at three exponents
    for j in range(128):
        A = float(np.float32((128 + j) / 128.0 * 2.0 ** exp))
        check_nv(_hazard_tensor(A), f"hazards, amax {A!r}")


def test_nv_hazard_values_two_pass_quantize_and_scale_search():
    # the same hazard tensors through the two-pass encoder (here its packed
    # form, which shares the block-scale table and quotient) and through the
    # scale search, whose candidates use the same corrected reciprocals
    import oracle.gemm as og
    for j in range(128):
        A = float(np.float32((128 + j) / 128.0 * 2.0 ** -6))
        t = _hazard_tensor(A)
        x = torch.zeros(1, 4096, dtype=torch.bfloat16)
        x[:, : t.shape[1]] = t
        announce(f"hazards two-pass packed quantize + search, amax {A!r}")
        got, sg = fp4.quantize_nvfp4_packed(dev(x))
        codes, scales, sgs = fp4.scale_search(dev(x))
        torch.cuda.synchronize()
        xo = oracle_view(x)
        p, sc, sg_ref, flags = oracle.nv_quantize(xo)
        assert flags == 0
        assert np.float32(sg.item()) == np.float32(sg_ref)
        assert_bytes_equal(host_u8(got), og.nv_pack_operand(p, sc, 1, 4096), f"packed, amax {A!r}")
        p, s, f2 = oracle.scale_search_with_scale(xo, sg_ref, 64, 0.5, 1.0)
        assert f2 == 0
        assert_bytes_equal(host_u8(scales), s, f"search scales, amax {A!r}")
        assert_bytes_equal(host_u8(codes), p, f"search codes, amax {A!r}")
