"""Pins for the oracle's packed (MFMA operand order) layout: a hand-listed
example, the padding rule, and a GEMM that reads packed operands the way the
scaled MFMA consumes its lanes, checked against the row-major binary64
product.  The layout itself is not fixed by the pages (OCP leaves it to the
implementation, "NVFP4 / MXFP4 format" page, section 7)."""
import numpy as np
import pytest

import oracle.gemm as og


def _rand(rows, K, seed):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 256, (rows, K // 2), dtype=np.uint8),
            rng.integers(118, 137, (rows, K // 32), dtype=np.uint8))


def test_hand_listed_example_one_row():
    # one row of 512 values: code bytes 0..255, scale bytes 100..115
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    scales = np.arange(100, 116, dtype=np.uint8).reshape(1, 16)
    p = og.pack_operand(codes, scales, 1, 512)
    assert len(p) == 32 * 256 + 32 * 16
    tile = p[:8 * 1024].reshape(8, 64, 16)       # 8 K steps x 64 lanes x 16 bytes
    assert list(tile[0, 0]) == list(range(0, 16))     # step 0, lane 0: block 0
    assert list(tile[0, 32]) == list(range(16, 32))   # step 0, lane 32: block 1
    assert list(tile[1, 0]) == list(range(32, 48))    # step 1, lane 0: block 2
    assert list(tile[7, 32]) == list(range(240, 256))  # step 7, lane 32: block 15
    assert not tile[:, 1:32].any() and not tile[:, 33:].any()   # rows 1..31 are padding
    sc = p[8 * 1024:].reshape(64, 8)              # one group of eight steps
    assert list(sc[0]) == [100, 102, 104, 106, 108, 110, 112, 114]   # K half 0: even blocks
    assert list(sc[32]) == [101, 103, 105, 107, 109, 111, 113, 115]  # K half 1: odd blocks
    assert (sc[1:32] == 127).all() and (sc[33:] == 127).all()


@pytest.mark.parametrize("rows,K", [(1, 512), (33, 512), (70, 1024), (64, 2048)])
def test_every_byte_lands_once(rows, K):
    """A permutation: the packed code bytes are the source bytes plus the
    zero padding rows, and the packed scale bytes the source scales plus 127
    for every padding row, as multisets."""
    codes, scales = _rand(rows, K, rows * K)
    p = og.pack_operand(codes, scales, rows, K)
    pad = (rows + 31) // 32 * 32 - rows
    nc = (rows + pad) * K // 2
    want_c = np.concatenate([codes.reshape(-1), np.zeros(pad * K // 2, np.uint8)])
    want_s = np.concatenate([scales.reshape(-1), np.full(pad * K // 32, 127, np.uint8)])
    assert np.array_equal(np.sort(p[:nc]), np.sort(want_c))
    assert np.array_equal(np.sort(p[nc:]), np.sort(want_s))
    assert len(p) == og.packed_bytes(rows, K)


@pytest.mark.parametrize("M,N,K", [(32, 32, 512), (40, 70, 1024), (1, 65, 512), (96, 33, 2048)])
def test_mfma_consumer_reproduces_the_product(M, N, K):
    a, sa = _rand(M, K, M + K)
    b, sb = _rand(N, K, N + 7 * K)
    ref = og.gemm_f64(a, sa, b, sb, M, N, K)
    got = og.gemm_from_packed(og.pack_operand(a, sa, M, K), og.pack_operand(b, sb, N, K), M, N, K)
    # values p 2^e with e in [-9, 9] and 32 K steps at most: every partial sum
    # is exact in binary64, so both orders give the same bits
    assert np.array_equal(got, ref)


def test_a_swapped_k_half_is_caught():
    """Planting a mistake in the packing (the two K halves of each step
    swapped) changes the product the consumer reads."""
    M, N, K = 32, 32, 512
    a, sa = _rand(M, K, 3)
    b, sb = _rand(N, K, 4)
    pa = og.pack_operand(a, sa, M, K)
    bad = pa.copy()
    tiles = bad[:M * K // 2].reshape(1, K // 64, 64, 16)
    tiles[:] = np.concatenate([tiles[:, :, 32:], tiles[:, :, :32]], axis=2)
    good = og.gemm_from_packed(pa, og.pack_operand(b, sb, N, K), M, N, K)
    wrong = og.gemm_from_packed(bad, og.pack_operand(b, sb, N, K), M, N, K)
    assert np.array_equal(good, og.gemm_f64(a, sa, b, sb, M, N, K))
    assert not np.array_equal(wrong, good)


# ---- NVFP4 packed layout --------------------------------------------------------

def _nv_rand(rows, K, seed):
    rng = np.random.default_rng(seed)
    # E4M3 bytes of both signs, finite (magnitude code below 0x7F)
    s = rng.integers(0, 127, (rows, K // 16), dtype=np.uint8) | (rng.integers(0, 2, (rows, K // 16), dtype=np.uint8) << 7)
    return rng.integers(0, 256, (rows, K // 2), dtype=np.uint8), s


def test_nv_hand_listed_example_one_row():
    # one row of 512 values: code bytes 0..255, scale bytes 1..32 (block j -> j + 1)
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    scales = np.arange(1, 33, dtype=np.uint8).reshape(1, 32)
    p = og.nv_pack_operand(codes, scales, 1, 512)
    assert len(p) == og.nv_packed_bytes(1, 512) == 32 * 256 + 32 * 32
    tile = p[:8 * 1024].reshape(8, 64, 16)
    assert list(tile[0, 0]) == list(range(0, 16)) and list(tile[7, 32]) == list(range(240, 256))
    sc = p[8 * 1024:].reshape(64, 16)
    # lane 0 takes blocks 0, 1 of every step (values 0..31), lane 32 blocks 2, 3
    assert list(sc[0]) == [1, 2, 5, 6, 9, 10, 13, 14, 17, 18, 21, 22, 25, 26, 29, 30]
    assert list(sc[32]) == [3, 4, 7, 8, 11, 12, 15, 16, 19, 20, 23, 24, 27, 28, 31, 32]
    assert not sc[1:32].any() and not sc[33:].any()


@pytest.mark.parametrize("rows,K", [(1, 512), (33, 512), (70, 1024)])
def test_nv_every_byte_lands_once(rows, K):
    codes, scales = _nv_rand(rows, K, rows + K)
    p = og.nv_pack_operand(codes, scales, rows, K)
    pad = (rows + 31) // 32 * 32 - rows
    nc = (rows + pad) * K // 2
    assert np.array_equal(np.sort(p[:nc]), np.sort(np.concatenate(
        [codes.reshape(-1), np.zeros(pad * K // 2, np.uint8)])))
    assert np.array_equal(np.sort(p[nc:]), np.sort(np.concatenate(
        [scales.reshape(-1), np.zeros(pad * K // 16, np.uint8)])))
    assert len(p) == og.nv_packed_bytes(rows, K)


@pytest.mark.parametrize("M,N,K", [(32, 32, 512), (40, 70, 1024), (1, 65, 512)])
def test_nv_mfma_consumer_reproduces_the_product(M, N, K):
    a, sa = _nv_rand(M, K, M + K)
    b, sb = _nv_rand(N, K, N + 3 * K)
    sg_a, sg_b = np.float32(0.375), np.float32(1.0 / 3.0)
    ref = og.nv_gemm_f64(a, sa, sg_a, b, sb, sg_b, M, N, K)
    got = og.nv_gemm_from_packed(og.nv_pack_operand(a, sa, M, K), sg_a,
                                 og.nv_pack_operand(b, sb, N, K), sg_b, M, N, K)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_nv_swapped_block_scales_are_caught():
    """A planted mistake in the packing (the two block scales of each lane
    and step swapped) changes the product the consumer reads."""
    M, N, K = 32, 32, 512
    a, sa = _nv_rand(M, K, 5)
    b, sb = _nv_rand(N, K, 6)
    pa, pb = og.nv_pack_operand(a, sa, M, K), og.nv_pack_operand(b, sb, N, K)
    bad = pa.copy()
    s = bad[M * K // 2:].reshape(-1, 2)
    s[:] = s[:, ::-1].copy()
    good = og.nv_gemm_from_packed(pa, 1.0, pb, 1.0, M, N, K)
    wrong = og.nv_gemm_from_packed(bad, 1.0, pb, 1.0, M, N, K)
    assert not np.allclose(wrong, good)
