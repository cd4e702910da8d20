"""Pins for the oracle's row-padded layout ("NVFP4 / MXFP4 format" page,
section 8: B = R * ceil(K / G) blocks, B (G/2 + 1) bytes plus 4 for the
NVFP4 tensor scale; decoding crops each row to the logical shape)."""
import numpy as np
import torch

import oracle
from tests._golden import rows


def _padded_rows():
    return [r for r in rows("storage_bytes.txt") if r[0] == "padded"]


def test_padded_storage_matches_the_page():
    (_, R, K, G, gb, nblocks, total), = _padded_rows()
    R, K, G, gb = int(R), int(K), int(G), int(gb)
    assert oracle.padded_storage_bytes(R, K, G, gb) == int(total)
    x = (np.arange(R * K, dtype=np.float32) - 10) / 7
    packed, scales, s_g, flags = oracle.nv_quantize_padded(x, R, K)
    assert flags == 0 and scales.size == int(nblocks)
    assert packed.size + scales.size + 4 == int(total)
    # flattening first would count ceil(R K / G) = 3 blocks, not the page's 4
    assert -(-R * K // G) != int(nblocks)


def test_complete_rows_equal_the_complete_block_encoders():
    g = torch.Generator().manual_seed(61)
    x = (torch.randn(6, 96, generator=g) * 3).numpy()
    p1, s1, f1 = oracle.mx_quantize_padded(x, 6, 96)
    p2, s2, f2 = oracle.mx_quantize(x.reshape(-1))
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
    p1, s1, g1, f1 = oracle.nv_quantize_padded(x, 6, 96)
    p2, s2, g2, f2 = oracle.nv_quantize(x.reshape(-1))
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2) and g1 == g2


def test_padding_is_zero_codes_and_rows_are_independent():
    g = torch.Generator().manual_seed(62)
    R, K = 5, 41
    x = (torch.randn(R, K, generator=g) * 2).numpy().astype(np.float32)
    # MX: each row on its own, padded with explicit zeros, gives the same bytes
    p, s, f = oracle.mx_quantize_padded(x, R, K)
    codes = oracle.unpack(p).reshape(R, 64)
    assert np.all(codes[:, K:] == 0)
    for r in range(R):
        row = np.zeros(64, np.float32)
        row[:K] = x[r]
        pr, sr, _ = oracle.mx_quantize(row)
        assert np.array_equal(p.reshape(R, 32)[r], pr) and np.array_equal(s.reshape(R, 2)[r], sr)
    # NV: the tensor scale comes from the logical elements alone
    p, s, s_g, f = oracle.nv_quantize_padded(x, R, K)
    assert s_g == oracle.nv_global_scale(x.reshape(-1))[0]
    assert np.all(oracle.unpack(p).reshape(R, 48)[:, K:] == 0)


def test_padded_decode_crops_each_row():
    g = torch.Generator().manual_seed(63)
    R, K = 3, 19
    x = (torch.randn(R, K, generator=g)).numpy().astype(np.float32)
    p, s, s_g, f = oracle.nv_quantize_padded(x, R, K)
    y = oracle.dequantize_padded(oracle.NV, p, s, R, K, s_g).reshape(R, K)
    full = oracle.dequantize(oracle.NV, p, s, s_g).reshape(R, 32)
    assert np.array_equal(y, full[:, :K])
    assert np.all(full[:, K:] == 0)
    # the decode is close to the input: within one E2M1 step of the block scale
    assert np.all(np.abs(y - x) <= np.abs(x).max() / 2)
