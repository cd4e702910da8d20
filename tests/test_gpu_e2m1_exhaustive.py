"""Every fp32 value the converter can be handed at scale 1, through the GPU
MXFP4 quantizer, against the oracle's RoundE2M1 ("NVFP4 / MXFP4 format"
page, section 1: nearest code, ties to the code with an even low bit,
saturating at 6, the sign kept, so -0 and negative values that round to
zero give code 8).

A block whose amax lies in [4, 8) has the floor-rule scale 2^0, so its
quotients are its values unchanged and the kernel's FP4 converter sees them
at scale 1.  Each block here is [7.5, v_1 .. v_31]: the v run over every
fp32 bit pattern of magnitude below 8 (0 .. 0x40FFFFFF, subnormals
included), both signs, 2 181 038 080 values in all, which is every value
an MXFP4 block quotient can take at that scale (the floor rule keeps
|q| < 8; the NVFP4 quotients stay below 6.5).  Codes must match bit for bit
and every scale byte must be 127."""
import numpy as np
import pytest
import torch

import mxfp4_block_amax_amd as fp4
import oracle
from tests._gpu import announce, oracle_split

pytestmark = pytest.mark.gpu

MAG_END = 0x41000000            # first fp32 pattern of magnitude 8
CHUNK = 1 << 25                 # magnitudes per pass (both signs: 2^26 values)
PIN = np.float32(7.5)


def _blocks_host(m0: int, m1: int) -> np.ndarray:
    mags = np.arange(m0, m1, dtype=np.uint32)
    v = np.concatenate([mags, mags | np.uint32(0x80000000)]).view(np.float32)
    nb = (v.size + 30) // 31
    x = np.zeros((nb, 32), np.float32)
    x[:, 0] = PIN
    flat = x[:, 1:].reshape(-1)
    flat[: v.size] = v
    x[:, 1:] = flat.reshape(nb, 31)
    return x


def _blocks_device(m0: int, m1: int) -> torch.Tensor:
    mags = torch.arange(m0, m1, dtype=torch.int64, device="cuda")
    v = torch.cat([mags, mags | 0x80000000]).to(torch.int64)
    v = torch.where(v >= 2**31, v - 2**32, v).to(torch.int32).view(torch.float32)
    nb = (v.numel() + 30) // 31
    x = torch.zeros(nb, 32, dtype=torch.float32, device="cuda")
    x[:, 0] = float(PIN)
    body = torch.zeros(nb * 31, dtype=torch.float32, device="cuda")
    body[: v.numel()] = v
    x[:, 1:] = body.view(nb, 31)
    return x


def _pack(codes: np.ndarray) -> np.ndarray:
    c = codes.reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)


def test_round_e2m1_every_fp32_below_8_at_scale_1():
    checked = 0
    for m0 in range(0, MAG_END, CHUNK):
        m1 = min(m0 + CHUNK, MAG_END)
        announce(f"RoundE2M1 sweep, magnitudes {m0:#010x}..{m1:#010x}")
        codes, scales = fp4.quantize_mxfp4(_blocks_device(m0, m1))
        x = _blocks_host(m0, m1)
        want = np.concatenate(oracle_split(oracle.e2m1_round_array, x.reshape(-1), 32))
        assert want.max() < 16
        sc = scales.cpu().numpy().reshape(-1)
        assert (sc == 127).all(), f"scale bytes other than 127 near {m0:#x}"
        got = codes.cpu().numpy().reshape(-1)
        ref = _pack(want)
        bad = np.nonzero(got != ref)[0]
        if bad.size:
            i = int(bad[0])
            vals = x.reshape(-1)[2 * i: 2 * i + 2]
            raise AssertionError(f"{bad.size} code bytes differ; first at byte {i}: values "
                                 f"{[hex(int(u)) for u in vals.view(np.uint32)]} got {got[i]:#04x} "
                                 f"want {ref[i]:#04x}")
        checked += 2 * (m1 - m0)
    assert checked == 2 * MAG_END
    print(f"{checked} fp32 values checked", flush=True)
