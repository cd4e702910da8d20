"""The stored oracle digests (tests/golden/workload_digests.json, which the
benchmark checks its timed buffers against) agree with the oracle run now on
the same seeded inputs: the 4096-element round trip in full, and the
8192 x 8192 weight's NVFP4 and MXFP4 outputs by digest."""
import hashlib
import json
import os

import numpy as np

import oracle
import workloads
from tests._golden import GOLDEN
from tests._gpu import oracle_view


def _load():
    with open(os.path.join(GOLDEN, "workload_digests.json")) as f:
        return json.load(f)


def _sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def _f32_hex(v):
    return "0x%08x" % int(np.float32(v).view(np.uint32))


def test_tiny_roundtrip_entry_is_the_oracles():
    d = _load()["tiny_roundtrip_4096_f32"]
    x = oracle_view(workloads.tiny_roundtrip())
    p, s, f = oracle.mx_quantize(x)
    assert f == 0
    assert d["mx"]["codes_hex"] == p.tobytes().hex() and d["mx"]["codes_sha256"] == _sha(p)
    assert d["mx"]["scales_hex"] == s.tobytes().hex()
    y = oracle.dequantize(oracle.MX, p, s).astype(np.float64)
    assert d["mx"]["mae"] == float(np.abs(y - x).mean())
    p, s, sg, f = oracle.nv_quantize(x)
    assert f == 0
    assert d["nv"]["codes_hex"] == p.tobytes().hex() and d["nv"]["s_g_bits"] == _f32_hex(sg)
    assert d["nv"]["scales_hex"] == s.tobytes().hex()
    # the encoded scales lose to the pages' ideal amax/6 scale at 32- and
    # 16-blocks (0.0901, 0.0747) by less than the one-block error (0.7238)
    assert d["mx"]["mae"] < 0.7238 and d["nv"]["mae"] < 0.7238


def test_weight_8192_entries_are_the_oracles():
    d = _load()["nvfp4_weight_8192x8192_bf16_seed0"]
    x = oracle_view(workloads.nvfp4_weight())
    p, s, sg, f = oracle.nv_quantize(x)
    assert f == 0
    assert d["nv"] == {"codes_sha256": _sha(p), "scales_sha256": _sha(s), "s_g_bits": _f32_hex(sg)}
    p, s, f = oracle.mx_quantize(x)
    assert f == 0
    assert d["mx"] == {"codes_sha256": _sha(p), "scales_sha256": _sha(s)}
