"""Write tests/golden/workload_digests.json: the oracle's outputs on the
seeded workload inputs, as SHA-256 digests (and, for the 4096-element
round-trip input, in full), so that the benchmark can check the buffers it
times without running the oracle.

Every value here comes from the CPU oracle (oracle/) on the inputs that
workloads/ generates; nothing is read from the GPU path.  Run from the
repository root:

    python tests/golden/make_workload_digests.py
"""
import hashlib
import json
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "workload_digests.json")
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def f32_hex(v) -> str:
    return "0x%08x" % int(np.float32(v).view(np.uint32))


def view(t):
    t = t.contiguous()
    if t.dtype.is_floating_point and t.element_size() == 2:
        return workloads.bf16_bits(t).reshape(-1)
    return t.numpy().reshape(-1)


def split(fn, x, unit):
    n = x.size
    per = max(1, (n // unit + 4 * THREADS - 1) // (4 * THREADS)) * unit
    with ThreadPoolExecutor(THREADS) as pool:
        return list(pool.map(fn, [x[i:i + per] for i in range(0, n, per)]))


def mx_entry(x):
    p, s, f = oracle.mx_quantize(x)
    assert f == 0
    return {"codes_sha256": sha(p), "scales_sha256": sha(s)}, p, s


def nv_entry(x):
    p, s, sg, f = oracle.nv_quantize(x)
    assert f == 0
    return {"codes_sha256": sha(p), "scales_sha256": sha(s), "s_g_bits": f32_hex(sg)}, p, s, sg


def search_entry(x, ncand=64, c_lo=0.5, c_hi=1.0):
    sg, f = oracle.nv_global_scale(x)
    assert f == 0
    res = split(lambda part: oracle.scale_search_with_scale(part, sg, ncand, c_lo, c_hi), x, 16)
    assert all(r[2] == 0 for r in res)
    p = np.concatenate([r[0] for r in res])
    s = np.concatenate([r[1] for r in res])
    return {"codes_sha256": sha(p), "scales_sha256": sha(s), "s_g_bits": f32_hex(sg)}


def main():
    d = {"_about": "oracle outputs on the seeded workload inputs (workloads/), written by "
                   "tests/golden/make_workload_digests.py; SHA-256 over the row-major uint8 "
                   "codes and scale arrays, s_g as fp32 bits"}

    x = view(workloads.tiny_roundtrip())
    mx, p, s = mx_entry(x)
    y = oracle.dequantize(oracle.MX, p, s).astype(np.float64)
    mx.update({"codes_hex": p.tobytes().hex(), "scales_hex": s.tobytes().hex(),
               "mae": float(np.abs(y - x.astype(np.float64)).mean())})
    nv, p, s, sg = nv_entry(x)
    y = oracle.dequantize(oracle.NV, p, s, sg).astype(np.float64)
    nv.update({"codes_hex": p.tobytes().hex(), "scales_hex": s.tobytes().hex(),
               "mae": float(np.abs(y - x.astype(np.float64)).mean())})
    d["tiny_roundtrip_4096_f32"] = {"mx": mx, "nv": nv, "input_sha256": sha(x)}
    print("tiny done", flush=True)

    x = view(workloads.nvfp4_weight())
    d["nvfp4_weight_8192x8192_bf16_seed0"] = {"nv": nv_entry(x)[0], "mx": mx_entry(x)[0],
                                              "input_sha256": sha(x)}
    x = view(workloads.nvfp4_weight(seed=1))
    d["nvfp4_weight_8192x8192_bf16_seed1"] = {"nv": nv_entry(x)[0], "input_sha256": sha(x)}
    print("weights done", flush=True)

    x = view(workloads.mxfp4_activation())
    d["mxfp4_activation_16384x7168_bf16"] = {"mx": mx_entry(x)[0], "input_sha256": sha(x)}
    print("activation done", flush=True)

    x = view(workloads.scale_search_input())
    d["scale_search_4096x14336_bf16"] = {"search_64_c0.5_1.0": search_entry(x),
                                         "input_sha256": sha(x)}
    print("search done", flush=True)

    a, bt = workloads.gemm_operands()
    d["gemm_operands_128x8192x8192"] = {"a_mx": mx_entry(view(a))[0], "bt_mx": mx_entry(view(bt))[0],
                                        "a_input_sha256": sha(view(a)),
                                        "bt_input_sha256": sha(view(bt))}
    a_bf16 = a.to(__import__("torch").bfloat16)
    d["gemm_operands_128x8192x8192"]["a_bf16_mx"] = mx_entry(view(a_bf16))[0]
    d["gemm_operands_128x8192x8192"]["a_nv"] = nv_entry(view(a))[0]

    with open(OUT, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
