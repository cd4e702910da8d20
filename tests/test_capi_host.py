"""Host-side tests of the C ABI: the library loads, exports every entry point
include/fp4.h declares, and rejects invalid arguments synchronously, before
any HIP call (so no GPU is needed).  No compute call is made here."""
import ctypes
import os
import re

import pytest

import mxfp4_block_amax_amd as fp4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4.h")

OK, E_ARG, E_SHAPE, E_DTYPE, E_ALIGN, E_WORKSPACE = 0, 1, 2, 3, 4, 5

pytestmark = pytest.mark.skipif(not os.path.exists(fp4.LIB_PATH), reason="libfp4.so not built")

# fake, never-dereferenced device addresses: validation must fail before use
A16 = ctypes.c_void_p(0x10000)
A1 = ctypes.c_void_p(0x10001)
NULL = None


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fp4_[a-z_0-9]+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(fp4.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = fp4.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    for code in range(7):
        assert fp4.status_str(code)
    assert fp4.status_str(0) == "ok"


def test_workspace_bytes():
    assert fp4.workspace_bytes(fp4.MXFP4, 8192, 8192) == 0
    assert fp4.workspace_bytes(fp4.NVFP4, 8192, 8192) >= 1024 * 4


def mx(x=A16, dt=fp4.BF16, rows=4, cols=64, block=32, codes=A16, scales=A16, status=NULL):
    return fp4.lib().fp4_quantize_mxfp4(x, dt, rows, cols, block, codes, scales, status, NULL)


def nv(x=A16, dt=fp4.BF16, rows=4, cols=64, block=16, codes=A16, scales=A16, sg=A16, ws=A16,
       wsb=1 << 20, status=NULL):
    return fp4.lib().fp4_quantize_nvfp4(x, dt, rows, cols, block, codes, scales, sg, ws, wsb,
                                        status, NULL)


def test_mx_validation():
    assert mx(x=NULL) == E_ARG
    assert mx(codes=NULL) == E_ARG
    assert mx(block=16) == E_ARG
    assert mx(dt=7) == E_DTYPE
    assert mx(cols=48) == E_SHAPE        # incomplete 32-block
    assert mx(rows=0) == E_SHAPE
    assert mx(cols=0) == E_SHAPE
    assert mx(x=A1) == E_ALIGN


def test_nv_validation():
    assert nv(sg=NULL) == E_ARG
    assert nv(block=32) == E_ARG
    assert nv(cols=17) == E_SHAPE         # the page's 17-element case
    assert nv(ws=NULL) == E_WORKSPACE
    assert nv(wsb=16) == E_WORKSPACE
    assert nv(x=A1) == E_ALIGN


def test_dequant_validation():
    L = fp4.lib()
    assert L.fp4_dequantize(5, A16, A16, A16, 4, 64, 32, A16, fp4.BF16, NULL) == E_DTYPE
    assert L.fp4_dequantize(fp4.NVFP4, A16, A16, NULL, 4, 64, 16, A16, fp4.BF16, NULL) == E_ARG
    assert L.fp4_dequantize(fp4.MXFP4, A16, A16, NULL, 4, 64, 16, A16, fp4.BF16, NULL) == E_ARG
    assert L.fp4_dequantize(fp4.MXFP4, A16, A16, NULL, 4, 40, 32, A16, fp4.BF16, NULL) == E_SHAPE
    assert L.fp4_dequantize(fp4.MXFP4, A16, A16, NULL, 4, 64, 32, A1, fp4.BF16, NULL) == E_ALIGN


def test_search_validation():
    L = fp4.lib()

    def s(n=64, lo=0.5, hi=1.0, block=16, cols=64):
        return L.fp4_scale_search(A16, fp4.BF16, 4, cols, block, n, lo, hi, A16, A16, A16, A16,
                                  1 << 20, NULL, NULL)
    assert s(n=1) == E_ARG
    assert s(lo=0.0) == E_ARG
    assert s(lo=1.0, hi=0.5) == E_ARG
    assert s(n=4) == E_ARG                # grid coarser than the E4M3 grid
    assert s(hi=5.0, n=4096) == E_ARG
    assert s(block=32) == E_ARG
    assert s(cols=24) == E_SHAPE
    # a block's codes are one 8-byte store
    assert L.fp4_scale_search(A16, fp4.BF16, 4, 64, 16, 64, 0.5, 1.0, ctypes.c_void_p(0x10004), A16,
                              A16, A16, 1 << 20, NULL, NULL) == E_ALIGN


def test_mx_rule_validation():
    L = fp4.lib()

    def r(rule=1, block=32, cols=64, x=A16, dt=fp4.BF16):
        return L.fp4_quantize_mxfp4_rule(x, dt, 4, cols, block, rule, A16, A16, NULL, NULL)
    assert r(rule=3) == E_ARG
    assert r(rule=-1) == E_ARG
    assert r(block=16) == E_ARG
    assert r(x=NULL) == E_ARG
    assert r(dt=9) == E_DTYPE
    assert r(cols=48) == E_SHAPE
    assert r(x=A1) == E_ALIGN


def test_exhaustive_search_validation():
    L = fp4.lib()

    def s(block=16, cols=64, ws=A16, wsb=1 << 20, sg=A16):
        return L.fp4_scale_search_exhaustive(A16, fp4.BF16, 4, cols, block, A16, A16, sg, ws, wsb,
                                             NULL, NULL)
    assert s(block=32) == E_ARG
    assert s(sg=NULL) == E_ARG
    assert s(cols=24) == E_SHAPE
    assert s(ws=NULL) == E_WORKSPACE
    assert s(wsb=8) == E_WORKSPACE
    assert L.fp4_scale_search_exhaustive(A16, fp4.BF16, 4, 64, 16, ctypes.c_void_p(0x10004), A16, A16,
                                         A16, 1 << 20, NULL, NULL) == E_ALIGN


def test_linear_validation():
    L = fp4.lib()

    def lin(x=A16, M=128, K=512, N=64, ws=A16, wsb=1 << 20, ac=A16, c=A16, xt=fp4.BF16, mode=0):
        return L.fp4_linear_mxfp4(x, xt, M, K, A16, A16, N, ac, A16, c, fp4.BF16, mode, ws, wsb,
                                  NULL, NULL)
    assert lin(mode=2) == E_ARG
    assert lin(x=NULL) == E_ARG
    assert lin(ac=NULL) == E_ARG
    assert lin(xt=4) == E_DTYPE
    assert lin(K=48) == E_SHAPE
    assert lin(M=0) == E_SHAPE
    assert lin(ws=NULL) == E_WORKSPACE
    assert lin(wsb=8) == E_WORKSPACE
    assert lin(x=A1) == E_ALIGN
    assert lin(ac=A1) == E_ALIGN


def test_gemm_nvfp4_validation():
    L = fp4.lib()

    def g(M=128, N=64, K=512, sga=A16, c=A16, ct=fp4.BF16):
        return L.fp4_gemm_nvfp4(A16, A16, sga, A16, A16, A16, M, N, K, c, ct, NULL)
    assert g(sga=NULL) == E_ARG
    assert g(ct=6) == E_DTYPE
    assert g(K=24) == E_SHAPE
    assert g(N=0) == E_SHAPE
    assert g(c=A1) == E_ALIGN


def test_padded_storage_and_validation():
    # the format page's section 8: two rows of 17 values, NVFP4 -> 40 bytes
    assert fp4.padded_storage_bytes(fp4.NVFP4, 2, 17) == 40
    assert fp4.padded_storage_bytes(fp4.MXFP4, 2, 17) == 2 * (16 + 1)
    assert fp4.padded_storage_bytes(fp4.NVFP4, 0, 17) == -1
    L = fp4.lib()

    def q(fmt=fp4.NVFP4, rows=2, cols=17, sg=A16, ws=A16, wsb=1 << 20, x=A16, codes=A16):
        return L.fp4_quantize_padded(fmt, x, fp4.BF16, rows, cols, codes, A16, sg, ws, wsb, NULL,
                                     NULL)
    assert q(fmt=5) == E_DTYPE
    assert q(sg=NULL) == E_ARG
    assert q(cols=0) == E_SHAPE
    assert q(ws=NULL) == E_WORKSPACE
    assert q(x=A1) == E_ALIGN
    assert q(codes=ctypes.c_void_p(0x10002)) == E_ALIGN
    assert L.fp4_dequantize_padded(fp4.MXFP4, A16, A16, NULL, 2, 0, A16, fp4.BF16, NULL) == E_SHAPE


def test_sr_validation():
    L = fp4.lib()

    def q(fmt=fp4.NVFP4, x=A16, dt=fp4.BF16, rows=4, cols=64, block=16, codes=A16, sg=A16,
          ws=A16, wsb=1 << 20, status=NULL):
        return L.fp4_quantize_sr(fmt, x, dt, rows, cols, block, 2**64 - 1, codes, A16, sg, ws,
                                 wsb, status, NULL)
    assert q(fmt=2) == E_DTYPE
    assert q(dt=9) == E_DTYPE
    assert q(x=NULL) == E_ARG
    assert q(sg=NULL) == E_ARG                       # NVFP4 needs s_g
    assert q(block=32) == E_ARG                      # NVFP4 blocks are 16
    assert q(fmt=fp4.MXFP4, block=16) == E_ARG       # MXFP4 blocks are 32
    assert q(cols=17) == E_SHAPE
    assert q(fmt=fp4.MXFP4, block=32, cols=48) == E_SHAPE
    assert q(rows=0) == E_SHAPE
    assert q(ws=NULL) == E_WORKSPACE
    assert q(wsb=16) == E_WORKSPACE
    assert q(x=A1) == E_ALIGN
    assert q(status=A1) == E_ALIGN
    assert q(ws=ctypes.c_void_p(0x10004)) == E_ALIGN


def test_splitk_workspace_sizes():
    # S = the fewest equal K ranges of at most 2048 K, each a multiple of 512
    ws = fp4.gemm_splitk_workspace_bytes
    assert ws(128, 8192, 8192) == 4 * 128 * 8192 * 4
    assert ws(128, 8192, 4096) == 2 * 128 * 8192 * 4
    assert ws(128, 8192, 2048) == 1 * 128 * 8192 * 4
    assert ws(1, 8, 512) == 1 * 1 * 8 * 4
    assert ws(64, 512, 3072) == 2 * 64 * 512 * 4      # 2 x 1536
    assert ws(64, 512, 2560) == 5 * 64 * 512 * 4      # 5 x 512 (2 x 1280 is not allowed)
    assert ws(64, 512, 16384) == 8 * 64 * 512 * 4
    assert ws(128, 8192, 256) == 0                     # K below 512
    assert ws(128, 8192, 8192 + 32) == 0               # K not a multiple of 512
    assert ws(128, 6, 8192) == 0                       # N not a multiple of 4
    assert ws(0, 8, 512) == 0


def test_splitk_validation():
    L = fp4.lib()

    def g(M=128, N=256, K=1024, a=A16, sa=A16, c=A16, ws=A16, wsb=1 << 30, ct=fp4.BF16):
        return L.fp4_gemm_mxfp4_splitk(a, sa, A16, A16, M, N, K, c, ct, ws, wsb, NULL)
    assert g(a=NULL) == E_ARG
    assert g(c=NULL) == E_ARG
    assert g(ct=5) == E_DTYPE
    assert g(K=480) == E_SHAPE
    assert g(N=6) == E_SHAPE
    assert g(M=0) == E_SHAPE
    assert g(ws=NULL) == E_WORKSPACE
    assert g(wsb=fp4.gemm_splitk_workspace_bytes(128, 256, 1024) - 1) == E_WORKSPACE
    assert g(a=A1) == E_ALIGN
    assert g(sa=ctypes.c_void_p(0x10008)) == E_ALIGN    # scales need 16 bytes
    assert g(c=ctypes.c_void_p(0x10008), ct=fp4.F32) == E_ALIGN
    assert g(ws=ctypes.c_void_p(0x10004)) == E_ALIGN


def test_gemm_validation():
    L = fp4.lib()

    def g(M=128, N=256, K=256, a=A16, c=A16):
        return L.fp4_gemm_mxfp4(a, A16, A16, A16, M, N, K, c, fp4.BF16, NULL)
    assert g(a=NULL) == E_ARG
    assert g(K=48) == E_SHAPE
    assert g(M=0) == E_SHAPE
    assert g(a=A1) == E_ALIGN


def test_debug_poll_limit_entry_points_validate_as_the_product_ones():
    """The grid barrier's poll limit is an argument of two debug entry points
    (no process-wide setting): they reject what fp4_quantize_nvfp4 and
    fp4_linear_mxfp4 reject, with the same codes, whatever the limit; the
    header's default matches the binding's; the binding checks the range."""
    m = re.search(r"#define FP4_BARRIER_SPIN_LIMIT_DEFAULT (\d+)u", open(HEADER).read())
    assert m and int(m.group(1)) == fp4.BARRIER_SPIN_LIMIT_DEFAULT
    L = fp4.lib()

    def nv2(spin, x=A16, block=16, cols=64, sg=A16, ws=A16, wsb=1 << 20):
        args = (x, fp4.BF16, 4, cols, block, A16, A16, sg, ws, wsb, NULL, NULL)
        return L.fp4_quantize_nvfp4(*args), L.fp4_debug_quantize_nvfp4_spin(*args, spin)

    def lin2(spin, x=A16, K=512, ws=A16, mode=0):
        args = (x, fp4.BF16, 128, K, A16, A16, 64, A16, A16, A16, fp4.BF16, mode, ws, 1 << 20,
                NULL, NULL)
        return L.fp4_linear_mxfp4(*args), L.fp4_debug_linear_mxfp4_spin(*args, spin)

    for spin in (0, 7, 2**32 - 1):
        assert nv2(spin, sg=NULL) == (E_ARG, E_ARG)
        assert nv2(spin, block=32) == (E_ARG, E_ARG)
        assert nv2(spin, cols=17) == (E_SHAPE, E_SHAPE)
        assert nv2(spin, ws=NULL) == (E_WORKSPACE, E_WORKSPACE)
        assert nv2(spin, x=A1) == (E_ALIGN, E_ALIGN)
        assert lin2(spin, mode=2) == (E_ARG, E_ARG)
        assert lin2(spin, K=48) == (E_SHAPE, E_SHAPE)
        assert lin2(spin, ws=NULL) == (E_WORKSPACE, E_WORKSPACE)
        assert lin2(spin, x=A1) == (E_ALIGN, E_ALIGN)
    for bad in (-1, 2**32):
        with pytest.raises(ValueError):
            fp4._spin(bad)


def test_packed_sizes_and_validation():
    L = fp4.lib()
    assert fp4.packed_operand_bytes(1, 512) == 32 * 256 + 32 * 16
    assert fp4.packed_operand_bytes(33, 1024) == 64 * 512 + 64 * 32
    assert fp4.packed_operand_bytes(128, 8192) == 128 * 4096 + 128 * 256
    assert fp4.packed_operand_bytes(1, 256) == 0        # K below 512
    assert fp4.packed_operand_bytes(1, 1000) == 0
    assert fp4.packed_operand_bytes(0, 512) == 0

    def p(c=A16, s=A16, rows=64, K=1024, out=A16, nb=1 << 20):
        return L.fp4_pack_mxfp4_operand(c, s, rows, K, out, nb, NULL)
    assert p(c=NULL) == E_ARG
    assert p(out=NULL) == E_ARG
    assert p(K=256) == E_SHAPE
    assert p(rows=0) == E_SHAPE
    assert p(nb=fp4.packed_operand_bytes(64, 1024) - 1) == E_WORKSPACE
    assert p(c=A1) == E_ALIGN
    assert p(out=ctypes.c_void_p(0x10008)) == E_ALIGN

    def g(a=A16, b=A16, M=128, N=256, K=2048, c=A16, ct=fp4.BF16):
        return L.fp4_gemm_mxfp4_packed(a, b, M, N, K, c, ct, NULL)
    assert g(a=NULL) == E_ARG
    assert g(c=NULL) == E_ARG
    assert g(ct=7) == E_DTYPE
    assert g(K=1024) == E_SHAPE
    assert g(K=3072) == E_SHAPE
    assert g(K=18432) == E_SHAPE
    assert g(M=0) == E_SHAPE
    assert g(N=1 << 20, K=16384) == E_SHAPE   # packed Bt above 1 GiB
    assert g(a=A1) == E_ALIGN
    assert g(c=ctypes.c_void_p(0x10002)) == E_ALIGN


def test_nv_packed_sizes_and_validation():
    L = fp4.lib()
    assert fp4.nv_packed_operand_bytes(1, 512) == 32 * 256 + 32 * 32
    assert fp4.nv_packed_operand_bytes(33, 1024) == 64 * 512 + 64 * 64
    assert fp4.nv_packed_operand_bytes(8192, 8192) == 8192 * 4096 + 8192 * 512
    assert fp4.nv_packed_operand_bytes(1, 256) == 0
    assert fp4.nv_packed_operand_bytes(0, 512) == 0

    def p(c=A16, s=A16, rows=64, K=1024, out=A16, nb=1 << 20):
        return L.fp4_pack_nvfp4_operand(c, s, rows, K, out, nb, NULL)
    assert p(s=NULL) == E_ARG
    assert p(K=1000) == E_SHAPE
    assert p(nb=fp4.nv_packed_operand_bytes(64, 1024) - 1) == E_WORKSPACE
    assert p(out=A1) == E_ALIGN

    def g(a=A16, sa=A16, b=A16, sb=A16, M=128, N=256, K=2048, c=A16, ct=fp4.BF16):
        return L.fp4_gemm_nvfp4_packed(a, sa, b, sb, M, N, K, c, ct, NULL)
    assert g(sa=NULL) == E_ARG
    assert g(sb=NULL) == E_ARG
    assert g(ct=7) == E_DTYPE
    assert g(K=1024) == E_SHAPE
    assert g(K=6144 + 512) == E_SHAPE
    assert g(K=18432) == E_SHAPE
    assert g(N=0) == E_SHAPE
    assert g(N=1 << 20, K=16384) == E_SHAPE   # packed Bt above 1 GiB
    assert g(b=A1) == E_ALIGN
    assert g(sa=ctypes.c_void_p(0x10002)) == E_ALIGN

    ws = fp4.workspace_bytes(fp4.NVFP4, 64, 1024)

    def q(x=A16, xt=fp4.F32, rows=64, cols=1024, out=A16, nb=1 << 20, sg=A16, w=A16, wb=ws, st=A16):
        return L.fp4_quantize_nvfp4_packed(x, xt, rows, cols, out, nb, sg, w, wb, st, NULL)
    assert q(sg=NULL) == E_ARG
    assert q(xt=9) == E_DTYPE
    assert q(cols=1000) == E_SHAPE
    assert q(nb=fp4.nv_packed_operand_bytes(64, 1024) - 1) == E_WORKSPACE
    assert q(w=NULL) == E_WORKSPACE
    assert q(wb=ws - 1) == E_WORKSPACE
    assert q(x=A1) == E_ALIGN

    def lin(M=128, K=2048, N=256, nb=1 << 20, w=A16, wb=ws, c=A16, sb=A16):
        return L.fp4_linear_nvfp4_packed(A16, fp4.F32, M, K, A16, sb, N, A16, nb, A16, c,
                                         fp4.BF16, w, wb, NULL, NULL)
    assert lin(sb=NULL) == E_ARG
    assert lin(K=1024) == E_SHAPE
    assert lin(N=0) == E_SHAPE
    assert lin(nb=fp4.nv_packed_operand_bytes(128, 2048) - 1) == E_WORKSPACE
    assert lin(w=NULL) == E_WORKSPACE
    assert lin(c=A1) == E_ALIGN


def test_packed_quantize_and_linear_validation():
    L = fp4.lib()

    def q(x=A16, rows=64, cols=1024, out=A16, nb=1 << 20, xt=fp4.BF16, st=NULL):
        return L.fp4_quantize_mxfp4_packed(x, xt, rows, cols, out, nb, st, NULL)
    assert q(x=NULL) == E_ARG
    assert q(out=NULL) == E_ARG
    assert q(xt=9) == E_DTYPE
    assert q(cols=1056) == E_SHAPE                   # not a multiple of 512
    assert q(rows=0) == E_SHAPE
    assert q(nb=fp4.packed_operand_bytes(64, 1024) - 1) == E_WORKSPACE
    assert q(x=A1) == E_ALIGN
    assert q(out=ctypes.c_void_p(0x10008)) == E_ALIGN
    assert q(st=ctypes.c_void_p(0x10002)) == E_ALIGN

    def lin(x=A16, M=128, K=2048, bt=A16, N=256, a=A16, nb=1 << 20, c=A16, ct=fp4.BF16):
        return L.fp4_linear_mxfp4_packed(x, fp4.F32, M, K, bt, N, a, nb, c, ct, NULL, NULL)
    assert lin(bt=NULL) == E_ARG
    assert lin(a=NULL) == E_ARG
    assert lin(ct=4) == E_DTYPE
    assert lin(K=1024) == E_SHAPE
    assert lin(K=20480) == E_SHAPE
    assert lin(nb=fp4.packed_operand_bytes(128, 2048) - 1) == E_WORKSPACE
    assert lin(a=ctypes.c_void_p(0x10008)) == E_ALIGN


def nv_noalloc(x=A16, dt=fp4.BF16, rows=4, cols=64, block=16, codes=A16, scales=A16, sg=A16,
               status=NULL):
    return fp4.lib().fp4_quantize_nvfp4_noalloc(x, dt, rows, cols, block, codes, scales, sg,
                                                status, NULL)


def test_nv_noalloc_validation():
    # every argument error comes back before the scratch is set up (no HIP call)
    assert nv_noalloc(x=NULL) == E_ARG
    assert nv_noalloc(sg=NULL) == E_ARG
    assert nv_noalloc(block=32) == E_ARG
    assert nv_noalloc(dt=7) == E_DTYPE
    assert nv_noalloc(cols=17) == E_SHAPE
    assert nv_noalloc(rows=0) == E_SHAPE
    assert nv_noalloc(x=A1) == E_ALIGN
    assert nv_noalloc(sg=ctypes.c_void_p(0x10002)) == E_ALIGN


def test_noalloc_scratch_holds_a_workspace():
    # the fixed scratch is at least the workspace of the largest accepted shape
    assert fp4.workspace_bytes(fp4.NVFP4, 1 << 20, 1 << 20) <= fp4.NOALLOC_SCRATCH_BYTES
    src = open(HEADER).read()
    assert f"#define FP4_NOALLOC_SCRATCH_BYTES {fp4.NOALLOC_SCRATCH_BYTES}u" in src


@pytest.mark.parametrize("lang,compiler,std", [("c", "gcc", "-std=c11"), ("c++", "g++", "-std=c++17")])
def test_header_compiles_for_c_and_cpp_callers(tmp_path, lang, compiler, std):
    # The header is the boundary for callers in either language: it must
    # compile cleanly as both, with every enumeration 32 bits wide.
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    check = ("_Static_assert" if lang == "c" else "static_assert")
    src.write_text(
        '#include "fp4.h"\n'
        f"{check}(sizeof(fp4_status) == 4, \"fp4_status is 32 bits\");\n"
        f"{check}(sizeof(fp4_dtype) == 4 && sizeof(fp4_format) == 4, \"32-bit enums\");\n"
        f"{check}(sizeof(fp4_mx_rule) == 4 && sizeof(fp4_linear_mode) == 4, \"32-bit enums\");\n"
        "int f(void) { return (int)fp4_status_str(FP4_OK)[0]; }\n")
    r = subprocess.run([compiler, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
