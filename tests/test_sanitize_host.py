"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two programs, each built here with the sanitizers and run once:

* tests/sanitize/oracle_check.c with the C oracle (gcc): every oracle
  routine on fp32 and bf16 inputs that reach its edge paths (zero blocks,
  subnormals, the largest finite values, NaN, infinities), with output
  buffers of exactly the stated sizes;
* tests/sanitize/capi_check.cpp with libfp4's sources (hipcc; the
  sanitizers instrument the host code only, the GPU code is built as usual
  and never run): every entry point with arguments its validation must
  reject, over sizes that break naive size arithmetic, plus the size
  helpers' results.

A sanitizer report ends the program with a nonzero status
(-fno-sanitize-recover), as does a failed check."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
sys.path.insert(0, ROOT)

from mxfp4_block_amax_amd import build as fp4_build  # noqa: E402

SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
          "-fno-fast-math", "-fexcess-precision=standard", "-Wall", "-Wextra", "-Werror",
          "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "fp4_oracle.c"), os.path.join(SAN, "oracle_check.c"),
          "-o", exe, "-lm"])
    out = _run([exe], env=SAN_ENV)
    print(out.strip())
    assert ", 0 failed checks" in out, out


@pytest.mark.skipif(not os.path.exists(fp4_build.HIPCC), reason="hipcc not found")
def test_capi_host_code_under_asan_ubsan(tmp_path):
    # the library's own flags, with the host pass instrumented (each sanitizer
    # flag after -Xarch_host, so the GPU code is compiled without them)
    san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", f]
    flags = [f for f in fp4_build.FLAGS if f != "-O3"] + ["-O1", "-g", *san]
    srcs = [os.path.join(fp4_build.CSRC, s) for s in fp4_build.SOURCES]
    srcs.append(os.path.join(SAN, "capi_check.cpp"))
    objs = [str(tmp_path / (os.path.basename(s) + ".o")) for s in srcs]
    procs = [subprocess.Popen([fp4_build.HIPCC, *flags, "-c", s, "-o", o],
                              stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
             for s, o in zip(srcs, objs)]
    for p, s in zip(procs, srcs):
        out = p.communicate()[0]
        assert p.returncode == 0, f"hipcc failed on {s}:\n{out[-4000:]}"
    exe = str(tmp_path / "capi_check")
    _run([fp4_build.HIPCC, "--offload-arch=gfx950", *san, *objs, "-o", exe])
    out = _run([exe], env=SAN_ENV)
    print(out.strip())
    assert ", 0 failures" in out, out
