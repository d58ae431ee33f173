"""Sanitizer builds (CPU only): the oracle, and the library's host code behind the C ABI,
under AddressSanitizer (with leak detection) and UndefinedBehaviorSanitizer.

- oracle/w4a8_oracle.c with oracle/sanitize_check.c (gcc): every oracle function on small,
  ragged and edge-case inputs.
- w4a8_codebook_gemm_amd/csrc/api.hip compiled with host-side sanitizers (hipcc, each
  -fsanitize after -Xarch_host, so the device code is built as usual), linked with the other
  sources' objects, and driven by tests/abi_check.c (clang): every entry point's argument
  validation and the metadata calls, none of which touches a GPU.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_check"
    run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
         "-Wno-unknown-pragmas", os.path.join(ROOT, "oracle", "w4a8_oracle.c"),
         os.path.join(ROOT, "oracle", "sanitize_check.c"), "-lm", "-o", str(exe)])
    r = run([str(exe)], env=SAN_ENV, timeout=300)
    assert r.stdout.strip().endswith("ok")


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_library_host_code_under_asan_ubsan(tmp_path):
    import w4a8_codebook_gemm_amd.build as B
    flags = [f for f in B.FLAGS]
    srcs = B.sources()
    api = [s for s in srcs if os.path.basename(s) == "api.hip"]
    assert api
    header = os.path.join(ROOT, "w4a8_codebook_gemm_amd", "csrc", "w4a8_internal.h")

    def obj_for(src):
        # the library build's object when it is newer than its source and the shared header
        built = os.path.join(B.BUILD, os.path.basename(src) + ".o")
        if os.path.exists(built) and os.path.getmtime(built) >= max(os.path.getmtime(src), os.path.getmtime(header)):
            return built
        out = str(tmp_path / (os.path.basename(src) + ".o"))
        run([HIPCC, *flags, "-c", src, "-o", out])
        return out

    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = str(tmp_path / "api_san.o")
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        fut = ex.submit(run, [HIPCC, *flags, "-O1", "-g", *san, "-c", api[0], "-o", api_obj])
        others = list(ex.map(obj_for, [s for s in srcs if s not in api]))
        fut.result()
    lib = str(tmp_path / "libw4a8_san.so")
    run([HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
         "-Xarch_host", "-fsanitize=undefined", api_obj, *others, "-o", lib])
    exe = str(tmp_path / "abi_check")
    run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g",
         f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "abi_check.c"),
         f"-L{tmp_path}", "-lw4a8_san", f"-Wl,-rpath,{tmp_path}", "-o", exe])
    r = run([exe], env=SAN_ENV, timeout=300)
    assert r.stdout.strip().endswith("ok")
