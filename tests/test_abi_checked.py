"""The C ABI's host-side validation and planning code under AddressSanitizer
and UndefinedBehaviorSanitizer (CPU only).

The library's sources are compiled again with the sanitizers on the host pass
only (the device code is the same gfx950 code), linked with ROCm's clang, and
driven by tests/abi_fuzz.c over random problem descriptions in and out of the
supported ranges: every call must return a status code of moe.h, workspace
sizes must behave, and no out-of-bounds access, overflow or other undefined
behaviour may occur on the way to the first HIP call."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

from sparse_mixture_experts_moe_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HOST_SAN = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _have_tools():
    try:
        B.hipcc()
    except RuntimeError:
        return False
    return os.path.exists(CLANG) and os.path.exists(CLANG + "++")


@pytest.mark.skipif(not _have_tools(), reason="needs ROCm's hipcc and clang")
def test_abi_validation_under_sanitizers(tmp_path):
    out = str(tmp_path)

    def comp(src):
        obj = os.path.join(out, src + ".o")
        r = subprocess.run([B.hipcc(), *B.CFLAGS, *HOST_SAN, "-c", os.path.join(B.CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        return obj

    with cf.ThreadPoolExecutor(min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(comp, B.SOURCES))
    lib = os.path.join(out, "libmoe_checked.so")
    rocm_lib = "/opt/rocm/lib"
    res = subprocess.run([CLANG, "-print-resource-dir"], capture_output=True, text=True).stdout.strip()
    san_lib = os.path.join(res, "lib", "linux")   # the sanitizer runtimes
    r = subprocess.run([CLANG + "++", "-shared", "-fsanitize=address,undefined", "-shared-libsan", *objs,
                        f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}", f"-Wl,-rpath,{san_lib}", "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = os.path.join(out, "abi_fuzz")
    r = subprocess.run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-shared-libsan", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "abi_fuzz.c"), lib, f"-Wl,-rpath,{out}", f"-Wl,-rpath,{san_lib}",
                        "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-6000:]
    assert r.stdout.startswith("ok"), r.stdout
    print(r.stdout.strip())
    shutil.rmtree(out, ignore_errors=True)
