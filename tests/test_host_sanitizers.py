"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
on a machine without a GPU: every source of the library is compiled with the
sanitizers on its host side only (device code unchanged), linked with a C11
driver (tests/host_sanitized/abi_checks.c) that exercises every entry point's
argument checks, workspace sizing and the pattern-search dynamic program, and
run.  No call in the driver reaches the GPU."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dsa_lightning_indexer_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/lib/llvm/bin/clang"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _sources():
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    assert "api.cpp" in srcs and "pattern_search.cpp" in srcs
    return srcs


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG) and shutil.which("gcc")),
                    reason="needs hipcc, ROCm's clang and gcc")
def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        r = subprocess.run([HIPCC, *FLAGS, *SAN_HOST, *lang, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr}"
        return obj
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, _sources()))
    driver = os.path.join(ROOT, "tests", "host_sanitized", "abi_checks.c")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include"]
    # the public header is plain C11 for a C compiler other than the one that built the library
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", *inc, driver],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # the driver itself instrumented too (same compiler family as the library)
    main_o = str(tmp_path / "abi_checks.o")
    r = subprocess.run([CLANG, "-x", "c", "-std=c11", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address",
                        "-fsanitize=undefined", "-fno-sanitize-recover=all", *inc, "-c", driver, "-o", main_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "abi_checks")
    # link line: no -Xarch_ option, so the sanitizers are kept off the device side explicitly
    link = [HIPCC, "--offload-arch=gfx950", "-fno-gpu-sanitize", "-fsanitize=address", "-fsanitize=undefined"]
    r = subprocess.run([*link, main_o, *objs, "-o", exe, "-L/opt/rocm/lib", "-lamdhip64"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "ALL OK" in r.stdout, out
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
