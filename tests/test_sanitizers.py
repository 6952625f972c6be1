"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

- The CPU oracle (oracle/moe_oracle.c) is compiled with gcc's ASan + UBSan and run
  through every entry point by oracle/sanitize_main.c, which also checks a cheap
  invariant after each call.
- The library's C-ABI translation unit (csrc/moe_api.hip: validation, sizing,
  dispatch) is compiled with the host-side sanitizers only (device code is built as
  usual) and linked with the library's other objects into
  tests/abi_sanitize_main.c, which exercises every entry point's validation paths.
  None of them reaches a kernel launch, so the run needs no GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_sanitize")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-o", exe,
          os.path.join(ROOT, "oracle", "sanitize_main.c"),
          os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    r = _run([exe], env=SAN_ENV)
    assert "all checks passed" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_abi_under_asan_ubsan():
    objs = [os.path.join(ROOT, "_build", f"{n}.o") for n in ("selection", "grouped_ffn", "fused_ffn", "combine",
                                                              "quant")]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built (run routing_aware_grouped_amd.build)")
    os.makedirs(OUT, exist_ok=True)
    api = os.path.join(OUT, "moe_api_san.o")
    # host-side sanitizers only: each -fsanitize applies to the host compilation
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-c",
          os.path.join(ROOT, "routing_aware_grouped_amd", "csrc", "moe_api.hip"), "-o", api])
    drv = os.path.join(OUT, "abi_main.o")
    _run([CLANG, "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-c",
          os.path.join(ROOT, "tests", "abi_sanitize_main.c"), "-o", drv])
    exe = os.path.join(OUT, "abi_sanitize")
    _run([CLANG + "++", "-fsanitize=address,undefined", "-o", exe, drv, api, *objs,
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = _run([exe], env=SAN_ENV)
    assert "all checks passed" in r.stdout
