"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two drivers under tests/sanitize/: oracle_checks.c runs every oracle entry
point on small seeded shapes (gcc); abi_checks.cpp links the C ABI's real host
code (argument checks, workspace layout, miss-policy replay) with kernel
launchers that abort if reached, and drives every validation path (hipcc with
the sanitizers on the host side only, clang++ to link). A sanitizer report, a
failed check or a launch reached from a rejected call fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routed_expert_quantized_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(SAN, "oracle_checks.c"), "-lm", "-o", exe],
         tmp_path)
    r = _run([exe], tmp_path)
    assert r.stdout.strip() == "ok" and "runtime error" not in r.stderr


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm toolchain missing")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["-x", "hip", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *san,
              "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = []
    # moe_api.cpp holds a device array, so it needs its device half (built without sanitizers)
    for src, extra in ((os.path.join(CSRC, "moe_api.cpp"), ["--offload-arch=gfx950"]),
                       (os.path.join(CSRC, "miss_replay.cpp"), ["--cuda-host-only"]),
                       (os.path.join(SAN, "abi_checks.cpp"), ["--cuda-host-only"])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, *extra, *common, "-c", src, "-o", obj], tmp_path)
        objs.append(obj)
    exe = str(tmp_path / "abi_checks")
    _run([CLANGXX, "-fsanitize=address,undefined", *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe], tmp_path)
    r = _run([exe], tmp_path)
    assert r.stdout.strip() == "ok" and "runtime error" not in r.stderr
