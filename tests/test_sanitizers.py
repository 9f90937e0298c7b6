"""CPU: AddressSanitizer and UndefinedBehaviorSanitizer over host code.

- the fp64 oracle (oracle/ddts_oracle.c), built by gcc with both sanitizers
  into a small driver (tests/sanitize/oracle_driver.c) that runs its forward,
  decode step and reverse mode on awkward shapes (T = 0, dk = dv = 1, odd
  widths, several threads);
- the library's host code (argument checks, plans, size queries in
  csrc/api.hip), compiled with host-only sanitizers (hipcc -Xarch_host),
  linked with the normally built kernel objects, and driven by the ABI tests
  (tests/test_abi.py) with the sanitizer runtime preloaded.
Any sanitizer report aborts the process (no recovery), failing the test."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["address", "undefined"]


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-pthread",
           "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
           "-fsanitize=" + ",".join(SAN),
           os.path.join(HERE, "sanitize", "oracle_driver.c"),
           os.path.join(ROOT, "oracle", "ddts_oracle.c"), "-lm", "-o", exe]
    subprocess.check_call(cmd)
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([exe], env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    print(p.stdout)
    assert p.returncode == 0, p.stdout
    assert "FAILED" not in p.stdout and p.stdout.count("ok") == 5


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not found")
def test_library_host_code_under_asan_ubsan(tmp_path):
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.o")))
    others = [o for o in objs if not o.endswith("api.hip.o")]
    if len(others) < 8:
        pytest.skip("the library's objects are not built (run the build first)")
    api = str(tmp_path / "api_san.o")
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", "-fsanitize=" + s]
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           *host_san, "-Xarch_host", "-fno-sanitize-recover=all",
                           "-I" + os.path.join(ROOT, "include"), "-c",
                           os.path.join(ROOT, "gated_linear_attention_rodimus_amd", "csrc",
                                        "api.hip"), "-o", api],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    lib = str(tmp_path / "librodimus_ddts_san.so")
    subprocess.check_call([CLANG, "-shared", "-fPIC", "-shared-libasan",
                           "-fsanitize=" + ",".join(SAN), "-o", lib, api, *others,
                           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    rt = subprocess.check_output([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 text=True).strip()
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="abort_on_error=1:detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([sys.executable, os.path.join(HERE, "sanitize", "abi_driver.py"), lib],
                       env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    print(p.stdout[-3000:])
    assert p.returncode == 0, p.stdout[-3000:]
    assert "passed" in p.stdout
