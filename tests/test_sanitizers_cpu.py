"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:
the oracle (built with gcc, then its pins run against it) and the C ABI's
argument validation (libmoe built with the sanitizers on its host code only,
then the ABI validation tests run against it).  A memory or UB error aborts the
sub-process, which fails the test.  GPU code is not instrumented."""
import concurrent.futures
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _run(cmd, env=None, timeout=900):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _gcc_runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libmoe_oracle_san.so")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", lib, "-lm"])
    driver = tmp_path / "run_pins.py"
    driver.write_text(
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import oracle\n"
        f"oracle._LIB = {lib!r}\n"
        "oracle.build = lambda force=False: oracle._LIB\n"
        "import pytest\n"
        f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_oracle_pins.py')!r}]))\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               LD_PRELOAD=f"{_gcc_runtime('libasan.so')}:{_gcc_runtime('libubsan.so')}")
    r = _run([sys.executable, str(driver)], env=env)
    assert " passed" in r.stdout


def test_abi_validation_under_asan_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not os.path.exists(HIPCC) or not rt:
        pytest.skip("hipcc or its sanitizer runtime is not installed")
    srcs = sorted(glob.glob(os.path.join(ROOT, "expert_grouped_gemm_top_amd", "csrc", "*.hip")) +
                  glob.glob(os.path.join(ROOT, "expert_grouped_gemm_top_amd", "csrc", "*.cpp")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), *SAN_HOST, "-shared-libsan", "-c", src, "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libmoe_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN_HOST, "-shared-libsan", *objs, "-o", lib])
    driver = tmp_path / "run_abi.py"
    driver.write_text(
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from expert_grouped_gemm_top_amd import moe\n"
        f"moe.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r},"
        " '-k', 'not exports_every']))\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", LD_PRELOAD=rt[-1])
    r = _run([sys.executable, str(driver)], env=env)
    assert " passed" in r.stdout
