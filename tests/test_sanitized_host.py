"""Host code under the sanitizers, on the CPU.

The C oracle is rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer and must pass its
pin tests; the library's host code (descriptor validation, workspace planning, the ABI entry
points' argument checks) is rebuilt with AddressSanitizer on the host pass only and must pass
the ABI tests. Both runs stop at the first report. Device code is not instrumented and no GPU
is touched.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_moe_layer_05_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
STOP = "detect_leaks=0:abort_on_error=1:halt_on_error=1"


def gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def clang_asan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def run(cmd, env_extra, cwd):
    env = dict(os.environ, **env_extra)
    return subprocess.run(cmd, cwd=cwd, env=env, capture_output=True, text=True, timeout=900)


@pytest.mark.slow
def test_oracle_pins_pass_under_asan_and_ubsan(tmp_path):
    asan, ubsan = gcc_runtime("libasan.so"), gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "_moe_oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                           "-ffp-contract=off", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", lib,
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    script = (
        "import sys; sys.path.insert(0, %r)\n"
        "from oracle import oracle as O\n"
        "O._LIB = %r\n"
        "O.build = lambda force=False: O._LIB\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-x', '-q', '-p', 'no:cacheprovider', %r]))\n"
    ) % (ROOT, lib, os.path.join(ROOT, "tests", "test_oracle_pins.py"))
    r = run([sys.executable, "-c", script],
            dict(LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS=STOP,
                 UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1"), str(tmp_path))
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout


@pytest.mark.slow
def test_abi_checks_pass_with_the_host_code_under_asan(tmp_path):
    asan = clang_asan_runtime()
    objs = [os.path.join(PKG, "_build", f) for f in ("gemm.o", "gemm_kt.o", "routing.o",
                                                      "stream.o", "backward.o", "static_ws.o")]
    if not asan or not os.path.exists(HIPCC):
        pytest.skip("clang AddressSanitizer runtime or hipcc not installed")
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built (run __graft_entry__.build())")
    # a copy of the package and of what the ABI tests read, with the ABI's host translation
    # unit rebuilt under AddressSanitizer
    tree = tmp_path / "tree"
    pkg = tree / "sparse_moe_layer_05_amd"
    pkg.mkdir(parents=True)
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            shutil.copy(os.path.join(PKG, f), pkg / f)
    shutil.copytree(os.path.join(ROOT, "include"), tree / "include")
    (tree / "tests").mkdir()
    for f in ("conftest.py", "test_abi.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tree / "tests" / f)
    api = str(tmp_path / "moe_api_asan.o")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    subprocess.check_call([HIPCC, *flags, "-c", os.path.join(PKG, "csrc", "moe_api.cpp"),
                           "-o", api])
    subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host",
                           "-fsanitize=address", "-shared-libsan", api, *objs, "-o",
                           str(pkg / "libmoe_mi355x.so")])
    r = run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
             "tests/test_abi.py"], dict(LD_PRELOAD=asan, ASAN_OPTIONS=STOP), str(tree))
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
