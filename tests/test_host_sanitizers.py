"""Host-side AddressSanitizer / UndefinedBehaviorSanitizer runs (CPU only).

  * the oracle (oracle.c) built with gcc's ASan + UBSan and driven by its own
    pin tests in a child process;
  * the C-ABI host layer of libbga (bga_abi.hip, argument validation) built
    with ASan + UBSan on the host side only and linked with the release kernel
    objects, driven by the C-ABI tests in a child process (every call there
    returns before any device call).

A sanitizer report aborts the child (halt_on_error, no recovery), so the test
fails on the first invalid access or undefined operation. Sanitizer runtimes
are preloaded into the child interpreter, which itself is not instrumented.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_OPTS = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def run_child(args, env_extra, timeout=600):
    env = dict(os.environ, **SAN_OPTS, **env_extra)
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *args], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=timeout)
    out = p.stdout + p.stderr
    assert p.returncode == 0 and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan(tmp_path):
    import oracle
    gcc_rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(gcc_rt):
        pytest.skip("gcc's libasan is not installed")
    lib = str(tmp_path / "liboracle_asan.so")
    flags = [f for f in oracle.GCC_FLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                          "-fsanitize=address,undefined",
                                                          "-fno-sanitize-recover=all"]
    subprocess.run(["gcc", *flags, os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"], check=True)
    out = run_child(["tests/test_oracle_pins.py"], {"LD_PRELOAD": gcc_rt, "BGA_ORACLE_LIB": lib})
    assert " passed" in out


def test_abi_host_layer_under_asan_ubsan(tmp_path):
    import attention_bga_packed_amd.build as hb
    hipcc = shutil.which(os.environ.get("HIPCC", "hipcc"))
    if hipcc is None:
        pytest.skip("hipcc not found")
    clang_rt = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "llvm", "bin", "clang"),
                               "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    rt = clang_rt.stdout.strip()
    if clang_rt.returncode != 0 or not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("clang's ASan runtime is not installed")
    hb.build()   # release kernel objects in _build/
    abi_obj = str(tmp_path / "bga_abi_asan.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    subprocess.run([hipcc, *hb.HIPCC_FLAGS, *san, "-c", os.path.join(hb.CSRC, "bga_abi.hip"), "-o", abi_obj],
                   check=True, capture_output=True)
    objs = [os.path.join(hb.BUILD, os.path.basename(s)[:-4] + ".o") for s in hb.sources()
            if os.path.basename(s) != "bga_abi.hip"]
    lib = str(tmp_path / "libbga_asan.so")
    subprocess.run([hipcc, f"--offload-arch={hb.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libasan", abi_obj, *objs, "-o", lib],
                   check=True, capture_output=True)
    out = run_child(["tests/test_abi.py"], {"LD_PRELOAD": rt, "BGA_LIBRARY": lib})
    assert " passed" in out
