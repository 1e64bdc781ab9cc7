"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libtidar is compiled with the sanitizers on its host side
(device code is built as usual and never runs: there is no launch here) and
linked with `abi_host_check.c`, which drives every entry point through its
argument checks and sweeps the workspace queries over extreme shapes (int32
limits included). The program fails on any unexpected status and the
sanitizers abort on any memory error, leak or undefined behaviour such as a
signed overflow in a size computation.
"""
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("tidar_build", os.path.join(ROOT, "ar_self_speculative_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.timeout(600)
def test_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = shutil.which("amdclang") or "/opt/rocm/bin/amdclang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not installed")
    b = _build_module()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    # the production flags with -O1 -g for readable reports; the sanitizers apply to host code only
    flags = [f for f in b.HIP_FLAGS if f != "-O3"] + ["-O1", "-g", "-fno-omit-frame-pointer", *san]
    procs, objs = [], []
    for src in b.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        objs.append(obj)
        cmd = [hipcc, "-x", "hip", *flags, *b.EXTRA_FLAGS.get(src, []), "-c", os.path.join(b.CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    for src, pr in procs:
        out, _ = pr.communicate()
        assert pr.returncode == 0, f"{src}:\n{out}"
    drv_o = str(tmp_path / "drv.o")
    r = subprocess.run([clang, "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                        f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(ROOT, "tests", "abi_host_check.c"),
                        "-o", drv_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "abi_host_check")
    r = subprocess.run([hipcc, f"--offload-arch={b.ARCH}", *san, drv_o, *objs, "-o", exe], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host ABI checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr
