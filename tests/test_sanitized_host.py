"""The CPU tests of the C ABI and of the input generator, run once more
against host code built with AddressSanitizer and UndefinedBehaviorSanitizer.

Built here, in a temporary folder:
  libready.so  ready_api.cpp (plans, argument validation, workspace sizes,
               status strings) and ready_static.hip, host parts sanitized
               (the device code of ready_static.hip is built as usual), with
               the kernel launchers replaced by stubs that report no device
               (tests/sanitize/launch_stubs.cpp): none of these tests reaches
               a launch.
  libsynth.so  synth/gdn_gen.c, the counter-based input generator.
Both use clang's shared sanitizer runtime, which the child pytest process
preloads; tests/sanitize/plugin.py points the binding and the generator at
these libraries.  Any sanitizer report ends the child with an error.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hla_recurrent_state_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
SUITES = ["tests/test_abi.py", "tests/test_abi_multi.py", "tests/test_synth.py"]
SAN_HOST = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer"]


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    res = subprocess.run([CLANG, "-print-resource-dir"], stdout=subprocess.PIPE, text=True)
    hits = sorted(glob.glob(os.path.join(res.stdout.strip(), "lib", "*", "libclang_rt.asan-x86_64.so")) +
                  glob.glob(os.path.join(res.stdout.strip(), "lib", "*", "libclang_rt.asan.so")))
    return hits[0] if hits else None


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-4000:]


def _instrumented(path):
    res = subprocess.run(["nm", "-D", "--undefined-only", path], stdout=subprocess.PIPE, text=True)
    return "__asan_init" in res.stdout or "__asan_report_load8" in res.stdout


@pytest.mark.timeout(900)
def test_abi_and_generator_tests_pass_under_asan_and_ubsan(tmp_path):
    asan = _asan_runtime()
    if asan is None or not os.path.exists(HIPCC):
        pytest.skip("clang sanitizer runtime or hipcc not found")
    rt_dir = os.path.dirname(asan)
    lib = str(tmp_path / "libready.so")
    host_flags = []
    for f in SAN_HOST:
        host_flags += ["-Xarch_host", f]
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
          "-I" + os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + host_flags +
         ["-shared-libsan", "-Wl,--no-undefined", "-Wl,-rpath," + rt_dir,
          "ready_api.cpp", "ready_static.hip", os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
          "-o", lib], cwd=CSRC)
    syn = str(tmp_path / "libsynth.so")
    _run([CLANG, "-O1", "-g", "-mavx2", "-mfma", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"] +
         SAN_HOST + ["-shared-libsan", "-Wl,-rpath," + rt_dir, "-Wl,-rpath,/opt/rocm/llvm/lib",
                     "gdn_gen.c", "-o", syn, "-lm"], cwd=os.path.join(ROOT, "synth"))
    assert _instrumented(lib) and _instrumented(syn)

    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": asan,
        # the interpreter and the HIP runtime are not built for leak checking
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:alloc_dealloc_mismatch=0:detect_odr_violation=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "READY_SAN_DIR": str(tmp_path),
        "PYTHONPATH": ROOT + os.pathsep + env.get("PYTHONPATH", ""),
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider",
                          "-p", "tests.sanitize.plugin", "-m", "not gpu"] + SUITES,
                         cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=600)
    out = res.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert res.returncode == 0, out[-6000:]
    assert " passed" in out and " failed" not in out, out[-3000:]
