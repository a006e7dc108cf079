"""Host-side sanitizer builds (CPU only).

The input generator (synth/synth.c) and the library's host code (argument
checks, planning, the C ABI in csrc/api.hip) are rebuilt with
AddressSanitizer and UndefinedBehaviorSanitizer on the host pass only (the
device code is compiled as usual and never runs here), and the CPU tests
that drive them - the ABI checks and the generator tests - run again in a
subprocess with the sanitizer runtime preloaded.  Any report fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.slow
def test_host_code_under_asan_and_ubsan(tmp_path):
    rt = _asan_runtime()
    if not (rt and os.path.exists(CLANG) and os.path.exists(HIPCC)):
        pytest.skip("ROCm clang / sanitizer runtime not found")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    synth_lib = tmp_path / "libsynth_san.so"
    r = subprocess.run([CLANG, "-O1", "-g", *san, "-shared-libsan", "-std=gnu11", "-fPIC", "-shared", "-pthread",
                        os.path.join(ROOT, "synth", "synth.c"), "-o", str(synth_lib), "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    phi_lib = tmp_path / "libphi_san.so"
    host = []
    for f in san:  # host pass only: each sanitizer flag right after -Xarch_host
        host += ["-Xarch_host", f]
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-g", "-std=c++17", "-fPIC", "-shared",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host, "-shared-libsan",
                        os.path.join(ROOT, "logits_parity_amd", "csrc", "api.hip"), "-o", str(phi_lib)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PHI_LIB=str(phi_lib), SYNTH_LIB=str(synth_lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_synth.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
