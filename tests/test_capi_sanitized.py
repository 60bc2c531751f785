"""The C ABI's argument validation with the host code under AddressSanitizer
and UndefinedBehaviorSanitizer (no GPU).

tests/test_capi_cpu.py runs again in a child process that loads libvae_san.so
(the same sources built with -fsanitize=address,undefined for the host
compilation; see diffusion_vae_decoder_amd/build.py) with the ASan runtime
preloaded.  Those tests walk every entry point's rejection paths and the
decoder's weight walk and workspace sizing: an out-of-bounds access, a use
after free or undefined behaviour on any of them aborts the child.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "diffusion_vae_decoder_amd", "libvae_san.so")


def asan_runtime():
    clang = shutil.which("clang++", path="/opt/rocm/llvm/bin") or shutil.which("amdclang++")
    if not clang:
        return None
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_validation_paths_under_host_sanitizers():
    if not os.path.exists(SAN_LIB):
        pytest.skip("libvae_san.so is not built (python -m diffusion_vae_decoder_amd.build --sanitized)")
    rt = asan_runtime()
    if rt is None:
        pytest.skip("the ASan runtime of the ROCm toolchain is not installed")
    env = dict(os.environ, LD_PRELOAD=rt, VAE_LIBRARY="libvae_san.so",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_capi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert " passed" in r.stdout and "skipped" not in r.stdout
