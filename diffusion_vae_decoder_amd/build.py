"""Build libvae.so for gfx950 with hipcc (run on any host; no GPU needed).

    python -m diffusion_vae_decoder_amd.build [--sanitized]

Every HIP source under csrc/ is compiled to an object in _build/ (in
parallel), then linked into diffusion_vae_decoder_amd/libvae.so next to this
file.  Always rebuilds.  With --sanitized (or build(sanitized=True)) the same
sources are built into libvae_san.so with the host code instrumented by
AddressSanitizer and UndefinedBehaviorSanitizer (the device code is not
instrumented); it loads only into a process that starts with the ASan runtime
preloaded (tests/test_capi_sanitized.py runs the C ABI's validation tests that
way, on the CPU).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvae.so")
SAN_LIB = os.path.join(PKG, "libvae_san.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # no packed-FP32 (v_pk_*_f32) code generation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# host-side sanitizers only: each -fsanitize= goes to the host compilation
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-O1"]


def _compile(src: str, sanitized: bool = False) -> str:
    out = os.path.join(BUILD, "san") if sanitized else BUILD
    obj = os.path.join(out, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *(SAN_FLAGS if sanitized else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(verbose: bool = True, sanitized: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, "san") if sanitized else BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitized), srcs))
    lib = SAN_LIB if sanitized else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if sanitized:
        cmd[1:1] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


if __name__ == "__main__":
    build(sanitized="--sanitized" in sys.argv[1:])
