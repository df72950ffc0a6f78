"""Build libfa.so (the HIP kernels and the C ABI of include/fa.h) for gfx950, in-tree.

    python -m attention_causal_gqa_attn_amd.build          # or build() from Python

Every source is compiled with hipcc --offload-arch=gfx950 -O3, with the packed-FP32 VALU
forms disabled (-Xclang -target-feature -Xclang -packed-fp32-ops); the objects are linked into
attention_causal_gqa_attn_amd/libfa.so next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
SOURCES = ["fa_api.cpp", "fa_prefill16.hip", "fa_decode.hip", "fa_dequant.hip", "fa_quant.hip",
           "fa_standard.hip", "fa_measure.hip"]
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")
    return path


def _quiet(out: str) -> str:
    # the host pass does not know the packed-fp32 feature and says so: harmless
    return "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)


# The prefill kernels issue some MFMAs and lane exchanges from inline asm and wait out their
# hazards with hand-counted s_nop drains; those counts were checked against the code this
# compiler emits. Another compiler may schedule around them differently: the build says so.
TESTED_HIPCC = "AMD clang version 22.0.0git (https://github.com/RadeonOpenCompute/llvm-project roc-7.2.0"
BUILD_INFO = os.path.join(HERE, "libfa.build.json")


def hipcc_version(hipcc=None) -> str:
    r = subprocess.run([hipcc or _hipcc(), "--version"], capture_output=True, text=True)
    return " | ".join(l.strip() for l in r.stdout.splitlines()[:2])


def build_info() -> dict:
    """What build() recorded about the library in this tree (empty if nothing was recorded)."""
    import json
    try:
        with open(BUILD_INFO) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


# host-side AddressSanitizer + UndefinedBehaviorSanitizer (the device code is built as usual):
# every flag goes after -Xarch_host so that it reaches the host compilation only
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, extra_flags=(), out_path: str = LIB,
          host_sanitize: bool = False) -> str:
    """Compile every source and link libfa.so at out_path (default: in-tree). host_sanitize:
    instrument the host code (the C ABI's checks, the launch planning) with ASan and UBSan; such a
    build needs the sanitizer runtime preloaded and is for tests only."""
    import json
    hipcc = _hipcc()
    if host_sanitize:
        extra_flags = tuple(extra_flags) + tuple(HOST_SANITIZE)
    version = hipcc_version(hipcc)
    tested = TESTED_HIPCC in version
    if verbose:
        print(f"hipcc: {version}", flush=True)
    if not tested:
        print(f"warning: {hipcc} is not the compiler the asm hazard drains were checked "
              f"against ({TESTED_HIPCC}...); run the GPU parity tests before trusting it",
              file=sys.stderr, flush=True)
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [hipcc, *COMMON, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".cpp"):
                cmd[1:1] = ["-x", "hip"]
            r = subprocess.run(cmd, capture_output=True, text=True)
            msg = _quiet(r.stdout + r.stderr)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{msg}")
            if verbose and msg.strip():
                print(msg, flush=True)
            return obj

        with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out = os.path.join(tmp, "libfa.so")
        # (a host-sanitized build leaves the sanitizer runtime's symbols to the preloaded runtime)
        cmd = [hipcc, "-shared", f"--offload-arch={ARCH}", *objs, "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{_quiet(r.stdout + r.stderr)}")
        shutil.copyfile(out, out_path + ".tmp")
        os.replace(out_path + ".tmp", out_path)
    if out_path == LIB:
        with open(BUILD_INFO, "w") as f:
            json.dump({"hipcc_version": version, "tested_compiler": tested, "arch": ARCH,
                       "flags": COMMON + list(extra_flags)}, f)
    if verbose:
        print(f"built {out_path}", flush=True)
    return out_path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
