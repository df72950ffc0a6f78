"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer: libfa.so with its host side
(the C ABI's argument checks, the launch planning) instrumented, and the C oracle, each loaded
into a child process with its sanitizer runtime preloaded, running the ABI rejection suite and
the oracle pin suite. No GPU is needed: none of these calls reaches a kernel launch."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _clang_asan():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _gcc_asan():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    except OSError:
        return None
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run(args, env_extra, timeout=600):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt_clang, rt_gcc = _clang_asan(), _gcc_asan()
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")) or not rt_clang \
            or not rt_gcc:
        pytest.skip("hipcc, gcc or a sanitizer runtime is missing")
    d = tmp_path_factory.mktemp("san")
    from attention_causal_gqa_attn_amd import build as fa_build
    lib = fa_build.build(out_path=str(d / "libfa_san.so"), host_sanitize=True)
    orc = str(d / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "fa_oracle.c"),
                    "-o", orc, "-lm"], check=True)
    return {"lib": lib, "orc": orc, "rt_clang": rt_clang, "rt_gcc": rt_gcc}


def test_abi_checks_under_asan_ubsan(sanitized):
    env = {"LD_PRELOAD": sanitized["rt_clang"], "FA_LIBRARY": sanitized["lib"]}
    which = _run(["-c", "import attention_causal_gqa_attn_amd as fa; fa.load(); print(fa.LIB_PATH)"],
                 env)
    assert which.returncode == 0, which.stderr[-2000:]
    assert which.stdout.strip() == sanitized["lib"]
    r = _run(["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"], env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])


def test_oracle_pins_under_asan_ubsan(sanitized):
    env = {"LD_PRELOAD": sanitized["rt_gcc"], "FA_ORACLE_LIB": sanitized["orc"]}
    which = _run(["-c", "import oracle; print(oracle.default().path)"], env)
    assert which.returncode == 0, which.stderr[-2000:]
    assert which.stdout.strip() == sanitized["orc"]
    # the mutation test compiles its own copies of the oracle: left to the plain suite
    r = _run(["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_oracle.py",
              "-k", "not planted"], env)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
