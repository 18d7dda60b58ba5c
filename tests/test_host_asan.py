"""The C ABI's host code under AddressSanitizer (CPU only).

The library's host side (argument validation, split planning, workspace
layout, the launch code up to the first HIP call) is rebuilt with
AddressSanitizer; its device code is the release build's (the sanitizer
flags go to the host compilation only). The ABI tests then run against that
build in a child process with the sanitizer's runtime preloaded: any
out-of-bounds or use-after-free access in the host code aborts the child.
No call here reaches a kernel (there is no GPU in the CPU test run)."""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "head_latent_attention_07_amd")
OUT = os.path.join(ROOT, "_build", "libmla_hip_asan.so")


def asan_runtime():
    from head_latent_attention_07_amd import build as b
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(b.hipcc()))), "llvm")
    pats = [os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"),
            "/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"]
    for pat in pats:
        hits = sorted(glob.glob(pat))
        if hits:
            return hits[-1]
    return None


def sources():
    out = [os.path.join(ROOT, "include", "mla.h")]
    out += glob.glob(os.path.join(PKG, "csrc", "*"))
    return out


def build_asan():
    """hipcc with the sanitizer on the host side only (each -fsanitize= right
    after -Xarch_host); rebuilt when a source is newer than the library."""
    from head_latent_attention_07_amd import build as b
    if os.path.exists(OUT) and os.path.getmtime(OUT) >= max(os.path.getmtime(s) for s in sources()):
        return OUT
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    host_only = ["-Xarch_host", "-fsanitize=address",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    cmd = [b.hipcc(), *b.HIPCC_FLAGS, *host_only, *b.SOURCES, "-o", OUT + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    os.replace(OUT + ".tmp", OUT)
    return OUT


@pytest.fixture(scope="module")
def asan_env():
    rt = asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime next to hipcc's clang")
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("LD_PRELOAD is already set in this environment; the sanitizer runtime "
                    "must be the first preloaded library")
    lib = build_asan()
    env = dict(os.environ, LD_PRELOAD=rt, MLA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1")
    return env, lib


def test_asan_build_is_instrumented(asan_env):
    env, lib = asan_env
    code = ("import ctypes, head_latent_attention_07_amd as m; m.load(); "
            "ctypes.CDLL(None).__asan_init; "
            "assert any('libclang_rt.asan' in l for l in open('/proc/self/maps')); "
            "assert m.status_string(0) == 'MLA_OK'; print('asan runtime live')")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert "__asan_report_load" in nm.stdout


def test_abi_suite_under_asan(asan_env):
    env, _ = asan_env
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    print(r.stdout[-1500:])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr
