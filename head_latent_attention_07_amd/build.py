"""Build the HIP library (libmla_hip.so, gfx950) in place next to this file."""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libmla_hip.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
# the same library with the debug checks of the device-resident integers
# (lengths, block-table entries, append positions) compiled in
DEBUG_LIB_PATH = os.path.join(HERE, "libmla_hip_debug.so")
# the benchmark's calibration kernel (a plain streaming read; not the MLA path)
CALIB_LIB_PATH = os.path.join(HERE, "libmla_calib.so")
CALIB_SOURCES = [os.path.join(HERE, "csrc", "calib.hip")]
SOURCES = [os.path.join(HERE, "csrc", "mla_api.hip")]
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 arithmetic is kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def m0_conflicts(asm_text: str) -> list:
    """Kernels whose inline assembly writes M0 without saving it (the decode
    kernels' direct-to-LDS loads) must not use M0 anywhere else: returns the
    names of those that do, from the device assembly of the library."""
    bad, fn, in_asm, asm_m0, other_m0 = [], None, False, False, False

    def close():
        if fn and asm_m0 and other_m0:
            bad.append(fn)

    for line in asm_text.splitlines():
        s = line.strip()
        m = re.match(r"^([A-Za-z_][\w.$]*):\s*(;.*)?$", s)
        if m and not s.startswith(".") and m.group(1).startswith("_Z"):
            close()
            fn, asm_m0, other_m0 = m.group(1), False, False
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith(";") or s.startswith("."):
            continue
        if re.search(r"\bm0\b", s):
            if in_asm:
                asm_m0 = True
            else:
                other_m0 = True
    close()
    return bad


_SCC_WRITE = re.compile(r"^s_(cmp|and|or|xor|andn2|orn2|nand|nor|xnor|add_|sub_|addk|lshl|lshr|"
                        r"ashr|bfe|min|max|not|abs|bcnt|absdiff)")
_SCC_READ = re.compile(r"^s_(cselect|cbranch_scc|addc|subb|cmov)")


def scc_conflicts(asm_text: str) -> list:
    """Places where the compiler reads SCC after an inline-assembly block that
    writes it and before anything redefines it (an undeclared SCC clobber):
    (kernel, instruction) pairs from the device assembly of the library."""
    bad, fn, in_asm, asm_writes, pending = [], None, False, False, False
    for line in asm_text.splitlines():
        s = line.strip()
        m = re.match(r"^(_Z[\w.$]*):", s)
        if m:
            fn, pending = m.group(1), False
            continue
        if s.startswith(";;#ASMSTART"):
            in_asm, asm_writes = True, False
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            pending = pending or asm_writes
            continue
        if not s or s.startswith(";") or s.startswith("."):
            if s.startswith(".LBB"):
                pending = False
            continue
        op = s.split()[0]
        if in_asm:
            asm_writes = asm_writes or bool(_SCC_WRITE.match(op))
            continue
        if pending:
            if _SCC_READ.match(op):
                bad.append((fn, s))
                pending = False
            elif _SCC_WRITE.match(op) or op.startswith("s_cbranch") or op.startswith("s_branch"):
                pending = False
    return bad


def build(verbose: bool = False, debug_checks: bool = False) -> str:
    """Compile the library (and, alongside, the device assembly for the M0
    and SCC checks); returns the path of the built .so. `debug_checks`
    builds libmla_hip_debug.so (MLA_DEBUG_CHECKS=1) instead."""
    lib_path = DEBUG_LIB_PATH if debug_checks else LIB_PATH
    flags = HIPCC_FLAGS + (["-DMLA_DEBUG_CHECKS=1"] if debug_checks else [])
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), *flags, *SOURCES, "-o", tmp]
    asm_path = lib_path + ".s.tmp"
    asm_flags = [f for f in flags if f not in ("-fPIC", "-shared")]
    asm_cmd = [hipcc(), *asm_flags, "--cuda-device-only", "-S", *SOURCES, "-o", asm_path]
    if verbose:
        print(" ".join(cmd), flush=True)
    lib_proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    asm_proc = subprocess.Popen(asm_cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    lib_out = lib_proc.communicate()
    asm_out = asm_proc.communicate()
    if lib_proc.returncode != 0:
        sys.stderr.write(lib_out[0] + lib_out[1])
        raise RuntimeError(f"hipcc failed with status {lib_proc.returncode}")
    if asm_proc.returncode != 0:
        sys.stderr.write(asm_out[0] + asm_out[1])
        raise RuntimeError(f"hipcc -S failed with status {asm_proc.returncode}")
    with open(asm_path) as f:
        asm_text = f.read()
    os.remove(asm_path)
    bad = m0_conflicts(asm_text)
    if bad:
        os.remove(tmp)
        raise RuntimeError("the compiler uses M0 in kernels whose direct-to-LDS loads assume it "
                           "does not: " + ", ".join(bad))
    bad_scc = scc_conflicts(asm_text)
    if bad_scc:
        os.remove(tmp)
        raise RuntimeError("SCC read after an inline-assembly block that writes it: " +
                           "; ".join(f"{f}: {i}" for f, i in bad_scc[:5]))
    os.replace(tmp, lib_path)
    return lib_path


def build_calib(verbose: bool = False) -> str:
    """The benchmark's calibration library (libmla_calib.so)."""
    tmp = CALIB_LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *CALIB_SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    os.replace(tmp, CALIB_LIB_PATH)
    return CALIB_LIB_PATH


def build_all(verbose: bool = False) -> list:
    """The release and the debug-checks libraries and the calibration one,
    built concurrently."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(3) as ex:
        futs = [ex.submit(build, verbose, dbg) for dbg in (False, True)]
        futs.append(ex.submit(build_calib, verbose))
        return [f.result() for f in futs]


if __name__ == "__main__":
    print("\n".join(build_all(verbose=True)))
