"""Build libspecv.so (HIP for gfx950) in-tree with hipcc.

    python -m draft_token_verification_flattened_amd.build [--sanitized-check]

The library is written next to this file so that it travels with the source
tree; every call recompiles. build_sanitized_check() compiles the same sources
and tests/abi_sanitized_check.cpp into one host executable with
AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (device
code is built as usual), for the C ABI's argument validation and host state.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libspecv.so")

SOURCES = ["abi.cpp", "schedule.hip", "verify.hip", "markov.hip", "attention.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Per-source flags. The verification kernels treat logits as finite numbers:
# without IEEE-mode NaN quieting, max over widened bf16 values needs no
# canonicalising instruction per element.
SOURCE_FLAGS = {"verify.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


# Kernels must not spill VGPRs. The compiler can place a spill store inside a
# lane-divergent block (an `if (lane == 0)` region), where it saves only the
# active lanes, and reload the value later with every lane active: the other
# lanes then read stale scratch memory (for an address, a wild access). Every
# kernel is kept within its register budget, and the build refuses one that is
# not.
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
_REMARK_NAME = re.compile(r"remark:\s+Function Name: (\S+)")
_REMARK_SPILL = re.compile(r"remark:\s+VGPRs Spill: (\d+)")


def vgpr_spills(remarks: str) -> dict:
    """{kernel: spilled VGPRs} for every kernel with spills in the compiler's
    kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = _REMARK_NAME.search(line)
        if m:
            cur = m.group(1)
            continue
        m = _REMARK_SPILL.search(line)
        if m and cur is not None and int(m.group(1)) > 0:
            out[cur] = int(m.group(1))
    return out


def _compile(src: str, hipcc: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    else:
        cmd += RESOURCE_REMARKS
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    spills = vgpr_spills(res.stderr)
    if spills:
        raise RuntimeError(f"{src}: kernels spill VGPRs (refused): {spills}")
    if verbose:
        rest = "\n".join(l for l in res.stderr.splitlines() if "remark:" not in l).strip()
        if rest:
            print(rest, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    hipcc = _hipcc()
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host code only: each sanitizer flag goes to the host compilation and link.
SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]
SAN_DIR = os.path.join(OBJDIR, "sanitized")
SAN_CHECK = os.path.join(SAN_DIR, "abi_sanitized_check")
SAN_DRIVER = os.path.join(ROOT, "tests", "abi_sanitized_check.cpp")


def build_sanitized_check(verbose: bool = False, planted: bool = False) -> str:
    """The sanitized host check executable (see the module docstring).
    planted=True builds a copy whose driver ends with a heap overflow, the
    control that shows the sanitizers are active (it must abort)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    hipcc = _hipcc()
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"] + SANITIZE
    if planted:
        flags.append("-DSPECV_PLANTED_OVERFLOW")
    tag = "_planted" if planted else ""

    def one(src):
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        obj = os.path.join(SAN_DIR, os.path.splitext(os.path.basename(src))[0] + tag + ".o")
        cmd = [hipcc, "-xhip", *flags, *SOURCE_FLAGS.get(os.path.basename(src), []), "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        objs = list(ex.map(one, SOURCES + [SAN_DRIVER]))
    exe = SAN_CHECK + tag
    cmd = [hipcc, f"--offload-arch={ARCH}", *SANITIZE, "-o", exe, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    return exe


if __name__ == "__main__":
    if "--sanitized-check" in sys.argv:
        print(build_sanitized_check(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
