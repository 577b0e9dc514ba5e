"""Build libdas.so for gfx950 with hipcc, in-tree.

Each source is compiled to an object with its device assembly kept, the
objects are linked into ``volumetric_delay_sum_amd/libdas.so``, and the kept
assembly is scanned for the one hazard the hand-written DPP arithmetic can
expose: a VALU write of a VGPR read through DPP fewer than two wait states
later (or an EXEC write fewer than five).  A build with such a hazard fails.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdas.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> tuple[str, str]:
    base = os.path.splitext(os.path.basename(src))[0]
    obj = os.path.join(BUILD_DIR, base + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd.insert(1, "-save-temps=obj")
        cmd += ["-x", "hip"] if False else []
    res = subprocess.run(cmd, cwd=BUILD_DIR, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj, res.stderr


_REG = re.compile(r"^-?\|?v(\d+)\|?$")
_RANGE = re.compile(r"^v\[(\d+):(\d+)\]$")


def _regs(tok: str) -> set[int]:
    tok = tok.strip().rstrip(",")
    m = _REG.match(tok)
    if m:
        return {int(m.group(1))}
    m = _RANGE.match(tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return set()


def scan_dpp_hazards(asm_text: str) -> list[str]:
    """Return a description of every DPP read too close to a VALU write of its source."""
    lines = []
    for raw in asm_text.splitlines():
        s = raw.split(";")[0].strip()
        if not s or s.startswith(".") or s.startswith("//"):
            continue
        lines.append(s)
    problems = []
    for i, s in enumerate(lines):
        op = s.split()[0]
        if "_dpp" not in op:
            continue
        ops = s[len(op):].split(",")
        if len(ops) < 2:
            continue
        src0 = _regs(ops[1].split()[0])
        waits = 0
        j = i - 1
        while j >= 0 and waits < 5:
            t = lines[j]
            if t.endswith(":"):
                if waits < 5:
                    # control can arrive from elsewhere: require the gap inside this block
                    problems.append(f"label within the DPP wait window before: {s}")
                break
            top = t.split()[0]
            if top == "s_nop":
                waits += int(t.split()[1], 0) + 1
            else:
                if top.startswith("v_") and waits < 2:
                    dst = _regs(t[len(top):].split(",")[0])
                    if dst & src0:
                        problems.append(f"VALU write '{t}' then DPP read '{s}' after {waits} wait states")
                if ("exec" in t.split(",")[0]) and not top.startswith("s_waitcnt"):
                    problems.append(f"EXEC write '{t}' then DPP '{s}' after {waits} wait states")
                waits += 1
            j -= 1
    return problems


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source for gfx950 and link libdas.so (always rebuilds)."""
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    for f in glob.glob(os.path.join(BUILD_DIR, "*")):
        if os.path.isfile(f):
            os.remove(f)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    problems = []
    for asm in glob.glob(os.path.join(BUILD_DIR, f"*-hip-amdgcn-amd-amdhsa-{ARCH}.s")):
        problems += [f"{os.path.basename(asm)}: {p}" for p in scan_dpp_hazards(open(asm).read())]
    if problems:
        raise RuntimeError("DPP hazard check failed:\n" + "\n".join(problems[:20]))
    tmp = LIB + f".tmp{os.getpid()}"
    res = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                         cwd=BUILD_DIR, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
