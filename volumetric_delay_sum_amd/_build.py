"""Build libdas.so for gfx950 with hipcc, in-tree.

Each source is compiled to an object with its device assembly kept, the
objects are linked into ``volumetric_delay_sum_amd/libdas.so``, and the kept
assembly is scanned for the one hazard the hand-written DPP arithmetic can
expose: a VALU write of a VGPR read through DPP fewer than two wait states
later (or a VALU write of EXEC fewer than five).  A build with such a hazard fails.
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


_LABEL = re.compile(r"^\.?[\w$.]+:$")


def scan_dpp_hazards(asm_text: str) -> list[str]:
    """Return a description of every DPP read too close to a VALU write of its source.

    The scan walks backwards from each DPP instruction until five wait states
    have passed.  At a label it continues into every predecessor (the
    fall-through and each branch to the label), so a hazard across a branch is
    found too; a walk that does not settle within a few predecessor hops is
    reported.  Functions are scanned separately.
    """
    lines = []
    for raw in asm_text.splitlines():
        s = raw.split(";")[0].strip()
        if not s or s.startswith("//"):
            continue
        if s.startswith(".") and not _LABEL.match(s):
            continue                # assembler directive
        lines.append(s)
    # branches to each label, by line index of the branch
    branches: dict[str, list[int]] = {}
    for i, s in enumerate(lines):
        top = s.split()[0]
        if top.startswith("s_cbranch") or top == "s_branch":
            parts = s.split()
            if len(parts) > 1:
                branches.setdefault(parts[-1], []).append(i)
    uncond = ("s_branch", "s_setpc_b64", "s_endpgm")
    problems = []

    def walk(dpp: str, src0: set, j: int, waits: int, hops: int):
        while j >= 0 and waits < 5:
            t = lines[j]
            if t.endswith(":"):
                if _LABEL.match(t) and not t.startswith("."):
                    return          # function entry: nothing runs before it
                if hops >= 6:
                    problems.append(f"unresolved control flow within the DPP wait window before: {dpp}")
                    return
                label = t[:-1]
                prev = lines[j - 1].split()[0] if j > 0 else "s_endpgm"
                if prev not in uncond:
                    walk(dpp, src0, j - 1, waits, hops + 1)
                for b in branches.get(label, []):
                    walk(dpp, src0, b - 1, waits, hops + 1)
                return
            top = t.split()[0]
            if top == "s_nop":
                waits += int(t.split()[1], 0) + 1
            else:
                if top.startswith("v_") and waits < 2:
                    dst = _regs(t[len(top):].split(",")[0])
                    if dst & src0:
                        problems.append(f"VALU write '{t}' then DPP read '{dpp}' after {waits} wait states")
                # a VALU write of EXEC (v_cmpx, or a VALU op targeting exec) needs 5 wait
                # states before a DPP op; scalar writes of EXEC are interlocked
                dst0 = t[len(top):].split(",")[0].strip()
                if top.startswith("v_cmpx") or (top.startswith("v_") and dst0 in ("exec", "exec_lo", "exec_hi")):
                    problems.append(f"VALU EXEC write '{t}' then DPP '{dpp}' after {waits} wait states")
                waits += 1
            j -= 1

    for i, s in enumerate(lines):
        op = s.split()[0]
        if "_dpp" not in op:
            continue
        ops = s[len(op):].split(",")
        if len(ops) < 2:
            continue
        walk(s, _regs(ops[1].split()[0]), i - 1, 0, 0)
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
