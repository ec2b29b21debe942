"""Compiles the HIP kernels and the C-ABI layer into page_selected_sparse_amd/libpsd.so.

Every source is compiled for gfx950 only, in parallel, then linked; the library is
replaced atomically. Run ``python -m page_selected_sparse_amd.build``.

The build fails when any kernel spills registers to scratch memory. Several kernels
issue their own ``s_waitcnt vmcnt`` waits for loads they track by count, and a
spilling build adds memory operations the hand-written counts do not name; the
compiler's resource report (``-Rpass-analysis=kernel-resource-usage``) is read for
every kernel, written to ``_build/kernel_resources.txt``, and any nonzero
``ScratchSize`` stops the build.
"""
from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpsd.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-variable", "-Wno-unused-function",
    # packed fp32 VALU ops stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build")
    return path


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


REPORT_FLAG = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]):\s*(\S+)")


def kernel_resources(stderr: str) -> list[dict]:
    """Per-kernel fields of the compiler's resource-usage remarks, in report order."""
    rows: list[dict] = []
    for line in stderr.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1).split()[0], m.group(2)
        if key == "Function":
            rows.append({"name": val})
        elif rows:
            rows[-1][key] = int(val) if val.isdigit() else val
    return rows


def _demangle(names: list[str]) -> list[str]:
    tool = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    if not tool or not names:
        return names
    res = subprocess.run([tool], input="\n".join(names), capture_output=True, text=True)
    out = res.stdout.splitlines()
    return out if len(out) == len(names) else names


def build(verbose: bool = False) -> str:
    """Compile every source and link libpsd.so. Returns the library path. Raises when a
    source fails to compile or any kernel uses scratch memory (register spills)."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()

    def compile_one(src: str):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [hipcc, *FLAGS, REPORT_FLAG, "-c", src, "-o", obj]
        if os.path.basename(src).endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        rows = kernel_resources(res.stderr)
        if verbose:  # diagnostics other than the resource remarks and their source snippets
            rest = [l for l in res.stderr.splitlines()
                    if "remark:" not in l and not re.match(r"\s*\d*\s*\|", l)
                    and "packed-fp32-ops" not in l and not l.startswith("In file included")]
            if rest:
                print("\n".join(rest))
        return obj, [dict(r, source=os.path.basename(src)) for r in rows]

    with ThreadPoolExecutor(max(1, min(len(srcs), os.cpu_count() or 1))) as ex:
        results = list(ex.map(compile_one, srcs))
    objs = [o for o, _ in results]
    kernels = [r for _, rows in results for r in rows]
    for r, name in zip(kernels, _demangle([r["name"] for r in kernels])):
        r["kernel"] = name.replace("psd::(anonymous namespace)::", "")
    with open(os.path.join(BUILD_DIR, "kernel_resources.txt"), "w") as fh:
        fh.write("scratch_bytes_per_lane vgprs agprs waves_per_simd lds_bytes source kernel\n")
        for r in kernels:
            fh.write(f"{r.get('ScratchSize', 0)} {r.get('VGPRs', 0)} {r.get('AGPRs', 0)} "
                     f"{r.get('Occupancy', 0)} {r.get('LDS', 0)} {r['source']} {r['kernel']}\n")
    spills = [r for r in kernels if r.get("ScratchSize", 0)]
    if spills:
        lines = "\n".join(f"  {r['ScratchSize']} B/lane  {r['source']}: {r['kernel']}" for r in spills)
        raise RuntimeError(f"kernels spill registers to scratch memory:\n{lines}")
    if not kernels:
        raise RuntimeError("the compiler printed no kernel resource report")
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
