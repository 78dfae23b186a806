"""Build libcce.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

Usage: python -m collective_overlap_amd.build [--jobs N]

The library links against the HIP runtime that torch ships (torch/lib), so
that the streams and device pointers torch hands over belong to the same
runtime instance; /opt/rocm/lib is the fallback search path when the library
is loaded without torch.
"""

from __future__ import annotations

import argparse
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcce.so")
ROOT = os.path.dirname(PKG)

SOURCES = ["gemm.hip", "epilogue.hip", "permute.hip", "plan.cpp", "abi.cpp"]
# Standalone measurement programs, not part of the library: the rate the
# matrix cores sustain on MFMAs and LDS operand reads alone (bench.py
# --mfma-ceiling runs it), and what HBM sustains for plain streaming kernels
# (bench.py --hbm-ceiling).
PROBES = ("mfma_ceiling", "hbm_ceiling")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def torch_lib_dir() -> str | None:
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec is None or not spec.submodule_search_locations:
            return None
        d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
        return d if os.path.exists(os.path.join(d, "libamdhip64.so")) else None
    except Exception:
        return None


COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 VALU ops stay off: hipcc -O3 would otherwise form them from
    # plain float code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Loops marked for full unrolling stay fully unrolled up to this size: the
    # GEMM epilogue's passes index the accumulator registers by the pass
    # number, and a pass left rolled would move them to scratch memory.
    "-mllvm", "-pragma-unroll-threshold=65536",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


# Kernels allowed to use scratch memory (register spills), with the bytes
# per lane this compiler gives them today: the 256 x 256 bf16 store without
# GELU (the local partial GEMM) and the 256 x 256 bf16 accumulate without GELU
# (only the last iteration of an AllGather case 2 with a bf16 output runs it),
# two registers each.  Any other spill, or a larger one, fails the build: in a
# GEMM it would otherwise show only as an unexplained slowdown.
KNOWN_SPILLS = {
    "_ZN3cce12_GLOBAL__N_116gemm_bf16_kernelILi256ELi256ELi2ELi2ELi64ELi2EDF16bLi0ELb0EEEvNS0_5KArgsE": 8,
    "_ZN3cce12_GLOBAL__N_116gemm_bf16_kernelILi256ELi256ELi2ELi2ELi64ELi2EDF16bLi1ELb0EEEvNS0_5KArgsE": 8,
}


def scratch_by_kernel(remarks: str) -> dict:
    """Kernel name -> scratch bytes per lane, from the compiler's
    kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and cur is not None:
            out[cur] = int(m.group(1))
    return out


def check_spills(scratch: dict, known=None) -> list:
    """Kernels whose scratch use is not in `known` or exceeds it."""
    known = KNOWN_SPILLS if known is None else known
    return sorted(f"{k}: {v} bytes/lane (allowed {known.get(k, 0)})"
                  for k, v in scratch.items() if v > known.get(k, 0))


def compile_one(src: str, extra=(), build_dir: str = BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    remarks = ["-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *extra, *remarks, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    bad = check_spills(scratch_by_kernel(r.stderr))
    if bad:
        raise RuntimeError(f"{src}: kernels spill to scratch memory:\n  " + "\n  ".join(bad))
    return obj


def build(jobs: int = 4, verbose: bool = False, extra=(), out: str = LIB,
          build_dir: str = BUILD) -> str:
    """Compile every source and link `out`.  `extra` adds compiler flags
    (e.g. the GEMM k-tile knob -DCCE_GEMM_BK=..)."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda src: compile_one(src, extra, build_dir), SOURCES))
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", out + ".tmp", *objs]
    tl = torch_lib_dir()
    if tl:
        link += [f"-L{tl}", f"-Wl,-rpath,{tl}"]
    link += ["-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(link)}\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)
    if out == LIB:
        for name in PROBES:
            build_probe(name)
    if verbose:
        print(f"built {out}")
    return out


def build_probe(name: str = "mfma_ceiling") -> str:
    """Compile a measurement program (an executable beside the library, not
    linked into it) from csrc/<name>.hip."""
    out = os.path.join(PKG, name)
    cmd = [hipcc(), *COMMON, "-x", "hip", os.path.join(CSRC, name + ".hip"), "-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)
    return out


def sources_at(rev: str) -> str:
    """Write the library's sources (csrc/ and include/cce.h) as of git
    revision `rev` under the build directory; returns the csrc copy, for
    building an older library beside the current one (A/B timing)."""
    top = os.path.join(BUILD, "rev_" + re.sub(r"[^0-9A-Za-z_.-]", "_", rev))
    csrc = os.path.join(top, "collective_overlap_amd", "csrc")
    os.makedirs(csrc, exist_ok=True)
    os.makedirs(os.path.join(top, "include"), exist_ok=True)

    def show(path):
        r = subprocess.run(["git", "-C", ROOT, "show", f"{rev}:{path}"], capture_output=True)
        return r.stdout if r.returncode == 0 else None

    hdr = show("include/cce.h")
    if hdr is None:
        raise RuntimeError(f"include/cce.h not found at {rev}")
    open(os.path.join(top, "include", "cce.h"), "wb").write(hdr)
    ls = subprocess.run(["git", "-C", ROOT, "ls-tree", "--name-only", f"{rev}:collective_overlap_amd/csrc"],
                        capture_output=True, text=True)
    if ls.returncode != 0:
        raise RuntimeError(ls.stderr.strip())
    for f in ls.stdout.split():
        open(os.path.join(csrc, f), "wb").write(show(f"collective_overlap_amd/csrc/{f}"))
    return csrc


def main(argv=None):
    global CSRC
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(4, os.cpu_count() or 1))
    ap.add_argument("--rev", help="build the sources of this git revision instead of the "
                                  "working tree (needs --out)")
    ap.add_argument("--out", help="library path (default: the package's libcce.so)")
    a = ap.parse_args(argv)
    if a.rev and not a.out:
        ap.error("--rev needs --out: the package's own library is built from the working tree")
    out = os.path.abspath(a.out) if a.out else LIB
    bd = BUILD
    if a.rev:
        CSRC = sources_at(a.rev)
        top = os.path.dirname(os.path.dirname(CSRC))
        # that revision's header, not the working tree's
        i = COMMON.index(os.path.join(ROOT, "include"))
        COMMON[i] = os.path.join(top, "include")
        SOURCES[:] = [f for f in SOURCES if os.path.exists(os.path.join(CSRC, f))]
        bd = os.path.join(top, "obj")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    build(a.jobs, verbose=True, out=out, build_dir=bd)


if __name__ == "__main__":
    sys.exit(main())
