"""The GEMM's k loop as compiled (CPU, hipcc): every bf16 kernel's main loop
waits for its global->LDS loads once per k tile, at the barrier, and not
after each load.  A compiler that cannot tell those loads' LDS target from
the loop's other LDS accesses inserts a full wait after every load instead;
that serialised the loop of one kernel variant and made it 4x slower, with
identical results -- so no parity test would notice."""

import os
import re
import shutil
import subprocess

import pytest

from collective_overlap_amd import build


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("no hipcc")
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    cmd = [hipcc, *build.COMMON, "-x", "hip", "-S", "--cuda-device-only",
           os.path.join(build.CSRC, "gemm.hip"), "-o", str(out)]
    cmd = [c for c in cmd if c != "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _k_loops(body):
    """Loop bodies (label .. backward branch to it) holding at least 32 MFMAs."""
    loops = []
    for m in re.finditer(r"s_cbranch_\w+ (\.LBB\d+_\d+)\n", body):
        lab = m.group(1)
        p = body.find(lab + ":")
        if 0 <= p < m.start():
            seg = body[p:m.start()]
            if seg.count("v_mfma") >= 32:
                loops.append(seg)
    return loops


def test_every_bf16_kernel_waits_once_per_k_tile(gemm_asm):
    names = re.findall(r"^(_ZN3cce12_GLOBAL__N_116gemm_bf16_kernel\S+):", gemm_asm, re.M)
    assert len(names) >= 24
    checked = 0
    for name in names:
        i = gemm_asm.index(name + ":")
        body = gemm_asm[i:gemm_asm.index("s_endpgm", i)]
        for seg in _k_loops(body):
            loads = len(re.findall(r"buffer_load_dwordx4 .* lds", seg))
            full_waits = len(re.findall(r"s_waitcnt vmcnt\(0\)", seg))
            assert loads >= 8, name
            assert full_waits == 1, f"{name}: {full_waits} full vmcnt waits for {loads} loads"
            checked += 1
    assert checked >= 16


def _longest_store_run(text):
    """The longest stretch of the kernel's code without a branch or label
    that holds 16-byte global stores: (number of stores, the lines)."""
    lines = [l.split(";")[0].strip() for l in text.splitlines()
             if l.strip() and not l.strip().startswith(";")]
    best, cur = (0, []), []
    for l in lines + [".LBB_end:"]:
        if l.startswith("s_cbranch") or l.startswith("s_branch") or l.startswith(".LBB"):
            n = sum("global_store_dwordx4" in x for x in cur)
            if n > best[0]:
                best = (n, cur)
            cur = []
        else:
            cur.append(l)
    return best


@pytest.mark.parametrize("variant", [
    "ILi256ELi256ELi2ELi2ELi64ELi2EfLi1ELb0E",       # fp32 accumulate (ReduceScatter)
    "ILi256ELi256ELi2ELi2ELi64ELi2EfLi0ELb0E",       # fp32 store
    "ILi256ELi256ELi2ELi2ELi64ELi2EDF16bLi0ELb1E",   # bf16 store + GELU (AllGather)
])
def test_whole_tile_stores_are_not_drained_one_by_one(gemm_asm, variant):
    """The staged epilogue of a whole tile stores its 32 chunks of a pass in
    one straight run, and waits for the memory counter there at most once
    (for the accumulator input): a per-chunk drain of the stores had cost
    the ReduceScatter's accumulate launches 3%."""
    name = "_ZN3cce12_GLOBAL__N_116gemm_bf16_kernel" + variant + "EEvNS0_5KArgsE"
    i = gemm_asm.index(name + ":")
    body = gemm_asm[i:gemm_asm.index(".Lfunc_end", i)]
    n, run = _longest_store_run(body)
    assert n >= 32, f"{variant}: longest straight run of stores {n}"
    first = next(k for k, l in enumerate(run) if "global_store_dwordx4" in l)
    drains = [l for l in run[first:] if re.match(r"s_waitcnt vmcnt\(0\)", l)]
    assert drains == [], f"{variant}: {len(drains)} full waits between the stores"
