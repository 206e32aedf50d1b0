"""Compile libfa.so (gfx950) in-tree with hipcc.

Every source under ``csrc/`` is compiled to an object in ``_build/`` (in
parallel) and linked into ``exact_tiled_attention_amd/libfa.so``.  Runs on a
machine without a GPU: hipcc cross-compiles for gfx950.

After compiling, the gfx950 code object of every object file is read back
(its kernel metadata: registers, LDS, scratch) and the build fails if any
kernel spills to scratch memory, which would silently cost the hot loop an
order of magnitude.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU ops.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libfa.so cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(hipcc, src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIP_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _llvm_tool(name):
    for d in (os.environ.get("ROCM_PATH", "/opt/rocm") + "/llvm/bin", "/opt/rocm/llvm/bin"):
        p = os.path.join(d, name)
        if os.path.exists(p):
            return p
    return None


def kernel_resources(obj: str) -> list[dict]:
    """Kernel metadata of the gfx950 code object embedded in a built object.

    Returns one dict per kernel: name, vgpr (VGPR + AGPR count), agpr, sgpr,
    lds (bytes), scratch (private segment bytes per lane), vgpr_spill,
    sgpr_spill.  Empty if the LLVM tools are not installed.
    """
    objcopy, bundler, readelf = (_llvm_tool(t) for t in ("llvm-objcopy", "clang-offload-bundler",
                                                         "llvm-readelf"))
    if not (objcopy and bundler and readelf):
        return []
    with tempfile.TemporaryDirectory() as td:
        fb, co = os.path.join(td, "fatbin"), os.path.join(td, "code.elf")
        subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fb}", obj, os.path.join(td, "host.o")],
                       check=True, capture_output=True)
        subprocess.run([bundler, "--unbundle", "--type=o", f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}",
                        f"--input={fb}", f"--output={co}"], check=True, capture_output=True)
        notes = subprocess.run([readelf, "--notes", co], check=True, capture_output=True, text=True).stdout
    keys = {"agpr_count": "agpr", "group_segment_fixed_size": "lds", "private_segment_fixed_size": "scratch",
            "sgpr_count": "sgpr", "sgpr_spill_count": "sgpr_spill", "vgpr_count": "vgpr",
            "vgpr_spill_count": "vgpr_spill"}
    out = []
    # kernel entries are the two-space-indented items of the amdhsa.kernels list
    body = notes[notes.index("amdhsa.kernels:"):] if "amdhsa.kernels:" in notes else ""
    for blk in re.split(r"\n  - (?=\.)", body)[1:]:
        m = re.search(r"\n    \.name:\s+(\S+)", blk)
        if not m:
            continue
        k = {"name": m.group(1)}
        for key, short in keys.items():
            v = re.search(r"(?:^|\n    )\." + key + r":\s+(\d+)", blk)
            k[short] = int(v.group(1)) if v else None
        out.append(k)
    return out


# Kernels allowed to use scratch: none.
SCRATCH_ALLOWED = ()


def check_no_scratch(objs) -> None:
    bad = []
    for obj in objs:
        for k in kernel_resources(obj):
            if k.get("scratch") and not any(a in k["name"] for a in SCRATCH_ALLOWED):
                bad.append(f"{k['name']}: {k['scratch']} bytes of scratch, {k['vgpr_spill']} VGPR spills")
    if bad:
        raise RuntimeError("kernels spill to scratch memory:\n  " + "\n  ".join(bad))


def build(verbose: bool = True) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), srcs))
    check_no_scratch([o for o in objs if o.endswith(".hip.o")])
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
