"""Build the HIP library libtsa.so in-tree for gfx950.

Every csrc/*.hip file is compiled separately (in parallel) with hipcc and the
objects are linked into tile_sparse_attention_amd/libtsa.so.  Objects go to
_build/ at the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtsa.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-command-line-argument",
    # packed fp32 VALU forms stay off; scalar fp32 code is generated instead
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source extra flags.  The bf16 attention kernels never see NaN scores
# (finite inputs), and without NaN handling a running max over MFMA results
# compiles to three-way max instructions with no operand quieting.
EXTRA = {name: ["-fno-honor-nans"] for name in ("attention_fwd_bf16.hip", "attention_fwd_fp8.hip", "attention_bwd.hip")}


def _flags(src: str) -> list:
    return [*CFLAGS, *EXTRA.get(os.path.basename(src), [])]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *_flags(src), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


SPILL_CHECKED = ("attention_fwd_bf16.hip", "attention_fwd_f32.hip", "attention_fwd_fp8.hip", "attention_bwd.hip")


def _check_no_spills(src: str) -> None:
    """Fail the build if a kernel of `src` spills registers to scratch memory.

    (SGPR spills into VGPR lanes cost no memory traffic and are allowed.)
    The attention kernels are tuned to fit the register file at two waves per
    SIMD; a spill means a change pushed them over, which costs both speed and
    (through scratch traffic interleaved with the LDS-DMA pipeline) has been
    seen to produce wrong results, so it is treated as a build error.
    """
    asm = os.path.join(BUILD, os.path.basename(src)[:-4] + ".s")
    cmd = [HIPCC, *_flags(src), "--offload-device-only", "-S", src, "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    spills = []
    name = None
    with open(asm) as f:
        for line in f:
            t = line.strip()
            if t.startswith(".name:"):
                name = t.split(None, 1)[1]
            elif t.startswith((".vgpr_spill_count:", ".private_segment_fixed_size:")):
                n = int(t.split()[1])
                if n:
                    spills.append(f"{name}: {t}")
    if spills:
        raise RuntimeError("register spills in " + src + ":\n  " + "\n  ".join(spills))


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    checked = [x for x in srcs if os.path.basename(x) in SPILL_CHECKED]
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
        list(ex.map(_check_no_spills, checked))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
