"""Build libllama_mi355x.so from csrc/*.hip for gfx950 with hipcc (in-tree).

Each translation unit compiles to an object under _build/ in parallel, then
one shared library is linked next to this file. Run as
`python -m decoder_only_transformer_llama_amd.build`.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libllama_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 arithmetic on the device
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every "#pragma unroll" loop over accumulator tiles must unroll fully: a
    # loop left rolled indexes the accumulator array dynamically, which moves
    # it to scratch memory; the remark below turns a refusal into a build error
    "-mllvm", "-pragma-unroll-threshold=262144",
    "-Rpass-missed=loop-unroll",
    # per-kernel resource report: a kernel that spills registers to scratch
    # memory fails the build (scratch loads also count against vmcnt, so one
    # spill can make every wait on in-flight tile loads drain them all)
    "-Rpass-analysis=kernel-resource-usage",
    "-Wno-unused-command-line-argument",
]
UNROLL_REFUSED = "Unable to fully unroll loop as directed by unroll pragma"
SCRATCH = re.compile(r"ScratchSize \[bytes/lane\]: ([0-9]+)")
FUNC = re.compile(r"Function Name: (\S+)")


def _scratch_kernels(log: str):
    """Kernels whose resource report shows scratch memory per lane."""
    bad, name = [], None
    for line in log.splitlines():
        m = FUNC.search(line)
        if m:
            name = m.group(1)
        m = SCRATCH.search(line)
        if m and int(m.group(1)) > 0:
            bad.append(f"{name} ({m.group(1)} bytes/lane)")
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    if UNROLL_REFUSED in r.stderr:
        raise RuntimeError(f"{src}: a '#pragma unroll' loop did not unroll fully:\n{r.stderr}")
    bad = _scratch_kernels(r.stderr)
    if bad:
        raise RuntimeError(f"{src}: kernels spill to scratch memory: " + ", ".join(bad))
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    # --no-undefined: a symbol missing from the sources fails the link, not the first load
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources")
    return LIB_PATH


if __name__ == "__main__":
    try:
        build()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
