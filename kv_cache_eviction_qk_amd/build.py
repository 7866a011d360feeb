"""Build libkvev.so (HIP, gfx950) in-tree.

    python -m kv_cache_eviction_qk_amd.build          # compile every source

Each .hip source is compiled to an object with hipcc for gfx950 (in
parallel), then linked into ``kv_cache_eviction_qk_amd/libkvev.so``; the HBM
read-rate probe (csrc/probe/) is built into ``libkvev_probe.so`` beside it.
Packed FP32 instructions are disabled in device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libkvev.so")
# the HBM read-rate probe, a library of its own (only the benchmark's probe mode loads it)
PROBE_SRC = os.path.join(CSRC, "probe", "hbm_read_probe.hip")
PROBE_OUT = os.path.join(HERE, "libkvev_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build", "kvev")
ARCH = os.environ.get("KVEV_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.hip", "score.hip", "select.hip", "compact.hip", "finish.hip", "measure.hip", "window_attn.hip", "h2o_step.hip", "vtoken.hip", "policy.hip", "ring_step.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-source extra flags.  finish.hip takes its compaction ticket with an
# atomic whose result is read only much later; the compiler's atomic optimizer
# would rewrite that atomic into a wave-wide form that reads the result at once,
# so the issuing wave would wait there for every load issued before it (the
# head's keys).  Its other atomics are issued by one lane or go to divergent
# LDS addresses, where the optimizer has nothing to combine.
FILE_FLAGS = {"finish.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    jobs = min(len(SOURCES), max(1, min(16, len(os.sched_getaffinity(0)))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    build_probe()
    return OUT


def build_probe() -> str:
    tmp = PROBE_OUT + ".tmp"
    cmd = [_hipcc(), *HIPCC_FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_OUT)
    return PROBE_OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
