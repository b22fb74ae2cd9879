"""Builds libh2o.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m kv_cache_eviction_03_amd.build   (or __graft_entry__.build())
Always recompiles. Objects go to kv_cache_eviction_03_amd/_build/, the shared
libraries (libh2o.so, and the measurement probes libh2o_probes.so) next to this file.
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
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libh2o.so")
PROBE_LIB = os.path.join(HERE, "libh2o_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the softmax reads them every tile, and the AGPR form
    # costs a v_accvgpr copy per element each way.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    """libh2o.so from csrc/*.hip, and the measurement probes (csrc/probes/*.hip, the HBM
    read and MFMA ceilings bench.py reports) as libh2o_probes.so."""
    os.makedirs(OUT_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probes = sorted(glob.glob(os.path.join(CSRC, "probes", "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources) + len(probes))) as ex:
        objs = list(ex.map(_compile, sources + probes))
    _link(objs[:len(sources)], LIB)
    _link(objs[len(sources):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
