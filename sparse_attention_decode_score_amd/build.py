"""Builds libdsa.so (the C ABI of the DSA decode path) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libdsa.so")
SOURCES = ["index_score.hip", "topk.hip", "sparse_mla.hip", "lse_combine.hip", "cache_append.hip",
           "capi.cpp"]
# measurement kernels used by the benchmark only (streaming-read ceiling, page-read rate)
PROBE_LIB = os.path.join(LIBDIR, "libdsa_probe.so")
PROBE_SOURCES = ["bandwidth_probe.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the DSA library needs ROCm's hipcc to build")


COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          # packed fp32 instructions stay off: plain float code only
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include")]


# per-source options: the indexer keeps its MFMA results in ordinary VGPRs (its head sum
# reads every result with vector ALU ops; accumulation registers would need one copy each)
EXTRA = {"index_score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.insert(1, "-xhip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")


def _link(sources, out, tmp):
    objs = [os.path.join(tmp, s + ".o") for s in sources]
    with cf.ThreadPoolExecutor(max_workers=min(len(sources), os.cpu_count() or 4)) as ex:
        list(ex.map(_compile, sources, objs))
    out_tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", out_tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(out_tmp, out)


def build(verbose: bool = False) -> str:
    """Compiles every source for gfx950 and links lib/libdsa.so (and the benchmark's
    measurement library lib/libdsa_probe.so); returns the path of libdsa.so."""
    os.makedirs(LIBDIR, exist_ok=True)
    with tempfile.TemporaryDirectory() as tmp:
        _link(SOURCES, LIB, tmp)
        _link(PROBE_SOURCES, PROBE_LIB, tmp)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
