"""Build the HIP library (libdsa.so) for gfx950, in-tree.

    python -m sparse_long_context_c4a_amd.build

Every HIP source under csrc/ is compiled with hipcc for gfx950 and linked
into sparse_long_context_c4a_amd/libdsa.so.  Packed-fp32 instruction
selection is switched off for all device code.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-source flags.  The indexer's scores are finite for finite inputs, so
# its ReLUs need no NaN quieting (a bare v_max_f32 instead of two), and its
# matrix-core results are consumed by VALU math at once, so they go to
# VGPRs rather than to accumulation registers that must be copied out.
_INDEXER_FLAGS = ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {"indexer.hip": _INDEXER_FLAGS, "prefill_index.hip": _INDEXER_FLAGS}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


PROBES = os.path.join(ROOT, "tests", "hw")


def build_probes(verbose=True):
    """Hardware probes the tests load (tests/hw/*.hip -> tests/hw/lib*.so);
    they are not part of libdsa.so."""
    if not os.path.isdir(PROBES):
        return []
    out = []
    for f in sorted(os.listdir(PROBES)):
        if not f.endswith(".hip"):
            continue
        lib = os.path.join(PROBES, "lib" + f[:-4] + ".so")
        cmd = [hipcc(), *FLAGS, "-shared", os.path.join(PROBES, f), "-o", lib + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {f}:\n{r.stderr}")
        os.replace(lib + ".tmp", lib)
        out.append(lib)
    if verbose and out:
        print(f"built {len(out)} test probe(s) under {PROBES}")
    return out


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    build_probes(verbose)
    return LIB


if __name__ == "__main__":
    try:
        build()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
