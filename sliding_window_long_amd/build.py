"""Build libsparse_attn.so (HIP, gfx950 only) in-tree with hipcc.

``python -m sliding_window_long_amd.build`` or ``build_library()``.  Each
source compiles to an object under ``_build/`` (in parallel), then hipcc
links the shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libsparse_attn.so")
SOURCES = ["sa_api.hip", "sa_attn.hip", "sa_blocks.hip", "sa_gate.hip", "sa_compact.hip",
           "sa_token.hip", "sa_decode.hip", "sa_cmp.hip", "sa_bwd.hip", "sa_fp8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # No packed-fp32 VALU instructions (v_pk_{add,mul,fma}_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The kernels never produce or consume NaN (masking uses -inf, and every
    # comparison is written NaN-free), so min/max need no quieting.  The
    # hardware IEEE mode stays at its default: switching it off differs from
    # the device library's functions, which then are not inlined (every
    # kernel would call out for its work-item and group ids).
    "-fno-honor-nans",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source additions.  The token passes read every matrix-core result with
# vector ops: the VGPR form of the MFMA ops saves a copy out of the
# accumulation registers per element.
EXTRA = {"sa_token.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, build_dir: str = BUILD_DIR, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *[f"-D{d}" for d in defines], "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build_library(jobs: int = 4, out: str = LIB_PATH, defines=(), build_dir: str = BUILD_DIR) -> str:
    """Compile and link; `defines` (NAME=VALUE strings) select build-time
    kernel variants, `out` and `build_dir` place a variant elsewhere."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(int(sys.argv[1]) if len(sys.argv) > 1 else 4))
