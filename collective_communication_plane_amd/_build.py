"""Build libccl.so for gfx950 in-tree with hipcc (no JIT, no torch extension)."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libccl.so")
BUILD_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["ccl_api.cpp", "ccl_plan.cpp", "ccl_collectives.hip", "ccl_reshard.hip",
           "ccl_rmsnorm.hip"]

# ccl_coll_inst.hip is compiled once per (kind, element type) slice.
INSTANCES = [
    ("ar_f32", "KIND_AR", "CCL_FLOAT32"), ("ar_bf16", "KIND_AR", "CCL_BFLOAT16"),
    ("ar_f16", "KIND_AR", "CCL_FLOAT16"), ("ar_i32", "KIND_AR", "CCL_INT32"),
    ("rs_f32", "KIND_RS", "CCL_FLOAT32"), ("rs_bf16", "KIND_RS", "CCL_BFLOAT16"),
    ("rs_f16", "KIND_RS", "CCL_FLOAT16"), ("rs_i32", "KIND_RS", "CCL_INT32"),
    ("ag_b16", "KIND_AG", "CCL_BFLOAT16"), ("ag_b32", "KIND_AG", "CCL_INT32"),
]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-ffp-contract=off",
    # keep the compiler from emitting packed fp32 ALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(job) -> str:
    src, defines, stem = job
    obj = os.path.join(BUILD_DIR, stem + ".o")
    cmd = [HIPCC, *FLAGS, *defines]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    """Compile every source and link libccl.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    work = [(src, [], os.path.splitext(src)[0]) for src in SOURCES]
    work += [("ccl_coll_inst.hip",
              [f"-DCCL_INST_KIND={kind}", f"-DCCL_INST_DT={dt}", f"-DCCL_INST_NAME=dispatch_{name}"],
              f"ccl_coll_{name}") for name, kind, dt in INSTANCES]
    # longest jobs first
    work.sort(key=lambda w: 0 if w[0] == "ccl_coll_inst.hip" else 1)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, work))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
