"""Build libisa.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

Usage: python long_context_sparse_indexpool_amd/build.py [--verbose]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libisa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "pool.hip", "indexer_decode.hip", "topk_rows.hip", "mla_decode.hip", "score_prefill.hip",
           "latent_fp8.hip", "kda.hip"]
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
         # packed fp32 instructions are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-source additions: the prefill contraction keeps its MFMA accumulators in
# ordinary VGPRs, so the epilogue reads them without accvgpr moves
EXTRA_FLAGS = {"score_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if resource_usage:
            cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj, r.stderr

    with ThreadPoolExecutor(min(len(SOURCES), 8)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    if verbose or resource_usage:
        for _, err in results:
            for line in err.splitlines():
                if "packed-fp32-ops" in line or "not a recognized feature" in line:
                    continue
                if resource_usage and "remark" not in line:
                    continue
                print(line)
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *[o for o, _ in results], "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv, resource_usage="--resources" in sys.argv)
    print(LIB)
