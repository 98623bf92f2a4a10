"""Build libkda.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m gated_delta_rule_87_amd.build

Compiles every source under csrc/ with hipcc for --offload-arch=gfx950 into
gated_delta_rule_87_amd/libkda.so. hipcc cross-compiles without a GPU.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

SOURCES = ["kda_api.cpp", "kda_sched.hip", "kda_intra.hip", "kda_chain.hip", "kda_scan.hip", "kda_recurrent.hip",
           "kda_noalloc.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    # MFMA results stay in VGPRs: no v_accvgpr_read before the VALU uses them
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra_flags, "-o", tmp, *[
        # hipcc treats .cpp as host C++ unless told otherwise; the API file is host-only
        s for s in srcs]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed building libkda.so")
    if verbose and err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
